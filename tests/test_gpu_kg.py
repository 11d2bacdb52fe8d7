"""GPU parity of the kernel-generation transformer (gkd_kg_transformer, HIP
through the C ABI) against the float64 oracle on the same seeded inputs.

Tolerance, from the arithmetic: the kernels round every matrix operand to
bfloat16 (unit roundoff u = 2^-9), i.e. the block input, Q, K, V, the
attention probabilities, the attention output and the FFN hidden layer,
and the final kernels once more. Each rounding adds an independent error
of at most u relative; about 8 of them per block reach an output, and
LayerNorm keeps the outputs at unit scale, so over 2 blocks the RMS error
is about u * sqrt(16 / 3) ~ 0.005. 3x that (0.015) bounds the RMS error, and
0.1 (about 6 sigma of the same estimate at the largest output magnitudes
of ~5) the largest one. A wrong head, mask or slot puts errors of order 1
on whole rows.
"""
import numpy as np
import pytest
import torch

import gkdsynth
from parity_util import dev_tensor

pytestmark = pytest.mark.gpu

TOL_RMS = 0.015
TOL_MAX = 0.1


@pytest.fixture(scope="module")
def gkd():
    import prompt_conditioned_keypoint_amd as m
    m.load()
    assert torch.cuda.is_available()
    return m


@pytest.fixture(scope="module")
def okg():
    from oracle import kg
    return kg


def case(seed, B, R, C, H, W, F, nb, p_vis=0.7, p_txt=0.6):
    rng = np.random.default_rng(seed)
    vis = gkdsynth.round_bf16_f32(rng.standard_normal((B, R, C)).astype(np.float32))
    txt = gkdsynth.round_bf16_f32(rng.standard_normal((B, R, C)).astype(np.float32))
    mv = (rng.random((B, R)) < p_vis).astype(np.uint8)
    mt = (rng.random((B, R)) < p_txt).astype(np.uint8)
    q = gkdsynth.round_bf16_f32(rng.standard_normal((B, C, H, W)).astype(np.float32))
    w = gkdsynth.kg_weights(C, F, nb, seed=seed + 1)
    return vis, mv, txt, mt, q, w


def bf(x):
    return dev_tensor(np.ascontiguousarray(x)).to(torch.bfloat16)


SENTINEL = 0x7FC1  # a bfloat16 NaN the kernels never write


def run(gkd, vis, mv, txt, mt, q, w, nb, F, tokens_skip=None, modalities="both"):
    """Kernels [B, 2R, C] in slot order; rows with no prompt in either
    modality are NaN (the call leaves them as they were, which is checked)."""
    if tokens_skip is None:
        query, kw = bf(q), {}
    else:
        B, C = q.shape[:2]
        tok = q.reshape(B, C, -1).transpose(0, 2, 1)
        lead = np.full((B, tokens_skip, C), 7.0, np.float32)
        query = bf(np.concatenate([lead, tok], axis=1))
        kw = dict(token_hw=q.shape[2:], token_skip=tokens_skip)
    B, R, C = txt.shape
    out = torch.full((2, B, R, C), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vkw = {} if modalities == "text" else dict(kern_vis=bf(vis), mask_vis=dev_tensor(mv))
    got = gkd.kg_transformer(query, bf(w), kern_txt=bf(txt), mask_txt=dev_tensor(mt),
                             n_blocks=nb, d_ff=F, out=out, **vkw, **kw)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    prompted = (mt > 0) if modalities == "text" else ((mv > 0) | (mt > 0))
    bits = out.view(torch.int16).cpu().numpy()
    idle = ~prompted
    assert np.all(bits[:, idle] == SENTINEL), "a row without a prompt was written"
    o = out.float().cpu().numpy().astype(np.float64)
    o[:, idle] = np.nan
    return np.concatenate([o[0], o[1]], axis=1)   # [B, 2R, C] slot order


def check(got, want):
    """Compares the slots of prompted rows (NaN in got marks the others)."""
    m = ~np.isnan(got)
    assert m.any()
    err = np.abs(got[m] - want[m])
    rms = float(np.sqrt(np.mean(err ** 2)))
    assert np.all(np.isfinite(got[m]))
    assert rms <= TOL_RMS, (rms, float(err.max()))
    assert err.max() <= TOL_MAX, (rms, float(err.max()))


@pytest.mark.parametrize("B,R,C,H,W,F", [(3, 7, 128, 5, 7, 192), (2, 40, 192, 9, 9, 128),
                                         (1, 3, 64, 1, 1, 64), (2, 9, 128, 48, 48, 128),
                                         (1, 5, 64, 25, 37, 64)])
def test_kg_matches_oracle_small(gkd, okg, B, R, C, H, W, F):
    """Ragged slot counts (14, 80, 6, 18, 10 slots against 16-query tiles),
    ragged key tails (35, 81, 1 keys; 2304 and 925 keys stream through the
    cross-attention's 64-key chunks in 36 and 15 chunks, the last one
    partial) and tiles past M and N."""
    vis, mv, txt, mt, q, w = case(B * 100 + R, B, R, C, H, W, F, 2)
    mv[0, -1] = mt[0, -1] = 0   # a padding row
    print(f"[kg] small B={B} R={R} C={C} HW={H * W} F={F}", flush=True)
    got = run(gkd, vis, mv, txt, mt, q, w, 2, F)
    want = okg.kg_transformer(vis, mv, txt, mt, q, w, 2, F)
    check(got, want)


def test_kg_unprompted_crop_one_block_and_text_only(gkd, okg):
    """A crop with no prompted row (nothing of it is written), one block,
    and a call with only the text modality."""
    vis, mv, txt, mt, q, w = case(5, 3, 9, 128, 4, 6, 128, 1)
    mv[1] = mt[1] = 0
    print("[kg] unprompted crop", flush=True)
    got = run(gkd, vis, mv, txt, mt, q, w, 1, 128)
    assert np.isnan(got[1]).all()
    want = okg.kg_transformer(vis, mv, txt, mt, q, w, 1, 128)
    check(got, want)
    got = run(gkd, vis, mv, txt, mt, q, w, 1, 128, modalities="text")
    check(got, okg.kg_transformer(None, None, txt, mt, q, w, 1, 128))


def test_kg_tokens_layout_is_bit_identical(gkd):
    vis, mv, txt, mt, q, w = case(9, 2, 11, 128, 6, 5, 128, 2)
    print("[kg] token layout", flush=True)
    a = run(gkd, vis, mv, txt, mt, q, w, 2, 128)
    b = run(gkd, vis, mv, txt, mt, q, w, 2, 128, tokens_skip=5)
    np.testing.assert_array_equal(a, b)


def test_kg_full_size_sampled(gkd, okg):
    """B=256 crops, C=1024, R=80 (160 slots), 24x24 query, d_ff=1024, 2
    blocks, launched as the benchmark launches it; the oracle recomputes 3
    sampled crops. Two runs are bit-identical."""
    B, R, C, H, W, F = 256, 80, 1024, 24, 24, 1024
    vis, mv, txt, mt, q, w = case(2026, B, R, C, H, W, F, 2)
    n = np.random.default_rng(1).integers(1, R + 1, B)
    pad = np.arange(R)[None, :] >= n[:, None]
    mv[pad] = 0
    mt[pad] = 0
    print("[kg] full size", flush=True)
    a = run(gkd, vis, mv, txt, mt, q, w, 2, F)
    b = run(gkd, vis, mv, txt, mt, q, w, 2, F)
    np.testing.assert_array_equal(a, b)   # NaN rows compare equal here
    for i in (0, 101, 255):
        want = okg.kg_transformer(vis[i:i + 1], mv[i:i + 1], txt[i:i + 1], mt[i:i + 1],
                                  q[i:i + 1], w, 2, F)
        check(a[i:i + 1], want)


def test_kg_highres_query_sampled(gkd, okg):
    """Crops of the high-resolution batch's shape: all 80 rows text-prompted
    (the 80 visual slots unprompted), C=1024, a 48x48 query (2304
    cross-attention keys a crop), d_ff=1024, 2 blocks; 32 crops, the oracle
    recomputes 2 sampled ones."""
    B, R, C, H, W, F = 32, 80, 1024, 48, 48, 1024
    vis, mv, txt, mt, q, w = case(77, B, R, C, H, W, F, 2, p_vis=0.0, p_txt=1.0)
    print("[kg] high-resolution query", flush=True)
    a = run(gkd, vis, mv, txt, mt, q, w, 2, F, modalities="text")
    for i in (0, 31):
        want = okg.kg_transformer(None, None, txt[i:i + 1], mt[i:i + 1], q[i:i + 1], w, 2, F)
        check(a[i:i + 1], want)
