"""GPU parity for kernel rows whose L2 norm is zero or below the clamp.

GKDT-L GGUF model card, section "Model": the head L2-normalises each kernel
row. The pages do not say what a zero row does; the reading taken (both
sides) is k / max(||k||, 1e-12), the torch F.normalize convention, so a
zero row gives an all-zero map and a row with 0 < ||k|| < 1e-12 is scaled
by 1e12 instead of 1 / ||k||.

Cases, on every path that forms the row weights (the bf16 streamed
contraction with the combined dual kernels parked in the heatmap rows, the
same with heatmap rows too short for them so the contraction combines step
by step, the keypoints-only contraction, and the general kernel in float32
and for bf16 shapes the streamed path does not take):
  * a dual row whose visual kernel is zero (its map is half the text map);
  * a dual row whose text kernel is zero;
  * a single-prompt row that is zero;
  * rows with a nonzero norm below 1e-12 (the clamp sets their scale);
  * a crop whose every valid row is zero in every modality: all maps are
    exactly zero, so every cell ties and the decode returns index 0 and
    score 0.
Each is compared with the oracle (heatmaps, indices, scores, sentinels).
"""
import numpy as np
import pytest
import torch

import gkdsynth
from parity_util import (check_decode, check_heatmaps, check_heatmaps_internal, dev_tensor,
                         floors_of, internal_bounds)

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0DEAD


@pytest.fixture(scope="module")
def gkd():
    import prompt_conditioned_keypoint_amd as m
    m.load()
    assert torch.cuda.is_available()
    return m


@pytest.fixture(scope="module")
def ora():
    import oracle
    oracle._load()
    return oracle


def sentinel(shape, dtype=torch.float32):
    t = torch.empty(shape, dtype=torch.int32, device="cuda").fill_(NAN_BITS)
    return t.view(torch.float32) if dtype == torch.float32 else t


def zero_norm_inputs(B, C, H, W, R, dtype, seed):
    """Crop 0: dual rows (zero visual row 0, zero text row 1, tiny rows 2
    and 3); crop 1: text only (zero row 0, tiny row 1); crop 2: dual, every
    kernel zero; crop 3 (if any): visual only with a zero row; the rest
    random dual/single rows."""
    assert B >= 3 and R >= 4
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, C, H, W)).astype(np.float32)
    kv = rng.standard_normal((B, R, C)).astype(np.float32)
    kt = rng.standard_normal((B, R, C)).astype(np.float32)
    mv = (rng.random((B, R)) < 0.6).astype(np.uint8)
    mt = (rng.random((B, R)) < 0.6).astype(np.uint8)
    # a norm of about 2^-46 sqrt(C) < 1e-12 for C <= 1024: the clamp
    # decides the scale, and the maps stay O(1e-1)
    tiny = np.float32(2.0 ** -46)
    mv[0, :4] = mt[0, :4] = 1
    kv[0, 0] = 0.0
    kt[0, 1] = 0.0
    kv[0, 2] *= tiny
    kt[0, 3] *= tiny
    mv[1] = 0
    mt[1, :2] = 1
    kt[1, 0] = 0.0
    kt[1, 1] *= tiny
    mv[2, :] = 0
    mt[2, :] = 0
    mv[2, : R // 2] = mt[2, : R // 2] = 1
    kv[2] = 0.0
    kt[2] = 0.0
    if B > 3:
        mt[3] = 0
        mv[3, :3] = 1
        kv[3, 1] = 0.0
    if dtype == "bf16":
        q, kv, kt = (gkdsynth.round_bf16_f32(a) for a in (q, kv, kt))
    return q, kv, mv, kt, mt


SHAPES = [
    # bf16 streamed path, combined kernels parked in the heatmap rows
    ("bf16", (4, 256, 24, 24, 16)),
    ("bf16", (4, 1024, 24, 24, 80)),
    # bf16 streamed path, heatmap rows too short: combined step by step
    ("bf16", (4, 256, 4, 4, 12)),
    # bf16 shapes the streamed path does not take (general kernel)
    ("bf16", (3, 40, 5, 7, 9)),
    # float32 (general kernel)
    ("f32", (4, 64, 8, 8, 16)),
    ("f32", (3, 1024, 24, 24, 20)),
]


@pytest.mark.parametrize("dtype,shape", SHAPES, ids=[f"{d}-{s}" for d, s in SHAPES])
def test_zero_and_tiny_norm_rows(gkd, ora, dtype, shape):
    B, C, H, W, R = shape
    q, kv, mv, kt, mt = zero_norm_inputs(B, C, H, W, R, dtype, seed=C + 7 * R + H)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"[zero-norm] {dtype} {shape}", flush=True)
    args = (dev_tensor(q, dt), dev_tensor(kv, dt), dev_tensor(mv), dev_tensor(kt, dt),
            dev_tensor(mt))
    heat, (idx, xy, score) = gkd.kernel_heatmap(*args, out=sentinel((B, R, 4 * H, 4 * W)))
    kp = (sentinel((B, R), torch.int32), sentinel((B, R, 2)), sentinel((B, R)))
    kp_idx, kp_xy, kp_score = gkd.kernel_heatmap(*args, out_decode=kp, with_heatmaps=False)
    torch.cuda.synchronize()

    oh = ora.kernel_heatmap(q, kv, mv, kt, mt)
    valid = ((mv | mt) > 0).astype(np.uint8)
    fl = floors_of(q)
    g = heat.cpu().numpy()
    check_heatmaps(g, oh, valid, dtype, fl)
    if dtype == "bf16":
        check_heatmaps_internal(g, oh, valid, internal_bounds(q))
    for dec in ((idx, xy, score), (kp_idx, kp_xy, kp_score)):
        check_decode(tuple(t.cpu().numpy() for t in dec), oh, valid, dtype, floors=fl)
    # masked rows keep their bytes
    assert np.all(heat.view(torch.int32).cpu().numpy()[valid == 0] == NAN_BITS)

    # the all-zero crop: exact zeros, every cell tied, the first one wins
    z = valid[2] > 0
    assert np.all(g[2][z] == 0.0)
    for i_t, xy_t, s_t in ((idx, xy, score), (kp_idx, kp_xy, kp_score)):
        i_np, xy_np, s_np = i_t.cpu().numpy(), xy_t.cpu().numpy(), s_t.cpu().numpy()
        assert np.all(i_np[2][z] == 0)
        assert np.all(s_np[2][z] == 0.0)
        assert np.allclose(xy_np[2][z], [1.0 / (4 * W) - 1.0, 1.0 / (4 * H) - 1.0], atol=1e-7)
        assert np.all(i_np[2][~z] == -1)

    # a dual row with one zero kernel is half the other modality's map
    half_t = ora.kernel_heatmap(q[:1], None, None, kt[:1], mt[:1])[0, 0] / 2.0
    np.testing.assert_allclose(oh[0, 0], half_t, rtol=0, atol=1e-12)
    tol = 1e-4 if dtype == "f32" else 2e-2 * np.abs(half_t).max() + fl[0]
    assert np.abs(g[0, 0] - half_t).max() <= tol
