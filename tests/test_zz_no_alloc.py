"""GPU test of gkd_kg_transformer_noalloc, the kernel-generation transformer
entry point for callers that cannot allocate (its workspace is the
library's static device array, shared by every call on the GPU).

Through the C ABI, two calls in a row (the second with fewer crops and a
different prompt pattern, so the array still holds the first call's larger
contents) must each equal, bit for bit, gkd_kg_transformer on the same
inputs with a caller-owned workspace: both run the same kernels in the
same order. A shape beyond the static workspace is rejected.
"""
import numpy as np
import pytest
import torch

import gkdsynth
from parity_util import dev_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gkd():
    import prompt_conditioned_keypoint_amd as m
    m.load()
    assert torch.cuda.is_available()
    return m


def bf(x):
    return dev_tensor(np.ascontiguousarray(x)).to(torch.bfloat16)


def inputs(seed, B, R, C, H, W, p_vis, p_txt):
    rng = np.random.default_rng(seed)
    vis = rng.standard_normal((B, R, C)).astype(np.float32)
    txt = rng.standard_normal((B, R, C)).astype(np.float32)
    mv = (rng.random((B, R)) < p_vis).astype(np.uint8)
    mt = (rng.random((B, R)) < p_txt).astype(np.uint8)
    q = rng.standard_normal((B, C, H, W)).astype(np.float32)
    return bf(vis), dev_tensor(mv), bf(txt), dev_tensor(mt), bf(q)


@pytest.mark.parametrize("tokens", [False, True])
def test_kg_noalloc_equals_workspace_call(gkd, tokens):
    C, H, W, R, F, nb = 1024, 24, 24, 80, 1024, 2
    w = bf(gkdsynth.kg_weights(C, F, nb, seed=11))
    for call, (B, seed, pv, pt) in enumerate([(6, 101, 0.7, 0.6), (3, 202, 0.3, 0.9)]):
        print(f"[kg-noalloc] tokens={tokens} call {call} B={B}", flush=True)
        vis, mv, txt, mt, q = inputs(seed, B, R, C, H, W, pv, pt)
        kw = {}
        if tokens:
            tok = q.reshape(B, C, H * W).transpose(1, 2)
            q = torch.cat([torch.full((B, 5, C), 3.0, dtype=torch.bfloat16, device="cuda"), tok],
                          1).contiguous()
            kw = dict(token_hw=(H, W), token_skip=5)
        # rows without a prompt are not written: both outputs start equal
        ref = torch.full((2, B, R, C), 7.0, dtype=torch.bfloat16, device="cuda")
        gkd.kg_transformer(q, w, kern_vis=vis, mask_vis=mv, kern_txt=txt, mask_txt=mt,
                           n_blocks=nb, d_ff=F, out=ref, **kw)
        out = torch.full_like(ref, 7.0)
        got = gkd.kg_transformer(q, w, kern_vis=vis, mask_vis=mv, kern_txt=txt, mask_txt=mt,
                                 n_blocks=nb, d_ff=F, out=out, workspace="static", **kw)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert bool(torch.isfinite(got.float()).all())
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), call


def test_kg_noalloc_rejects_beyond_static_workspace(gkd):
    C, H, W, R, F, nb = 1024, 24, 24, 80, 1024, 2
    B = 11
    assert gkd.kg_workspace_size(B, C, H, W, R, F) > gkd.binding.GKD_KG_STATIC_WORKSPACE_BYTES
    vis, mv, txt, mt, q = inputs(5, B, R, C, H, W, 0.5, 0.5)
    w = bf(gkdsynth.kg_weights(C, F, nb, seed=11))
    with pytest.raises(gkd.GkdError) as e:
        gkd.kg_transformer(q, w, kern_vis=vis, mask_vis=mv, kern_txt=txt, mask_txt=mt,
                           n_blocks=nb, d_ff=F, workspace="static")
    assert e.value.status == 4
