"""Helpers for the GPU-vs-oracle parity tests (test infrastructure).

Tolerances (floating point), per valid row of a heatmap:
  * float32 inputs: max |gpu - oracle| <= 1e-4;
  * bfloat16 inputs: max |gpu - oracle| <= 2e-2 * max |oracle row| + floor,
    floor = 1e-6 * sqrt(C) * max |F_b|: every heatmap value is a sum of
    normalised-kernel terms bounded by ||G_p|| <= sqrt(C) max |F_b|, so a
    row that cancels to zero exactly (opposite dual kernels) still carries
    float32 rounding of that size.
Argmax: the decision is taken in float32 on both sides (the oracle's
double heatmap rounded to float32, then a first-maximum scan). Indices must
agree exactly wherever the oracle's top-2 gap exceeds GAP_TOL; elsewhere the
GPU's pick must hold a value within GAP_TOL of the oracle maximum.
Prototypes: float32 within 1e-5 * max |oracle row|; bfloat16 within one
bfloat16 ulp of the oracle's rounded value.

Internal bound (bfloat16 inputs, the same values on both sides): beside
the 2e-2 relative bar, every heatmap value must lie within
INTERNAL_REL * sqrt(C) * max |F_b| of the oracle. The GPU's error is pure
float32 evaluation, bounded term by term in the worst case:
  * bf16 x bf16 products are exact in float32; a sum of C terms taken 32
    at a time and accumulated K-step by K-step is off by at most about
    (C/32 + 32) 2^-24 of sum |k^_c G_c| <= ||G(p)||_2 <= sqrt(C) max |F_b|
    (Cauchy-Schwarz with ||k^|| = 1; G is a convex combination of F);
  * the row norm, a float32 sum of at most C/4 squares per thread (256 at
    C = 1024), is off by at most C/4 2^-24 relative, so the weight 1/||k||
    by half that;
  * a two-prompt row's combined kernel, carried as bfloat16 hi + lo parts,
    is within 2^-18 of its value per element;
  * the expand's two fma stages add a few ulps of max |P|.
Together about 1.5e-5 * sqrt(C) max |F_b| at C <= 1024; the bound is 2e-5
(typical errors are a hundred times smaller). A wrong expand tap or a
fusion weight off by 1% is far outside it.
"""
from __future__ import annotations

import numpy as np
import torch

GAP_TOL = 1e-3
F32_ATOL = 1e-4
BF16_RTOL = 2e-2
INTERNAL_REL = 2e-5


def floors_of(query):
    """Per-crop float32 evaluation floor 1e-6 sqrt(C) max |F_b|."""
    q = np.asarray(query)
    return 1e-6 * np.sqrt(q.shape[1]) * np.abs(q).reshape(q.shape[0], -1).max(1)


def internal_bounds(query):
    """Per-crop float32-evaluation bound INTERNAL_REL sqrt(C) max |F_b|."""
    q = np.asarray(query)
    return INTERNAL_REL * np.sqrt(q.shape[1]) * np.abs(q).reshape(q.shape[0], -1).max(1)


def check_heatmaps_internal(gpu, ora, valid, bounds):
    """gpu [b,R,Ho,Wo] float32 vs ora (float64) on valid rows, held to the
    float32-evaluation bound of crop b (identical bf16 inputs only)."""
    worst = 0.0
    for b in range(gpu.shape[0]):
        for r in range(gpu.shape[1]):
            if not valid[b, r]:
                continue
            err = np.abs(gpu[b, r].astype(np.float64) - ora[b, r]).max()
            assert err <= bounds[b], (b, r, err, bounds[b])
            worst = max(worst, err / bounds[b])
    return worst


def dev_tensor(a, dtype=None, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return t.to(dtype) if dtype is not None else t


def feat_dtype(d):
    return torch.bfloat16 if d["dtype"] == "bf16" else torch.float32


def bf16_ulp(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    return np.where(x > 0, 2.0 ** (e - 7), 2.0 ** -133)


def check_protos(gpu, ora, valid, dtype, fmax):
    """gpu/ora [B,R,C]; only rows with valid set are compared. fmax [B] is
    max |support| per crop: the GPU forms each prototype in float32 from
    weights carried to ~2^-18 relative (bf16 hi + lo) and float32 sums, so
    its pre-rounding value is within 1e-5 * max |fibre| of the exact one.
    float32: |g - o| <= 1e-5 max|S_b|; bfloat16: additionally one ulp of
    the larger of the two rounded values."""
    g = np.asarray(gpu, np.float64)
    o = np.asarray(ora, np.float64)
    eps = 1e-5 * np.asarray(fmax, np.float64)[:, None, None]
    tol = np.broadcast_to(eps, g.shape)
    if dtype != "f32":
        tol = tol + bf16_ulp(np.maximum(np.abs(g), np.abs(o)))
    m = np.broadcast_to((valid > 0)[..., None], g.shape)
    assert np.isfinite(g[m]).all()
    bad = (np.abs(g - o) > tol) & m
    assert not bad.any(), (np.argwhere(bad)[:5], g[bad][:5], o[bad][:5])


def row_tol(o, dtype, floor):
    if dtype == "f32":
        return F32_ATOL
    return BF16_RTOL * np.abs(o).max() + floor


def check_heatmaps(gpu, ora, valid, dtype, floors=None):
    """gpu [b,R,Ho,Wo] float32, ora float64 (NaN where masked); floors [b]
    = 1e-6 sqrt(C) max|F_b| (see the module docstring), default 0."""
    worst = 0.0
    for b in range(gpu.shape[0]):
        for r in range(gpu.shape[1]):
            if not valid[b, r]:
                continue
            o = ora[b, r]
            g = gpu[b, r].astype(np.float64)
            err = np.abs(g - o).max()
            tol = row_tol(o, dtype, 0.0 if floors is None else floors[b])
            assert err <= tol, (b, r, err, tol)
            worst = max(worst, err / (tol if tol > 0 else 1))
    return worst


def check_decode(gpu_dec, ora_heat, valid, dtype, gap_tol=GAP_TOL, floors=None):
    """gpu_dec = (idx, xy, score) numpy for the same rows as ora_heat."""
    import oracle
    idx, xy, score = gpu_dec
    o_idx, o_xy, o_score, o_gap = oracle.peak_decode(
        ora_heat.astype(np.float32).astype(np.float64), valid)
    _, _, _, gap64 = oracle.peak_decode(np.nan_to_num(ora_heat, nan=0.0), valid)
    B, R, Ho, Wo = ora_heat.shape
    n_exact = n_near = 0
    for b in range(B):
        for r in range(R):
            if not valid[b, r]:
                assert idx[b, r] == -1
                assert np.isnan(xy[b, r]).all() and score[b, r] == -np.inf
                continue
            if gap64[b, r] > gap_tol:
                assert idx[b, r] == o_idx[b, r], (b, r, idx[b, r], o_idx[b, r], gap64[b, r])
                n_exact += 1
            else:
                h = ora_heat[b, r].reshape(-1)
                assert 0 <= idx[b, r] < Ho * Wo
                assert h[idx[b, r]] >= h.max() - gap_tol, (b, r)
                n_near += 1
            p = int(idx[b, r])
            y, x = divmod(p, Wo)
            assert abs(xy[b, r, 0] - ((2 * x + 1) / Wo - 1)) < 1e-6
            assert abs(xy[b, r, 1] - ((2 * y + 1) / Ho - 1)) < 1e-6
            ref = ora_heat[b, r].reshape(-1)[p]
            tol = row_tol(ora_heat[b, r], dtype, 0.0 if floors is None else floors[b])
            assert abs(score[b, r] - ref) <= tol, (b, r, score[b, r], ref)
    return n_exact, n_near
