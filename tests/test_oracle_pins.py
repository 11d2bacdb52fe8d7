"""Pins for the CPU oracle: closed forms, invariants, library routines and
exact rational brute force. None of these re-types the oracle's own
formula in floating point; each would fail on a plausible slip (a dropped
term, a wrong half-pixel offset, sigma vs sigma^2, a sum instead of a mean,
a transposed index, a last-occurrence argmax).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def dyadic(rng, shape, denom=8, span=16):
    return rng.integers(-span, span + 1, size=shape).astype(np.float64) / denom


# --------------------------------------------------------------------------
# bilinear 4x upsample
# --------------------------------------------------------------------------
def _load_delta_golden():
    rows = []
    with open(os.path.join(HERE, "golden", "upsample4_delta.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            t = line.split()
            rows.append((t[0], int(t[1]), int(t[2]), int(t[3]),
                         [float(v) for v in t[4:]]))
    return rows


@pytest.mark.parametrize("case", _load_delta_golden(), ids=lambda c: c[0])
def test_upsample_delta_closed_form(oracle_mod, case):
    _, n_in, at, first, weights = case
    # 2-D delta on an n_in x 3 map; the column profile through x of the delta
    F = np.zeros((1, n_in, 3))
    F[0, at, 1] = 1.0
    G = oracle_mod.upsample4(F)[0]
    col = G[:, 4 * 1 + 1]          # x = 5 sits fully on source column 1
    assert G[:, 5].tolist() == G[:, 6].tolist()  # 7/8 both sides of centre
    expect = np.zeros(4 * n_in)
    expect[first:first + len(weights)] = weights
    # x=5 has weight 7/8 on column 1, so the profile is scaled by 7/8
    np.testing.assert_array_equal(col, expect * 0.875)


def test_upsample_matches_torch_interpolate_on_dyadic(oracle_mod):
    rng = np.random.default_rng(1)
    F = dyadic(rng, (3, 5, 7))
    G = oracle_mod.upsample4(F)
    ref = torch.nn.functional.interpolate(
        torch.from_numpy(F)[None], scale_factor=4, mode="bilinear",
        align_corners=False)[0].numpy()
    np.testing.assert_array_equal(G, ref)


def test_upsample_close_to_torch_on_random(oracle_mod):
    rng = np.random.default_rng(2)
    F = rng.standard_normal((2, 24, 24))
    G = oracle_mod.upsample4(F)
    ref = torch.nn.functional.interpolate(
        torch.from_numpy(F)[None], scale_factor=4, mode="bilinear",
        align_corners=False)[0].numpy()
    np.testing.assert_allclose(G, ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("H,W", [(5, 7), (1, 6), (6, 1), (24, 24)])
def test_upsample_corners_matches_torch_interpolate(oracle_mod, H, W):
    """The align_corners=True grid against torch's bilinear interpolate
    with align_corners=True (float64), the corners exactly on the source
    corners."""
    rng = np.random.default_rng(H * 31 + W)
    F = rng.standard_normal((3, H, W))
    G = oracle_mod.upsample4(F, corners=True)
    ref = torch.nn.functional.interpolate(torch.from_numpy(F)[None], scale_factor=4,
                                          mode="bilinear", align_corners=True)[0].numpy()
    np.testing.assert_allclose(G, ref, rtol=0, atol=1e-12)
    assert np.array_equal(G[:, 0, 0], F[:, 0, 0]) and np.array_equal(G[:, -1, -1], F[:, -1, -1])


def test_heatmap_corners_is_conv_of_corner_upsample(oracle_mod):
    """With corners the heatmap is the normalised kernel applied to the
    align_corners=True upsample (torch's), mask-averaged like the default."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 8, 5, 6))
    k = rng.standard_normal((2, 3, 8))
    m = np.array([[1, 0, 1], [1, 1, 1]], np.uint8)
    h = oracle_mod.kernel_heatmap(q, k, m, corners=True)
    up = torch.nn.functional.interpolate(torch.from_numpy(q), scale_factor=4, mode="bilinear",
                                         align_corners=True).numpy()
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    ref = np.einsum("brc,bcyx->bryx", kn, up)
    ok = m > 0
    np.testing.assert_allclose(h[ok], ref[ok], rtol=0, atol=1e-12)
    assert np.all(np.isnan(h[~ok]))


def test_upsample_constant_ramp_and_edge_duplicates(oracle_mod):
    F = np.full((1, 4, 5), 2.5)
    assert np.all(oracle_mod.upsample4(F) == 2.5)
    # ramp along y: exact source position inside, clamped at the borders
    H = 6
    F = np.tile(np.arange(H, dtype=np.float64)[:, None], (1, 3))[None]
    G = oracle_mod.upsample4(F)[0][:, 0]
    for y in range(4 * H):
        src = min(max((y + 0.5) / 4 - 0.5, 0.0), H - 1.0)
        assert G[y] == src
    rng = np.random.default_rng(3)
    G = oracle_mod.upsample4(rng.standard_normal((2, 5, 6)))
    assert np.array_equal(G[:, 0], G[:, 1])
    assert np.array_equal(G[:, -2], G[:, -1])
    assert np.array_equal(G[:, :, 0], G[:, :, 1])
    assert np.array_equal(G[:, :, -2], G[:, :, -1])


# --------------------------------------------------------------------------
# kernel heatmaps
# --------------------------------------------------------------------------
UNIT4 = np.array([0.5, -0.5, 0.5, 0.5])        # dyadic unit vector
UNIT4B = np.array([0.5, 0.5, -0.5, 0.5])       # orthogonal to UNIT4


def _delta_response(H, W, i, j):
    d = np.zeros((1, H, W))
    d[0, i, j] = 1.0
    return torch.nn.functional.interpolate(
        torch.from_numpy(d)[None], scale_factor=4, mode="bilinear",
        align_corners=False)[0, 0].numpy()


def test_heatmap_planted_peak_closed_form(oracle_mod):
    H, W, alpha = 5, 6, 4.0
    F = np.zeros((1, 4, H, W))
    F[0, :, 2, 3] = alpha * UNIT4
    k = 3.0 * UNIT4                               # norm 3, normalises exactly
    hm = oracle_mod.kernel_heatmap(F, None, None, k[None, None],
                                   np.ones((1, 1), np.uint8))
    np.testing.assert_array_equal(hm[0, 0], alpha * _delta_response(H, W, 2, 3))


def test_heatmap_dual_is_mean_of_modalities(oracle_mod):
    H, W = 4, 5
    F = np.zeros((1, 4, H, W))
    F[0, :, 1, 1] = 2.0 * UNIT4
    F[0, :, 3, 4] = 6.0 * UNIT4B
    kv = (5.0 * UNIT4)[None, None]
    kt = (0.25 * UNIT4B)[None, None]
    one = np.ones((1, 1), np.uint8)
    hm = oracle_mod.kernel_heatmap(F, kv, one, kt, one)[0, 0]
    expect = (2.0 * _delta_response(H, W, 1, 1)
              + 6.0 * _delta_response(H, W, 3, 4)) / 2
    np.testing.assert_array_equal(hm, expect)
    # one mask off reduces exactly to the single modality
    zero = np.zeros((1, 1), np.uint8)
    hv = oracle_mod.kernel_heatmap(F, kv, one, kt, zero)[0, 0]
    np.testing.assert_array_equal(hv, 2.0 * _delta_response(H, W, 1, 1))
    ht = oracle_mod.kernel_heatmap(F, kv, zero, kt, one)[0, 0]
    np.testing.assert_array_equal(ht, 6.0 * _delta_response(H, W, 3, 4))


def _frac_heatmap(F, kerns):
    """Exact rational heatmap of one row: F [C,H,W] dyadic, kerns = list of
    integer kernel rows with perfect-square squared norms."""
    C, H, W = F.shape
    Ho, Wo = 4 * H, 4 * W

    def taps(o, n):
        num = Fraction(2 * o + 1, 8) - Fraction(1, 2)
        src = max(num, Fraction(0))
        i0 = math.floor(src)
        i1 = min(i0 + 1, n - 1)
        lam = src - i0
        out = {}
        out[i0] = out.get(i0, 0) + (1 - lam)
        out[i1] = out.get(i1, 0) + lam
        return out

    Ff = [[[Fraction(float(F[c, i, j])) for j in range(W)] for i in range(H)]
          for c in range(C)]
    khat = []
    for k in kerns:
        n2 = sum(int(v) * int(v) for v in k)
        n = math.isqrt(n2)
        assert n * n == n2
        khat.append([Fraction(int(v), n) for v in k])
    out = np.zeros((Ho, Wo), dtype=object)
    for y in range(Ho):
        ty = taps(y, H)
        for x in range(Wo):
            tx = taps(x, W)
            total = Fraction(0)
            for kh in khat:
                m = Fraction(0)
                for c in range(C):
                    g = sum(a * b * Ff[c][i][j] for i, a in ty.items()
                            for j, b in tx.items())
                    m += kh[c] * g
                total += m
            out[y, x] = total / len(khat)
    return out


def test_heatmap_exact_rational_brute_force(oracle_mod):
    rng = np.random.default_rng(4)
    C, H, W = 3, 3, 2
    F = dyadic(rng, (1, C, H, W))
    kv = np.array([[[1, 2, 2], [2, -3, 6], [0, 3, 4]]], np.float64)
    kt = np.array([[[-2, 1, 2], [4, 4, 7], [1, 2, 2]]], np.float64)
    mv = np.array([[1, 1, 0]], np.uint8)
    mt = np.array([[0, 1, 1]], np.uint8)
    hm = oracle_mod.kernel_heatmap(F, kv, mv, kt, mt)[0]
    rows = [[kv[0, 0]], [kv[0, 1], kt[0, 1]], [kt[0, 2]]]
    for r, ks in enumerate(rows):
        exact = _frac_heatmap(F[0], ks)
        ex = np.array([[float(v) for v in row] for row in exact])
        np.testing.assert_allclose(hm[r], ex, rtol=1e-15, atol=1e-15)


def test_heatmap_commutes_with_upsample_library_route(oracle_mod):
    """conv at low resolution then torch bilinear == oracle (upsample first)."""
    rng = np.random.default_rng(5)
    B, C, H, W, R = 2, 16, 5, 7, 3
    F = rng.standard_normal((B, C, H, W))
    kv = rng.standard_normal((B, R, C))
    kt = rng.standard_normal((B, R, C))
    mv = np.array([[1, 0, 1], [1, 1, 0]], np.uint8)
    mt = np.array([[0, 1, 1], [1, 0, 0]], np.uint8)
    hm = oracle_mod.kernel_heatmap(F, kv, mv, kt, mt)
    for b in range(B):
        for r in range(R):
            acc, n = 0.0, 0
            for k, m in ((kv, mv), (kt, mt)):
                if m[b, r]:
                    kh = k[b, r] / np.linalg.norm(k[b, r])
                    low = np.tensordot(kh, F[b], axes=(0, 0))
                    acc = acc + torch.nn.functional.interpolate(
                        torch.from_numpy(low)[None, None], scale_factor=4,
                        mode="bilinear", align_corners=False)[0, 0].numpy()
                    n += 1
            if n:
                np.testing.assert_allclose(hm[b, r], acc / n, rtol=0,
                                           atol=1e-12)
            else:
                assert np.isnan(hm[b, r]).all()


def test_heatmap_scale_invariance_sign_and_linearity(oracle_mod):
    rng = np.random.default_rng(6)
    F1 = rng.standard_normal((1, 32, 4, 4))
    F2 = rng.standard_normal((1, 32, 4, 4))
    k = rng.standard_normal((1, 1, 32))
    one = np.ones((1, 1), np.uint8)
    h = oracle_mod.kernel_heatmap(F1, None, None, k, one)
    np.testing.assert_allclose(
        oracle_mod.kernel_heatmap(F1, None, None, 3.7 * k, one), h,
        rtol=0, atol=1e-12)
    np.testing.assert_allclose(
        oracle_mod.kernel_heatmap(F1, None, None, -0.01 * k, one), -h,
        rtol=0, atol=1e-12)
    h12 = oracle_mod.kernel_heatmap(F1 + F2, None, None, k, one)
    h2 = oracle_mod.kernel_heatmap(F2, None, None, k, one)
    np.testing.assert_allclose(h12, h + h2, rtol=0, atol=1e-12)


def test_heatmap_zero_kernel_and_masked_rows(oracle_mod):
    rng = np.random.default_rng(7)
    F = rng.standard_normal((1, 8, 3, 3))
    k = np.zeros((1, 3, 8))
    k[0, 1] = np.nan                      # masked row: must never be read
    k[0, 2] = rng.standard_normal(8)
    m = np.array([[1, 0, 1]], np.uint8)
    hm = oracle_mod.kernel_heatmap(F, None, None, k, m)
    assert np.all(hm[0, 0] == 0.0)        # zero kernel -> all-zero map
    assert np.isnan(hm[0, 1]).all()       # untouched
    assert np.isfinite(hm[0, 2]).all()


# --------------------------------------------------------------------------
# peak decode
# --------------------------------------------------------------------------
def test_decode_matches_numpy_argmax_and_partition(oracle_mod):
    rng = np.random.default_rng(8)
    h = rng.integers(0, 6, size=(3, 4, 8, 12)).astype(np.float64)  # many ties
    h[0, 0] = 7.0                                              # constant map
    idx, xy, score, gap = oracle_mod.peak_decode(h)
    flat = h.reshape(3, 4, -1)
    np.testing.assert_array_equal(idx, flat.argmax(-1))
    assert idx[0, 0] == 0
    np.testing.assert_array_equal(score, flat.max(-1))
    top2 = -np.sort(-flat, axis=-1)[..., :2]
    np.testing.assert_array_equal(gap, top2[..., 0] - top2[..., 1])
    # coordinate map: cell centres of the Ho x Wo grid in -1..1
    Ho, Wo = 8, 12
    np.testing.assert_allclose(xy[..., 0], (2 * (idx % Wo) + 1) / Wo - 1,
                               rtol=0, atol=0)
    corner = np.zeros((1, 1, Ho, Wo))
    corner[0, 0, -1, -1] = 1.0
    i2, xy2, _, _ = oracle_mod.peak_decode(corner)
    assert i2[0, 0] == Ho * Wo - 1
    assert abs(xy2[0, 0, 0] - (1 - 1 / Wo)) < 1e-15
    assert abs(xy2[0, 0, 1] - (1 - 1 / Ho)) < 1e-15
    corner[0, 0] = 0
    corner[0, 0, 0, 0] = 1.0
    _, xy3, _, _ = oracle_mod.peak_decode(corner)
    assert abs(xy3[0, 0, 0] - (-1 + 1 / Wo)) < 1e-15
    assert abs(xy3[0, 0, 1] - (-1 + 1 / Ho)) < 1e-15


@pytest.mark.parametrize("Ho,Wo", [(96, 96), (7, 5), (1, 4), (3, 1)])
def test_decode_corner_coordinates_are_linspace(oracle_mod, Ho, Wo):
    """Corner-aligned coordinates: index i of n sits at numpy's
    linspace(-1, 1, n)[i] (0 for a one-cell axis); the default cell-centre
    coordinates are the midpoints of n equal cells of [-1, 1]. Every cell is
    made the peak once."""
    P = Ho * Wo
    heat = np.zeros((1, P, Ho, Wo))
    heat.reshape(P, P)[np.arange(P), np.arange(P)] = 1.0
    idx, xy, _, _ = oracle_mod.peak_decode(heat, corners=True)
    _, xyc, _, _ = oracle_mod.peak_decode(heat)
    lx = np.linspace(-1, 1, Wo) if Wo > 1 else np.zeros(1)
    ly = np.linspace(-1, 1, Ho) if Ho > 1 else np.zeros(1)
    np.testing.assert_array_equal(idx[0], np.arange(P))
    np.testing.assert_allclose(xy[0, :, 0], lx[np.arange(P) % Wo], rtol=0, atol=1e-15)
    np.testing.assert_allclose(xy[0, :, 1], ly[np.arange(P) // Wo], rtol=0, atol=1e-15)
    mid_x = (np.linspace(-1, 1, Wo + 1)[:-1] + np.linspace(-1, 1, Wo + 1)[1:]) / 2
    np.testing.assert_allclose(xyc[0, :, 0], mid_x[np.arange(P) % Wo], rtol=0, atol=1e-15)


def test_decode_sentinel_rows(oracle_mod):
    h = np.random.default_rng(9).standard_normal((2, 3, 4, 4))
    valid = np.array([[1, 0, 1], [0, 0, 1]], np.uint8)
    idx, xy, score, gap = oracle_mod.peak_decode(h, valid)
    assert idx[0, 1] == -1 and idx[1, 0] == -1
    assert np.isnan(xy[0, 1]).all() and score[0, 1] == -np.inf
    assert idx[0, 0] >= 0 and np.isfinite(score[1, 2])


def test_decode_planted_peak_interior_and_border(oracle_mod):
    rng = np.random.default_rng(10)
    C, H, W = 64, 6, 7
    u = rng.standard_normal(C)
    u /= np.linalg.norm(u)
    one = np.ones((1, 1), np.uint8)
    for (i, j) in [(2, 3), (0, 4), (5, 0), (3, 6)]:
        F = rng.standard_normal((1, C, H, W))
        F[0, :, i, j] += 50.0 * u
        hm = oracle_mod.kernel_heatmap(F, None, None, u[None, None], one)
        idx, _, _, _ = oracle_mod.peak_decode(hm)
        y, x = divmod(int(idx[0, 0]), 4 * W)
        ys = {0} if i == 0 else ({4 * H - 2} if i == H - 1 else
                                 {4 * i + 1, 4 * i + 2})
        xs = {0} if j == 0 else ({4 * W - 2} if j == W - 1 else
                                 {4 * j + 1, 4 * j + 2})
        assert y in ys and x in xs, (i, j, y, x)


def test_round_trip_support_keypoint_to_decoded_coordinate(oracle_mod):
    """Keypoint at a cell centre -> VKP kernel -> planted query -> decode
    lands within one output cell (1/Wo) of the keypoint's -1..1 coordinate."""
    rng = np.random.default_rng(11)
    C, H, W, s = 128, 6, 8, 16.0
    i, j = 3, 2
    support = rng.standard_normal((1, C, H, W))
    kx, ky = (j + 0.5) * s, (i + 0.5) * s
    proto = oracle_mod.vkp_pool(support, np.array([[[kx, ky]]]),
                                np.ones((1, 1), np.uint8), s, 14.0)
    u = proto[0, 0] / np.linalg.norm(proto[0, 0])
    q = rng.standard_normal((1, C, H, W))
    q[0, :, i, j] += 60.0 * u
    hm = oracle_mod.kernel_heatmap(q, proto, np.ones((1, 1), np.uint8))
    _, xy, _, _ = oracle_mod.peak_decode(hm)
    nx, ny = 2 * kx / (W * s) - 1, 2 * ky / (H * s) - 1
    assert abs(abs(xy[0, 0, 0] - nx) - 1 / (4 * W)) < 1e-12
    assert abs(abs(xy[0, 0, 1] - ny) - 1 / (4 * H)) < 1e-12


# --------------------------------------------------------------------------
# VKP Gaussian pooling
# --------------------------------------------------------------------------
def test_vkp_sigma_to_zero_picks_the_cell(oracle_mod):
    rng = np.random.default_rng(12)
    S = rng.standard_normal((2, 5, 4, 6))
    kp = np.array([[[(2 + 0.5) * 16, (1 + 0.5) * 16]],
                   [[(5 + 0.5) * 16, (3 + 0.5) * 16]]])
    out = oracle_mod.vkp_pool(S, kp, np.ones((2, 1), np.uint8), 16.0, 0.01)
    np.testing.assert_array_equal(out[0, 0], S[0, :, 1, 2])
    np.testing.assert_array_equal(out[1, 0], S[1, :, 3, 5])


def test_vkp_sigma_to_infinity_is_global_mean(oracle_mod):
    rng = np.random.default_rng(13)
    S = rng.standard_normal((1, 7, 5, 5))
    out = oracle_mod.vkp_pool(S, np.array([[[10.0, 70.0]]]),
                              np.ones((1, 1), np.uint8), 16.0, 1e8)
    np.testing.assert_allclose(out[0, 0], S[0].reshape(7, -1).mean(-1),
                               rtol=0, atol=1e-12)


def test_vkp_constant_map_and_three_cell_closed_form(oracle_mod):
    S = np.full((1, 3, 4, 4), -1.75)
    out = oracle_mod.vkp_pool(S, np.array([[[21.0, 40.0]]]),
                              np.ones((1, 1), np.uint8), 16.0, 14.0)
    np.testing.assert_allclose(out[0, 0], -1.75, rtol=1e-15, atol=0)
    # 1 x 3 grid, keypoint on the centre cell: weights e^-a, 1, e^-a with
    # a = stride^2 / (2 sigma^2)
    f = np.array([[[[1.0, 2.0, 7.0]]]])
    s, sig = 16.0, 14.0
    out = oracle_mod.vkp_pool(f, np.array([[[1.5 * s, 0.5 * s]]]),
                              np.ones((1, 1), np.uint8), s, sig)
    e = math.exp(-s * s / (2 * sig * sig))
    assert abs(out[0, 0, 0] - (e * 1.0 + 2.0 + e * 7.0) / (1 + 2 * e)) < 1e-14


def test_vkp_matches_scipy_normal_pdf_weights(oracle_mod):
    from scipy.stats import norm
    rng = np.random.default_rng(14)
    B, C, H, W, R = 2, 9, 6, 5, 3
    S = rng.standard_normal((B, C, H, W))
    kp = rng.uniform(0, [W * 16, H * 16], size=(B, R, 2))
    valid = np.array([[1, 0, 1], [1, 1, 1]], np.uint8)
    out = oracle_mod.vkp_pool(S, kp, valid, 16.0, 14.0)
    cx = (np.arange(W) + 0.5) * 16
    cy = (np.arange(H) + 0.5) * 16
    for b in range(B):
        for r in range(R):
            if not valid[b, r]:
                assert np.isnan(out[b, r]).all()
                continue
            w = np.outer(norm.pdf(cy, kp[b, r, 1], 14.0),
                         norm.pdf(cx, kp[b, r, 0], 14.0))
            ref = (S[b] * w).sum((1, 2)) / w.sum()
            np.testing.assert_allclose(out[b, r], ref, rtol=1e-13, atol=1e-14)


def test_round_bf16_matches_torch_and_ties_to_even(oracle_mod):
    rng = np.random.default_rng(15)
    x = rng.standard_normal(5000).astype(np.float32).astype(np.float64) * 37
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double()
    np.testing.assert_array_equal(oracle_mod.round_bf16(x), ref.numpy())
    # halfway cases: 1 + 2^-8 -> 1 (even); 1 + 3*2^-8 -> 1 + 2^-6 (even)
    assert oracle_mod.round_bf16(1 + 2 ** -8) == 1.0
    assert oracle_mod.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6
    assert oracle_mod.round_bf16(-(1 + 2 ** -8 + 2 ** -30)) == -(1 + 2 ** -7)


def test_vkp_rounds_to_dtype(oracle_mod):
    rng = np.random.default_rng(16)
    S = rng.standard_normal((1, 40, 3, 4))
    kp = np.array([[[20.0, 30.0]]])
    one = np.ones((1, 1), np.uint8)
    d = oracle_mod.vkp_pool(S, kp, one, dtype="f64")
    np.testing.assert_array_equal(oracle_mod.vkp_pool(S, kp, one, dtype="bf16"),
                                  oracle_mod.round_bf16(d))
    np.testing.assert_array_equal(oracle_mod.vkp_pool(S, kp, one, dtype="f32"),
                                  d.astype(np.float32).astype(np.float64))


def test_round_bf16_subnormal_and_overflow_branches(oracle_mod):
    """The two range branches of the oracle's bfloat16 rounding, against
    torch's float32 -> bfloat16 cast (round to nearest even on the bit
    pattern, which covers subnormals and the overflow to infinity):
      * float32 subnormals (|v| < 2^-126, fixed quantum 2^-133 in bf16),
        including halfway cases and the round-up into the smallest normal;
      * the top binade, up to and past the largest finite bfloat16
        (2 - 2^-7) 2^127: halfway to 2^128 rounds to even, i.e. to
        infinity, and anything above it too."""
    rng = np.random.default_rng(41)
    sub_bits = rng.integers(1, 1 << 23, size=4000, dtype=np.uint32)
    sub = sub_bits.view(np.float32)
    sign = np.where(rng.random(4000) < 0.5, -1.0, 1.0).astype(np.float32)
    sub = sub * sign
    # halfway between bf16 subnormals (low 16 bits 0x8000), and the largest
    # float32 subnormals (round up to 2^-126)
    halves = (np.arange(1, 128, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    top_sub = np.array([0x007FFFFF, 0x007F8000, 0x007F7FFF], np.uint32).view(np.float32)
    top_bits = rng.integers(0x7F000000, 0x7F800000, size=4000, dtype=np.uint32)
    big = top_bits.view(np.float32)
    edge = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0x7F7F0000,
                     0x7F7E8000], np.uint32).view(np.float32)
    x32 = np.concatenate([sub, halves, -halves, top_sub, big, -big, edge, -edge])
    ref = torch.from_numpy(x32.copy()).to(torch.bfloat16).double().numpy()
    got = oracle_mod.round_bf16(x32.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    assert np.isinf(got).sum() > 0 and (np.abs(got[np.isfinite(got)]) < 2.0 ** -126).sum() > 0
    # doubles between float32 values: rounded once, from the double
    q = 2.0 ** -133
    assert oracle_mod.round_bf16(5.5 * q) == 6 * q            # tie to even (up)
    assert oracle_mod.round_bf16(4.5 * q) == 4 * q            # tie to even (down)
    assert oracle_mod.round_bf16(4.5 * q + 2.0 ** -160) == 5 * q
    assert oracle_mod.round_bf16(255.5 * 2.0 ** 120 - 2.0 ** 80) == 255 * 2.0 ** 120
    assert oracle_mod.round_bf16(255.5 * 2.0 ** 120) == np.inf
    assert oracle_mod.round_bf16(-1e300) == -np.inf
