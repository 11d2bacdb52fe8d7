"""Pins for the oracle's ROI stage (crop, resize so the longer side is the
input size, centre-pad with the mean colour, ImageNet normalisation, and
the back-projection of -1..1 keypoints into the image).

The resize is pinned to torch's bilinear interpolation (half-pixel
centres, no antialiasing) on the cropped pixels, the normalisation to
torch's batch norm in inference mode with the ImageNet statistics, the
resized sizes and pads to exact rational rounding, and the
back-projection to the forward map written in closed form. A slip in the
half-pixel offset, the pad split, the rounding of the shorter side, a
swapped axis or a channel order would fail one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

MEAN = (0.485, 0.456, 0.406)   # ImageNet statistics (published constants)
STD = (0.229, 0.224, 0.225)
PAD = (124, 116, 104)           # the card's pad colour


def torch_normalise(v):
    """[B, 3, h, w] float64 in 0..255 -> ImageNet-normalised, via torch's
    batch norm in inference mode (mean, var = std^2; eps = 1e-300 vanishes
    against var in double)."""
    x = torch.from_numpy(np.ascontiguousarray(v)) / 255.0
    m = torch.tensor(MEAN, dtype=torch.float64)
    var = torch.tensor(STD, dtype=torch.float64) ** 2
    return torch.nn.functional.batch_norm(x, m, var, training=False, eps=1e-300).numpy()


def rounded_size(side, longer, L):
    """round(side * L / longer) with halves up, in exact rationals."""
    q = Fraction(side * L, longer)
    n = int(q + Fraction(1, 2))  # floor(q + 1/2) for q >= 0
    return max(n, 1)


def geometry(box, H, W, L):
    x0, y0, x1, y1 = box
    x0, x1 = min(max(x0, 0), W), min(max(x1, 0), W)
    y0, y1 = min(max(y0, 0), H), min(max(y1, 0), H)
    bw, bh = max(x1 - x0, 0), max(y1 - y0, 0)
    if bw == 0 or bh == 0:
        return None
    lng = max(bw, bh)
    nw, nh = rounded_size(bw, lng, L), rounded_size(bh, lng, L)
    return x0, y0, bw, bh, nw, nh, (L - nw) // 2, (L - nh) // 2


def pad_value():
    return torch_normalise(np.array(PAD, dtype=np.float64).reshape(1, 3, 1, 1))[0, :, 0, 0]


BOXES = [(0, 0, 40, 30), (5, 5, 9, 7), (3, 1, 38, 29), (10, 2, 13, 29), (0, 0, 1, 1),
         (7, 4, 27, 5), (-6, -3, 12, 50), (20, 10, 21, 30)]


@pytest.mark.parametrize("L", [16, 23, 64])
def test_roi_resize_matches_torch_interpolate(oracle_mod, L):
    rng = np.random.default_rng(L)
    img = rng.integers(0, 256, (30, 40, 3)).astype(np.uint8)
    out = oracle_mod.roi_preprocess(img, BOXES, size=L)
    pv = pad_value()
    for b, box in enumerate(BOXES):
        x0, y0, bw, bh, nw, nh, px, py = geometry(box, 30, 40, L)
        crop = img[y0:y0 + bh, x0:x0 + bw].astype(np.float64).transpose(2, 0, 1)[None]
        ref = torch.nn.functional.interpolate(torch.from_numpy(crop), size=(nh, nw),
                                              mode="bilinear", align_corners=False,
                                              antialias=False).numpy()
        ref = torch_normalise(ref)[0]
        got = out[b]
        np.testing.assert_allclose(got[:, py:py + nh, px:px + nw], ref, rtol=0, atol=1e-12)
        mask = np.ones((L, L), bool)
        mask[py:py + nh, px:px + nw] = False
        for c in range(3):
            assert np.all(got[c][mask] == pv[c]) or np.allclose(got[c][mask], pv[c], atol=1e-15)


@pytest.mark.parametrize("box", [(0, 0, 100, 50), (0, 0, 50, 100), (0, 0, 99, 1), (0, 0, 1, 99),
                                 (0, 0, 3, 2), (0, 0, 2, 3), (0, 0, 7, 5), (0, 0, 384, 383),
                                 (0, 0, 1000, 999), (0, 0, 999, 1000)])
def test_roi_sizes_and_pad_split(oracle_mod, box):
    """The content rectangle (a constant white crop on the pad colour) sits
    where exact rational rounding and a floor split of the pad put it."""
    H, W = box[3], box[2]
    L = 384
    img = np.full((H, W, 3), 255, np.uint8)
    out = oracle_mod.roi_preprocess(img, [box], size=L)[0]
    white = torch_normalise(np.full((1, 3, 1, 1), 255.0))[0, :, 0, 0]
    inside = np.isclose(out[0], white[0], atol=1e-12)
    ys, xs = np.nonzero(inside)
    _, _, bw, bh, nw, nh, px, py = geometry(box, H, W, L)
    assert (ys.min(), ys.max() + 1, xs.min(), xs.max() + 1) == (py, py + nh, px, px + nw)
    assert inside.sum() == nw * nh
    assert max(nw, nh) == L


def test_roi_identity_scale_is_the_normalised_image(oracle_mod):
    """A box whose longer side already equals L is pasted unresampled."""
    rng = np.random.default_rng(1)
    img = rng.integers(0, 256, (24, 32, 3)).astype(np.uint8)
    out = oracle_mod.roi_preprocess(img, [(0, 0, 32, 24)], size=32)[0]
    ref = torch_normalise(img.astype(np.float64).transpose(2, 0, 1)[None])[0]
    np.testing.assert_allclose(out[:, 4:28, :], ref, rtol=0, atol=1e-12)
    pv = pad_value()
    assert np.allclose(out[:, :4, :], pv[:, None, None], atol=1e-15)
    assert np.allclose(out[:, 28:, :], pv[:, None, None], atol=1e-15)


def test_roi_affine_image_closed_form(oracle_mod):
    """Bilinear resampling reproduces an affine image exactly wherever no
    tap is clamped: value = a x + b y + c_k at the source position
    ((u + 1/2) bw / nw - 1/2, (v + 1/2) bh / nh - 1/2) of the crop."""
    H, W = 60, 80
    y, x = np.mgrid[0:H, 0:W]
    img = np.stack([x + 2 * y, 2 * x + y, 40 + x + y], axis=-1)
    assert img.max() <= 255
    img = img.astype(np.uint8)
    box = (6, 9, 69, 40)
    L = 50
    out = oracle_mod.roi_preprocess(img, [box], size=L)[0]
    x0, y0, bw, bh, nw, nh, px, py = geometry(box, H, W, L)
    coef = [(1, 2, 0), (2, 1, 0), (1, 1, 40)]
    checked = 0
    for v in range(nh):
        sy = Fraction(2 * v + 1, 2) * Fraction(bh, nh) - Fraction(1, 2)
        if sy < 0 or sy > bh - 1:
            continue
        for u in range(nw):
            sx = Fraction(2 * u + 1, 2) * Fraction(bw, nw) - Fraction(1, 2)
            if sx < 0 or sx > bw - 1:
                continue
            for c, (a, b_, k) in enumerate(coef):
                val = a * (x0 + sx) + b_ * (y0 + sy) + k
                want = (float(val) / 255.0 - MEAN[c]) / STD[c]
                assert abs(out[c, py + v, px + u] - want) < 1e-12
                checked += 1
    assert checked > 3 * 0.8 * nw * nh


def test_roi_2x_downscale_is_the_2x2_mean(oracle_mod):
    """Resizing by exactly 1/2 samples every output between two source
    pixels on each axis: the mean of the 2x2 block."""
    rng = np.random.default_rng(3)
    img = rng.integers(0, 256, (12, 16, 3)).astype(np.uint8)
    out = oracle_mod.roi_preprocess(img, [(0, 0, 16, 12)], size=8)[0]
    blocks = img.astype(np.float64).reshape(6, 2, 8, 2, 3).mean(axis=(1, 3))
    ref = torch_normalise(blocks.transpose(2, 0, 1)[None])[0]
    np.testing.assert_allclose(out[:, 1:7, :], ref, rtol=0, atol=1e-12)


def test_roi_clamped_empty_and_outside_boxes(oracle_mod):
    rng = np.random.default_rng(4)
    img = rng.integers(0, 256, (30, 40, 3)).astype(np.uint8)
    out = oracle_mod.roi_preprocess(img, [(-6, -3, 12, 50), (0, -3, 12, 30), (45, 0, 60, 10),
                                          (10, 10, 10, 20), (12, 5, 3, 9)], size=16)
    np.testing.assert_array_equal(out[0], out[1])  # both clamp to (0, 0, 12, 30)
    pv = pad_value()
    for b in (2, 3, 4):
        assert np.allclose(out[b], pv[:, None, None], atol=1e-15)


def test_roi_backproject_inverts_the_forward_map(oracle_mod):
    """An image point inside the box, sent to the canvas's -1..1 frame by
    the forward map in closed form, comes back to itself; box corners map
    to the content corners; empty boxes give NaN."""
    rng = np.random.default_rng(5)
    H, W, L = 300, 500, 384
    boxes = [(0, 0, 500, 300), (33, 38, 241, 310), (100, 20, 130, 290), (7, 9, 8, 10),
             (10, 10, 10, 50)]
    R = 16
    pts = np.zeros((len(boxes), R, 2))
    want = np.zeros_like(pts)
    for b, box in enumerate(boxes):
        g = geometry(box, H, W, L)
        if g is None:
            continue
        x0, y0, bw, bh, nw, nh, px, py = g
        xi = x0 + rng.random(R) * bw
        yi = y0 + rng.random(R) * bh
        xi[0], yi[0] = x0, y0                       # top-left corner
        xi[1], yi[1] = x0 + bw, y0 + bh             # bottom-right corner
        want[b, :, 0], want[b, :, 1] = xi, yi
        xc = px + (xi - x0) * nw / bw
        yc = py + (yi - y0) * nh / bh
        pts[b, :, 0], pts[b, :, 1] = 2 * xc / L - 1, 2 * yc / L - 1
        assert pts[b, 0, 0] == 2 * px / L - 1 and pts[b, 1, 1] == 2 * (py + nh) / L - 1
    got = oracle_mod.roi_backproject(pts, boxes, (H, W), size=L)
    np.testing.assert_allclose(got[:4], want[:4], rtol=0, atol=1e-9)
    assert np.all(np.isnan(got[4]))
    # the box clamps first: (33, 38, 241, 310) is (33, 38, 241, 300) in a 300-row image
    c = oracle_mod.roi_backproject(pts[1:2], [(33, 38, 241, 300)], (H, W), size=L)
    np.testing.assert_array_equal(c, got[1:2])
