"""GPU parity of the ROI stage: gkd_roi_preprocess and gkd_roi_backproject
(HIP, through the C ABI) against the CPU oracle on the same seeded inputs.

Tolerances, from the arithmetic:
  * float32 canvas: the bilinear value of 8-bit samples carries at most a
    few roundings of 255 * 2^-24 (the tap fractions are exact integer
    ratios rounded once), and the normalisation one fma with rounded
    constants; both stay below 2e-6 in normalised units, so 1e-5 is used;
  * bfloat16 canvas: the kernel rounds its float32 value, the oracle its
    double value, to nearest even; two roundings to nearest differ by at
    most the distance of what they round plus one bfloat16 ulp, so the
    float32 bound plus one ulp is allowed (near zero, where the
    normalisation cancels, the float32 error spans many bfloat16 ulps);
  * back-projection: float32 image coordinates below 2^11 px carry a few
    ulps of 2^-13 px, so 1e-3 px is used.
"""
import numpy as np
import pytest
import torch

import gkdsynth
from parity_util import dev_tensor

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_PX = 1e-3


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


def bf16_ulp(x):
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


EDGE_BOXES = [
    (0, 0, 500, 300),      # the whole image (downscale, wide)
    (33, 38, 241, 300),    # tall
    (100, 20, 400, 60),    # very wide
    (7, 9, 8, 10),         # one pixel
    (10, 10, 12, 13),      # 2 x 3 (large upscale)
    (450, 250, 700, 500),  # past the bottom-right border: clamped
    (-50, -20, 40, 90),    # past the top-left border: clamped
    (600, 10, 700, 50),    # entirely outside: empty
    (40, 40, 40, 80),      # zero width: empty
    (90, 90, 30, 30),      # inverted: empty
    (0, 0, 384, 300),      # longer side already 384 (unresampled rows)
    (123, 45, 310, 232),   # square
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("size", [384, 97, 64])
def test_roi_preprocess_matches_oracle(gkd, ora, dtype, size):
    rng = np.random.default_rng(size)
    img = rng.integers(0, 256, (300, 500, 3)).astype(np.uint8)
    boxes = np.array(EDGE_BOXES, np.int32)
    print(f"[roi] preprocess {dtype} size={size}", flush=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    got = gkd.roi_preprocess(dev_tensor(img), dev_tensor(boxes), size=size, dtype=tdt)
    torch.cuda.synchronize()
    want = ora.roi_preprocess(img, boxes, size=size)
    g = got.float().cpu().numpy().astype(np.float64)
    if dtype == "f32":
        err = np.abs(g - want)
        assert err.max() <= TOL_F32, (err.max(), np.unravel_index(err.argmax(), err.shape))
    else:
        w16 = ora.round_bf16(want)
        err = np.abs(g - w16)
        assert np.all(err <= bf16_ulp(w16) + TOL_F32), err.max()
        assert np.mean(g == w16) > 0.99


def test_roi_preprocess_bf16_both_forms(gkd, ora):
    """bfloat16 canvases up to 2048 wide take the separable kernel, wider ones
    the direct kernel; both against the oracle, with the size-384 edge boxes
    (up- and downscaled, clamped, one-pixel and empty)."""
    rng = np.random.default_rng(21)
    img = rng.integers(0, 256, (300, 500, 3)).astype(np.uint8)
    boxes = np.array([EDGE_BOXES[i] for i in (0, 1, 4, 5, 7)], np.int32)
    for size in (2048, 2050):
        print(f"[roi] bf16 size={size}", flush=True)
        got = gkd.roi_preprocess(dev_tensor(img), dev_tensor(boxes), size=size, dtype=torch.bfloat16)
        torch.cuda.synchronize()
        want = ora.roi_preprocess(img, boxes, size=size)
        g = got.float().cpu().numpy().astype(np.float64)
        w16 = ora.round_bf16(want)
        assert np.all(np.abs(g - w16) <= bf16_ulp(w16) + TOL_F32), size
        assert np.mean(g == w16) > 0.99, size
        del got, g, want, w16


def test_roi_preprocess_full_workload_sampled(gkd, ora):
    """256 detector boxes on a 1920x1080 image, launched as the benchmark
    launches them; the oracle recomputes 12 sampled boxes."""
    d = gkdsynth.make_roi()
    print("[roi] full workload", flush=True)
    img, boxes = dev_tensor(d["image"]), dev_tensor(d["boxes"])
    for tdt in (torch.float32, torch.bfloat16):
        got = gkd.roi_preprocess(img, boxes, size=d["size"], dtype=tdt)
        torch.cuda.synchronize()
        pick = np.random.default_rng(7).choice(d["B"], 12, replace=False)
        want = ora.roi_preprocess(d["image"], d["boxes"][pick], size=d["size"])
        g = got[torch.from_numpy(pick).cuda()].float().cpu().numpy().astype(np.float64)
        if tdt == torch.float32:
            assert np.abs(g - want).max() <= TOL_F32
        else:
            w16 = ora.round_bf16(want)
            assert np.all(np.abs(g - w16) <= bf16_ulp(w16) + TOL_F32)


def test_roi_preprocess_writes_every_value_once(gkd):
    """Every canvas value is written (a sentinel fill disappears), also for
    empty boxes and sizes that are not a multiple of 4."""
    rng = np.random.default_rng(11)
    img = rng.integers(0, 256, (40, 50, 3)).astype(np.uint8)
    boxes = np.array([(0, 0, 50, 40), (60, 0, 70, 10), (3, 3, 9, 30)], np.int32)
    for size in (30, 31):
        for dt in (torch.float32, torch.bfloat16):
            out = torch.full((3, 3, size, size), float("nan"), device="cuda", dtype=dt)
            gkd.roi_preprocess(dev_tensor(img), dev_tensor(boxes), size=size, dtype=dt, out=out)
            torch.cuda.synchronize()
            assert not torch.isnan(out).any(), (size, dt)


def test_roi_backproject_matches_oracle(gkd, ora):
    d = gkdsynth.make_roi(seed=3, B=64, R=40)
    boxes = d["boxes"].copy()
    boxes[5] = (10, 10, 10, 20)   # empty: NaN out
    print("[roi] backproject", flush=True)
    got = gkd.roi_backproject(dev_tensor(d["xy"]), dev_tensor(boxes), (d["H"], d["W"]),
                              size=d["size"])
    torch.cuda.synchronize()
    want = ora.roi_backproject(d["xy"].astype(np.float64), boxes, (d["H"], d["W"]),
                               size=d["size"])
    g = got.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(g), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.abs(g[ok] - want[ok]).max() <= TOL_PX
    assert np.all(np.isnan(g[5]))
