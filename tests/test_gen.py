"""The seeded workload generator: determinism, shapes and the recipe."""
import numpy as np
import pytest
import torch

import gkdsynth
from gkdsynth import make, round_bf16_f32


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(20000).astype(np.float32)
    x = np.concatenate([x * 1e3, x * 1e-30, [0.0, -0.0, 3.0e38]]).astype(
        np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(round_bf16_f32(x), ref)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(gkdsynth.bf16_bits(x), bits.view(np.uint16))


@pytest.mark.parametrize("name", ["tiny_visual", "text_f32"])
def test_deterministic_and_shapes(name):
    a, b = make(name), make(name)
    for k in ("query", "kpts", "kern_txt", "mask_vis", "mask_txt"):
        np.testing.assert_array_equal(a[k], b[k])
    B, C, H, W, R = a["B"], a["C"], a["H"], a["W"], a["R"]
    assert a["query"].shape == (B, C, H, W) and a["query"].dtype == np.float32
    assert a["kern_txt"].shape == (B, R, C) and R == 80
    c = make(name, seed=a["seed"] + 1)
    assert not np.array_equal(a["query"], c["query"])


def test_tiny_visual_recipe():
    d = make("tiny_visual")
    assert d["mask_vis"].sum() == 5 and d["mask_txt"].sum() == 0
    assert np.all(d["mask_vis"][0, :5] == 1)
    k = d["kpts"][0, :5]
    assert np.all((k >= 0) & (k < 24 * 16))
    assert np.isnan(d["kpts"][0, 5:]).all()          # masked rows poisoned
    assert np.isnan(d["kern_txt"]).all()
    assert d["support"].shape == d["query"].shape
    assert np.all(d["planted_alpha"][0, :5, 0] == 4.0)
    cells = d["planted_cell"][0, :5, 0]
    assert len(set(cells.tolist())) == 5


def test_text_f32_recipe():
    d = make("text_f32")
    assert d["mask_txt"][0, :20].all() and d["mask_txt"][0, 20:].sum() == 0
    assert np.all(d["planted_alpha"][0, :17, 0] == 3.0)
    assert np.all(d["planted_cell"][0, 17:20] == -1)
    assert d["support"] is None


def test_dual_bf16_reduced_is_bf16_representable():
    d = make("dual_bf16", B=3)
    for k in ("query", "support"):
        assert np.array_equal(round_bf16_f32(d[k]), d[k])
    kt = d["kern_txt"][d["mask_txt"] > 0]
    assert np.array_equal(round_bf16_f32(kt), kt)
    assert np.all(d["mask_vis"][:, :17] == 1) and np.all(d["mask_txt"][:, :17])
    a = d["planted_alpha"][:, :17, 0]
    assert np.all((a >= 1) & (a <= 5))


def test_visual_direction_is_planted_in_support():
    """The 3x3 support fibres around a keypoint share the row's direction;
    the same direction is planted in the query at the planted cell."""
    d = make("tiny_visual")
    for r in range(5):
        x, y = d["kpts"][0, r]
        i, j = int(y // 16), int(x // 16)
        blk = d["support"][0, :, max(i - 1, 0):i + 2, max(j - 1, 0):j + 2]
        m = blk.reshape(d["C"], -1).mean(1).astype(np.float64)
        u = m / np.linalg.norm(m)
        qi, qj = divmod(int(d["planted_cell"][0, r, 0]), d["W"])
        proj = d["query"][0, :, qi, qj].astype(np.float64) @ u
        assert proj > 2.0, (r, proj)      # ~0.95 * alpha = 3.8 +- 1


def test_longtail_full_recipe():
    d = make("longtail_bf16")
    assert d["B"] == 256 and d["query"].shape == (256, 1024, 24, 24)
    valid = (d["mask_vis"] | d["mask_txt"]) > 0
    rv = valid.sum(1)
    assert rv.min() >= 1 and rv.max() <= 80
    assert np.all(valid[np.arange(80)[None, :] < rv[:, None]])  # leading rows
    counts = np.bincount(d["mode"], minlength=3)
    assert counts.min() > 256 / 3 * 0.7
    vis = d["mode"] == 0
    assert d["mask_txt"][vis].sum() == 0 and d["mask_vis"][d["mode"] == 1].sum() == 0
    weak = (d["planted_alpha"][:, 0, 0] < 0.5) & valid[:, 0]
    assert weak.sum() == round(0.1 * 256)


def test_highres_pairs_far_apart():
    d = make("highres_bf16", B=2)
    W = d["W"]
    assert d["H"] == 48 and W == 48
    for b in range(2):
        cells = d["planted_cell"][b].reshape(-1)
        assert len(set(cells.tolist())) == 160
        for c1, c2 in d["planted_cell"][b]:
            (i1, j1), (i2, j2) = divmod(int(c1), W), divmod(int(c2), W)
            assert max(abs(i1 - i2), abs(j1 - j2)) >= 2
        assert np.all(d["planted_alpha"][b] == [4.0, 3.5])
