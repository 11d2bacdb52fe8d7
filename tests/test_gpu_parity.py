"""GPU parity: libgkdhead (HIP, through the C ABI) against the CPU oracle
on the same seeded inputs. Small workloads are compared in full; the
full-size batches run on the GPU exactly as the benchmark launches them
and the oracle recomputes sampled crops one by one.
"""
import numpy as np
import pytest
import torch

import gkdsynth
from parity_util import (check_decode, check_heatmaps, check_heatmaps_internal, check_protos,
                         dev_tensor, feat_dtype, floors_of, internal_bounds)

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0DEAD  # sentinel fill: any write shows up bitwise


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


_CACHE = {}


def workload(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _CACHE:
        _CACHE[key] = gkdsynth.make(name, **kw)
    return _CACHE[key]


def oracle_protos(ora, d, crops=None):
    crops = range(d["B"]) if crops is None else crops
    out = np.full((d["B"], d["R"], d["C"]), np.nan)
    if d["support"] is None:
        return out
    for b in crops:
        if d["mask_vis"][b].any():
            out[b:b + 1] = ora.vkp_pool(d["support"][b:b + 1], d["kpts"][b:b + 1],
                                        d["mask_vis"][b:b + 1], d["stride"], d["sigma"],
                                        dtype=d["dtype"])
    return out


def run_heatmap(gkd, d, kern_vis_np, decode=True):
    dt = feat_dtype(d)
    q = dev_tensor(d["query"], dt)
    kv = mv = kt = mt = None
    if d["mask_vis"].any():
        kv = dev_tensor(np.nan_to_num(kern_vis_np, nan=0.0).astype(np.float32), dt)
        mv = dev_tensor(d["mask_vis"])
    if d["mask_txt"].any():
        kt = dev_tensor(d["kern_txt"], dt)
        mt = dev_tensor(d["mask_txt"])
    out = sentinel((d["B"], d["R"], 4 * d["H"], 4 * d["W"]))
    res = gkd.kernel_heatmap(q, kv, mv, kt, mt, decode=decode, out=out)
    torch.cuda.synchronize()
    return res


def valid_rows(d):
    return ((d["mask_vis"] | d["mask_txt"]) > 0).astype(np.uint8)


def oracle_heat(ora, d, protos, crops):
    sl = list(crops)
    mv = d["mask_vis"][sl] if d["mask_vis"].any() else None
    mt = d["mask_txt"][sl] if d["mask_txt"].any() else None
    kv = protos[sl] if mv is not None else None
    kt = d["kern_txt"][sl] if mt is not None else None
    return ora.kernel_heatmap(d["query"][sl], kv, mv, kt, mt)


# sampled crops for the large batches: every prompt mode and extreme row count
def sample_crops(d, n):
    B = d["B"]
    rv = valid_rows(d).sum(1)
    picks = {0, B - 1, int(np.argmax(rv)), int(np.argmin(rv))}
    for m in (0, 1, 2):
        hit = np.nonzero(d["mode"] == m)[0]
        if len(hit):
            picks.add(int(hit[0]))
    rng = np.random.default_rng(99)
    while len(picks) < min(n, B):
        picks.add(int(rng.integers(0, B)))
    return sorted(picks)


CASES = [("tiny_visual", {}, None), ("text_f32", {}, None), ("dual_bf16", {}, 8),
         ("longtail_bf16", {}, 12), ("highres_bf16", {}, 6), ("longtail_dense", {}, 8)]


@pytest.mark.parametrize("name,kw,nsample", CASES, ids=[c[0] for c in CASES])
def test_vkp_pool_parity(gkd, ora, name, kw, nsample):
    d = workload(name, **kw)
    if d["support"] is None:
        pytest.skip("text-only workload")
    dt = feat_dtype(d)
    print(f"[vkp] {name} B={d['B']} C={d['C']} {d['H']}x{d['W']}", flush=True)
    out = sentinel((d["B"], d["R"], d["C"]), torch.int32)
    out = out.view(torch.float32) if dt == torch.float32 else \
        torch.empty((d["B"], d["R"], d["C"]), dtype=torch.int16, device="cuda").fill_(
            0x7FC1).view(torch.bfloat16)
    before = out.clone()
    gkd.vkp_pool(dev_tensor(d["support"], dt), dev_tensor(d["kpts"]),
                 dev_tensor(d["mask_vis"]), d["stride"], d["sigma"], out=out)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    crops = list(range(d["B"])) if nsample is None else sample_crops(d, nsample)
    o = oracle_protos(ora, d, crops)
    fmax = np.abs(d["support"][crops]).reshape(len(crops), -1).max(1)
    check_protos(g[crops], o[crops], d["mask_vis"][crops], d["dtype"], fmax)
    # rows without a keypoint are untouched, bit for bit
    inval = torch.from_numpy(d["mask_vis"] == 0).cuda()
    assert torch.equal(out[inval].view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       before[inval].view(torch.int16 if dt == torch.bfloat16 else torch.int32))


@pytest.mark.parametrize("name,kw,nsample", CASES, ids=[c[0] for c in CASES])
def test_kernel_heatmap_parity(gkd, ora, name, kw, nsample):
    """Stage parity: both sides get the same kernels (visual rows: the
    oracle's prototypes rounded to the feature dtype)."""
    d = workload(name, **kw)
    print(f"[heatmap] {name} B={d['B']} C={d['C']} {d['H']}x{d['W']}", flush=True)
    crops = list(range(d["B"])) if nsample is None else sample_crops(d, nsample)
    protos = oracle_protos(ora, d)  # all crops: every crop's kernels go to the GPU
    heat, (idx, xy, score) = run_heatmap(gkd, d, protos)
    valid = valid_rows(d)
    g = heat.cpu().numpy()
    oh = oracle_heat(ora, d, protos, crops)
    fl = floors_of(d["query"][crops])
    check_heatmaps(g[crops], oh, valid[crops], d["dtype"], fl)
    if d["dtype"] == "bf16":
        # the same bf16 values on both sides: float32-evaluation bound too
        check_heatmaps_internal(g[crops], oh, valid[crops], internal_bounds(d["query"][crops]))
    n_exact, n_near = check_decode((idx.cpu().numpy()[crops], xy.cpu().numpy()[crops],
                                    score.cpu().numpy()[crops]), oh, valid[crops],
                                   d["dtype"], floors=fl)
    assert n_exact > 0
    # rows with no prompt: heatmap untouched, decode sentinel
    gi = heat.view(torch.int32).cpu().numpy()
    assert np.all(gi[valid == 0] == NAN_BITS)
    assert np.all(idx.cpu().numpy()[valid == 0] == -1)


@pytest.mark.parametrize("name", ["longtail_bf16", "longtail_dense"])
def test_every_valid_row_finished(gkd, name):
    """Full batch, every row: whether the contraction kernel expanded a row
    itself or parked it for the expand kernel, the row ends finite
    everywhere (no parked map or tag is left behind) and its keypoint is
    set; rows with no prompt keep their bytes."""
    d = workload(name)
    protos = gkdsynth.round_bf16_f32(np.asarray(
        np.random.default_rng(6).standard_normal((d["B"], d["R"], d["C"])), np.float32))
    print(f"[finished] {name}", flush=True)
    heat, (idx, xy, score) = run_heatmap(gkd, d, protos)
    v = dev_tensor(valid_rows(d)).bool()
    rows = heat.view(d["B"], d["R"], -1)
    assert bool(torch.isfinite(rows[v]).all())
    assert bool((idx[v] >= 0).all()) and bool(torch.isfinite(score[v]).all())
    assert bool((rows.view(torch.int32)[~v] == NAN_BITS).all())


def test_fused_decode_equals_standalone_decode(gkd):
    d = workload("longtail_bf16")
    protos = np.asarray(np.random.default_rng(5).standard_normal((d["B"], d["R"], d["C"])),
                        np.float32)
    protos = gkdsynth.round_bf16_f32(protos)
    heat, (idx, xy, score) = run_heatmap(gkd, d, protos)
    v = dev_tensor(valid_rows(d))
    idx2, xy2, score2 = gkd.peak_decode(heat, v)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(score.view(torch.int32), score2.view(torch.int32))
    assert torch.equal(torch.nan_to_num(xy, 7.0), torch.nan_to_num(xy2, 7.0))


def test_peak_decode_bitexact_on_identical_input(gkd, ora):
    """Same float32 maps on both sides: index and score bit-exact, including
    exact ties (integer-valued maps) and constant maps."""
    rng = np.random.default_rng(17)
    B, R, Ho, Wo = 3, 37, 96, 96
    h = rng.standard_normal((B, R, Ho, Wo)).astype(np.float32)
    h[0] = rng.integers(0, 4, size=(R, Ho, Wo)).astype(np.float32)   # many ties
    h[1, :5] = 2.5                                                   # constant maps
    h[2, 3, -1, -1] = 1e9                                            # last cell
    valid = (rng.random((B, R)) > 0.2).astype(np.uint8)
    idx, xy, score = gkd.peak_decode(dev_tensor(h), dev_tensor(valid))
    torch.cuda.synchronize()
    o_idx, o_xy, o_score, _ = ora.peak_decode(h.astype(np.float64), valid)
    idx, xy, score = idx.cpu().numpy(), xy.cpu().numpy(), score.cpu().numpy()
    np.testing.assert_array_equal(idx, o_idx)
    m = valid > 0
    np.testing.assert_array_equal(score[m], o_score[m].astype(np.float32))
    assert np.all(score[~m] == -np.inf) and np.isnan(xy[~m]).all()
    np.testing.assert_allclose(xy[m], o_xy[m], rtol=0, atol=1e-6)
    # odd map size: scalar path
    h2 = rng.standard_normal((2, 3, 5, 7)).astype(np.float32)
    i2, _, s2 = gkd.peak_decode(dev_tensor(h2))
    torch.cuda.synchronize()
    o2 = ora.peak_decode(h2.astype(np.float64))
    np.testing.assert_array_equal(i2.cpu().numpy(), o2[0])


def test_chain_vkp_heatmap_decode(gkd, ora):
    """End to end: GPU VKP -> GPU heatmap vs the oracle's own chain."""
    d = workload("dual_bf16")
    dt = feat_dtype(d)
    crops = [0, 7, 33, 63]
    protos = gkd.vkp_pool(dev_tensor(d["support"], dt), dev_tensor(d["kpts"]),
                          dev_tensor(d["mask_vis"]))
    heat, (idx, xy, score) = gkd.kernel_heatmap(
        dev_tensor(d["query"], dt), protos, dev_tensor(d["mask_vis"]),
        dev_tensor(d["kern_txt"], dt), dev_tensor(d["mask_txt"]))
    torch.cuda.synchronize()
    o_protos = oracle_protos(ora, d, crops)
    oh = oracle_heat(ora, d, o_protos, crops)
    valid = valid_rows(d)[crops]
    g = heat.cpu().numpy()[crops]
    fl = floors_of(d["query"][crops])
    check_heatmaps(g, oh, valid, "bf16", fl)
    # prototypes may differ by one bf16 ulp, so the argmax is held to the
    # gap the heatmap error allows
    err = max(np.abs(g[b, r] - oh[b, r]).max() for b in range(len(crops))
              for r in range(d["R"]) if valid[b, r])
    check_decode((idx.cpu().numpy()[crops], xy.cpu().numpy()[crops],
                  score.cpu().numpy()[crops]), oh, valid, "bf16",
                 gap_tol=max(1e-3, 4 * err), floors=fl)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 40, 5, 7, 19), (2, 3, 1, 1, 4), (2, 72, 9, 10, 33),
                                   (5, 256, 24, 24, 80), (1, 1, 2, 3, 2), (3, 64, 8, 8, 16),
                                   (2, 96, 16, 16, 40), (9, 128, 24, 24, 37),
                                   (2, 64, 32, 32, 8), (1, 32, 2, 72, 6), (2, 64, 8, 8, 200),
                                   (3, 256, 4, 4, 12)])
def test_ragged_shapes(gkd, ora, dtype, shape):
    """Ragged channel counts, maps that do not fill a pixel chunk,
    degenerate 1x1 maps, random masks (dual, single, none). The bf16 shapes
    with C % 32 == 0 and H*W % 16 == 0 take the two-launch path
    (contraction + expand): several pixel chunks (32x32), rows wider than a
    wave (W = 72), more valid rows than one item holds (R = 200, up to four
    row blocks), idle waves, heatmap rows too short to hold a two-prompt
    row's combined kernel (4x4 maps with C = 256: combined step by step in
    the contraction); the rest take the general kernel."""
    B, C, H, W, R = shape
    rng = np.random.default_rng(B * 1000 + C + H * 10 + W + R)
    q = rng.standard_normal((B, C, H, W)).astype(np.float32)
    kv = rng.standard_normal((B, R, C)).astype(np.float32)
    kt = rng.standard_normal((B, R, C)).astype(np.float32)
    mv = (rng.random((B, R)) < 0.5).astype(np.uint8)
    mt = (rng.random((B, R)) < 0.5).astype(np.uint8)
    mv[0, 0] = mt[0, 0] = 1
    if B > 1:
        mv[1] = mt[1] = 0            # a crop with no prompt at all
    if dtype == "bf16":
        q, kv, kt = (gkdsynth.round_bf16_f32(a) for a in (q, kv, kt))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"[ragged] {dtype} {shape}", flush=True)
    out = sentinel((B, R, 4 * H, 4 * W))
    heat, (idx, xy, score) = gkd.kernel_heatmap(
        dev_tensor(q, dt), dev_tensor(kv, dt), dev_tensor(mv), dev_tensor(kt, dt),
        dev_tensor(mt), out=out)
    torch.cuda.synchronize()
    oh = ora.kernel_heatmap(q, kv, mv, kt, mt)
    valid = ((mv | mt) > 0).astype(np.uint8)
    fl = floors_of(q)
    check_heatmaps(heat.cpu().numpy(), oh, valid, dtype, fl)
    if dtype == "bf16":
        check_heatmaps_internal(heat.cpu().numpy(), oh, valid, internal_bounds(q))
    check_decode((idx.cpu().numpy(), xy.cpu().numpy(), score.cpu().numpy()), oh, valid, dtype,
                 floors=fl)
    assert np.all(heat.view(torch.int32).cpu().numpy()[valid == 0] == NAN_BITS)
    # VKP on the same shape
    kp = rng.uniform(0, [W * 16, H * 16], size=(B, R, 2)).astype(np.float32)
    pv = gkd.vkp_pool(dev_tensor(q, dt), dev_tensor(kp), dev_tensor(mv))
    torch.cuda.synchronize()
    op = ora.vkp_pool(q, kp, mv, 16.0, 14.0, dtype=dtype)
    check_protos(pv.float().cpu().numpy(), op, mv, dtype, np.abs(q).reshape(B, -1).max(1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 64, 8, 8, 16), (5, 256, 24, 24, 80), (2, 64, 8, 8, 200),
                                   (1, 32, 2, 72, 6), (3, 256, 4, 4, 12), (3, 40, 5, 7, 19),
                                   (2, 64, 32, 32, 8), (9, 128, 24, 24, 37)])
def test_keypoints_only(gkd, ora, dtype, shape):
    """Heatmaps NULL: the keypoints equal, bit for bit, those of the same
    call with heatmaps (the contraction finds the peaks itself on bf16
    features with H*W <= 576: several row blocks, W > 64, one and both
    prompts; otherwise the general kernel runs without stores), rows with no
    mask get the sentinel, and they agree with the oracle's decode (maps of
    bf16 features beyond 576 pixels decode in the general kernel, so there
    only the oracle comparison applies)."""
    B, C, H, W, R = shape
    rng = np.random.default_rng(5 * B + C + 13 * H + W + R)
    q = rng.standard_normal((B, C, H, W)).astype(np.float32)
    kv = rng.standard_normal((B, R, C)).astype(np.float32)
    kt = rng.standard_normal((B, R, C)).astype(np.float32)
    mv = (rng.random((B, R)) < 0.5).astype(np.uint8)
    mt = (rng.random((B, R)) < 0.5).astype(np.uint8)
    mv[0, 0] = mt[0, 0] = 1
    if B > 1:
        mv[1] = mt[1] = 0
    if B > 2:
        mt[2] = 0                    # a crop with one prompt only
    if dtype == "bf16":
        q, kv, kt = (gkdsynth.round_bf16_f32(a) for a in (q, kv, kt))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"[kp-only] {dtype} {shape}", flush=True)
    args = (dev_tensor(q, dt), dev_tensor(kv, dt), dev_tensor(mv), dev_tensor(kt, dt),
            dev_tensor(mt))
    heat, full = gkd.kernel_heatmap(*args, out=sentinel((B, R, 4 * H, 4 * W)))
    fill = lambda shp, dtp: sentinel(shp, dtp) if dtp == torch.int32 else sentinel(shp)
    kp = (fill((B, R), torch.int32), fill((B, R, 2), torch.float32), fill((B, R), torch.float32))
    got = gkd.kernel_heatmap(*args, out_decode=kp, with_heatmaps=False)
    torch.cuda.synchronize()
    # bf16 maps larger than one workgroup's pixel chunk (576) take the
    # streamed path with heatmaps but the general kernel without: another
    # summation order, so only the oracle comparison below applies there
    same_path = not (dtype == "bf16" and C % 32 == 0 and (H * W) % 16 == 0 and H * W > 576)
    if same_path:
        for g, f in zip(got, full):
            assert torch.equal(g.view(torch.int32), f.view(torch.int32))
    oh = ora.kernel_heatmap(q, kv, mv, kt, mt)
    valid = ((mv | mt) > 0).astype(np.uint8)
    check_decode(tuple(t.cpu().numpy() for t in got), oh, valid, dtype, floors=floors_of(q))


def test_keypoints_only_ties(gkd):
    """Keypoints only on maps with exact ties: plateaus of identical feature
    vectors (a ridge, a block, a 2x2 at a corner, one flat crop) equal the
    decode of the call with heatmaps, bit for bit. The contraction's peak
    search evaluates only the neighbourhoods of cells near the maximum and
    falls back to the full scan on flat maps; either way the first
    occurrence must win."""
    B, C, H, W, R = 4, 64, 24, 24, 16
    rng = np.random.default_rng(91)
    q = rng.standard_normal((B, C, H, W)).astype(np.float32)
    kv = rng.standard_normal((B, R, C)).astype(np.float32)
    v = rng.standard_normal(C).astype(np.float32)
    kv[:, ::2] = v                           # every other row peaks on the plateaus
    q[0, :, 7, 2:22] = v[:, None]            # a ridge of 20 cells
    q[1, :, 10:16, 3:9] = v[:, None, None]   # a 6x6 block (36 cells)
    q[2, :, 22:, 22:] = v[:, None, None]     # a 2x2 block at the corner
    q[2, :, 0, 0] = v                        # and a lone cell at the other
    q[3] = v[:, None, None]                  # flat crop: every cell ties
    mv = np.ones((B, R), np.uint8)
    mv[1, 3] = 0
    q, kv = gkdsynth.round_bf16_f32(q), gkdsynth.round_bf16_f32(kv)
    print("[kp-only] ties", flush=True)
    args = (dev_tensor(q, torch.bfloat16), dev_tensor(kv, torch.bfloat16), dev_tensor(mv))
    _, full = gkd.kernel_heatmap(*args)
    got = gkd.kernel_heatmap(*args, with_heatmaps=False)
    torch.cuda.synchronize()
    for g, f in zip(got, full):
        assert torch.equal(g.view(torch.int32), f.view(torch.int32))


def test_keypoints_only_longtail(gkd):
    """The long-tail batch, keypoints only: equal to the decode of the call
    with heatmaps, bit for bit."""
    d = workload("longtail_bf16")
    q = dev_tensor(d["query"], torch.bfloat16)
    kv = dev_tensor(np.nan_to_num(gkdsynth.round_bf16_f32(np.random.default_rng(3).standard_normal(
        (d["B"], d["R"], d["C"])).astype(np.float32))), torch.bfloat16)
    mv, mt = dev_tensor(d["mask_vis"]), dev_tensor(d["mask_txt"])
    kt = dev_tensor(np.nan_to_num(d["kern_txt"]), torch.bfloat16)
    print("[kp-only] longtail", flush=True)
    _, full = gkd.kernel_heatmap(q, kv, mv, kt, mt)
    got = gkd.kernel_heatmap(q, kv, mv, kt, mt, with_heatmaps=False)
    torch.cuda.synchronize()
    for g, f in zip(got, full):
        assert torch.equal(g.view(torch.int32), f.view(torch.int32))


BF16_SENTINEL = 0x7FC1  # bfloat16 NaN pattern no rounding produces


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 64, 8, 8, 16), (5, 256, 24, 24, 80), (2, 64, 32, 32, 8),
                                   (3, 256, 4, 4, 12), (3, 40, 5, 7, 19), (2, 64, 8, 8, 200)])
def test_bf16_heatmap_output(gkd, ora, dtype, shape):
    """GKD_HEATMAP_BF16: every valid heatmap value is the same call's float32
    value rounded to nearest even, bit for bit (streamed path, rows too short
    to park the combined kernels, several row blocks, and the general kernel
    for float32 features and odd channel counts); the fused decode is the
    float32 one; rows with no mask are not written; against the oracle within
    the bfloat16 row tolerance."""
    B, C, H, W, R = shape
    rng = np.random.default_rng(7 * B + C + 11 * H + W + R)
    q = rng.standard_normal((B, C, H, W)).astype(np.float32)
    kv = rng.standard_normal((B, R, C)).astype(np.float32)
    kt = rng.standard_normal((B, R, C)).astype(np.float32)
    mv = (rng.random((B, R)) < 0.5).astype(np.uint8)
    mt = (rng.random((B, R)) < 0.5).astype(np.uint8)
    mv[0, 0] = mt[0, 0] = 1
    if B > 1:
        mv[1] = mt[1] = 0
    if dtype == "bf16":
        q, kv, kt = (gkdsynth.round_bf16_f32(a) for a in (q, kv, kt))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"[bf16-heat] {dtype} {shape}", flush=True)
    args = (dev_tensor(q, dt), dev_tensor(kv, dt), dev_tensor(mv), dev_tensor(kt, dt),
            dev_tensor(mt))
    h32, (i32, xy32, s32) = gkd.kernel_heatmap(*args, out=sentinel((B, R, 4 * H, 4 * W)))
    out16 = torch.full((B, R, 4 * H, 4 * W), BF16_SENTINEL, dtype=torch.int16,
                       device="cuda").view(torch.bfloat16)
    h16, (i16, xy16, s16) = gkd.kernel_heatmap(*args, out=out16, heat_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert h16.dtype == torch.bfloat16 and h16.data_ptr() == out16.data_ptr()
    valid = torch.from_numpy(((mv | mt) > 0)).cuda()
    bits16 = h16.view(torch.int16)
    ref16 = h32.to(torch.bfloat16).view(torch.int16)  # torch rounds to nearest even
    assert torch.equal(bits16[valid], ref16[valid])
    assert bool((bits16[~valid] == BF16_SENTINEL).all())
    assert torch.equal(i16, i32)
    assert torch.equal(xy16.view(torch.int32), xy32.view(torch.int32))
    assert torch.equal(s16.view(torch.int32), s32.view(torch.int32))
    oh = ora.kernel_heatmap(q, kv, mv, kt, mt)
    check_heatmaps(h16.float().cpu().numpy(), oh, valid.cpu().numpy().astype(np.uint8), "bf16",
                   floors_of(q))


def test_bf16_heatmap_output_longtail(gkd):
    """The long-tail batch with bfloat16 heatmaps: equal to the float32
    heatmaps of the same call rounded to nearest even on every valid row,
    same decode."""
    d = workload("longtail_bf16")
    q = dev_tensor(d["query"], torch.bfloat16)
    kv = dev_tensor(np.nan_to_num(gkdsynth.round_bf16_f32(np.random.default_rng(3).standard_normal(
        (d["B"], d["R"], d["C"])).astype(np.float32))), torch.bfloat16)
    mv, mt = dev_tensor(d["mask_vis"]), dev_tensor(d["mask_txt"])
    kt = dev_tensor(np.nan_to_num(d["kern_txt"]), torch.bfloat16)
    B, R, H, W = d["B"], d["R"], d["H"], d["W"]
    print("[bf16-heat] longtail", flush=True)
    h32, dec32 = gkd.kernel_heatmap(q, kv, mv, kt, mt, out=sentinel((B, R, 4 * H, 4 * W)))
    out16 = torch.full((B, R, 4 * H, 4 * W), BF16_SENTINEL, dtype=torch.int16,
                       device="cuda").view(torch.bfloat16)
    h16, dec16 = gkd.kernel_heatmap(q, kv, mv, kt, mt, out=out16, heat_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    valid = (mv > 0) | (mt > 0)
    assert torch.equal(h16.view(torch.int16)[valid], h32.to(torch.bfloat16).view(torch.int16)[valid])
    assert bool((h16.view(torch.int16)[~valid] == BF16_SENTINEL).all())
    for a16, a32 in zip(dec16, dec32):
        assert torch.equal(a16.view(torch.int32), a32.view(torch.int32))


@pytest.mark.parametrize("shape,p_valid", [
    ((3, 48, 9, 8, 30), 0.6),      # H not a multiple of the row-ring depth; C < one block
    ((5, 272, 12, 8, 30), 0.6),    # H a multiple of the ring depth: the ring runs on into
                                   #   the next item (two channel blocks, the second partial)
    ((2, 32, 5, 16, 12), 0.7),     # short maps, no cross-item prefetch
    ((2, 16, 1, 8, 5), 1.0),       # a one-row map
    ((2, 144, 8, 16, 10), 0.5),    # a partial channel block (one wave of eight)
    ((1, 16, 32, 32, 6), 1.0),     # the largest map of the bf16 fast path
    ((2, 32, 8, 8, 256), 0.8),     # R = 256: up to four row blocks per crop
    ((4100, 16, 8, 8, 4), 0.5),    # more crops than one launch lists (two launches)
    ((1030, 16, 8, 8, 256), 0.1),  # four row blocks per crop: 1024 crops per launch
])
def test_vkp_bf16_fast_path_shapes(gkd, ora, shape, p_valid):
    """The persistent bf16 VKP kernel off the benchmark's shape: rings that do
    not run on into the next item, idle waves, several row blocks, crops
    without a visual prompt, and batches split over several launches."""
    B, C, H, W, R = shape
    rng = np.random.default_rng(B + C * 7 + H * 31 + W * 131 + R)
    q = gkdsynth.round_bf16_f32(rng.standard_normal((B, C, H, W)).astype(np.float32))
    mv = (rng.random((B, R)) < p_valid).astype(np.uint8)
    mv[0, 0] = 1
    if B > 1:
        mv[1] = 0                    # a crop with no visual prompt
    kp = rng.uniform(0, [W * 16, H * 16], size=(B, R, 2)).astype(np.float32)
    print(f"[vkp-fast] {shape} valid={int(mv.sum())}", flush=True)
    out = torch.empty((B, R, C), dtype=torch.int16, device="cuda").fill_(0x7FC1).view(
        torch.bfloat16)
    before = out.clone()
    gkd.vkp_pool(dev_tensor(q, torch.bfloat16), dev_tensor(kp), dev_tensor(mv), out=out)
    torch.cuda.synchronize()
    op = ora.vkp_pool(q, kp, mv, 16.0, 14.0, dtype="bf16")
    check_protos(out.float().cpu().numpy(), op, mv, "bf16", np.abs(q).reshape(B, -1).max(1))
    inval = torch.from_numpy(mv == 0).cuda()
    assert torch.equal(out[inval].view(torch.int16), before[inval].view(torch.int16))


def test_empty_batch_and_no_prompt_crops(gkd):
    q = torch.zeros((0, 64, 24, 24), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((0, 80, 64), dtype=torch.bfloat16, device="cuda")
    m = torch.zeros((0, 80), dtype=torch.uint8, device="cuda")
    heat, (idx, _, _) = gkd.kernel_heatmap(q, k, m)
    assert heat.shape == (0, 80, 96, 96) and idx.shape == (0, 80)
    # a batch whose crops carry no prompt: nothing written, sentinels only
    q = torch.randn((4, 64, 24, 24), device="cuda").to(torch.bfloat16)
    k = torch.randn((4, 80, 64), device="cuda").to(torch.bfloat16)
    m = torch.zeros((4, 80), dtype=torch.uint8, device="cuda")
    out = sentinel((4, 80, 96, 96))
    heat, (idx, xy, score) = gkd.kernel_heatmap(q, k, m, out=out)
    torch.cuda.synchronize()
    assert torch.all(heat.view(torch.int32) == NAN_BITS)
    assert torch.all(idx == -1) and torch.all(score == -float("inf"))


def test_guard_bands_untouched(gkd):
    """Outputs are written only inside their own extent."""
    d = workload("dual_bf16", B=9, C=256)
    dt = torch.bfloat16
    B, R, Ho, Wo = d["B"], d["R"], 4 * d["H"], 4 * d["W"]
    n = B * R * Ho * Wo
    pad = 1024  # 4 KiB of float32 on each side
    big = sentinel((n + 2 * pad,))
    out = big[pad:pad + n].view(B, R, Ho, Wo)
    pbig = torch.empty((B * R * 256 + 2 * pad * 2,), dtype=torch.int16,
                       device="cuda").fill_(0x7FC1)
    protos = pbig[2 * pad:2 * pad + B * R * 256].view(torch.bfloat16).view(B, R, 256)
    gkd.vkp_pool(dev_tensor(d["support"], dt), dev_tensor(d["kpts"]),
                 dev_tensor(d["mask_vis"]), out=protos)
    gkd.kernel_heatmap(dev_tensor(d["query"], dt), protos, dev_tensor(d["mask_vis"]),
                       dev_tensor(d["kern_txt"], dt), dev_tensor(d["mask_txt"]), out=out)
    torch.cuda.synchronize()
    bi = big.view(torch.int32)
    assert torch.all(bi[:pad] == NAN_BITS) and torch.all(bi[pad + n:] == NAN_BITS)
    assert torch.all(pbig[:2 * pad] == 0x7FC1) and torch.all(pbig[2 * pad + B * R * 256:] == 0x7FC1)


def test_deterministic_and_power_of_two_scaling(gkd):
    d = workload("longtail_bf16")
    dt = torch.bfloat16
    q = dev_tensor(d["query"], dt)
    kt = dev_tensor(np.nan_to_num(d["kern_txt"]), dt)
    mt = dev_tensor(d["mask_txt"])
    h1, (i1, _, s1) = gkd.kernel_heatmap(q, None, None, kt, mt)
    h2, (i2, _, s2) = gkd.kernel_heatmap(q, None, None, kt, mt)
    h3, (i3, _, s3) = gkd.kernel_heatmap(q, None, None, kt * 8, mt)   # exact in bf16
    torch.cuda.synchronize()
    v = torch.from_numpy(d["mask_txt"] > 0).cuda()
    for h in (h2, h3):
        assert torch.equal(h1[v].view(torch.int32), h[v].view(torch.int32))
    assert torch.equal(i1, i2) and torch.equal(i1, i3)
    assert torch.equal(s1.view(torch.int32), s3.view(torch.int32))


def test_planted_peaks_recovered_at_high_snr(gkd):
    """alpha = 50 planted peaks land in the planted cell's 2x2 centre."""
    rng = np.random.default_rng(23)
    B, C, H, W, R = 4, 256, 24, 24, 12
    q = rng.standard_normal((B, C, H, W)).astype(np.float32)
    k = rng.standard_normal((B, R, C)).astype(np.float32)
    cells = np.stack([rng.choice(np.arange(1, H - 1) * W + 5, R, replace=False)
                      for _ in range(B)])
    for b in range(B):
        for r in range(R):
            i, j = divmod(int(cells[b, r]), W)
            q[b, :, i, j] += 50 * k[b, r] / np.linalg.norm(k[b, r])
    q, k = gkdsynth.round_bf16_f32(q), gkdsynth.round_bf16_f32(k)
    m = np.ones((B, R), np.uint8)
    _, (idx, _, _) = gkd.kernel_heatmap(dev_tensor(q, torch.bfloat16),
                                        None, None, dev_tensor(k, torch.bfloat16),
                                        dev_tensor(m))
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for b in range(B):
        for r in range(R):
            i, j = divmod(int(cells[b, r]), W)
            y, x = divmod(int(idx[b, r]), 4 * W)
            assert y in (4 * i + 1, 4 * i + 2) and x in (4 * j + 1, 4 * j + 2)


def _corner_xy(idx, Ho, Wo):
    x, y = idx % Wo, idx // Wo
    return np.stack([2.0 * x / (Wo - 1) - 1.0, 2.0 * y / (Ho - 1) - 1.0], axis=-1)


def test_corner_coordinates(gkd, ora):
    """GKD_COORDS_CORNERS: the standalone decode matches the oracle's corner
    convention (same index, coordinates within two float32 roundings); the
    fused decode of the streamed, general and keypoints-only paths returns
    the same indices and scores as with cell centres and the corner-aligned
    coordinates of those indices."""
    rng = np.random.default_rng(17)
    h = rng.standard_normal((3, 7, 40, 24)).astype(np.float32)
    valid = (rng.random((3, 7)) < 0.7).astype(np.uint8)
    print("[corners] standalone decode", flush=True)
    idx, xy, score = gkd.peak_decode(dev_tensor(h), dev_tensor(valid), coords="corners")
    torch.cuda.synchronize()
    o_idx, o_xy, o_score, _ = ora.peak_decode(h.astype(np.float64), valid, corners=True)
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    ok = valid > 0
    assert np.abs(xy.cpu().numpy()[ok] - o_xy[ok]).max() <= 2.0 ** -23
    assert np.all(np.isnan(xy.cpu().numpy()[~ok]))
    d = workload("longtail_bf16")
    q = dev_tensor(d["query"], torch.bfloat16)
    kv = dev_tensor(np.nan_to_num(gkdsynth.round_bf16_f32(np.random.default_rng(3).standard_normal(
        (d["B"], d["R"], d["C"])).astype(np.float32))), torch.bfloat16)
    mv, mt = dev_tensor(d["mask_vis"]), dev_tensor(d["mask_txt"])
    kt = dev_tensor(np.nan_to_num(d["kern_txt"]), torch.bfloat16)
    Ho, Wo = 4 * d["H"], 4 * d["W"]
    valid = (d["mask_vis"] | d["mask_txt"]) > 0
    for kw in ({}, {"with_heatmaps": False}):
        print(f"[corners] fused {kw}", flush=True)
        a = gkd.kernel_heatmap(q, kv, mv, kt, mt, **kw)
        c = gkd.kernel_heatmap(q, kv, mv, kt, mt, coords="corners", **kw)
        torch.cuda.synchronize()
        (ia, _, sa), (ic, xc, sc) = (a if kw else a[1]), (c if kw else c[1])
        assert torch.equal(ia, ic) and torch.equal(sa.view(torch.int32), sc.view(torch.int32))
        want = _corner_xy(ic.cpu().numpy(), Ho, Wo)
        assert np.abs(xc.cpu().numpy()[valid] - want[valid]).max() <= 2.0 ** -23
    # the general kernel (float32 features)
    rng = np.random.default_rng(23)
    qf = rng.standard_normal((2, 64, 8, 8)).astype(np.float32)
    kf = rng.standard_normal((2, 5, 64)).astype(np.float32)
    m = np.ones((2, 5), np.uint8)
    print("[corners] general kernel", flush=True)
    _, (ia, _, _) = gkd.kernel_heatmap(dev_tensor(qf), dev_tensor(kf), dev_tensor(m))
    _, (ic, xc, _) = gkd.kernel_heatmap(dev_tensor(qf), dev_tensor(kf), dev_tensor(m),
                                        coords="corners")
    torch.cuda.synchronize()
    assert torch.equal(ia, ic)
    assert np.abs(xc.cpu().numpy() - _corner_xy(ic.cpu().numpy(), 32, 32)).max() <= 2.0 ** -23


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 64, 8, 8, 16), (2, 256, 24, 24, 40), (1, 64, 32, 32, 6),
                                   (3, 40, 5, 7, 9), (2, 32, 1, 8, 4), (3, 256, 4, 4, 12)])
def test_align_corners_upsample(gkd, ora, dtype, shape):
    """GKD_UPSAMPLE_CORNERS against the oracle's align_corners=True heatmaps
    (streamed path with one and several pixel chunks, general kernel, a
    one-row map, maps too small to park the combined kernels), the fused
    decode, bfloat16 heatmaps (the float32 values rounded) and keypoints
    only (the same keypoints, bit for bit, where the path is the same)."""
    B, C, H, W, R = shape
    rng = np.random.default_rng(3 * B + C + 7 * H + W + R)
    q = rng.standard_normal((B, C, H, W)).astype(np.float32)
    kv = rng.standard_normal((B, R, C)).astype(np.float32)
    kt = rng.standard_normal((B, R, C)).astype(np.float32)
    mv = (rng.random((B, R)) < 0.5).astype(np.uint8)
    mt = (rng.random((B, R)) < 0.5).astype(np.uint8)
    mv[0, 0] = mt[0, 0] = 1
    if B > 1:
        mv[1] = mt[1] = 0
    if dtype == "bf16":
        q, kv, kt = (gkdsynth.round_bf16_f32(a) for a in (q, kv, kt))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"[corners-up] {dtype} {shape}", flush=True)
    args = (dev_tensor(q, dt), dev_tensor(kv, dt), dev_tensor(mv), dev_tensor(kt, dt),
            dev_tensor(mt))
    out = sentinel((B, R, 4 * H, 4 * W))
    heat, (idx, xy, score) = gkd.kernel_heatmap(*args, out=out, align_corners=True)
    out16 = torch.empty((B, R, 4 * H, 4 * W), dtype=torch.bfloat16, device="cuda")
    h16, _ = gkd.kernel_heatmap(*args, out=out16, heat_dtype=torch.bfloat16, align_corners=True)
    kp = gkd.kernel_heatmap(*args, with_heatmaps=False, align_corners=True)
    torch.cuda.synchronize()
    oh = ora.kernel_heatmap(q, kv, mv, kt, mt, corners=True)
    valid = ((mv | mt) > 0).astype(np.uint8)
    fl = floors_of(q)
    check_heatmaps(heat.cpu().numpy(), oh, valid, dtype, fl)
    check_decode((idx.cpu().numpy(), xy.cpu().numpy(), score.cpu().numpy()), oh, valid, dtype,
                 floors=fl)
    assert np.all(heat.view(torch.int32).cpu().numpy()[valid == 0] == NAN_BITS)
    v = torch.from_numpy(valid > 0).cuda()
    assert torch.equal(h16.view(torch.int16)[v], heat.to(torch.bfloat16).view(torch.int16)[v])
    check_decode(tuple(t.cpu().numpy() for t in kp), oh, valid, dtype, floors=fl)
    same_path = not (dtype == "bf16" and C % 32 == 0 and (H * W) % 16 == 0 and H * W > 576)
    if same_path:
        for g, f in zip(kp, (idx, xy, score)):
            assert torch.equal(g.view(torch.int32), f.view(torch.int32))


def _tokens(q, skip, rng):
    """[B, C, H, W] -> the ViT's token sequence [B, skip + H*W, C] with
    random leading tokens."""
    B, C, H, W = q.shape
    t = np.empty((B, skip + H * W, C), q.dtype)
    t[:, :skip] = rng.standard_normal((B, skip, C)).astype(q.dtype) * 100
    t[:, skip:] = q.reshape(B, C, H * W).transpose(0, 2, 1)
    return np.ascontiguousarray(t)


@pytest.mark.parametrize("skip", [0, 5])
@pytest.mark.parametrize("shape", [(3, 64, 8, 8, 16), (2, 256, 24, 24, 40), (1, 64, 32, 32, 6),
                                   (3, 256, 4, 4, 12), (2, 32, 6, 8, 200), (2, 96, 8, 8, 24)])
def test_query_tokens_layout(gkd, ora, shape, skip):
    """GKD_QUERY_TOKENS: the token sequence [B, skip + H*W, C] gives, bit
    for bit, the results of the same call on [B, C, H, W] (heatmaps,
    bfloat16 heatmaps, the fused decode and keypoints only: the channel
    order of every K step and the accumulation order are the same), and
    the heatmaps match the oracle."""
    B, C, H, W, R = shape
    rng = np.random.default_rng(B + C + H + W + R + skip)
    q = gkdsynth.round_bf16_f32(rng.standard_normal((B, C, H, W)).astype(np.float32))
    kv = gkdsynth.round_bf16_f32(rng.standard_normal((B, R, C)).astype(np.float32))
    kt = gkdsynth.round_bf16_f32(rng.standard_normal((B, R, C)).astype(np.float32))
    mv = (rng.random((B, R)) < 0.5).astype(np.uint8)
    mt = (rng.random((B, R)) < 0.5).astype(np.uint8)
    mv[0, 0] = mt[0, 0] = 1
    tok = dev_tensor(_tokens(q, skip, rng), torch.bfloat16)
    bf = torch.bfloat16
    rest = (dev_tensor(kv, bf), dev_tensor(mv), dev_tensor(kt, bf), dev_tensor(mt))
    print(f"[tokens] {shape} skip={skip}", flush=True)
    for kw in ({}, {"heat_dtype": bf}):
        h0, d0 = gkd.kernel_heatmap(dev_tensor(q, bf), *rest, **kw)
        h1, d1 = gkd.kernel_heatmap(tok, *rest, token_hw=(H, W), token_skip=skip, **kw)
        torch.cuda.synchronize()
        valid = torch.from_numpy((mv | mt) > 0).cuda()
        iv = torch.int16 if kw else torch.int32
        assert torch.equal(h0.view(iv)[valid], h1.view(iv)[valid])
        for a, b in zip(d0, d1):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        if not kw:
            oh = ora.kernel_heatmap(q, kv, mv, kt, mt)
            check_heatmaps(h1.cpu().numpy(), oh, ((mv | mt) > 0).astype(np.uint8), "bf16",
                           floors_of(q))
    if H * W <= 576:
        k0 = gkd.kernel_heatmap(dev_tensor(q, bf), *rest, with_heatmaps=False)
        k1 = gkd.kernel_heatmap(tok, *rest, with_heatmaps=False, token_hw=(H, W), token_skip=skip)
        torch.cuda.synchronize()
        for a, b in zip(k0, k1):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_query_tokens_longtail(gkd):
    """The long-tail batch with the query as tokens (5 leading tokens): the
    same heatmaps and keypoints, bit for bit, as the [B, C, H, W] call."""
    d = workload("longtail_bf16")
    rng = np.random.default_rng(8)
    q = dev_tensor(d["query"], torch.bfloat16)
    tok = dev_tensor(_tokens(d["query"], 5, rng), torch.bfloat16)
    kv = dev_tensor(np.nan_to_num(gkdsynth.round_bf16_f32(np.random.default_rng(3).standard_normal(
        (d["B"], d["R"], d["C"])).astype(np.float32))), torch.bfloat16)
    mv, mt = dev_tensor(d["mask_vis"]), dev_tensor(d["mask_txt"])
    kt = dev_tensor(np.nan_to_num(d["kern_txt"]), torch.bfloat16)
    print("[tokens] longtail", flush=True)
    h0, d0 = gkd.kernel_heatmap(q, kv, mv, kt, mt)
    h1, d1 = gkd.kernel_heatmap(tok, kv, mv, kt, mt, token_hw=(d["H"], d["W"]), token_skip=5)
    torch.cuda.synchronize()
    valid = torch.from_numpy((d["mask_vis"] | d["mask_txt"]) > 0).cuda()
    assert torch.equal(h0.view(torch.int32)[valid], h1.view(torch.int32)[valid])
    for a, b in zip(d0, d1):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 64, 5, 7, 9), (3, 128, 24, 24, 80), (2, 32, 6, 8, 20),
                                   (2, 256, 32, 32, 40), (3, 64, 16, 16, 7)])
def test_support_tokens_layout(gkd, ora, dtype, shape):
    """gkd_vkp_pool with the support map as tokens [B, 5 + H*W, C]: the
    oracle's prototypes within the prototype tolerance, and bit for bit the
    channel-row call (both layouts take the same kernel: the fast separable
    one for bfloat16 maps up to 32x32 with W % 8 == 0, the general one
    otherwise, and feed its MFMAs the same values in the same order)."""
    B, C, H, W, R = shape
    rng = np.random.default_rng(B + C + H + W + R)
    s = rng.standard_normal((B, C, H, W)).astype(np.float32)
    if dtype == "bf16":
        s = gkdsynth.round_bf16_f32(s)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kp = rng.uniform(0, [W * 16, H * 16], size=(B, R, 2)).astype(np.float32)
    mv = (rng.random((B, R)) < 0.7).astype(np.uint8)
    tok = _tokens(s, 5, rng)
    print(f"[tokens-vkp] {dtype} {shape}", flush=True)
    p1 = gkd.vkp_pool(dev_tensor(tok, dt), dev_tensor(kp), dev_tensor(mv), token_hw=(H, W),
                      token_skip=5, out=torch.zeros((B, R, C), dtype=dt, device="cuda"))
    p0 = gkd.vkp_pool(dev_tensor(s, dt), dev_tensor(kp), dev_tensor(mv),
                      out=torch.zeros((B, R, C), dtype=dt, device="cuda"))
    torch.cuda.synchronize()
    op = ora.vkp_pool(s, kp, mv, 16.0, 14.0, dtype=dtype)
    check_protos(p1.float().cpu().numpy(), op, mv, dtype, np.abs(s).reshape(B, -1).max(1))
    v = torch.from_numpy(mv > 0).cuda()
    iv = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(p0.view(iv)[v], p1.view(iv)[v])
