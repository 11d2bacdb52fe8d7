"""Benchmark of the GKDT detection head on one MI355X.

One step = one pass of the whole hot path over one batch: Gaussian-pooled
visual prototypes (gkd_vkp_pool) for the crops with a visual prompt, then
the kernel heatmaps with the fused peak decode (gkd_kernel_heatmap) for
every crop. Default workload: the long-tail batch (B=256 crops, C=1024
bfloat16 features at 24x24 -> 96x96 heatmaps, rows padded to 80 with
U{1..80} valid rows, prompt mode drawn per crop from visual/text/dual),
synthetic and seeded. Inputs are resident in HBM before timing starts.

Prints one JSON line. `value` is heatmaps/s over the whole step (a heatmap
is one valid (crop, row) map written and decoded). `roofline` rates the
dominant kernel (gkd_kernel_heatmap) by its algorithmic bytes over its
average duration, timed with events on the stream it runs on.
`cpu_baseline` times the CPU oracle on a bounded sample of the same
workload on this host.

The headline steps run back to back (steady state: each step's VKP starts
behind the previous call's heatmap write stream). The heatmap call is also
timed alone with a 1 GiB buffer write between calls (`cold`: nothing of
the inputs is left in L2 or the memory-side cache), median/p10/p90 of 50.

  python bench.py [--steps K] [--warmup W] [--gpus 1]
  python bench.py --copy-only      # plain copy kernel of known size, for
                                   # scaling rocprofv3 byte counters
  python bench.py --no-modes       # headline only (profiling runs)
  python bench.py --roi-only       # the ROI stage only (profiling runs)
  python bench.py --kg-only        # the KG transformer only (profiling runs)
  python bench.py --workload dual_bf16 --no-modes   # one config's call
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "heatmaps/sec (96×96, C=1024, K=80, B=256) + % of HBM roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "heatmap_bf16_longtail_traffic.txt")
CSRC = os.path.join(ROOT, "prompt_conditioned_keypoint_amd", "csrc")
# sources of the heatmap call's kernels (the counters are void once they change)
HEATMAP_SRCS = [os.path.join(CSRC, n) for n in
                ("heatmap.hip", "heatmap_stream.hip", "gkd_device.hpp", "launch.hpp")]


class TimingEvent:
    """A HIP timing event recorded on torch's current stream, created with
    hipEventDisableSystemFence: recording it writes a timestamp without the
    system-scope release (cache write-back) of a default event, which would
    otherwise add to every step it brackets. Read with hipEventElapsedTime."""
    _hip = None

    def __init__(self, torch):
        import ctypes
        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._ct = ctypes
        self._torch = torch
        self.h = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.h),
                                                     ctypes.c_uint(0x20000000))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        stream = self._ct.c_void_p(self._torch.cuda.current_stream().cuda_stream)
        rc = TimingEvent._hip.hipEventRecord(self.h, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        ms = self._ct.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if TimingEvent._hip is not None and self.h:
            TimingEvent._hip.hipEventDestroy(self.h)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(d):
    """Bytes the heatmap call must move, and those of the VKP call."""
    B, C, H, W, R = d["B"], d["C"], d["H"], d["W"], d["R"]
    S = H * W
    e = 2 if d["dtype"] == "bf16" else 4
    mv, mt = d["mask_vis"] > 0, d["mask_txt"] > 0
    rv = (mv | mt).sum()
    rk = mv.sum() + mt.sum()
    heat = B * C * S * e + rk * C * e + 2 * B * R + rv * 16 * S * 4 + 16 * rv
    vis_crops = mv.any(1).sum()
    vkp = vis_crops * C * S * e + B * R * (8 + 1) + mv.sum() * C * e
    return int(heat), int(vkp), int(rv)


def src_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """Measured HBM bytes per heatmap launch from the committed rocprofv3
    counter summary, or None if it was taken on another kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("heatmap_src_sha256_16") != src_hash(HEATMAP_SRCS):
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_bandwidth(torch, nbytes=1 << 30, iters=10):
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / iters
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def host_cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(d, gpu_protos, target_s=20.0, max_crops=None):
    """Time the oracle on the first crops of the workload until ~target_s of
    CPU work: VKP (the oracle's own prototypes, compared with the GPU's),
    then the heatmaps from the GPU's prototypes (the kernels the timed GPU
    call used, so the heatmap stage compares like with like; its cost does
    not depend on the kernel values). Returns rows/s of the two stages
    together, the sample, and the oracle's prototypes and heatmaps."""
    import oracle
    rows = crops = 0
    t_vkp = t_heat = 0.0
    heat, protos = {}, {}
    max_crops = d["B"] if max_crops is None else max_crops
    while crops < min(max_crops, d["B"]) and t_vkp + t_heat < target_s:
        b = crops
        sl = slice(b, b + 1)
        mv, mt = d["mask_vis"][sl], d["mask_txt"][sl]
        t0 = time.perf_counter()
        if mv.any():
            protos[b] = oracle.vkp_pool(d["support"][sl], d["kpts"][sl], mv, d["stride"],
                                        d["sigma"], dtype=d["dtype"])
        t1 = time.perf_counter()
        kv = np.nan_to_num(gpu_protos[sl]) if mv.any() else None
        heat[b] = oracle.kernel_heatmap(d["query"][sl], kv, mv if mv.any() else None,
                                        d["kern_txt"][sl] if mt.any() else None,
                                        mt if mt.any() else None)
        t2 = time.perf_counter()
        t_vkp += t1 - t0
        t_heat += t2 - t1
        rows += int(((mv | mt) > 0).sum())
        crops += 1
    dt = t_vkp + t_heat
    # and one crop on one host thread
    nthreads = oracle.max_threads()
    oracle.set_threads(1)
    t1 = time.perf_counter()
    mv, mt = d["mask_vis"][:1], d["mask_txt"][:1]
    kv = (oracle.vkp_pool(d["support"][:1], d["kpts"][:1], mv, d["stride"], d["sigma"],
                          dtype=d["dtype"]) if mv.any() else None)
    oracle.kernel_heatmap(d["query"][:1], kv, mv if mv.any() else None,
                          d["kern_txt"][:1] if mt.any() else None, mt if mt.any() else None)
    one = time.perf_counter() - t1
    oracle.set_threads(nthreads)
    return rows / dt, dict(crops=crops, rows=rows, seconds=dt, vkp_s=t_vkp, heat_s=t_heat,
                           one_crop_1thread_s=one,
                           one_crop_rows=int(((mv | mt) > 0).sum())), heat, protos


GAP_TOL = 1e-3  # the argmax contract: bit-exact where the oracle's top-2 gap exceeds it


def check_parity(d, heat_gpu, idx_gpu, ora_heat, protos_gpu=None, ora_protos=None):
    """Compare the timed GPU outputs with the oracle on the sampled crops.
    The oracle's heatmaps were computed from the same kernels as the GPU's
    (its prototypes included), so the contract applies as it stands:
    heatmaps within 2e-2 of the row maximum (bf16 features; 1e-4 absolute
    for float32), and the index bit-exact wherever the oracle's top-2 gap
    exceeds 1e-3, else on a cell within 1e-3 of the maximum; a row that
    meets neither counts as a mismatch. The prototypes are compared with
    the oracle's own within one bf16 ulp (plus 1e-5 max |support|)."""
    import oracle
    worst = worst_abs_scaled = 0.0
    exact = near = bad = 0
    scale = np.sqrt(d["C"])
    for b, oh in ora_heat.items():
        valid = ((d["mask_vis"][b] | d["mask_txt"][b]) > 0)
        g = heat_gpu[b]
        fmax = np.abs(d["query"][b]).max()
        _, _, _, gap = oracle.peak_decode(np.nan_to_num(oh), valid[None].astype(np.uint8))
        o_idx, _, _, _ = oracle.peak_decode(oh.astype(np.float32).astype(np.float64),
                                            valid[None].astype(np.uint8))
        for r in np.nonzero(valid)[0]:
            o = oh[0, r]
            dif = np.abs(g[r].astype(np.float64) - o).max()
            worst = max(worst, dif / max(np.abs(o).max(), 1e-30))
            worst_abs_scaled = max(worst_abs_scaled, dif / (scale * fmax))
            gi = int(idx_gpu[b, r])
            if gap[0, r] > GAP_TOL:
                if gi == o_idx[0, r]:
                    exact += 1
                else:
                    bad += 1
            elif 0 <= gi < o.size and o.reshape(-1)[gi] >= o.max() - GAP_TOL:
                near += 1
            else:
                bad += 1
    rel_bar = 2e-2 if d["dtype"] == "bf16" else None
    ok = bad == 0 and (worst <= rel_bar if rel_bar else True)
    res = dict(crops=len(ora_heat), max_rel_err=float(worst),
               max_err_over_sqrtC_maxF=float(worst_abs_scaled),
               argmax_exact=exact, argmax_near_tie=near, argmax_mismatch=bad,
               gap_tol=GAP_TOL)
    if ora_protos:
        pw = 0.0
        for b, op in ora_protos.items():
            m = d["mask_vis"][b] > 0
            gp = protos_gpu[b][m].astype(np.float64)
            o = op[0][m]
            ulp = np.abs(o) * 2.0 ** -7 + 1e-5 * np.abs(d["support"][b]).max()
            pw = max(pw, float((np.abs(gp - o) / ulp).max()))
        res["protos_err_in_ulps_max"] = round(pw, 4)
        ok = ok and pw <= 1.0
    res["ok"] = bool(ok)
    return res


def timed_calls(torch, fn, n, flush=None):
    """Durations (ms) of n calls of fn, each bracketed by fence-free events on
    the current stream; with flush, flush() runs between calls, outside the
    events."""
    evs = [[TimingEvent(torch) for _ in range(2)] for _ in range(n)]
    torch.cuda.synchronize()
    for k in range(n):
        if flush is not None:
            flush()
        evs[k][0].record()
        fn()
        evs[k][1].record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def make_flush(torch, nbytes=1 << 30):
    """A 1 GiB buffer whose fill between timed calls evicts the L2s and the
    memory-side cache (256 MB on MI355X)."""
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    return lambda: buf.fill_(1.0)


def stats(ms):
    return {"mean": round(float(ms.mean()), 4), "p10_p50_p90":
            [round(float(x), 4) for x in np.percentile(ms, [10, 50, 90])]}


def roi_stage(torch, gkd, n=50, with_cpu=True):
    """The ROI stage on its own workload (256 detector boxes on a 1920x1080
    8-bit image -> [256, 3, 384, 384]): gkd_roi_preprocess in float32 and
    bfloat16, rated by its algorithmic bytes (the canvas written once, the
    image and boxes read once) over its event-timed duration, and
    gkd_roi_backproject of 80 keypoints per box."""
    import gkdsynth
    d = gkdsynth.make_roi()
    dev = "cuda"
    img = torch.from_numpy(d["image"]).to(dev)
    boxes = torch.from_numpy(d["boxes"]).to(dev)
    xy = torch.from_numpy(d["xy"]).to(dev)
    B, L = d["B"], d["size"]
    res = {"note": "ROI stage: 256 detector boxes on a 1920x1080 RGB image -> "
                   "[256,3,384,384]; not the headline",
           "workload": {"B": B, "image": [d["H"], d["W"]], "size": L}}
    for name, dt, e in (("f32", torch.float32, 4), ("bf16", torch.bfloat16, 2)):
        out = torch.empty((B, 3, L, L), dtype=dt, device=dev)
        for _ in range(5):
            gkd.roi_preprocess(img, boxes, size=L, dtype=dt, out=out)
        evs = [[TimingEvent(torch) for _ in range(2)] for _ in range(n)]
        torch.cuda.synchronize()
        for k in range(n):
            evs[k][0].record()
            gkd.roi_preprocess(img, boxes, size=L, dtype=dt, out=out)
            evs[k][1].record()
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        nbytes = B * 3 * L * L * e + d["H"] * d["W"] * 3 + B * 16
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "boxes_per_s": round(B / (ms * 1e-3), 1),
                     "alg_bytes": nbytes, "gbps": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        del out
    out = torch.empty_like(xy)
    evs = [[TimingEvent(torch) for _ in range(2)] for _ in range(n)]
    torch.cuda.synchronize()
    for k in range(n):
        evs[k][0].record()
        gkd.roi_backproject(xy, boxes, (d["H"], d["W"]), size=L, out=out)
        evs[k][1].record()
    torch.cuda.synchronize()
    res["backproject_ms"] = round(float(np.mean([a.elapsed_time(b) for a, b in evs])), 4)
    if with_cpu:
        import oracle
        k = 8
        t0 = time.perf_counter()
        oracle.roi_preprocess(d["image"], d["boxes"][:k], size=L)
        sec = time.perf_counter() - t0
        res["cpu_oracle"] = {"boxes_per_s": round(k / sec, 2), "sample": f"first {k} boxes",
                             "cores": oracle.max_threads()}
    return res


def dense_mode(torch, gkd, n=50):
    """The dense long-tail variant (same shapes, text prompts, all 80 rows
    valid: 20,480 heatmaps), the heatmap call alone (no VKP is needed),
    timed with events like the headline call."""
    import gkdsynth
    d = gkdsynth.make("longtail_dense")
    heat_bytes, _, rows = algorithmic_bytes(d)
    B, C, H, W, R = d["B"], d["C"], d["H"], d["W"], d["R"]
    dev = "cuda"
    dt = torch.bfloat16 if d["dtype"] == "bf16" else torch.float32
    q = torch.from_numpy(d["query"]).to(dev).to(dt)
    kt = torch.from_numpy(np.nan_to_num(d["kern_txt"])).to(dev).to(dt)
    mt = torch.from_numpy(d["mask_txt"]).to(dev)
    heat = torch.empty((B, R, 4 * H, 4 * W), dtype=torch.float32, device=dev)
    idx = torch.empty((B, R), dtype=torch.int32, device=dev)
    xy = torch.empty((B, R, 2), dtype=torch.float32, device=dev)
    score = torch.empty((B, R), dtype=torch.float32, device=dev)
    call = lambda: gkd.kernel_heatmap(q, None, None, kt, mt, out=heat, out_decode=(idx, xy, score))
    for _ in range(5):
        call()
    evs = [[TimingEvent(torch) for _ in range(2)] for _ in range(n)]
    torch.cuda.synchronize()
    for k in range(n):
        evs[k][0].record()
        call()
        evs[k][1].record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    gbs = heat_bytes / (ms.mean() * 1e-3) / 1e9
    return {"note": "longtail_dense: B=256, C=1024 bf16, text prompts, all 80 rows valid; "
                    "heatmap call alone; not the headline",
            "heatmaps": rows, "call_ms": round(float(ms.mean()), 4),
            "call_ms_p10_p50_p90": [round(float(x), 4) for x in np.percentile(ms, [10, 50, 90])],
            "heatmaps_per_s": round(rows / (ms.mean() * 1e-3), 1),
            "alg_bytes": heat_bytes, "gbps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def tokens_mode(torch, gkd, d, kv, mv, kt, mt, heat, dec, heat_bytes, rows, n=50):
    """The headline heatmap call with the query as the ViT's token sequence
    [B, 5 + H*W, C] (class + storage tokens first; GKD_QUERY_TOKENS), timed
    with events like the headline call (the results equal the headline's),
    and the whole step with both feature maps as tokens (wall clock)."""
    B, C, H, W = d["B"], d["C"], d["H"], d["W"]

    def as_tokens(f):
        t = np.concatenate([np.zeros((B, 5, C), np.float32),
                            f.reshape(B, C, H * W).transpose(0, 2, 1)], axis=1)
        return torch.from_numpy(np.ascontiguousarray(t)).to("cuda").to(torch.bfloat16)
    tok = as_tokens(d["query"])
    call = lambda: gkd.kernel_heatmap(tok, kv, mv, kt, mt, out=heat, out_decode=dec,
                                      token_hw=(H, W), token_skip=5)
    for _ in range(5):
        call()
    evs = [[TimingEvent(torch) for _ in range(2)] for _ in range(n)]
    torch.cuda.synchronize()
    for k in range(n):
        evs[k][0].record()
        call()
        evs[k][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    gbs = heat_bytes / (ms * 1e-3) / 1e9
    res = {"note": "headline heatmap call (and step) with the feature maps as "
                   "[B, 5 + H*W, C] tokens (GKD_QUERY_TOKENS); not the headline",
           "call_ms": round(ms, 4), "heatmaps_per_s_call": round(rows / (ms * 1e-3), 1),
           "gbps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    if kv is not None and d["support"] is not None:
        stok = as_tokens(d["support"])
        kp = torch.from_numpy(np.nan_to_num(d["kpts"])).to("cuda")

        def step():
            gkd.vkp_pool(stok, kp, mv, d["stride"], d["sigma"], out=kv, token_hw=(H, W),
                         token_skip=5)
            call()
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / n
        res["step_ms"] = round(ms_step, 4)
        res["heatmaps_per_s"] = round(rows / (ms_step * 1e-3), 1)
    return res


def kg_flops(B, C, HW, R, F, nb):
    """Flops of the kernel-generation transformer if every slot of the 2R per
    crop ran through every block (multiply-adds count 2): the padded count."""
    T, M = 2 * R, B * 2 * R
    blk = (2 * M * C * 3 * C + 4 * B * T * T * C + 2 * M * C * C      # SA
           + 2 * M * C * C + 2 * B * HW * C * 2 * C + 4 * B * T * HW * C + 2 * M * C * C  # CA
           + 4 * M * C * F)                                             # FFN
    return nb * blk


def kg_flops_prompted(mask_vis, mask_txt, C, HW, F, nb):
    """Flops of the method's own work: only the 2 n_b slots of the n_b rows
    with a prompt in crop b enter the attention and the dense layers, and
    the query's keys and values are projected for crops with such rows."""
    n = ((mask_vis > 0) | (mask_txt > 0)).sum(1).astype(np.int64)
    T = 2 * n
    M = int(T.sum())
    crops = int((n > 0).sum())
    blk = (2 * M * C * 3 * C + 4 * int((T * T).sum()) * C + 2 * M * C * C      # SA
           + 2 * M * C * C + 2 * crops * HW * C * 2 * C + 4 * M * HW * C
           + 2 * M * C * C                                                     # CA
           + 4 * M * C * F)                                                    # FFN
    return nb * blk


def kg_mode(torch, gkd, d, protos, mv, kt, mt, q, kp, rows, n=20):
    """The kernel-generation transformer (2 blocks, d_ff 1024, seeded
    synthetic weights) on the long-tail batch: the call alone (events), and
    the whole step VKP -> KG -> heatmap call with the fused decode (wall
    clock), the head taking the KG's kernels."""
    import gkdsynth
    B, C, H, W, R = d["B"], d["C"], d["H"], d["W"], d["R"]
    F, nb = 1024, 2
    wt = torch.from_numpy(gkdsynth.kg_weights(C, F, nb, seed=5)).to("cuda").to(torch.bfloat16)
    out = torch.empty((2, B, R, C), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gkd.kg_workspace_size(B, C, H, W, R, F), dtype=torch.uint8, device="cuda")
    call = lambda: gkd.kg_transformer(q, wt, kern_vis=protos, mask_vis=mv, kern_txt=kt,
                                      mask_txt=mt, n_blocks=nb, d_ff=F, out=out, workspace=ws)
    for _ in range(3):
        call()
    evs = [[TimingEvent(torch) for _ in range(2)] for _ in range(n)]
    torch.cuda.synchronize()
    for k in range(n):
        evs[k][0].record()
        call()
        evs[k][1].record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    fl = kg_flops(B, C, H * W, R, F, nb)
    flp = kg_flops_prompted(d["mask_vis"], d["mask_txt"], C, H * W, F, nb)
    res = {"note": "kernel-generation transformer with synthetic weights (perf only); "
                   "not the headline",
           "shape": {"B": B, "slots": 2 * R, "C": C, "HW": H * W, "d_ff": F, "blocks": nb,
                     "heads": C // 64,
                     "prompted_slots": int(2 * ((d["mask_vis"] | d["mask_txt"]) > 0).sum())},
           "call_ms": round(ms, 4),
           "alg_tflop": round(flp / 1e12, 4),
           "tflops": round(flp / (ms * 1e-3) / 1e12, 1),
           "mfma_frac": round(flp / (ms * 1e-3) / 1e12 / 2500.0, 4),
           "padded_tflop": round(fl / 1e12, 4),
           "padded_tflops": round(fl / (ms * 1e-3) / 1e12, 1)}
    heat = torch.empty((B, R, 4 * H, 4 * W), dtype=torch.float32, device="cuda")

    def step():
        gkd.vkp_pool(d["support_t"], kp, mv, d["stride"], d["sigma"], out=protos)
        call()
        gkd.kernel_heatmap(q, out[0], mv, out[1], mt, out=heat)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / n
    res["step_ms"] = round(ms_step, 4)
    res["heatmaps_per_s_with_kg"] = round(rows / (ms_step * 1e-3), 1)
    return res


def kg_highres_mode(torch, gkd, n=10):
    """The kernel-generation transformer on the high-resolution batch (B=128,
    80 text-prompted rows a crop, C=1024, a 48x48 query: 2304 cross-attention
    keys a crop), 2 blocks, d_ff 1024, synthetic weights: the call alone."""
    import gkdsynth
    d = gkdsynth.make("highres_bf16")
    B, C, H, W, R = d["B"], d["C"], d["H"], d["W"], d["R"]
    F, nb = 1024, 2
    q = torch.from_numpy(d["query"]).to("cuda").to(torch.bfloat16)
    kt = torch.from_numpy(np.nan_to_num(d["kern_txt"])).to("cuda").to(torch.bfloat16)
    mt = torch.from_numpy(d["mask_txt"]).to("cuda")
    wt = torch.from_numpy(gkdsynth.kg_weights(C, F, nb, seed=5)).to("cuda").to(torch.bfloat16)
    out = torch.empty((2, B, R, C), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gkd.kg_workspace_size(B, C, H, W, R, F), dtype=torch.uint8, device="cuda")
    call = lambda: gkd.kg_transformer(q, wt, kern_txt=kt, mask_txt=mt, n_blocks=nb, d_ff=F,
                                      out=out, workspace=ws)
    for _ in range(2):
        call()
    evs = [[TimingEvent(torch) for _ in range(2)] for _ in range(n)]
    torch.cuda.synchronize()
    for k in range(n):
        evs[k][0].record()
        call()
        evs[k][1].record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    flp = kg_flops_prompted(np.zeros_like(d["mask_txt"]), d["mask_txt"], C, H * W, F, nb)
    return {"note": "kernel-generation transformer on the high-resolution batch (text "
                    "prompts, 48x48 query), synthetic weights, call alone; not the headline",
            "shape": {"B": B, "slots": 2 * R, "C": C, "HW": H * W, "d_ff": F, "blocks": nb,
                      "prompted_slots": int(2 * (d["mask_txt"] > 0).sum())},
            "call_ms": round(ms, 4),
            "alg_tflop": round(flp / 1e12, 4),
            "tflops": round(flp / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flp / (ms * 1e-3) / 1e12 / 2500.0, 4)}


def config_mode(torch, gkd, name, n=50, flush=None):
    """One workload's heatmap call at its own shape, alone: warm (calls back
    to back) and cold (a 1 GiB write between calls, so no input byte is
    left in L2 or the memory-side cache), median/p10/p90 of n event-timed
    calls, rated by its algorithmic bytes; the VKP call likewise; and the
    whole step (VKP, then the call with the fused decode), wall clock."""
    import gkdsynth
    d = gkdsynth.make(name)
    heat_bytes, vkp_bytes, rows = algorithmic_bytes(d)
    B, C, H, W, R = d["B"], d["C"], d["H"], d["W"], d["R"]
    dev = "cuda"
    dt = torch.bfloat16 if d["dtype"] == "bf16" else torch.float32
    q = torch.from_numpy(d["query"]).to(dev).to(dt)
    has_vis = d["support"] is not None and d["mask_vis"].any()
    has_txt = bool(d["mask_txt"].any())
    sup = torch.from_numpy(d["support"]).to(dev).to(dt) if has_vis else None
    kp = torch.from_numpy(np.nan_to_num(d["kpts"])).to(dev)
    mv = torch.from_numpy(d["mask_vis"]).to(dev)
    mt = torch.from_numpy(d["mask_txt"]).to(dev)
    kt = torch.from_numpy(np.nan_to_num(d["kern_txt"])).to(dev).to(dt)
    protos = torch.zeros((B, R, C), dtype=dt, device=dev)
    heat = torch.empty((B, R, 4 * H, 4 * W), dtype=torch.float32, device=dev)
    dec = (torch.empty((B, R), dtype=torch.int32, device=dev),
           torch.empty((B, R, 2), dtype=torch.float32, device=dev),
           torch.empty((B, R), dtype=torch.float32, device=dev))
    vkp = lambda: gkd.vkp_pool(sup, kp, mv, d["stride"], d["sigma"], out=protos)
    call = lambda: gkd.kernel_heatmap(q, protos if has_vis else None, mv if has_vis else None,
                                      kt if has_txt else None, mt if has_txt else None,
                                      out=heat, out_decode=dec)

    def step():
        if has_vis:
            vkp()
        call()
    for _ in range(5):
        step()
    warm = timed_calls(torch, call, n)
    res = {"workload": f"{name}: B={B}, C={C} {d['dtype']}, {H}x{W} -> {4 * H}x{4 * W}, "
                       f"rows padded to {R}, {rows} valid",
           "heatmaps": rows, "alg_bytes": heat_bytes,
           "call_ms_warm": stats(warm),
           "gbps_warm": round(heat_bytes / (np.median(warm) * 1e-3) / 1e9, 1),
           "hbm_frac_warm": round(heat_bytes / (np.median(warm) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "heatmaps_per_s_call": round(rows / (np.median(warm) * 1e-3), 1)}
    if flush is not None:
        cold = timed_calls(torch, call, n, flush)
        res["call_ms_cold"] = stats(cold)
        res["gbps_cold"] = round(heat_bytes / (np.median(cold) * 1e-3) / 1e9, 1)
        res["hbm_frac_cold"] = round(heat_bytes / (np.median(cold) * 1e-3) / 1e9
                                     / HBM_PEAK_GBS, 4)
    if has_vis:
        vw = timed_calls(torch, vkp, n)
        res["vkp"] = {"alg_bytes": vkp_bytes, "ms_warm": stats(vw),
                      "hbm_frac_warm": round(vkp_bytes / (np.median(vw) * 1e-3) / 1e9
                                             / HBM_PEAK_GBS, 4)}
        if flush is not None:
            vc = timed_calls(torch, vkp, n, flush)
            res["vkp"]["ms_cold"] = stats(vc)
            res["vkp"]["hbm_frac_cold"] = round(vkp_bytes / (np.median(vc) * 1e-3) / 1e9
                                                / HBM_PEAK_GBS, 4)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / n
    res["step_ms"] = round(ms_step, 4)
    res["heatmaps_per_s_step"] = round(rows / (ms_step * 1e-3), 1)
    return res


def oracle_timing(names=("tiny_visual", "text_f32", "dual_bf16", "longtail_bf16",
                         "highres_bf16"), budget_s=4.0):
    """The oracle chain (VKP, then the heatmaps) timed on the first crops of
    each workload, all host threads, until about budget_s seconds each."""
    import gkdsynth
    import oracle
    out = {"cores": oracle.max_threads(), "cpu_model": host_cpu_model()}
    for name in names:
        d = gkdsynth.make(name)
        crops = rows = 0
        t0 = time.perf_counter()
        while crops < d["B"] and time.perf_counter() - t0 < budget_s:
            sl = slice(crops, crops + 1)
            mv, mt = d["mask_vis"][sl], d["mask_txt"][sl]
            kv = (oracle.vkp_pool(d["support"][sl], d["kpts"][sl], mv, d["stride"], d["sigma"],
                                  dtype=d["dtype"]) if mv.any() else None)
            oracle.kernel_heatmap(d["query"][sl], kv, mv if mv.any() else None,
                                  d["kern_txt"][sl] if mt.any() else None,
                                  mt if mt.any() else None)
            rows += int(((mv | mt) > 0).sum())
            crops += 1
        sec = time.perf_counter() - t0
        out[name] = {"crops": crops, "of": d["B"], "heatmaps": rows, "seconds": round(sec, 3),
                     "heatmaps_per_s": round(rows / sec, 2), "crops_per_s": round(crops / sec, 3)}
    return out


def latency_mode(torch, gkd, n=50):
    """Latency of the small single-crop configs (launch-bound): one tiny
    visual crop (C=256 float32, 5 valid rows) and one text crop (C=1024
    float32, 20 valid rows), whole step (VKP when there is a visual prompt,
    then the heatmap call with the fused decode), median of n event-timed
    runs."""
    import gkdsynth
    out = {}
    for name in ("tiny_visual", "text_f32"):
        d = gkdsynth.make(name)
        B, C, H, W, R = d["B"], d["C"], d["H"], d["W"], d["R"]
        dev = "cuda"
        q = torch.from_numpy(d["query"]).to(dev)
        mv = torch.from_numpy(d["mask_vis"]).to(dev)
        mt = torch.from_numpy(d["mask_txt"]).to(dev)
        has_vis = d["support"] is not None and d["mask_vis"].any()
        has_txt = bool(d["mask_txt"].any())
        sup = torch.from_numpy(d["support"]).to(dev) if has_vis else None
        kp = torch.from_numpy(np.nan_to_num(d["kpts"])).to(dev)
        kt = torch.from_numpy(np.nan_to_num(d["kern_txt"])).to(dev)
        protos = torch.zeros((B, R, C), device=dev)

        def step():
            if has_vis:
                gkd.vkp_pool(sup, kp, mv, d["stride"], d["sigma"], out=protos)
            gkd.kernel_heatmap(q, protos if has_vis else None, mv if has_vis else None,
                               kt if has_txt else None, mt if has_txt else None)
        for _ in range(5):
            step()
        evs = [[TimingEvent(torch) for _ in range(2)] for _ in range(n)]
        torch.cuda.synchronize()
        for k in range(n):
            evs[k][0].record()
            step()
            evs[k][1].record()
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
        out[name] = {"step_us_p10_p50_p90": [round(float(x), 1) for x in
                                              np.percentile(us, [10, 50, 90])],
                     "heatmaps": int(((d["mask_vis"] | d["mask_txt"]) > 0).sum())}
    out["note"] = "single-crop configs, launch-latency bound; not the headline"
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="longtail_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-only", action="store_true")
    ap.add_argument("--roi-only", action="store_true",
                    help="time only the ROI stage and print its JSON (profiling runs)")
    ap.add_argument("--kg-only", action="store_true",
                    help="time only the kernel-generation transformer (profiling runs)")
    ap.add_argument("--no-modes", action="store_true",
                    help="headline only: skip the secondary modes and configs (profiling runs)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache (1 GiB write between calls) timings")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the head shards over crops with no "
              "exchange, so multi-GPU runs are not part of this benchmark "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_only:
        gbs = copy_bandwidth(torch)
        print(json.dumps({"copy_bytes": 2 * (1 << 30), "copy_gbps": round(gbs, 1)}))
        return

    import gkdsynth
    import prompt_conditioned_keypoint_amd as gkd
    gkd.load()
    if args.roi_only:
        print(json.dumps(roi_stage(torch, gkd, n=args.steps, with_cpu=False)), flush=True)
        return

    log(f"[bench] generating workload {args.workload}")
    d = gkdsynth.make(args.workload)
    heat_bytes, vkp_bytes, rows = algorithmic_bytes(d)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if d["dtype"] == "bf16" else torch.float32
    B, C, H, W, R = d["B"], d["C"], d["H"], d["W"], d["R"]
    q = torch.from_numpy(d["query"]).to(dev).to(dt)
    has_vis = d["support"] is not None and d["mask_vis"].any()
    sup = torch.from_numpy(d["support"]).to(dev).to(dt) if has_vis else None
    kp = torch.from_numpy(np.nan_to_num(d["kpts"])).to(dev)
    mv = torch.from_numpy(d["mask_vis"]).to(dev)
    mt = torch.from_numpy(d["mask_txt"]).to(dev)
    kt = torch.from_numpy(np.nan_to_num(d["kern_txt"])).to(dev).to(dt)
    protos = torch.zeros((B, R, C), dtype=dt, device=dev)
    heat = torch.empty((B, R, 4 * H, 4 * W), dtype=torch.float32, device=dev)
    idx = torch.empty((B, R), dtype=torch.int32, device=dev)
    xy = torch.empty((B, R, 2), dtype=torch.float32, device=dev)
    score = torch.empty((B, R), dtype=torch.float32, device=dev)
    has_txt = bool(d["mask_txt"].any())
    torch.cuda.synchronize()

    if args.kg_only:
        if not (has_vis and has_txt and q.dtype == torch.bfloat16):
            sys.exit("--kg-only needs a bf16 workload with both prompt modalities")
        gkd.vkp_pool(sup, kp, mv, d["stride"], d["sigma"], out=protos)
        d["support_t"] = sup
        print(json.dumps(kg_mode(torch, gkd, d, protos, mv, kt, mt, q, kp, rows,
                                 n=max(3, args.steps))), flush=True)
        return

    heat16 = None  # bfloat16 heatmaps (GKD_HEATMAP_BF16), for the secondary mode

    def heatmap_call(bf16_heat=False, kp_only=False):
        if kp_only:
            gkd.kernel_heatmap(q, protos if has_vis else None, mv if has_vis else None,
                               kt if has_txt else None, mt if has_txt else None,
                               out_decode=(idx, xy, score), with_heatmaps=False)
        else:
            gkd.kernel_heatmap(q, protos if has_vis else None, mv if has_vis else None,
                               kt if has_txt else None, mt if has_txt else None,
                               out=heat16 if bf16_heat else heat, out_decode=(idx, xy, score),
                               heat_dtype=torch.bfloat16 if bf16_heat else torch.float32)

    def vkp_call():
        if has_vis:
            gkd.vkp_pool(sup, kp, mv, d["stride"], d["sigma"], out=protos)

    def step(ev=None, bf16_heat=False, kp_only=False):
        # ev: events around the heatmap call (the roofline's kernel);
        # bf16_heat / kp_only: the same step with bfloat16 heatmaps, or with
        # the keypoints only (separate passes)
        vkp_call()
        if ev is not None:
            ev[0].record()
        heatmap_call(bf16_heat, kp_only)
        if ev is not None:
            ev[1].record()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, wall clock between two synchronisations
    log(f"[bench] timing {args.steps} steps")
    # (two events per step, around the heatmap call only, on the stream it
    # is launched on; every recorded event adds a little to the step)
    evs = [[TimingEvent(torch) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    hm_all = np.array([e[0].elapsed_time(e[1]) for e in evs])
    hm_ms = float(hm_all.mean())
    # the VKP launch duration, from a separate pass (event-timed, back to back)
    vkp_all = timed_calls(torch, vkp_call, 20) if has_vis else np.zeros(1)
    vkp_ms = float(vkp_all.mean())
    # keep the outputs of the timed steps for the parity check
    heat_keep = heat.cpu().numpy() if not args.no_cpu_baseline else None
    idx_keep = idx.cpu().numpy()
    protos_keep = protos.float().cpu().numpy() if has_vis else None

    cold = None
    flush = None
    if not args.no_cold:
        log("[bench] cold-cache calls")
        flush = make_flush(torch)
        hm_cold = timed_calls(torch, lambda: heatmap_call(), 50, flush)
        cold = {"note": "the heatmap call alone with a 1 GiB buffer write between calls "
                        "(no input byte left in L2 or the memory-side cache), 50 calls",
                "call_ms": stats(hm_cold),
                "hbm_frac": round(heat_bytes / (np.median(hm_cold) * 1e-3) / 1e9
                                  / HBM_PEAK_GBS, 4)}
        if has_vis:
            vkp_cold = timed_calls(torch, vkp_call, 50, flush)
            cold["vkp_ms"] = stats(vkp_cold)
            cold["vkp_hbm_frac"] = round(vkp_bytes / (np.median(vkp_cold) * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 4)

    modes = None
    if not args.no_modes:
        # secondary modes, outside the headline: the same steps with bfloat16
        # heatmaps (half the bytes of the dominant output stream)
        heat16 = torch.empty((B, R, 4 * H, 4 * W), dtype=torch.bfloat16, device=dev)
        n16 = max(20, args.steps // 4)
        for _ in range(args.warmup):
            step(bf16_heat=True)
        ev16 = [[TimingEvent(torch) for _ in range(2)] for _ in range(n16)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(n16):
            step(ev16[k], bf16_heat=True)
        torch.cuda.synchronize()
        ms16 = (time.perf_counter() - t0) * 1e3 / n16
        hm16 = float(np.mean([e[0].elapsed_time(e[1]) for e in ev16]))
        heat16_bytes = heat_bytes - rows * 16 * H * W * 2  # 2 of the 4 bytes per heatmap value
        del heat16
        heat16 = None

        # and with the keypoints only (no heatmaps at all)
        for _ in range(args.warmup):
            step(kp_only=True)
        evk = [[TimingEvent(torch) for _ in range(2)] for _ in range(n16)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(n16):
            step(evk[k], kp_only=True)
        torch.cuda.synchronize()
        mskp = (time.perf_counter() - t0) * 1e3 / n16
        hmkp = float(np.mean([e[0].elapsed_time(e[1]) for e in evk]))
        kp_bytes = heat_bytes - rows * 16 * H * W * 4  # no heatmap bytes
        log("[bench] other configurations")
        cfgs = {}
        for name in ("dual_bf16", "highres_bf16"):
            if name != args.workload:
                cfgs[name] = config_mode(torch, gkd, name, flush=flush)
        log("[bench] ROI stage")
        roi = roi_stage(torch, gkd, with_cpu=not args.no_cpu_baseline)
        log("[bench] dense long-tail batch")
        dense = dense_mode(torch, gkd)
        log("[bench] kernel-generation transformer")
        kgr = None
        if has_vis and has_txt and q.dtype == torch.bfloat16:
            d["support_t"] = sup
            kgr = kg_mode(torch, gkd, d, protos, mv, kt, mt, q, kp, rows)
        log("[bench] kernel-generation transformer, high-resolution query")
        kgh = kg_highres_mode(torch, gkd)
        log("[bench] small-config latency")
        lat = latency_mode(torch, gkd)
        log("[bench] token-layout query")
        toks = tokens_mode(torch, gkd, d, protos if has_vis else None, mv if has_vis else None,
                           kt if has_txt else None, mt if has_txt else None, heat,
                           (idx, xy, score), heat_bytes, rows)
        modes = {
            "configs": cfgs,
            "kg_transformer": kgr,
            "kg_transformer_highres": kgh,
            "latency_small": lat,
            "query_tokens": toks,
            "longtail_dense": dense,
            "roi_stage": roi,
            "heatmap_bf16": {
                "note": "same workload, heatmaps stored as bfloat16 (GKD_HEATMAP_BF16); "
                        "not the headline",
                "steps": n16, "ms_per_step": round(ms16, 4),
                "heatmaps_per_s": round(rows / (ms16 * 1e-3), 1),
                "heatmap_call_ms": round(hm16, 4), "heatmap_call_alg_bytes": heat16_bytes,
                "heatmap_call_gbps": round(heat16_bytes / (hm16 * 1e-3) / 1e9, 1),
            },
            "keypoints_only": {
                "note": "same workload, keypoints only (heatmaps NULL); not the headline",
                "steps": n16, "ms_per_step": round(mskp, 4),
                "keypoints_per_s": round(rows / (mskp * 1e-3), 1),
                "call_ms": round(hmkp, 4), "call_alg_bytes": kp_bytes,
                "call_gbps": round(kp_bytes / (hmkp * 1e-3) / 1e9, 1),
            },
        }

    achieved = heat_bytes / (hm_ms * 1e-3) / 1e9
    copy_gbs = copy_bandwidth(torch)
    # the counter summary covers the long-tail batch only
    traffic = read_traffic() if args.workload == "longtail_bf16" else None

    cpu = None
    parity = None
    oracle_cfgs = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) on a bounded sample")
        import oracle
        rate, sample, ora_heat, ora_protos = cpu_baseline(d, protos_keep)
        cpu = {"value": round(rate, 3), "unit": "heatmaps/s",
               "cores": oracle.max_threads(), "kind": "oracle",
               "cpu_model": host_cpu_model(),
               "sample": (f"first {sample['crops']} crops of the {args.workload} batch "
                          f"({sample['rows']} heatmaps; VKP {sample['vkp_s']:.1f} s + "
                          f"heatmaps {sample['heat_s']:.1f} s)"),
               "one_crop_one_thread_s": round(sample["one_crop_1thread_s"], 3),
               "one_crop_rows": sample["one_crop_rows"]}
        # parity of the timed outputs on the sampled crops
        parity = check_parity(d, heat_keep, idx_keep, ora_heat, protos_keep, ora_protos)
        if not args.no_modes:
            log("[bench] oracle timing per configuration")
            oracle_cfgs = oracle_timing()

    value = rows / (ms_step * 1e-3)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "heatmaps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if d["dtype"] == "bf16" else "f32",
        "data": "synthetic (seeded planted-peak features and prompts)",
        "config": {"workload": f"{args.workload}: B={B} crops, C={C}, {H}x{W} -> "
                               f"{4 * H}x{4 * W} heatmaps, rows padded to {R}, "
                               f"{rows} valid rows, VKP + kernel heatmap + fused decode",
                   "B": B, "C": C, "H": H, "W": W, "R": R, "valid_rows": rows},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "keypoints_per_s": round(value, 1),
        "crops_per_s": round(B / (ms_step * 1e-3), 1),
        "timing": "steady state: steps back to back, each VKP behind the previous "
                  "call's write stream; kernel times are fence-free events around each call",
        "kernels": {
            "gkd_kernel_heatmap": {"ms": round(hm_ms, 4), "alg_bytes": heat_bytes,
                                   "gbps": round(achieved, 1),
                                   "ms_p10_p50_p90": [round(float(x), 4) for x in
                                                      np.percentile(hm_all, [10, 50, 90])]},
            "gkd_vkp_pool": {"ms": round(vkp_ms, 4), "alg_bytes": vkp_bytes,
                             "gbps": round(vkp_bytes / (vkp_ms * 1e-3) / 1e9, 1)
                             if vkp_ms > 0 else None,
                             "ms_p10_p50_p90": [round(float(x), 4) for x in
                                                np.percentile(vkp_all, [10, 50, 90])]},
        },
        "cold": cold,
        "step_hbm_frac": round((heat_bytes + vkp_bytes) / (ms_step * 1e-3) / 1e9
                               / HBM_PEAK_GBS, 4),
        "copy_gbps_measured": round(copy_gbs, 1),
        "modes": modes,
        "oracle_per_config": oracle_cfgs,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
