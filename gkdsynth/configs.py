"""Named synthetic workloads and the seeded generator that builds them.

Each workload is a dict of plain numpy arrays:

  query      float32 [B, C, H, W]  query feature map (values exactly
                                   representable in bf16 when dtype is bf16)
  support    float32 [B, C, H, W]  support feature map, or None (text only)
  kpts       float32 [B, R, 2]     support keypoints (x, y) in input px
  mask_vis   uint8   [B, R]        1 = row has a visual prompt (keypoint)
  kern_txt   float32 [B, R, C]     text kernels (bf16-representable if bf16)
  mask_txt   uint8   [B, R]        1 = row has a text prompt
  mode       int8    [B]           0 visual, 1 text, 2 dual
  planted_cell  int32 [B, R, 2]    low-res flat cell index of each planted
                                   peak (-1 = none)
  planted_alpha float32 [B, R, 2]  planted amplitude (0 = none)

Rows that carry no prompt of a modality are filled with NaN in that
modality's arrays (kernels, keypoints), so any read of a masked row shows up
as NaN downstream.

Draw order per workload (one numpy Generator, seed fixed per workload):
  1. query noise, 2. support noise (if any visual rows), 3. the set of
  weak-peak crops (long-tail workloads), 4. per crop in order: mode, valid
  row count, alphas, then per row: keypoint, visual direction, text kernel;
  then the crop's planted cells.
"""
from __future__ import annotations

import numpy as np

STRIDE_PX = 16.0   # ViT-L/16 patch stride (384 px input -> 24x24 grid)
SIGMA_PX = 14.0    # VKP Gaussian sigma, input px (model card "Prompts")
R_PAD = 80         # prompt rows padded to 80 (model card "Model")

MODE_VIS, MODE_TXT, MODE_DUAL = 0, 1, 2

# name -> spec. seed = 20260 + index of the workload in the list below.
CONFIGS = {
    "tiny_visual": dict(index=0, B=1, C=256, H=24, W=24, dtype="f32",
                        modes="visual", rows="fixed:5", alpha="const:4"),
    "text_f32": dict(index=1, B=1, C=1024, H=24, W=24, dtype="f32",
                     modes="text", rows="fixed:20", alpha="text17x3+3x0"),
    "dual_bf16": dict(index=2, B=64, C=1024, H=24, W=24, dtype="bf16",
                      modes="dual", rows="fixed:17", alpha="uniform:1:5"),
    "longtail_bf16": dict(index=3, B=256, C=1024, H=24, W=24, dtype="bf16",
                          modes="mixed", rows="uniform:1:80",
                          alpha="longtail"),
    "highres_bf16": dict(index=4, B=128, C=1024, H=48, W=48, dtype="bf16",
                         modes="text", rows="fixed:80", alpha="two:4:3.5"),
    "longtail_dense": dict(index=5, B=256, C=1024, H=24, W=24, dtype="bf16",
                           modes="text", rows="fixed:80", alpha="longtail"),
}

SEED_BASE = 20260


def config_names():
    return list(CONFIGS)


def round_bf16_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 precision (nearest, ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    NaN stays NaN; finite inputs in the configs never overflow.
    """
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    nan = np.isnan(u.view(np.float32))
    t = u >> 16
    t &= 1
    t += 0x7FFF
    u += t          # no wrap: finite |x| <= FLT_MAX stays below 2^32
    u &= np.uint32(0xFFFF0000)
    if nan.any():
        u[nan] = np.uint32(0x7FC00000)
    return u.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The bfloat16 bit pattern (uint16) of float32 values, rounded RNE."""
    return (round_bf16_f32(x).view(np.uint32) >> 16).astype(np.uint16)


def _unit(v: np.ndarray) -> np.ndarray:
    return (v / np.linalg.norm(v.astype(np.float64))).astype(np.float32)


def _draw_cells(rng, S, W, n_single, n_pairs):
    """Distinct low-res cells: n_single singles, then n_pairs pairs whose
    members are >= 2 cells apart in Chebyshev distance."""
    perm = list(rng.permutation(S))
    singles = perm[:n_single]
    rest = perm[n_single:]
    pairs = []
    for _ in range(n_pairs):
        a = rest.pop(0)
        ai, aj = divmod(a, W)
        for k, b in enumerate(rest):
            bi, bj = divmod(b, W)
            if max(abs(ai - bi), abs(aj - bj)) >= 2:
                pairs.append((a, rest.pop(k)))
                break
        else:  # pragma: no cover - impossible at the configured sizes
            raise RuntimeError("no cell pair far enough apart")
    return singles, pairs


def make(name: str, seed: int | None = None, B: int | None = None,
         C: int | None = None, H: int | None = None, W: int | None = None,
         poison_masked: bool = True) -> dict:
    """Build the named workload. B/C/H/W may be overridden (smaller test
    variants keep the recipe); seed defaults to 20260 + workload index."""
    spec = dict(CONFIGS[name])
    for k, v in (("B", B), ("C", C), ("H", H), ("W", W)):
        if v is not None:
            spec[k] = v
    B, C, H, W = spec["B"], spec["C"], spec["H"], spec["W"]
    R, S = R_PAD, spec["H"] * spec["W"]
    if seed is None:
        seed = SEED_BASE + spec["index"]
    rng = np.random.default_rng(seed)
    bf16 = spec["dtype"] == "bf16"

    query = rng.standard_normal((B, C, H, W), dtype=np.float32)
    any_visual = spec["modes"] in ("visual", "dual", "mixed")
    support = (rng.standard_normal((B, C, H, W), dtype=np.float32)
               if any_visual else None)

    nan = np.float32(np.nan) if poison_masked else np.float32(0)
    kpts = np.full((B, R, 2), nan, np.float32)
    kern_txt = np.full((B, R, C), nan, np.float32)
    mask_vis = np.zeros((B, R), np.uint8)
    mask_txt = np.zeros((B, R), np.uint8)
    mode = np.zeros(B, np.int8)
    planted_cell = np.full((B, R, 2), -1, np.int32)
    planted_alpha = np.zeros((B, R, 2), np.float32)
    sqrtC = np.float32(np.sqrt(C))
    img_w, img_h = W * STRIDE_PX, H * STRIDE_PX

    n_weak = int(round(0.1 * B)) if spec["alpha"] == "longtail" else 0
    weak = np.zeros(B, bool)
    if n_weak:
        weak[rng.choice(B, size=n_weak, replace=False)] = True

    for b in range(B):
        m = {"visual": MODE_VIS, "text": MODE_TXT, "dual": MODE_DUAL}.get(
            spec["modes"])
        if m is None:
            m = int(rng.integers(0, 3))
        mode[b] = m
        kind, _, arg = spec["rows"].partition(":")
        if kind == "fixed":
            rv = int(arg)
        else:
            lo, hi = (int(t) for t in arg.split(":"))
            rv = int(rng.integers(lo, hi + 1))
        rv = min(rv, R)

        a = spec["alpha"]
        if a.startswith("const:"):
            alphas = np.full(rv, float(a[6:]), np.float32)
        elif a == "text17x3+3x0":
            alphas = np.array([3.0] * 17 + [0.0] * (rv - 17), np.float32)
        elif a.startswith("uniform:"):
            lo, hi = (float(t) for t in a[8:].split(":"))
            alphas = rng.uniform(lo, hi, rv).astype(np.float32)
        elif a == "longtail":
            if weak[b]:
                alphas = rng.uniform(0.0, 0.5, rv).astype(np.float32)
            else:
                alphas = rng.uniform(1.0, 5.0, rv).astype(np.float32)
        elif a.startswith("two:"):
            alphas = None
        else:  # pragma: no cover
            raise ValueError(a)

        dirs = np.zeros((rv, C), np.float32)
        for r in range(rv):
            u = None
            if m in (MODE_VIS, MODE_DUAL):
                mask_vis[b, r] = 1
                x = rng.uniform(0.0, img_w)
                y = rng.uniform(0.0, img_h)
                kpts[b, r] = (x, y)
                u = _unit(rng.standard_normal(C).astype(np.float32))
                ci, cj = int(y // STRIDE_PX), int(x // STRIDE_PX)
                ci, cj = min(ci, H - 1), min(cj, W - 1)
                i0, i1 = max(ci - 1, 0), min(ci + 2, H)
                j0, j1 = max(cj - 1, 0), min(cj + 2, W)
                support[b, :, i0:i1, j0:j1] += (sqrtC * u)[:, None, None]
            if m in (MODE_TXT, MODE_DUAL):
                mask_txt[b, r] = 1
                k = rng.standard_normal(C).astype(np.float32)
                kern_txt[b, r] = k
                ku = _unit(k)
                u = ku if u is None else _unit(u + ku)
            dirs[r] = u

        if alphas is None:  # two peaks per row
            _, pairs = _draw_cells(rng, S, W, 0, rv)
            lo_a, hi_a = (float(t) for t in spec["alpha"][4:].split(":"))
            for r, (c1, c2) in enumerate(pairs):
                planted_cell[b, r] = (c1, c2)
                planted_alpha[b, r] = (lo_a, hi_a)
        else:
            singles, _ = _draw_cells(rng, S, W, rv, 0)
            for r in range(rv):
                if alphas[r] > 0:
                    planted_cell[b, r, 0] = singles[r]
                    planted_alpha[b, r, 0] = alphas[r]
        for r in range(rv):
            for t in range(2):
                cell = planted_cell[b, r, t]
                if cell >= 0:
                    i, j = divmod(int(cell), W)
                    query[b, :, i, j] += planted_alpha[b, r, t] * dirs[r]

    if bf16:
        query = round_bf16_f32(query)
        if support is not None:
            support = round_bf16_f32(support)
        kern_txt = round_bf16_f32(kern_txt)

    return dict(name=name, seed=seed, B=B, C=C, H=H, W=W, R=R,
                dtype=spec["dtype"], stride=STRIDE_PX, sigma=SIGMA_PX,
                query=query, support=support, kpts=kpts, mask_vis=mask_vis,
                kern_txt=kern_txt, mask_txt=mask_txt, mode=mode,
                planted_cell=planted_cell, planted_alpha=planted_alpha)
