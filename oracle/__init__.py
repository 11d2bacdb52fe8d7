"""CPU oracle for the GKDT parameter-free detection head.

TEST INFRASTRUCTURE. Only the test suite (tests/), the smoke check
(__graft_entry__.smoke) and the CPU-baseline leg of bench.py may import or
call anything in this package. The GPU library never does, and this package
never imports the GPU library.

The arithmetic lives in gko.c (plain C, double precision, compiled with
-O2 and no fast-math); this module only marshals numpy arrays through
ctypes. See gko.c for the passages each function follows and the readings
taken where the pages are silent.

Functions return float64 arrays. Rows that a mask excludes come back as NaN
(heatmaps, protos) so that any accidental use is loud.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gko.c")
_LIB_PATH = os.path.join(_HERE, "libgko.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double


def build(force: bool = True) -> str:
    """Compile gko.c into libgko.so (gcc -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC",
                        "-shared", "-Wall", "-Wno-unknown-pragmas", _SRC,
                        "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.gko_version.restype = _I
        lib.gko_max_threads.restype = _I
        lib.gko_set_threads.restype = None
        lib.gko_set_threads.argtypes = [_I]
        lib.gko_round_bf16.restype = _D
        lib.gko_round_bf16.argtypes = [_D]
        lib.gko_vkp_pool.restype = _I
        lib.gko_vkp_pool.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _D, _D,
                                     _I, _P]
        lib.gko_upsample4.restype = _I
        lib.gko_upsample4.argtypes = [_P, _I, _I, _I, _I, _P]
        lib.gko_kernel_heatmap.restype = _I
        lib.gko_kernel_heatmap.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I,
                                           _I, _I, _I, _P]
        lib.gko_roi_preprocess.restype = _I
        lib.gko_roi_preprocess.argtypes = [_P, _I, _I, _P, _I, _I, _P]
        lib.gko_roi_backproject.restype = _I
        lib.gko_roi_backproject.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P]
        lib.gko_peak_decode.restype = _I
        lib.gko_peak_decode.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _P,
                                        _P, _P]
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _u8(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.uint8)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def max_threads() -> int:
    return _load().gko_max_threads()


def set_threads(n: int) -> None:
    """OpenMP threads for the following calls (timing only)."""
    _load().gko_set_threads(int(n))


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value (ties to even)."""
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    return np.vectorize(lib.gko_round_bf16, otypes=[np.float64])(x)


_DTYPES = {"f32": 0, "bf16": 1, "f64": 2}


def vkp_pool(support, kpts, valid, stride=16.0, sigma=14.0, dtype="f64"):
    """support [B,C,H,W], kpts [B,R,2], valid [B,R] -> protos [B,R,C].

    Protos are rounded to `dtype` ('f32', 'bf16' or 'f64'); invalid rows
    are NaN."""
    lib = _load()
    s = _f64(support)
    B, C, H, W = s.shape
    k = _f64(kpts)
    R = k.shape[1]
    v = _u8(valid)
    out = np.full((B, R, C), np.nan)
    _check(lib.gko_vkp_pool(_ptr(s), _ptr(k), _ptr(v), B, C, H, W, R,
                            float(stride), float(sigma), _DTYPES[dtype],
                            _ptr(out)), "vkp_pool")
    return out


def upsample4(F, corners=False):
    """F [C,H,W] -> G [C,4H,4W] (half-pixel bilinear, edge clamp; with
    corners the align_corners=True grid)."""
    lib = _load()
    f = _f64(F)
    C, H, W = f.shape
    G = np.empty((C, 4 * H, 4 * W))
    _check(lib.gko_upsample4(_ptr(f), C, H, W, 1 if corners else 0, _ptr(G)), "upsample4")
    return G


def kernel_heatmap(query, kern_vis=None, mask_vis=None, kern_txt=None,
                   mask_txt=None, corners=False):
    """query [B,C,H,W]; kernels [B,R,C] + masks [B,R] per modality (None =
    modality absent) -> heatmaps [B,R,4H,4W], NaN where no mask is set.
    corners: upsample on the align_corners=True grid."""
    lib = _load()
    q = _f64(query)
    B, C, H, W = q.shape
    if (kern_vis is None) != (mask_vis is None) or \
       (kern_txt is None) != (mask_txt is None):
        raise ValueError("kernel and mask must be given together")
    R = (mask_vis if mask_vis is not None else mask_txt).shape[1]
    kv = None if kern_vis is None else _f64(kern_vis)
    kt = None if kern_txt is None else _f64(kern_txt)
    out = np.full((B, R, 4 * H, 4 * W), np.nan)
    _check(lib.gko_kernel_heatmap(_ptr(q), _ptr(kv), _ptr(_u8(mask_vis)),
                                  _ptr(kt), _ptr(_u8(mask_txt)), B, C, H, W,
                                  R, 1 if corners else 0, _ptr(out)), "kernel_heatmap")
    return out


def peak_decode(heat, row_valid=None, corners=False):
    """heat [B,R,Ho,Wo] -> (idx int32 [B,R], xy [B,R,2], score [B,R],
    gap [B,R]); the values are compared in float64, so pass the heatmap
    already rounded to the precision the decision is taken in. corners:
    corner-aligned -1..1 coordinates instead of cell centres."""
    lib = _load()
    h = _f64(heat)
    B, R, Ho, Wo = h.shape
    idx = np.empty((B, R), np.int32)
    xy = np.empty((B, R, 2))
    score = np.empty((B, R))
    gap = np.empty((B, R))
    _check(lib.gko_peak_decode(_ptr(h), _ptr(_u8(row_valid)), B, R, Ho, Wo,
                               1 if corners else 0, _ptr(idx), _ptr(xy), _ptr(score),
                               _ptr(gap)),
           "peak_decode")
    return idx, xy, score, gap


def _boxes(boxes):
    b = np.ascontiguousarray(boxes, dtype=np.int32)
    if b.ndim != 2 or b.shape[1] != 4:
        raise ValueError("boxes must be [B, 4]")
    return b


def roi_preprocess(image, boxes, size=384):
    """image [H, W, 3] uint8 RGB, boxes [B, 4] int (x0, y0, x1, y1) ->
    [B, 3, size, size] float64: crop, resize the longer side to `size`,
    centre-pad with the mean colour, ImageNet-normalise."""
    lib = _load()
    img = np.ascontiguousarray(image, dtype=np.uint8)
    if img.ndim != 3 or img.shape[2] != 3:
        raise ValueError("image must be [H, W, 3]")
    b = _boxes(boxes)
    out = np.empty((b.shape[0], 3, size, size), dtype=np.float64)
    _check(lib.gko_roi_preprocess(_ptr(img), img.shape[0], img.shape[1], _ptr(b),
                                  b.shape[0], size, _ptr(out)), "roi_preprocess")
    return out


def roi_backproject(xy, boxes, image_hw, size=384):
    """xy [B, R, 2] in the canvas's -1..1 frame -> image coordinates
    [B, R, 2] (continuous: pixel i covers [i, i + 1)); NaN for empty boxes."""
    lib = _load()
    x = _f64(xy)
    b = _boxes(boxes)
    if x.ndim != 3 or x.shape[2] != 2 or x.shape[0] != b.shape[0]:
        raise ValueError("xy must be [B, R, 2]")
    out = np.empty_like(x)
    _check(lib.gko_roi_backproject(_ptr(x), _ptr(b), x.shape[0], x.shape[1],
                                   int(image_hw[0]), int(image_hw[1]), size, _ptr(out)),
           "roi_backproject")
    return out


from .kg import kg_transformer  # noqa: E402  (pure NumPy, float64)
