"""ctypes binding of libgkdhead (the GKDT detection head on gfx950).

Argument marshalling only: shape/dtype/device checks, output allocation
with torch, and the call through the C ABI declared in include/gkdhead.h.
Every step of the computation runs in the library's HIP kernels. There is
no fallback: if libgkdhead.so is missing or a call fails, this module
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgkdhead.so")

GKD_DTYPE_F32, GKD_DTYPE_BF16 = 0, 1
GKD_ABI_VERSION = 9          # include/gkdhead.h
GKD_KG_STATIC_WORKSPACE_BYTES = 64 << 20  # the no-allocation KG call's static workspace
GKD_HEATMAP_BF16 = 0x1       # gkd_kernel_heatmap flag: bfloat16 heatmaps
GKD_UPSAMPLE_CORNERS = 0x2   # gkd_kernel_heatmap flag: align_corners=True upsample
GKD_COORDS_CORNERS = 0x4     # decode flag: corner-aligned -1..1 coordinates
GKD_QUERY_TOKENS = 0x8       # query as [B, skip + H*W, C] tokens; skip in bits 8..15
STATUS = {0: "GKD_OK", 1: "GKD_ERR_NULL", 2: "GKD_ERR_SHAPE", 3: "GKD_ERR_DTYPE",
          4: "GKD_ERR_VALUE", 5: "GKD_ERR_UNSUPPORTED", 6: "GKD_ERR_HIP",
          7: "GKD_ERR_ALIGN"}

_lib = None
_P, _I, _U32, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_float


class GkdError(RuntimeError):
    """A gkd_* call returned a non-OK status."""

    def __init__(self, status: int, text: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {text}")


def load():
    """Load libgkdhead.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import "
            "__graft_entry__ as g; g.build()'` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.gkd_abi_version.restype = _I
    lib.gkd_status_string.restype = ctypes.c_char_p
    lib.gkd_status_string.argtypes = [_I]
    lib.gkd_last_error.restype = ctypes.c_char_p
    lib.gkd_vkp_pool.restype = _I
    lib.gkd_vkp_pool.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _I, _U32,
                                 _P, _P]
    lib.gkd_kernel_heatmap.restype = _I
    lib.gkd_kernel_heatmap.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                       _U32, _P, _P, _P, _P, _P]
    lib.gkd_peak_decode.restype = _I
    lib.gkd_peak_decode.argtypes = [_P, _P, _I, _I, _I, _I, _U32, _P, _P, _P, _P]
    lib.gkd_roi_preprocess.restype = _I
    lib.gkd_roi_preprocess.argtypes = [_P, _I, _I, _P, _I, _I, _I, _U32, _P, _P]
    lib.gkd_roi_backproject.restype = _I
    lib.gkd_roi_backproject.argtypes = [_P, _P, _I, _I, _I, _I, _I, _U32, _P, _P]
    lib.gkd_kg_workspace_size.restype = ctypes.c_size_t
    lib.gkd_kg_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I, _U32]
    lib.gkd_kg_transformer.restype = _I
    lib.gkd_kg_transformer.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _I, _I,
                                       _U32, _P, _P, ctypes.c_size_t, _P]
    lib.gkd_kg_transformer_noalloc.restype = _I
    lib.gkd_kg_transformer_noalloc.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I,
                                               _I, _I, _U32, _P, _P]
    if lib.gkd_abi_version() != GKD_ABI_VERSION:
        raise ImportError("libgkdhead ABI version mismatch")
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise GkdError(status, load().gkd_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GKD_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return GKD_DTYPE_BF16
    raise TypeError(f"features must be float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def vkp_pool(support: torch.Tensor, kpts: torch.Tensor, kpt_valid: torch.Tensor,
             stride: float = 16.0, sigma: float = 14.0,
             out: torch.Tensor | None = None, token_hw=None,
             token_skip: int = 0) -> torch.Tensor:
    """support [B,C,H,W] (f32|bf16), kpts [B,R,2] f32 px, kpt_valid [B,R] u8
    -> protos [B,R,C] in the support dtype (rows with kpt_valid == 0 are
    left as they are in `out`). token_hw=(H, W): the support map is the
    ViT's token sequence [B, token_skip + H*W, C] (GKD_QUERY_TOKENS)."""
    lib = load()
    if token_hw is None:
        _dev(support, "support", ndim=4)
        B, C, H, W = support.shape
        flags = 0
    else:
        _dev(support, "support", ndim=3)
        H, W = (int(v) for v in token_hw)
        B, T, C = support.shape
        if not 0 <= token_skip <= 255 or T != token_skip + H * W:
            raise ValueError("support must be [B, token_skip + H*W, C] with 0 <= token_skip <= 255")
        flags = GKD_QUERY_TOKENS | (token_skip << 8)
    _dev(kpts, "kpts", torch.float32, 3)
    _dev(kpt_valid, "kpt_valid", torch.uint8, 2)
    R = kpt_valid.shape[1]
    if kpts.shape != (B, R, 2) or kpt_valid.shape != (B, R):
        raise ValueError("kpts must be [B,R,2] and kpt_valid [B,R]")
    if out is None:
        out = torch.empty((B, R, C), dtype=support.dtype, device=support.device)
    _dev(out, "out", support.dtype)
    if out.shape != (B, R, C):
        raise ValueError("out must be [B,R,C]")
    _check(lib.gkd_vkp_pool(_ptr(support), _ptr(kpts), _ptr(kpt_valid), B, C, H, W, R,
                            float(stride), float(sigma), _dtype_code(support), flags,
                            _ptr(out), _stream(support.device)))
    return out


def kernel_heatmap(query: torch.Tensor, kern_vis=None, mask_vis=None, kern_txt=None,
                   mask_txt=None, decode: bool = True, out=None, out_decode=None,
                   heat_dtype=torch.float32, with_heatmaps: bool = True,
                   coords: str = "centres", align_corners: bool = False,
                   token_hw=None, token_skip: int = 0):
    """query [B,C,H,W] (f32|bf16); kern_* [B,R,C] in the query dtype with
    mask_* [B,R] u8 (None = modality absent).

    Returns heatmaps [B,R,4H,4W] in heat_dtype (float32, or bfloat16 via
    the GKD_HEATMAP_BF16 flag) and, if decode, (idx [B,R] i32, xy [B,R,2]
    f32, score [B,R] f32). Rows with no mask set are not written (they keep
    whatever `out` held). with_heatmaps=False computes the keypoints only
    (heatmaps NULL in the C call; decode must be True) and returns
    (idx, xy, score). coords: "centres" or "corners" (GKD_COORDS_CORNERS);
    align_corners: upsample on the align_corners=True grid
    (GKD_UPSAMPLE_CORNERS). token_hw=(H, W): the query is the ViT's token
    sequence [B, token_skip + H*W, C] (GKD_QUERY_TOKENS)."""
    lib = load()
    if token_hw is None:
        _dev(query, "query", ndim=4)
        B, C, H, W = query.shape
    else:
        _dev(query, "query", ndim=3)
        H, W = (int(v) for v in token_hw)
        B, T, C = query.shape
        if not 0 <= token_skip <= 255 or T != token_skip + H * W:
            raise ValueError("query must be [B, token_skip + H*W, C] with 0 <= token_skip <= 255")
    R = None
    for k, m, name in ((kern_vis, mask_vis, "vis"), (kern_txt, mask_txt, "txt")):
        if (k is None) != (m is None):
            raise ValueError(f"kern_{name} and mask_{name} go together")
        if k is not None:
            _dev(k, f"kern_{name}", query.dtype, 3)
            _dev(m, f"mask_{name}", torch.uint8, 2)
            if R is None:
                R = m.shape[1]
            if k.shape != (B, R, C) or m.shape != (B, R):
                raise ValueError(f"kern_{name} must be [B,R,C], mask_{name} [B,R]")
    if R is None:
        raise ValueError("at least one prompt modality is required")
    if heat_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"heat_dtype must be float32 or bfloat16, got {heat_dtype}")
    flags = ((GKD_HEATMAP_BF16 if heat_dtype == torch.bfloat16 else 0) | _coords_flag(coords) |
             (GKD_UPSAMPLE_CORNERS if align_corners else 0) |
             (GKD_QUERY_TOKENS | (token_skip << 8) if token_hw is not None else 0))
    if not with_heatmaps:
        if not decode:
            raise ValueError("with_heatmaps=False needs decode=True")
        if out is not None:
            raise ValueError("with_heatmaps=False takes no heatmap buffer")
    elif out is None:
        out = torch.empty((B, R, 4 * H, 4 * W), dtype=heat_dtype, device=query.device)
    if out is not None:
        _dev(out, "out", heat_dtype)
        if out.shape != (B, R, 4 * H, 4 * W):
            raise ValueError("out must be [B,R,4H,4W]")
    idx = xy = score = None
    if decode:
        if out_decode is None:
            idx = torch.empty((B, R), dtype=torch.int32, device=query.device)
            xy = torch.empty((B, R, 2), dtype=torch.float32, device=query.device)
            score = torch.empty((B, R), dtype=torch.float32, device=query.device)
        else:
            idx, xy, score = out_decode
    _check(lib.gkd_kernel_heatmap(_ptr(query), _ptr(kern_vis), _ptr(mask_vis),
                                  _ptr(kern_txt), _ptr(mask_txt), B, C, H, W, R,
                                  _dtype_code(query), flags, _ptr(out), _ptr(idx), _ptr(xy),
                                  _ptr(score), _stream(query.device)))
    if not with_heatmaps:
        return idx, xy, score
    if decode:
        return out, (idx, xy, score)
    return out


def _coords_flag(coords: str) -> int:
    if coords not in ("centres", "corners"):
        raise ValueError("coords must be 'centres' or 'corners'")
    return GKD_COORDS_CORNERS if coords == "corners" else 0


def peak_decode(heat: torch.Tensor, row_valid: torch.Tensor | None = None,
                coords: str = "centres"):
    """heat [B,R,Ho,Wo] f32, row_valid [B,R] u8 or None -> (idx [B,R] i32,
    xy [B,R,2] f32, score [B,R] f32); invalid rows get (-1, NaN, -inf).
    coords: "centres" ((2x + 1)/Wo - 1) or "corners" (2x/(Wo - 1) - 1)."""
    lib = load()
    _dev(heat, "heat", torch.float32, 4)
    B, R, Ho, Wo = heat.shape
    if row_valid is not None:
        _dev(row_valid, "row_valid", torch.uint8, 2)
        if row_valid.shape != (B, R):
            raise ValueError("row_valid must be [B,R]")
    idx = torch.empty((B, R), dtype=torch.int32, device=heat.device)
    xy = torch.empty((B, R, 2), dtype=torch.float32, device=heat.device)
    score = torch.empty((B, R), dtype=torch.float32, device=heat.device)
    _check(lib.gkd_peak_decode(_ptr(heat), _ptr(row_valid), B, R, Ho, Wo, _coords_flag(coords),
                               _ptr(idx), _ptr(xy), _ptr(score), _stream(heat.device)))
    return idx, xy, score


def roi_preprocess(image: torch.Tensor, boxes: torch.Tensor, size: int = 384,
                   dtype=torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    """image [H,W,3] u8 RGB, boxes [B,4] i32 (x0, y0, x1, y1) -> the
    backbone input [B,3,size,size] in dtype (float32 or bfloat16): each box
    cropped, resized so its longer side is `size`, centre-padded with the
    mean colour and ImageNet-normalised."""
    lib = load()
    _dev(image, "image", torch.uint8, 3)
    _dev(boxes, "boxes", torch.int32, 2)
    if image.shape[2] != 3 or boxes.shape[1] != 4:
        raise ValueError("image must be [H,W,3] and boxes [B,4]")
    if dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("dtype must be float32 or bfloat16")
    B = boxes.shape[0]
    if out is None:
        out = torch.empty((B, 3, size, size), dtype=dtype, device=image.device)
    else:
        _dev(out, "out", dtype, 4)
        if out.shape != (B, 3, size, size):
            raise ValueError("out must be [B,3,size,size]")
    _check(lib.gkd_roi_preprocess(_ptr(image), image.shape[0], image.shape[1], _ptr(boxes), B,
                                  size, 1 if dtype == torch.bfloat16 else 0, 0, _ptr(out),
                                  _stream(image.device)))
    return out


def roi_backproject(xy: torch.Tensor, boxes: torch.Tensor, image_hw, size: int = 384,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """xy [B,R,2] f32 in the ROI canvas's -1..1 frame -> image coordinates
    [B,R,2] f32 (continuous, pixel i covers [i, i + 1)); NaN stays NaN."""
    lib = load()
    _dev(xy, "xy", torch.float32, 3)
    _dev(boxes, "boxes", torch.int32, 2)
    B, R, two = xy.shape
    if two != 2 or boxes.shape != (B, 4):
        raise ValueError("xy must be [B,R,2] and boxes [B,4]")
    if out is None:
        out = torch.empty_like(xy)
    else:
        _dev(out, "out", torch.float32, 3)
        if out.shape != xy.shape:
            raise ValueError("out must be [B,R,2]")
    _check(lib.gkd_roi_backproject(_ptr(xy), _ptr(boxes), B, R, int(image_hw[0]),
                                   int(image_hw[1]), size, 0, _ptr(out), _stream(xy.device)))
    return out


def kg_workspace_size(B: int, C: int, H: int, W: int, R: int, d_ff: int = 1024,
                      tokens: bool = False) -> int:
    """Bytes of workspace gkd_kg_transformer needs for these sizes."""
    return int(load().gkd_kg_workspace_size(B, C, H, W, R, d_ff,
                                            GKD_QUERY_TOKENS if tokens else 0))


def kg_transformer(query: torch.Tensor, weights: torch.Tensor, kern_vis=None, mask_vis=None,
                   kern_txt=None, mask_txt=None, n_blocks: int = 2, d_ff: int = 1024,
                   token_hw=None, token_skip: int = 0, out=None,
                   workspace=None) -> torch.Tensor:
    """Kernel-generation transformer: prototypes [B,R,C] bf16 (with their
    [B,R] u8 masks) -> kernels [2,B,R,C] bf16: out[0] from the visual slots,
    out[1] from the text slots, ready as the heatmap call's kern_vis and
    kern_txt.
    query [B,C,H,W] bf16, or with token_hw=(H, W) the token sequence
    [B, token_skip + H*W, C]; weights: the flat bf16 array. workspace: a
    uint8 CUDA tensor of at least kg_workspace_size() bytes (allocated here
    when None), or "static" for gkd_kg_transformer_noalloc (the library's
    static workspace of GKD_KG_STATIC_WORKSPACE_BYTES per GPU; nothing is
    allocated by the call, `out` included when it is given)."""
    lib = load()
    if token_hw is None:
        _dev(query, "query", torch.bfloat16, 4)
        B, C, H, W = query.shape
        flags = 0
    else:
        _dev(query, "query", torch.bfloat16, 3)
        H, W = (int(v) for v in token_hw)
        B, T, C = query.shape
        if not 0 <= token_skip <= 255 or T != token_skip + H * W:
            raise ValueError("query must be [B, token_skip + H*W, C] with 0 <= token_skip <= 255")
        flags = GKD_QUERY_TOKENS | (token_skip << 8)
    _dev(weights, "weights", torch.bfloat16, 1)
    masks = [m for m in (mask_vis, mask_txt) if m is not None]
    if not masks:
        raise ValueError("give mask_vis, mask_txt or both")
    R = masks[0].shape[1]
    for k, m, name in ((kern_vis, mask_vis, "vis"), (kern_txt, mask_txt, "txt")):
        if m is None:
            continue
        _dev(m, "mask_" + name, torch.uint8, 2)
        _dev(k, "kern_" + name, torch.bfloat16, 3)
        if m.shape != (B, R) or k.shape != (B, R, C):
            raise ValueError(f"kern_{name} must be [B,R,C] and mask_{name} [B,R]")
    if out is None:
        out = torch.empty((2, B, R, C), dtype=torch.bfloat16, device=query.device)
    _dev(out, "out", torch.bfloat16, 4)
    if out.shape != (2, B, R, C):
        raise ValueError("out must be [2,B,R,C]")
    args = (_ptr(kern_vis) if mask_vis is not None else None, _ptr(mask_vis),
            _ptr(kern_txt) if mask_txt is not None else None, _ptr(mask_txt), _ptr(query),
            B, C, H, W, R, _ptr(weights), n_blocks, d_ff, 1, flags, _ptr(out))
    if workspace == "static":
        # no workspace argument: the library's own static device array
        _check(lib.gkd_kg_transformer_noalloc(*args, _stream(query.device)))
        return out
    need = int(lib.gkd_kg_workspace_size(B, C, H, W, R, d_ff, flags))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=query.device)
    _dev(workspace, "workspace", torch.uint8, 1)
    _check(lib.gkd_kg_transformer(*args, _ptr(workspace), workspace.numel(),
                                  _stream(query.device)))
    return out
