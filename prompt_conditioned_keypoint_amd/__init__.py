"""GKDT parameter-free detection head on AMD MI355X (gfx950).

Calls over the C ABI of libgkdhead (include/gkdhead.h):
  vkp_pool         Gaussian-pooled visual keypoint prototypes
  kernel_heatmap   normalised 1x1 kernels x 4x-upsampled features, fused per
                   row over the prompt modalities, with the peak decode fused
  peak_decode      per-row argmax -> -1..1 keypoint + score
  roi_preprocess   detector boxes of an image -> the backbone's normalised
                   square input (crop, resize, centre pad, normalise)
  roi_backproject  -1..1 keypoints -> image coordinates
  kg_transformer   kernel-generation transformer: prototypes -> kernels
"""
from .binding import (GkdError, LIB_PATH, kernel_heatmap, kg_transformer, kg_workspace_size,
                      load, peak_decode, roi_backproject, roi_preprocess, vkp_pool)

__all__ = ["GkdError", "LIB_PATH", "kernel_heatmap", "kg_transformer", "kg_workspace_size",
           "load", "peak_decode", "roi_backproject", "roi_preprocess", "vkp_pool"]
