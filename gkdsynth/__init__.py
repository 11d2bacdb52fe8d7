"""Seeded synthetic workloads for the GKDT detection head.

This module only draws random numbers and lays them out in the shapes the
head consumes. It holds none of the head's arithmetic (no Gaussian pooling,
no upsampling, no convolution, no fusion, no argmax); both the CPU oracle
and the GPU library consume its arrays unchanged.

Shapes follow the GKDT-L model card (Hugging Face page "Asher-1/GKD_GGUF",
section "Model"): a 384 px crop through a stride-16 ViT-L gives 24x24 patch
features with D=1024 channels, the head emits 96x96 heatmaps, and prompt
rows are padded to 80 with a validity mask. The paper summary (agihunt.info,
GKDT, pipeline paragraph) gives the three prompt modes: visual, text, both.

Recipe (every config):
  * features are N(0,1) drawn in float32, planted in float32, and only then
    rounded to bfloat16 (round to nearest even) when the config is bf16;
  * text kernels are N(0,1) rows of length C;
  * support keypoints are uniform over the padded input, [0, W*16)^2 px;
  * a "planted peak" adds alpha * u to the query fibre at one low-res cell,
    with u a unit vector along the row's prompt direction; planted cells are
    uniform over the grid and distinct within a crop;
  * visual rows get their prompt direction from the support map: the
    generator draws a random unit vector u_r and adds sqrt(C) * u_r (per
    channel RMS 1, the same scale as the noise) to the 3x3 block of support
    fibres around the keypoint's cell. Gaussian pooling (sigma 14 px) then
    yields a prototype whose direction is close to u_r (cosine ~0.9 at
    C=1024), and the query peak is planted along u_r;
  * dual rows plant along unit(u_r + unit(k_txt)).
"""
from .configs import CONFIGS, config_names, make, round_bf16_f32, bf16_bits
from .roi import make_roi

from .kg import kg_weights  # noqa: E402

__all__ = ["CONFIGS", "config_names", "make", "make_roi", "kg_weights", "round_bf16_f32",
           "bf16_bits"]
