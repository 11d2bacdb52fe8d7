"""Seeded synthetic weights for the kernel-generation transformer.

The pages publish no weights, so the transformer is exercised with random
ones: linear weights N(0, 1/fan_in) (unit-variance inputs give unit-variance
outputs), biases N(0, 0.02^2), LayerNorm weights 1 + N(0, 0.1^2) and biases
N(0, 0.1^2), the mask token N(0, 1). All values are rounded to bfloat16
(round to nearest even) so that both sides of a comparison see the same
numbers. Only random draws and the layout of the flat array live here.
"""
import numpy as np

from .configs import round_bf16_f32


def kg_weights(C: int = 1024, d_ff: int = 1024, n_blocks: int = 2, seed: int = 0):
    """Flat float32 array (bfloat16-exact values) in the documented order."""
    rng = np.random.default_rng(seed)
    parts = [rng.standard_normal(C)]
    for _ in range(n_blocks):
        for rows, cols, ln in ((3 * C, C, False), (C, C, True), (3 * C, C, False),
                               (C, C, True), (d_ff, C, False), (C, d_ff, True)):
            parts.append(rng.standard_normal(rows * cols) / np.sqrt(cols))
            parts.append(0.02 * rng.standard_normal(rows))
            if ln:
                parts.append(1.0 + 0.1 * rng.standard_normal(C))
                parts.append(0.1 * rng.standard_normal(C))
    return round_bf16_f32(np.concatenate(parts).astype(np.float32))
