"""Seeded synthetic inputs for the ROI stage (detector boxes on one image).

Only random numbers: an 8-bit RGB image of uniform noise (every pixel
differs from its neighbours, so a resampling slip shows at full strength)
and detector-like boxes. Box centres are uniform over the image, widths
log-uniform in [32, 900] px and aspect ratios (height / width) log-uniform
in [1/2, 3], so boxes cover wide, tall and near-square crops, both up- and
downscaled to the 384 px input; some boxes reach past the image border and
are clamped there. The model card's 384 px input and the top-down use (one
box per detected object) set the shapes; no public dataset is involved.
"""
import numpy as np


def make_roi(seed: int = 0, B: int = 256, H: int = 1080, W: int = 1920, R: int = 80,
             size: int = 384):
    rng = np.random.default_rng(seed)
    image = rng.integers(0, 256, size=(H, W, 3), dtype=np.uint8)
    w = 32.0 * (900.0 / 32.0) ** rng.random(B)        # log-uniform widths
    h = w * 0.5 * (3.0 / 0.5) ** rng.random(B)         # log-uniform aspect
    cx, cy = rng.uniform(0, W, B), rng.uniform(0, H, B)
    boxes = np.stack([cx - w / 2, cy - h / 2, cx + w / 2, cy + h / 2], axis=1)
    boxes = np.round(boxes).astype(np.int32)
    boxes[:, 2] = np.maximum(boxes[:, 2], boxes[:, 0] + 1)
    boxes[:, 3] = np.maximum(boxes[:, 3], boxes[:, 1] + 1)
    # keypoints in the canvas's -1..1 frame, uniform, some rows invalid (NaN)
    xy = rng.uniform(-1.0, 1.0, size=(B, R, 2)).astype(np.float32)
    xy[rng.random((B, R)) < 0.2] = np.nan
    return {"image": image, "boxes": boxes, "xy": xy, "B": B, "H": H, "W": W, "R": R,
            "size": size}
