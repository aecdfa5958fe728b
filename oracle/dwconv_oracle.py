"""fp64 CPU oracle of the depth-wise 3x3 convolution over the token grid.

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
use it. It shares no code with the HIP library and does not import the package.

What it computes. Vision-TTT adds a depth-wise convolution that aggregates local 2D token
correlations before the scan (Vision-TTT summary on gist.science, "Methodologie" item 2, the
Conv2d module; the Vision-TTT review on nubint.ai calls it Conv2d-based preprocessing of the
dataset); ViT^3 runs a 3x3 depth-wise convolution branch beside its main branch (ViT^3 review on
techloop.online, "TTT Block" section and the section on the official code). The pages give no
formula, so this takes the plainest reading, the convolution layer of deep learning: a token
sequence of N = height * width tokens in raster order, [B, N, C] with C channels, viewed as a
[B, height, width, C] image; each channel c has its own 3x3 kernel w[c] and bias b[c]; the
output is the cross-correlation with zero padding of one token on each side ("same" size):
    y[b, i, j, c] = b[c] + sum_{u, v in 0..2} w[c, u, v] * x[b, i + u - 1, j + v - 1, c],
terms outside the image being zero.

Parity status: pinned by tests/test_oracle_pins_dwconv.py (identity and shift kernels, torch's
convolution, linearity, shift equivariance, channel independence, brute force on tiny inputs).
"""
from __future__ import annotations

import numpy as np


def dwconv3x3(x, weight, bias, height: int, width: int):
    """x: [B, height * width, C]; weight: [C, 3, 3]; bias: [C] or None. Returns float64 [B, N, C]."""
    x = np.asarray(x, dtype=np.float64)
    B, N, C = x.shape
    if N != height * width:
        raise ValueError(f"{N} tokens are not a {height} x {width} grid")
    w = np.asarray(weight, dtype=np.float64)
    if w.shape != (C, 3, 3):
        raise ValueError(f"weight must be [{C}, 3, 3]")
    img = x.reshape(B, height, width, C)
    pad = np.zeros((B, height + 2, width + 2, C))
    pad[:, 1:-1, 1:-1] = img
    y = np.zeros((B, height, width, C)) if bias is None else np.broadcast_to(
        np.asarray(bias, dtype=np.float64), (B, height, width, C)).copy()
    for u in range(3):
        for v in range(3):
            y += w[:, u, v] * pad[:, u:u + height, v:v + width]
    return y.reshape(B, N, C)
