"""fp64 CPU oracle of the ViT^3 block epilogue.

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
use it. It shares no code with the HIP library and does not import the package.

What it computes. The ViT^3 block runs two branches in parallel, a GLU-style main branch and a
3x3 depth-wise convolution branch, then concatenates their outputs and projects them back to the
block's width (ViT^3 review on techloop.online, "TTT Block" section and the section on the
official code). The pages give no formula; the plainest reading, with the gating of the original
gated linear unit (a sigmoid gate): for each token, with O the TTT layer's output, G its gate
input and X the convolution branch's output (all [M, C]),
    y = [O * sigmoid(G), X] Wo^T + b,
Wo [C_out, 2C] (a linear layer's [out, in] layout), b [C_out] or none.

Parity status: pinned by tests/test_oracle_pins_block.py (torch's glu and linear layer, the
split of the projection into its two halves, the saturated gate).
"""
from __future__ import annotations

import numpy as np


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def block_epilogue(o, gate, xconv, w_proj, bias=None):
    o, gate, xconv = (np.asarray(t, dtype=np.float64) for t in (o, gate, xconv))
    w = np.asarray(w_proj, dtype=np.float64)
    cat = np.concatenate([o * sigmoid(gate), xconv], axis=-1)
    y = cat @ w.T
    return y if bias is None else y + np.asarray(bias, dtype=np.float64)
