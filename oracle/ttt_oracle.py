"""fp64 CPU oracle for the TTT-layer forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module: only
tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may use it.
It shares no code with the HIP library (test_sequence_layers_amd/csrc) and does
not import the package; the two meet only through the seeded input generator.

What it computes, per (batch, head) pair -- every head is an independent inner
model (Vision-TTT summary on gist.science, "Methodologie" item 3: the hidden
state is split over several heads):

* Tokens are rows. The inner linear model predicts k.W with W of shape [D, D];
  the inner MLP predicts GELU(k.W1).W2.
* The self-supervised loss of one token is l(W; k, v) = 1/2 ||f_W(k) - v||^2
  (reconstruction loss: Vision-TTT summary, "Methodologie" item 1; ViT^3
  review on techloop.online, design-space study: an MSE-type loss). A step over
  a batch of n tokens averages the per-token gradients, so the step is
  W <- W - (eta/n) * sum_j grad l_j(W) (the gradient-descent rule in
  "Methodologie" item 1 of the Vision-TTT summary, with mini-batches of
  "Methodologie" item 3).
* Gradients are hand-derived closed forms, not autograd (ViT^3 review, section
  on the official code: the authors write the inner gradient by hand).

Everything is evaluated in the PRIMAL form: the weights each output is read with
are materialised explicitly. The GPU path uses different algebra (dual forms,
affine segment maps), so the two share neither code nor association order.

Inputs are [B, N, H, D] arrays (already rounded to the I/O dtype; they are
widened to float64 here); inner states are [H, ...] (shared over the batch) or
[B, H, ...] (one per batch element).

Parity status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, special cases, finite differences, autograd, exact rational
arithmetic; chunked_bidir_2d and grid_transpose in test_oracle_pins_2d.py) and
tests/test_oracle_pins_epochs.py (fullbatch_epochs: closed form
with orthogonal keys, convergence to least squares) and tests/test_oracle_pins_vjp.py
(fullbatch_vjp: finite differences, torch autograd, eta = 0) and
tests/test_oracle_pins_chunked_vjp.py (chunked_causal_vjp, chunked_bidir_vjp: finite differences,
torch autograd of the dual form, eta = 0, one chunk = the full-batch gradients). None is "parity
unpinned".
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _bhnd(x) -> np.ndarray:
    """[B, N, H, D] -> float64 [B, H, N, D]."""
    return np.ascontiguousarray(np.transpose(np.asarray(x, dtype=np.float64), (0, 2, 1, 3)))


def _bnhd(x) -> np.ndarray:
    """float64 [B, H, N, D] -> [B, N, H, D]."""
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))


def _state(w, B: int, H: int) -> np.ndarray:
    """[H, r, c] or [B, H, r, c] -> float64 [B, H, r, c] (a private copy)."""
    w = np.asarray(w, dtype=np.float64)
    if w.ndim == 3:
        w = np.broadcast_to(w, (B,) + w.shape)
    if w.shape[:2] != (B, H):
        raise ValueError(f"state shape {w.shape} does not match B={B}, H={H}")
    return np.array(w)


def _t(x: np.ndarray) -> np.ndarray:
    """Transpose of the last two axes."""
    return np.swapaxes(x, -1, -2)


def _check_chunk(N: int, chunk: int) -> None:
    if chunk <= 0 or N % chunk != 0:
        raise ValueError(f"sequence length {N} is not a multiple of the mini-batch size {chunk}")


# --------------------------------------------------------------------------------------------
# Variant (a): single-epoch full-batch update (ViT^3)
# --------------------------------------------------------------------------------------------
def fullbatch(q, k, v, w0, eta: float):
    """One full-batch gradient step on all N (k, v) pairs, then read out Q.

    ViT^3 review (techloop.online), "core idea" section: train the inner model on
    (K, V), get W*, output F_{W*}(Q); design-space study: one epoch, full batch,
    inner learning rate 1.0. With l_j = 1/2 ||k_j W - v_j||^2 averaged over N:
        W* = W0 - (eta/N) K^T (K W0 - V),   O = Q W*.
    Returns (O [B,N,H,D], W* [B,H,D,D]).
    """
    Q, K, V = _bhnd(q), _bhnd(k), _bhnd(v)
    B, H, N, _ = Q.shape
    W0 = _state(w0, B, H)
    E = K @ W0 - V                       # residuals f_W0(k_j) - v_j, one row per token
    G = _t(K) @ E                        # sum_j of per-token gradients k_j^T e_j
    W = W0 - (eta / N) * G
    return _bnhd(Q @ W), W


def fullbatch_vjp(q, k, v, w0, eta: float, d_o):
    """Gradients of the full-batch layer for the outer training loop: given dO = dL/dO, returns
    (dL/dq, dL/dk, dL/dv, dL/dW0) of the one-step forward above, in closed form (the pages'
    authors likewise derive the inner gradient by hand rather than by autograd: ViT^3 review,
    section on the official code). With s = eta/N, E = K W0 - V, W* = W0 - s K^T E and
    G = Q^T dO = dL/dW*:
        dQ  = dO W*^T
        dW0 = (I - s K^T K) G                 (dW*/dW0 = I - s K^T K, symmetric)
        dV  = s K G                            (W* depends on V through s K^T V)
        dK  = -s (E G^T + K G W0^T)            (from d(K^T (K W0 - V)) = dK^T E + K^T dK W0)
    Inputs as for fullbatch, d_o [B,N,H,D]. Returns ([B,N,H,D] x 3, [B,H,D,D]).
    """
    Q, K, V, dO = _bhnd(q), _bhnd(k), _bhnd(v), _bhnd(d_o)
    B, H, N, D = Q.shape
    W0 = _state(w0, B, H)
    s = eta / N
    E = K @ W0 - V
    Ws = W0 - s * (_t(K) @ E)
    G = _t(Q) @ dO
    dQ = dO @ _t(Ws)
    dW0 = G - s * (_t(K) @ (K @ G))
    dV = s * (K @ G)
    dK = -s * (E @ _t(G) + K @ G @ _t(W0))
    return _bnhd(dQ), _bnhd(dK), _bnhd(dV), dW0


def fullbatch_epochs(q, k, v, w0, eta: float, epochs: int):
    """Several full-batch epochs of the inner training before the read-out.

    ViT^3 review (techloop.online), design-space study: how many epochs one inner update runs is
    one of the studied choices (single epoch is the one the final models keep). Epoch e takes one
    full-batch gradient step from the previous epoch's weights:
        W_{e+1} = W_e - (eta/N) K^T (K W_e - V),   W_0 = W0,   O = Q W_epochs.
    Returns (O [B,N,H,D], W_epochs [B,H,D,D]).
    """
    if epochs < 1:
        raise ValueError("at least one epoch")
    Q, K, V = _bhnd(q), _bhnd(k), _bhnd(v)
    B, H, N, _ = Q.shape
    W = _state(w0, B, H)
    for _ in range(epochs):
        W = W - (eta / N) * (_t(K) @ (K @ W - V))
    return _bnhd(Q @ W), W


# --------------------------------------------------------------------------------------------
# Variant (b): bidirectional chunked scan (Vision-TTT)
# --------------------------------------------------------------------------------------------
def _scan_noncausal(Q, K, V, W0, eta: float, b: int):
    """Mini-batch GD over consecutive chunks of b tokens; each chunk is read out
    with the state *after* its own update (non-causal inside the chunk)."""
    N = Q.shape[2]
    W = W0.copy()
    O = np.empty_like(Q)
    for c0 in range(0, N, b):
        Kc, Vc = K[:, :, c0:c0 + b], V[:, :, c0:c0 + b]
        W = W - (eta / b) * (_t(Kc) @ (Kc @ W - Vc))
        O[:, :, c0:c0 + b] = Q[:, :, c0:c0 + b] @ W
    return O, W


def chunked_bidir(q, k, v, w0, eta: float, chunk: int):
    """Forward scan plus a scan of the token-reversed sequence, both from W0, summed.

    Vision-TTT summary (gist.science), "Methodologie" item 2: tokens are scanned
    both forwards and backwards; item 3: mini-batch gradient steps of b tokens.
    The reversed run's outputs are flipped back to token order before the sum.
    Returns (O, W_fwd_end, W_rev_end).
    """
    Q, K, V = _bhnd(q), _bhnd(k), _bhnd(v)
    B, H, N, _ = Q.shape
    _check_chunk(N, chunk)
    W0 = _state(w0, B, H)
    Of, Wf = _scan_noncausal(Q, K, V, W0, eta, chunk)
    rev = slice(None, None, -1)
    Or, Wr = _scan_noncausal(Q[:, :, rev], K[:, :, rev], V[:, :, rev], W0, eta, chunk)
    return _bnhd(Of + Or[:, :, rev]), Wf, Wr


def grid_transpose(x, height: int, width: int):
    """[B, height * width, ...] tokens in raster order -> the same tokens in column order (the
    raster order of the transposed [width, height] grid)."""
    x = np.asarray(x)
    B = x.shape[0]
    rest = x.shape[2:]
    return np.ascontiguousarray(np.swapaxes(x.reshape((B, height, width) + rest), 1, 2).reshape((B, height * width) + rest))


def chunked_bidir_2d(q, k, v, w0, eta: float, chunk: int, height: int, width: int):
    """Bidirectional scans in raster order and in column order, summed.

    The Vision-TTT summary (gist.science, "De Oplossing": the bidirectional scanner reads the image
    left to right, right to left, and top to bottom) adds a column scan to the raster scans. Read
    here as: the bidirectional scan of chunked_bidir over the tokens in raster order, plus the same
    over the tokens in column order (top to bottom, column by column), its outputs put back in
    raster order; all four directions start from the same W0.
    Returns (O, [raster fwd end, raster rev end, column fwd end, column rev end]).
    """
    O1, Wf1, Wr1 = chunked_bidir(q, k, v, w0, eta, chunk)
    qt, kt, vt = (grid_transpose(t, height, width) for t in (q, k, v))
    O2t, Wf2, Wr2 = chunked_bidir(qt, kt, vt, w0, eta, chunk)
    O2 = grid_transpose(O2t, width, height)
    return O1 + O2, [Wf1, Wr1, Wf2, Wr2]


# --------------------------------------------------------------------------------------------
# Variant (c): causal mini-batch TTT-Linear and TTT-MLP
# --------------------------------------------------------------------------------------------
def chunked_causal(q, k, v, w0, eta: float, chunk: int):
    """TTT-Linear (TTT-Linear/TTT-MLP abstract: the hidden state is a linear model
    updated by a self-supervised step) with causal mini-batches of b tokens.

    Inside a chunk every gradient is taken at the chunk's start state W_s; token i
    is read out with W_s - (eta/b) * sum_{j <= i} grad l_j(W_s) (its own gradient
    included), and the chunk hands W_s - (eta/b) * sum_{all j} grad l_j(W_s) on.
    Returns (O, W_end).
    """
    Q, K, V = _bhnd(q), _bhnd(k), _bhnd(v)
    B, H, N, D = Q.shape
    _check_chunk(N, chunk)
    a = eta / chunk
    W = _state(w0, B, H)
    O = np.empty_like(Q)
    for c0 in range(0, N, chunk):
        Ws = W
        S = np.zeros_like(Ws)
        for i in range(c0, c0 + chunk):
            ki, vi, qi = K[:, :, i:i + 1], V[:, :, i:i + 1], Q[:, :, i:i + 1]
            S = S + _t(ki) @ (ki @ Ws - vi)          # grad of 1/2||k_i W - v_i||^2 at W_s
            O[:, :, i:i + 1] = qi @ (Ws - a * S)     # token i's own weights
        W = Ws - a * S
    return _bnhd(O), W


def _scan_vjp(Q, K, V, W0, dO, eta: float, b: int, causal: bool):
    """Reverse mode through the primal mini-batch loop of one scan direction ([B, H, N, D] arrays,
    tokens in the scan's order).

    Forward, per chunk with start state W_s and a = eta/b: e_j = k_j W_s - v_j, S_i = sum over the
    chunk's tokens j <= i (causal) or all of them (read-out after the update) of k_j^T e_j,
    o_i = q_i (W_s - a S_i), and the chunk hands W_s - a S_last on. Backward, chunks last to first,
    with lam = dL/d(state handed on) (zero after the last chunk):
        dq_i   = do_i (W_s - a S_i)^T
        Gam_j  = -a (lam + sum of q_i^T do_i over the outputs i whose S_i contains token j)
        de_j   = k_j Gam_j                 (S_i holds k_j^T e_j)
        dk_j   = e_j Gam_j^T + de_j W_s^T  (through k_j^T e_j and through e_j = k_j W_s - v_j)
        dv_j   = -de_j
        lam   <- lam + sum_i q_i^T do_i + sum_j k_j^T de_j   (= dL/dW_s)
    Returns (dQ, dK, dV, dW0) with dW0 [B, H, D, D]."""
    B, H, N, D = Q.shape
    a = eta / b
    starts = []
    W = W0.copy()
    for c0 in range(0, N, b):  # forward pass: every chunk's start state
        starts.append(W)
        Kc, Vc = K[:, :, c0:c0 + b], V[:, :, c0:c0 + b]
        W = W - a * (_t(Kc) @ (Kc @ W - Vc))
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    lam = np.zeros_like(W0)
    for ci in range(N // b - 1, -1, -1):
        c0 = ci * b
        Ws = starts[ci]
        rows = [c0 + i for i in range(b)]
        e = {j: K[:, :, j:j + 1] @ Ws - V[:, :, j:j + 1] for j in rows}
        qdo = {i: _t(Q[:, :, i:i + 1]) @ dO[:, :, i:i + 1] for i in rows}
        S = np.zeros_like(Ws)
        total_qdo = sum(qdo.values())
        S_all = sum(_t(K[:, :, j:j + 1]) @ e[j] for j in rows)
        for i in rows:  # read-out weights of each output
            S = S + _t(K[:, :, i:i + 1]) @ e[i]
            Wi = Ws - a * (S if causal else S_all)
            dQ[:, :, i:i + 1] = dO[:, :, i:i + 1] @ _t(Wi)
        lam_prev = lam + total_qdo
        later = np.zeros_like(Ws)  # sum of q_i^T do_i over outputs i >= j (causal)
        for j in reversed(rows):
            later = later + qdo[j]
            Gam = -a * (lam + (later if causal else total_qdo))
            kj = K[:, :, j:j + 1]
            de = kj @ Gam
            dK[:, :, j:j + 1] = e[j] @ _t(Gam) + de @ _t(Ws)
            dV[:, :, j:j + 1] = -de
            lam_prev = lam_prev + _t(kj) @ de
        lam = lam_prev
    return dQ, dK, dV, lam


def chunked_causal_vjp(q, k, v, w0, eta: float, chunk: int, d_o):
    """Gradients of the causal chunked TTT-Linear layer (chunked_causal) for the outer training
    loop: (dL/dq, dL/dk, dL/dv, dL/dW0) for L = <dO, O>, by reverse mode through the primal loop
    (the pages' authors derive the inner gradient by hand: ViT^3 review, section on the official
    code; the outer gradient here follows the same closed-form style). dW0 is per batch element
    [B, H, D, D]; a W0 shared over the batch gets the sum over B."""
    Q, K, V, dO = _bhnd(q), _bhnd(k), _bhnd(v), _bhnd(d_o)
    B, H, N, D = Q.shape
    _check_chunk(N, chunk)
    dQ, dK, dV, dW0 = _scan_vjp(Q, K, V, _state(w0, B, H), dO, eta, chunk, causal=True)
    return _bnhd(dQ), _bnhd(dK), _bnhd(dV), dW0


def chunked_bidir_vjp(q, k, v, w0, eta: float, chunk: int, d_o):
    """Gradients of the bidirectional scan (chunked_bidir): the forward scan's and the reversed
    scan's gradients summed (both read the same q, k, v, W0 and receive the same dO, the reversed
    one in its own token order). Returns (dq, dk, dv [B,N,H,D], dW0 [B,H,D,D])."""
    Q, K, V, dO = _bhnd(q), _bhnd(k), _bhnd(v), _bhnd(d_o)
    B, H, N, D = Q.shape
    _check_chunk(N, chunk)
    W0 = _state(w0, B, H)
    gf = _scan_vjp(Q, K, V, W0, dO, eta, chunk, causal=False)
    rev = slice(None, None, -1)
    gr = _scan_vjp(Q[:, :, rev], K[:, :, rev], V[:, :, rev], W0, dO[:, :, rev], eta, chunk, causal=False)
    grads = [_bnhd(f + r[:, :, rev]) for f, r in zip(gf[:3], gr[:3])]
    return grads[0], grads[1], grads[2], gf[3] + gr[3]


def gelu(x):
    """Exact GELU, x * Phi(x)."""
    return 0.5 * x * (1.0 + erf(x / _SQRT2))


def gelu_prime(x):
    """d/dx [x Phi(x)] = Phi(x) + x phi(x)."""
    return 0.5 * (1.0 + erf(x / _SQRT2)) + x * np.exp(-0.5 * x * x) * _INV_SQRT_2PI


def mlp_token_grad(k, v, W1, W2):
    """Hand-derived gradient of l = 1/2 ||GELU(k W1) W2 - v||^2 for one token per (b, h).

    k, v: [..., 1, D]; W1: [..., D, Dh]; W2: [..., Dh, D]. Returns (dl/dW1, dl/dW2).
    """
    z = k @ W1
    x = gelu(z)
    e = x @ W2 - v
    g2 = _t(x) @ e
    dz = (e @ _t(W2)) * gelu_prime(z)
    g1 = _t(k) @ dz
    return g1, g2


def mlp_causal(q, k, v, w1, w2, eta: float, chunk: int):
    """TTT-MLP (TTT-Linear/TTT-MLP abstract: the hidden state is a two-layer MLP)
    with causal mini-batches of b tokens; f(x) = GELU(x W1) W2, no bias.

    Token i is read out with (W1_s - (eta/b) A1_i, W2_s - (eta/b) A2_i), where
    A*_i sums the per-token gradients of tokens j <= i in the chunk, each taken at
    the chunk's start state (W1_s, W2_s). Returns (O, W1_end, W2_end).
    """
    Q, K, V = _bhnd(q), _bhnd(k), _bhnd(v)
    B, H, N, D = Q.shape
    _check_chunk(N, chunk)
    a = eta / chunk
    W1 = _state(w1, B, H)
    W2 = _state(w2, B, H)
    O = np.empty_like(Q)
    for c0 in range(0, N, chunk):
        W1s, W2s = W1, W2
        A1 = np.zeros_like(W1s)
        A2 = np.zeros_like(W2s)
        for i in range(c0, c0 + chunk):
            ki, vi, qi = K[:, :, i:i + 1], V[:, :, i:i + 1], Q[:, :, i:i + 1]
            g1, g2 = mlp_token_grad(ki, vi, W1s, W2s)
            A1 = A1 + g1
            A2 = A2 + g2
            O[:, :, i:i + 1] = gelu(qi @ (W1s - a * A1)) @ (W2s - a * A2)
        W1 = W1s - a * A1
        W2 = W2s - a * A2
    return _bnhd(O), W1, W2


def run(inputs, w_override=None):
    """Run the oracle on a synth.Inputs object; returns the output [B,N,H,D] float64.

    w_override replaces the initial state(s): a [B,H,..] array for TTT-Linear or
    a (W1, W2) pair for TTT-MLP.
    """
    wl = inputs.wl
    q, k, v = inputs.q64, inputs.k64, inputs.v64
    if wl.op == "fullbatch":
        return fullbatch(q, k, v, inputs.w0 if w_override is None else w_override, wl.eta)[0]
    if wl.op == "bidir":
        return chunked_bidir(q, k, v, inputs.w0 if w_override is None else w_override, wl.eta, wl.chunk)[0]
    if wl.op == "causal":
        return chunked_causal(q, k, v, inputs.w0 if w_override is None else w_override, wl.eta, wl.chunk)[0]
    if wl.op == "mlp":
        w1, w2 = (inputs.w1, inputs.w2) if w_override is None else w_override
        return mlp_causal(q, k, v, w1, w2, wl.eta, wl.chunk)[0]
    raise ValueError(wl.op)
