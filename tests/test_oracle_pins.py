"""Pins of the fp64 oracle to what the mathematics fixes (no GPU).

Every oracle function is checked against something other than its own formula:
closed forms and textbook special cases (linear attention, the delta rule),
finite differences and torch autograd for every hand-derived gradient, an
independent dual-form evaluation, invariants (reversal, permutation inside a
chunk, state carry), and exact rational arithmetic on tiny integer inputs.
Each test names the kind of mistake it would catch.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import ttt_oracle as O
from test_sequence_layers_amd import synth

RNG = np.random.default_rng(20260301)


def _rand(B, N, H, D, scale=None):
    s = (1.0 / np.sqrt(D)) if scale is None else scale
    return [RNG.standard_normal((B, N, H, D)) * s for _ in range(3)]


def _w(B, H, r, c, scale=0.02, per_batch=False):
    shape = (B, H, r, c) if per_batch else (H, r, c)
    return RNG.standard_normal(shape) * scale


def _heads(x):  # [B,N,H,D] -> [B,H,N,D]
    return np.transpose(x, (0, 2, 1, 3))


# ------------------------------------------------------------------ full-batch
def test_fullbatch_w0_zero_is_linear_attention():
    """W0 = 0 turns the step into linear attention, O = (eta/N) (Q K^T) V, here evaluated through
    the N x N score matrix (ViT^3 review, core idea: linear attention compresses K, V into one state).
    Catches a wrong sign, a dropped 1/N, or a transposed operand in the update."""
    B, N, H, D = 2, 37, 3, 8
    q, k, v = _rand(B, N, H, D)
    eta = 0.7
    o, _ = O.fullbatch(q, k, v, np.zeros((H, D, D)), eta)
    Q, K, V = _heads(q), _heads(k), _heads(v)
    ref = (eta / N) * (Q @ np.swapaxes(K, -1, -2)) @ V
    np.testing.assert_allclose(_heads(o), ref, rtol=0, atol=1e-14)


def _loss_fullbatch_loops(K, V, W):
    """(1/2N) sum_t sum_c ((k_t W)_c - v_tc)^2 with explicit loops (one head)."""
    N, D = K.shape
    tot = 0.0
    for t in range(N):
        pred = [sum(K[t, i] * W[i, c] for i in range(D)) for c in range(D)]
        tot += sum((pred[c] - V[t, c]) ** 2 for c in range(D))
    return tot / (2 * N)


def test_fullbatch_step_is_gradient_of_mean_squared_loss_fd():
    """(W0 - W*)/eta must equal the finite-difference gradient of the mean reconstruction loss.
    Catches a wrong loss scale (1/N vs 2/(N D)), a wrong sign or a transposed gradient."""
    B, N, H, D = 1, 9, 1, 4
    q, k, v = _rand(B, N, H, D, scale=0.5)
    w0 = _w(B, H, D, D, scale=0.3)
    eta = 1.0
    _, W = O.fullbatch(q, k, v, w0, eta)
    K, V, W0 = _heads(k)[0, 0], _heads(v)[0, 0], w0[0]
    h = 1e-6
    fd = np.zeros((D, D))
    for i in range(D):
        for c in range(D):
            Wp, Wm = W0.copy(), W0.copy()
            Wp[i, c] += h
            Wm[i, c] -= h
            fd[i, c] = (_loss_fullbatch_loops(K, V, Wp) - _loss_fullbatch_loops(K, V, Wm)) / (2 * h)
    np.testing.assert_allclose((W0 - W[0, 0]) / eta, fd, rtol=1e-6, atol=1e-9)


def test_fullbatch_step_matches_autograd():
    """Same statement through torch autograd, on a batch of heads and a per-batch W0."""
    B, N, H, D = 2, 50, 2, 16
    q, k, v = _rand(B, N, H, D)
    w0 = _w(B, H, D, D, per_batch=True)
    eta = 1.0
    o, W = O.fullbatch(q, k, v, w0, eta)
    K, V = torch.tensor(_heads(k)), torch.tensor(_heads(v))
    Wt = torch.tensor(w0, requires_grad=True)
    loss = 0.5 * ((K @ Wt - V) ** 2).sum(dim=(-1, -2)) / N
    loss.sum().backward()
    Wref = w0 - eta * Wt.grad.numpy()
    np.testing.assert_allclose(W, Wref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(_heads(o), _heads(q) @ Wref, rtol=0, atol=1e-14)


# ------------------------------------------------------------------ eta = 0 for every variant
@pytest.mark.parametrize("variant", ["fullbatch", "bidir", "causal", "mlp"])
def test_eta_zero_reads_out_initial_state(variant):
    """No learning: O = Q W0 (bidir: both scans read Q W0, so 2 Q W0), MLP: GELU(Q W1) W2.
    Catches readout bugs independent of the update."""
    B, N, H, D = 2, 32, 2, 8
    q, k, v = _rand(B, N, H, D)
    Q = _heads(q)
    if variant == "mlp":
        w1, w2 = _w(B, H, D, 12, 0.3), _w(B, H, 12, D, 0.3)
        o = O.mlp_causal(q, k, v, w1, w2, 0.0, 8)[0]
        ref = O.gelu(Q @ w1) @ w2
    else:
        w0 = _w(B, H, D, D, 0.3)
        if variant == "fullbatch":
            o = O.fullbatch(q, k, v, w0, 0.0)[0]
        elif variant == "bidir":
            o = O.chunked_bidir(q, k, v, w0, 0.0, 8)[0]
        else:
            o = O.chunked_causal(q, k, v, w0, 0.0, 8)[0]
        ref = Q @ w0 * (2.0 if variant == "bidir" else 1.0)
    np.testing.assert_allclose(_heads(o), ref, rtol=0, atol=1e-14)


# ------------------------------------------------------------------ bidirectional
def test_bidir_single_chunk_is_twice_fullbatch():
    """b = N: each scan is one full-batch step on all tokens (order does not matter for a sum),
    so the two directions agree and O = 2 * full-batch O. Catches reading out with the pre-update
    state (the chunk read-out is non-causal, after the update)."""
    B, N, H, D = 2, 48, 2, 16
    q, k, v = _rand(B, N, H, D)
    w0 = _w(B, H, D, D)
    o, wf, wr = O.chunked_bidir(q, k, v, w0, 1.0, N)
    of, w_star = O.fullbatch(q, k, v, w0, 1.0)
    np.testing.assert_allclose(o, 2 * of, rtol=0, atol=1e-14)
    np.testing.assert_allclose(wf, w_star, rtol=0, atol=1e-14)
    np.testing.assert_allclose(wr, w_star, rtol=0, atol=1e-14)


def test_bidir_first_chunk_is_fullbatch_on_that_chunk():
    """The forward scan's first chunk is a full-batch step on its own b tokens, and the reverse scan
    reaches that chunk last, with its end state. So on chunk 0: O = fullbatch(chunk 0) + Q_0 W_rev_end.
    Catches a wrong chunk boundary, divisor, or a reverse output left unflipped."""
    B, N, H, D, b = 1, 40, 2, 8, 8
    q, k, v = _rand(B, N, H, D)
    w0 = _w(B, H, D, D)
    o, _, wr = O.chunked_bidir(q, k, v, w0, 1.0, b)
    of0, _ = O.fullbatch(q[:, :b], k[:, :b], v[:, :b], w0, 1.0)
    rev_part = _heads(o)[:, :, :b] - _heads(of0)
    np.testing.assert_allclose(rev_part, _heads(q)[:, :, :b] @ wr, rtol=0, atol=1e-13)


def test_bidir_reversal_equivariance():
    """Reversing the token order of Q, K, V reverses the output and swaps the two end states."""
    B, N, H, D, b = 2, 64, 2, 8, 16
    q, k, v = _rand(B, N, H, D)
    w0 = _w(B, H, D, D)
    o, wf, wr = O.chunked_bidir(q, k, v, w0, 1.0, b)
    fl = slice(None, None, -1)
    o2, wf2, wr2 = O.chunked_bidir(q[:, fl], k[:, fl], v[:, fl], w0, 1.0, b)
    np.testing.assert_allclose(o2[:, fl], o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(wf2, wr, rtol=0, atol=1e-14)
    np.testing.assert_allclose(wr2, wf, rtol=0, atol=1e-14)


def test_bidir_permutation_inside_chunk_equivariance():
    """Non-causal inside a chunk: permuting tokens within each chunk permutes the output the same way.
    Catches an accidental causal mask or per-token state in the bidirectional path."""
    B, N, H, D, b = 1, 48, 2, 8, 16
    q, k, v = _rand(B, N, H, D)
    w0 = _w(B, H, D, D)
    perm = np.concatenate([c * b + RNG.permutation(b) for c in range(N // b)])
    o = O.chunked_bidir(q, k, v, w0, 1.0, b)[0]
    op = O.chunked_bidir(q[:, perm], k[:, perm], v[:, perm], w0, 1.0, b)[0]
    np.testing.assert_allclose(op, o[:, perm], rtol=0, atol=1e-14)


# ------------------------------------------------------------------ causal TTT-Linear
def test_causal_chunk_one_is_delta_rule():
    """b = 1: the per-token delta rule W_i = W_{i-1} - eta k_i^T (k_i W_{i-1} - v_i), o_i = q_i W_i."""
    B, N, H, D = 2, 30, 2, 8
    q, k, v = _rand(B, N, H, D)
    w0 = _w(B, H, D, D)
    eta = 0.9
    o, wend = O.chunked_causal(q, k, v, w0, eta, 1)
    for bb in range(B):
        for h in range(H):
            W = w0[h].copy()
            for i in range(N):
                ki, vi, qi = k[bb, i, h], v[bb, i, h], q[bb, i, h]
                W = W - eta * np.outer(ki, ki @ W - vi)
                np.testing.assert_allclose(o[bb, i, h], qi @ W, rtol=0, atol=1e-14)
            np.testing.assert_allclose(wend[bb, h], W, rtol=0, atol=1e-14)


def test_causal_primal_equals_dual_form():
    """Dual form of one causal chunk: O_c = Q_c W_s - (eta/b) tril(Q_c K_c^T) (K_c W_s - V_c),
    W_next = W_s - (eta/b) K_c^T (K_c W_s - V_c) (diagonal included). Catches an exclusive mask
    (token not seeing its own gradient) or a running-count divisor."""
    B, N, H, D, b = 2, 64, 3, 16, 16
    q, k, v = _rand(B, N, H, D)
    w0 = _w(B, H, D, D)
    eta = 1.0
    o, wend = O.chunked_causal(q, k, v, w0, eta, b)
    Q, K, V = _heads(q), _heads(k), _heads(v)
    W = np.broadcast_to(w0, (B,) + w0.shape).copy()
    a = eta / b
    ref = np.empty_like(Q)
    mask = np.tril(np.ones((b, b)))
    for c0 in range(0, N, b):
        Qc, Kc, Vc = Q[:, :, c0:c0 + b], K[:, :, c0:c0 + b], V[:, :, c0:c0 + b]
        E = Kc @ W - Vc
        ref[:, :, c0:c0 + b] = Qc @ W - a * ((Qc @ np.swapaxes(Kc, -1, -2)) * mask) @ E
        W = W - a * np.swapaxes(Kc, -1, -2) @ E
    np.testing.assert_allclose(_heads(o), ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(wend, W, rtol=0, atol=1e-13)


def test_causal_matches_autograd_per_token():
    """Token i uses W_s - (eta/b) sum_{j<=i} grad l_j(W_s), with the gradients from torch autograd."""
    B, N, H, D, b = 1, 16, 1, 8, 8
    q, k, v = _rand(B, N, H, D)
    w0 = _w(B, H, D, D, scale=0.2)
    eta = 1.0
    o, _ = O.chunked_causal(q, k, v, w0, eta, b)
    W = torch.tensor(w0[0])
    for c0 in range(0, N, b):
        grads = []
        for j in range(c0, c0 + b):
            Wj = W.clone().requires_grad_(True)
            kj, vj = torch.tensor(k[0, j, 0]), torch.tensor(v[0, j, 0])
            (0.5 * ((kj @ Wj - vj) ** 2).sum()).backward()
            grads.append(Wj.grad)
        acc = torch.zeros_like(W)
        for i in range(c0, c0 + b):
            acc = acc + grads[i - c0]
            ref = torch.tensor(q[0, i, 0]) @ (W - eta / b * acc)
            np.testing.assert_allclose(o[0, i, 0], ref.numpy(), rtol=0, atol=1e-14)
        W = W - eta / b * acc


@pytest.mark.parametrize("variant", ["causal", "mlp", "bidir_fwd_state"])
def test_state_carry_split_equals_one_call(variant):
    """Running N tokens equals N/2 tokens, then N/2 more from the carried end state."""
    B, N, H, D, b = 2, 64, 2, 8, 16
    q, k, v = _rand(B, N, H, D)
    h2 = N // 2
    if variant == "mlp":
        w1, w2 = _w(B, H, D, 12, 0.3), _w(B, H, 12, D, 0.3)
        o, e1, e2 = O.mlp_causal(q, k, v, w1, w2, 1.0, b)
        oa, m1, m2 = O.mlp_causal(q[:, :h2], k[:, :h2], v[:, :h2], w1, w2, 1.0, b)
        ob, f1, f2 = O.mlp_causal(q[:, h2:], k[:, h2:], v[:, h2:], m1, m2, 1.0, b)
        np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, rtol=0, atol=1e-14)
        np.testing.assert_allclose(f1, e1, rtol=0, atol=1e-14)
        np.testing.assert_allclose(f2, e2, rtol=0, atol=1e-14)
        return
    w0 = _w(B, H, D, D)
    if variant == "causal":
        o, e = O.chunked_causal(q, k, v, w0, 1.0, b)
        oa, m = O.chunked_causal(q[:, :h2], k[:, :h2], v[:, :h2], w0, 1.0, b)
        ob, f = O.chunked_causal(q[:, h2:], k[:, h2:], v[:, h2:], m, 1.0, b)
        np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, rtol=0, atol=1e-14)
        np.testing.assert_allclose(f, e, rtol=0, atol=1e-14)
    else:
        _, wf, _ = O.chunked_bidir(q, k, v, w0, 1.0, b)
        _, m, _ = O.chunked_bidir(q[:, :h2], k[:, :h2], v[:, :h2], w0, 1.0, b)
        _, f, _ = O.chunked_bidir(q[:, h2:], k[:, h2:], v[:, h2:], m, 1.0, b)
        np.testing.assert_allclose(f, wf, rtol=0, atol=1e-14)


# ------------------------------------------------------------------ TTT-MLP
def test_gelu_against_torch_and_identities():
    """GELU is the exact erf form (torch's approximate='none'); GELU' matches finite differences
    and torch autograd; gelu(x) - gelu(-x) = x."""
    x = np.linspace(-6, 6, 2001)
    xt = torch.tensor(x, requires_grad=True)
    y = torch.nn.functional.gelu(xt, approximate="none")
    y.sum().backward()
    np.testing.assert_allclose(O.gelu(x), y.detach().numpy(), rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.gelu_prime(x), xt.grad.numpy(), rtol=0, atol=1e-14)
    h = 1e-5
    np.testing.assert_allclose(O.gelu_prime(x), (O.gelu(x + h) - O.gelu(x - h)) / (2 * h), rtol=0, atol=1e-9)
    np.testing.assert_allclose(O.gelu(x) - O.gelu(-x), x, rtol=0, atol=1e-14)
    assert O.gelu(0.0) == 0.0 and O.gelu_prime(0.0) == 0.5


def _mlp_loss(k, v, W1, W2):
    return 0.5 * float(np.sum((O.gelu(k @ W1) @ W2 - v) ** 2))


def test_mlp_token_grad_finite_difference():
    """Hand-derived TTT-MLP gradients against central finite differences (d = 8, Dh = 12)."""
    D, Dh = 8, 12
    k = RNG.standard_normal((1, D))
    v = RNG.standard_normal((1, D))
    W1 = RNG.standard_normal((D, Dh)) * 0.5
    W2 = RNG.standard_normal((Dh, D)) * 0.5
    g1, g2 = O.mlp_token_grad(k, v, W1, W2)
    h = 1e-6
    for W, g in ((W1, g1), (W2, g2)):
        fd = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            old = W[idx]
            W[idx] = old + h
            lp = _mlp_loss(k, v, W1, W2)
            W[idx] = old - h
            lm = _mlp_loss(k, v, W1, W2)
            W[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_mlp_causal_matches_autograd_per_token():
    """Token i is read out with (W1_s, W2_s) - (eta/b) sum_{j<=i} grad l_j, gradients from autograd."""
    B, N, H, D, Dh, b = 1, 8, 1, 4, 6, 4
    q, k, v = _rand(B, N, H, D, scale=0.7)
    w1, w2 = _w(B, H, D, Dh, 0.5), _w(B, H, Dh, D, 0.5)
    eta = 1.0
    o, e1, e2 = O.mlp_causal(q, k, v, w1, w2, eta, b)
    W1, W2 = torch.tensor(w1[0]), torch.tensor(w2[0])
    gelu = lambda t: torch.nn.functional.gelu(t, approximate="none")  # noqa: E731
    for c0 in range(0, N, b):
        A1, A2 = torch.zeros_like(W1), torch.zeros_like(W2)
        for i in range(c0, c0 + b):
            a1, a2 = W1.clone().requires_grad_(True), W2.clone().requires_grad_(True)
            kk, vv = torch.tensor(k[0, i, 0]), torch.tensor(v[0, i, 0])
            (0.5 * ((gelu(kk @ a1) @ a2 - vv) ** 2).sum()).backward()
            A1, A2 = A1 + a1.grad, A2 + a2.grad
            ref = gelu(torch.tensor(q[0, i, 0]) @ (W1 - eta / b * A1)) @ (W2 - eta / b * A2)
            np.testing.assert_allclose(o[0, i, 0], ref.numpy(), rtol=0, atol=1e-14)
        W1, W2 = W1 - eta / b * A1, W2 - eta / b * A2
    np.testing.assert_allclose(e1[0, 0], W1.numpy(), rtol=0, atol=1e-14)
    np.testing.assert_allclose(e2[0, 0], W2.numpy(), rtol=0, atol=1e-14)


def test_mlp_primal_equals_dual_form():
    """Dual form of one TTT-MLP chunk (all gradients at the chunk start):
    Z1 = K W1, X2 = GELU(Z1), E = X2 W2 - V, D1 = (E W2^T) * GELU'(Z1);
    Z1q = Q W1 - a tril(Q K^T) D1; X2q = GELU(Z1q); O = X2q W2 - a tril(X2q X2^T) E;
    W1 -= a K^T D1; W2 -= a X2^T E."""
    B, N, H, D, Dh, b = 2, 48, 2, 8, 24, 16
    q, k, v = _rand(B, N, H, D)
    w1, w2 = _w(B, H, D, Dh, 0.2), _w(B, H, Dh, D, 0.2)
    eta = 1.0
    o, e1, e2 = O.mlp_causal(q, k, v, w1, w2, eta, b)
    Q, K, V = _heads(q), _heads(k), _heads(v)
    W1 = np.broadcast_to(w1, (B,) + w1.shape).copy()
    W2 = np.broadcast_to(w2, (B,) + w2.shape).copy()
    a = eta / b
    T = lambda x: np.swapaxes(x, -1, -2)  # noqa: E731
    mask = np.tril(np.ones((b, b)))
    ref = np.empty_like(Q)
    for c0 in range(0, N, b):
        Qc, Kc, Vc = Q[:, :, c0:c0 + b], K[:, :, c0:c0 + b], V[:, :, c0:c0 + b]
        Z1 = Kc @ W1
        X2 = O.gelu(Z1)
        E = X2 @ W2 - Vc
        D1 = (E @ T(W2)) * O.gelu_prime(Z1)
        Z1q = Qc @ W1 - a * ((Qc @ T(Kc)) * mask) @ D1
        X2q = O.gelu(Z1q)
        ref[:, :, c0:c0 + b] = X2q @ W2 - a * ((X2q @ T(X2)) * mask) @ E
        W1 = W1 - a * T(Kc) @ D1
        W2 = W2 - a * T(X2) @ E
    np.testing.assert_allclose(_heads(o), ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(e1, W1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(e2, W2, rtol=0, atol=1e-13)


# ------------------------------------------------------------------ exact arithmetic on tiny inputs
def _fmat(a):
    return [[Fraction(int(x)) for x in row] for row in a]


def _mm(A, B):
    return [[sum(A[i][t] * B[t][j] for t in range(len(B))) for j in range(len(B[0]))] for i in range(len(A))]


def _sub(A, B, s=Fraction(1)):
    return [[A[i][j] - s * B[i][j] for j in range(len(A[0]))] for i in range(len(A))]


def _tr(A):
    return [list(r) for r in zip(*A)]


def test_exact_rational_tiny_cases():
    """Small integer inputs with eta = 1 make every result rational. Evaluated exactly with Fractions,
    token by token (delta-style accumulation for causal, explicit chunk loop for the bidir scan), the
    fp64 oracle must agree to rounding. Catches indexing mistakes that symmetric random data hides."""
    rs = np.random.default_rng(5)
    N, D, b = 6, 3, 2
    Qi, Ki, Vi = (rs.integers(-3, 4, (N, D)) for _ in range(3))
    W0i = rs.integers(-2, 3, (D, D))
    q, k, v = (x.reshape(1, N, 1, D).astype(np.float64) for x in (Qi, Ki, Vi))
    w0 = W0i.reshape(1, D, D).astype(np.float64)
    Q, K, V, W0 = _fmat(Qi), _fmat(Ki), _fmat(Vi), _fmat(W0i)
    # full batch
    E = _sub(_mm(K, W0), V)
    Wst = _sub(W0, _mm(_tr(K), E), Fraction(1, N))
    ref = _mm(Q, Wst)
    got = O.fullbatch(q, k, v, w0, 1.0)[0][0, :, 0]
    np.testing.assert_allclose(got, np.array(ref, dtype=float), rtol=1e-13, atol=1e-12)
    # causal, b = 2: token by token with the chunk-start state
    W = W0
    ref = []
    for c0 in range(0, N, b):
        S = [[Fraction(0)] * D for _ in range(D)]
        for i in range(c0, c0 + b):
            ki, vi = [K[i]], [V[i]]
            S = _sub(S, _mm(_tr(ki), _sub(_mm(ki, W), vi)), Fraction(-1))
            ref.append(_mm([Q[i]], _sub(W, S, Fraction(1, b)))[0])
        W = _sub(W, S, Fraction(1, b))
    got = O.chunked_causal(q, k, v, w0, 1.0, b)[0][0, :, 0]
    np.testing.assert_allclose(got, np.array(ref, dtype=float), rtol=1e-12, atol=1e-10)
    # bidirectional, b = 2
    def scan(order):
        W = W0
        out = {}
        for c in range(0, N, b):
            idx = order[c:c + b]
            Kc, Vc = [K[i] for i in idx], [V[i] for i in idx]
            W = _sub(W, _mm(_tr(Kc), _sub(_mm(Kc, W), Vc)), Fraction(1, b))
            for i in idx:
                out[i] = _mm([Q[i]], W)[0]
        return out
    f, r = scan(list(range(N))), scan(list(range(N))[::-1])
    ref = [[f[i][j] + r[i][j] for j in range(D)] for i in range(N)]
    got = O.chunked_bidir(q, k, v, w0, 1.0, b)[0][0, :, 0]
    np.testing.assert_allclose(got, np.array(ref, dtype=float), rtol=1e-12, atol=1e-9)


def test_oracle_rejects_ragged_chunking():
    q, k, v = _rand(1, 10, 1, 4)
    with pytest.raises(ValueError):
        O.chunked_causal(q, k, v, np.zeros((1, 4, 4)), 1.0, 4)


def test_run_dispatch_on_workload_inputs():
    """oracle.run on a generated workload equals calling the variant directly."""
    wl = synth.WORKLOADS["fullbatch_tiny_fp32"]
    x = synth.make_inputs(wl)
    np.testing.assert_array_equal(O.run(x), O.fullbatch(x.q64, x.k64, x.v64, x.w0, 1.0)[0])
