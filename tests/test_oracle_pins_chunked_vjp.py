"""Pins of the chunked backward (vector-Jacobian product) oracles, causal and bidirectional:
central finite differences of the forward oracles, torch autograd of the layers written in their
dual (matrix) form, the eta = 0 closed form, and the one-chunk case, which is the full-batch layer
(whose gradients are pinned on their own)."""
import numpy as np
import pytest
import torch

from oracle import ttt_oracle as O

RNG = np.random.default_rng(31)


def _case(B=2, N=12, H=2, D=5):
    q, k, v = [RNG.standard_normal((B, N, H, D)) / np.sqrt(D) for _ in range(3)]
    w0 = RNG.standard_normal((B, H, D, D)) * 0.3
    d_o = RNG.standard_normal((B, N, H, D))
    return q, k, v, w0, d_o


FWD = {"causal": O.chunked_causal, "bidir": O.chunked_bidir}
VJP = {"causal": O.chunked_causal_vjp, "bidir": O.chunked_bidir_vjp}


@pytest.mark.parametrize("kind", ["causal", "bidir"])
@pytest.mark.parametrize("chunk", [1, 3, 4])
@pytest.mark.parametrize("which", [0, 1, 2, 3])
def test_directional_finite_differences(kind, chunk, which):
    """<grad, delta> equals the central difference of L = <dO, O> along a random delta, for each
    input and several chunk sizes (a wrong sign, a transposed factor, a dropped term or a wrong
    mask in any gradient changes the directional derivative)."""
    q, k, v, w0, d_o = _case()
    eta = 0.8
    args = [q, k, v, w0]
    grads = VJP[kind](q, k, v, w0, eta, chunk, d_o)
    delta = RNG.standard_normal(args[which].shape)
    h = 1e-6

    def L(x):
        a = list(args)
        a[which] = x
        return float(np.sum(d_o * FWD[kind](*a, eta, chunk)[0]))

    fd = (L(args[which] + h * delta) - L(args[which] - h * delta)) / (2 * h)
    np.testing.assert_allclose(np.sum(grads[which] * delta), fd, rtol=1e-7, atol=1e-9)


def _dual_scan(Q, K, V, W0, eta, b, causal):
    """One scan direction in the dual form, in torch: per chunk E = K W - V, O = Q W - a M(Q K^T) E
    with M the lower-triangular mask (causal) or all ones (read-out after the update)."""
    N = Q.shape[2]
    a = eta / b
    W = W0
    outs = []
    mask = torch.tril(torch.ones(b, b, dtype=Q.dtype)) if causal else torch.ones(b, b, dtype=Q.dtype)
    for c0 in range(0, N, b):
        Qc, Kc, Vc = Q[:, :, c0:c0 + b], K[:, :, c0:c0 + b], V[:, :, c0:c0 + b]
        E = Kc @ W - Vc
        outs.append(Qc @ W - a * ((Qc @ Kc.transpose(-1, -2)) * mask) @ E)
        W = W - a * Kc.transpose(-1, -2) @ E
    return torch.cat(outs, dim=2)


@pytest.mark.parametrize("kind", ["causal", "bidir"])
def test_matches_torch_autograd_of_dual_form(kind):
    """torch autograd (float64) of the layer written in the dual form, an algebra the oracle does
    not use (it runs the primal per-token loop)."""
    q, k, v, w0, d_o = _case(B=1, N=16, H=2, D=4)
    eta, chunk = 1.1, 4
    tq, tk, tv, tw = [torch.tensor(x, requires_grad=True) for x in (q, k, v, w0)]
    Q, K, V = [t.permute(0, 2, 1, 3) for t in (tq, tk, tv)]
    if kind == "causal":
        out = _dual_scan(Q, K, V, tw, eta, chunk, True)
    else:
        rev = torch.arange(Q.shape[2] - 1, -1, -1)
        out = _dual_scan(Q, K, V, tw, eta, chunk, False) + \
            _dual_scan(Q[:, :, rev], K[:, :, rev], V[:, :, rev], tw, eta, chunk, False)[:, :, rev]
    (out.permute(0, 2, 1, 3) * torch.tensor(d_o)).sum().backward()
    got = VJP[kind](q, k, v, w0, eta, chunk, d_o)
    for g, t in zip(got, (tq, tk, tv, tw)):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("kind", ["causal", "bidir"])
def test_eta_zero(kind):
    """eta = 0: every output is q W0 (once per scan direction), so dQ = n dO W0^T and dW0 = n Q^T dO
    (n = 1 causal, 2 bidirectional) and dK = dV = 0."""
    q, k, v, w0, d_o = _case()
    n = 1 if kind == "causal" else 2
    dq, dk, dv, dw0 = VJP[kind](q, k, v, w0, 0.0, 4, d_o)
    Qh, dOh = np.transpose(q, (0, 2, 1, 3)), np.transpose(d_o, (0, 2, 1, 3))
    np.testing.assert_allclose(np.transpose(dq, (0, 2, 1, 3)), n * dOh @ np.swapaxes(w0, -1, -2), atol=1e-13)
    np.testing.assert_allclose(dw0, n * np.swapaxes(Qh, -1, -2) @ dOh, atol=1e-12)
    assert np.abs(dk).max() == 0 and np.abs(dv).max() == 0


def test_bidir_one_chunk_is_twice_fullbatch():
    """With a single chunk both directions are the full-batch layer (read-out after one step on
    all tokens), so the gradients are twice fullbatch_vjp's."""
    q, k, v, w0, d_o = _case(N=8)
    eta = 0.7
    got = O.chunked_bidir_vjp(q, k, v, w0, eta, 8, d_o)
    ref = O.fullbatch_vjp(q, k, v, w0, eta, d_o)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, 2 * r, rtol=1e-12, atol=1e-13)


def test_linear_in_d_o():
    """The gradients are linear in dO."""
    q, k, v, w0, d_o = _case()
    d2 = RNG.standard_normal(d_o.shape)
    g1 = O.chunked_causal_vjp(q, k, v, w0, 0.9, 3, d_o)
    g2 = O.chunked_causal_vjp(q, k, v, w0, 0.9, 3, d2)
    g12 = O.chunked_causal_vjp(q, k, v, w0, 0.9, 3, 2 * d_o - d2)
    for a, b, c in zip(g1, g2, g12):
        np.testing.assert_allclose(c, 2 * a - b, rtol=1e-11, atol=1e-12)
