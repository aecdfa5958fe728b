"""Pins of the full-batch backward (vector-Jacobian product) oracle: central finite differences of
the forward oracle, torch autograd of the forward definition, and the eta = 0 special case."""
import numpy as np
import pytest
import torch

from oracle import ttt_oracle as O

RNG = np.random.default_rng(29)


def _case(B=2, N=23, H=2, D=5):
    q, k, v = [RNG.standard_normal((B, N, H, D)) / np.sqrt(D) for _ in range(3)]
    w0 = RNG.standard_normal((B, H, D, D)) * 0.3
    d_o = RNG.standard_normal((B, N, H, D))
    return q, k, v, w0, d_o


@pytest.mark.parametrize("which", [0, 1, 2, 3])
def test_directional_finite_differences(which):
    """<grad, delta> equals the central difference of L = <dO, O> along a random delta, for each
    input (catches a wrong sign, a transposed factor or a missing term in any gradient)."""
    q, k, v, w0, d_o = _case()
    eta = 0.9
    args = [q, k, v, w0]
    grads = O.fullbatch_vjp(q, k, v, w0, eta, d_o)
    delta = RNG.standard_normal(args[which].shape)
    h = 1e-6

    def L(x):
        a = list(args)
        a[which] = x
        return float(np.sum(d_o * O.fullbatch(*a, eta)[0]))

    fd = (L(args[which] + h * delta) - L(args[which] - h * delta)) / (2 * h)
    np.testing.assert_allclose(np.sum(grads[which] * delta), fd, rtol=1e-7, atol=1e-9)


def test_matches_torch_autograd():
    """torch autograd (float64) of the forward definition W* = W0 - (eta/N) K^T (K W0 - V),
    O = Q W*, for L = <dO, O>."""
    q, k, v, w0, d_o = _case(B=1, N=17, H=3, D=4)
    eta = 1.3
    tq, tk, tv, tw = [torch.tensor(a, requires_grad=True) for a in (q, k, v, w0)]
    Q, K, V = [t.permute(0, 2, 1, 3) for t in (tq, tk, tv)]
    N = q.shape[1]
    Ws = tw - (eta / N) * K.transpose(-1, -2) @ (K @ tw - V)
    O_ = (Q @ Ws).permute(0, 2, 1, 3)
    (O_ * torch.tensor(d_o)).sum().backward()
    got = O.fullbatch_vjp(q, k, v, w0, eta, d_o)
    for g, t in zip(got, (tq, tk, tv, tw)):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_eta_zero():
    """eta = 0: O = Q W0, so only dQ = dO W0^T and dW0 = Q^T dO are nonzero."""
    q, k, v, w0, d_o = _case()
    dq, dk, dv, dw0 = O.fullbatch_vjp(q, k, v, w0, 0.0, d_o)
    Qh, dOh = np.transpose(q, (0, 2, 1, 3)), np.transpose(d_o, (0, 2, 1, 3))
    np.testing.assert_allclose(np.transpose(dq, (0, 2, 1, 3)), dOh @ np.swapaxes(w0, -1, -2), atol=1e-14)
    np.testing.assert_allclose(dw0, np.swapaxes(Qh, -1, -2) @ dOh, atol=1e-13)
    assert np.abs(dk).max() == 0 and np.abs(dv).max() == 0
