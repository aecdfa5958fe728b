"""Pins of the multi-epoch full-batch oracle (no GPU)."""
import numpy as np
import pytest

from oracle import ttt_oracle as O

RNG = np.random.default_rng(11)


def _qkv(B, N, H, D):
    return [RNG.standard_normal((B, N, H, D)) / np.sqrt(D) for _ in range(3)]


def test_one_epoch_is_the_full_batch_step():
    q, k, v = _qkv(2, 40, 3, 8)
    w0 = RNG.standard_normal((3, 8, 8)) * 0.02
    o1, w1 = O.fullbatch_epochs(q, k, v, w0, 0.8, 1)
    o, w = O.fullbatch(q, k, v, w0, 0.8)
    np.testing.assert_allclose(o1, o, rtol=0, atol=1e-15)
    np.testing.assert_allclose(w1, w, rtol=0, atol=1e-15)


@pytest.mark.parametrize("epochs", [2, 3, 7])
def test_closed_form_with_orthogonal_keys(epochs):
    """K with orthogonal columns of squared norm c (K^T K = c I): each epoch contracts the distance
    to the solution K^T V / c by (1 - s c), s = eta / N, so
    W_E = (1 - s c)^E W0 + (1 - (1 - s c)^E) K^T V / c. Catches a missing epoch, a wrong step
    size or a step taken from W0 instead of the previous epoch."""
    N, D, eta = 32, 8, 1.0
    c = 5.0
    Qm, _ = np.linalg.qr(RNG.standard_normal((N, D)))
    K = np.sqrt(c) * Qm
    V = RNG.standard_normal((N, D))
    W0 = RNG.standard_normal((D, D))
    q = RNG.standard_normal((1, N, 1, D))
    o, w = O.fullbatch_epochs(q, K[None, :, None], V[None, :, None], W0[None], eta, epochs)
    r = (1 - eta / N * c) ** epochs
    ref = r * W0 + (1 - r) * (K.T @ V) / c
    np.testing.assert_allclose(w[0, 0], ref, atol=1e-12)
    np.testing.assert_allclose(o[0, :, 0], q[0, :, 0] @ ref, atol=1e-12)


def test_many_epochs_converge_to_least_squares():
    """With a step below 2 / lambda_max(K^T K / N), the epochs converge to the least-squares fit
    of V by K (numpy's lstsq), whatever W0."""
    N, D = 64, 6
    K = RNG.standard_normal((N, D))
    V = RNG.standard_normal((N, D))
    lam = np.linalg.eigvalsh(K.T @ K / N).max()
    eta = 1.0 / lam
    _, w = O.fullbatch_epochs(np.zeros((1, N, 1, D)), K[None, :, None], V[None, :, None],
                              RNG.standard_normal((1, D, D)), eta, 3000)
    np.testing.assert_allclose(w[0, 0], np.linalg.lstsq(K, V, rcond=None)[0], atol=1e-9)


def test_epochs_must_be_positive():
    q, k, v = _qkv(1, 8, 1, 4)
    with pytest.raises(ValueError):
        O.fullbatch_epochs(q, k, v, np.zeros((1, 4, 4)), 1.0, 0)
