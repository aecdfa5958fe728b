"""Pins of the depth-wise 3x3 convolution oracle (no GPU). Each test names the mistake it catches."""
import numpy as np
import pytest
import torch

from oracle.dwconv_oracle import dwconv3x3

RNG = np.random.default_rng(7)


def _case(B=2, Hi=5, Wi=7, C=6):
    return RNG.standard_normal((B, Hi * Wi, C)), RNG.standard_normal((C, 3, 3)), RNG.standard_normal(C), Hi, Wi


def test_identity_kernel():
    """Centre tap 1, bias 0: the output is the input (catches an off-by-one in the window)."""
    x, _, _, Hi, Wi = _case()
    w = np.zeros((x.shape[2], 3, 3))
    w[:, 1, 1] = 1.0
    assert np.array_equal(dwconv3x3(x, w, None, Hi, Wi), x)


@pytest.mark.parametrize("u,v", [(0, 0), (0, 2), (2, 1), (1, 0)])
def test_single_tap_is_a_shift_with_zero_padding(u, v):
    """One tap w[u, v] = 1: y[i, j] = x[i + u - 1, j + v - 1], zero where that leaves the image.
    Pins the orientation (cross-correlation, not a flipped kernel), the row/column order of the
    taps and the zero padding."""
    x, _, _, Hi, Wi = _case()
    C = x.shape[2]
    w = np.zeros((C, 3, 3))
    w[:, u, v] = 1.0
    img = x.reshape(2, Hi, Wi, C)
    ref = np.zeros_like(img)
    for i in range(Hi):
        for j in range(Wi):
            ii, jj = i + u - 1, j + v - 1
            if 0 <= ii < Hi and 0 <= jj < Wi:
                ref[:, i, j] = img[:, ii, jj]
    assert np.array_equal(dwconv3x3(x, w, None, Hi, Wi), ref.reshape(x.shape))


def test_matches_torch_grouped_convolution():
    """torch's Conv2d with groups = channels and padding 1 (the library routine of the convolution
    layer) in float64."""
    x, w, b, Hi, Wi = _case(B=3, Hi=6, Wi=4, C=5)
    B, N, C = x.shape
    xt = torch.from_numpy(x.reshape(B, Hi, Wi, C)).permute(0, 3, 1, 2)
    ref = torch.nn.functional.conv2d(xt, torch.from_numpy(w)[:, None], torch.from_numpy(b), padding=1, groups=C)
    ref = ref.permute(0, 2, 3, 1).reshape(B, N, C).numpy()
    np.testing.assert_allclose(dwconv3x3(x, w, b, Hi, Wi), ref, rtol=0, atol=1e-13)


def test_linear_in_input_and_weights():
    """Without bias the convolution is linear in x and in w (catches a squared term or a stray
    constant)."""
    x1, w1, _, Hi, Wi = _case()
    x2, w2, _, _, _ = _case()
    a, c = 0.75, -1.5
    np.testing.assert_allclose(dwconv3x3(a * x1 + c * x2, w1, None, Hi, Wi),
                               a * dwconv3x3(x1, w1, None, Hi, Wi) + c * dwconv3x3(x2, w1, None, Hi, Wi), atol=1e-13)
    np.testing.assert_allclose(dwconv3x3(x1, a * w1 + c * w2, None, Hi, Wi),
                               a * dwconv3x3(x1, w1, None, Hi, Wi) + c * dwconv3x3(x1, w2, None, Hi, Wi), atol=1e-13)


def test_shift_equivariance_in_the_interior():
    """Shifting the image by one row and one column shifts the output, away from the borders
    (catches a position-dependent weight or a wrong row stride)."""
    x, w, b, Hi, Wi = _case(B=1, Hi=8, Wi=9, C=3)
    img = x.reshape(1, Hi, Wi, 3)
    sh = np.roll(img, (1, 1), axis=(1, 2))
    y = dwconv3x3(x, w, b, Hi, Wi).reshape(1, Hi, Wi, 3)
    ys = dwconv3x3(sh.reshape(x.shape), w, b, Hi, Wi).reshape(1, Hi, Wi, 3)
    np.testing.assert_allclose(ys[:, 2:-1, 2:-1], y[:, 1:-2, 1:-2], atol=1e-13)


def test_channels_are_independent():
    """Changing one channel of the input changes only that channel of the output (depth-wise)."""
    x, w, b, Hi, Wi = _case()
    x2 = x.copy()
    x2[:, :, 3] += RNG.standard_normal(x.shape[1])
    d = dwconv3x3(x2, w, b, Hi, Wi) - dwconv3x3(x, w, b, Hi, Wi)
    assert np.abs(np.delete(d, 3, axis=2)).max() == 0.0
    assert np.abs(d[:, :, 3]).max() > 0


def test_brute_force_loops_on_a_tiny_grid():
    """Every output element by explicit loops over the 3 x 3 taps."""
    x, w, b, Hi, Wi = _case(B=1, Hi=3, Wi=4, C=2)
    img = x.reshape(Hi, Wi, 2)
    ref = np.zeros((Hi, Wi, 2))
    for i in range(Hi):
        for j in range(Wi):
            for c in range(2):
                s = b[c]
                for u in range(3):
                    for v in range(3):
                        ii, jj = i + u - 1, j + v - 1
                        if 0 <= ii < Hi and 0 <= jj < Wi:
                            s += w[c, u, v] * img[ii, jj, c]
                ref[i, j, c] = s
    np.testing.assert_allclose(dwconv3x3(x, w, b, Hi, Wi), ref.reshape(1, Hi * Wi, 2), atol=1e-14)


def test_rejects_a_token_count_that_is_not_the_grid():
    x, w, b, _, _ = _case()
    with pytest.raises(ValueError):
        dwconv3x3(x, w, b, 4, 7)
