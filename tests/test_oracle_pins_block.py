"""Pins of the ViT^3 block-epilogue oracle (no GPU)."""
import numpy as np
import torch

from oracle.block_oracle import block_epilogue

RNG = np.random.default_rng(53)


def _case(M=37, C=12, Co=10):
    return (RNG.standard_normal((M, C)), RNG.standard_normal((M, C)), RNG.standard_normal((M, C)),
            RNG.standard_normal((Co, 2 * C)), RNG.standard_normal(Co))


def test_matches_torch_glu_and_linear():
    """torch.nn.functional.glu on [O, G] (O * sigmoid(G)), concatenated with X, through
    torch.nn.functional.linear, in float64."""
    o, g, x, w, b = _case()
    t = lambda a: torch.from_numpy(a)  # noqa: E731
    main = torch.nn.functional.glu(torch.cat([t(o), t(g)], dim=-1), dim=-1)
    ref = torch.nn.functional.linear(torch.cat([main, t(x)], dim=-1), t(w), t(b)).numpy()
    np.testing.assert_allclose(block_epilogue(o, g, x, w, b), ref, atol=1e-12)


def test_projection_splits_into_the_two_branches():
    """The first C input columns of the projection act on the gated main branch only, the last C on
    the convolution branch only (catches a swapped concatenation or a transposed weight)."""
    o, g, x, w, _ = _case()
    C = o.shape[1]
    w_main = w.copy()
    w_main[:, C:] = 0
    w_conv = w.copy()
    w_conv[:, :C] = 0
    both = block_epilogue(o, g, x, w, None)
    np.testing.assert_allclose(block_epilogue(o, g, x, w_main, None) + block_epilogue(o, g, x, w_conv, None), both,
                               atol=1e-12)
    assert np.abs(block_epilogue(o, g, np.zeros_like(x), w_conv, None)).max() == 0


def test_saturated_and_zero_gate():
    """A gate of +60 passes O through, -60 closes it, 0 halves it."""
    o, _, x, w, b = _case()
    C = o.shape[1]
    open_ = block_epilogue(o, np.full_like(o, 60.0), x, w, b)
    np.testing.assert_allclose(open_, np.concatenate([o, x], -1) @ w.T + b, atol=1e-12)
    closed = block_epilogue(o, np.full_like(o, -60.0), x, w, b)
    np.testing.assert_allclose(closed, x @ w[:, C:].T + b, atol=1e-12)
    half = block_epilogue(o, np.zeros_like(o), x, w, None)
    np.testing.assert_allclose(half, np.concatenate([o / 2, x], -1) @ w.T, atol=1e-12)
