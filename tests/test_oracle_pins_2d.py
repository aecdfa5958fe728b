"""Pins of the 2-D bidirectional scan oracle (raster-order plus column-order bidirectional scans)."""
import numpy as np
import pytest

from oracle import ttt_oracle as O

RNG = np.random.default_rng(41)


def _qkv(B, N, H, D):
    return [RNG.standard_normal((B, N, H, D)) / np.sqrt(D) for _ in range(3)]


def test_grid_transpose_by_index():
    """Token (i, j) of a height x width grid moves from raster index i * width + j to column index
    j * height + i; transposing twice is the identity."""
    B, Hg, Wg = 2, 3, 5
    x = RNG.standard_normal((B, Hg * Wg, 4))
    t = O.grid_transpose(x, Hg, Wg)
    for i in range(Hg):
        for j in range(Wg):
            assert np.array_equal(t[:, j * Hg + i], x[:, i * Wg + j])
    assert np.array_equal(O.grid_transpose(t, Wg, Hg), x)


def test_one_row_image_scans_the_same_order_twice():
    """A 1 x W image: the column order is the raster order, so the output is twice the
    bidirectional scan's."""
    q, k, v = _qkv(2, 32, 2, 4)
    w0 = RNG.standard_normal((2, 4, 4)) * 0.1
    o2d, _ = O.chunked_bidir_2d(q, k, v, w0, 0.7, 8, 1, 32)
    o, _, _ = O.chunked_bidir(q, k, v, w0, 0.7, 8)
    np.testing.assert_allclose(o2d, 2 * o, atol=1e-14)


def test_transposed_image_gives_the_transposed_output():
    """Scanning the transposed image (width x height) swaps the raster and column scans, so the
    output is the transposed output (catches a transposition in the wrong direction)."""
    Hg, Wg = 4, 6
    q, k, v = _qkv(1, Hg * Wg, 2, 4)
    w0 = RNG.standard_normal((2, 4, 4)) * 0.1
    o, _ = O.chunked_bidir_2d(q, k, v, w0, 0.9, 4, Hg, Wg)
    tq, tk, tv = (O.grid_transpose(t, Hg, Wg) for t in (q, k, v))
    ot, _ = O.chunked_bidir_2d(tq, tk, tv, w0, 0.9, 4, Wg, Hg)
    np.testing.assert_allclose(ot, O.grid_transpose(o, Hg, Wg), atol=1e-13)


def test_one_chunk_is_four_full_batch_readouts():
    """b = N: each of the four directions takes one full-batch step on all tokens and reads them
    out after it, so the output is 4 x the full-batch layer's."""
    Hg, Wg = 3, 5
    q, k, v = _qkv(2, Hg * Wg, 1, 4)
    w0 = RNG.standard_normal((1, 4, 4)) * 0.1
    o, ends = O.chunked_bidir_2d(q, k, v, w0, 1.0, Hg * Wg, Hg, Wg)
    of, wf = O.fullbatch(q, k, v, w0, 1.0)
    np.testing.assert_allclose(o, 4 * of, atol=1e-13)
    for w in ends:
        np.testing.assert_allclose(w, wf, atol=1e-14)
