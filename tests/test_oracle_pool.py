"""The process-pool evaluation of the TTT-MLP oracle (tests/oracle_pool.py) gives the same result
as one call over all (batch, head) pairs, up to fp64 rounding (the batched products may take other
summation orders for other batch shapes): the pairs are independent inner models."""
import numpy as np

from oracle import ttt_oracle as O
from oracle_pool import mlp_causal_sliced
from test_sequence_layers_amd import synth


def test_sliced_mlp_oracle_equals_one_call():
    wl = synth.WORKLOADS["ttt_mlp_causal_8k"].with_(B=2, N=32, H=5, D=8, Dh=12, chunk=8, seed=9)
    x = synth.make_inputs(wl)
    whole = O.mlp_causal(x.q64, x.k64, x.v64, x.w1, x.w2, wl.eta, wl.chunk)[0]
    sliced = mlp_causal_sliced(x.q64, x.k64, x.v64, x.w1, x.w2, wl.eta, wl.chunk, heads_per_task=2)
    assert np.abs(whole - sliced).max() <= 1e-12 * np.abs(whole).max()


def test_sliced_chunked_vjp_matches_direct_call():
    """The pool's slice-by-slice evaluation of the chunked backward oracles (shared and per-batch
    W0) equals the direct call."""
    from oracle import ttt_oracle as O
    from oracle_pool import chunked_vjp_sliced

    rng = np.random.default_rng(41)
    B, N, H, D = 2, 24, 3, 4
    q, k, v, do = [rng.standard_normal((B, N, H, D)) for _ in range(4)]
    for w0 in (rng.standard_normal((H, D, D)) * 0.2, rng.standard_normal((B, H, D, D)) * 0.2):
        for kind, fn in (("causal", O.chunked_causal_vjp), ("bidir", O.chunked_bidir_vjp)):
            got = chunked_vjp_sliced(kind, q, k, v, w0, 0.7, 8, do)
            ref = fn(q, k, v, w0, 0.7, 8, do)
            for g, r in zip(got, ref):
                np.testing.assert_allclose(g, r, rtol=1e-12, atol=1e-12)
