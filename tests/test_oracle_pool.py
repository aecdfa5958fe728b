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
