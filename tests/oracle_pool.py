"""Runs the fp64 oracle over independent (batch, head) slices in worker processes.

Every (batch, head) pair of a TTT layer is an independent inner model, so a slice of the inputs
gives exactly that slice of the outputs. The workers are started with the "spawn" method: they
import only numpy, scipy and the oracle (never the GPU runtime), and a process that has touched
the GPU is never forked. Test infrastructure only.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np


def workers() -> int:
    """Worker count: the host's cores, at most 16 (a host's share per GPU)."""
    n = int(os.environ.get("OMP_NUM_THREADS") or 0) or (os.cpu_count() or 1)
    return max(1, min(16, n, os.cpu_count() or 1))


def _mlp_slice(args):
    from oracle import ttt_oracle as O

    b, h0, h1, q, k, v, w1, w2, eta, chunk = args
    return b, h0, h1, O.mlp_causal(q, k, v, w1, w2, eta, chunk)[0]


def mlp_causal_sliced(q64, k64, v64, w1, w2, eta, chunk, heads_per_task: int = 3):
    """O of the TTT-MLP oracle for [B, N, H, D] inputs and per-head states [H, ...], computed
    slice by slice in a process pool. Returns float64 [B, N, H, D]."""
    B, N, H, D = q64.shape
    tasks = []
    for b in range(B):
        for h0 in range(0, H, heads_per_task):
            h1 = min(H, h0 + heads_per_task)
            sl = (slice(b, b + 1), slice(None), slice(h0, h1))
            tasks.append((b, h0, h1, np.ascontiguousarray(q64[sl]), np.ascontiguousarray(k64[sl]),
                          np.ascontiguousarray(v64[sl]), w1[h0:h1], w2[h0:h1], eta, chunk))
    out = np.empty((B, N, H, D), dtype=np.float64)
    with ProcessPoolExecutor(max_workers=min(workers(), len(tasks)), mp_context=mp.get_context("spawn")) as ex:
        for b, h0, h1, o in ex.map(_mlp_slice, tasks):
            out[b:b + 1, :, h0:h1] = o
    return out


def _vjp_slice(args):
    from oracle import ttt_oracle as O

    kind, b, h0, h1, q, k, v, w0, eta, chunk, d_o = args
    fn = O.chunked_causal_vjp if kind == "causal" else O.chunked_bidir_vjp
    return b, h0, h1, fn(q, k, v, w0, eta, chunk, d_o)


def chunked_vjp_sliced(kind, q64, k64, v64, w0, eta, chunk, do64, heads_per_task: int = 1):
    """(dq, dk, dv, dW0) of the chunked backward oracles ("causal" or "bidir") for [B, N, H, D]
    inputs and states [H, D, D] or [B, H, D, D], slice by slice in a process pool."""
    B, N, H, D = q64.shape
    w0 = np.asarray(w0, dtype=np.float64)
    tasks = []
    for b in range(B):
        for h0 in range(0, H, heads_per_task):
            h1 = min(H, h0 + heads_per_task)
            sl = (slice(b, b + 1), slice(None), slice(h0, h1))
            ws = w0[h0:h1] if w0.ndim == 3 else w0[b:b + 1, h0:h1]
            tasks.append((kind, b, h0, h1, np.ascontiguousarray(q64[sl]), np.ascontiguousarray(k64[sl]),
                          np.ascontiguousarray(v64[sl]), ws, eta, chunk, np.ascontiguousarray(do64[sl])))
    grads = [np.empty((B, N, H, D)) for _ in range(3)]
    dw0 = np.empty((B, H, D, D))
    with ProcessPoolExecutor(max_workers=min(workers(), len(tasks)), mp_context=mp.get_context("spawn")) as ex:
        for b, h0, h1, g in ex.map(_vjp_slice, tasks):
            for i in range(3):
                grads[i][b:b + 1, :, h0:h1] = g[i]
            dw0[b:b + 1, h0:h1] = g[3]
    return grads[0], grads[1], grads[2], dw0
