"""Seeded synthetic inputs for TTT-layer forward passes.

This module is shared by the GPU path's tests and bench and by the oracle's tests.
It holds none of the TTT method's arithmetic: only a counter-based SplitMix64
stream (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014), Box-Muller normals, and fp32 -> bf16
round-to-nearest-even.

Recipe (the pages use image and language workloads; i.i.d. Gaussians of the
same shapes stand in for them, and since no kernel has data-dependent control
flow the work and the bytes moved are the same):
  * every tensor has its own SplitMix64 stream, keyed by (seed, tensor tag);
  * element i of a tensor (row-major order) is normal number i of that stream;
  * Q, K, V ~ N(0, 1) / sqrt(D); inner weights W0 / W1 / W2 ~ N(0, 0.02^2);
  * Q, K, V are rounded to the I/O dtype (bf16 by RNE, or fp32); weights are
    fp32 (the inner state is always fp32).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Stream tags, one per tensor.
TAG_W0 = 1  # W0 of TTT-Linear, or W1 of TTT-MLP
TAG_W2 = 2  # W2 of TTT-MLP
TAG_Q = 3
TAG_K = 4
TAG_V = 5


def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(state: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs start .. start+n-1 of the SplitMix64 sequence whose state starts at `state`.

    Output i is mix64(state + (i + 1) * gamma), so any slice can be produced on its own.
    """
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(np.uint64(state) + i * _GAMMA)


def stream_key(seed: int, tag: int) -> int:
    """Starting state of the stream for (seed, tag)."""
    z = np.array([(int(seed) << 20) ^ int(tag)], dtype=np.uint64)
    with np.errstate(over="ignore"):
        return int(_mix64(z + _GAMMA)[0])


def normals(seed: int, tag: int, count: int) -> np.ndarray:
    """`count` standard normals (float64) from stream (seed, tag), Box-Muller on pairs of 53-bit uniforms."""
    pairs = (count + 1) // 2
    z = splitmix64(stream_key(seed, tag), 2 * pairs)
    u = ((z >> np.uint64(11)).astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    th = (2.0 * math.pi) * u2
    out = np.empty(2 * pairs, dtype=np.float64)
    out[0::2] = r * np.cos(th)
    out[1::2] = r * np.sin(th)
    return out[:count]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 by round-to-nearest-even; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    with np.errstate(over="ignore"):
        r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and settings of one TTT-layer forward call."""

    name: str
    op: str  # "fullbatch" | "causal" | "bidir" | "mlp"
    B: int
    N: int
    H: int
    D: int
    dtype: str  # "bf16" | "fp32"
    seed: int
    chunk: int = 0  # mini-batch size b (0 for full-batch)
    Dh: int = 0  # TTT-MLP hidden width
    eta: float = 1.0

    @property
    def tokens(self) -> int:
        return self.B * self.N

    @property
    def io_bytes(self) -> int:
        """Algorithmic HBM bytes: read Q, K, V once and write O once."""
        s = 2 if self.dtype == "bf16" else 4
        return 4 * self.B * self.N * self.H * self.D * s

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads the library is measured and checked on.
WORKLOADS = {
    # tiny full-batch check in fp32 I/O: batch 1, 2 heads, 64 tokens, head dim 16
    "fullbatch_tiny_fp32": Workload("fullbatch_tiny_fp32", "fullbatch", 1, 64, 2, 16, "fp32", 1),
    # ViT^3-S layer: 64 images of 14x14 tokens, 6 heads x 64
    "vit3s_fullbatch": Workload("vit3s_fullbatch", "fullbatch", 64, 196, 6, 64, "bf16", 2),
    # H-ViT^3-T stage 1: 64 images of 56x56 tokens, 2 heads x 32
    "hvit3t_stage1_fullbatch": Workload("hvit3t_stage1_fullbatch", "fullbatch", 64, 3136, 2, 32, "bf16", 3),
    # Vision-TTT layer at 1280x1280 with 16-px patches: 8 images of 80x80 tokens, 3 heads x 64, b = 64
    "vittt_bidir_1280": Workload("vittt_bidir_1280", "bidir", 8, 6400, 3, 64, "bf16", 4, chunk=64),
    # TTT-MLP language layer: batch 4, 8192 tokens, 12 heads x 64, hidden 256, b = 16
    "ttt_mlp_causal_8k": Workload("ttt_mlp_causal_8k", "mlp", 4, 8192, 12, 64, "bf16", 5, chunk=16, Dh=256),
    # TTT-Linear language layer at 16384 tokens: batch 2, 12 heads x 64, b = 16
    "ttt_linear_causal_16k": Workload("ttt_linear_causal_16k", "causal", 2, 16384, 12, 64, "bf16", 11, chunk=16),
    # N = 16384 sweep points
    "ttt_mlp_causal_16k": Workload("ttt_mlp_causal_16k", "mlp", 2, 16384, 12, 64, "bf16", 12, chunk=16, Dh=256),
    "fullbatch_16k": Workload("fullbatch_16k", "fullbatch", 16, 16384, 2, 32, "bf16", 13),
    "bidir_16k": Workload("bidir_16k", "bidir", 8, 16384, 3, 64, "bf16", 14, chunk=64),
}


@dataclasses.dataclass
class Inputs:
    """Host-side inputs. q/k/v are uint16 bf16 bit patterns ([B,N,H,D]) or float32 arrays;
    q64/k64/v64 give the same values widened to float64 (what the oracle consumes)."""

    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    w0: np.ndarray | None = None  # fp32 [H,D,D]
    w1: np.ndarray | None = None  # fp32 [H,D,Dh]
    w2: np.ndarray | None = None  # fp32 [H,Dh,D]

    def _wide(self, x):
        if self.wl.dtype == "bf16":
            return bf16_bits_to_f32(x).astype(np.float64)
        return x.astype(np.float64)

    @property
    def q64(self):
        return self._wide(self.q)

    @property
    def k64(self):
        return self._wide(self.k)

    @property
    def v64(self):
        return self._wide(self.v)


def _activation(seed, tag, shape, scale, dtype):
    x = (normals(seed, tag, int(np.prod(shape))) * scale).astype(np.float32).reshape(shape)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def make_inputs(wl: Workload, zero_w: bool = False) -> Inputs:
    """Draw the inputs of workload `wl` from its seed. zero_w gives W0 = 0 (or W1 = W2 = 0)."""
    shp = (wl.B, wl.N, wl.H, wl.D)
    sc = 1.0 / math.sqrt(wl.D)
    q = _activation(wl.seed, TAG_Q, shp, sc, wl.dtype)
    k = _activation(wl.seed, TAG_K, shp, sc, wl.dtype)
    v = _activation(wl.seed, TAG_V, shp, sc, wl.dtype)
    if wl.op == "mlp":
        w1 = (normals(wl.seed, TAG_W0, wl.H * wl.D * wl.Dh) * 0.02).astype(np.float32).reshape(wl.H, wl.D, wl.Dh)
        w2 = (normals(wl.seed, TAG_W2, wl.H * wl.Dh * wl.D) * 0.02).astype(np.float32).reshape(wl.H, wl.Dh, wl.D)
        if zero_w:
            w1[:] = 0
            w2[:] = 0
        return Inputs(wl, q, k, v, w1=w1, w2=w2)
    w0 = (normals(wl.seed, TAG_W0, wl.H * wl.D * wl.D) * 0.02).astype(np.float32).reshape(wl.H, wl.D, wl.D)
    if zero_w:
        w0[:] = 0
    return Inputs(wl, q, k, v, w0=w0)
