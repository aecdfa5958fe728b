"""GPU parity of the depth-wise 3x3 convolution (ttt_dwconv3x3) against the fp64 oracle, element by
element, and of the Vision-TTT preprocessing chain: the convolution of K and V followed by the
bidirectional scan, against the same chain of oracles.

Metric: max |gpu - oracle| / max |oracle| per batch image; 1e-2 for bf16 I/O, 1e-4 for fp32.
"""
import numpy as np
import pytest

from oracle import ttt_oracle as O
from oracle.dwconv_oracle import dwconv3x3
from test_sequence_layers_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _inputs(B, Hi, Wi, C, dtype, seed, bias=True):
    rs = np.random.default_rng(seed)
    x = (rs.standard_normal((B, Hi * Wi, C)) / np.sqrt(C)).astype(np.float32)
    w = (rs.standard_normal((C, 3, 3)) / 3.0).astype(np.float32)
    b = (rs.standard_normal(C) * 0.1).astype(np.float32) if bias else None
    if dtype == "bf16":
        xb = synth.f32_to_bf16_bits(x)
        return xb, synth.bf16_bits_to_f32(xb).astype(np.float64), w, b
    return x, x.astype(np.float64), w, b


def _dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _err(got, ref):
    num = np.abs(got - ref).reshape(got.shape[0], -1).max(axis=1)
    den = np.abs(ref).reshape(ref.shape[0], -1).max(axis=1)
    return float((num / np.maximum(den, 1e-30)).max())


CASES = [
    (2, 5, 7, 16, "bf16", True),
    (1, 9, 13, 64, "fp32", True),
    (3, 8, 8, 24, "bf16", False),
    (1, 1, 1, 8, "bf16", True),         # a single token: only the centre tap
    (1, 1, 33, 40, "fp32", False),      # one image row
    (2, 17, 1, 32, "bf16", True),       # one image column
    (1, 23, 41, 136, "bf16", True),     # rows not a multiple of 8, a ragged last workgroup
    (2, 56, 56, 64, "bf16", True),      # H-ViT^3-T stage-1 grid, C = 2 x 32
    (8, 80, 80, 192, "bf16", True),     # Vision-TTT at 1280^2 (80 x 80 tokens), C = 3 x 64
]


@pytest.mark.parametrize("B,Hi,Wi,C,dtype,bias", CASES, ids=lambda v: str(v))
def test_dwconv_parity(B, Hi, Wi, C, dtype, bias):
    import test_sequence_layers_amd as T

    print(f"dwconv B={B} {Hi}x{Wi} C={C} {dtype} bias={bias}", flush=True)
    x, x64, w, b = _inputs(B, Hi, Wi, C, dtype, seed=B * 1000 + Hi * 10 + C, bias=bias)
    y = T.ttt_dwconv3x3(_dev(x, dtype), torch.from_numpy(w).cuda(), None if b is None else torch.from_numpy(b).cuda(),
                        height=Hi, width=Wi)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    ref = dwconv3x3(x64, w, b, Hi, Wi)
    err = _err(got, ref)
    print(f"  max err {err:.3e}", flush=True)
    assert err <= (1e-2 if dtype == "bf16" else 1e-4)


def test_dwconv_preprocessing_then_bidirectional_scan():
    """Vision-TTT's chain at a reduced 1280^2 shape (2 images of 80 x 80 tokens, 3 heads of 64,
    b = 64): K and V each through their own depth-wise convolution, then the bidirectional scan.
    The oracle chain rounds the convolved K and V to bf16, the scan's input dtype."""
    import test_sequence_layers_amd as T

    wl = synth.WORKLOADS["vittt_bidir_1280"].with_(B=2, seed=150)
    Hi = Wi = 80
    x = synth.make_inputs(wl)
    C = wl.H * wl.D
    rs = np.random.default_rng(151)
    wk, wv = [(rs.standard_normal((C, 3, 3)) / 3.0).astype(np.float32) for _ in range(2)]
    bk, bv = [(rs.standard_normal(C) * 0.05).astype(np.float32) for _ in range(2)]
    q, k, v = _dev(x.q, "bf16"), _dev(x.k, "bf16"), _dev(x.v, "bf16")
    kc = T.ttt_dwconv3x3(k, torch.from_numpy(wk).cuda(), torch.from_numpy(bk).cuda(), height=Hi, width=Wi)
    vc = T.ttt_dwconv3x3(v, torch.from_numpy(wv).cuda(), torch.from_numpy(bv).cuda(), height=Hi, width=Wi)
    out = T.ttt_forward_chunked_bidir(q, kc, vc, torch.from_numpy(x.w0).cuda(), wl.chunk, wl.eta)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)

    def conv_bf16(t64, w, b):
        y = dwconv3x3(t64.reshape(wl.B, wl.N, C), w, b, Hi, Wi).astype(np.float32)
        return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(y)).astype(np.float64).reshape(t64.shape)

    ref = O.chunked_bidir(x.q64, conv_bf16(x.k64, wk, bk), conv_bf16(x.v64, wv, bv), x.w0, wl.eta, wl.chunk)[0]
    num = np.abs(got - ref).max(axis=(1, 3))
    den = np.abs(ref).max(axis=(1, 3))
    err = float((num / den).max())
    print(f"conv + bidir: max err {err:.3e}", flush=True)
    assert err <= 1e-2
