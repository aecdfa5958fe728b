"""GPU parity of the ViT^3 block epilogue (ttt_block_epilogue) against the fp64 oracle, alone and
composed into a ViT^3-style block with the full-batch layer and the depth-wise convolution.
Metric: max |gpu - oracle| / max |oracle| over the output; 1e-2 for bf16, 1e-4 for fp32."""
import numpy as np
import pytest

from oracle import ttt_oracle as O
from oracle.block_oracle import block_epilogue
from oracle.dwconv_oracle import dwconv3x3
from test_sequence_layers_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _round(a, dtype):
    a = np.asarray(a, dtype=np.float32)
    return synth.f32_to_bf16_bits(a) if dtype == "bf16" else a


def _wide(a, dtype):
    return synth.bf16_bits_to_f32(a).astype(np.float64) if dtype == "bf16" else a.astype(np.float64)


def _dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("M,C,Co,dtype,bias", [
    (1000, 64, 64, "bf16", True),
    (77, 192, 192, "bf16", True),     # ragged token tile, Vision-TTT width
    (51200, 192, 192, "bf16", False), # Vision-TTT 1280^2: 8 x 6400 tokens
    (200704, 64, 64, "bf16", True),   # H-ViT^3-T stage 1: 64 x 3136 tokens
    (100, 32, 128, "fp32", True),
    (33, 64, 64, "fp32", False),
])
def test_epilogue_parity(M, C, Co, dtype, bias):
    import test_sequence_layers_amd as T

    print(f"epilogue M={M} C={C} C_out={Co} {dtype} bias={bias}", flush=True)
    rs = np.random.default_rng(M + C + Co)
    o = _round(rs.standard_normal((M, C)) * 0.3, dtype)
    g = _round(rs.standard_normal((M, C)), dtype)
    x = _round(rs.standard_normal((M, C)) * 0.3, dtype)
    w = _round(rs.standard_normal((Co, 2 * C)) / np.sqrt(2 * C), dtype)
    b = (rs.standard_normal(Co) * 0.1).astype(np.float32) if bias else None
    y = T.ttt_block_epilogue(_dev(o, dtype), _dev(g, dtype), _dev(x, dtype), _dev(w, dtype),
                             None if b is None else torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    ref = block_epilogue(_wide(o, dtype), _wide(g, dtype), _wide(x, dtype), _wide(w, dtype), b)
    err = float(np.abs(got - ref).max() / np.abs(ref).max())
    print(f"  max err {err:.3e}", flush=True)
    assert err <= (1e-2 if dtype == "bf16" else 1e-4)


def test_vit3_style_block_at_hvit3t_stage1():
    """The full-batch TTT layer's output, a 3x3 depth-wise convolution of V over the 56 x 56 grid
    and a gate, through the epilogue (C = C_out = 64), against the same chain of oracles (each
    intermediate rounded to bf16, the dtype the next step reads)."""
    import test_sequence_layers_amd as T

    wl = synth.WORKLOADS["hvit3t_stage1_fullbatch"].with_(B=4, seed=191)
    x = synth.make_inputs(wl)
    C = wl.H * wl.D
    rs = np.random.default_rng(192)
    wc = (rs.standard_normal((C, 3, 3)) / 3).astype(np.float32)
    gate = synth.f32_to_bf16_bits(rs.standard_normal((wl.B * wl.N, C)).astype(np.float32))
    wp = synth.f32_to_bf16_bits((rs.standard_normal((C, 2 * C)) / np.sqrt(2 * C)).astype(np.float32))
    bias = (rs.standard_normal(C) * 0.05).astype(np.float32)
    q, k, v = _dev(x.q, "bf16"), _dev(x.k, "bf16"), _dev(x.v, "bf16")
    o = T.ttt_forward_fullbatch(q, k, v, torch.from_numpy(x.w0).cuda(), wl.eta)
    xc = T.ttt_dwconv3x3(v, torch.from_numpy(wc).cuda(), None, height=56, width=56)
    y = T.ttt_block_epilogue(o.view(-1, C), _dev(gate, "bf16"), xc.view(-1, C), _dev(wp, "bf16"),
                             torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    rb = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(a, np.float32))).astype(np.float64)  # noqa: E731
    o_ref = rb(O.fullbatch(x.q64, x.k64, x.v64, x.w0, wl.eta)[0].reshape(-1, C))
    xc_ref = rb(dwconv3x3(x.v64.reshape(wl.B, wl.N, C), wc, None, 56, 56).reshape(-1, C))
    ref = block_epilogue(o_ref, synth.bf16_bits_to_f32(gate).astype(np.float64), xc_ref,
                         synth.bf16_bits_to_f32(wp).astype(np.float64), bias)
    err = float(np.abs(got - ref).max() / np.abs(ref).max())
    print(f"ViT^3-style block: max err {err:.3e}", flush=True)
    assert err <= 1e-2
