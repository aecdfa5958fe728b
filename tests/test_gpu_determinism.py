"""Repeat calls of the entry points added beside the forward layers give bit-identical results (fixed
reduction orders, no atomics), on the default stream and on a side stream: the backward passes, the
convolution, the block epilogue, the 2-D scan and the full-batch epochs."""
import numpy as np
import pytest

from test_sequence_layers_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _same(xs, ys):
    for x, y in zip(xs, ys):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def _calls():
    import test_sequence_layers_amd as T

    rs = np.random.default_rng(77)
    W = synth.WORKLOADS
    out = {}
    for name, wl, fn in (("fullbatch_bwd", W["hvit3t_stage1_fullbatch"].with_(B=4, N=1000, seed=301),
                          lambda d, wl: T.ttt_backward_fullbatch(d["q"], d["k"], d["v"], d["w0"], d["do"], wl.eta)),
                         ("causal_bwd", W["ttt_linear_causal_16k"].with_(B=1, N=2048, H=2, seed=302),
                          lambda d, wl: T.ttt_backward_chunked_causal(d["q"], d["k"], d["v"], d["w0"], d["do"],
                                                                      wl.chunk, wl.eta)),
                         ("bidir_bwd", W["vittt_bidir_1280"].with_(B=1, N=1280, H=2, seed=303),
                          lambda d, wl: T.ttt_backward_chunked_bidir(d["q"], d["k"], d["v"], d["w0"], d["do"],
                                                                     wl.chunk, wl.eta)),
                         ("epochs", W["hvit3t_stage1_fullbatch"].with_(B=4, N=1000, seed=304),
                          lambda d, wl: (T.ttt_forward_fullbatch_epochs(d["q"], d["k"], d["v"], d["w0"], 3, wl.eta),)),
                         ("bidir2d", W["vittt_bidir_1280"].with_(B=1, N=32 * 40, H=2, seed=305),
                          lambda d, wl: (T.ttt_forward_chunked_bidir2d(d["q"], d["k"], d["v"], d["w0"], wl.chunk, 32,
                                                                       40, wl.eta),))):
        x = synth.make_inputs(wl)
        do = synth.f32_to_bf16_bits((rs.standard_normal((wl.B, wl.N, wl.H, wl.D)) / 8).astype(np.float32))
        d = {"q": _dev(x.q, "bf16"), "k": _dev(x.k, "bf16"), "v": _dev(x.v, "bf16"),
             "w0": torch.from_numpy(x.w0).cuda(), "do": _dev(do, "bf16")}
        out[name] = (lambda d=d, wl=wl, fn=fn: fn(d, wl))
    xc = _dev(synth.f32_to_bf16_bits((rs.standard_normal((2, 30 * 30, 64))).astype(np.float32)), "bf16")
    wc = torch.from_numpy((rs.standard_normal((64, 3, 3)) / 3).astype(np.float32)).cuda()
    bc = torch.from_numpy((rs.standard_normal(64) * 0.1).astype(np.float32)).cuda()
    out["dwconv"] = lambda: (T.ttt_dwconv3x3(xc, wc, bc, height=30, width=30),)
    act = [_dev(synth.f32_to_bf16_bits((rs.standard_normal((777, 64)) * 0.3).astype(np.float32)), "bf16")
           for _ in range(3)]
    wo = _dev(synth.f32_to_bf16_bits((rs.standard_normal((128, 128)) / 11).astype(np.float32)), "bf16")
    out["epilogue"] = lambda: (T.ttt_block_epilogue(act[0], act[1], act[2], wo, None),)
    return out


@pytest.mark.parametrize("name", ["fullbatch_bwd", "causal_bwd", "bidir_bwd", "epochs", "bidir2d", "dwconv",
                                  "epilogue"])
def test_repeat_calls_bit_identical(name):
    print(f"determinism: {name}", flush=True)
    call = _calls()[name]
    first = [t.clone() for t in call()]
    torch.cuda.synchronize()
    again = [t.clone() for t in call()]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        on_side = [t.clone() for t in call()]
    side.synchronize()
    torch.cuda.synchronize()
    _same(first, again)
    _same(first, on_side)
