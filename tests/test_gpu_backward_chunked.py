"""GPU parity of the chunked backward passes (ttt_backward_chunked_causal, ttt_backward_chunked_bidir)
against the fp64 oracle: dQ, dK, dV per (batch, head) slice (max |gpu - oracle| / max |oracle|) and
dW0 per (batch, head); 1e-2 for bf16 I/O, 1e-4 for fp32. Cases span one and many segments (the
sequence is split into segments whose maps are composed and folded), ragged last segments, every
head width and chunk size, per-batch initial states and the full-size causal TTT-Linear and
Vision-TTT bidirectional layers."""
import numpy as np
import pytest

from test_sequence_layers_amd import synth
from oracle_pool import chunked_vjp_sliced

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CAUSAL = W["ttt_linear_causal_16k"]
BIDIR = W["vittt_bidir_1280"]


def _dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _slice_err(got, ref):
    num = np.abs(got - ref).max(axis=(1, 3))
    den = np.abs(ref).max(axis=(1, 3))
    return float((num / np.maximum(den, 1e-30)).max())


CASES = [
    ("causal", CAUSAL),                                                        # full size: 1024 chunks of 16
    ("causal", CAUSAL.with_(B=1, N=2048, H=2, seed=181)),                     # many segments, ragged last one
    ("causal", CAUSAL.with_(B=2, N=64, H=3, seed=182)),                       # one segment
    ("causal", CAUSAL.with_(B=1, N=1536, H=4, D=32, chunk=32, seed=183)),
    ("causal", CAUSAL.with_(B=2, N=1024, H=2, D=16, chunk=64, seed=184)),
    ("causal", CAUSAL.with_(B=1, N=1280, H=2, chunk=64, seed=185)),
    ("causal", CAUSAL.with_(B=1, N=256, H=2, D=32, dtype="fp32", seed=186)),
    ("causal", CAUSAL.with_(B=1, N=512, H=1, chunk=64, dtype="fp32", seed=187)),
    ("bidir", BIDIR),                                                          # full size: 100 chunks of 64
    ("bidir", BIDIR.with_(B=1, N=1280, H=2, seed=191)),
    ("bidir", BIDIR.with_(B=2, N=128, H=2, seed=192)),                         # one segment
    ("bidir", BIDIR.with_(B=1, N=2048, H=2, D=32, chunk=16, seed=193)),
    ("bidir", BIDIR.with_(B=1, N=1024, H=4, D=16, chunk=32, seed=194)),
    ("bidir", BIDIR.with_(B=1, N=512, H=2, D=64, chunk=16, seed=195)),
    ("bidir", BIDIR.with_(B=1, N=256, H=2, D=32, chunk=16, dtype="fp32", seed=196)),
    ("bidir", BIDIR.with_(B=1, N=384, H=1, chunk=64, dtype="fp32", seed=197)),
]


def _ids(c):
    kind, w = c
    return f"{kind}-{w.dtype}-B{w.B}N{w.N}H{w.H}D{w.D}b{w.chunk}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
@pytest.mark.parametrize("per_batch_w0", [False, True])
def test_chunked_backward_parity(case, per_batch_w0):
    import test_sequence_layers_amd as T

    kind, wl = case
    if per_batch_w0 and wl.N * wl.B * wl.H > 200000:
        pytest.skip("full-size cases run once, with the shared W0")
    print(f"backward {kind} {wl.dtype} B={wl.B} N={wl.N} H={wl.H} D={wl.D} b={wl.chunk} "
          f"per-batch W0={per_batch_w0}", flush=True)
    x = synth.make_inputs(wl)
    rs = np.random.default_rng(wl.seed + 600)
    w0 = (rs.standard_normal((wl.B, wl.H, wl.D, wl.D)) * 0.05).astype(np.float32) if per_batch_w0 else x.w0
    do = (rs.standard_normal((wl.B, wl.N, wl.H, wl.D)) / np.sqrt(wl.D)).astype(np.float32)
    if wl.dtype == "bf16":
        do = synth.f32_to_bf16_bits(do)
        do64 = synth.bf16_bits_to_f32(do).astype(np.float64)
    else:
        do64 = do.astype(np.float64)
    fn = T.ttt_backward_chunked_causal if kind == "causal" else T.ttt_backward_chunked_bidir
    dq, dk, dv, dw0 = fn(_dev(x.q, wl.dtype), _dev(x.k, wl.dtype), _dev(x.v, wl.dtype),
                         torch.from_numpy(np.ascontiguousarray(w0)).cuda(), _dev(do, wl.dtype), wl.chunk, wl.eta)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    gw = dw0.cpu().numpy().astype(np.float64)
    ref = chunked_vjp_sliced(kind, x.q64, x.k64, x.v64, w0, wl.eta, wl.chunk, do64)
    tol = 1e-2 if wl.dtype == "bf16" else 1e-4
    for name, g, r in zip(("dq", "dk", "dv"), got, ref[:3]):
        err = _slice_err(g, r)
        print(f"  {name}: max err {err:.3e}", flush=True)
        assert err <= tol, name
    err = float((np.abs(gw - ref[3]).max(axis=(2, 3)) / np.abs(ref[3]).max(axis=(2, 3))).max())
    print(f"  dw0: max err {err:.3e}", flush=True)
    assert err <= tol


@pytest.mark.parametrize("kind", ["causal", "bidir"])
def test_chunked_backward_is_the_gradient_of_the_gpu_forward(kind):
    """Consistency of the GPU entry points on a small fp32 case: <dL/dx, delta> from the backward
    equals the central difference of <dO, forward(x +- h delta)> from the forward, for x = q, k, v
    and W0."""
    import test_sequence_layers_amd as T

    wl = CAUSAL.with_(B=1, N=128, H=2, D=16, dtype="fp32", seed=198)
    x = synth.make_inputs(wl)
    rs = np.random.default_rng(199)
    do = rs.standard_normal((wl.B, wl.N, wl.H, wl.D)).astype(np.float32)
    args = [x.q, x.k, x.v, np.broadcast_to(x.w0, (wl.B,) + x.w0.shape).astype(np.float32)]
    fwd = T.ttt_forward_chunked_causal if kind == "causal" else T.ttt_forward_chunked_bidir
    bwd = T.ttt_backward_chunked_causal if kind == "causal" else T.ttt_backward_chunked_bidir
    dev = [_dev(a, "fp32") for a in args]
    grads = bwd(*dev, _dev(do, "fp32"), wl.chunk, wl.eta)
    h = 1e-2
    for i in range(4):
        delta = rs.standard_normal(args[i].shape).astype(np.float32)

        def L(sign):
            a = [d for d in dev]
            a[i] = _dev(args[i] + sign * h * delta, "fp32")
            return float((fwd(*a, wl.chunk, wl.eta).cpu().numpy().astype(np.float64) * do).sum())

        fd = (L(1) - L(-1)) / (2 * h)
        an = float((grads[i].cpu().numpy().astype(np.float64) * delta).sum())
        print(f"{kind} input {i}: backward {an:.6e}, forward difference {fd:.6e}", flush=True)
        assert abs(an - fd) <= 2e-3 * max(abs(fd), 1e-3)
