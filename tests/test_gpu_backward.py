"""GPU parity of the full-batch backward pass (ttt_backward_fullbatch) against the fp64 oracle:
dQ, dK, dV per (batch, head) slice (max |gpu - oracle| / max |oracle|) and dW0 per (batch, head);
1e-2 for bf16 I/O, 1e-4 for fp32."""
import numpy as np
import pytest

from oracle import ttt_oracle as O
from test_sequence_layers_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _slice_err(got, ref):
    num = np.abs(got - ref).max(axis=(1, 3))
    den = np.abs(ref).max(axis=(1, 3))
    return float((num / np.maximum(den, 1e-30)).max())


CASES = [
    W["hvit3t_stage1_fullbatch"],                                   # H-ViT^3-T stage 1, full size
    W["vit3s_fullbatch"].with_(B=4, seed=171),                      # one head of 64 per group
    W["hvit3t_stage1_fullbatch"].with_(B=2, N=1000, H=4, D=16, seed=172),  # four heads of 16 per row
    W["hvit3t_stage1_fullbatch"].with_(B=1, N=333, H=3, seed=173),  # one head of 32 per group, ragged
    W["fullbatch_tiny_fp32"],
    W["fullbatch_tiny_fp32"].with_(B=2, N=150, H=2, D=64, seed=174),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: f"{w.dtype}-B{w.B}N{w.N}H{w.H}D{w.D}")
@pytest.mark.parametrize("per_batch_w0", [False, True])
def test_backward_parity(wl, per_batch_w0):
    import test_sequence_layers_amd as T

    print(f"backward {wl.dtype} B={wl.B} N={wl.N} H={wl.H} D={wl.D} per-batch W0={per_batch_w0}", flush=True)
    x = synth.make_inputs(wl)
    rs = np.random.default_rng(wl.seed + 500)
    w0 = (rs.standard_normal((wl.B, wl.H, wl.D, wl.D)) * 0.05).astype(np.float32) if per_batch_w0 else x.w0
    do = (rs.standard_normal((wl.B, wl.N, wl.H, wl.D)) / np.sqrt(wl.D)).astype(np.float32)
    if wl.dtype == "bf16":
        do = synth.f32_to_bf16_bits(do)
        do64 = synth.bf16_bits_to_f32(do).astype(np.float64)
    else:
        do64 = do.astype(np.float64)
    dq, dk, dv, dw0 = T.ttt_backward_fullbatch(_dev(x.q, wl.dtype), _dev(x.k, wl.dtype), _dev(x.v, wl.dtype),
                                               torch.from_numpy(np.ascontiguousarray(w0)).cuda(),
                                               _dev(do, wl.dtype), wl.eta)
    torch.cuda.synchronize()
    ref = O.fullbatch_vjp(x.q64, x.k64, x.v64, w0, wl.eta, do64)
    tol = 1e-2 if wl.dtype == "bf16" else 1e-4
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        err = _slice_err(g.float().cpu().numpy().astype(np.float64), r)
        print(f"  {name}: max err {err:.3e}", flush=True)
        assert err <= tol, name
    gw = dw0.cpu().numpy().astype(np.float64)
    err = float((np.abs(gw - ref[3]).max(axis=(2, 3)) / np.abs(ref[3]).max(axis=(2, 3))).max())
    print(f"  dw0: max err {err:.3e}", flush=True)
    assert err <= tol


def test_backward_is_the_gradient_of_the_gpu_forward():
    """Consistency of the two GPU entry points on one small fp32 case: <dL/dk, delta> from the
    backward equals the central difference of <dO, forward(k +- h delta)> from the forward."""
    import test_sequence_layers_amd as T

    wl = W["fullbatch_tiny_fp32"].with_(B=1, N=96, H=2, D=16, seed=175)
    x = synth.make_inputs(wl)
    rs = np.random.default_rng(176)
    do = (rs.standard_normal((wl.B, wl.N, wl.H, wl.D))).astype(np.float32)
    delta = (rs.standard_normal((wl.B, wl.N, wl.H, wl.D))).astype(np.float32)
    q, k, v = _dev(x.q, "fp32"), _dev(x.k, "fp32"), _dev(x.v, "fp32")
    w0 = torch.from_numpy(x.w0).cuda()
    _, dk, _, _ = T.ttt_backward_fullbatch(q, k, v, w0, _dev(do, "fp32"), wl.eta)
    h = 1e-2
    kp = _dev(x.k + h * delta, "fp32")
    km = _dev(x.k - h * delta, "fp32")
    lp = float((T.ttt_forward_fullbatch(q, kp, v, w0, wl.eta).cpu().numpy().astype(np.float64) * do).sum())
    lm = float((T.ttt_forward_fullbatch(q, km, v, w0, wl.eta).cpu().numpy().astype(np.float64) * do).sum())
    fd = (lp - lm) / (2 * h)
    an = float((dk.cpu().numpy().astype(np.float64) * delta).sum())
    print(f"directional derivative: backward {an:.6e}, forward difference {fd:.6e}", flush=True)
    assert abs(an - fd) <= 1e-3 * max(abs(fd), 1e-6)
