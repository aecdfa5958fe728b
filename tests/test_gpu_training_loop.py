"""The forward and backward entry points in an outer training loop: gradient descent on a shared W0
for L = 1/2 ||O - target||^2, with the layer's O from the forward call and dL/dW0 from the backward
call (summed over the batch, W0 being shared). The same loop driven by the fp64 oracle (forward and
chunked_causal_vjp / fullbatch_vjp) gives the reference trajectory; the GPU run must follow it
step by step (fp32 I/O: 1e-4 relative on W0 after every step) and the loss must fall."""
import numpy as np
import pytest

from oracle import ttt_oracle as O
from test_sequence_layers_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["causal", "fullbatch"])
def test_outer_gradient_descent_follows_the_oracle(kind):
    import test_sequence_layers_amd as T

    wl = synth.WORKLOADS["ttt_linear_causal_16k"].with_(B=2, N=256, H=2, D=32, dtype="fp32", seed=401)
    x = synth.make_inputs(wl)
    rs = np.random.default_rng(402)
    target = rs.standard_normal((wl.B, wl.N, wl.H, wl.D)) * 0.1
    lr, steps = 0.05, 4  # the loss curvature in W0 is about B N / d = 16: below 2 / 16 for a stable descent
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (x.q, x.k, x.v))
    tgt = torch.from_numpy(target.astype(np.float32)).cuda()
    w_gpu = torch.from_numpy(x.w0.copy()).cuda()
    w_ref = x.w0.astype(np.float64)
    losses = []
    for it in range(steps):
        if kind == "causal":
            o = T.ttt_forward_chunked_causal(q, k, v, w_gpu, wl.chunk, wl.eta)
            d_o = o - tgt
            _, _, _, dw0 = T.ttt_backward_chunked_causal(q, k, v, w_gpu, d_o, wl.chunk, wl.eta)
            o_ref = O.chunked_causal(x.q64, x.k64, x.v64, w_ref, wl.eta, wl.chunk)[0]
            g_ref = O.chunked_causal_vjp(x.q64, x.k64, x.v64, w_ref, wl.eta, wl.chunk, o_ref - target)[3]
        else:
            o = T.ttt_forward_fullbatch(q, k, v, w_gpu, wl.eta)
            d_o = o - tgt
            _, _, _, dw0 = T.ttt_backward_fullbatch(q, k, v, w_gpu, d_o, wl.eta)
            o_ref = O.fullbatch(x.q64, x.k64, x.v64, w_ref, wl.eta)[0]
            g_ref = O.fullbatch_vjp(x.q64, x.k64, x.v64, w_ref, wl.eta, o_ref - target)[3]
        losses.append(0.5 * float(((o_ref - target) ** 2).sum()))
        w_gpu = w_gpu - lr * dw0.sum(dim=0)          # W0 is shared over the batch
        w_ref = w_ref - lr * g_ref.sum(axis=0)
        got = w_gpu.cpu().numpy().astype(np.float64)
        err = np.abs(got - w_ref).max() / np.abs(w_ref).max()
        print(f"{kind} step {it}: loss {losses[-1]:.6f}, W0 rel err {err:.3e}", flush=True)
        assert err <= 1e-4
    assert losses[-1] < losses[0]
