"""ttt_forward_fullbatch_noalloc (the full-batch forward with the library's static per-device scratch
instead of a workspace) through the C ABI, against ttt_forward_fullbatch on the same inputs: the
same kernels and the same split plan, so the outputs and end states must be bit-identical. Two
calls in a row, the second smaller than the first, so that the second finds the first's records
in the scratch; then a call too large for the scratch, which must fail without touching o."""
import numpy as np
import pytest

from test_sequence_layers_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _pair(T, wl):
    x = synth.make_inputs(wl)
    q, k, v = _dev(x.q), _dev(x.k), _dev(x.v)
    w0 = torch.from_numpy(x.w0).cuda()
    o_ref = torch.empty_like(q)
    w_ref = torch.full((wl.B, wl.H, wl.D, wl.D), float("nan"), device="cuda")
    T.ttt_forward_fullbatch(q, k, v, w0, wl.eta, o=o_ref, w_out=w_ref)
    o = torch.full_like(q, float("nan"))
    w = torch.full((wl.B, wl.H, wl.D, wl.D), float("nan"), device="cuda")
    T.ttt_forward_fullbatch_noalloc(q, k, v, w0, wl.eta, o=o, w_out=w)
    torch.cuda.synchronize()
    return o_ref, w_ref, o, w


def test_noalloc_matches_the_workspace_entry_point():
    import test_sequence_layers_amd as T

    big = synth.WORKLOADS["hvit3t_stage1_fullbatch"]               # 64 x 3136, 2 heads of 32: 7.3 MB of records
    small = synth.WORKLOADS["vit3s_fullbatch"].with_(B=8, seed=7)  # 8 x 196, 6 heads of 64
    for wl in (big, small):
        need = T.ttt_workspace_size(T.TTT_OP_FULLBATCH, T.TTT_BF16, wl.B, wl.H, wl.N, wl.D)
        print(f"noalloc B={wl.B} N={wl.N} H={wl.H} D={wl.D}: scratch {need} bytes", flush=True)
        assert 0 < need <= T.TTT_NOALLOC_SCRATCH_BYTES
        o_ref, w_ref, o, w = _pair(T, wl)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(w, w_ref)


def test_noalloc_rejects_a_call_too_large_for_its_scratch():
    import test_sequence_layers_amd as T

    B, N, H, D = 4096, 16, 6, 64
    assert T.ttt_workspace_size(T.TTT_OP_FULLBATCH, T.TTT_BF16, B, H, N, D) > T.TTT_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, N, H, D, dtype=torch.bfloat16, device="cuda")
    w0 = torch.zeros(H, D, D, device="cuda")
    o = torch.full_like(q, 7.0)
    with pytest.raises(T.TTTError) as e:
        T.ttt_forward_fullbatch_noalloc(q, q, q, w0, 1.0, o=o)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool((o.float() == 7.0).all())
