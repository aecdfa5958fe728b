"""The C ABI without a GPU: the library loads, exports every declared symbol, sizes workspaces,
and rejects bad arguments before launching anything.

Every call below that passes pointers is built to FAIL VALIDATION (the pointers are fake but never
dereferenced, because the library validates all arguments before it enqueues work).
"""
import ctypes
import os
import re

import pytest

import test_sequence_layers_amd as T
from test_sequence_layers_amd import ttt as binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "ttt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted([
        "ttt_forward_fullbatch", "ttt_forward_chunked_causal", "ttt_forward_chunked_bidir", "ttt_mlp_forward",
        "ttt_workspace_size", "ttt_status_string", "ttt_forward_fullbatch_noalloc", "ttt_dwconv3x3",
        "ttt_forward_fullbatch_epochs", "ttt_backward_fullbatch", "ttt_forward_chunked_bidir2d",
        "ttt_block_epilogue", "ttt_backward_chunked_causal", "ttt_backward_chunked_bidir"])


def test_block_epilogue_validation():
    lib = T.load_library()
    call = lambda C=64, Co=64, y=4, o=0: lib.ttt_block_epilogue(T.TTT_BF16, 128, C, Co, None if o is None else _p(o),  # noqa: E731
                                                               _p(1), _p(2), _p(3), None, None if y is None else _p(y),
                                                               None)
    assert call(o=None) == 1
    assert call(y=None) == 1
    assert call(C=48) == 2
    assert call(Co=96) == 2
    assert call(y=0) == 1


def test_bidir2d_validation_rejects_before_launch():
    lib = T.load_library()
    # 80 x 80 tokens in chunks of 64: several segments per scan, so that a workspace is required
    call = lambda hg=80, wg=80, chunk=64, ws=5, wsb=1 << 30, o=4, wout=None: lib.ttt_forward_chunked_bidir2d(  # noqa: E731
        T.TTT_BF16, 1, 1, hg, wg, 64, chunk, 1.0, _p(0), _p(1), _p(2), _p(3), 0, None if o is None else _p(o),
        None if wout is None else _p(wout), None if ws is None else _p(ws), wsb, None)
    assert call(hg=0) == 1
    assert call(o=None) == 1
    assert call(chunk=24) == 2
    assert call(hg=5, wg=5) == 1          # 25 tokens: not a multiple of the chunk
    assert call(ws=None) == 3
    assert call(wsb=64) == 3
    assert call(wout=1) == 1              # end states overlap k
    # bf16: the scans' workspace only (the column-order scan reads and adds in place); fp32 also holds
    # column-order copies of q, k, v and of the output
    for dt, es in ((T.TTT_BF16, 2), (T.TTT_F32, 4)):
        scan = T.ttt_workspace_size(T.TTT_OP_BIDIR, dt, 8, 3, 6400, 64, 0, 64)
        two_d = T.ttt_workspace_size(T.TTT_OP_BIDIR2D, dt, 8, 3, 6400, 64, 0, 64)
        assert two_d == scan if dt == T.TTT_BF16 else two_d >= 4 * 8 * 6400 * 3 * 64 * es + scan


def test_backward_validation_rejects_before_launch():
    lib = T.load_library()
    call = lambda do=5, dq=6, dk=7, dv=8, dw=9, ws=10, wsb=1 << 30, D=64: lib.ttt_backward_fullbatch(  # noqa: E731
        T.TTT_BF16, 1, 1, 64, D, 1.0, _p(0), _p(1), _p(2), _p(3), 0, None if do is None else _p(do),
        None if dq is None else _p(dq), None if dk is None else _p(dk), None if dv is None else _p(dv),
        None if dw is None else _p(dw), None if ws is None else _p(ws), wsb, None)
    assert call(do=None) == 1
    assert call(dw=None) == 1
    assert call(dk=0) == 1               # a gradient output overlaps q
    assert call(dv=6) == 1               # two outputs overlap
    assert call(ws=None) == 3
    assert call(wsb=16) == 3
    assert call(D=48) == 2
    assert T.ttt_workspace_size(T.TTT_OP_FULLBATCH_BWD, T.TTT_BF16, 64, 2, 3136, 32) > 0


@pytest.mark.parametrize("fn", ["ttt_backward_chunked_causal", "ttt_backward_chunked_bidir"])
def test_chunked_backward_validation_rejects_before_launch(fn):
    lib = T.load_library()
    f = getattr(lib, fn)
    call = lambda do=5, dq=6, dk=7, dv=8, dw=9, ws=10, wsb=1 << 30, D=64, N=1024, chunk=16: f(  # noqa: E731
        T.TTT_BF16, 1, 1, N, D, chunk, 1.0, _p(0), _p(1), _p(2), _p(3), 0, None if do is None else _p(do),
        None if dq is None else _p(dq), None if dk is None else _p(dk), None if dv is None else _p(dv),
        None if dw is None else _p(dw), None if ws is None else _p(ws), wsb, None)
    assert call(do=None) == 1
    assert call(dw=None) == 1
    assert call(dk=0) == 1               # a gradient output overlaps q
    assert call(dv=6) == 1               # two outputs overlap
    assert call(ws=None) == 3            # 1024 tokens of 16: several segments, workspace needed
    assert call(wsb=16) == 3
    assert call(D=48) == 2
    assert call(chunk=24) == 2
    assert call(N=1000) == 1             # not a multiple of the chunk
    op = T.TTT_OP_CAUSAL_BWD if "causal" in fn else T.TTT_OP_BIDIR_BWD
    assert T.ttt_workspace_size(op, T.TTT_BF16, 2, 12, 16384, 64, 0, 16) > 0
    assert T.ttt_workspace_size(op, T.TTT_BF16, 2, 12, 16384, 64, 0, 24) == 0
    # fp32: the scan's states, C + 1 per (b, h)
    assert T.ttt_workspace_size(op, T.TTT_F32, 2, 3, 256, 32, 0, 16) == 2 * 3 * 17 * 32 * 32 * 4


def test_chunked_backward_workspace_holds_the_segment_states():
    """The backward always keeps its segments' forward states (bf16, d x d each) in the workspace; a
    single-segment causal sequence needs only those (C + 1 states), the bidirectional one also
    holds one scan's fp32 partial gradients."""
    ring = (2 + 1) * 64 * 64 * 2
    assert T.ttt_workspace_size(T.TTT_OP_CAUSAL_BWD, T.TTT_BF16, 1, 1, 32, 64, 0, 16) == ring
    assert T.ttt_workspace_size(T.TTT_OP_BIDIR_BWD, T.TTT_BF16, 1, 1, 32, 64, 0, 16) == ring + 3 * 32 * 64 * 4


def test_fullbatch_epochs_validation():
    lib = T.load_library()
    call = lambda e: lib.ttt_forward_fullbatch_epochs(T.TTT_BF16, 1, 1, 64, 64, e, 1.0, _p(0), _p(1), _p(2), _p(3),  # noqa: E731
                                                      0, _p(4), None, _p(5), 1 << 30, None)
    assert call(0) == 1
    assert call(-3) == 1
    assert call(257) == 2


def test_dwconv_validation_rejects_before_launch():
    lib = T.load_library()
    call = lambda dt=T.TTT_BF16, B=1, Hi=4, Wi=4, C=64, x=0, w=1, b=2, y=3: lib.ttt_dwconv3x3(  # noqa: E731
        dt, B, Hi, Wi, C, None if x is None else _p(x), None if w is None else _p(w), None if b is None else _p(b),
        None if y is None else _p(y), None)
    assert call(x=None) == 1
    assert call(y=None) == 1
    assert call(w=None) == 1
    assert call(B=0) == 1
    assert call(dt=5) == 1
    assert call(C=62) == 2               # channels not a multiple of 4
    assert call(y=0) == 1                # output overlaps the input
    st = lib.ttt_dwconv3x3(T.TTT_BF16, 1, 4, 4, 64, ctypes.c_void_p(FAKE + 8), _p(1), None, _p(3), None)
    assert st == 1                       # misaligned input


def test_noalloc_rejects_calls_beyond_its_scratch_before_any_device_call():
    """The no-alloc full-batch entry point validates everything, the scratch size included, before
    it touches the device (so this runs without a GPU), and reports calls too large for its static
    scratch as a workspace error."""
    lib = T.load_library()
    B, H, D = 4096, 6, 64  # 256-group plan: one split per group, 2 * 6 * 64 * 64 * 4 bytes each
    assert T.ttt_workspace_size(T.TTT_OP_FULLBATCH, T.TTT_BF16, B, H, 196, D) > T.TTT_NOALLOC_SCRATCH_BYTES
    call = lambda B=B, o=4, N=196: lib.ttt_forward_fullbatch_noalloc(T.TTT_BF16, B, H, N, D, 1.0, _p(0), _p(1),  # noqa: E731
                                                                     _p(2), _p(3), 0, None if o is None else _p(o),
                                                                     None, None)
    assert call() == binding.TTT_ERR_WORKSPACE
    assert call(o=None) == binding.TTT_ERR_INVALID
    assert call(o=0) == binding.TTT_ERR_INVALID  # output aliases q
    assert call(N=0) == binding.TTT_ERR_INVALID


def test_library_exports_every_declared_symbol():
    lib = T.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert name in binding.SIGNATURES, name


def test_status_strings():
    assert T.status_string(0) == "ok"
    assert "invalid" in T.status_string(1)
    assert "unsupported" in T.status_string(2)
    assert "workspace" in T.status_string(3)
    assert "HIP" in T.status_string(4)
    assert T.status_string(99) == "unknown status"


def test_workspace_sizes():
    ws = T.ttt_workspace_size
    # full-batch: split partials (K^T K and K^T V, d x d fp32 each per (b, h)) + W*
    assert ws(T.TTT_OP_FULLBATCH, T.TTT_BF16, 1, 2, 64, 16) > 0
    assert ws(T.TTT_OP_FULLBATCH, T.TTT_BF16, 64, 2, 3136, 32) % 256 == 0
    # the split count is capped, so the workspace stays bounded as N grows (linear in B*H only)
    # (2 heads of 32 share a 128-byte row: 4 groups, at most ~4096 splits in total)
    bound = (4096 + 2 * 4) * 2 * 2 * 32 * 32 * 4 + 4 * 2 * 32 * 32 * 4 + 4096
    for n in (100000, 200000, 4000000):
        assert 0 < ws(T.TTT_OP_FULLBATCH, T.TTT_BF16, 4, 2, n, 32) <= bound
    # unsupported sizes report 0
    assert ws(T.TTT_OP_FULLBATCH, T.TTT_BF16, 1, 1, 64, 48) == 0
    assert ws(T.TTT_OP_CAUSAL, T.TTT_BF16, 1, 1, 100, 64, 0, 16) == 0  # N % chunk != 0
    assert ws(T.TTT_OP_BIDIR, T.TTT_BF16, 1, 1, 128, 64, 0, 8) == 0    # chunk unsupported
    assert ws(T.TTT_OP_FULLBATCH, T.TTT_BF16, 0, 1, 64, 64) == 0


FAKE = 1 << 32  # 16-byte aligned, never dereferenced


def _p(i):
    return ctypes.c_void_p(FAKE * (i + 1))


def _fullbatch(dt=T.TTT_BF16, B=1, H=1, N=64, D=64, eta=1.0, q=0, k=1, v=2, w0=3, o=4, w_out=None, ws=5,
               ws_bytes=1 << 30, w0s=0):
    lib = T.load_library()
    ptr = lambda i: None if i is None else _p(i)  # noqa: E731
    return lib.ttt_forward_fullbatch(dt, B, H, N, D, eta, ptr(q), ptr(k), ptr(v), ptr(w0), w0s, ptr(o),
                                     ptr(w_out), ptr(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=0), T.TTT_ERR_INVALID if hasattr(T, "TTT_ERR_INVALID") else 1),
    (dict(N=-5), 1),
    (dict(D=48), 2),
    (dict(D=128), 2),
    (dict(dt=7), 1),
    (dict(eta=float("nan")), 1),
    (dict(q=None), 1),
    (dict(o=None), 1),
    (dict(o=0), 1),              # output aliases q
    (dict(w_out=1), 1),          # state output aliases k
    (dict(ws=None), 3),          # workspace needed but missing
    (dict(ws_bytes=16), 3),      # workspace too small
    (dict(w0s=7), 1),            # batch stride smaller than one batch of states
    (dict(B=2, w0s=64 * 64 + 2), 1),  # batch stride that misaligns the second batch's states
])
def test_fullbatch_validation_rejects_before_launch(kw, expect):
    assert _fullbatch(**kw) == expect


def test_misaligned_pointer_rejected():
    lib = T.load_library()
    st = lib.ttt_forward_fullbatch(T.TTT_BF16, 1, 1, 64, 64, 1.0, ctypes.c_void_p(FAKE + 2), _p(1), _p(2), _p(3),
                                   0, _p(4), None, _p(5), 1 << 30, None)
    assert st == 1


def _chunked(fn, chunk, N=128, D=64, dt=T.TTT_BF16):
    lib = T.load_library()
    return getattr(lib, fn)(dt, 1, 1, N, D, chunk, 1.0, _p(0), _p(1), _p(2), _p(3), 0, None, None, _p(5),
                            1 << 30, None)


@pytest.mark.parametrize("fn", ["ttt_forward_chunked_causal", "ttt_forward_chunked_bidir"])
def test_chunked_validation(fn):
    assert _chunked(fn, 16) == 1          # o is NULL
    lib = T.load_library()
    call = lambda chunk, N=128, D=64: getattr(lib, fn)(T.TTT_BF16, 1, 1, N, D, chunk, 1.0, _p(0), _p(1), _p(2),  # noqa: E731
                                                        _p(3), 0, _p(4), None, _p(5), 16, None)
    assert call(0) == 1                   # non-positive chunk
    assert call(8) == 2                   # unsupported chunk
    assert call(48) == 2
    assert call(16, N=100) == 1           # ragged tail
    assert call(16, D=24) == 2


def test_mlp_validation():
    lib = T.load_library()
    call = lambda dt=T.TTT_BF16, D=64, Dh=256, chunk=16, N=64, o=4, wbs=0: lib.ttt_mlp_forward(  # noqa: E731
        dt, 2, 1, N, D, Dh, chunk, 1.0, _p(0), _p(1), _p(2), _p(3), _p(6), wbs,
        None if o is None else _p(o), None, None, None, 0, None)
    assert call(o=None) == 1
    # supported sizes and dtypes get as far as the (missing) workspace
    assert call() == 3
    assert call(dt=T.TTT_F32) == 3
    assert call(D=32) == 3
    assert call(Dh=128) == 3
    assert call(Dh=1024) == 3
    assert call(chunk=32, N=64) == 3
    assert call(D=48) == 2
    assert call(Dh=100) == 2
    assert call(Dh=2048) == 2
    assert call(chunk=8) == 2
    assert call(N=40) == 1
    assert call(o=0) == 1                 # output aliases q
    assert call(wbs=100) == 1             # batch stride below one batch of states
    assert call(wbs=64 * 256 + 2) == 1    # batch stride that misaligns the second batch's states


def test_binding_fails_loudly_without_gpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 16, 1, 16)
    with pytest.raises(TypeError):
        T.ttt_forward_fullbatch(x, x, x, torch.zeros(1, 16, 16))


# ------------------------------------------------------------------ binding checks (no launch)
# The Python binding checks every tensor against the layout the C ABI assumes before it calls the
# library. These run on CPU with fake CUDA tensors (shape, dtype and device only, no storage); the
# library handle is replaced by one that fails the test if any entry point is reached.
class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"the binding reached the library ({name}) with invalid arguments")


@pytest.fixture
def fake_cuda(monkeypatch):
    torch = pytest.importorskip("torch")
    from torch._subclasses.fake_tensor import FakeTensorMode

    monkeypatch.setattr(binding, "_lib", _NoCalls())
    mode = FakeTensorMode()

    def make(*shape, dtype=torch.bfloat16):
        with mode:
            return torch.empty(*shape, dtype=dtype, device="cuda")

    return torch, make


def _linear_cases(torch, make):
    B, N, H, D = 2, 64, 3, 32
    q = make(B, N, H, D)
    w0 = make(H, D, D, dtype=torch.float32)
    f32 = torch.float32
    return q, w0, [
        ("o wrong shape", dict(o=make(B, N, H, 16))),
        ("o wrong dtype", dict(o=make(B, N, H, D, dtype=f32))),
        ("w_out wrong shape", dict(w_out=make(B, H, D, 16, dtype=f32))),
        ("w_out wrong dtype", dict(w_out=make(B, H, D, D))),
        ("w_out of one direction only (bidir needs two)", dict(w_out=make(B, H, D, D, dtype=f32), bidir_only=True)),
        ("w0 wrong trailing dims", dict(w0=make(H, D, 16, dtype=f32))),
        ("w0 wrong dtype", dict(w0=make(H, D, D))),
        ("w0 wrong batch", dict(w0=make(B + 1, H, D, D, dtype=f32))),
        ("k wrong shape", dict(k=make(B, N, H, 16))),
        ("v wrong dtype", dict(v=make(B, N, H, D, dtype=f32))),
        ("o transposed view", dict(o=make(B, H, N, D).transpose(1, 2))),
    ]


@pytest.mark.parametrize("fn", ["ttt_forward_fullbatch", "ttt_forward_chunked_causal", "ttt_forward_chunked_bidir"])
def test_binding_rejects_bad_tensors_before_launch(fake_cuda, fn):
    torch, make = fake_cuda
    q, w0, cases = _linear_cases(torch, make)
    f = getattr(T, fn)
    for what, kw in cases:
        if kw.pop("bidir_only", False) and fn != "ttt_forward_chunked_bidir":
            continue
        args = dict(q=q, k=kw.pop("k", q), v=kw.pop("v", q), w0=kw.pop("w0", w0))
        call = (lambda: f(args["q"], args["k"], args["v"], args["w0"], 1.0, **kw)) if fn == "ttt_forward_fullbatch" \
            else (lambda: f(args["q"], args["k"], args["v"], args["w0"], 16, 1.0, **kw))
        with pytest.raises((ValueError, TypeError)):
            call()
        print("rejected:", what)


@pytest.mark.parametrize("fn", ["ttt_backward_fullbatch", "ttt_backward_chunked_causal",
                                "ttt_backward_chunked_bidir"])
def test_binding_rejects_bad_backward_tensors_before_launch(fake_cuda, fn):
    torch, make = fake_cuda
    f32 = torch.float32
    B, N, H, D = 2, 64, 3, 32
    q = make(B, N, H, D)
    w0 = make(H, D, D, dtype=f32)
    f = getattr(T, fn)
    cases = [
        dict(d_o=make(B, N, H, 16)),
        dict(d_o=make(B, N, H, D, dtype=f32)),
        dict(d_q=make(B, N, H, 16)),
        dict(d_k=make(B, N, H, D, dtype=f32)),
        dict(d_w0=make(H, D, D, dtype=f32)),             # per batch element: [B, H, D, D]
        dict(d_w0=make(B, H, D, D)),                     # bf16 instead of fp32
        dict(w0=make(H, D, 16, dtype=f32)),
    ]
    for kw in cases:
        d_o = kw.pop("d_o", q)
        a_w0 = kw.pop("w0", w0)
        with pytest.raises((ValueError, TypeError)):
            if fn == "ttt_backward_fullbatch":
                f(q, q, q, a_w0, d_o, 1.0, **kw)
            else:
                f(q, q, q, a_w0, d_o, 16, 1.0, **kw)


def test_binding_rejects_bad_mlp_tensors_before_launch(fake_cuda):
    torch, make = fake_cuda
    f32 = torch.float32
    B, N, H, D, Dh = 2, 64, 3, 64, 256
    q = make(B, N, H, D)
    w1, w2 = make(H, D, Dh, dtype=f32), make(H, Dh, D, dtype=f32)
    cases = [
        dict(w1=make(H, D, 128, dtype=f32)),                      # hidden widths disagree with w2
        dict(w2=make(H, D, Dh, dtype=f32)),                       # w2 transposed
        dict(w2=make(B, H, Dh, D, dtype=f32)),                    # batched w2 with shared w1
        dict(o=make(B, N, H, 32)),
        dict(w1_out=make(B, H, Dh, D, dtype=f32)),
        dict(w2_out=make(H, Dh, D, dtype=f32)),
        dict(w2_out=make(B, H, Dh, D)),
    ]
    for kw in cases:
        a1, a2 = kw.pop("w1", w1), kw.pop("w2", w2)
        with pytest.raises((ValueError, TypeError)):
            T.ttt_mlp_forward(q, q, q, a1, a2, 16, 1.0, **kw)
