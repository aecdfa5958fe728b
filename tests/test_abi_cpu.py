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
    return sorted(set(re.findall(r"\b(ttt_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted([
        "ttt_forward_fullbatch", "ttt_forward_chunked_causal", "ttt_forward_chunked_bidir", "ttt_mlp_forward",
        "ttt_workspace_size", "ttt_status_string"])


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
    assert call(dt=T.TTT_F32) == 2
    assert call(D=32) == 2
    assert call(Dh=128) == 2
    assert call(chunk=32) == 2
    assert call(N=40) == 1
    assert call(o=0) == 1                 # output aliases q
    assert call(wbs=100) == 1             # batch stride below one batch of states
    assert call(wbs=64 * 256 + 2) == 1    # batch stride that misaligns the second batch's states


def test_binding_fails_loudly_without_gpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 16, 1, 16)
    with pytest.raises(TypeError):
        T.ttt_forward_fullbatch(x, x, x, torch.zeros(1, 16, 16))
