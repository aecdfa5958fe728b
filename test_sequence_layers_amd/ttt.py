"""Thin ctypes binding of libttt.so (the C ABI declared in include/ttt.h).

Argument marshalling only: every step of the layer runs in the HIP kernels. torch supplies the
device memory and the current HIP stream. There is no CPU fallback: without the built library,
or without a GPU, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libttt.so")

TTT_OK, TTT_ERR_INVALID, TTT_ERR_UNSUPPORTED, TTT_ERR_WORKSPACE, TTT_ERR_HIP = range(5)
TTT_F32, TTT_BF16 = 0, 1
TTT_OP_FULLBATCH, TTT_OP_CAUSAL, TTT_OP_BIDIR, TTT_OP_MLP = range(4)

# Every symbol include/ttt.h declares, with its ctypes signature.
_c_int, _c_float, _c_ll, _vp, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "ttt_forward_fullbatch": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp, _vp, _c_ll,
                                       _vp, _vp, _vp, _sz, _vp]),
    "ttt_forward_chunked_causal": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp,
                                            _vp, _c_ll, _vp, _vp, _vp, _sz, _vp]),
    "ttt_forward_chunked_bidir": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp,
                                           _vp, _c_ll, _vp, _vp, _vp, _sz, _vp]),
    "ttt_mlp_forward": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp,
                                 _vp, _vp, _c_ll, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ttt_workspace_size": (_sz, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "ttt_status_string": (ctypes.c_char_p, [_c_int]),
}

_lib = None


class TTTError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libttt.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libttt.so not built ({path}); run __graft_entry__.build() or "
                           "python -m test_sequence_layers_amd.build")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ttt_status_string(status).decode()


def ttt_workspace_size(op: int, dtype: int, B: int, H: int, N: int, D: int, Dh: int = 0, chunk: int = 0) -> int:
    return int(load_library().ttt_workspace_size(op, dtype, B, H, N, D, Dh, chunk))


# ------------------------------------------------------------------------------------ helpers
def _torch():
    import torch  # imported lazily so that the CPU-only checks need no GPU

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TTT_BF16
    if t.dtype == torch.float32:
        return TTT_F32
    raise TypeError(f"unsupported I/O dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_io(q, k, v):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, N, H, D]")
        if t.dim() != 4 or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q's shape [B, N, H, D] and dtype")


def _state_stride(w, B: int, H: int, per_head: int) -> int:
    torch = _torch()
    if w.dtype != torch.float32 or not w.is_cuda or not w.is_contiguous():
        raise ValueError("inner states must be contiguous fp32 device tensors")
    if w.dim() == 3:
        if w.shape[0] != H:
            raise ValueError("state of shape [H, ...] expected")
        return 0
    if w.dim() == 4 and w.shape[0] == B and w.shape[1] == H:
        return H * per_head
    raise ValueError("state must be [H, r, c] or [B, H, r, c]")


def _workspace(op, dt, B, H, N, D, Dh, chunk, workspace):
    torch = _torch()
    need = ttt_workspace_size(op, dt, B, H, N, D, Dh, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
    size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, size


def _raise(status, where):
    if status != TTT_OK:
        raise TTTError(status, where)


# ------------------------------------------------------------------------------- entry points
def ttt_forward_fullbatch(q, k, v, w0, eta: float = 1.0, *, o=None, w_out=None, workspace=None, stream=None):
    """O = Q W*, W* = W0 - (eta/N) K^T (K W0 - V) per (b, h). Returns o."""
    lib = load_library()
    _check_io(q, k, v)
    B, N, H, D = q.shape
    dt = _dtype_code(q)
    stride = _state_stride(w0, B, H, D * D)
    o = _torch().empty_like(q) if o is None else o
    ws, ws_size = _workspace(TTT_OP_FULLBATCH, dt, B, H, N, D, 0, 0, workspace)
    st = lib.ttt_forward_fullbatch(dt, B, H, N, D, float(eta), _ptr(q), _ptr(k), _ptr(v), _ptr(w0), stride,
                                   _ptr(o), _ptr(w_out), _ptr(ws), ws_size, _stream(stream))
    _raise(st, "ttt_forward_fullbatch")
    return o


def ttt_forward_chunked_causal(q, k, v, w0, chunk: int, eta: float = 1.0, *, o=None, w_out=None, workspace=None,
                               stream=None):
    """Causal mini-batch TTT-Linear. Returns o."""
    lib = load_library()
    _check_io(q, k, v)
    B, N, H, D = q.shape
    dt = _dtype_code(q)
    stride = _state_stride(w0, B, H, D * D)
    o = _torch().empty_like(q) if o is None else o
    ws, ws_size = _workspace(TTT_OP_CAUSAL, dt, B, H, N, D, 0, chunk, workspace)
    st = lib.ttt_forward_chunked_causal(dt, B, H, N, D, int(chunk), float(eta), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(w0), stride, _ptr(o), _ptr(w_out), _ptr(ws), ws_size, _stream(stream))
    _raise(st, "ttt_forward_chunked_causal")
    return o


def ttt_forward_chunked_bidir(q, k, v, w0, chunk: int, eta: float = 1.0, *, o=None, w_out=None, workspace=None,
                              stream=None):
    """Bidirectional chunked scan (forward + reversed-sequence scans, summed). Returns o."""
    lib = load_library()
    _check_io(q, k, v)
    B, N, H, D = q.shape
    dt = _dtype_code(q)
    stride = _state_stride(w0, B, H, D * D)
    o = _torch().empty_like(q) if o is None else o
    ws, ws_size = _workspace(TTT_OP_BIDIR, dt, B, H, N, D, 0, chunk, workspace)
    st = lib.ttt_forward_chunked_bidir(dt, B, H, N, D, int(chunk), float(eta), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(w0), stride, _ptr(o), _ptr(w_out), _ptr(ws), ws_size, _stream(stream))
    _raise(st, "ttt_forward_chunked_bidir")
    return o


def ttt_mlp_forward(q, k, v, w1, w2, chunk: int, eta: float = 1.0, *, o=None, w1_out=None, w2_out=None,
                    workspace=None, stream=None):
    """Causal mini-batch TTT-MLP, f(x) = GELU(x W1) W2. Returns o."""
    lib = load_library()
    _check_io(q, k, v)
    B, N, H, D = q.shape
    dt = _dtype_code(q)
    Dh = w1.shape[-1]
    stride = _state_stride(w1, B, H, D * Dh)
    if _state_stride(w2, B, H, D * Dh) != stride:
        raise ValueError("w1 and w2 must both be shared over the batch or both per batch element")
    o = _torch().empty_like(q) if o is None else o
    ws, ws_size = _workspace(TTT_OP_MLP, dt, B, H, N, D, Dh, chunk, workspace)
    st = lib.ttt_mlp_forward(dt, B, H, N, D, Dh, int(chunk), float(eta), _ptr(q), _ptr(k), _ptr(v), _ptr(w1),
                             _ptr(w2), stride, _ptr(o), _ptr(w1_out), _ptr(w2_out), _ptr(ws), ws_size,
                             _stream(stream))
    _raise(st, "ttt_mlp_forward")
    return o
