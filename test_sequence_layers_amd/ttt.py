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
(TTT_OP_FULLBATCH, TTT_OP_CAUSAL, TTT_OP_BIDIR, TTT_OP_MLP, TTT_OP_FULLBATCH_BWD, TTT_OP_BIDIR2D, TTT_OP_CAUSAL_BWD,
 TTT_OP_BIDIR_BWD) = range(8)
TTT_NOALLOC_SCRATCH_BYTES = 32 << 20  # static scratch of ttt_forward_fullbatch_noalloc, per device

# Every symbol include/ttt.h declares, with its ctypes signature.
_c_int, _c_float, _c_ll, _vp, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "ttt_forward_fullbatch": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp, _vp, _c_ll,
                                       _vp, _vp, _vp, _sz, _vp]),
    "ttt_forward_fullbatch_epochs": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp,
                                              _vp, _vp, _c_ll, _vp, _vp, _vp, _sz, _vp]),
    "ttt_backward_fullbatch": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp, _vp, _c_ll,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ttt_backward_chunked_causal": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp,
                                             _vp, _c_ll, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ttt_backward_chunked_bidir": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp,
                                            _vp, _c_ll, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ttt_forward_chunked_bidir2d": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp,
                                             _vp, _vp, _vp, _c_ll, _vp, _vp, _vp, _sz, _vp]),
    "ttt_forward_chunked_causal": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp,
                                            _vp, _c_ll, _vp, _vp, _vp, _sz, _vp]),
    "ttt_forward_chunked_bidir": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp,
                                           _vp, _c_ll, _vp, _vp, _vp, _sz, _vp]),
    "ttt_mlp_forward": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp,
                                 _vp, _vp, _c_ll, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ttt_forward_fullbatch_noalloc": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp, _vp,
                                               _c_ll, _vp, _vp, _vp]),
    "ttt_dwconv3x3": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp]),
    "ttt_block_epilogue": (_c_int, [_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
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
# The binding is the only layer that sees tensor shapes: it checks every tensor against the layout
# the C ABI assumes (include/ttt.h) before calling it, so that a wrongly shaped output or state can
# never make a kernel write past its buffer. Everything below is argument marshalling only.
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


def _stream(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_tensor(name, t, shape, dtype, device):
    """t must be a contiguous device tensor of exactly this shape and dtype, on `device`."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, q on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, not {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_io(q, k, v):
    torch = _torch()
    if not isinstance(q, torch.Tensor) or not q.is_cuda:
        raise TypeError("q must be a CUDA (HIP) tensor")
    if q.dim() != 4:
        raise ValueError("q must be [B, N, H, D]")
    _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)


def _state_stride(name, w, B: int, H: int, rows: int, cols: int, device) -> int:
    """Batch stride (elements) of an initial state [H, rows, cols] (shared, stride 0) or
    [B, H, rows, cols] (one per batch element)."""
    torch = _torch()
    if isinstance(w, torch.Tensor) and w.dim() == 3:
        _check_tensor(name, w, (H, rows, cols), torch.float32, device)
        return 0
    _check_tensor(name, w, (B, H, rows, cols), torch.float32, device)
    return H * rows * cols


def _check_out(name, t, shape, dtype, device):
    if t is not None:
        _check_tensor(name, t, shape, dtype, device)


def _workspace(op, dt, B, H, N, D, Dh, chunk, workspace, device):
    torch = _torch()
    need = ttt_workspace_size(op, dt, B, H, N, D, Dh, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or workspace.device != device:
            raise ValueError(f"workspace must be a device tensor on {device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
    size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, size


def _raise(status, where):
    if status != TTT_OK:
        raise TTTError(status, where)


def _linear(op, fn_name, q, k, v, w0, chunk, eta, o, w_out, workspace, stream, epochs=None):
    lib = load_library()
    _check_io(q, k, v)
    torch = _torch()
    B, N, H, D = q.shape
    dev = q.device
    dt = _dtype_code(q)
    stride = _state_stride("w0", w0, B, H, D, D, dev)
    _check_out("o", o, q.shape, q.dtype, dev)
    _check_out("w_out", w_out, ((2,) if op == TTT_OP_BIDIR else ()) + (B, H, D, D), torch.float32, dev)
    with torch.cuda.device(dev):
        o = torch.empty_like(q) if o is None else o
        ws, ws_size = _workspace(op, dt, B, H, N, D, 0, chunk, workspace, dev)
        args = [dt, B, H, N, D] + ([] if op == TTT_OP_FULLBATCH else [int(chunk)]) + \
            ([] if epochs is None else [int(epochs)])
        st = getattr(lib, fn_name)(*args, float(eta), _ptr(q), _ptr(k), _ptr(v), _ptr(w0), stride, _ptr(o),
                                   _ptr(w_out), _ptr(ws), ws_size, _stream(stream, dev))
    _raise(st, fn_name)
    return o


# ------------------------------------------------------------------------------- entry points
def ttt_forward_fullbatch(q, k, v, w0, eta: float = 1.0, *, o=None, w_out=None, workspace=None, stream=None):
    """O = Q W*, W* = W0 - (eta/N) K^T (K W0 - V) per (b, h). Returns o.

    q, k, v, o: [B, N, H, D] bf16 or fp32; w0: fp32 [H, D, D] or [B, H, D, D]; w_out: fp32 [B, H, D, D]."""
    return _linear(TTT_OP_FULLBATCH, "ttt_forward_fullbatch", q, k, v, w0, 0, eta, o, w_out, workspace, stream)


def ttt_forward_fullbatch_epochs(q, k, v, w0, epochs: int, eta: float = 1.0, *, o=None, w_out=None, workspace=None,
                                 stream=None):
    """`epochs` full-batch steps W <- W - (eta/N) K^T (K W - V) from W0, then O = Q W. Returns o."""
    return _linear(TTT_OP_FULLBATCH, "ttt_forward_fullbatch_epochs", q, k, v, w0, 0, eta, o, w_out, workspace,
                   stream, epochs=epochs)


def _backward(op, name, q, k, v, w0, d_o, chunk, eta, d_q, d_k, d_v, d_w0, workspace, stream):
    lib = load_library()
    _check_io(q, k, v)
    torch = _torch()
    B, N, H, D = q.shape
    dev = q.device
    dt = _dtype_code(q)
    stride = _state_stride("w0", w0, B, H, D, D, dev)
    _check_tensor("d_o", d_o, q.shape, q.dtype, dev)
    for nm, t in (("d_q", d_q), ("d_k", d_k), ("d_v", d_v)):
        _check_out(nm, t, q.shape, q.dtype, dev)
    _check_out("d_w0", d_w0, (B, H, D, D), torch.float32, dev)
    with torch.cuda.device(dev):
        d_q = torch.empty_like(q) if d_q is None else d_q
        d_k = torch.empty_like(q) if d_k is None else d_k
        d_v = torch.empty_like(q) if d_v is None else d_v
        d_w0 = torch.empty((B, H, D, D), dtype=torch.float32, device=dev) if d_w0 is None else d_w0
        ws, ws_size = _workspace(op, dt, B, H, N, D, 0, chunk, workspace, dev)
        args = [dt, B, H, N, D] + ([int(chunk)] if op != TTT_OP_FULLBATCH_BWD else []) + [
            float(eta), _ptr(q), _ptr(k), _ptr(v), _ptr(w0), stride, _ptr(d_o), _ptr(d_q), _ptr(d_k), _ptr(d_v),
            _ptr(d_w0), _ptr(ws), ws_size, _stream(stream, dev)]
        st = getattr(lib, name)(*args)
    _raise(st, name)
    return d_q, d_k, d_v, d_w0


def ttt_backward_fullbatch(q, k, v, w0, d_o, eta: float = 1.0, *, d_q=None, d_k=None, d_v=None, d_w0=None,
                           workspace=None, stream=None):
    """Gradients (dq, dk, dv, dW0) of the full-batch layer for the outer loop, given d_o = dL/dO.
    d_w0 is [B, H, D, D] per batch element (sum it over the batch when w0 is shared)."""
    return _backward(TTT_OP_FULLBATCH_BWD, "ttt_backward_fullbatch", q, k, v, w0, d_o, 0, eta, d_q, d_k, d_v, d_w0,
                     workspace, stream)


def ttt_backward_chunked_causal(q, k, v, w0, d_o, chunk: int, eta: float = 1.0, *, d_q=None, d_k=None, d_v=None,
                                d_w0=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv, dW0) of the causal chunked layer given d_o = dL/dO (no gradient through
    the end state). d_w0 is [B, H, D, D] per batch element."""
    return _backward(TTT_OP_CAUSAL_BWD, "ttt_backward_chunked_causal", q, k, v, w0, d_o, chunk, eta, d_q, d_k, d_v,
                     d_w0, workspace, stream)


def ttt_backward_chunked_bidir(q, k, v, w0, d_o, chunk: int, eta: float = 1.0, *, d_q=None, d_k=None, d_v=None,
                               d_w0=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv, dW0) of the bidirectional scan (both scans summed) given d_o = dL/dO."""
    return _backward(TTT_OP_BIDIR_BWD, "ttt_backward_chunked_bidir", q, k, v, w0, d_o, chunk, eta, d_q, d_k, d_v,
                     d_w0, workspace, stream)


def ttt_forward_fullbatch_noalloc(q, k, v, w0, eta: float = 1.0, *, o, w_out=None, stream=None):
    """ttt_forward_fullbatch for callers that cannot allocate: the library's static per-device scratch
    replaces the workspace, and the caller passes the output `o`. Returns o."""
    lib = load_library()
    _check_io(q, k, v)
    torch = _torch()
    B, N, H, D = q.shape
    dev = q.device
    dt = _dtype_code(q)
    stride = _state_stride("w0", w0, B, H, D, D, dev)
    _check_tensor("o", o, q.shape, q.dtype, dev)
    _check_out("w_out", w_out, (B, H, D, D), torch.float32, dev)
    with torch.cuda.device(dev):
        st = lib.ttt_forward_fullbatch_noalloc(dt, B, H, N, D, float(eta), _ptr(q), _ptr(k), _ptr(v), _ptr(w0),
                                               stride, _ptr(o), _ptr(w_out), _stream(stream, dev))
    _raise(st, "ttt_forward_fullbatch_noalloc")
    return o


def ttt_forward_chunked_causal(q, k, v, w0, chunk: int, eta: float = 1.0, *, o=None, w_out=None, workspace=None,
                               stream=None):
    """Causal mini-batch TTT-Linear. Returns o. w_out: fp32 [B, H, D, D] end state."""
    return _linear(TTT_OP_CAUSAL, "ttt_forward_chunked_causal", q, k, v, w0, chunk, eta, o, w_out, workspace,
                   stream)


def ttt_forward_chunked_bidir(q, k, v, w0, chunk: int, eta: float = 1.0, *, o=None, w_out=None, workspace=None,
                              stream=None):
    """Bidirectional chunked scan (forward + reversed-sequence scans, summed). Returns o.
    w_out: fp32 [2, B, H, D, D] (forward end state, reverse end state)."""
    return _linear(TTT_OP_BIDIR, "ttt_forward_chunked_bidir", q, k, v, w0, chunk, eta, o, w_out, workspace,
                   stream)


def ttt_forward_chunked_bidir2d(q, k, v, w0, chunk: int, height: int, width: int, eta: float = 1.0, *, o=None,
                                w_out=None, workspace=None, stream=None):
    """Bidirectional scans in raster order and in column order of the height x width token grid,
    summed. w_out: fp32 [4, B, H, D, D]. Returns o."""
    lib = load_library()
    _check_io(q, k, v)
    torch = _torch()
    B, N, H, D = q.shape
    if N != height * width:
        raise ValueError(f"{N} tokens are not a {height} x {width} grid")
    dev = q.device
    dt = _dtype_code(q)
    stride = _state_stride("w0", w0, B, H, D, D, dev)
    _check_out("o", o, q.shape, q.dtype, dev)
    _check_out("w_out", w_out, (4, B, H, D, D), torch.float32, dev)
    with torch.cuda.device(dev):
        o = torch.empty_like(q) if o is None else o
        ws, ws_size = _workspace(TTT_OP_BIDIR2D, dt, B, H, N, D, 0, chunk, workspace, dev)
        st = lib.ttt_forward_chunked_bidir2d(dt, B, H, int(height), int(width), D, int(chunk), float(eta), _ptr(q),
                                             _ptr(k), _ptr(v), _ptr(w0), stride, _ptr(o), _ptr(w_out), _ptr(ws),
                                             ws_size, _stream(stream, dev))
    _raise(st, "ttt_forward_chunked_bidir2d")
    return o


def ttt_mlp_forward(q, k, v, w1, w2, chunk: int, eta: float = 1.0, *, o=None, w1_out=None, w2_out=None,
                    workspace=None, stream=None):
    """Causal mini-batch TTT-MLP, f(x) = GELU(x W1) W2. Returns o.

    w1: fp32 [H, D, Dh] or [B, H, D, Dh]; w2: fp32 [H, Dh, D] or [B, H, Dh, D] (batched like w1);
    w1_out / w2_out: fp32 [B, H, D, Dh] / [B, H, Dh, D] end states."""
    lib = load_library()
    _check_io(q, k, v)
    torch = _torch()
    B, N, H, D = q.shape
    dev = q.device
    dt = _dtype_code(q)
    if not isinstance(w1, torch.Tensor) or w1.dim() not in (3, 4):
        raise ValueError("w1 must be [H, D, Dh] or [B, H, D, Dh]")
    Dh = int(w1.shape[-1])
    stride = _state_stride("w1", w1, B, H, D, Dh, dev)
    if w2.dim() != w1.dim():
        raise ValueError("w1 and w2 must both be shared over the batch or both per batch element")
    _state_stride("w2", w2, B, H, Dh, D, dev)
    _check_out("o", o, q.shape, q.dtype, dev)
    _check_out("w1_out", w1_out, (B, H, D, Dh), torch.float32, dev)
    _check_out("w2_out", w2_out, (B, H, Dh, D), torch.float32, dev)
    with torch.cuda.device(dev):
        o = torch.empty_like(q) if o is None else o
        ws, ws_size = _workspace(TTT_OP_MLP, dt, B, H, N, D, Dh, chunk, workspace, dev)
        st = lib.ttt_mlp_forward(dt, B, H, N, D, Dh, int(chunk), float(eta), _ptr(q), _ptr(k), _ptr(v), _ptr(w1),
                                 _ptr(w2), stride, _ptr(o), _ptr(w1_out), _ptr(w2_out), _ptr(ws), ws_size,
                                 _stream(stream, dev))
    _raise(st, "ttt_mlp_forward")
    return o


def ttt_dwconv3x3(x, weight, bias=None, *, height: int, width: int, y=None, stream=None):
    """Depth-wise 3x3 convolution over the token grid. x: [B, height * width, C] or [B, N, H, D]
    (then C = H * D) bf16 or fp32; weight fp32 [C, 3, 3]; bias fp32 [C] or None. Returns y (x's shape)."""
    lib = load_library()
    torch = _torch()
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError("x must be a CUDA (HIP) tensor")
    dev = x.device
    dt = _dtype_code(x)
    if x.dim() not in (3, 4) or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, N, C] or [B, N, H, D] tensor")
    B, N = int(x.shape[0]), int(x.shape[1])
    C = int(x.numel() // max(B * N, 1))
    if N != height * width:
        raise ValueError(f"{N} tokens are not a {height} x {width} grid")
    _check_tensor("weight", weight, (C, 3, 3), torch.float32, dev)
    _check_out("bias", bias, (C,), torch.float32, dev)
    _check_out("y", y, x.shape, x.dtype, dev)
    with torch.cuda.device(dev):
        y = torch.empty_like(x) if y is None else y
        st = lib.ttt_dwconv3x3(dt, B, int(height), int(width), C, _ptr(x), _ptr(weight), _ptr(bias), _ptr(y),
                               _stream(stream, dev))
    _raise(st, "ttt_dwconv3x3")
    return y


def ttt_block_epilogue(o, gate, xconv, w_proj, bias=None, *, y=None, stream=None):
    """y = [o * sigmoid(gate), xconv] w_proj^T + bias per token. o, gate, xconv: [..., C] (the
    leading dims are the tokens); w_proj [C_out, 2C] of the same dtype; bias fp32 [C_out] or None.
    Returns y [..., C_out]."""
    lib = load_library()
    torch = _torch()
    if not isinstance(o, torch.Tensor) or not o.is_cuda:
        raise TypeError("o must be a CUDA (HIP) tensor")
    dev = o.device
    dt = _dtype_code(o)
    C = int(o.shape[-1])
    M = int(o.numel() // C)
    for name, t in (("o", o), ("gate", gate), ("xconv", xconv)):
        _check_tensor(name, t, o.shape, o.dtype, dev)
    if w_proj.dim() != 2 or int(w_proj.shape[1]) != 2 * C:
        raise ValueError("w_proj must be [C_out, 2C]")
    Co = int(w_proj.shape[0])
    _check_tensor("w_proj", w_proj, (Co, 2 * C), o.dtype, dev)
    _check_out("bias", bias, (Co,), torch.float32, dev)
    out_shape = tuple(o.shape[:-1]) + (Co,)
    _check_out("y", y, out_shape, o.dtype, dev)
    with torch.cuda.device(dev):
        y = torch.empty(out_shape, dtype=o.dtype, device=dev) if y is None else y
        st = lib.ttt_block_epilogue(dt, M, C, Co, _ptr(o), _ptr(gate), _ptr(xconv), _ptr(w_proj), _ptr(bias), _ptr(y),
                                    _stream(stream, dev))
    _raise(st, "ttt_block_epilogue")
    return y
