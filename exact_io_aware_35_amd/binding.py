"""Thin ctypes binding over the C ABI in include/fa.h (libfa_mi355x.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind fa_forward / fa_backward. PyTorch supplies device memory and
the current stream. If the shared library is missing the calls raise; there
is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa_mi355x.so")

FA_DTYPE_BF16 = 0
FA_DTYPE_F32 = 1
FA_DTYPE_F16 = 2

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_WORKSPACE = 3
FA_ERR_HIP = 4

# (name, restype, argtypes) of every entry point the header declares.
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
SIGNATURES = [
    ("fa_forward", _I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P]),
    ("fa_backward_workspace_size", _SZ, [_I, _I, _I, _I, _I]),
    ("fa_backward", _I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I,
                         _I, _P, _SZ, _P]),
    ("fa_forward_ex", _I, [_P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I,
                           _P]),
    ("fa_backward_ex", _I, [_P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                            _F, _I, _I, _I, _I, _P, _SZ, _P]),
    ("fa_forward_fp8", _I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _F, _F, _F, _I, _I, _I,
                            _P]),
    ("fa_backward_noalloc", _I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I,
                                 _I, _I, _I, _P]),
    ("fa_status_string", ctypes.c_char_p, [_I]),
    ("fa_last_error_message", ctypes.c_char_p, []),
]

_lib = None


class FaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


def load_library(path: str | None = None):
    """Load libfa_mi355x.so (once) and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FaError(-1, f"{p} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(p)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(lib, status):
    if status != FA_OK:
        msg = lib.fa_last_error_message().decode() or lib.fa_status_string(status).decode()
        raise FaError(status, msg)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    if t.dtype == torch.float16:
        return FA_DTYPE_F16
    raise FaError(FA_ERR_UNSUPPORTED, f"dtype {t.dtype} is not supported")


def _stream_handle(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise FaError(FA_ERR_INVALID_ARG, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise FaError(FA_ERR_INVALID_ARG, f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t, name, shape, dtypes, device=None):
    """Reject a caller-supplied tensor whose shape, dtype or device differs
    from what the kernels read or write through its pointer (the C ABI sees
    only the pointer, so a short buffer would be read or written past its
    end)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise FaError(FA_ERR_INVALID_ARG,
                      f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        want = " or ".join(str(d) for d in dtypes)
        raise FaError(FA_ERR_INVALID_ARG, f"{name} must be {want}, got {t.dtype}")
    if device is not None and t.device != device:
        raise FaError(FA_ERR_INVALID_ARG, f"{name} is on {t.device}, the inputs on {device}")


def _check_forward_buffers(q, k, v, shape, out, lse, seqlens_k, out_dtypes, in_dtypes=None):
    """Shapes, dtypes and device of a forward call's tensors (k, v None when
    the input is packed). k and v must have q's dtype unless ``in_dtypes``
    names the accepted ones."""
    import torch
    B, N, H, D = shape
    for t, name in ((k, "k"), (v, "v")):
        _expect(t, name, shape, in_dtypes or (q.dtype,), q.device)
    _expect(out, "out", shape, out_dtypes, q.device)
    _expect(lse, "lse", (B, H, N), (torch.float32,), q.device)
    _expect(seqlens_k, "seqlens_k", (B,), (torch.int32,), q.device)


def _alibi(alibi_slopes, batch, heads):
    """(pointer, batch stride) of optional ALiBi slopes: fp32 device [H] or [B, H]."""
    import torch
    if alibi_slopes is None:
        return None, 0
    if alibi_slopes.dtype != torch.float32:
        raise FaError(FA_ERR_INVALID_ARG, "alibi_slopes must be float32")
    if tuple(alibi_slopes.shape) == (heads,):
        stride = 0
    elif tuple(alibi_slopes.shape) == (batch, heads):
        stride = heads
    else:
        raise FaError(FA_ERR_INVALID_ARG,
                      f"alibi_slopes must have shape ({heads},) or ({batch}, {heads})")
    return _dev_ptr(alibi_slopes, "alibi_slopes"), stride


def _forward(q, k, v, packed, shape, causal, window, softmax_scale, seqlens_k, alibi_slopes,
             out, lse, stream):
    import torch
    _check_forward_buffers(q, k, v, shape, out, lse, seqlens_k, (q.dtype,))
    lib = load_library()
    B, N, H, D = shape
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty(shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    slopes, bstride = _alibi(alibi_slopes, B, H)
    st = lib.fa_forward_ex(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), int(packed),
                           _dev_ptr(out, "out"), _dev_ptr(lse, "lse"),
                           _dev_ptr(seqlens_k, "seqlens_k"), slopes, bstride, B, H, N, D, scale,
                           int(bool(causal)), int(window[0]), int(window[1]), _dtype_code(q),
                           _stream_handle(stream, q.device))
    _check(lib, st)
    return out, lse


def forward(q, k, v, causal=False, window=(-1, -1), softmax_scale=None, seqlens_k=None,
            alibi_slopes=None, out=None, lse=None, stream=None):
    """O, LSE = exact attention of q, k, v ([batch, seqlen, heads, headdim]).

    softmax_scale defaults to 1/sqrt(headdim). seqlens_k: int32 [batch] key
    lengths on the device, or None. alibi_slopes: fp32 [heads] or [batch,
    heads] on the device, or None. Returns (out, lse) with lse [B, H, N] fp32.
    """
    if k.shape != q.shape or v.shape != q.shape:
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v must have the same shape")
    return _forward(q, k, v, False, tuple(q.shape), causal, window, softmax_scale, seqlens_k,
                    alibi_slopes, out, lse, stream)


def forward_qkvpacked(qkv, causal=False, window=(-1, -1), softmax_scale=None, seqlens_k=None,
                      alibi_slopes=None, out=None, lse=None, stream=None):
    """forward() of one packed qkv tensor [batch, seqlen, 3, heads, headdim]."""
    if qkv.dim() != 5 or qkv.shape[2] != 3:
        raise FaError(FA_ERR_INVALID_ARG, "qkv must have shape (batch, seqlen, 3, heads, headdim)")
    B, N, _, H, D = qkv.shape
    return _forward(qkv, None, None, True, (B, N, H, D), causal, window, softmax_scale,
                    seqlens_k, alibi_slopes, out, lse, stream)


def forward_fp8(q8, k8, v8, descale_q=1.0, descale_k=1.0, descale_v=1.0, causal=False,
                window=(-1, -1), softmax_scale=None, seqlens_k=None, out=None, lse=None,
                stream=None):
    """O (bf16), LSE of attention over fp8 inputs (fa_forward_fp8).

    q8, k8, v8: e4m3 bytes [batch, seqlen, heads, headdim] on the device, as
    torch.uint8 or torch.float8_e4m3fn; element x of q8 stands for
    e4m3(x) * descale_q (likewise k8, v8). Returns (out bf16, lse fp32).
    """
    import torch
    if k8.shape != q8.shape or v8.shape != q8.shape:
        raise FaError(FA_ERR_INVALID_ARG, "q8, k8, v8 must have the same shape")
    for t, name in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise FaError(FA_ERR_INVALID_ARG,
                          f"{name} must be torch.uint8 (e4m3 bytes) or torch.float8_e4m3fn")
    _check_forward_buffers(q8, k8, v8, tuple(q8.shape), out, lse, seqlens_k, (torch.bfloat16,),
                           (torch.uint8, torch.float8_e4m3fn))
    lib = load_library()
    B, N, H, D = q8.shape
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    st = lib.fa_forward_fp8(_dev_ptr(q8, "q8"), _dev_ptr(k8, "k8"), _dev_ptr(v8, "v8"),
                            _dev_ptr(out, "out"), _dev_ptr(lse, "lse"),
                            _dev_ptr(seqlens_k, "seqlens_k"), B, H, N, D, scale,
                            float(descale_q), float(descale_k), float(descale_v),
                            int(bool(causal)), int(window[0]), int(window[1]),
                            _stream_handle(stream, q8.device))
    _check(lib, st)
    return out, lse


class PreparedCall:
    """An entry point with its arguments marshalled once.

    Calling it re-issues the same launch on the same stream, skipping the
    per-call checks and conversions of forward()/backward(); the tensors it
    was built from must stay alive and keep their storage.
    """

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep  # tensors whose storage the raw pointers refer to

    def __call__(self):
        st = self._fn(*self._args)
        if st != FA_OK:
            _check(load_library(), st)


def prepare_forward(q, k, v, out, lse, causal=False, window=(-1, -1), softmax_scale=None,
                    seqlens_k=None, stream=None):
    """forward() with every argument marshalled once; returns a callable."""
    import torch
    if out is None or lse is None:
        raise FaError(FA_ERR_INVALID_ARG, "prepare_forward needs out and lse")
    _check_forward_buffers(q, k, v, tuple(q.shape), out, lse, seqlens_k, (q.dtype,))
    lib = load_library()
    B, N, H, D = q.shape
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    args = (_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(out, "out"),
            _dev_ptr(lse, "lse"), _dev_ptr(seqlens_k, "seqlens_k"), B, H, N, D, scale,
            int(bool(causal)), int(window[0]), int(window[1]), _dtype_code(q),
            _stream_handle(stream, q.device))
    call = PreparedCall(lib.fa_forward, args, (q, k, v, out, lse, seqlens_k))
    call()  # surfaces argument errors now
    return call


def prepare_forward_fp8(q8, k8, v8, out, lse, descale_q, descale_k, descale_v, causal=False,
                        window=(-1, -1), softmax_scale=None, seqlens_k=None, stream=None):
    """forward_fp8() with every argument marshalled once; returns a callable."""
    import torch
    for t, name in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise FaError(FA_ERR_INVALID_ARG,
                          f"{name} must be torch.uint8 (e4m3 bytes) or torch.float8_e4m3fn")
    if out is None or lse is None:
        raise FaError(FA_ERR_INVALID_ARG, "prepare_forward_fp8 needs out and lse")
    _check_forward_buffers(q8, k8, v8, tuple(q8.shape), out, lse, seqlens_k, (torch.bfloat16,),
                           (torch.uint8, torch.float8_e4m3fn))
    lib = load_library()
    B, N, H, D = q8.shape
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    args = (_dev_ptr(q8, "q8"), _dev_ptr(k8, "k8"), _dev_ptr(v8, "v8"), _dev_ptr(out, "out"),
            _dev_ptr(lse, "lse"), _dev_ptr(seqlens_k, "seqlens_k"), B, H, N, D, scale,
            float(descale_q), float(descale_k), float(descale_v), int(bool(causal)),
            int(window[0]), int(window[1]), _stream_handle(stream, q8.device))
    call = PreparedCall(lib.fa_forward_fp8, args, (q8, k8, v8, out, lse, seqlens_k))
    call()  # surfaces argument errors now
    return call


def workspace_size(batch, heads, seqlen, headdim, dtype_code=FA_DTYPE_BF16):
    return int(load_library().fa_backward_workspace_size(batch, heads, seqlen, headdim, dtype_code))


def _backward(q, k, v, packed, shape, out, lse, dout, causal, window, softmax_scale, seqlens_k,
              alibi_slopes, grads, workspace, stream):
    import torch
    _check_forward_buffers(q, k, v, shape, out, lse, seqlens_k, (q.dtype,))
    if out is None or lse is None or dout is None:
        raise FaError(FA_ERR_INVALID_ARG, "out, lse and dout are required")
    _expect(dout, "dout", shape, (q.dtype,), q.device)
    if packed:
        _expect(grads[0], "dqkv", tuple(q.shape), (q.dtype,), q.device)
    else:
        for t, name in zip(grads, ("dq", "dk", "dv")):
            _expect(t, name, shape, (q.dtype,), q.device)
    lib = load_library()
    B, N, H, D = shape
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    code = _dtype_code(q)
    need = int(lib.fa_backward_workspace_size(B, H, N, D, code))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    slopes, bstride = _alibi(alibi_slopes, B, H)
    st = lib.fa_backward_ex(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), int(packed),
                            _dev_ptr(out, "out"), _dev_ptr(lse, "lse"), _dev_ptr(dout, "dout"),
                            _dev_ptr(grads[0], "dq"), _dev_ptr(grads[1], "dk"),
                            _dev_ptr(grads[2], "dv"), _dev_ptr(seqlens_k, "seqlens_k"), slopes,
                            bstride, B, H, N, D, scale, int(bool(causal)), int(window[0]),
                            int(window[1]), code, _dev_ptr(workspace, "workspace"),
                            workspace.numel() * workspace.element_size(),
                            _stream_handle(stream, q.device))
    _check(lib, st)


def backward(q, k, v, out, lse, dout, causal=False, window=(-1, -1), softmax_scale=None,
             seqlens_k=None, alibi_slopes=None, dq=None, dk=None, dv=None, workspace=None,
             stream=None):
    """dQ, dK, dV of exact attention, recomputing P from the forward's LSE."""
    import torch
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _backward(q, k, v, False, tuple(q.shape), out, lse, dout, causal, window, softmax_scale,
              seqlens_k, alibi_slopes, (dq, dk, dv), workspace, stream)
    return dq, dk, dv


def backward_qkvpacked(qkv, out, lse, dout, causal=False, window=(-1, -1), softmax_scale=None,
                       seqlens_k=None, alibi_slopes=None, dqkv=None, workspace=None, stream=None):
    """dqkv [batch, seqlen, 3, heads, headdim] for a packed qkv input."""
    import torch
    B, N, _, H, D = qkv.shape
    dqkv = torch.empty_like(qkv) if dqkv is None else dqkv
    _backward(qkv, None, None, True, (B, N, H, D), out, lse, dout, causal, window,
              softmax_scale, seqlens_k, alibi_slopes, (dqkv, None, None), workspace, stream)
    return dqkv


def backward_noalloc(q, k, v, out, lse, dout, causal=False, window=(-1, -1), softmax_scale=None,
                     seqlens_k=None, dq=None, dk=None, dv=None, stream=None):
    """backward() through fa_backward_noalloc: the library's static scratch
    array stands in for the workspace (no device allocation inside the call;
    the output tensors are allocated here unless given)."""
    import torch
    shape = tuple(q.shape)
    _check_forward_buffers(q, k, v, shape, out, lse, seqlens_k, (q.dtype,))
    if out is None or lse is None or dout is None:
        raise FaError(FA_ERR_INVALID_ARG, "out, lse and dout are required")
    _expect(dout, "dout", shape, (q.dtype,), q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, name in zip((dq, dk, dv), ("dq", "dk", "dv")):
        _expect(t, name, shape, (q.dtype,), q.device)
    lib = load_library()
    B, N, H, D = shape
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    st = lib.fa_backward_noalloc(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                 _dev_ptr(out, "out"), _dev_ptr(lse, "lse"),
                                 _dev_ptr(dout, "dout"), _dev_ptr(dq, "dq"), _dev_ptr(dk, "dk"),
                                 _dev_ptr(dv, "dv"), _dev_ptr(seqlens_k, "seqlens_k"), B, H, N, D,
                                 scale, int(bool(causal)), int(window[0]), int(window[1]),
                                 _dtype_code(q), _stream_handle(stream, q.device))
    _check(lib, st)
    return dq, dk, dv
