"""The Python binding rejects caller-supplied tensors whose shape, dtype or
device does not match what the kernels read or write through their pointers.
These checks run before any device access, so CPU tensors exercise them; a
tensor that passes them then fails on the device check."""

import pytest
import torch

from exact_io_aware_35_amd import binding as bd

B, N, H, D = 2, 40, 3, 64


def t(shape=(B, N, H, D), dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def raises(match, fn, *a, **kw):
    with pytest.raises(bd.FaError, match=match) as e:
        fn(*a, **kw)
    assert e.value.status == bd.FA_ERR_INVALID_ARG


def test_forward_buffers():
    q = t()
    raises(r"^k must be torch.bfloat16, got torch.float16", bd.forward, q, t(dtype=torch.float16), t())
    raises(r"^v must be torch.bfloat16", bd.forward, q, t(), t(dtype=torch.float32))
    raises(r"^out must have shape \(2, 40, 3, 64\), got \(2, 39, 3, 64\)", bd.forward, q, t(), t(),
           out=t((B, N - 1, H, D)))
    raises(r"^out must be torch.bfloat16, got torch.float32", bd.forward, q, t(), t(),
           out=t(dtype=torch.float32))
    raises(r"^lse must have shape \(2, 3, 40\)", bd.forward, q, t(), t(),
           lse=t((B, N, H), torch.float32))
    raises(r"^lse must be torch.float32", bd.forward, q, t(), t(), lse=t((B, H, N), torch.bfloat16))
    raises(r"^seqlens_k must be torch.int32, got torch.int64", bd.forward, q, t(), t(),
           seqlens_k=torch.full((B,), N, dtype=torch.int64))
    raises(r"^seqlens_k must have shape \(2,\)", bd.forward, q, t(), t(),
           seqlens_k=torch.full((B + 1,), N, dtype=torch.int32))
    # Matching buffers pass the checks and stop at the device check.
    raises(r"device tensor", bd.forward, q, t(), t(), out=t(), lse=t((B, H, N), torch.float32),
           seqlens_k=torch.full((B,), N, dtype=torch.int32))


def test_packed_forward_buffers():
    qkv = t((B, N, 3, H, D))
    raises(r"^out must have shape \(2, 40, 3, 64\)", bd.forward_qkvpacked, qkv, out=t((B, N, H, 32)))
    raises(r"device tensor", bd.forward_qkvpacked, qkv)


def test_backward_buffers():
    q, k, v, o, do = t(), t(), t(), t(), t()
    lse = t((B, H, N), torch.float32)
    raises(r"^dout must be torch.bfloat16", bd.backward, q, k, v, o, lse, t(dtype=torch.float16))
    raises(r"^dk must have shape", bd.backward, q, k, v, o, lse, do, dk=t((B, N, H, D - 8)))
    raises(r"^dq must be torch.bfloat16", bd.backward, q, k, v, o, lse, do,
           dq=t(dtype=torch.float32))
    raises(r"^out must have shape", bd.backward, q, k, v, t((B, N, H + 1, D)), lse, do)
    raises(r"^lse must be torch.float32", bd.backward, q, k, v, o, t((B, H, N)), do)
    raises(r"^out, lse and dout are required", bd.backward, q, k, v, o, lse, None)
    qkv = t((B, N, 3, H, D))
    raises(r"^dqkv must have shape \(2, 40, 3, 3, 64\)", bd.backward_qkvpacked, qkv, o, lse, do,
           dqkv=t((B, N, 3, H, D // 2)))
    raises(r"device tensor", bd.backward, q, k, v, o, lse, do)


def test_fp8_buffers():
    q8 = t(dtype=torch.uint8)
    k8 = t(dtype=torch.float8_e4m3fn)  # either byte type is accepted for any input
    raises(r"^out must be torch.bfloat16, got torch.float32", bd.forward_fp8, q8, k8, q8,
           out=t(dtype=torch.float32))
    raises(r"^lse must have shape", bd.forward_fp8, q8, k8, q8, lse=t((B, N), torch.float32))
    raises(r"^k8 must be torch.uint8", bd.forward_fp8, q8, t(dtype=torch.bfloat16), q8)
    raises(r"device tensor", bd.forward_fp8, q8, k8, q8)


def test_prepared_calls_need_their_outputs():
    q = t()
    raises(r"^prepare_forward needs out and lse", bd.prepare_forward, q, t(), t(), None, None)
    raises(r"^out must have shape", bd.prepare_forward, q, t(), t(), t((B, N, H, 8)),
           t((B, H, N), torch.float32))
    q8 = t(dtype=torch.uint8)
    raises(r"^prepare_forward_fp8 needs out and lse", bd.prepare_forward_fp8, q8, q8, q8, None,
           None, 1.0, 1.0, 1.0)
