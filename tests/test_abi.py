"""C-ABI checks that need no GPU: the library loads, exports every function
include/fa.h declares, and rejects bad arguments before any launch."""

import os
import re

import pytest

from exact_io_aware_35_amd import binding as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fb.LIB_PATH),
                                reason="libfa_mi355x.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(
        ["fa_forward", "fa_backward", "fa_forward_ex", "fa_backward_ex", "fa_forward_fp8",
         "fa_backward_workspace_size", "fa_backward_noalloc", "fa_status_string",
         "fa_last_error_message"])


def test_library_exports_every_declared_symbol():
    lib = fb.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(n for n, _, _ in fb.SIGNATURES) == declared_functions()


def test_status_strings():
    lib = fb.load_library()
    for code in range(5):
        assert lib.fa_status_string(code)
    assert lib.fa_status_string(99) == b"unknown status"


FAKE = 0x100000  # a 16-byte aligned non-null address; never dereferenced


def fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, seqlens=None, B=1, H=1, N=16, D=64,
             scale=0.125, causal=0, wl=-1, wr=-1, dtype=fb.FA_DTYPE_BF16)
    a.update(kw)
    return lib.fa_forward(a["q"], a["k"], a["v"], a["out"], a["lse"], a["seqlens"], a["B"],
                          a["H"], a["N"], a["D"], a["scale"], a["causal"], a["wl"], a["wr"],
                          a["dtype"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(B=-1), fb.FA_ERR_INVALID_ARG, "batch"),
    (dict(H=-1), fb.FA_ERR_INVALID_ARG, "batch"),
    (dict(N=-3), fb.FA_ERR_INVALID_ARG, "batch"),
    (dict(N=0, D=96), fb.FA_ERR_UNSUPPORTED, "headdim"),
    (dict(B=0, scale=0.0), fb.FA_ERR_INVALID_ARG, "softmax_scale"),
    (dict(N=(1 << 24) + 1), fb.FA_ERR_INVALID_ARG, "seqlen"),
    (dict(B=1 << 16, H=1 << 8, N=1 << 8), fb.FA_ERR_INVALID_ARG, "2^31"),
    (dict(D=96), fb.FA_ERR_UNSUPPORTED, "headdim"),
    (dict(H=64, N=1 << 17, D=128), fb.FA_ERR_UNSUPPORTED, "2^31 bytes"),
    (dict(dtype=7), fb.FA_ERR_UNSUPPORTED, "dtype"),
    (dict(scale=float("nan")), fb.FA_ERR_INVALID_ARG, "softmax_scale"),
    (dict(scale=0.0), fb.FA_ERR_INVALID_ARG, "softmax_scale"),
    (dict(scale=-1.0), fb.FA_ERR_INVALID_ARG, "softmax_scale"),
    (dict(wl=-2), fb.FA_ERR_INVALID_ARG, "window"),
    (dict(wr=-5), fb.FA_ERR_INVALID_ARG, "window"),
    (dict(q=None), fb.FA_ERR_INVALID_ARG, "q is null"),
    (dict(lse=None), fb.FA_ERR_INVALID_ARG, "lse is null"),
    (dict(v=FAKE + 8), fb.FA_ERR_INVALID_ARG, "v is not 16-byte aligned"),
    (dict(seqlens=FAKE + 2), fb.FA_ERR_INVALID_ARG, "seqlens_k"),
])
def test_forward_rejects_before_launch(kw, status, needle):
    lib = fb.load_library()
    assert fwd(lib, **kw) == status
    assert needle in lib.fa_last_error_message().decode()


def bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             seqlens=None, B=2, H=3, N=100, D=64, scale=0.125, causal=1, wl=-1, wr=-1,
             dtype=fb.FA_DTYPE_BF16, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return lib.fa_backward(a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["dq"],
                           a["dk"], a["dv"], a["seqlens"], a["B"], a["H"], a["N"], a["D"],
                           a["scale"], a["causal"], a["wl"], a["wr"], a["dtype"], a["ws"],
                           a["wsb"], None)


@pytest.mark.parametrize("zero", [dict(B=0), dict(H=0), dict(N=0)])
def test_empty_calls_return_ok_without_reading_pointers(zero):
    """No rows, valid scalars: every entry point returns FA_OK with all its
    pointers null (it must neither check nor read them)."""
    lib = fb.load_library()
    none = dict(q=None, k=None, v=None, out=None, lse=None)
    assert fwd(lib, **none, **zero) == fb.FA_OK
    assert fwd_fp8(lib, **none, **zero) == fb.FA_OK
    assert bwd(lib, **none, dout=None, dq=None, dk=None, dv=None, ws=None, wsb=0,
               **zero) == fb.FA_OK
    assert lib.fa_backward_workspace_size(zero.get("B", 2), zero.get("H", 3), zero.get("N", 100),
                                          64, fb.FA_DTYPE_BF16) == 0
    # A bad scalar is still reported.
    assert bwd(lib, **zero, dtype=fb.FA_DTYPE_F32) == fb.FA_ERR_UNSUPPORTED
    assert fwd_fp8(lib, **zero, dq=0.0) == fb.FA_ERR_INVALID_ARG


def test_workspace_size():
    lib = fb.load_library()
    need = lib.fa_backward_workspace_size(2, 3, 100, 64, fb.FA_DTYPE_BF16)
    assert need >= 2 * 3 * 100 * 4 and need % 256 == 0
    assert lib.fa_backward_workspace_size(0, 3, 100, 64, fb.FA_DTYPE_BF16) == 0
    assert lib.fa_backward_workspace_size(2, 3, 100, 80, fb.FA_DTYPE_BF16) == 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(ws=None), fb.FA_ERR_WORKSPACE, "workspace"),
    (dict(wsb=16), fb.FA_ERR_WORKSPACE, "workspace"),
    (dict(ws=FAKE + 4), fb.FA_ERR_INVALID_ARG, "workspace"),
    (dict(dout=None), fb.FA_ERR_INVALID_ARG, "dout is null"),
    (dict(dk=FAKE + 2), fb.FA_ERR_INVALID_ARG, "dk is not 16-byte aligned"),
    (dict(D=32), fb.FA_ERR_UNSUPPORTED, "headdim"),
    (dict(dtype=fb.FA_DTYPE_F32), fb.FA_ERR_UNSUPPORTED, "bf16"),
    (dict(wl=-3), fb.FA_ERR_INVALID_ARG, "window"),
])
def test_backward_rejects_before_launch(kw, status, needle):
    lib = fb.load_library()
    assert bwd(lib, **kw) == status
    assert needle in lib.fa_last_error_message().decode()


def test_binding_without_library_fails_loudly(tmp_path):
    with pytest.raises(fb.FaError):
        fb.load_library(str(tmp_path / "missing.so"))


def fwd_ex(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, packed=0, out=FAKE, lse=FAKE, seqlens=None, slopes=None,
             bstride=0, B=2, H=4, N=64, D=128, scale=0.125, causal=0, wl=-1, wr=-1,
             dtype=fb.FA_DTYPE_BF16)
    a.update(kw)
    return lib.fa_forward_ex(a["q"], a["k"], a["v"], a["packed"], a["out"], a["lse"],
                             a["seqlens"], a["slopes"], a["bstride"], a["B"], a["H"], a["N"],
                             a["D"], a["scale"], a["causal"], a["wl"], a["wr"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(packed=1), fb.FA_ERR_INVALID_ARG, "k and v must be null"),
    (dict(packed=1, k=None, v=None, q=None), fb.FA_ERR_INVALID_ARG, "qkv is null"),
    (dict(packed=1, k=None, v=None, q=FAKE + 8), fb.FA_ERR_INVALID_ARG, "qkv is not 16-byte"),
    (dict(k=None), fb.FA_ERR_INVALID_ARG, "k is null"),
    (dict(slopes=FAKE + 2), fb.FA_ERR_INVALID_ARG, "alibi_slopes"),
    (dict(slopes=FAKE, bstride=3), fb.FA_ERR_INVALID_ARG, "alibi_batch_stride"),
    # Packed rows are 3x wider: (N + 128) * 3 * H * D * 2 >= 2^31 here, unpacked < 2^31.
    (dict(packed=1, k=None, v=None, H=64, N=1 << 16, D=128), fb.FA_ERR_UNSUPPORTED, "2^31 bytes"),
])
def test_forward_ex_rejects_before_launch(kw, status, needle):
    lib = fb.load_library()
    assert fwd_ex(lib, **kw) == status
    assert needle in lib.fa_last_error_message().decode()


def test_packed_slice_limit_is_three_times_wider():
    lib = fb.load_library()
    # Same sizes unpacked stay below the limit: rejected later, on a null pointer.
    assert fwd_ex(lib, H=64, N=1 << 16, D=128, lse=None) == fb.FA_ERR_INVALID_ARG
    assert "lse is null" in lib.fa_last_error_message().decode()


def bwd_ex(lib, **kw):
    a = dict(q=FAKE, k=None, v=None, packed=1, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=None,
             dv=None, seqlens=None, slopes=None, bstride=0, B=2, H=3, N=100, D=64, scale=0.125,
             causal=1, wl=-1, wr=-1, dtype=fb.FA_DTYPE_BF16, ws=FAKE, wsb=1 << 24)
    a.update(kw)
    return lib.fa_backward_ex(a["q"], a["k"], a["v"], a["packed"], a["out"], a["lse"],
                              a["dout"], a["dq"], a["dk"], a["dv"], a["seqlens"], a["slopes"],
                              a["bstride"], a["B"], a["H"], a["N"], a["D"], a["scale"],
                              a["causal"], a["wl"], a["wr"], a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dk=FAKE), fb.FA_ERR_INVALID_ARG, "dk and dv must be null"),
    (dict(dq=None), fb.FA_ERR_INVALID_ARG, "dqkv is null"),
    (dict(packed=0, k=FAKE, v=FAKE, dk=FAKE, dv=None), fb.FA_ERR_INVALID_ARG, "dv is null"),
    (dict(slopes=FAKE, bstride=1), fb.FA_ERR_INVALID_ARG, "alibi_batch_stride"),
    (dict(ws=None), fb.FA_ERR_WORKSPACE, "workspace"),
    (dict(dtype=fb.FA_DTYPE_F32), fb.FA_ERR_UNSUPPORTED, "bf16"),
])
def test_backward_ex_rejects_before_launch(kw, status, needle):
    lib = fb.load_library()
    assert bwd_ex(lib, **kw) == status
    assert needle in lib.fa_last_error_message().decode()


def fwd_fp8(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, seqlens=None, B=2, H=4, N=64, D=128,
             scale=0.125, dq=0.5, dk=0.25, dv=2.0, causal=0, wl=-1, wr=-1)
    a.update(kw)
    return lib.fa_forward_fp8(a["q"], a["k"], a["v"], a["out"], a["lse"], a["seqlens"], a["B"],
                              a["H"], a["N"], a["D"], a["scale"], a["dq"], a["dk"], a["dv"],
                              a["causal"], a["wl"], a["wr"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dq=0.0), fb.FA_ERR_INVALID_ARG, "descale_q"),
    (dict(dk=float("nan")), fb.FA_ERR_INVALID_ARG, "descale_k"),
    (dict(dv=float("inf")), fb.FA_ERR_INVALID_ARG, "descale_v"),
    (dict(dv=-1.0), fb.FA_ERR_INVALID_ARG, "descale_v"),
    (dict(dq=1e30, dk=1e30), fb.FA_ERR_INVALID_ARG, "finite positive"),
    (dict(dq=1e9, dk=1e9), fb.FA_ERR_INVALID_ARG, "too large"),
    (dict(scale=0.0), fb.FA_ERR_INVALID_ARG, "softmax_scale"),
    (dict(D=96), fb.FA_ERR_UNSUPPORTED, "headdim"),
    (dict(B=-2), fb.FA_ERR_INVALID_ARG, "batch"),
    (dict(wl=-2), fb.FA_ERR_INVALID_ARG, "window"),
    (dict(q=None), fb.FA_ERR_INVALID_ARG, "q is null"),
    (dict(v=FAKE + 8), fb.FA_ERR_INVALID_ARG, "v is not 16-byte aligned"),
    (dict(out=None), fb.FA_ERR_INVALID_ARG, "out is null"),
    (dict(lse=FAKE + 4), fb.FA_ERR_INVALID_ARG, "lse is not 16-byte aligned"),
    (dict(seqlens=FAKE + 2), fb.FA_ERR_INVALID_ARG, "seqlens_k"),
    # One byte per element: (N + 128) * H * D >= 2^31 needs H = 128 at N = 2^17.
    (dict(H=128, N=1 << 17, D=128), fb.FA_ERR_UNSUPPORTED, "2^31 bytes"),
])
def test_forward_fp8_rejects_before_launch(kw, status, needle):
    lib = fb.load_library()
    assert fwd_fp8(lib, **kw) == status
    assert needle in lib.fa_last_error_message().decode()


def test_fp8_slice_limit_counts_one_byte_per_element():
    lib = fb.load_library()
    # 2-byte elements would exceed 2^31 here; one byte does not: the call gets
    # past the size check and stops at the null lse.
    assert fwd_fp8(lib, H=64, N=1 << 17, D=128, lse=None) == fb.FA_ERR_INVALID_ARG
    assert "lse is null" in lib.fa_last_error_message().decode()


def test_fp8_binding_rejects_other_byte_types():
    import torch
    x = torch.zeros((1, 4, 1, 64), dtype=torch.float8_e5m2)
    with pytest.raises(fb.FaError, match="e4m3"):
        fb.forward_fp8(x, x, x)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """fa_backward_noalloc refuses sizes whose workspace exceeds the static
    scratch before it reads a pointer or touches the GPU; an empty call is
    accepted and does nothing."""
    lib = fb.load_library()
    limit = 128 << 20
    B, H, N, D = 64, 16, 4096, 128
    assert lib.fa_backward_workspace_size(B, H, N, D, fb.FA_DTYPE_BF16) > limit
    st = lib.fa_backward_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                 B, H, N, D, 0.1, 0, -1, -1, fb.FA_DTYPE_BF16, None)
    assert st == fb.FA_ERR_WORKSPACE
    msg = lib.fa_last_error_message().decode()
    assert "no-alloc scratch holds 134217728" in msg, msg
    st = lib.fa_backward_noalloc(None, None, None, None, None, None, None, None, None, None,
                                 0, H, N, D, 0.1, 0, -1, -1, fb.FA_DTYPE_BF16, None)
    assert st == fb.FA_OK
    st = lib.fa_backward_noalloc(None, None, None, None, None, None, None, None, None, None,
                                 1, 1, 16, 96, 0.1, 0, -1, -1, fb.FA_DTYPE_BF16, None)
    assert st == fb.FA_ERR_UNSUPPORTED
