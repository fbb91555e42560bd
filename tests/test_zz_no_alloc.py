"""fa_backward_noalloc (the backward for callers that cannot allocate) against
fa_backward with a caller workspace, through the C ABI: two calls in a row,
the second smaller, each compared with the regular entry point's gradients
and with the oracle."""

import numpy as np
import pytest
import torch

from exact_io_aware_35_amd import backward, backward_noalloc, forward
from exact_io_aware_35_amd.inputs import make_case
from oracle import attention_backward

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_noalloc_backward_matches_workspace_backward(dtype):
    cases = [  # the second call is smaller, so stale scratch contents would show
        dict(B=2, N=700, H=3, D=128, seed=41, causal=True, seqlens=[700, 333], window=(-1, -1)),
        dict(B=1, N=190, H=2, D=64, seed=42, causal=False, seqlens=None, window=(50, 7)),
    ]
    for c in cases:
        print(f"no-alloc case {c} {dtype}", flush=True)
        d = make_case(c["B"], c["N"], c["H"], c["D"], dtype=dtype, seed=c["seed"], backward=True,
                      seqlens_k=c["seqlens"])
        q, k, v, do = (d[x].to(DEV) for x in ("q", "k", "v", "dout"))
        sk = None if d["seqlens_k"] is None else d["seqlens_k"].to(DEV)
        kw = dict(causal=c["causal"], window=c["window"], seqlens_k=sk)
        o, lse = forward(q, k, v, **kw)
        want = backward(q, k, v, o, lse, do, **kw)
        got = [torch.full_like(q, float("nan")) for _ in range(3)]
        backward_noalloc(q, k, v, o, lse, do, dq=got[0], dk=got[1], dv=got[2], **kw)
        torch.cuda.synchronize()
        ref = attention_backward(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["dout"]),
                                 causal=c["causal"], window=c["window"],
                                 seqlens_k=None if c["seqlens"] is None else c["seqlens"])
        for name, g, w, r in zip(("dQ", "dK", "dV"), got, want, ref):
            g64, w64 = np64(g), np64(w)
            assert np.isfinite(g64).all(), name
            assert np.abs(g64 - w64).max() <= TOL, name
            assert np.abs(g64 - r).max() <= TOL, name
        # dK and dV come from the same kernels on the same inputs: bitwise equal.
        assert torch.equal(got[1], want[1]) and torch.equal(got[2], want[2])
