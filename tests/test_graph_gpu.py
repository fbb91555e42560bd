"""The forward and backward captured in one HIP graph (torch.cuda.graph over
the C-ABI calls). The library enqueues kernels only: no allocation, memset or
synchronisation. Each replay follows eager work that rewrites the inputs, and
every replay is compared bitwise with an eager run on the same inputs (the
kernels are deterministic), and the first replay also with the oracle."""

import numpy as np
import pytest
import torch

from exact_io_aware_35_amd import backward, forward, workspace_size
from exact_io_aware_35_amd.inputs import make_case
from oracle import attention_backward, attention_forward

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("B,N,H,D,causal,window,pad", [
    (2, 300, 4, 128, True, (-1, -1), None),
    (3, 257, 2, 64, False, (40, 7), (100, 257)),
])
def test_forward_backward_graph_replays_match_eager(B, N, H, D, causal, window, pad):
    print(f"graph case B{B} N{N} H{H} D{D} causal={causal} window={window} pad={pad}", flush=True)
    cases = [make_case(B, N, H, D, seed=s, backward=True, pad_range=pad) for s in range(5)]
    sk = cases[0]["seqlens_k"]
    sk = None if sk is None else sk.to(DEV)
    q, k, v, do = (cases[0][x].to(DEV) for x in ("q", "k", "v", "dout"))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(workspace_size(B, H, N, D), dtype=torch.uint8, device=DEV)
    kw = dict(causal=causal, window=window, seqlens_k=sk)

    def step():
        forward(q, k, v, out=out, lse=lse, **kw)
        backward(q, k, v, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for r, c in enumerate(cases[1:]):
        # Eager work between replays: new inputs in place, then an eager reference.
        for t, x in ((q, "q"), (k, "k"), (v, "v"), (do, "dout"), (sk, "seqlens_k")):
            if t is not None:
                t.copy_(c[x].to(DEV))
        ref_o, ref_lse = forward(q, k, v, **kw)
        ref = backward(q, k, v, ref_o, ref_lse, do, **kw)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_lse), f"replay {r}: forward"
        for got, want, name in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
            assert torch.equal(got, want), f"replay {r}: {name}"
        if r == 0:
            cq, ck, cv, cdo = (_np(c[x]) for x in ("q", "k", "v", "dout"))
            skn = None if c["seqlens_k"] is None else c["seqlens_k"].numpy()
            o64, l64 = attention_forward(cq, ck, cv, None, causal, window, skn)
            fin = np.isfinite(l64)
            assert np.abs(_np(out) - o64).max() <= 2e-2
            assert np.abs(_np(lse)[fin] - l64[fin]).max() <= 1e-3
            grads = attention_backward(cq, ck, cv, cdo, None, causal, window, skn)
            for got, want in zip((dq, dk, dv), grads):
                assert np.abs(_np(got) - want).max() <= 2e-2
