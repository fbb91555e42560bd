"""GPU parity of the fp16 (IEEE half) path through the C ABI (dtype
FA_DTYPE_F16): the same kernels as bf16 with the 16-bit element type switched,
against the fp64 oracle on identical seeded inputs (cast to fp16 with round to
nearest even). fp16 keeps three more mantissa bits than bf16, so the bf16
bounds (O, dQ, dK, dV 2e-2; LSE 1e-3) hold with room to spare."""

import dataclasses

import numpy as np
import pytest
import torch

from exact_io_aware_35_amd import backward, backward_qkvpacked, forward, forward_qkvpacked
from exact_io_aware_35_amd.inputs import WORKLOADS, make_case, make_inputs
from oracle import attention_backward, attention_forward

from test_parity_gpu import MASKS, assert_close, assert_lse, dev, np64

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE, TOL_G = 2e-2, 1e-3, 2e-2


def fwd_check(d, causal=False, window=(-1, -1), scale=None, alibi=None):
    sk = dev(d["seqlens_k"])
    o, lse = forward(dev(d["q"]), dev(d["k"]), dev(d["v"]), causal=causal, window=window,
                     softmax_scale=scale, seqlens_k=sk,
                     alibi_slopes=None if alibi is None else dev(alibi))
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    ro, rl = attention_forward(np64(d["q"]), np64(d["k"]), np64(d["v"]), scale, causal, window,
                               None if d["seqlens_k"] is None else d["seqlens_k"].numpy(),
                               None if alibi is None else alibi.numpy())
    assert_close(o.cpu(), ro, TOL_O, "O")
    assert_lse(lse.cpu(), rl, TOL_LSE)
    return o, lse


def bwd_check(d, causal=False, window=(-1, -1), scale=None):
    q, k, v, do = dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["dout"])
    sk = dev(d["seqlens_k"])
    o, lse = forward(q, k, v, causal=causal, window=window, softmax_scale=scale, seqlens_k=sk)
    dq, dk, dv = backward(q, k, v, o, lse, do, causal=causal, window=window, softmax_scale=scale,
                          seqlens_k=sk)
    torch.cuda.synchronize()
    assert dq.dtype == dk.dtype == dv.dtype == torch.float16
    ref = attention_backward(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["dout"]), scale,
                             causal, window,
                             None if d["seqlens_k"] is None else d["seqlens_k"].numpy())
    return {name: assert_close(got.cpu(), want, TOL_G, name)
            for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref)}


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=lambda m: "-".join(f"{k}{v}" for k, v in m.items()) or "none")
def test_f16_forward_small(D, mask):
    fwd_check(make_case(2, 300, 3, D, dtype="f16", seed=41), **mask)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", MASKS[:4], ids=lambda m: "-".join(f"{k}{v}" for k, v in m.items()) or "none")
def test_f16_backward_small(D, mask):
    bwd_check(make_case(2, 300, 3, D, dtype="f16", seed=42, backward=True), **mask)


@pytest.mark.parametrize("seqlens,mask", [([300, 17], dict()), ([0, 129], dict(causal=True))])
def test_f16_key_padding(seqlens, mask):
    d = make_case(2, 300, 2, 128, dtype="f16", seed=43, backward=True, seqlens_k=seqlens)
    fwd_check(d, **mask)
    bwd_check(d, **mask)


@pytest.mark.parametrize("N", [1, 63, 65, 257])
def test_f16_lengths(N):
    d = make_case(1, N, 2, 64, dtype="f16", seed=44, backward=True)
    fwd_check(d, causal=True)
    bwd_check(d, causal=True)


def test_f16_large_scores_take_the_exact_path():
    """std-8 Q and K give scores of magnitude ~1e2: with fp16 P operands the
    fast path must hand any tile whose P would leave fp16's range to the exact
    path (the forward's bound on the tile's row sums is 2^15 for fp16)."""
    d = make_case(1, 300, 2, 64, dtype="f16", std=8.0, seed=45)
    d["v"] = d["v"] / 8
    o, _ = fwd_check(d, scale=0.05)
    assert torch.isfinite(o.float()).all()


def test_f16_alibi_and_packed():
    d = make_case(2, 257, 3, 128, dtype="f16", seed=46, backward=True)
    slopes = torch.tensor([0.5, 0.25, 0.125], dtype=torch.float32)
    fwd_check(d, causal=True, alibi=slopes)
    qkv = torch.stack([dev(d["q"]), dev(d["k"]), dev(d["v"])], dim=2).contiguous()
    o1, l1 = forward_qkvpacked(qkv, causal=True)
    o2, l2 = forward(dev(d["q"]), dev(d["k"]), dev(d["v"]), causal=True)
    dqkv = backward_qkvpacked(qkv, o1, l1, dev(d["dout"]), causal=True)
    g2 = backward(dev(d["q"]), dev(d["k"]), dev(d["v"]), o2, l2, dev(d["dout"]), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for i in range(3):
        assert torch.equal(dqkv[:, :, i], g2[i])


@pytest.mark.parametrize("name", ["fwdbwd_bf16_b8h12n1024d64_causal",
                                  "fwdbwd_bf16_b32h16n512d64_keypad"])
def test_f16_workload_fwd_bwd_full(name):
    """The two training-shaped workloads with fp16 inputs, in full."""
    w = dataclasses.replace(WORKLOADS[name], dtype="f16")
    d = make_inputs(w, 0)
    fwd_check(d, w.causal, w.window, w.softmax_scale)
    errs = bwd_check(d, w.causal, w.window, w.softmax_scale)
    print(name, {k: f"{v:.4g}" for k, v in errs.items()})


@pytest.mark.parametrize("name,count", [("fwd_bf16_b2h8n4096d128", 256),
                                        ("fwd_bf16_b1h16n65536d128_causal", 0)])
def test_f16_workload_sampled_rows(name, count):
    """The metric shape and the 64K causal shape with fp16 inputs, at full size: every row
    is computed on the GPU, and sampled rows are compared with the oracle."""
    from oracle import attention_forward_rows
    w = dataclasses.replace(WORKLOADS[name], dtype="f16")
    print(f"f16 {name}", flush=True)
    d = make_inputs(w, 0)
    o, lse = forward(dev(d["q"]), dev(d["k"]), dev(d["v"]), causal=w.causal, window=w.window,
                     softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    o, lse = o.cpu(), lse.cpu()
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    if count:  # workloads without their own row sample: seeded rows plus both ends
        g = torch.Generator().manual_seed(7)
        rows = torch.stack([torch.cat([torch.randperm(w.seqlen, generator=g)[:count],
                                       torch.tensor([0, w.seqlen - 1])]) for _ in range(w.heads)])
    else:
        rows = d["rows"]
    rows = rows.numpy()
    ro, rl = attention_forward_rows(np64(d["q"]), np64(d["k"]), np64(d["v"]), rows,
                                    w.softmax_scale, w.causal, w.window)
    for b in range(w.batch):
        for h in range(w.heads):
            r = rows[h]
            assert_close(o[b, r, h, :], ro[b, h], TOL_O, f"O[b={b},h={h}]")
            assert_lse(lse[b, h, r].numpy().astype(np.float64), rl[b, h], TOL_LSE)
