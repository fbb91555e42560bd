"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
identical seeded inputs.

Tolerances (max-abs): fp32 path 1e-5 on O and LSE; bf16 path 2e-2 on O, dQ,
dK, dV and 1e-3 on LSE. Small cases span several tiles with a ragged tail;
the named workloads run at full size, compared in full where the oracle is
quick and on sampled query rows otherwise.
"""

import numpy as np
import pytest
import torch

from exact_io_aware_35_amd import (backward, backward_qkvpacked, forward, forward_qkvpacked,
                                  workspace_size)
from exact_io_aware_35_amd.inputs import WORKLOADS, make_case, make_inputs
from oracle import attention_backward, attention_forward, attention_forward_rows

pytestmark = pytest.mark.gpu

TOL = {"bf16": dict(o=2e-2, lse=1e-3, grad=2e-2), "f32": dict(o=1e-5, lse=1e-5, grad=1e-5)}
DEV = "cuda:0"


def np64(t):
    return None if t is None else t.float().numpy().astype(np.float64)


def dev(t):
    return None if t is None else t.to(DEV)


def gpu_forward(d, causal, window, scale=None):
    o, lse = forward(dev(d["q"]), dev(d["k"]), dev(d["v"]), causal=causal, window=window,
                     softmax_scale=scale, seqlens_k=dev(d["seqlens_k"]))
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def assert_lse(got, want, tol, what="lse"):
    got = got.numpy().astype(np.float64) if isinstance(got, torch.Tensor) else got
    inf_w, inf_g = np.isneginf(want), np.isneginf(got)
    assert (inf_w == inf_g).all(), f"{what}: -inf rows differ"
    fin = ~inf_w
    err = np.abs(got[fin] - want[fin]).max() if fin.any() else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3g} > {tol}"
    return err


def assert_close(got, want, tol, what, rel=0.0):
    """max |got - want| <= tol (+ rel |want| elementwise, where a test says why)."""
    got = got.float().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else got
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    excess = np.abs(got - want) - rel * np.abs(want)
    err = np.abs(got - want).max()
    assert excess.max() <= tol, f"{what}: max abs err {err:.3g} > {tol} (+{rel} |ref|)"
    return err


# A bf16 output of magnitude x is rounded by up to 2^-8 |x| (half an ulp); at
# |x| >= 8 that alone exceeds the absolute 2e-2 bound. Cases whose structure
# concentrates gradient mass (a steep ALiBi bias funnelling many rows onto the
# last visible key) reach such magnitudes, so their bound adds that rounding.
BF16_HALF_ULP = 2.0 ** -8


def check_forward(d, dtype, causal=False, window=(-1, -1), scale=None):
    o, lse = gpu_forward(d, causal, window, scale)
    ro, rl = attention_forward(np64(d["q"]), np64(d["k"]), np64(d["v"]), scale, causal, window,
                               None if d["seqlens_k"] is None else d["seqlens_k"].numpy())
    t = TOL[dtype]
    assert_close(o, ro, t["o"], "O")
    assert_lse(lse, rl, t["lse"])
    return o, lse


MASKS = [
    dict(),
    dict(causal=True),
    dict(window=(37, 5)),
    dict(window=(0, 0)),
    dict(causal=True, window=(50, 0)),
    dict(window=(-1, 70)),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=lambda m: "-".join(f"{k}{v}" for k, v in m.items()) or "none")
def test_forward_small(dtype, D, mask):
    d = make_case(2, 300, 3, D, dtype=dtype, seed=1)
    check_forward(d, dtype, **mask)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("seqlens,mask", [
    ([300, 17], dict()),
    ([300, 17], dict(causal=True)),
    ([0, 129], dict()),
    ([5, 300], dict(window=(0, 0))),
    ([64, 200], dict(causal=True, window=(20, 0))),
])
def test_forward_key_padding(dtype, seqlens, mask):
    d = make_case(2, 300, 2, 64, dtype=dtype, seed=2, seqlens_k=seqlens)
    check_forward(d, dtype, **mask)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N", [1, 7, 63, 64, 65, 128, 129, 257])
def test_forward_lengths(dtype, N):
    d = make_case(1, N, 2, 128, dtype=dtype, seed=3)
    check_forward(d, dtype)
    check_forward(d, dtype, causal=True)


@pytest.mark.parametrize("shape", [(2, 0, 3, 64), (0, 40, 3, 128)], ids=["no-rows", "no-batch"])
def test_empty_inputs_give_empty_outputs(shape):
    """Zero rows: every call succeeds, launches nothing and returns outputs of
    the right (empty) shapes."""
    from exact_io_aware_35_amd import forward_fp8
    dev = "cuda:0"
    q, k, v, do = (torch.zeros(shape, dtype=torch.bfloat16, device=dev) for _ in range(4))
    o, lse = forward(q, k, v, causal=True)
    assert o.shape == shape and lse.shape == (shape[0], shape[2], shape[1])
    dq, dk, dv = backward(q, k, v, o, lse, do, causal=True)
    assert dq.shape == dk.shape == dv.shape == shape
    b8 = torch.zeros(shape, dtype=torch.uint8, device=dev)
    o8, lse8 = forward_fp8(b8, b8, b8, 1.0, 1.0, 1.0)
    assert o8.shape == shape and lse8.shape == lse.shape
    torch.cuda.synchronize()


def test_forward_large_magnitude_and_scale():
    """Scores of magnitude ~1e2 (std-8 Q, K) exercise the max shift: without
    it exp would overflow fp32. V is scaled back to std 1 (exact: a power of
    two) so that |O| stays where bf16 output rounding is below 2e-2.

    The fp32 path's 1e-5 bound is for N(0,1) inputs. Here the fp32 score
    itself carries the dot-product rounding error |delta| <= gamma_D c
    sum_d |q_d k_d| with gamma_D = D u / (1 - D u), u = 2^-24 (the standard
    bound for a length-D dot product), plus a few roundings of the scaled
    score and of the log. A score error delta moves O by at most
    2 max|delta| max|V| and LSE by max|delta|; the fp32 tolerances add those
    terms to 1e-5."""
    for dtype, n, scales in (("bf16", 300, (None, 0.05)), ("f32", 200, (0.3,))):
        d = make_case(1, n, 2, 64, dtype=dtype, std=8.0, seed=4)
        d["v"] = d["v"] / 8
        for scale in scales:
            c = scale if scale is not None else 0.125
            q64, k64 = d["q"].double(), d["k"].double()
            smax = c * float(torch.einsum("bihd,bjhd->bhij", q64, k64).abs().max())
            sabs = c * float(torch.einsum("bihd,bjhd->bhij", q64.abs(), k64.abs()).max())
            u, D = 2.0 ** -24, 64
            delta = D * u / (1 - D * u) * sabs + 4 * u * smax
            vmax = float(d["v"].double().abs().max())
            tol_o = TOL[dtype]["o"] + (2 * delta * vmax if dtype == "f32" else 0.0)
            tol_l = TOL[dtype]["lse"] + (delta if dtype == "f32" else 0.0)
            for causal in (False, True):
                o, lse = gpu_forward(d, causal, (-1, -1), scale)
                ro, rl = attention_forward(np64(d["q"]), np64(d["k"]), np64(d["v"]), scale,
                                           causal)
                assert smax > 89.0       # exp(max score) alone would overflow fp32
                assert_close(o, ro, tol_o, "O")
                assert_lse(lse, rl, tol_l)


def test_forward_zero_query_is_mean_of_visible_values():
    d = make_case(1, 190, 2, 64, dtype="bf16", seed=5)
    d["q"] = torch.zeros_like(d["q"])
    o, lse = gpu_forward(d, True, (-1, -1))
    n = torch.arange(1, 191, dtype=torch.float64)
    assert torch.allclose(lse.double(), torch.log(n).expand(1, 2, 190), atol=1e-3)
    prefix = torch.cumsum(d["v"].double(), dim=1) / n[None, :, None, None]
    assert (o.double() - prefix).abs().max() < 2e-2


def test_forward_is_deterministic_and_writes_everything():
    d = make_case(2, 333, 3, 128, dtype="bf16", seed=6)
    q, k, v = dev(d["q"]), dev(d["k"]), dev(d["v"])
    o1 = torch.full_like(q, float("nan"))
    l1 = torch.full((2, 3, 333), float("nan"), device=DEV)
    forward(q, k, v, causal=True, out=o1, lse=l1)
    o2, l2 = forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_forward_on_side_stream():
    d = make_case(1, 257, 2, 64, dtype="bf16", seed=7)
    s = torch.cuda.Stream()
    q, k, v = dev(d["q"]), dev(d["k"]), dev(d["v"])
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = forward(q, k, v, stream=s)
    s.synchronize()
    ro, rl = attention_forward(np64(d["q"]), np64(d["k"]), np64(d["v"]))
    assert_close(o.cpu(), ro, 2e-2, "O")
    assert_lse(lse.cpu(), rl, 1e-3)


# ---------------------------------------------------------------- backward

def check_backward(d, causal=False, window=(-1, -1), scale=None):
    q, k, v, do = dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["dout"])
    sk = dev(d["seqlens_k"])
    o, lse = forward(q, k, v, causal=causal, window=window, softmax_scale=scale, seqlens_k=sk)
    dq, dk, dv = backward(q, k, v, o, lse, do, causal=causal, window=window,
                          softmax_scale=scale, seqlens_k=sk)
    torch.cuda.synchronize()
    ref = attention_backward(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["dout"]), scale,
                             causal, window,
                             None if d["seqlens_k"] is None else d["seqlens_k"].numpy())
    errs = {}
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        errs[name] = assert_close(got.cpu(), want, TOL["bf16"]["grad"], name)
    return errs


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=lambda m: "-".join(f"{k}{v}" for k, v in m.items()) or "none")
def test_backward_small(D, mask):
    d = make_case(2, 300, 3, D, dtype="bf16", seed=11, backward=True)
    check_backward(d, **mask)


@pytest.mark.parametrize("seqlens,mask", [
    ([300, 17], dict()),
    ([200, 300], dict(causal=True)),
    ([5, 300], dict(window=(0, 0))),
    ([0, 100], dict()),
])
def test_backward_key_padding(seqlens, mask):
    d = make_case(2, 300, 2, 64, dtype="bf16", seed=12, backward=True, seqlens_k=seqlens)
    check_backward(d, **mask)


@pytest.mark.parametrize("N", [1, 33, 64, 100, 129])
def test_backward_lengths(N):
    d = make_case(1, N, 2, 64, dtype="bf16", seed=13, backward=True)
    check_backward(d, causal=True)
    check_backward(d)


@pytest.mark.parametrize("mask", [dict(), dict(causal=True), dict(causal=True, window=(300, 0)),
                                  dict(window=(90, 400))],
                         ids=["none", "causal", "causal-window300", "window90-400"])
def test_backward_d128_several_blocks(mask):
    # 1000 keys: 8 key blocks of 128 (the last ragged) and 4 query blocks.
    d = make_case(1, 1000, 2, 128, dtype="bf16", seed=15, backward=True)
    check_backward(d, **mask)


def test_backward_d128_key_padding():
    d = make_case(2, 700, 2, 128, dtype="bf16", seed=16, backward=True, seqlens_k=[650, 129])
    check_backward(d, causal=True)
    check_backward(d)


def test_window_at_or_past_seqlen_is_unbounded():
    # A window bound >= seqlen excludes nothing; the library treats it as -1.
    d = make_case(1, 200, 2, 64, dtype="bf16", seed=17, backward=True)
    q, k, v, do = dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["dout"])
    big = 2 ** 31 - 1
    ref_o, ref_lse = forward(q, k, v)
    ref_g = backward(q, k, v, ref_o, ref_lse, do)
    for window in [(big, big), (200, 200), (200, -1), (-1, big)]:
        o, lse = forward(q, k, v, window=window)
        g = backward(q, k, v, o, lse, do, window=window)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse), window
        for a, b in zip(g, ref_g):
            assert torch.equal(a, b), window


def test_backward_is_deterministic_and_writes_everything():
    d = make_case(2, 300, 2, 64, dtype="bf16", seed=14, backward=True)
    q, k, v, do = dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["dout"])
    o, lse = forward(q, k, v, causal=True)
    outs = []
    for _ in range(2):
        g = [torch.full_like(q, float("nan")) for _ in range(3)]
        ws = torch.full((workspace_size(2, 2, 300, 64),), 255, dtype=torch.uint8, device=DEV)
        backward(q, k, v, o, lse, do, causal=True, dq=g[0], dk=g[1], dv=g[2], workspace=ws)
        outs.append(g)
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert not torch.isnan(a).any()
        assert torch.equal(a, b)


# ---------------------------------------------------------------- named workloads, full size

def _rows_compare(w, d, o, lse):
    rows = d["rows"].numpy()
    ro, rl = attention_forward_rows(d["q"].float().numpy(), d["k"].float().numpy(),
                                    d["v"].float().numpy(), rows, w.softmax_scale, w.causal,
                                    w.window,
                                    None if d["seqlens_k"] is None else d["seqlens_k"].numpy())
    t = TOL[w.dtype]
    for b in range(w.batch):
        for h in range(w.heads):
            r = rows[h]
            assert_close(o[b, r, h, :], ro[b, h], t["o"], f"O[b={b},h={h}]")
            assert_lse(lse[b, h, r].numpy().astype(np.float64), rl[b, h], t["lse"])


def _sample_rows(n, heads, count, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.stack([torch.randperm(n, generator=g)[:count] for _ in range(heads)])


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", ["fwd_f32_b1h1n256d64"])
def test_workload_small_full(name, seed):
    w = WORKLOADS[name]
    d = make_inputs(w, seed)
    check_forward(d, w.dtype, w.causal, w.window, w.softmax_scale)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_workload_b2h8n4096d128_full(seed):
    """The metric shape, launched as the benchmark launches it: O and LSE of
    every query row of all 16 (batch, head) slices against the oracle (the
    whole blocked output against standard attention, as [scratch] §3.2
    verifies its implementation)."""
    w = WORKLOADS["fwd_bf16_b2h8n4096d128"]
    print(f"metric shape full compare, seed {seed}", flush=True)
    d = make_inputs(w, seed)
    check_forward(d, w.dtype, w.causal, w.window, w.softmax_scale)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", ["fwdbwd_bf16_b8h12n1024d64_causal",
                                  "fwdbwd_bf16_b32h16n512d64_keypad"])
def test_workload_fwd_bwd_full(name, seed):
    w = WORKLOADS[name]
    d = make_inputs(w, seed)
    check_forward(d, w.dtype, w.causal, w.window, w.softmax_scale)
    errs = check_backward(d, w.causal, w.window, w.softmax_scale)
    print(name, seed, {k: f"{v:.4g}" for k, v in errs.items()})


@pytest.mark.parametrize("causal", [False, True])
def test_backward_b2h8n4096d128_full(causal):
    """Full-size backward in the launch configuration the benchmark times:
    every gradient of all 16 (batch, head) slices against the oracle."""
    w = WORKLOADS["fwd_bf16_b2h8n4096d128"]
    print(f"metric shape backward, causal {causal}", flush=True)
    d = make_inputs(w, 0)
    g = torch.Generator().manual_seed(5)
    d["dout"] = torch.randn(d["q"].shape, generator=g).to(torch.bfloat16)
    check_backward(d, causal, (-1, -1), w.softmax_scale)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", ["fwd_bf16_b1h16n65536d128_causal",
                                  "fwd_bf16_b1h16n65536d128_window4096"])
def test_workload_long_context_sampled_rows(name, seed):
    w = WORKLOADS[name]
    print(f"long context {name} seed {seed}", flush=True)
    d = make_inputs(w, seed)
    o, lse = gpu_forward(d, w.causal, w.window, w.softmax_scale)
    _rows_compare(w, d, o, lse)


# ---------------------------------------------------------------- ALiBi and packed qkv

def geometric_slopes(heads):
    """The usual ALiBi slopes 2^(-8 (h + 1) / heads), fp32."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / heads) for h in range(heads)],
                        dtype=torch.float32)


SLOPE_CASES = {
    "per-head": lambda B, H: geometric_slopes(H),
    "per-batch-head": lambda B, H: torch.tensor([[0.0, 1.0, 0.05], [0.3, 0.0, 2.0 ** -6]][:B],
                                                dtype=torch.float32)[:, :H],
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("slopes", sorted(SLOPE_CASES))
@pytest.mark.parametrize("mask", [dict(), dict(causal=True), dict(window=(37, 5))],
                         ids=["none", "causal", "window37-5"])
def test_forward_alibi(dtype, D, slopes, mask):
    d = make_case(2, 300, 3, D, dtype=dtype, seed=21)
    sl = SLOPE_CASES[slopes](2, 3)
    o, lse = forward(dev(d["q"]), dev(d["k"]), dev(d["v"]), alibi_slopes=dev(sl), **mask)
    torch.cuda.synchronize()
    ro, rl = attention_forward(np64(d["q"]), np64(d["k"]), np64(d["v"]), alibi_slopes=sl.numpy(),
                               **mask)
    assert_close(o.cpu(), ro, TOL[dtype]["o"], "O")
    assert_lse(lse.cpu(), rl, TOL[dtype]["lse"])


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("slopes", sorted(SLOPE_CASES))
@pytest.mark.parametrize("mask", [dict(), dict(causal=True), dict(causal=True, window=(50, 0))],
                         ids=["none", "causal", "causal-window50"])
def test_backward_alibi(D, slopes, mask):
    d = make_case(2, 300, 3, D, dtype="bf16", seed=22, backward=True, seqlens_k=[300, 211])
    sl = SLOPE_CASES[slopes](2, 3)
    q, k, v, do, sk = dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["dout"]), dev(d["seqlens_k"])
    o, lse = forward(q, k, v, seqlens_k=sk, alibi_slopes=dev(sl), **mask)
    grads = backward(q, k, v, o, lse, do, seqlens_k=sk, alibi_slopes=dev(sl), **mask)
    torch.cuda.synchronize()
    ref = attention_backward(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["dout"]),
                             seqlens_k=d["seqlens_k"].numpy(), alibi_slopes=sl.numpy(), **mask)
    for name, got, want in zip(("dQ", "dK", "dV"), grads, ref):
        assert_close(got.cpu(), want, TOL["bf16"]["grad"], name, rel=BF16_HALF_ULP)


def test_alibi_zero_slopes_equal_no_alibi():
    d = make_case(1, 333, 2, 128, dtype="bf16", seed=23, backward=True)
    q, k, v, do = dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["dout"])
    zero = torch.zeros(2, dtype=torch.float32, device=DEV)
    o0, l0 = forward(q, k, v, causal=True)
    o1, l1 = forward(q, k, v, causal=True, alibi_slopes=zero)
    g0 = backward(q, k, v, o0, l0, do, causal=True)
    g1 = backward(q, k, v, o1, l1, do, causal=True, alibi_slopes=zero)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_qkvpacked_equals_separate_tensors(dtype, D):
    # The packed layout only changes strides: results must be bitwise those of
    # three separate tensors (which the other tests compare with the oracle).
    d = make_case(2, 257, 3, D, dtype=dtype, seed=24, backward=True, seqlens_k=[257, 100])
    q, k, v, sk = dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["seqlens_k"])
    qkv = torch.stack([q, k, v], dim=2).contiguous()
    sl = dev(geometric_slopes(3))
    for kw in [dict(causal=True), dict(window=(40, 7), alibi_slopes=sl)]:
        o1, l1 = forward(q, k, v, seqlens_k=sk, **kw)
        o2, l2 = forward_qkvpacked(qkv, seqlens_k=sk, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        if dtype == "bf16":
            do = dev(d["dout"])
            g = backward(q, k, v, o1, l1, do, seqlens_k=sk, **kw)
            dqkv = torch.full_like(qkv, float("nan"))
            backward_qkvpacked(qkv, o2, l2, do, seqlens_k=sk, dqkv=dqkv, **kw)
            torch.cuda.synchronize()
            for i in range(3):
                assert torch.equal(dqkv[:, :, i], g[i])


def test_qkvpacked_alibi_against_oracle():
    d = make_case(2, 300, 2, 128, dtype="bf16", seed=25, backward=True)
    qkv = torch.stack([dev(d["q"]), dev(d["k"]), dev(d["v"])], dim=2).contiguous()
    sl = torch.tensor([[0.5, 0.01], [0.0, 0.2]], dtype=torch.float32)
    o, lse = forward_qkvpacked(qkv, causal=True, alibi_slopes=dev(sl))
    dqkv = backward_qkvpacked(qkv, o, lse, dev(d["dout"]), causal=True, alibi_slopes=dev(sl))
    torch.cuda.synchronize()
    args = (np64(d["q"]), np64(d["k"]), np64(d["v"]))
    ro, rl = attention_forward(*args, causal=True, alibi_slopes=sl.numpy())
    assert_close(o.cpu(), ro, TOL["bf16"]["o"], "O")
    assert_lse(lse.cpu(), rl, TOL["bf16"]["lse"])
    ref = attention_backward(*args, np64(d["dout"]), causal=True, alibi_slopes=sl.numpy())
    for i, name in enumerate(("dQ", "dK", "dV")):
        assert_close(dqkv[:, :, i].cpu(), ref[i], TOL["bf16"]["grad"], name, rel=BF16_HALF_ULP)


def test_autograd_function_matches_direct_calls_and_oracle():
    """The torch.autograd wrapper returns the C-ABI forward's O and, through
    loss.backward(), exactly the gradients a direct fa_backward call gives for
    dO = d loss / d O; those match the oracle's."""
    from exact_io_aware_35_amd import flash_attention
    d = make_case(2, 260, 3, 64, dtype="bf16", seed=31, backward=True, seqlens_k=[260, 190])
    q, k, v = (dev(d[x]).requires_grad_() for x in ("q", "k", "v"))
    sk = dev(d["seqlens_k"])
    out = flash_attention(q, k, v, causal=True, seqlens_k=sk)
    do = dev(d["dout"])
    (out.float() * do.float()).sum().backward()
    torch.cuda.synchronize()
    o2, lse2 = forward(dev(d["q"]), dev(d["k"]), dev(d["v"]), causal=True, seqlens_k=sk)
    g2 = backward(dev(d["q"]), dev(d["k"]), dev(d["v"]), o2, lse2, do, causal=True, seqlens_k=sk)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), o2)
    for got, want in zip((q.grad, k.grad, v.grad), g2):
        assert torch.equal(got, want)
    rg = attention_backward(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["dout"]),
                            causal=True, seqlens_k=d["seqlens_k"].numpy())
    for name, got, want in zip(("dQ", "dK", "dV"), (q.grad, k.grad, v.grad), rg):
        assert_close(got.cpu(), want, TOL["bf16"]["grad"], name)


def test_forward_and_backward_keep_memory_linear_in_n():
    """The memory side of the method ([interview] section "Online Softmax":
    the N x N score and probability matrices are never stored, so memory
    drops from O(N^2) to O(N)): at N = 32768 a head's fp32 score matrix would
    take 4 GiB, yet a forward into preallocated outputs and a backward with a
    preallocated workspace leave the device's free memory exactly unchanged,
    and the backward workspace grows linearly with N."""
    B, H, N, D = 1, 2, 32768, 128
    g = torch.Generator(device=DEV).manual_seed(0)
    q, k, v, do = (torch.randn((B, N, H, D), generator=g, device=DEV).to(torch.bfloat16)
                   for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(workspace_size(B, H, N, D), dtype=torch.uint8, device=DEV)
    for _ in range(2):  # the first round loads code objects
        forward(q, k, v, causal=True, out=o, lse=lse)
        backward(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info(DEV)[0]
    forward(q, k, v, causal=True, out=o, lse=lse)
    backward(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info(DEV)[0] == free_before
    sizes = [workspace_size(B, H, n, D) for n in (4096, 8192, 16384, 32768)]
    for a, b in zip(sizes, sizes[1:]):
        assert abs(b / a - 2.0) < 0.01
    assert sizes[-1] < 2 * 4 * B * H * N * D  # a few copies of the inputs, no N^2 term


def test_alibi_workload_b2h8n4096d128_sampled_rows():
    """ALiBi (the usual per-head slopes) at the metric shape, full size, on sampled rows."""
    w = WORKLOADS["fwd_bf16_b2h8n4096d128"]
    d = make_inputs(w, 3)
    slopes = geometric_slopes(w.heads)
    o, lse = forward(dev(d["q"]), dev(d["k"]), dev(d["v"]), softmax_scale=w.softmax_scale,
                     alibi_slopes=dev(slopes))
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    rows = torch.cat([_sample_rows(4096, w.heads, 128, 31),
                      torch.tensor([[0, 2047, 4095]] * w.heads)], dim=1).numpy()
    ro, rl = attention_forward_rows(np64(d["q"]), np64(d["k"]), np64(d["v"]), rows,
                                    w.softmax_scale, alibi_slopes=slopes.numpy())
    for b in range(w.batch):
        for h in range(w.heads):
            r = rows[h]
            assert_close(o[b, r, h, :], ro[b, h], TOL["bf16"]["o"], f"O[b={b},h={h}]")
            assert_lse(lse[b, h, r].numpy().astype(np.float64), rl[b, h], TOL["bf16"]["lse"])


# ---------------------------------------------------------------- operand range of the backward

RANGE_CASES = {
    # dtype: exponents (Q, K, V, dO) applied to a standard case. bf16: Q and V
    # far above fp16's 65504, K and dO far below its normal range (gradients
    # around 1e-7). fp16: V and dO large enough that dP = dO V^T, unscaled,
    # would leave fp16's range in dS.
    "bf16": (20, -20, 17, -24),
    "f16": (0, 0, 6, 6),
}


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("alibi", [False, True], ids=["plain", "alibi"])
def test_backward_operand_range(dtype, D, alibi):
    """Inputs that are exact power-of-two multiples of a standard case,
    Q 2^a, K 2^b, V 2^c, dO 2^d, give exactly the standard case's results
    times the matching powers: O 2^c and the same LSE; dV 2^d, dK 2^(a+c+d),
    dQ 2^(b+c+d) (S is unchanged, dP, D and dS carry 2^(c+d)). The backward
    rescales each slice's fp16 operand copies by a power of two when its
    maximum leaves [2^-6, 8] (into [4, 8)), so with the standard slices'
    maxima in [4, 8) the scaled case runs on the same fp16 operands and must
    match bitwise; both also match the oracle, with the tolerance scaled like
    the result ([scratch] §5.2, keeping intermediates inside the format's
    range)."""
    ea, eb, ec, ed = RANGE_CASES[dtype]
    d = make_case(2, 300, 3, D, dtype=dtype, seed=51, backward=True, seqlens_k=[300, 211])
    # Bring each (b, h) slice's largest magnitude into [4, 8) by a power of
    # two (exact), where the scaled case's copies land too: both cases then
    # run on the same fp16 operands (fp16 subnormals would not scale exactly).
    for x in ("q", "k", "v", "dout"):
        t = d[x].double()
        m = t.abs().amax(dim=(1, 3), keepdim=True)
        d[x] = (t * torch.exp2(2.0 - torch.floor(torch.log2(m)))).to(d[x].dtype)
        m = d[x].double().abs().amax(dim=(1, 3))
        assert ((m >= 4) & (m < 8)).all()
    mask = dict(causal=True)
    sl = dev(geometric_slopes(3)) if alibi else None
    tdt = d["q"].dtype
    sc = lambda t, e: (t.double() * 2.0 ** e).to(tdt)
    std = [dev(d[x]) for x in ("q", "k", "v", "dout")]
    big = [dev(sc(d[x], e)) for x, e in zip(("q", "k", "v", "dout"), (ea, eb, ec, ed))]
    for t, s_, e in zip(big, std, (ea, eb, ec, ed)):  # the scaling itself is exact
        assert torch.equal(t.double(), s_.double() * 2.0 ** e)
    sk = dev(d["seqlens_k"])
    runs = []
    for q, k, v, do in (std, big):
        o, lse = forward(q, k, v, seqlens_k=sk, alibi_slopes=sl, **mask)
        g = backward(q, k, v, o, lse, do, seqlens_k=sk, alibi_slopes=sl, **mask)
        runs.append((o, lse, *g))
    torch.cuda.synchronize()
    (o0, l0, dq0, dk0, dv0), (o1, l1, dq1, dk1, dv1) = runs
    assert torch.equal(l1, l0)
    exps = {"O": ec, "dQ": eb + ec + ed, "dK": ea + ec + ed, "dV": ed}
    # An fp16 result in fp16's subnormal range (below 2^-14) is rounded on an
    # absolute grid of 2^-24, which does not scale: there the scaled result
    # may differ by one such step, times the power of two.
    sub = 2.0 ** -24 if dtype == "f16" else 0.0
    for name, a, b in (("O", o1, o0), ("dQ", dq1, dq0), ("dK", dk1, dk0), ("dV", dv1, dv0)):
        s = 2.0 ** exps[name]
        err = (a.double() - b.double() * s).abs()
        lim = torch.where(b.double().abs() < 2.0 ** -14, sub * s, 0.0)
        assert (err <= lim).all(), f"{name} is not the standard result times 2^{exps[name]}"
    f64 = lambda t: t.double().cpu().numpy()
    ref = attention_backward(*(f64(t) for t in big), seqlens_k=d["seqlens_k"].numpy(),
                             alibi_slopes=None if sl is None else sl.cpu().numpy(), **mask)
    # The normalised slices are larger than N(0, 1) draws, and so are the
    # gradients: the bound adds the output's own rounding (2^-8 |ref|, as in
    # the ALiBi cases).
    for name, got, want in zip(("dQ", "dK", "dV"), (dq1, dk1, dv1), ref):
        s = 2.0 ** exps[name]
        assert_close(got.cpu() / s, want / s, TOL["bf16"]["grad"], name, rel=BF16_HALF_ULP)
