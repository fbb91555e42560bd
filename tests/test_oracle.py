"""Pins for the fp64 CPU oracle (no GPU).

Each test checks the oracle against something other than itself: values the
pages print, closed forms, brute-force enumeration, the blocked online
recurrence, finite differences, and library routines on special cases.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (attention_backward, attention_forward,
                    attention_forward_rows, blocked_online_forward,
                    online_softmax_trace, visible_mask, visible_pair_count)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# ---------------------------------------------------------------- worked example

def _golden_example():
    with open(os.path.join(GOLDEN, "online_softmax_worked_example.json")) as f:
        return json.load(f)


def test_worked_example_intermediates():
    g = _golden_example()
    pr = g["printed"]
    tol = 0.5 * 10 ** -g["printed_decimals"] + 1e-9
    _, tr = online_softmax_trace(g["scores"], g["block"])
    b1, b2 = tr
    assert b1["block_max"] == pr["block1_max"]
    np.testing.assert_allclose(b1["e_local"], pr["block1_e"], atol=tol)
    assert abs(b1["l_local"] - pr["block1_l"]) <= tol
    np.testing.assert_allclose(b1["local_softmax"], pr["block1_local_softmax"], atol=tol)
    assert b2["m"] == pr["block2_running_max"]
    assert abs(b2["l_old_rescaled"] - pr["block1_l_rescaled"]) <= tol
    assert abs(b2["l_block"] - pr["block2_l"]) <= tol
    assert abs(b2["l"] - pr["l_total"]) <= tol


def _closed_form_softmax(x):
    e = [math.exp(t) for t in x]
    s = sum(e)
    return [t / s for t in e], math.log(s)


def test_worked_example_final_vector_by_definition():
    """The oracle's P row for scores [2,1,5,3] equals exp(x)/sum exp(x)."""
    g = _golden_example()
    x = g["scores"]
    want, want_lse = _closed_form_softmax(x)
    # Scores [2,1,5,3] for query 0: q0 = e0, k_j = x_j e0, scale 1; V = I.
    n = 4
    q = np.zeros((1, n, 1, n)); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, n, 1, n)); k[0, :, 0, 0] = x
    v = np.eye(n).reshape(1, n, 1, n)
    o, lse = attention_forward(q, k, v, softmax_scale=1.0)
    np.testing.assert_allclose(o[0, 0, 0], want, rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 0] - want_lse) < 1e-14
    # The recurrence gives the same vector.
    p, _ = online_softmax_trace(x, 2)
    np.testing.assert_allclose(p, want, atol=1e-15)
    # The page's own third entry (1 / l_total) agrees with the definition.
    assert abs(want[2] - g["printed"]["final_softmax"][2]) < 5e-4


def test_worked_example_printed_vector_is_the_diagnosed_mistake():
    """Documents why the printed final vector differs: p1, p2 carry a spurious
    factor l1 (e1 * l1_rescaled / l_total) and p4 is 1 minus the others."""
    g = _golden_example()
    pr = g["printed"]["final_softmax"]
    _, (b1, b2) = online_softmax_trace(g["scores"], 2)
    wrong12 = b1["e_local"] * b2["l_old_rescaled"] / b2["l"]
    np.testing.assert_allclose(wrong12, pr[:2], atol=5e-4)
    assert abs((1 - wrong12.sum() - 1 / b2["l"]) - pr[3]) < 1e-3
    want, _ = _closed_form_softmax(g["scores"])
    assert abs(want[0] - pr[0]) > 1e-2          # the printed vector is not softmax


# ---------------------------------------------------------------- masks

def _brute_visible(n, causal, wl, wr, key_len):
    out = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            ok = True
            if causal and not (j <= i):
                ok = False
            if wl >= 0 and j < i - wl:
                ok = False
            if wr >= 0 and j > i + wr:
                ok = False
            if j >= key_len:
                ok = False
            out[i, j] = ok
    return out


MASK_CASES = [(False, -1, -1, 37), (True, -1, -1, 37), (False, 3, 5, 37),
              (True, 4, -1, 37), (True, 4, 0, 37), (False, 0, 0, 37),
              (False, -1, 2, 20), (True, -1, -1, 11), (False, 7, -1, 0),
              (True, 0, 0, 37)]


@pytest.mark.parametrize("causal,wl,wr,kl", MASK_CASES)
def test_mask_brute_force(causal, wl, wr, kl):
    n = 37
    got = visible_mask(n, n, causal, wl, wr, kl)
    assert (got == _brute_visible(n, causal, wl, wr, kl)).all()
    assert visible_pair_count(n, causal, (wl, wr), [kl]) == int(got.sum())


def test_mask_rows_subset():
    n = 50
    rows = np.array([0, 7, 49, 13])
    full = visible_mask(n, n, True, 6, 0, 40)
    part = visible_mask(len(rows), n, True, 6, 0, 40, q_pos=rows)
    assert (part == full[rows]).all()


# ---------------------------------------------------------------- closed forms

def _count_visible_rows(n, causal, wl, wr, kl):
    return _brute_visible(n, causal, wl, wr, kl).sum(axis=1)


@pytest.mark.parametrize("causal,wl,wr,kl", MASK_CASES)
def test_zero_query_gives_mean_of_visible_values(causal, wl, wr, kl):
    """Q = 0 makes every visible score 0, so P is uniform over the visible
    keys: O_i = mean of visible V rows and LSE_i = ln(#visible_i)."""
    n, d = 37, 5
    q = np.zeros((1, n, 1, d))
    k = rnd((1, n, 1, d), 1)
    v = rnd((1, n, 1, d), 2)
    o, lse = attention_forward(q, k, v, causal=causal, window=(wl, wr),
                               seqlens_k=[kl])
    vis = _brute_visible(n, causal, wl, wr, kl)
    cnt = vis.sum(axis=1)
    for i in range(n):
        if cnt[i] == 0:
            assert (o[0, i, 0] == 0).all() and lse[0, 0, i] == -np.inf
            continue
        want = sum(v[0, j, 0] for j in range(n) if vis[i, j]) / cnt[i]
        np.testing.assert_allclose(o[0, i, 0], want, atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(cnt[i])) < 1e-14


def test_rows_sum_to_one():
    """With V = 1 every visible row of O is sum_j P_ij = 1."""
    n, d = 64, 16
    q, k = rnd((2, n, 3, d), 3, 2.0), rnd((2, n, 3, d), 4, 2.0)
    v = np.ones((2, n, 3, d))
    for causal, win in [(False, (-1, -1)), (True, (-1, -1)), (False, (5, 9))]:
        o, _ = attention_forward(q, k, v, causal=causal, window=win)
        np.testing.assert_allclose(o, 1.0, atol=1e-14)


def test_causal_first_row_and_window_zero():
    n, d = 33, 8
    q, k, v = rnd((1, n, 2, d), 5), rnd((1, n, 2, d), 6), rnd((1, n, 2, d), 7)
    c = 0.3
    o, lse = attention_forward(q, k, v, softmax_scale=c, causal=True)
    np.testing.assert_allclose(o[0, 0], v[0, 0], atol=1e-15)
    np.testing.assert_allclose(lse[0, :, 0], c * (q[0, 0] * k[0, 0]).sum(-1), atol=1e-14)
    o, lse = attention_forward(q, k, v, softmax_scale=c, window=(0, 0))
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse, c * np.einsum("bnhd,bnhd->bhn", q, k), atol=1e-13)


def test_single_key():
    q, k, v = rnd((3, 1, 2, 8), 8), rnd((3, 1, 2, 8), 9), rnd((3, 1, 2, 8), 10)
    o, lse = attention_forward(q, k, v)
    np.testing.assert_allclose(o, v, atol=1e-15)


def test_default_scale_is_inverse_sqrt_headdim():
    q, k, v = rnd((1, 9, 1, 16), 11), rnd((1, 9, 1, 16), 12), rnd((1, 9, 1, 16), 13)
    o1, l1 = attention_forward(q, k, v)
    o2, l2 = attention_forward(q, k, v, softmax_scale=0.25)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_key_permutation_invariance():
    """Without masks, permuting keys and values together leaves O unchanged
    (catches a transposed or mis-indexed operand)."""
    q, k, v = rnd((1, 40, 2, 8), 14), rnd((1, 40, 2, 8), 15), rnd((1, 40, 2, 8), 16)
    perm = np.random.default_rng(0).permutation(40)
    o1, l1 = attention_forward(q, k, v)
    o2, l2 = attention_forward(q, k[:, perm], v[:, perm])
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


# ---------------------------------------------------------------- library special case

def _sdpa_fp64(q, k, v, scale, causal=False, key_len=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3)))
    B, N = q.shape[:2]
    mask = None
    if key_len is not None:
        mask = torch.zeros(B, 1, N, N, dtype=torch.bool)
        for b in range(B):
            mask[b, :, :, : key_len[b]] = True
        if causal:
            mask &= torch.ones(N, N, dtype=torch.bool).tril()
        causal = False
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=mask, is_causal=causal, scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("std", [1.0, 8.0])
def test_matches_torch_sdpa_fp64(causal, std):
    q, k, v = rnd((2, 70, 3, 16), 20, std), rnd((2, 70, 3, 16), 21, std), rnd((2, 70, 3, 16), 22)
    o, lse = attention_forward(q, k, v, causal=causal)
    np.testing.assert_allclose(o, _sdpa_fp64(q, k, v, 0.25, causal), atol=1e-12)
    assert np.isfinite(lse).all()


def test_matches_torch_sdpa_fp64_padding():
    q, k, v = rnd((3, 48, 2, 8), 23), rnd((3, 48, 2, 8), 24), rnd((3, 48, 2, 8), 25)
    kl = [48, 30, 1]
    o, _ = attention_forward(q, k, v, seqlens_k=kl)
    np.testing.assert_allclose(o, _sdpa_fp64(q, k, v, 8 ** -0.5, False, kl), atol=1e-12)


# ---------------------------------------------------------------- blocked online recurrence

@pytest.mark.parametrize("block", [1, 2, 3, 64, 97])
@pytest.mark.parametrize("mask", [dict(), dict(causal=True), dict(window=(9, 3)),
                                  dict(causal=True, window=(20, 0), seqlens_k=[60, 11])])
def test_blocked_online_equals_one_shot(block, mask):
    q, k, v = rnd((2, 97, 2, 8), 30, 3.0), rnd((2, 97, 2, 8), 31, 3.0), rnd((2, 97, 2, 8), 32)
    o1, l1 = attention_forward(q, k, v, **mask)
    o2, l2 = blocked_online_forward(q, k, v, block_q=block, block_k=block, **mask)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    fin = np.isfinite(l1)
    assert (fin == np.isfinite(l2)).all()
    np.testing.assert_allclose(l2[fin], l1[fin], atol=1e-12)


def test_forward_rows_matches_full():
    q, k, v = rnd((1, 80, 3, 8), 33), rnd((1, 80, 3, 8), 34), rnd((1, 80, 3, 8), 35)
    rows = np.array([[0, 5, 79], [1, 40, 2], [79, 78, 77]])
    for kw in [dict(causal=True), dict(causal=True, window=(7, 0))]:
        o, l = attention_forward(q, k, v, **kw)
        orow, lrow = attention_forward_rows(q, k, v, rows, **kw)
        for h in range(3):
            np.testing.assert_allclose(orow[0, h], o[0, rows[h], h], atol=1e-14)
            np.testing.assert_allclose(lrow[0, h], l[0, h, rows[h]], atol=1e-14)


# ---------------------------------------------------------------- backward

def _loss(q, k, v, do, **kw):
    o, _ = attention_forward(q, k, v, **kw)
    return float((o * do).sum())


def _fd_check(shape, kw, seed, n_samples=None, rtol=1e-6):
    q, k, v = rnd(shape, seed), rnd(shape, seed + 1), rnd(shape, seed + 2)
    do = rnd(shape, seed + 3)
    grads = attention_backward(q, k, v, do, **kw)
    eps = 1e-6
    rng = np.random.default_rng(seed)
    for x, g in zip((q, k, v), grads):
        idx = list(np.ndindex(*shape))
        if n_samples is not None:
            idx = [idx[i] for i in rng.choice(len(idx), n_samples, replace=False)]
        for ix in idx:
            old = x[ix]
            x[ix] = old + eps
            lp = _loss(q, k, v, do, **kw)
            x[ix] = old - eps
            lm = _loss(q, k, v, do, **kw)
            x[ix] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[ix]) <= rtol * max(1.0, abs(fd)) + 1e-8, (ix, fd, g[ix])


@pytest.mark.parametrize("kw", [dict(), dict(causal=True), dict(window=(2, 1)),
                                dict(seqlens_k=[5]), dict(causal=True, window=(3, 0))])
def test_backward_finite_differences_tiny(kw):
    _fd_check((1, 8, 1, 4), kw, 40)


@pytest.mark.parametrize("kw", [dict(), dict(causal=True), dict(seqlens_k=[41])])
def test_backward_finite_differences_n64_d32(kw):
    _fd_check((1, 64, 1, 32), kw, 50, n_samples=60)


def test_backward_matches_torch_autograd_fp64():
    shape = (2, 33, 2, 8)
    q, k, v, do = (rnd(shape, 60 + i) for i in range(4))
    kl = [33, 20]
    for causal in (False, True):
        dq, dk, dv = attention_backward(q, k, v, do, causal=causal, seqlens_k=kl)
        tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v))
        s = tq @ tk.transpose(-1, -2) / math.sqrt(8)
        mask = torch.zeros(2, 1, 33, 33, dtype=torch.bool)
        for b in range(2):
            mask[b, :, :, : kl[b]] = True
        if causal:
            mask &= torch.ones(33, 33, dtype=torch.bool).tril()
        o = torch.softmax(s.masked_fill(~mask, float("-inf")), -1) @ tv
        o.backward(torch.tensor(do.transpose(0, 2, 1, 3)))
        for mine, ref in ((dq, tq), (dk, tk), (dv, tv)):
            np.testing.assert_allclose(mine, ref.grad.numpy().transpose(0, 2, 1, 3), atol=1e-12)


def test_backward_invariants():
    """sum_j dK_j = 0 (adding a vector to every key shifts each row of S by a
    constant); sum_j dV_j = sum_i dO_i over rows with visible keys (rows of P
    sum to 1); padded keys get exactly zero gradient."""
    shape = (2, 50, 3, 8)
    q, k, v, do = (rnd(shape, 70 + i) for i in range(4))
    kl = [50, 23]
    dq, dk, dv = attention_backward(q, k, v, do, causal=True, seqlens_k=kl)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-12)
    assert (dk[1, 23:] == 0).all() and (dv[1, 23:] == 0).all()


def test_empty_rows_have_zero_gradient():
    shape = (1, 12, 1, 4)
    q, k, v, do = (rnd(shape, 80 + i) for i in range(4))
    o, lse = attention_forward(q, k, v, window=(0, 0), seqlens_k=[5])
    assert (o[0, 5:] == 0).all() and np.isneginf(lse[0, 0, 5:]).all()
    dq, dk, dv = attention_backward(q, k, v, do, window=(0, 0), seqlens_k=[5])
    assert (dq[0, 5:] == 0).all() and np.isfinite(dq).all()
    np.testing.assert_allclose(dv[0, :5], do[0, :5], atol=1e-15)


# ---------------------------------------------------------------- ALiBi

def _alibi_closed_form(n, slope, causal):
    """Softmax weights of the scores -slope |i - j| (Q = 0), from geometric
    sums: Z_i = sum_{d=0}^{i} r^d (+ sum_{d=1}^{n-1-i} r^d without a causal
    mask), r = e^{-slope}. Returns (W [n, n], ln Z [n])."""
    r = math.exp(-slope)
    w = np.zeros((n, n))
    lnz = np.zeros(n)
    for i in range(n):
        z = (1 - r ** (i + 1)) / (1 - r)
        if not causal:
            z += r * (1 - r ** (n - 1 - i)) / (1 - r)
        lnz[i] = math.log(z)
        for j in range(n):
            if causal and j > i:
                continue
            w[i, j] = r ** abs(i - j) / z
    return w, lnz


@pytest.mark.parametrize("causal", [False, True])
def test_alibi_zero_query_closed_form(causal):
    # Q = 0 leaves only the bias: O_i = sum_j w_ij V_j with geometric weights;
    # a softmax scale other than 1 must not scale the bias.
    n, d, h = 20, 6, 2
    slopes = np.array([[0.5, 0.125]])  # [B=1, H=2]
    v = rnd((1, n, h, d), 90)
    o, lse = attention_forward(np.zeros((1, n, h, d)), rnd((1, n, h, d), 91), v,
                               softmax_scale=0.37, causal=causal, alibi_slopes=slopes)
    for hh in range(h):
        w, lnz = _alibi_closed_form(n, slopes[0, hh], causal)
        np.testing.assert_allclose(lse[0, hh], lnz, atol=1e-12)
        np.testing.assert_allclose(o[0, :, hh], w @ v[0, :, hh], atol=1e-12)


def test_alibi_zero_slope_is_plain_attention():
    shape = (2, 17, 3, 5)
    q, k, v, do = (rnd(shape, 92 + i) for i in range(4))
    for kw in [dict(), dict(causal=True, window=(4, 0))]:
        o0, l0 = attention_forward(q, k, v, **kw)
        o1, l1 = attention_forward(q, k, v, alibi_slopes=np.zeros(3), **kw)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
        for a, b in zip(attention_backward(q, k, v, do, **kw),
                        attention_backward(q, k, v, do, alibi_slopes=np.zeros((2, 3)), **kw)):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_alibi_matches_torch_sdpa_float_mask(causal):
    # torch's fp64 SDPA adds a float attn_mask to the scaled scores.
    B, N, H, D = 2, 23, 2, 8
    q, k, v = (rnd((B, N, H, D), 96 + i) for i in range(3))
    slopes = np.array([[0.25, 0.0625], [1.0, 0.5]])
    o, _ = attention_forward(q, k, v, causal=causal, alibi_slopes=slopes)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    bias = -slopes[:, :, None, None] * np.abs(i - j)[None, None]
    if causal:
        bias = np.where(j <= i, bias, -np.inf)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.tensor(x.transpose(0, 2, 1, 3)) for x in (q, k, v)), attn_mask=torch.tensor(bias))
    np.testing.assert_allclose(o, ref.numpy().transpose(0, 2, 1, 3), atol=1e-12)


def test_alibi_rows_match_full():
    shape = (1, 40, 2, 4)
    q, k, v = rnd(shape, 99), rnd(shape, 100), rnd(shape, 101)
    rows = np.array([[0, 7, 39], [3, 20, 38]])
    kw = dict(causal=True, window=(9, 0), alibi_slopes=np.array([0.3, 0.05]))
    o, l = attention_forward(q, k, v, **kw)
    orow, lrow = attention_forward_rows(q, k, v, rows, **kw)
    for h in range(2):
        np.testing.assert_allclose(orow[0, h], o[0, rows[h], h], atol=1e-14)
        np.testing.assert_allclose(lrow[0, h], l[0, h, rows[h]], atol=1e-14)


@pytest.mark.parametrize("kw", [dict(alibi_slopes=[0.4]), dict(causal=True, alibi_slopes=[1.5])])
def test_alibi_backward_finite_differences(kw):
    _fd_check((1, 8, 1, 4), kw, 110)
