"""The oracle's pins are sensitive: each plausible mistake planted in a copy of
the oracle (dropped term, wrong sign or index, transposed operand, wrong mask
bound) makes at least one pin fail. Runs on the CPU only; the planted copies
live in memory and are never used elsewhere."""

import math
import os
import types

import numpy as np
import pytest

from oracle import blocked_online_forward

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "attention.py")

MUTANTS = {
    "no_scale": ("s = scale * (qh @ kh.T)", "s = (qh @ kh.T)"),
    "causal_strict": ("vis &= j <= i\n", "vis &= j < i\n"),
    "window_left_sign": ("vis &= j >= i - window_left", "vis &= j >= i + window_left"),
    "window_right_exclusive": ("vis &= j <= i + window_right", "vis &= j < i + window_right"),
    "padding_inclusive": ("vis &= j < int(key_len)", "vis &= j <= int(key_len)"),
    "lse_without_max": ("lse = np.where(finite, shift + np.log(l), -np.inf)",
                        "lse = np.where(finite, np.log(l), -np.inf)"),
    "no_normalise": ("e / np.where(finite, l, 1.0)[:, None]", "e"),
    "bwd_drop_rowsum": ("ds = p * (dp - drow[:, None])", "ds = p * dp"),
    "bwd_rowsum_wrong_axis": ("drow = (p * dp).sum(axis=1)", "drow = (p * dp).sum(axis=0)"),
    "bwd_dq_unscaled": ("dq[b, :, h] = scale * (ds @ kh)", "dq[b, :, h] = (ds @ kh)"),
    "bwd_dk_transposed": ("dk[b, :, h] = scale * (ds.T @ qh)", "dk[b, :, h] = scale * (ds @ qh)"),
    "bwd_dv_untransposed": ("dv[b, :, h] = p.T @ doh", "dv[b, :, h] = p @ doh"),
    "bwd_dp_transposed": ("dp = doh @ vh.T", "dp = (doh @ vh.T).T"),
    "alibi_sign": ("s = s - slope * np.abs(i - j)", "s = s + slope * np.abs(i - j)"),
    "alibi_scaled": ("s = s - slope * np.abs(i - j)", "s = s - scale * slope * np.abs(i - j)"),
    "alibi_no_abs": ("s = s - slope * np.abs(i - j)", "s = s - slope * (i - j)"),
}


def _load(mutation):
    src = open(SRC).read()
    old, new = mutation
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def rnd(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _pins(m):
    """Yield (name, passed) for a battery of pins evaluated on module m."""
    n, d = 12, 4
    # Q = 0 closed form under several masks.
    k, v = rnd((1, n, 1, d), 1), rnd((1, n, 1, d), 2)
    for causal, wl, wr, kl in [(True, -1, -1, n), (False, 2, 3, n), (False, -1, -1, 7),
                               (True, 3, 0, 9)]:
        o, lse = m.attention_forward(np.zeros((1, n, 1, d)), k, v, causal=causal,
                                     window=(wl, wr), seqlens_k=[kl])
        ok = True
        for i in range(n):
            vis = [j for j in range(n) if (not causal or j <= i) and (wl < 0 or j >= i - wl)
                   and (wr < 0 or j <= i + wr) and j < kl]
            if not vis:
                continue
            ok &= np.allclose(o[0, i, 0], v[0, vis, 0].mean(axis=0), atol=1e-12)
            ok &= abs(lse[0, 0, i] - math.log(len(vis))) < 1e-12
        yield "zero_q", ok
    # ALiBi with Q = 0: weights r^|i-j| / Z_i, r = e^-slope (geometric sums).
    for causal, slope in [(True, 0.5), (False, 0.25)]:
        o, lse = m.attention_forward(np.zeros((1, n, 1, d)), k, v, softmax_scale=0.6,
                                     causal=causal, alibi_slopes=[slope])
        r = math.exp(-slope)
        ok = True
        for i in range(n):
            js = range(i + 1) if causal else range(n)
            wts = np.array([r ** abs(i - j) for j in js])
            ok &= abs(lse[0, 0, i] - math.log(wts.sum())) < 1e-12
            ok &= np.allclose(o[0, i, 0], (wts[:, None] * v[0, list(js), 0]).sum(0) / wts.sum(),
                              atol=1e-12)
        yield "alibi_zero_q", ok
    # Causal first row: LSE_0 = c q0.k0.
    q = rnd((1, n, 1, d), 3)
    o, lse = m.attention_forward(q, k, v, softmax_scale=0.7, causal=True)
    yield "causal_row0", np.isclose(lse[0, 0, 0], 0.7 * (q[0, 0, 0] @ k[0, 0, 0]), atol=1e-12)
    # Blocked online recurrence (independent derivation) agreement.
    for kw in [dict(), dict(window=(2, 3)), dict(softmax_scale=0.3)]:
        o1, l1 = m.attention_forward(q, k, v, **kw)
        o2, l2 = blocked_online_forward(q, k, v, block_q=5, block_k=5, **kw)
        yield "blocked", np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)
    # Finite differences on a tiny shape.
    do = rnd((1, n, 1, d), 4)
    for kw in [dict(), dict(causal=True)]:
        grads = m.attention_backward(q, k, v, do, **kw)
        ok = True
        for x, g in zip((q, k, v), grads):
            for ix in [(0, 0, 0, 0), (0, 5, 0, 2), (0, n - 1, 0, 3)]:
                old = x[ix]
                x[ix] = old + 1e-6
                lp = float((m.attention_forward(q, k, v, **kw)[0] * do).sum())
                x[ix] = old - 1e-6
                lm = float((m.attention_forward(q, k, v, **kw)[0] * do).sum())
                x[ix] = old
                ok &= abs((lp - lm) / 2e-6 - g[ix]) < 1e-6
        yield "finite_diff", ok


def test_unmutated_oracle_passes_battery():
    m = _load(("import numpy as np", "import numpy as np"))
    failed = [name for name, ok in _pins(m) if not ok]
    assert not failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    m = _load(MUTANTS[name])
    failed = [pin for pin, ok in _pins(m) if not ok]
    assert failed, f"mutant {name} passed every pin"
