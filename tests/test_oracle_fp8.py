"""Pins of the fp8 part of the oracle (oracle/fp8.py), CPU only.

The e4m3 decoder is checked against the format's closed-form values and
against torch's float8_e4m3fn conversion over all 256 codes; the rounding
against torch's conversion and its ties; the attention over decoded inputs
against closed forms; the bound on P's rounding against simulations of that
rounding at several factors the contract allows (the row's largest weight
mapped to 1, 8 or 448, or each key block's largest weight mapped to 448), with
cases that bring the simulated error to the bound. A planted mistake in a copy
of the module fails at least one pin.
"""

import math
import os
import types

import numpy as np
import pytest
import torch

import oracle.fp8 as fp8

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fp8.py")


def codes_of(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ------------------------------------------------------------------ pins


def pin_decode_closed_form(m):
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x3f: 1.875, 0x40: 2.0, 0x7e: 448.0, 0x77: 240.0, 0xb8: -1.0,
             0x80: -0.0, 0xfe: -448.0}
    got = m.e4m3_decode(np.array(list(table), dtype=np.uint8))
    ok = np.array_equal(got, np.array(list(table.values())))
    nan = m.e4m3_decode(np.array([0x7f, 0xff], dtype=np.uint8))
    return ok and np.isnan(nan).all() and np.signbit(m.e4m3_decode(np.array([0x80], np.uint8)))[0]


def pin_decode_torch(m):
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = m.e4m3_decode(codes)
    both_nan = np.isnan(want) & np.isnan(got)
    return bool(((got == want) | both_nan).all())


def pin_round(m):
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-2.0 ** -5, 2.0 ** -5, 4000),
                        np.exp2(rng.uniform(-12, 8.8, 4000)), [0.0, 448.0, -448.0]])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    if not np.array_equal(m.e4m3_round(x), want):
        return False
    # Ties go to the even mantissa: 1 + 1/16 -> 1, 1 + 3/16 -> 1.25, 2^-10 -> 0,
    # 3 * 2^-10 -> 2^-8, 2^8 (1 + 1/16) -> 2^8, and every code maps to itself.
    ties = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 272.0, -1.0625])
    want = np.array([1.0, 1.25, 0.0, 2.0 ** -8, 256.0, -1.0])
    finite = m.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = finite[np.isfinite(finite)]
    return np.array_equal(m.e4m3_round(ties), want) and np.array_equal(m.e4m3_round(finite), finite)


def _case(n=40, h=2, d=16, seed=0, std=1.0, b=1):
    g = torch.Generator().manual_seed(seed)
    out = []
    for _ in range(3):
        x = torch.randn((b, n, h, d), generator=g) * std * 32
        out.append(x.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    return out


def pin_attention_closed_forms(m):
    q8, _, v8 = _case(seed=1)
    k8 = np.zeros_like(q8)                 # all scores 0: uniform weights
    dq, dk, dv = 0.25, 0.5, 0.125
    o, lse = m.attention_forward_fp8(q8, k8, v8, dq, dk, dv, causal=True)
    v = m.e4m3_decode(v8) * dv
    n = q8.shape[1]
    ok = True
    for i in range(n):
        ok &= np.allclose(o[0, i], v[0, : i + 1].mean(axis=0), atol=1e-14, rtol=0)
        ok &= abs(lse[0, 0, i] - math.log(i + 1)) < 1e-12
    # Row 0 of a causal mask sees key 0 only: O = v_0 for any Q, K.
    q8, k8, v8 = _case(seed=2)
    o, _ = m.attention_forward_fp8(q8, k8, v8, 1.0, 1.0, 0.5, causal=True)
    ok &= np.array_equal(o[0, 0], m.e4m3_decode(v8[0, 0]) * 0.5)
    return bool(ok)


def pin_bound_covers_rounding(m):
    """The bound covers the rounding at every scale the contract allows that
    is tried here: the row's largest weight mapped to 1 (the smallest factor
    (ii) allows), to 8 and to 448 (the largest (i) allows), and one factor per
    block of 16 keys mapping each block's largest weight to 448."""
    ok = True
    worst = 0.0
    scales = [dict(top=1.0), dict(top=8.0), dict(top=448.0), dict(key_block=16)]
    for seed, mask, std in [(3, dict(), 1.0), (4, dict(causal=True), 2.0),
                            (5, dict(window=(5, 3)), 1.0), (6, dict(seqlens_k=[17]), 4.0)]:
        q8, k8, v8 = _case(seed=seed, std=std)
        args = (q8, k8, v8, 1 / 32, 1 / 32, 1 / 32)
        o, _ = m.attention_forward_fp8(*args, **mask)
        bnd = m.fp8_output_bound(*args, **mask)
        for sc in scales:
            r = m.attention_forward_fp8_rounded(*args, **mask, **sc)
            err = np.abs(r - o)
            ok &= bool((err <= bnd + 1e-15).all())
            worst = max(worst, float((err / (bnd + 1e-300)).max()))
    return ok and worst > 0.05


def _two_key_error(m, ratio, top=1.0):
    """Query row 1 of a two-key case sees scores 0 and ln(ratio), V rows 0 and
    (1, 1, ...): returns (|O_rounded - O_exact|, bound) of its first element,
    with the larger weight mapped to ``top``. The scores are realised with
    decoded Q = (1, 0, ...), K rows 0 and (ln ratio, 0, ...) (one e4m3 code
    -1 with descale_k = -ln ratio)."""
    s2 = math.log(ratio)
    q8 = np.zeros((1, 2, 1, 16), np.uint8)
    k8 = np.zeros((1, 2, 1, 16), np.uint8)
    v8 = np.zeros((1, 2, 1, 16), np.uint8)
    q8[0, :, 0, 0] = codes_of([1.0])[0]
    k8[0, 1, 0, 0] = codes_of([-1.0])[0]
    v8[0, 1, 0, :] = codes_of([1.0])[0]
    args = (q8, k8, v8, 1.0, -s2, 1.0)
    o, _ = m.attention_forward_fp8(*args, softmax_scale=1.0)
    r = m.attention_forward_fp8_rounded(*args, softmax_scale=1.0, top=top)
    bnd = m.fp8_output_bound(*args, softmax_scale=1.0)
    return abs(r[0, 1, 0, 0] - o[0, 1, 0, 0]), bnd[0, 1, 0, 0]


def pin_bound_near_tight(m):
    """Cases where one rounding reaches, or nearly reaches, the bound, with the
    larger weight w_1 mapped to 1 (c = 1 / w_1, the smallest factor the
    contract allows), so the smaller one is rounded at y = ratio:
    y = 2^-2 (1 + 1/16) is a tie that rounds to 2^-2, an error of 2^-4 of the
    value below it (the relative term, 94% of the bound);
    y = 3 * 2^-10, in the subnormal range, is a tie that rounds to 2^-8, an
    error of 2^-10 w_1 (the absolute term, all of the bound; the relative
    term alone gives 3/16 of it);
    y = 2^-17 rounds to 0, an error of the whole weight w_2, far below
    2^-10 w_1 (the min in the absolute term, all of the bound).
    A larger factor makes the same subnormal rounding smaller against the
    weight: with w_1 mapped to 8, a ratio of 3 * 2^-13 is rounded at
    y = 3 * 2^-10 and errs by 2^-10 / c = 2^-13 w_1, a third of the bound
    (which is w_2 = 3 * 2^-13 w_1 there)."""
    err, bnd = _two_key_error(m, 1.0625 / 4)
    ok = 0.9 * bnd <= err <= bnd
    err, bnd = _two_key_error(m, 3 * 2.0 ** -10)
    ok = ok and 0.99 * bnd <= err <= bnd
    err, bnd = _two_key_error(m, 2.0 ** -17)
    ok = ok and 0.99 * bnd <= err <= bnd
    err, bnd = _two_key_error(m, 3 * 2.0 ** -13, top=8.0)
    return bool(ok and abs(err / bnd - 1 / 3) < 1e-9)


def pin_rounded_rejects_scales_outside_contract(m):
    for top in (0.5, 449.0):
        try:
            q8, k8, v8 = _case(n=4, seed=8)
            m.attention_forward_fp8_rounded(q8, k8, v8, 1 / 32, 1 / 32, 1 / 32, top=top)
        except ValueError:
            continue
        return False
    return True


PINS = [pin_decode_closed_form, pin_decode_torch, pin_round, pin_attention_closed_forms,
        pin_bound_covers_rounding, pin_bound_near_tight, pin_rounded_rejects_scales_outside_contract]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    assert pin(fp8)


def test_round_rejects_out_of_range():
    with pytest.raises(ValueError):
        fp8.e4m3_round(np.array([449.0]))


def test_rows_variant_matches_full():
    q8, k8, v8 = _case(n=50, seed=7)
    args = (q8, k8, v8, 1 / 32, 1 / 32, 1 / 32)
    rows = np.array([[0, 7, 49], [3, 3, 20]])
    o, lse = fp8.attention_forward_fp8(*args, causal=True)
    ro, rl = fp8.attention_forward_fp8_rows(*args, rows=rows, causal=True)
    bnd = fp8.fp8_output_bound(*args, causal=True)
    rb = fp8.fp8_output_bound(*args, causal=True, rows=rows)
    for h in range(2):
        assert np.allclose(ro[0, h], o[0, rows[h], h], atol=1e-14, rtol=0)
        assert np.allclose(rl[0, h], lse[0, h, rows[h]], atol=1e-14, rtol=0)
        assert np.allclose(rb[0, h], bnd[0, rows[h], h], atol=1e-16, rtol=0)


# --------------------------------------------------------------- mutants

MUTANTS = {
    "exponent_bias_8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "subnormal_step": ("m * 2.0 ** -9, (1.0", "m * 2.0 ** -10, (1.0"),
    "no_nan": ("(e == 15) & ((c & 7) == 7)", "(e == 16)"),
    "no_sign": ("sign = np.where(c >> 7, -1.0, 1.0)", "sign = 1.0"),
    "ties_away": ("np.round(a / step)", "np.floor(a / step + 0.5)"),
    "normal_step": ("np.exp2(ex - 3.0)", "np.exp2(ex - 2.0)"),
    "subnormal_threshold": ("np.where(a < 2.0 ** -6, 2.0 ** -9", "np.where(a < 2.0 ** -7, 2.0 ** -9"),
    "no_descale_v": ("e4m3_decode(v8) * float(descale_v)", "e4m3_decode(v8)"),
    "bound_half": ("np.maximum(2.0 ** -4 * w,", "np.maximum(2.0 ** -5 * w,"),
    "bound_no_subnormal_term": ("np.maximum(2.0 ** -4 * w, np.minimum(w, 2.0 ** -10 * wmax))",
                                "2.0 ** -4 * w"),
    "bound_subnormal_without_min": ("np.minimum(w, 2.0 ** -10 * wmax))",
                                    "2.0 ** -10 * wmax * (w > 0))"),
    "bound_subnormal_tighter": ("np.minimum(w, 2.0 ** -10 * wmax))", "np.minimum(w, 2.0 ** -13 * wmax))"),
    "rounded_unscaled": ("(e4m3_round(y) / c) @", "(e4m3_round(y)) @"),
    "rounded_no_rounding": ("(e4m3_round(y) / c) @", "(y / c) @"),
    "rounded_top_ignored": ("target = top\n", "target = 8.0\n"),
    "rounded_no_range_check": ("if not 1.0 <= top <= E4M3_MAX:", "if False:"),
}


def _load(mutation):
    src = open(SRC).read()
    old, new = mutation
    assert src.count(old) == 1, old
    src = src.replace(old, new).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("oracle_fp8_mutant")
    exec(compile(src, "oracle_fp8_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    m = _load(MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            ok = pin(m)
        except Exception:  # a crash counts as a failed pin
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passes every pin"


def test_unmutated_copy_passes():
    m = _load(("E4M3_MAX = 448.0", "E4M3_MAX = 448.0"))
    for pin in PINS:
        assert pin(m), pin.__name__
