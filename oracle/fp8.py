"""FP8 (OCP e4m3) forward: decoding, exact attention over the decoded inputs,
and the bound on the error that rounding P to e4m3 adds (test infrastructure).

What the pages fix: FlashAttention-3 offers an FP8 forward ([interview]
"v1 → v2 → v3 演进", the v3 row; [wiki] "典型例子", the paragraph on the
official repository). They say nothing of its arithmetic, so this module takes
the plainest reading:

* Inputs are bytes in the OCP 8-bit e4m3 format, one fp32 dequantisation
  factor per tensor: byte x of Q stands for e4m3(x) * descale_q (likewise K, V).
* The result approximates exact attention ([wiki] "边界与常见误解": the method
  is exact) over the dequantised values. ``attention_forward_fp8`` is that
  exact attention: the definitions of ``attention.py`` applied to the decoded
  inputs, in fp64.
* The one further rounding an fp8 P V product forces is that of the
  probabilities, which must enter it as e4m3 values. The contract: the
  softmax weight w_j of key j (the exact probability, sum_j w_j = 1) enters as
  e4m3(c w_j) / c, rounded to nearest (ties to even), for some factor c > 0
  that may differ between groups of keys of a row, under two conditions:
    (i)  c w_j <= 448 for every weight rounded with it (nothing saturates);
    (ii) c w_max >= 1, w_max the row's largest weight.
  The LSE is computed from the unrounded weights. ``fp8_output_bound`` bounds
  what this rounding can do to O; it depends on the format and on (i), (ii)
  only, not on how an implementation picks c.

e4m3 (OCP): sign bit, 4 exponent bits with bias 7, 3 mantissa bits. Exponent
field 0 holds subnormals m * 2^-9; exponent field e > 0 holds (1 + m/8) 2^(e-7);
the two codes with all exponent and mantissa bits set (0x7f, 0xff) are NaN;
there are no infinities; the largest finite magnitude is 448.

The bound. Let y = c w be a value rounded to e4m3, 0 <= y <= 448 by (i).
Normal range (y >= 2^-6): y lies in [2^e, 2^(e+1)) with e >= -6, where the
spacing is 2^(e-3), so rounding to nearest errs by at most 2^(e-4) <= 2^-4 y.
Subnormal range (y < 2^-6): the spacing is 2^-9, so the error is at most half
of it, 2^-10; and a value at or below 2^-10 rounds to 0, erring by y itself.
In both ranges, |e4m3(y) - y| <= max(2^-4 y, min(y, 2^-10)) (in the normal
range the second term is 2^-10 <= 2^-4 y; in the subnormal range the first is
below the second). Dividing by c, and using 1/c <= w_max from (ii), the weight
of key j moves by at most max(2^-4 w_j, min(w_j, 2^-10 w_max)). O is the sum
of the weights times V, so per output element

    |O_fp8 - O| <= sum_j max(2^-4 w_j, min(w_j, 2^-10 w_max)) |v_j|

(v the dequantised V, the sums over visible keys). An implementation's other
roundings (fp32 scores from exact products, the fp32 exponential, the bf16
output) are bounded separately by the tests that use this.

Parity of this module: pinned by tests/test_oracle_fp8.py (the decoder against
the format's closed-form values and torch's float8_e4m3fn, the rounding's ties,
closed forms of the attention, and the bound against simulations of the
rounding it bounds at several scales the contract allows, some of them
reaching it).
"""

from __future__ import annotations

import numpy as np

from .attention import _key_len, _softmax_rows, visible_mask, attention_forward, \
    attention_forward_rows

E4M3_MAX = 448.0


def _e4m3_values(c):
    """float64 value of each code in the int64 array c, by the format's definition."""
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


_E4M3_TABLE = _e4m3_values(np.arange(256, dtype=np.int64))


def e4m3_decode(codes):
    """float64 values of e4m3 codes (uint8 array-like): the definition above,
    evaluated once per code and looked up (large inputs decode quickly)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_round(x):
    """Nearest e4m3 value of each x (ties to even), as float64.

    Magnitudes above 448 (excluded by condition (i)) raise ValueError.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if (a > E4M3_MAX).any():
        raise ValueError("value outside the e4m3 range")
    # Spacing of representable values: 2^-9 below 2^-6, else 2^(floor(log2 a) - 3).
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(ex - 3.0))
    r = np.round(a / step) * step          # numpy rounds halves to even
    return np.copysign(r, x)


def dequantise(q8, k8, v8, descale_q, descale_k, descale_v):
    """Decoded Q, K, V (float64) times their factors."""
    return (e4m3_decode(q8) * float(descale_q), e4m3_decode(k8) * float(descale_k),
            e4m3_decode(v8) * float(descale_v))


def attention_forward_fp8(q8, k8, v8, descale_q, descale_k, descale_v, softmax_scale=None,
                          causal=False, window=(-1, -1), seqlens_k=None):
    """Exact O [B,N,H,D] and LSE [B,H,N] over the dequantised inputs."""
    q, k, v = dequantise(q8, k8, v8, descale_q, descale_k, descale_v)
    return attention_forward(q, k, v, softmax_scale, causal, window, seqlens_k)


def attention_forward_fp8_rows(q8, k8, v8, descale_q, descale_k, descale_v, rows,
                               softmax_scale=None, causal=False, window=(-1, -1),
                               seqlens_k=None):
    """The same for the query rows ``rows`` ([H, R] or [R]); O [B,H,R,D], LSE [B,H,R]."""
    q, k, v = dequantise(q8, k8, v8, descale_q, descale_k, descale_v)
    return attention_forward_rows(q, k, v, rows, softmax_scale, causal, window, seqlens_k)


def _weights(qh, kh, scale, vis):
    s = np.where(vis, scale * (qh @ kh.T), -np.inf)
    p, _ = _softmax_rows(s)
    return p


def fp8_output_bound(q8, k8, v8, descale_q, descale_k, descale_v, softmax_scale=None,
                     causal=False, window=(-1, -1), seqlens_k=None, rows=None):
    """Per-element bound on |O_fp8 - O_exact| from rounding the weights to
    e4m3 under the contract of the module notes:
    sum_j max(2^-4 w_ij, min(w_ij, 2^-10 max_k w_ik)) |v_jd|.

    Returns [B,N,H,D], or [B,H,R,D] for the query rows ``rows`` ([H, R] or [R]).
    """
    q, k, v = dequantise(q8, k8, v8, descale_q, descale_k, descale_v)
    B, N, H, D = q.shape
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        if rows.ndim == 1:
            rows = np.broadcast_to(rows, (H, rows.shape[0]))
        out = np.zeros((B, H, rows.shape[1], D))
    else:
        out = np.zeros((B, N, H, D))
    for b in range(B):
        kl = _key_len(seqlens_k, b, N)
        for h in range(H):
            r = np.arange(N) if rows is None else rows[h]
            vis = visible_mask(len(r), N, causal, window[0], window[1], kl, q_pos=r)
            w = _weights(q[b, r, h, :], k[b, :, h, :], scale, vis)
            wmax = w.max(axis=1, keepdims=True)
            per_key = np.maximum(2.0 ** -4 * w, np.minimum(w, 2.0 ** -10 * wmax))
            bound = per_key @ np.abs(v[b, :, h, :])
            if rows is None:
                out[b, :, h, :] = bound
            else:
                out[b, h] = bound
    return out


def attention_forward_fp8_rounded(q8, k8, v8, descale_q, descale_k, descale_v,
                                  softmax_scale=None, causal=False, window=(-1, -1),
                                  seqlens_k=None, top=1.0, key_block=None):
    """O with the weights rounded to e4m3 as the contract allows: weight w_j
    enters as e4m3(c w_j) / c. One instance of the rounding
    ``fp8_output_bound`` covers, for checking that bound.

    Choice of c: with ``key_block`` None, one factor per row that maps the
    row's largest weight to ``top`` (1 <= top <= 448, the range conditions (i)
    and (ii) allow). With ``key_block`` = n, one factor per row and block of
    n consecutive keys, mapping the block's largest weight to 448: the largest
    factor (i) allows for that block, and c w_max >= 448 w_max / (block max)
    >= 448 satisfies (ii).
    """
    if not 1.0 <= top <= E4M3_MAX:
        raise ValueError("top must lie in [1, 448]")
    q, k, v = dequantise(q8, k8, v8, descale_q, descale_k, descale_v)
    B, N, H, D = q.shape
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out = np.zeros((B, N, H, D))
    for b in range(B):
        vis = visible_mask(N, N, causal, window[0], window[1], _key_len(seqlens_k, b, N))
        for h in range(H):
            w = _weights(q[b, :, h, :], k[b, :, h, :], scale, vis)
            if key_block is None:
                ref = np.broadcast_to(w.max(axis=1, keepdims=True), w.shape)
                target = top
            else:
                starts = np.arange(0, N, key_block)
                ref = np.repeat(np.maximum.reduceat(w, starts, axis=1),
                                np.diff(np.append(starts, N)), axis=1)
                target = E4M3_MAX
            c = np.where(ref > 0, target / np.where(ref > 0, ref, 1.0), 1.0)
            # c w can exceed the target by one fp64 rounding; the clip removes
            # only that excess.
            y = np.minimum(c * w, target)
            out[b, :, h, :] = (e4m3_round(y) / c) @ v[b, :, h, :]
    return out
