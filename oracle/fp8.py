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
* The one further rounding the fp8 product forces is that of P: the P V
  product runs on fp8 operands, so P is rounded to e4m3 (to nearest, ties to
  even) as P' = 2^(x - M + 3), M the tile's reference max (below). The LSE is
  computed from the unrounded P. ``fp8_output_bound`` bounds the effect.

e4m3 (OCP): sign bit, 4 exponent bits with bias 7, 3 mantissa bits. Exponent
field 0 holds subnormals m * 2^-9; exponent field e > 0 holds (1 + m/8) 2^(e-7);
the two codes with all exponent and mantissa bits set (0x7f, 0xff) are NaN;
there are no infinities; the largest finite magnitude is 448.

The bound. Let P'_j = 2^(x_j - M + 3) be the kernel's probability of key j at
the reference M of its tile (x_j the score in log2 units). M is only ever set
to the exact running max of the scores seen so far, and every P'_j <= 448 (a
tile whose per-lane sum of P' exceeds 448 is redone against a raised M). Let
P^_j be the e4m3 rounding of P'_j. Round-to-nearest gives
|P^_j - P'_j| <= 2^-4 P'_j where P'_j is in the normal range (>= 2^-6), and at
most min(P'_j, 2^-10) below it (half the subnormal step, or the value itself
when it rounds to 0). Each tile's contribution is later multiplied by
alpha = 2^(M - M_final) <= 1, and O is divided by l = sum_j alpha P'_j. M_final
is the score of some key, whose term is 2^3, so l >= 2^3 sum_j 2^(x_j - x_max)
= 2^3 / w_max. With w_j = alpha P'_j / l the exact softmax weights,

    |O_fp8 - O| <= 2^-4 sum_j w_j |v_j| + sum_j min(w_j, 2^-13 w_max) |v_j|

per output element (v the dequantised V, the sums over visible keys). The kernel's other roundings (fp32
scores from exact products, the fp32 exponential, the bf16 output) are far
smaller or are bounded separately by the tests.

Parity of this module: pinned by tests/test_oracle_fp8.py (the decoder against
the format's closed-form values and torch's float8_e4m3fn, the rounding's ties,
closed forms of the attention, and the bound against a simulation of the
rounding it bounds).
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

    Magnitudes above 448 (which the forward never produces) raise ValueError.
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
    """Per-element bound on |O_fp8 - O_exact| from rounding P to e4m3 (module notes):
    2^-4 sum_j w_ij |v_jd| + sum_j min(w_ij, 2^-13 max_j w_ij) |v_jd|.

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
            av = np.abs(v[b, :, h, :])
            wmax = w.max(axis=1, keepdims=True)
            bound = 2.0 ** -4 * (w @ av) + np.minimum(w, 2.0 ** -13 * wmax) @ av
            if rows is None:
                out[b, :, h, :] = bound
            else:
                out[b, h] = bound
    return out


def attention_forward_fp8_rounded(q8, k8, v8, descale_q, descale_k, descale_v,
                                  softmax_scale=None, causal=False, window=(-1, -1),
                                  seqlens_k=None):
    """O with P rounded to e4m3 at the final reference: P' = 2^3 P / max_j P
    (row max -> 2^3), O = sum_j e4m3(P'_j) v_j / sum_j P'_j. One instance of the
    rounding ``fp8_output_bound`` covers (the tests use it to check the bound)."""
    q, k, v = dequantise(q8, k8, v8, descale_q, descale_k, descale_v)
    B, N, H, D = q.shape
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out = np.zeros((B, N, H, D))
    for b in range(B):
        vis = visible_mask(N, N, causal, window[0], window[1], _key_len(seqlens_k, b, N))
        for h in range(H):
            s = np.where(vis, scale * (q[b, :, h, :] @ k[b, :, h, :].T), -np.inf)
            m = s.max(axis=1)
            fin = np.isfinite(m)
            pp = np.where(fin[:, None], np.exp(s - np.where(fin, m, 0.0)[:, None]) * 2.0 ** 3, 0.0)
            l = pp.sum(axis=1)
            num = e4m3_round(pp) @ v[b, :, h, :]
            out[b, :, h, :] = np.where(fin[:, None], num / np.where(fin, l, 1.0)[:, None], 0.0)
    return out
