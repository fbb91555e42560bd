"""Exact attention by its definition, in fp64 on the CPU (test infrastructure).

The method is exact: it reaches the same result as standard attention and only
changes the order of work and the memory traffic ([wiki] "工作机制" and
"边界与常见误解"; [interview] "Online Softmax"; [notes] FAQ "FlashAttention 是
近似算法嗎？"). So this oracle is the definition written out, with the full
score matrix S and probability matrix P materialised per (batch, head):

    S = c * Q K^T                    ([scratch] §1.1; [interview] 标准注意力)
    S_ij = -inf where (i, j) is not visible       (masks, see visible_mask)
    LSE_i = m_i + ln sum_j exp(S_ij - m_i),  m_i = max_j S_ij   ([scratch] §3.1, §5.2)
    P = exp(S - LSE),   O = P V

Backward ([interview] 反向传播; [scratch] §3.3, softmax Jacobian
dp_j/ds_i = p_i (delta_ij - p_j) applied over the whole row):

    dP = dO V^T
    D_i = sum_j P_ij dP_ij                (the full-row sum)
    dS = P * (dP - D)
    dQ = c dS K,   dK = c dS^T Q,   dV = P^T dO

Readings where the pages are silent or wrong:
* Rows with no visible key (possible only with windows/padding) give O = 0,
  LSE = -inf and no gradient.
* Causal keeps j <= i (the extracted comparison operator is lost; the comment
  beside it says a query sees only keys at or before it).
* Key padding: keys j >= L_b of sequence b are invisible to every query row of
  that sequence; query rows are all still computed.
* ALiBi ([notes] docstring, the ``alibi_slopes`` argument: one fp32 slope
  per head, or per batch and head, lowering the score of query i and key j
  by slope times their distance): the bias joins the scaled score,
  S = c q.k - slope |i - j|, before masking and softmax. It does not depend on Q or K, so the backward's
  formulas are unchanged (dS is the gradient of the biased score, and the
  biased score's derivative in q.k is still c).

Tensors use the (batch, seqlen, nheads, headdim) layout of [notes]. Every
array argument is converted to float64 first. Parity: pinned by the tests in
tests/test_oracle.py (worked example, closed forms, brute-force masks, blocked
online recurrence, finite differences, library special case).
"""

from __future__ import annotations

import numpy as np


def visible_mask(n_q, n_k, causal=False, window_left=-1, window_right=-1,
                 key_len=None, q_pos=None):
    """Boolean [n_q, n_k]: may query i attend to key j?

    [notes] docstring: a window (left, right) restricts query i to keys in
    [i - left, i + right] inclusive; -1 leaves that side unbounded.
    [scratch] §5.3: causal keeps keys j <= i. Both may be given; they
    intersect. ``key_len`` (padding) hides keys j >= key_len. ``q_pos``
    gives the query positions of the rows (default 0..n_q-1).
    """
    i = (np.arange(n_q) if q_pos is None else np.asarray(q_pos))[:, None]
    j = np.arange(n_k)[None, :]
    vis = np.ones((n_q, n_k), dtype=bool)
    if causal:
        vis &= j <= i
    if window_left >= 0:
        vis &= j >= i - window_left
    if window_right >= 0:
        vis &= j <= i + window_right
    if key_len is not None:
        vis &= j < int(key_len)
    return vis


def _key_len(seqlens_k, b, n):
    if seqlens_k is None:
        return n
    return int(min(max(int(seqlens_k[b]), 0), n))


def _softmax_rows(s):
    """Row softmax of an fp64 score block that may hold -inf entries.

    Returns (P, LSE). A row that is entirely -inf gives P = 0, LSE = -inf.
    """
    m = s.max(axis=1)
    finite = np.isfinite(m)
    shift = np.where(finite, m, 0.0)
    e = np.exp(s - shift[:, None])          # exp(-inf) = 0 for masked entries
    l = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(finite, shift + np.log(l), -np.inf)
    p = np.where(finite[:, None], e / np.where(finite, l, 1.0)[:, None], 0.0)
    return p, lse


def _slopes(alibi_slopes, B, H):
    """ALiBi slopes as a float64 [B, H] array (zeros when there is no bias)."""
    if alibi_slopes is None:
        return np.zeros((B, H))
    a = np.asarray(alibi_slopes, dtype=np.float64)
    if a.shape == (H,):
        return np.broadcast_to(a, (B, H))
    if a.shape == (B, H):
        return a
    raise ValueError(f"alibi_slopes must have shape ({H},) or ({B}, {H}), got {a.shape}")


def _scores(qh, kh, scale, vis, slope=0.0, q_pos=None):
    """Masked scores c q.k - slope |i - j| of query rows q_pos (default 0..) and keys 0..."""
    s = scale * (qh @ kh.T)
    if slope != 0.0:
        i = (np.arange(qh.shape[0]) if q_pos is None else np.asarray(q_pos))[:, None]
        j = np.arange(kh.shape[0])[None, :]
        s = s - slope * np.abs(i - j)
    return np.where(vis, s, -np.inf)


def attention_forward(q, k, v, softmax_scale=None, causal=False,
                      window=(-1, -1), seqlens_k=None, alibi_slopes=None):
    """O [B,N,H,D] and LSE [B,H,N] (natural log) of exact attention.

    ``softmax_scale`` defaults to 1/sqrt(headdim) ([notes] docstring).
    ``alibi_slopes``: None, [H] or [B, H] (see the module notes).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, H, D = q.shape
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    slopes = _slopes(alibi_slopes, B, H)
    out = np.zeros((B, N, H, D))
    lse = np.zeros((B, H, N))
    for b in range(B):
        vis = visible_mask(N, N, causal, window[0], window[1],
                           _key_len(seqlens_k, b, N))
        for h in range(H):
            s = _scores(q[b, :, h, :], k[b, :, h, :], scale, vis, slopes[b, h])
            p, lse[b, h] = _softmax_rows(s)
            out[b, :, h, :] = p @ v[b, :, h, :]
    return out, lse


def attention_forward_rows(q, k, v, rows, softmax_scale=None, causal=False,
                           window=(-1, -1), seqlens_k=None, alibi_slopes=None):
    """The same definition evaluated only for query rows ``rows[h]``.

    ``rows`` is an int array [H, R] (or [R], shared by all heads) of query
    positions. Returns O [B,H,R,D] and LSE [B,H,R] for those rows. Used where
    the full N x N matrix is too large for the CPU (long sequences).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, N, H, D = q.shape
    rows = np.asarray(rows, dtype=np.int64)
    if rows.ndim == 1:
        rows = np.broadcast_to(rows, (H, rows.shape[0]))
    R = rows.shape[1]
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    slopes = _slopes(alibi_slopes, B, H)
    out = np.zeros((B, H, R, D))
    lse = np.zeros((B, H, R))
    for b in range(B):
        kl = _key_len(seqlens_k, b, N)
        for h in range(H):
            r = rows[h]
            vis = visible_mask(R, N, causal, window[0], window[1], kl, q_pos=r)
            qh = np.asarray(q[b, r, h, :], dtype=np.float64)
            kh = np.asarray(k[b, :, h, :], dtype=np.float64)
            vh = np.asarray(v[b, :, h, :], dtype=np.float64)
            s = _scores(qh, kh, scale, vis, slopes[b, h], q_pos=r)
            p, lse[b, h] = _softmax_rows(s)
            out[b, h] = p @ vh
    return out, lse


def attention_backward(q, k, v, dout, softmax_scale=None, causal=False,
                       window=(-1, -1), seqlens_k=None, alibi_slopes=None):
    """dQ, dK, dV [B,N,H,D] of exact attention for upstream gradient dO.

    P is rebuilt from the definition (the method rebuilds it from the saved
    LSE; in exact arithmetic the two agree). D_i is the full-row sum
    sum_j P_ij dP_ij, which equals sum_d dO_id O_id.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    B, N, H, D = q.shape
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    slopes = _slopes(alibi_slopes, B, H)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        vis = visible_mask(N, N, causal, window[0], window[1],
                           _key_len(seqlens_k, b, N))
        for h in range(H):
            qh, kh, vh, doh = q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h]
            p, _ = _softmax_rows(_scores(qh, kh, scale, vis, slopes[b, h]))
            dp = doh @ vh.T
            drow = (p * dp).sum(axis=1)
            ds = p * (dp - drow[:, None])
            dq[b, :, h] = scale * (ds @ kh)
            dk[b, :, h] = scale * (ds.T @ qh)
            dv[b, :, h] = p.T @ doh
    return dq, dk, dv


def visible_pair_count(n, causal=False, window=(-1, -1), seqlens_k=None,
                       batch=1):
    """Number of visible (query, key) pairs summed over the batch (per head).

    Used to report FLOPs over visible pairs for windowed/padded work.
    Computed row by row in closed form (no N x N matrix).
    """
    total = 0
    i = np.arange(n, dtype=np.int64)
    for b in range(batch):
        kl = _key_len(seqlens_k, b, n)
        lo = np.zeros(n, dtype=np.int64)
        hi = np.full(n, kl - 1, dtype=np.int64)
        if causal:
            hi = np.minimum(hi, i)
        if window[0] >= 0:
            lo = np.maximum(lo, i - window[0])
        if window[1] >= 0:
            hi = np.minimum(hi, i + window[1])
        total += int(np.clip(hi - lo + 1, 0, None).sum())
    return total
