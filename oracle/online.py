"""The online-softmax recurrence in fp64 (test infrastructure, used to pin the
definition-based oracle in attention.py; never used as the oracle itself).

The recurrence is the prose version on the pages ([interview] "Online Softmax
（增量式 softmax）"; [scratch] §2.2 "Online Softmax"): keep, per row, the
running maximum m and the running sum l of exponentials taken relative to m.
For each new block x_b:

    m_new = max(m, max(x_b))
    l     = l * exp(m - m_new) + sum(exp(x_b - m_new))      (rescale old, add new)
    acc   = acc * exp(m - m_new) + exp(x_b - m_new) @ V_b    (same rescale for O)

with m = -inf, l = 0, acc = 0 before the first block, so that the first block
needs no special case ([scratch] §3.1, on the -inf initial value). At the end
O = acc / l and LSE = m + ln l.

Reading: [scratch] §3.1's printed blocked code reuses the LSE slot as the
running maximum and stores log(l) without adding m back; applied literally it
does not reproduce standard attention. The prose recurrence above (m and l kept
apart, LSE = m + ln l) is the one that agrees with the definition, and is the
one implemented here.
"""

from __future__ import annotations

import numpy as np


def online_softmax_trace(x, block):
    """Softmax of one row x by the blocked recurrence, with its intermediates.

    Returns (p, trace) where trace is a list of per-block dicts holding the
    block max, the block's exponentials relative to its own max, the block's
    local sum and local softmax, the running max after the block, the old sum
    rescaled to the new max, the block's sum relative to the new max, and the
    running sum -- the quantities the worked example in [scratch] §2.2 prints.
    """
    x = np.asarray(x, dtype=np.float64)
    m = -np.inf
    l = 0.0
    trace = []
    for s in range(0, x.shape[0], block):
        xb = x[s:s + block]
        bmax = xb.max()
        e_local = np.exp(xb - bmax)
        m_new = max(m, bmax)
        l_old_rescaled = l * np.exp(m - m_new) if np.isfinite(m) else 0.0
        l_block = np.exp(xb - m_new).sum()
        l = l_old_rescaled + l_block
        trace.append(dict(block_max=bmax, e_local=e_local,
                          l_local=e_local.sum(),
                          local_softmax=e_local / e_local.sum(),
                          m=m_new, l_old_rescaled=l_old_rescaled,
                          l_block=l_block, l=l))
        m = m_new
    p = np.exp(x - m) / l
    return p, trace


def blocked_online_forward(q, k, v, softmax_scale=None, causal=False,
                           window=(-1, -1), seqlens_k=None, block_q=64,
                           block_k=64):
    """Tiled forward in fp64: query blocks outside, key blocks inside
    ([scratch] §3.1 loop structure), with the prose recurrence per row.

    Returns O [B,N,H,D] and LSE [B,H,N]. Masked scores are -inf; a row whose
    keys are all masked so far keeps m = -inf and contributes nothing.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, H, D = q.shape
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    wl, wr = window
    out = np.zeros((B, N, H, D))
    lse = np.zeros((B, H, N))
    for b in range(B):
        kl = N if seqlens_k is None else min(max(int(seqlens_k[b]), 0), N)
        for h in range(H):
            for q0 in range(0, N, block_q):
                qi = np.arange(q0, min(q0 + block_q, N))
                qb = q[b, qi, h, :]
                m = np.full(qi.shape[0], -np.inf)
                l = np.zeros(qi.shape[0])
                acc = np.zeros((qi.shape[0], D))
                for k0 in range(0, N, block_k):
                    kj = np.arange(k0, min(k0 + block_k, N))
                    s = scale * (qb @ k[b, kj, h, :].T)
                    ok = np.ones(s.shape, dtype=bool)
                    if causal:
                        ok &= kj[None, :] <= qi[:, None]
                    if wl >= 0:
                        ok &= kj[None, :] >= qi[:, None] - wl
                    if wr >= 0:
                        ok &= kj[None, :] <= qi[:, None] + wr
                    ok &= kj[None, :] < kl
                    s = np.where(ok, s, -np.inf)
                    m_new = np.maximum(m, s.max(axis=1))
                    live = np.isfinite(m_new)
                    ref = np.where(live, m_new, 0.0)
                    alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
                    e = np.exp(s - ref[:, None])
                    l = l * alpha + e.sum(axis=1)
                    acc = acc * alpha[:, None] + e @ v[b, kj, h, :]
                    m = m_new
                live = l > 0
                out[b, qi, h, :] = np.where(
                    live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
                with np.errstate(divide="ignore"):
                    lse[b, h, qi] = np.where(live, m + np.log(l), -np.inf)
    return out, lse
