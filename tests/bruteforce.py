"""Independent fp64 brute force used to pin the oracle (test-only).

Written from the mathematics, not from the oracle: dense masked softmax
attention with a library matmul, and the block decisions of the BLASST skip
test evaluated non-incrementally.  Because the running max of the online
softmax never depends on which blocks were skipped (a skipped block has
m~ < m + ln(lambda) <= m for every row, so max(m, m~) = m anyway), the running
max before block j equals the plain maximum of the scores of blocks 0..j-1;
this module uses that closed form instead of any running state.
"""
import math

import numpy as np


def scores(q, k, scale):
    """S = scale * q k^T for q [R,d], k [N,d]."""
    return scale * (q @ k.T)


def prefill_mask(L, causal, window=0):
    """Visible[i, c] for Lq = Lk = L; ``window`` > 0 keeps c > i - window only."""
    if not causal:
        return np.ones((L, L), dtype=bool)
    m = np.tril(np.ones((L, L), dtype=bool))
    if window > 0:
        m &= ~np.tril(np.ones((L, L), dtype=bool), -window)
    return m


def masked_softmax_attention(S, mask, v):
    """softmax over the visible entries of each row, times v; rows with no visible key give 0."""
    Sm = np.where(mask, S, -np.inf)
    mx = Sm.max(axis=1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    p = np.where(mask, np.exp(Sm - mx), 0.0)
    den = p.sum(axis=1, keepdims=True)
    out = (p @ v) / np.where(den > 0, den, 1.0)
    return np.where(den > 0, out, 0.0)


def dense_probs(S, mask):
    Sm = np.where(mask, S, -np.inf)
    mx = Sm.max(axis=1, keepdims=True)
    p = np.where(mask, np.exp(Sm - mx), 0.0)
    return p / p.sum(axis=1, keepdims=True)


def block_decisions(S, mask, rows_of_unit, block_cols, lam, init=None):
    """Decisions of one unit by the closed form of the running max.

    S, mask: [R_all, N] for the unit's rows (already selected); block_cols:
    list of column ranges, in visiting order; init: per-row running max before
    the first block (default -inf).  Returns (skip list, gap list) with 255 /
    -inf for unvisited blocks.
    """
    lnlam = -math.inf if lam == 0 else math.log(lam)
    R = S.shape[0]
    prev_max = np.full(R, -np.inf) if init is None else np.array(init, dtype=np.float64)
    skips, gaps = [], []
    for (c0, c1) in block_cols:
        m_blk = mask[:, c0:c1]
        if not m_blk.any():
            skips.append(255)
            gaps.append(-math.inf)
            continue
        mt = np.where(m_blk, S[:, c0:c1], -np.inf).max(axis=1)
        d = np.where(mt == -np.inf, -np.inf,
                     np.where(prev_max == -np.inf, np.inf, mt - np.where(np.isfinite(prev_max), prev_max, 0.0)))
        g = d.max()
        gaps.append(g)
        skips.append(1 if g < lnlam else 0)
        prev_max = np.maximum(prev_max, mt)
    return skips, gaps
