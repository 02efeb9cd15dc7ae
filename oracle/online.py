"""Block-by-block (online-softmax) forward in fp64, for self-tests only.

TEST INFRASTRUCTURE (see the package docstring).  These routines exist so the
tests can check, in fp64, that the incremental softmax the method relies on
reaches the plain definition of ``attention.forward`` whatever the block size.
They are written from the pages' description, not from any listing:

* ``merge_stats`` -- the two-part combination rule of [FA-guide]
  "Artımsal Softmax Takibi": for a vector split into x1 and x2,
  m = max(m1, m2) and l = e^(m1 - m) l1 + e^(m2 - m) l2.
* ``tiled_forward_rescaled`` -- [FA-guide] "Yöntem", steps 1-4 for query block
  i and key/value block j: block scores, block-local max / exp / row sum,
  update of the running (m, l), and the running output renormalised by
  diag(l_new)^-1 after every block.
* ``tiled_forward_deferred`` -- [Week-13] Step 2: per query block keep (m, d, o)
  unnormalised; on a new maximum the old d and o are multiplied by
  e^(m_old - m_new); divide by d once at the end.

Both treat a block whose entries are all masked as contributing nothing: the
block max is -inf and no exp(-inf - (-inf)) is ever formed ([Week-13]
"Типичные ошибки").  m starts at -inf, l (or d) at 0, O at 0.
"""

from __future__ import annotations

import numpy as np

from .attention import keep_matrix, MASK_BLOCK


def _exp_diff(a, b):
    """e^(a - b) elementwise, defined as 0 where a = -inf (also when b = -inf),
    so a fully masked part never produces NaN."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    out = np.zeros(np.broadcast(a, b).shape)
    ok = np.broadcast_to(np.isfinite(a) & np.isfinite(b), out.shape)
    with np.errstate(invalid="ignore"):
        diff = np.broadcast_to(a, out.shape) - np.broadcast_to(b, out.shape)
    np.exp(diff, out=out, where=ok)
    return out


def merge_stats(m1, l1, m2, l2):
    """Combine the (max, sum-of-exp) statistics of two parts of a row."""
    m = np.maximum(m1, m2)
    l = _exp_diff(m1, m) * l1 + _exp_diff(m2, m) * l2
    return m, l


def _block_scores(q, k, scale, keep, i0, i1, j0, j1):
    s = scale * (q[i0:i1] @ k[j0:j1].T)
    return np.where(keep[i0:i1, j0:j1], s, -np.inf)


def tiled_forward_rescaled(q, k, v, scale, block_rows, block_cols,
                           causal=False, block_mask=None,
                           mask_block=MASK_BLOCK):
    """One head ([N, d] each): forward via [FA-guide] steps 1-4.

    Returns (O, m, l); the log-sum-exp is m + ln l.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    N, d = q.shape
    keep = keep_matrix(N, N, causal, block_mask, mask_block)
    O = np.zeros((N, d))
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    for i0 in range(0, N, block_rows):
        i1 = min(N, i0 + block_rows)
        for j0 in range(0, N, block_cols):
            j1 = min(N, j0 + block_cols)
            s = _block_scores(q, k, scale, keep, i0, i1, j0, j1)     # step 1
            m_blk = s.max(axis=1)                                     # step 2
            p_blk = _exp_diff(s, m_blk[:, None])
            l_blk = p_blk.sum(axis=1)
            m_old, l_old = m[i0:i1], l[i0:i1]
            m_new, l_new = merge_stats(m_old, l_old, m_blk, l_blk)    # step 3
            a_old = _exp_diff(m_old, m_new)                           # step 4
            a_blk = _exp_diff(m_blk, m_new)
            num = (l_old * a_old)[:, None] * O[i0:i1] \
                + a_blk[:, None] * (p_blk @ v[j0:j1])
            with np.errstate(invalid="ignore", divide="ignore"):
                O[i0:i1] = np.where(l_new[:, None] > 0,
                                    num / np.where(l_new > 0, l_new, 1.0)[:, None],
                                    0.0)
            m[i0:i1], l[i0:i1] = m_new, l_new
    return O, m, l


def tiled_forward_deferred(q, k, v, scale, block_rows, block_cols,
                           causal=False, block_mask=None,
                           mask_block=MASK_BLOCK):
    """One head: forward with unnormalised running (m, d, o) ([Week-13]).

    Returns (O, m, l) like ``tiled_forward_rescaled``.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    N, dh = q.shape
    keep = keep_matrix(N, N, causal, block_mask, mask_block)
    O = np.zeros((N, dh))
    m_all = np.full(N, -np.inf)
    l_all = np.zeros(N)
    for i0 in range(0, N, block_rows):
        i1 = min(N, i0 + block_rows)
        m = np.full(i1 - i0, -np.inf)
        dsum = np.zeros(i1 - i0)
        o = np.zeros((i1 - i0, dh))
        for j0 in range(0, N, block_cols):
            j1 = min(N, j0 + block_cols)
            s = _block_scores(q, k, scale, keep, i0, i1, j0, j1)
            m_new = np.maximum(m, s.max(axis=1))
            alpha = _exp_diff(m, m_new)          # rescale old d and o
            p = _exp_diff(s, m_new[:, None])
            dsum = alpha * dsum + p.sum(axis=1)
            o = alpha[:, None] * o + p @ v[j0:j1]
            m = m_new
        with np.errstate(invalid="ignore", divide="ignore"):
            O[i0:i1] = np.where(dsum[:, None] > 0,
                                o / np.where(dsum > 0, dsum, 1.0)[:, None], 0.0)
        m_all[i0:i1], l_all[i0:i1] = m, dsum
    return O, m_all, l_all
