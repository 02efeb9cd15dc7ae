"""Plain fp64 attention: materialised S and P, closed-form backward.

TEST INFRASTRUCTURE (see the package docstring): never called by the product
path.

What is computed, per (batch, head), on the values the caller passes (the GPU
receives the very same values, already rounded to its storage type):

  1. S = scale * Q K^T                       (N x N)
     The attention formula softmax(Q K^T / sqrt(d)) V is [Training-FA] §1;
     [FA-guide] "Problem ve motivasyon" writes S = Q K^T without the scale,
     which is the case scale = 1.  The scale is a parameter here.
  2. Masking: a pair (i, j) is kept when (not causal or j <= i) and (no block
     mask or M[i // 128][j // 128] != 0).  Dropped pairs get S_ij = -inf.
     Causal tile skipping is [Week-13] Step 2; the block mask
     M in {0,1}^{N/B_r x N/B_c} is [FA-guide] "Blok-Seyrek FlashAttention".
     Reading: the mask has a fixed 128 x 128 granularity (parameter
     ``mask_block`` so tiny tests can use smaller blocks) and one mask is
     shared by every (batch, head).
  3. Forward: m_i = max_j S_ij, P = exp(S - m) / rowsum, O = P V and the
     per-row log-sum-exp LSE_i = m_i + ln sum_j exp(S_ij - m_i).  Only O and
     this per-row statistic are what the method keeps for the backward
     ([Training-FA] §2.1 and §3.1; [Week-13] Step 2 stores the logsumexp;
     [FA-guide] "Temel fikirler" stores (l, m)).
     Reading for a row that keeps no key (possible only with a block mask that
     drops a diagonal tile): P_i = 0, O_i = 0, LSE_i = -inf, no NaN
     ([Week-13] "Типичные ошибки" warns about exp(-inf - (-inf))).
  4. Backward, by the chain rule through softmax (the pages print a garbled
     dQ/dK in [Training-FA] §3; the closed form below is what differentiating
     step 3 gives and is pinned by finite differences in the tests):
        dV = P^T dO
        dP = dO V^T
        D_i = sum_k dO_ik O_ik
        dS = P * (dP - D 1^T)
        dQ = scale * dS K
        dK = scale * dS^T Q
     Recomputing S and P here (instead of storing them) mirrors
     [Training-FA] §3.1; the result is the same either way.

Everything is fp64.  Tensors are [B, H, N, d] numpy arrays (any float dtype;
converted to fp64).  Heads are processed one at a time so memory stays at a few
N x N fp64 matrices.
"""

from __future__ import annotations

import numpy as np

MASK_BLOCK = 128


def keep_matrix(n_q: int, n_k: int, causal: bool, block_mask=None,
                mask_block: int = MASK_BLOCK) -> np.ndarray:
    """Boolean [n_q, n_k] matrix of kept (query, key) pairs (step 2 above).

    ``n_q == n_k`` for self-attention; the two sizes are separate only so that
    row subsets can be evaluated (``rows`` index the query side).
    """
    return keep_rows(np.arange(n_q), n_k, causal, block_mask, mask_block)


def keep_rows(rows, n_k: int, causal: bool, block_mask=None,
              mask_block: int = MASK_BLOCK) -> np.ndarray:
    """Kept pairs for the query rows ``rows`` (absolute indices) against all
    ``n_k`` keys."""
    return keep_pairs(rows, np.arange(n_k), causal, block_mask, mask_block)


def keep_pairs(rows, cols, causal: bool, block_mask=None,
               mask_block: int = MASK_BLOCK) -> np.ndarray:
    """Kept pairs for query rows ``rows`` and key rows ``cols`` (absolute
    indices), as a [len(rows), len(cols)] boolean matrix."""
    i = np.asarray(rows)[:, None]
    j = np.asarray(cols)[None, :]
    keep = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if causal:
        keep &= j <= i
    if block_mask is not None:
        bm = np.asarray(block_mask)
        keep &= bm[i // mask_block, j // mask_block] != 0
    return keep


def _softmax_rows(s: np.ndarray):
    """Row softmax of a score block whose dropped entries are -inf.

    Returns (P, m, lse).  A row with every entry -inf gives P = 0,
    m = -inf, lse = -inf.
    """
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for dropped pairs
    l = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(l[:, None] > 0, e / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = np.where(l > 0, m_safe + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return p, m, lse


def _head_forward(q, k, v, scale, keep):
    s = scale * (q @ k.T)
    s = np.where(keep, s, -np.inf)
    p, _, lse = _softmax_rows(s)
    o = p @ v
    return p, o, lse


def _head_backward(q, k, v, o, do, p, scale):
    dv = p.T @ do
    dp = do @ v.T
    dvec = (do * o).sum(axis=1)
    ds = p * (dp - dvec[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def forward(q, k, v, scale: float, causal: bool = False, block_mask=None,
            mask_block: int = MASK_BLOCK):
    """Exact forward.  Returns (O [B,H,N,d], LSE [B,H,N]) in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    keep = keep_matrix(N, N, causal, block_mask, mask_block)
    o = np.empty_like(q)
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            _, o[b, h], lse[b, h] = _head_forward(q[b, h], k[b, h], v[b, h],
                                                  scale, keep)
    return o, lse


def forward_backward(q, k, v, do, scale: float, causal: bool = False,
                     block_mask=None, mask_block: int = MASK_BLOCK):
    """Exact forward and backward.

    Returns a dict with O, LSE, dQ, dK, dV (fp64).  The backward uses the
    oracle's own O for D = rowsum(dO * O).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    keep = keep_matrix(N, N, causal, block_mask, mask_block)
    out = {name: np.empty_like(q) for name in ("O", "dQ", "dK", "dV")}
    out["LSE"] = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            p, o, lse = _head_forward(q[b, h], k[b, h], v[b, h], scale, keep)
            dq, dk, dv = _head_backward(q[b, h], k[b, h], v[b, h], o,
                                        do[b, h], p, scale)
            out["O"][b, h], out["LSE"][b, h] = o, lse
            out["dQ"][b, h], out["dK"][b, h], out["dV"][b, h] = dq, dk, dv
    return out


def backward(q, k, v, do, scale: float, causal: bool = False, block_mask=None,
             mask_block: int = MASK_BLOCK):
    """Exact gradients (dQ, dK, dV) of sum(O * dO), recomputing S and P."""
    r = forward_backward(q, k, v, do, scale, causal, block_mask, mask_block)
    return r["dQ"], r["dK"], r["dV"]


# --------------------------------------------------------------------------
# Row-restricted evaluation for large sizes.  Each query row of the forward,
# and each query row of dQ, depends only on that row of S; each key row of
# dK and dV needs one column of S and the per-row statistics (LSE, D) of every
# query row.  These helpers evaluate the same formulas as above, restricted to
# the requested rows, so a full-size result can be checked on a sample.
# --------------------------------------------------------------------------

def forward_rows(q, k, v, scale: float, rows, causal: bool = False,
                 block_mask=None, mask_block: int = MASK_BLOCK):
    """O and LSE of one head for the query rows ``rows``.

    q, k, v: [N, d] (one head).  Returns (O [len(rows), d], LSE [len(rows)]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.asarray(rows)
    keep = keep_rows(rows, k.shape[0], causal, block_mask, mask_block)
    _, o, lse = _head_forward(q[rows], k, v, scale, keep)
    return o, lse


def query_rows(q, k, v, do, scale: float, rows, causal: bool = False,
               block_mask=None, mask_block: int = MASK_BLOCK):
    """O, LSE and dQ of one head for the query rows ``rows``.

    q, k, v, do: [N, d] (one head).  D_i uses the oracle's own O_i.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    rows = np.asarray(rows)
    keep = keep_rows(rows, k.shape[0], causal, block_mask, mask_block)
    p, o, lse = _head_forward(q[rows], k, v, scale, keep)
    dp = do[rows] @ v.T
    dvec = (do[rows] * o).sum(axis=1)
    ds = p * (dp - dvec[:, None])
    dq = scale * (ds @ k)
    return {"O": o, "LSE": lse, "dQ": dq}


def key_rows(q, k, v, do, scale: float, cols, causal: bool = False,
             block_mask=None, mask_block: int = MASK_BLOCK, row_chunk: int = 2048):
    """dK and dV of one head for the key rows ``cols``.

    Needs LSE_i and D_i of every query row; they are computed from full rows
    of S, ``row_chunk`` query rows at a time (each row's softmax is evaluated
    exactly as in the full forward).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    cols = np.asarray(cols)
    N = q.shape[0]
    lse = np.empty(N)
    dvec = np.empty(N)
    for r0 in range(0, N, row_chunk):
        rows = np.arange(r0, min(N, r0 + row_chunk))
        keep = keep_rows(rows, N, causal, block_mask, mask_block)
        _, o, lse[rows] = _head_forward(q[rows], k, v, scale, keep)
        dvec[rows] = (do[rows] * o).sum(axis=1)
    # Column block of S for the requested keys, over all query rows.
    keep_c = keep_pairs(np.arange(N), cols, causal, block_mask, mask_block)
    s = scale * (q @ k[cols].T)
    with np.errstate(invalid="ignore"):
        p = np.where(keep_c & np.isfinite(lse)[:, None],
                     np.exp(np.where(keep_c, s, 0.0)
                            - np.where(np.isfinite(lse), lse, 0.0)[:, None]),
                     0.0)
    dv = p.T @ do
    dp = do @ v[cols].T
    ds = p * (dp - dvec[:, None])
    dk = scale * (ds.T @ q)
    return {"dK": dk, "dV": dv}


# --------------------------------------------------------------------------
# Work accounting (cross-checks the library's own pair counting).
# --------------------------------------------------------------------------

def kept_pairs(N: int, causal: bool, block_mask=None,
               mask_block: int = MASK_BLOCK) -> int:
    """Number of kept (query, key) pairs of one head."""
    if block_mask is None and not causal:
        return N * N
    if block_mask is None:
        return N * (N + 1) // 2
    return int(keep_matrix(N, N, causal, block_mask, mask_block).sum())

