"""Attention with dropout on the probabilities: plain fp64 reference.

TEST INFRASTRUCTURE (see the package docstring): never called by the product
path.

[FA-guide] "Temel fikirler" lists dropout among the operations the method
fuses into its one kernel next to the matrix products, masking and softmax;
the pages say nothing more about it.  Readings taken here (the plainest ones
the rest of the pages support):

  * Dropout acts on the attention probabilities: with keep mask Z (Z_ij in
    {0, 1}, kept with probability 1 - p) and M = Z / (1 - p),
        O = (P * M) V.
    The softmax statistics (row max, row sum, LSE) are those of the
    undropped P, so LSE is unchanged by dropout.
  * Backward, by the chain rule through the same formula:
        dV = (P * M)^T dO
        dP = (dO V^T) * M
        D_i = sum_k dO_ik O_ik      (still equals sum_j P_ij dP_ij)
        dS = P * (dP - D 1^T),  dQ = scale dS K,  dK = scale dS^T Q.
  * The mask is not stored: forward and backward regenerate it from a
    counter-based generator, Philox4x32 with 10 rounds (Salmon, Moraes, Dror,
    Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011).  One call
    serves a 2 x 4 block of the score matrix: element (i, j) of head bh
    (= b H + h) takes word j mod 4 of
        Philox4x32-10(counter = (j // 4, i // 2, bh, 0), key = (seed mod 2^32,
                      seed // 2^32)),
    its low 16 bits for even i and its high 16 bits for odd i, and is kept
    iff that 16-bit value is >= T = floor(p 2^16) (clamped to 2^16 - 1; p = 0
    keeps all).  The drop probability is so T / 2^16, within 2^-16 of p; the
    kept probabilities are still scaled by 1 / (1 - p).

The generator is written from its published definition below, in numpy
uint64 arithmetic; nothing is shared with the GPU library.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64, _softmax_rows, keep_matrix, MASK_BLOCK

# Philox4x32 constants from the paper: the two round multipliers and the two
# Weyl increments of the key schedule.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32(ctr, key, rounds: int = 10):
    """Philox4x32-R on arrays.

    ctr: four uint32 arrays (broadcastable), key: two uint32 values or
    arrays.  One round maps (c0, c1, c2, c3) with key (k0, k1) to
        (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),  hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0))
    where hi/lo are the upper/lower 32 bits of the 64-bit product; between
    rounds the key advances by (W0, W1) modulo 2^32.  Returns four uint32
    arrays.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in ctr)
    k0 = np.uint64(int(key[0]) & MASK32)
    k1 = np.uint64(int(key[1]) & MASK32)
    for r in range(rounds):
        if r > 0:
            k0 = np.uint64((int(k0) + PHILOX_W0) & MASK32)
            k1 = np.uint64((int(k1) + PHILOX_W1) & MASK32)
        p0 = c0 * np.uint64(PHILOX_M0)          # < 2^64: no overflow
        p1 = c2 * np.uint64(PHILOX_M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


MASK16 = 0xFFFF


def threshold(p: float) -> int:
    """Integer keep threshold T = floor(p 2^16) (clamped to 2^16 - 1)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    return min(int(np.floor(p * 65536.0)), MASK16)


def keep_mask(bh: int, rows, cols, p: float, seed: int) -> np.ndarray:
    """Boolean keep mask Z[rows, cols] of head bh (see the module docstring)."""
    rows = np.asarray(rows, dtype=np.uint64)[:, None]
    cols = np.asarray(cols, dtype=np.uint64)[None, :]
    words = philox4x32((cols >> np.uint64(2), rows >> np.uint64(1), np.full_like(cols, bh),
                        np.zeros_like(cols)),
                       (seed & MASK32, (seed >> 32) & MASK32))
    w = np.stack(np.broadcast_arrays(*words), axis=-1)          # [rows, cols, 4]
    pick = (cols & np.uint64(3)).astype(np.int64)
    r = np.take_along_axis(w, np.broadcast_to(pick, w.shape[:2])[..., None], axis=-1)[..., 0]
    half = (r.astype(np.uint64) >> (np.uint64(16) * (rows & np.uint64(1)))) & np.uint64(MASK16)
    return half >= np.uint64(threshold(p))


def _head(q, k, v, do, keep, scale: float, p: float, seed: int, bh: int):
    """One head (2-D arrays): the formulas of the module docstring with the
    keep mask of head index bh."""
    N = q.shape[0]
    idx = np.arange(N)
    s = scale * (q @ k.T)
    s = np.where(keep, s, -np.inf)
    pr, _, lse = _softmax_rows(s)
    m = keep_mask(bh, idx, idx, p, seed) * (1.0 / (1.0 - p))
    o = (pr * m) @ v
    dv = (pr * m).T @ do
    dp = (do @ v.T) * m
    dvec = (do * o).sum(axis=1)
    ds = pr * (dp - dvec[:, None])
    return {"O": o, "LSE": lse, "dQ": scale * (ds @ k), "dK": scale * (ds.T @ q), "dV": dv}


def forward_backward(q, k, v, do, scale: float, p: float, seed: int, causal: bool = False,
                     block_mask=None, mask_block: int = MASK_BLOCK):
    """Forward and backward of attention with dropout (module docstring).

    Returns a dict with O, LSE, dQ, dK, dV (fp64).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    keep = keep_matrix(N, N, causal, block_mask, mask_block)
    out = {name: np.empty_like(q) for name in ("O", "dQ", "dK", "dV")}
    out["LSE"] = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            r = _head(q[b, h], k[b, h], v[b, h], do[b, h], keep, scale, p, seed, b * H + h)
            for name in out:
                out[name][b, h] = r[name]
    return out


def head_outputs(q, k, v, do, scale: float, p: float, seed: int, b: int, h: int,
                 causal: bool = False, block_mask=None, mask_block: int = MASK_BLOCK):
    """The outputs of head (b, h) of [B, H, N, d] inputs alone (full-size
    checks on a few heads): the per-head step of ``forward_backward``, with
    the head's own mask index b H + h."""
    H = q.shape[1]
    keep = keep_matrix(q.shape[2], q.shape[2], causal, block_mask, mask_block)
    return _head(_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _f64(do[b, h]), keep, scale, p,
                 seed, b * H + h)
