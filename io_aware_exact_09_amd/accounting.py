"""Work accounting for the benchmark: kept (query, key) pairs, algorithmic
FLOPs and algorithmic HBM bytes per kernel.  Host logic only.

Algorithmic FLOPs count the contractions the method needs on kept pairs:
forward 4 d per pair (S = Q K^T and P V), backward 10 d per pair (recomputed
S, dV = P^T dO, dP = dO V^T, dQ = dS K, dK = dS^T Q).  Per kernel:
  fwd     4 d P
  dkdv    8 d P   (S, dP, dV, dK)
  dq      2 d P   (dQ; its recomputation of S and dP is not counted)
"""

from __future__ import annotations

import numpy as np

MASK_BLOCK = 128


def kept_pairs(N: int, causal: bool, mask=None, block: int = MASK_BLOCK) -> int:
    """Kept (query, key) pairs of one head, counted tile by tile."""
    T = -(-N // block)
    sizes = np.array([min(block, N - t * block) for t in range(T)], dtype=np.int64)
    full = np.outer(sizes, sizes)
    keep = np.ones((T, T), dtype=bool) if mask is None else (np.asarray(mask) != 0)
    if causal:
        tri = np.tril(np.ones((T, T), dtype=bool), -1)
        diag = sizes * (sizes + 1) // 2
        return int(full[keep & tri].sum() + diag[np.diag(keep)].sum())
    return int(full[keep].sum())


def flops(B: int, H: int, N: int, d: int, causal: bool, mask=None) -> dict:
    p = B * H * kept_pairs(N, causal, mask)
    return {"pairs": p, "fwd": 4 * d * p, "bwd": 10 * d * p,
            "fwd_kernel": 4 * d * p, "dkdv_kernel": 8 * d * p, "dq_kernel": 2 * d * p,
            "dq_kernel_executed": 6 * d * p}


def hbm_bytes(B: int, H: int, N: int, d: int, elem: int) -> dict:
    """Minimal algorithmic HBM bytes per kernel: every [B,H,N,d] tensor the
    kernel touches is read or written once (d * elem bytes per row), LSE and
    D are 4 bytes per row."""
    rows = B * H * N
    t = rows * d * elem
    r = rows * 4
    return {
        "fwd_kernel": 3 * t + t + r,                 # read Q K V, write O, LSE
        "pre_kernel": 2 * t + r,                     # read O dO, write D
        "dkdv_kernel": 4 * t + 2 * r + 2 * t,        # read Q K V dO LSE D, write dK dV
        "dq_kernel": 4 * t + 2 * r + t,              # read Q K V dO LSE D, write dQ
        "dq_and_d_kernel": 5 * t + 2 * r + t,        # read Q K V O dO LSE, write D dQ
    }


def decode_bytes(B: int, Hq: int, Hkv: int, Nq: int, d: int, elem: int, seqlens) -> dict:
    """Minimal algorithmic HBM bytes of one decode call: the visible cache rows
    of K and V read once (each cache head once, whatever the number of query
    heads sharing it), Q read and O written once, LSE 4 bytes per row.  Also
    the matrix FLOPs (4 d per query row and visible key; causal rows of the
    Nq new tokens see slightly fewer keys, which is ignored)."""
    kv_rows = int(np.asarray(seqlens, dtype=np.int64).sum()) * Hkv
    rows = B * Hq * Nq
    cache = 2 * kv_rows * d * elem
    qo = 2 * rows * d * elem + 4 * rows
    flops = 4 * d * Nq * (Hq // Hkv) * kv_rows
    return {"cache": cache, "q_o_lse": qo, "total": cache + qo, "flops": flops}
