"""Attention with grouped key/value heads (GQA / MQA) in the training path:
plain fp64 reference for the forward and the backward.

TEST INFRASTRUCTURE (see the package docstring): never called by the product
path.

[Week-13] (its decode bullet) names GQA: groups of query heads share one key
and value head, so the cache is smaller and each byte of it serves several
heads.  Readings taken here (the plainest ones the pages support):

  * Q, O, dO, dQ: [B, Hq, N, d]; K, V, dK, dV: [B, Hkv, N, d], Hq = G Hkv;
    query head h attends with key/value head h // G (consecutive query heads
    share a head), under the same causal / block mask as the plain path.
  * Forward: per query head exactly the plain attention of oracle.attention.
  * Backward: dQ per query head as in the plain path; a shared key or value
    head receives the sum over its G query heads of their contributions
    (dK_k = sum_{h: h//G = k} scale dS_h^T Q_h, dV_k = sum P_h^T dO_h), which
    is what the chain rule gives when one tensor feeds G heads.
  * MQA is the case Hkv = 1; Hkv = Hq is the plain path.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64, _head_backward, _head_forward, keep_matrix, MASK_BLOCK


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """Key/value head used by query head h."""
    return h // (Hq // Hkv)


def _accumulate(grad, head, contribution):
    """A shared head's gradient is the sum of its query heads' contributions."""
    grad[head] += contribution


def forward_backward(q, k, v, do, scale: float, causal: bool = False, block_mask=None,
                     mask_block: int = MASK_BLOCK):
    """O, LSE, dQ ([B, Hq, ...]) and dK, dV ([B, Hkv, ...]) in fp64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("the query head count must be a multiple of the key/value head count")
    keep = keep_matrix(N, N, causal, block_mask, mask_block)
    out = {"O": np.empty_like(q), "dQ": np.empty_like(q), "LSE": np.empty((B, Hq, N)),
           "dK": np.zeros_like(k), "dV": np.zeros_like(v)}
    for b in range(B):
        for h in range(Hq):
            c = kv_head(h, Hq, Hkv)
            p, o, lse = _head_forward(q[b, h], k[b, c], v[b, c], scale, keep)
            dq, dk, dv = _head_backward(q[b, h], k[b, c], v[b, c], o, do[b, h], p, scale)
            out["O"][b, h], out["LSE"][b, h], out["dQ"][b, h] = o, lse, dq
            _accumulate(out["dK"], (b, c), dk)
            _accumulate(out["dV"], (b, c), dv)
    return out


def query_rows(q, k, v, do, scale: float, h: int, rows, causal: bool = False,
               block_mask=None, mask_block: int = MASK_BLOCK):
    """O, LSE, dQ of query head h of one batch entry for the rows ``rows``
    (q, do: [Hq, N, d]; k, v: [Hkv, N, d])."""
    from .attention import query_rows as plain_rows
    c = kv_head(h, q.shape[0], k.shape[0])
    return plain_rows(q[h], k[c], v[c], do[h], scale, rows, causal, block_mask, mask_block)


def key_rows(q, k, v, do, scale: float, c: int, cols, causal: bool = False,
             block_mask=None, mask_block: int = MASK_BLOCK):
    """dK and dV of key/value head c of one batch entry for the key rows
    ``cols``: the sum over the query heads that share head c (q, do:
    [Hq, N, d]; k, v: [Hkv, N, d])."""
    from .attention import key_rows as plain_key_rows
    Hq, Hkv = q.shape[0], k.shape[0]
    dk = dv = 0.0
    for h in range(Hq):
        if kv_head(h, Hq, Hkv) == c:
            r = plain_key_rows(q[h], k[c], v[c], do[h], scale, cols, causal, block_mask,
                               mask_block)
            dk = dk + r["dK"]
            dv = dv + r["dV"]
    return {"dK": dk, "dV": dv}
