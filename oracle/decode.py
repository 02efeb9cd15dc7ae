"""Attention of a few new query rows against a long key/value cache
(inference decode) with grouped key/value heads: plain fp64 reference.

TEST INFRASTRUCTURE (see the package docstring): never called by the product
path.

[Week-13] (the bullet on decode attention next to "Критический размер
батча") observes that in decode every request reads its own cache, so its
arithmetic intensity is about (query heads / key-value heads) FLOP per byte
whatever the batch, and that grouped key/value heads (GQA) make each byte of
cache serve several query heads.  The same page quotes a context of 8K and a
decode batch of 64 requests; speculative decoding checks B (gamma + 1) new
tokens at once.  Readings taken here (the plainest ones the pages support):

  * Shapes: Q [B, Hq, Nq, d] (the Nq newest tokens of each sequence), a cache
    K, V [B, Hkv, Nkv, d] with Hkv dividing Hq; query head h reads cache head
    h // G, G = Hq / Hkv (consecutive query heads share a cache head).
  * Sequence b holds L_b = seqlens[b] valid cache rows (all Nkv when no
    lengths are given); rows at or past L_b are never read.
  * The Nq new tokens are the last Nq positions of the sequence.  Without
    causal masking every query row sees all L_b keys; with it, query row i
    sees key j iff j <= L_b - Nq + i (the causal mask aligned to the end of
    the sequence).  For L_b = Nq this is the training path's causal mask.
  * O = softmax(scale Q K^T) V over the visible keys and LSE = m + ln l, as in
    the training forward; a row that sees no key gets O = 0, LSE = -inf.

How the GPU splits the keys into chunks and merges the partial results
(the two-part rule of [FA-guide] "Artımsal Softmax Takibi") is its own
business: the definition here takes all keys at once.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64, _softmax_rows


def visible_keys(L: int, Nq: int, causal: bool) -> np.ndarray:
    """Boolean [Nq, L] matrix: query row i sees key j (module docstring)."""
    i = np.arange(Nq)[:, None]
    j = np.arange(L)[None, :]
    if causal:
        return j <= L - Nq + i
    return np.ones((Nq, L), dtype=bool)


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """Cache head read by query head h (module docstring)."""
    return h // (Hq // Hkv)


def decode_forward(q, k, v, scale: float, seqlens=None, causal: bool = False):
    """O [B, Hq, Nq, d] and LSE [B, Hq, Nq] (fp64) of the module docstring."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, d = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("the query head count must be a multiple of the key/value head count")
    lens = np.full(B, Nkv) if seqlens is None else np.asarray(seqlens)
    o = np.zeros((B, Hq, Nq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        L = int(lens[b])
        if not 0 <= L <= Nkv:
            raise ValueError("sequence lengths must lie in [0, Nkv]")
        if L == 0:
            continue
        vis = visible_keys(L, Nq, causal)
        for h in range(Hq):
            kvh = kv_head(h, Hq, Hkv)
            s = scale * (q[b, h] @ k[b, kvh, :L].T)
            s = np.where(vis, s, -np.inf)
            p, _, lse[b, h] = _softmax_rows(s)
            o[b, h] = p @ v[b, kvh, :L]
    return o, lse
