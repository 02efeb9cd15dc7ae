"""Seeded synthetic inputs for the attention workloads.

This module draws the inputs that both the HIP path and the CPU oracle receive.
It holds none of the attention arithmetic: only random draws, the block-mask
pattern and round-to-nearest-even conversion to bf16 storage.  It imports
numpy only, so tests and the oracle's callers can use it without the GPU
library.

The five workloads stand in for the shapes the FlashAttention reading guide
(xyznot.com/tr/paper/2205.14135, "Sonuçlar") reports on, without their data:

  tiny      B=1  H=2  N=128   d=64   fp32  dense          exact fp32 check
  gpt2      B=8  H=12 N=1024  d=64   bf16  causal         GPT-2-small attention
  long      B=2  H=16 N=4096  d=128  bf16  causal         1% of K rows x20
  sparse    B=4  H=8  N=8192  d=64   bf16  128-tile block mask, Bernoulli(0.25)
                                           keep pattern plus the diagonal
  verylong  B=1  H=8  N=16384 d=128  bf16  causal         sigma = 0.5
  long_gqa  as long (1% of K rows x20), 4 key/value heads shared by the
            16 query heads
  long_fp8  as long, quantized to FP8 (E4M3) for the FP8 forward
  verylong_shard  B=1 H=1 N=16384 d=128 bf16 causal sigma = 0.5: one GPU's
            share of verylong split by heads over eight GPUs

Recipe (the same for every workload): ``rng = numpy.random.default_rng(seed)``
(PCG64); draw Q, K, V, dO in that order, each
``rng.standard_normal((B, H, N, d), dtype=float32) * sigma`` (K and V with the
key/value head count when it differs); then, for
``long``, choose floor(0.01 * B*H*N) rows of the flattened [B*H*N] K row index
without replacement and multiply those rows by 20; then, for ``sparse``, draw
the [T, T] keep pattern (T = ceil(N/128)) as ``rng.random((T, T)) < 0.25`` and
set its diagonal.  The scale is 1/sqrt(d).  bf16 workloads are rounded to bf16
(round to nearest, ties to even) after all draws; the rounded values are the
inputs of both sides.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

MASK_BLOCK = 128


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str              # "bf16" or "fp32"
    causal: bool
    sigma: float = 1.0
    k_row_frac: float = 0.0  # fraction of K rows scaled by k_row_gain
    k_row_gain: float = 1.0
    mask_density: Optional[float] = None   # Bernoulli keep probability
    seed: int = 0
    Hkv: Optional[int] = None  # key/value heads when grouped (None: H, one per query head)

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hkv is None else self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def tiles(self) -> int:
        return -(-self.N // MASK_BLOCK)

    def with_shape(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 128, 64, "fp32", False, seed=1001),
    "gpt2": Workload("gpt2", 8, 12, 1024, 64, "bf16", True, seed=1002),
    "long": Workload("long", 2, 16, 4096, 128, "bf16", True,
                     k_row_frac=0.01, k_row_gain=20.0, seed=1003),
    "sparse": Workload("sparse", 4, 8, 8192, 64, "bf16", False,
                       mask_density=0.25, seed=1004),
    "verylong": Workload("verylong", 1, 8, 16384, 128, "bf16", True,
                         sigma=0.5, seed=1005),
    # long-context training with grouped key/value heads (4 query heads per
    # key/value head, the grouping of the week-13 page's Llama-3-8B example),
    # with the long workload's large logits: 1% of the K rows x20
    "long_gqa": Workload("long_gqa", 2, 16, 4096, 128, "bf16", True,
                         k_row_frac=0.01, k_row_gain=20.0, seed=1006, Hkv=4),
    # the long-context shape as FP8 (E4M3) inputs for the FP8 forward: Q, K, V
    # drawn as for long (x20 rows included), then quantized by quantize_fp8
    "long_fp8": Workload("long_fp8", 2, 16, 4096, 128, "fp8", True,
                         k_row_frac=0.01, k_row_gain=20.0, seed=1007),
    # the long-context shape without the causal mask (every query row sees
    # every key, as in an encoder), iid N(0, 1) inputs
    "long_nc": Workload("long_nc", 2, 16, 4096, 128, "bf16", False, seed=1008),
    # one GPU's share of verylong when its eight heads are split over eight
    # GPUs (heads are independent): one head of 16K rows, drawn as verylong
    "verylong_shard": Workload("verylong_shard", 1, 1, 16384, 128, "bf16", True,
                               sigma=0.5, seed=1009),
}


@dataclass(frozen=True)
class DecodeWorkload:
    """A few new query rows per sequence against a key/value cache, with
    Hkv cache heads shared by groups of Hq / Hkv query heads."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    d: int
    dtype: str
    causal: bool
    lengths: str = "full"     # "full": every sequence Nkv long; "uniform": U{1..Nkv}
    sigma: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def with_shape(self, **kw) -> "DecodeWorkload":
        return replace(self, **kw)


# Decode shapes from the week-13 page's decode discussion: a batch of 64
# requests at an 8K context, 32 query heads over 8 cache heads (the Llama-3-8B
# grouping it quotes), d = 128; "spec" checks 4 draft tokens per request at
# once (speculative decoding with gamma = 3), causal among themselves.
# Recipe: rng = default_rng(seed); Q [B, Hq, Nq, d], then K, V [B, Hkv, Nkv, d]
# as standard_normal(float32) * sigma; then the lengths (``uniform``:
# rng.integers(1, Nkv + 1, B)); then bf16 rounding.
DECODE_WORKLOADS = {
    "decode": DecodeWorkload("decode", 64, 32, 8, 1, 8192, 128, "bf16", False, seed=1101),
    "decode_mix": DecodeWorkload("decode_mix", 64, 32, 8, 1, 8192, 128, "bf16", False,
                                 lengths="uniform", seed=1102),
    "decode_spec": DecodeWorkload("decode_spec", 64, 32, 8, 4, 8192, 128, "bf16", True,
                                  lengths="uniform", seed=1103),
}


def make_decode_inputs(w: DecodeWorkload, seed: Optional[int] = None) -> dict:
    """Draw the inputs of decode workload ``w``: dict(q [B,Hq,Nq,d],
    k, v [B,Hkv,Nkv,d] float32 holding the storage-type values, seqlens int32
    [B], scale, causal, dtype)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    sig = np.float32(w.sigma)
    q = rng.standard_normal((w.B, w.Hq, w.Nq, w.d), dtype=np.float32) * sig
    k = rng.standard_normal((w.B, w.Hkv, w.Nkv, w.d), dtype=np.float32) * sig
    v = rng.standard_normal((w.B, w.Hkv, w.Nkv, w.d), dtype=np.float32) * sig
    if w.lengths == "full":
        lens = np.full(w.B, w.Nkv, dtype=np.int32)
    elif w.lengths == "uniform":
        lens = rng.integers(1, w.Nkv + 1, size=w.B).astype(np.int32)
    else:
        raise ValueError(f"unknown length mix {w.lengths!r}")
    if w.dtype == "bf16":
        q, k, v = (bf16_round(t) for t in (q, k, v))
    return dict(q=q, k=k, v=v, seqlens=lens, scale=w.scale, causal=w.causal, dtype=w.dtype)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """OCP E4M3 codes (uint8) of float values: round to nearest, ties to even,
    saturating at +-448 (inputs must be finite)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    tiny = a < 2.0 ** -6
    e = np.floor(np.log2(np.where(tiny, 1.0, a)))
    m = np.rint(np.where(tiny, a / 2.0 ** -9, (a / np.exp2(e) - 1.0) * 8.0))   # half to even
    carry = ~tiny & (m == 8)
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code = np.where(tiny, m, (e + 7) * 8 + m).astype(np.int64)
    code = np.minimum(code, 0x7E)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_fp8(q, k, v, block: int = MASK_BLOCK) -> dict:
    """FP8 (E4M3) inputs of the FP8 forward: Q and K with one fp32 scale per
    (batch, head, 128-row block), V with one per (batch, head), scale =
    amax / 448 (1 for an all-zero block); V's codes transposed to [B, H, d, N]."""
    def rows(x):
        B, H, N, d = x.shape
        nb = -(-N // block)
        codes = np.empty(x.shape, np.uint8)
        sc = np.empty((B, H, nb), np.float32)
        for t in range(nb):
            blk = x[:, :, t * block:(t + 1) * block].astype(np.float64)
            amax = np.abs(blk).max(axis=(2, 3))
            s = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
            sc[:, :, t] = s
            codes[:, :, t * block:(t + 1) * block] = e4m3_encode(
                blk / s.astype(np.float64)[:, :, None, None])
        return codes, sc
    q8, sq = rows(q)
    k8, sk = rows(k)
    v64 = np.asarray(v, np.float64)
    amax = np.abs(v64).max(axis=(2, 3))
    sv = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    vt8 = np.ascontiguousarray(e4m3_encode(v64 / sv.astype(np.float64)[:, :, None, None])
                               .transpose(0, 1, 3, 2))
    return dict(q8=q8, k8=k8, vt8=vt8, sq=sq, sk=sk, sv=sv)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32
    holding exactly representable bf16 values.  Inputs must be finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((bits >> 16) & 1)
    bits = ((bits + bias) & 0xFFFF0000).astype(np.uint32)
    return bits.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The uint16 bf16 encoding of float32 values that are already bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def make_block_mask(rng: np.random.Generator, tiles: int, density: float) -> np.ndarray:
    """[T, T] uint8 keep pattern: Bernoulli(density) with the diagonal set."""
    keep = rng.random((tiles, tiles)) < density
    keep[np.arange(tiles), np.arange(tiles)] = True
    return keep.astype(np.uint8)


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw the inputs of workload ``w``.

    Returns dict(q, k, v, do: float32 [B,H,N,d] holding the storage-type
    values, mask: uint8 [T,T] or None, scale, causal, dtype).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    kv_shape = (w.B, w.kv_heads, w.N, w.d)
    q = rng.standard_normal(shape, dtype=np.float32) * np.float32(w.sigma)
    k = rng.standard_normal(kv_shape, dtype=np.float32) * np.float32(w.sigma)
    v = rng.standard_normal(kv_shape, dtype=np.float32) * np.float32(w.sigma)
    do = rng.standard_normal(shape, dtype=np.float32) * np.float32(w.sigma)
    if w.k_row_frac > 0.0:
        rows_total = w.B * w.kv_heads * w.N
        count = int(math.floor(w.k_row_frac * rows_total))
        idx = rng.choice(rows_total, size=count, replace=False)
        flat = k.reshape(rows_total, w.d)
        flat[idx] *= np.float32(w.k_row_gain)
    mask = None
    if w.mask_density is not None:
        mask = make_block_mask(rng, w.tiles, w.mask_density)
    if w.dtype == "bf16":
        q, k, v, do = (bf16_round(t) for t in (q, k, v, do))
    return dict(q=q, k=k, v=v, do=do, mask=mask, scale=w.scale,
                causal=w.causal, dtype=w.dtype)


def random_inputs(B, H, N, d, dtype="bf16", seed=0, sigma=1.0):
    """Plain iid N(0, sigma^2) Q, K, V, dO of any shape (edge-case tests)."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    ts = [rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
          for _ in range(4)]
    if dtype == "bf16":
        ts = [bf16_round(t) for t in ts]
    return dict(zip(("q", "k", "v", "do"), ts))


def random_block_mask(N: int, density: float, seed: int, keep_diag=True) -> np.ndarray:
    """Seeded [ceil(N/128)]^2 uint8 block mask (for edge-case tests)."""
    rng = np.random.default_rng(seed)
    t = -(-N // MASK_BLOCK)
    keep = rng.random((t, t)) < density
    if keep_diag:
        keep[np.arange(t), np.arange(t)] = True
    return keep.astype(np.uint8)
