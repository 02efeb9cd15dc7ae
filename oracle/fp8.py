"""8-bit floating point (FP8 E4M3) attention forward: plain fp64 reference.

TEST INFRASTRUCTURE (see the package docstring): never called by the product
path.

[Training-FA] (its list of FlashAttention versions) and [Week-13] (its note on
FA2 and FA3) say only that FlashAttention-3 supports FP8.  Readings taken here
(the plainest ones the pages support; the number format is fixed by the OCP
8-bit floating point specification, OFP8, E4M3 variant, which is the FP8
format of the gfx950 matrix cores):

  * E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
    is subnormal (value m 2^-9), the code S.1111.111 is NaN, there is no
    infinity, the largest finite magnitude is 448.  Conversion rounds to the
    nearest code, ties to the code with an even mantissa, and saturates to
    +-448.
  * Inputs are quantized in blocks: Q and K per (batch, head, 128-row block),
    V per (batch, head), each with an fp32 scale s = amax / 448 (1 for an
    all-zero block), code = E4M3(x / s); the value a code stands for is
    decode(code) * s.  V is supplied transposed, [B, H, d, N], so that the
    P V product contracts over contiguous bytes.
  * What the method computes is exact attention on those values:
        O = softmax(scale * Qd Kd^T) Vd,  LSE as in the plain forward,
    Qd, Kd, Vd the dequantized tensors.  The GPU also rounds the probabilities
    to E4M3 before the P V product (as FlashAttention-3 does); that error is
    bounded in ``o_error_bound``.
  * The FP8 matrix instruction does not add its 64 products in full fp32
    precision (measured on gfx950 with a one-wave probe, and re-checked by the
    GPU tests): it returns C + sum_k p_k up to an error of a few units of
    2^(E - 14), E = floor(log2 max(|C|, max_k |p_k|)) -- at most 8.8 such units
    over 40,960 random sums, unbiased for products of mixed sign.  The scores,
    and so LSE, carry that error; ``lse_allowance`` bounds it with 16 units
    per instruction (about twice the largest seen).  Products of two E4M3
    values are exact, so the scores' only other error is this one.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64, _head_forward, keep_matrix, MASK_BLOCK

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


# Non-negative finite codes 0x00 .. 0x7E in increasing order of value.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = decode(_POS_CODES)


def encode(x) -> np.ndarray:
    """E4M3 codes of float values: nearest code, ties to the even mantissa,
    saturating to +-448.  NaN inputs give the NaN code."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, 0x7E)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x), E4M3_NAN, code)
    return code.astype(np.uint8)


def quantize_rows(x, block: int = MASK_BLOCK):
    """Per (batch, head, row block) quantization of [B, H, N, d] values:
    returns (codes uint8 [B, H, N, d], scales float32 [B, H, ceil(N/block)])."""
    x = _f64(x)
    B, H, N, d = x.shape
    nb = -(-N // block)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    for t in range(nb):
        blk = x[:, :, t * block:(t + 1) * block]
        amax = np.abs(blk).max(axis=(2, 3))
        s = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
        scales[:, :, t] = s
        codes[:, :, t * block:(t + 1) * block] = encode(blk / s.astype(np.float64)[:, :, None, None])
    return codes, scales


def quantize_heads_transposed(v):
    """Per (batch, head) quantization of V [B, H, N, d], returned transposed:
    (codes uint8 [B, H, d, N], scales float32 [B, H])."""
    v = _f64(v)
    amax = np.abs(v).max(axis=(2, 3))
    s = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
    codes = encode(v / s.astype(np.float64)[:, :, None, None])
    return np.ascontiguousarray(codes.transpose(0, 1, 3, 2)), s


def dequantize(q8, k8, vt8, sq, sk, sv, block: int = MASK_BLOCK):
    """fp64 Q, K, V [B, H, N, d] that the codes and scales stand for."""
    rows = np.arange(q8.shape[2]) // block
    q = decode(q8) * np.asarray(sq, np.float64)[:, :, rows, None]
    k = decode(k8) * np.asarray(sk, np.float64)[:, :, rows, None]
    v = decode(vt8).transpose(0, 1, 3, 2) * np.asarray(sv, np.float64)[:, :, None, None]
    return q, k, v


def forward(q8, k8, vt8, sq, sk, sv, scale: float, causal: bool = False, block_mask=None,
            mask_block: int = MASK_BLOCK):
    """Exact attention on the dequantized inputs: (O, LSE) in fp64."""
    q, k, v = dequantize(q8, k8, vt8, sq, sk, sv, mask_block)
    B, H, N, d = q.shape
    keep = keep_matrix(N, N, causal, block_mask, mask_block)
    o = np.empty_like(q)
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            _, o[b, h], lse[b, h] = _head_forward(q[b, h], k[b, h], v[b, h], scale, keep)
    return o, lse


def o_error_bound(q8, k8, vt8, sq, sk, sv, scale: float, causal: bool = False,
                  block_mask=None, mask_block: int = MASK_BLOCK, shift: int = 8):
    """Elementwise bound on |O_gpu - O| from rounding the probabilities to
    E4M3 before the P V product.

    The GPU forms P~_j = 2^(shift + s_j log2 e - m) with m a reference that
    trails the running max by less than 0.75 (so a kept P~ is at most
    2^(shift + 0.75) < 448, still a normal E4M3 value, and the row sum
    l >= 2^shift, the key that set m contributing 2^shift), rescales by
    alpha <= 1 when m moves, and divides by the fp32 row sum of the
    unrounded P~.  A rounded normal value is within 2^-4 relative, a
    subnormal one (below 2^-6) within 2^-10 absolute, so
        |O_gpu - O|_ik <= s_v (2^-4 (P |V8|)_ik + 2^-10 2^-shift sum_j |V8_jk|)
    over kept keys j, V8 the decoded codes.  Returns that bound.
    """
    q, k, v = dequantize(q8, k8, vt8, sq, sk, sv, mask_block)
    v8 = decode(vt8).transpose(0, 1, 3, 2)
    B, H, N, d = q.shape
    keep = keep_matrix(N, N, causal, block_mask, mask_block)
    bound = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            p, _, _ = _head_forward(q[b, h], k[b, h], v[b, h], scale, keep)
            av = np.abs(v8[b, h])
            bound[b, h] = float(sv[b, h]) * (2.0 ** -4 * (p @ av)
                                             + 2.0 ** (-10 - shift) * (keep @ av))
    return bound


def head_rows(q8, k8, vt8, sq, sk, sv, b: int, h: int, rows, scale: float,
              causal: bool = False, block_mask=None, mask_block: int = MASK_BLOCK,
              shift: int = 8):
    """O, LSE and the P-rounding bound of ``o_error_bound`` (same ``shift``)
    for the query rows ``rows`` of head (b, h) (full-size checks on a
    sample): the same formulas as ``forward`` and ``o_error_bound``,
    restricted to those rows."""
    from .attention import keep_rows
    sl = (slice(b, b + 1), slice(h, h + 1))
    q, k, v = dequantize(q8[sl], k8[sl], vt8[sl], np.asarray(sq)[sl], np.asarray(sk)[sl],
                         np.asarray(sv)[sl], mask_block)
    q, k, v = q[0, 0], k[0, 0], v[0, 0]
    rows = np.asarray(rows)
    keep = keep_rows(rows, k.shape[0], causal, block_mask, mask_block)
    p, o, lse = _head_forward(q[rows], k, v, scale, keep)
    av = np.abs(decode(vt8[b, h]).T)
    bound = float(sv[b, h]) * (2.0 ** -4 * (p @ av) + 2.0 ** (-10 - shift) * (keep @ av))
    return {"O": o, "LSE": lse, "bound": bound}


# Accumulation model of the FP8 matrix instruction (module docstring): the
# result is within UNITS * 2^(E - WINDOW) of the exact C + sum of products.
MFMA_WINDOW = 14
MFMA_UNITS = 16.0
MFMA_GROUP = 64          # products per instruction and output element


def _pow2_floor(x):
    """2^floor(log2 x) for x > 0, 0 for x == 0."""
    x = np.asarray(x, np.float64)
    out = np.zeros_like(x)
    pos = x > 0
    out[pos] = np.exp2(np.floor(np.log2(x[pos])))
    return out


def lse_allowance(q8, k8, sq, sk, scale: float, causal: bool = False, block_mask=None,
                  mask_block: int = MASK_BLOCK, units: float = MFMA_UNITS,
                  window: int = MFMA_WINDOW):
    """Per-row bound [B, H, N] on |LSE_gpu - LSE| that the FP8 instruction's
    accumulation allows.

    Score s_ij = scale sQ_i sK_j S_ij with S_ij = sum_k a_ik b_jk over the
    decoded codes, formed by d / 64 instructions in order; instruction g adds
    the products of its 64 dimensions to the partial sum C_g of the earlier
    ones, with an error of at most units * 2^(E_g - window),
    E_g = floor(log2 max(|C_g|, max_k |a_ik b_jk|)) (products bounded by the
    row maxima of the codes in that group).  LSE_i = ln sum_j exp(s_ij) moves
    by at most the largest change of a kept score, so the allowance of row i
    is max over kept j of |scale| sQ_i sK_j sum_g units 2^(E_g - window).
    (A row that keeps nothing has no LSE to move: allowance 0.)
    """
    from .attention import keep_rows
    a_all, b_all = decode(q8), decode(k8)
    B, H, N, d = a_all.shape
    rows_blk = np.arange(N) // mask_block
    out = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            a, bk = a_all[b, h], b_all[b, h]
            fq = abs(scale) * np.asarray(sq, np.float64)[b, h][rows_blk]        # per query row
            fk = np.asarray(sk, np.float64)[b, h][rows_blk]                      # per key row
            partial = np.zeros((N, N))
            err = np.zeros((N, N))
            for g0 in range(0, d, MFMA_GROUP):
                ga, gb = a[:, g0:g0 + MFMA_GROUP], bk[:, g0:g0 + MFMA_GROUP]
                pmax = np.abs(ga).max(1)[:, None] * np.abs(gb).max(1)[None, :]
                err += units * _pow2_floor(np.maximum(np.abs(partial), pmax)) * 2.0 ** -window
                partial = partial + ga @ gb.T
            ds = fq[:, None] * fk[None, :] * err
            keep = keep_rows(np.arange(N), N, causal, block_mask, mask_block)
            out[b, h] = np.where(keep, ds, 0.0).max(1)
    return out
