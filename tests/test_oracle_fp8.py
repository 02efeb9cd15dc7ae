"""Pins of the FP8 oracle (oracle/fp8.py): the E4M3 code table against values
the OCP 8-bit floating point specification fixes, rounding against brute-force
nearest search, block quantization within its half-ulp bound, the exact
attention on dequantized inputs against the plain oracle, and the stated
probability-rounding bound against a direct emulation of the rounding.
Planted mistakes in the encoder (truncation, ties away from zero, the E4M3
bias of the FNUZ variant) each fail a pin.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import fp8


def test_code_table_fixed_points():
    d = fp8.decode
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert d(0x38) == 1.0 and d(0xB8) == -1.0
    assert d(0x01) == 2.0 ** -9           # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9       # largest subnormal
    assert d(0x08) == 2.0 ** -6           # smallest normal
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    assert d(0x40) == 2.0 and d(0x3C) == 1.5 and d(0x30) == 0.5
    vals = d(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0)      # positive codes ordered by value
    assert len(np.unique(vals)) == 127


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    np.testing.assert_array_equal(fp8.encode(fp8.decode(codes)), codes)


def test_rounding_is_nearest_with_ties_to_even():
    e = fp8.encode
    assert e(1.0 + 1 / 16) == 0x38        # tie between 1.0 and 1.125 -> even (1.0)
    assert e(1.0 + 3 / 16) == 0x3A        # tie between 1.125 and 1.25 -> even (1.25)
    assert e(1.0 + 1 / 16 + 1e-9) == 0x39
    assert e(0.96875) == 0x38             # tie across a binade -> 1.0
    assert e(2.0 ** -10) == 0x00          # half the smallest subnormal: tie to 0
    assert e(1.5 * 2.0 ** -9) == 0x02     # tie between 1 and 2 subnormal steps -> even
    assert e(1000.0) == 0x7E and e(-1e9) == 0xFE and e(464.0) == 0x7E
    assert e(float("nan")) == 0x7F


def test_rounding_matches_brute_force_nearest():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.uniform(-4, 2.6, 4000),
                        rng.uniform(-460, 460, 1000)])
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    vals = fp8.decode(codes)
    got = fp8.encode(x)
    for xi, gi in zip(x, got):
        xs = min(max(xi, -448.0), 448.0)
        err = np.abs(vals - xs)
        best = err.min()
        cands = codes[err == best]
        assert abs(fp8.decode(gi) - xs) == best
        if len(cands) > 1 and best > 0:   # a tie: the even mantissa wins
            assert gi & 1 == 0


def test_block_quantization_within_half_ulp():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 300, 16)) * 3.0
    x[0, 1, 128:256] = 0.0                # an all-zero block
    codes, s = fp8.quantize_rows(x)
    assert s.shape == (2, 3, 3) and s[0, 1, 1] == 1.0
    back = fp8.decode(codes) * s.astype(np.float64)[:, :, np.arange(300) // 128, None]
    y = np.abs(x / s.astype(np.float64)[:, :, np.arange(300) // 128, None])
    bound = np.where(y >= 2.0 ** -6, 2.0 ** -4 * y, 2.0 ** -10) * s.astype(np.float64)[:, :, np.arange(300) // 128, None]
    assert np.all(np.abs(back - x) <= bound * (1 + 1e-12))
    # every block uses its full range: its largest magnitude encodes to +-448
    assert np.abs(fp8.decode(codes[0, 0, :128])).max() == 448.0


def test_forward_is_plain_attention_on_dequantized_values():
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((1, 2, 200, 8)) for _ in range(3))
    q8, sq = fp8.quantize_rows(q)
    k8, sk = fp8.quantize_rows(k)
    vt8, sv = fp8.quantize_heads_transposed(v)
    assert vt8.shape == (1, 2, 8, 200)
    qd, kd, vd = fp8.dequantize(q8, k8, vt8, sq, sk, sv)
    o, lse = fp8.forward(q8, k8, vt8, sq, sk, sv, 0.3, causal=True)
    o_ref, lse_ref = oracle.forward(qd, kd, vd, 0.3, True)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(lse, lse_ref)
    # and the dequantized values are close to the originals
    assert np.abs(vd - v).max() <= 2.0 ** -4 * np.abs(v).max() * 1.01


def _emulate_p_rounding(q8, k8, vt8, sq, sk, sv, scale, tile, shift=8):
    """O with the probabilities rounded to E4M3 as the GPU forms them: tiles of
    `tile` keys, running max m, P~ = 2^(shift + s log2 e - m), rescale on a
    new max, divide by the sum of the unrounded P~."""
    q, k, v = fp8.dequantize(q8, k8, vt8, sq, sk, sv)
    B, H, N, d = q.shape
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            s = scale * q[b, h] @ k[b, h].T * math.log2(math.e)
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, d))
            for j0 in range(0, N, tile):
                st = s[:, j0:j0 + tile]
                m_new = np.maximum(m, st.max(axis=1))
                alpha = np.where(np.isfinite(m), np.exp2(m - m_new), 0.0)
                pt = np.exp2(shift + st - m_new[:, None])
                acc = acc * alpha[:, None] + fp8.decode(fp8.encode(pt)) @ v[b, h, j0:j0 + tile]
                l = l * alpha + pt.sum(axis=1)
                m = m_new
            out[b, h] = acc / l[:, None]
    return out


def test_probability_rounding_bound_holds():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 2, 256, 16)) for _ in range(3))
    k[0, 0, 17] *= 20.0                   # a large-logit key
    q8, sq = fp8.quantize_rows(q)
    k8, sk = fp8.quantize_rows(k)
    vt8, sv = fp8.quantize_heads_transposed(v)
    o, _ = fp8.forward(q8, k8, vt8, sq, sk, sv, 0.25)
    bound = fp8.o_error_bound(q8, k8, vt8, sq, sk, sv, 0.25)
    for tile in (16, 64, 256):
        emu = _emulate_p_rounding(q8, k8, vt8, sq, sk, sv, 0.25, tile)
        err = np.abs(emu - o)
        assert np.all(err <= bound), (tile, float((err / bound).max()))
        assert err.max() > 0                # the rounding is visible
    # without the shift the subnormal term grows 256-fold
    b0 = fp8.o_error_bound(q8, k8, vt8, sq, sk, sv, 0.25, shift=0)
    assert np.all(b0 >= bound)


def test_planted_mistakes_fail(monkeypatch):
    x = np.array([1.0 + 1 / 16, 1.0 + 3 / 16, 0.3, -2.7, 100.0])
    good = fp8.encode(x)
    # truncation instead of rounding
    trunc = np.array([fp8._POS_CODES[np.searchsorted(fp8._POS_VALUES, abs(t), side="right") - 1]
                      | (0x80 if t < 0 else 0) for t in x], dtype=np.uint8)
    assert not np.array_equal(trunc, good)
    # a decoder with the bias of the FNUZ variant (8) disagrees with the fixed points
    with monkeypatch.context() as mp:
        real = fp8.decode
        mp.setattr(fp8, "decode", lambda c: real(c) / 2.0)
        with pytest.raises(AssertionError):
            test_code_table_fixed_points()
    # ties away from zero break the tie pin
    with monkeypatch.context() as mp:
        mp.setattr(fp8, "encode", lambda v: np.where(np.asarray(v) == 1.0 + 1 / 16, 0x39,
                                                       good[0]).astype(np.uint8))
        with pytest.raises(AssertionError):
            test_rounding_is_nearest_with_ties_to_even()


@pytest.mark.parametrize("shift", [8, 0, 3])
def test_head_rows_equals_rows_of_the_full_results(shift):
    """The row helper used by the full-size FP8 check is the full forward and
    the full bound restricted to the sampled rows: masked, causal, several
    heads, a large-logit key and a zero key block, every shift."""
    rng = np.random.default_rng(5)
    B, H, N, d, blk = 2, 3, 96, 16, 32
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    k[1, 2, 40] *= 20.0
    k[0, 1, 64:96] = 0.0
    q8, sq = fp8.quantize_rows(q, blk)
    k8, sk = fp8.quantize_rows(k, blk)
    vt8, sv = fp8.quantize_heads_transposed(v)
    mask = np.array([[1, 0, 0], [1, 1, 0], [0, 1, 1]], np.uint8)
    o, lse = fp8.forward(q8, k8, vt8, sq, sk, sv, 0.4, True, mask, blk)
    bound = fp8.o_error_bound(q8, k8, vt8, sq, sk, sv, 0.4, True, mask, blk, shift=shift)
    rows = np.array([0, 5, 31, 32, 50, 95])
    for b in range(B):
        for h in range(H):
            r = fp8.head_rows(q8, k8, vt8, sq, sk, sv, b, h, rows, 0.4, True, mask, blk,
                              shift=shift)
            np.testing.assert_allclose(r["O"], o[b, h, rows], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(r["LSE"], lse[b, h, rows], rtol=1e-13)
            np.testing.assert_allclose(r["bound"], bound[b, h, rows], rtol=1e-13, atol=0)


def test_head_rows_subnormal_term_follows_shift():
    """A planted fixed subnormal term (the shift-8 value at shift 0) breaks
    the equality with o_error_bound."""
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((1, 1, 64, 16)) for _ in range(3))
    q8, sq = fp8.quantize_rows(q)
    k8, sk = fp8.quantize_rows(k)
    vt8, sv = fp8.quantize_heads_transposed(v)
    rows = np.arange(64)
    full0 = fp8.o_error_bound(q8, k8, vt8, sq, sk, sv, 0.3, True, shift=0)[0, 0]
    good = fp8.head_rows(q8, k8, vt8, sq, sk, sv, 0, 0, rows, 0.3, True, shift=0)["bound"]
    wrong = fp8.head_rows(q8, k8, vt8, sq, sk, sv, 0, 0, rows, 0.3, True, shift=8)["bound"]
    np.testing.assert_allclose(good, full0, rtol=1e-13)
    assert not np.allclose(wrong, full0, rtol=1e-6)


def _lse_with_instruction_errors(q8, k8, sq, sk, scale, causal, sign, units=fp8.MFMA_UNITS,
                                 window=fp8.MFMA_WINDOW):
    """LSE from scores formed instruction by instruction, each instruction's
    result pushed by sign * units * 2^(E - window) (the model's extreme),
    written out with loops over rows, keys and 64-wide groups."""
    a, b = fp8.decode(q8), fp8.decode(k8)
    B, H, N, d = a.shape
    lse = np.empty((B, H, N))
    for bb in range(B):
        for h in range(H):
            for i in range(N):
                s = np.full(N, -np.inf)
                for j in range(N):
                    if causal and j > i:
                        continue
                    c = 0.0
                    for g0 in range(0, d, 64):
                        p = a[bb, h, i, g0:g0 + 64] * b[bb, h, j, g0:g0 + 64]
                        m = max(abs(c), float(np.abs(p).max()))
                        e = 2.0 ** (math.floor(math.log2(m)) - window) if m > 0 else 0.0
                        c = c + float(p.sum()) + sign * units * e
                    s[j] = scale * float(sq[bb, h, i // 128]) * float(sk[bb, h, j // 128]) * c
                mx = s.max()
                lse[bb, h, i] = mx + math.log(np.exp(s - mx).sum())
    return lse


@pytest.mark.parametrize("d,causal,scale", [(64, False, 0.3), (128, True, -0.2)])
def test_lse_allowance_covers_the_instruction_model(d, causal, scale):
    """Scores pushed to the model's extreme in either direction move LSE by
    at most the allowance (equality when every kept score moves by the same
    amount), on inputs with a large-logit key; a narrower window (a planted
    mistake) gives an allowance the same extreme exceeds."""
    rng = np.random.default_rng(8)
    q, k = (rng.standard_normal((1, 2, 20, d)) for _ in range(2))
    k[0, 1, 3] *= 20.0
    q8, sq = fp8.quantize_rows(q)
    k8, sk = fp8.quantize_rows(k)
    _, lse = fp8.forward(q8, k8, fp8.quantize_heads_transposed(q)[0], sq, sk,
                         np.ones((1, 2), np.float32), scale, causal)
    allow = fp8.lse_allowance(q8, k8, sq, sk, scale, causal)
    assert np.all(allow > 0)
    worst = 0.0
    for sign in (1.0, -1.0):
        moved = _lse_with_instruction_errors(q8, k8, sq, sk, scale, causal, sign)
        dl = np.abs(moved - lse)
        assert np.all(dl <= allow * (1 + 1e-9) + 1e-12)
        worst = max(worst, float((dl / allow).max()))
    assert worst > 0.3                     # the allowance is not vacuous
    narrow = fp8.lse_allowance(q8, k8, sq, sk, scale, causal, window=fp8.MFMA_WINDOW + 4)
    moved = _lse_with_instruction_errors(q8, k8, sq, sk, scale, causal, 1.0)
    assert np.any(np.abs(moved - lse) > narrow * (1 + 1e-9))


def test_lse_allowance_zero_codes_and_masked_rows():
    q8 = np.zeros((1, 1, 8, 64), np.uint8)
    k8 = fp8.encode(np.random.default_rng(9).standard_normal((1, 1, 8, 64)))
    ones = np.ones((1, 1, 1), np.float32)
    assert np.all(fp8.lse_allowance(q8, k8, ones, ones, 0.5) == 0.0)   # all products zero
    mask = np.zeros((1, 1), np.uint8)                                  # nothing kept
    q8 = fp8.encode(np.ones((1, 1, 8, 64)))
    assert np.all(fp8.lse_allowance(q8, k8, ones, ones, 0.5, block_mask=mask) == 0.0)
