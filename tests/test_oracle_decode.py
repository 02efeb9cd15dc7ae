"""Pins of the decode oracle (oracle/decode.py) against facts fixed outside it:
the training oracle (itself pinned in test_oracle.py) on the cases the decode
definition reduces to, a library softmax, scalar brute force, closed forms,
and the pages' two-part merge rule ([FA-guide] "Artımsal Softmax Takibi").
Planted mistakes in the oracle (head mapping, causal alignment, ignored
lengths) each fail one of these pins.
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import attention as A
from oracle import decode as OD
from oracle import online


def _draw(B, Hq, Hkv, Nq, Nkv, d, seed, sigma=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, d)) * sigma
    k = rng.standard_normal((B, Hkv, Nkv, d)) * sigma
    v = rng.standard_normal((B, Hkv, Nkv, d)) * sigma
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
def test_mha_full_length_is_training_forward(causal):
    """G = 1 and L = Nq = Nkv: decode is the training forward (end-aligned
    causal equals the training causal mask when L = Nq)."""
    q, k, v = _draw(2, 3, 3, 9, 9, 5, seed=1)
    o, lse = OD.decode_forward(q, k, v, 0.4, causal=causal)
    o_ref, lse_ref = A.forward(q, k, v, 0.4, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def _rows_reference(q, k, v, scale, lens, causal):
    """Each (b, h) through the training oracle's row evaluation: the Nq new
    queries placed at positions L-Nq .. L-1 of an L-row sequence whose cache
    is the first L rows of the query head's cache head."""
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.zeros(q.shape)
    lse = np.full(q.shape[:3], -np.inf)
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            kc, vc = k[b, h // G, :L], v[b, h // G, :L]
            for i in range(Nq):
                pos = L - Nq + i                       # position of new token i
                if causal:
                    if pos < 0:
                        continue                       # sees no key
                    rows_q = np.zeros((L, d))
                    rows_q[pos] = q[b, h, i]
                    oi, li = A.forward_rows(rows_q, kc, vc, scale, [pos], causal=True)
                else:
                    if L == 0:
                        continue
                    oi, li = A.forward_rows(q[b, h, i][None], kc, vc, scale, [0], causal=False)
                o[b, h, i], lse[b, h, i] = oi[0], li[0]
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_lengths_against_training_rows(causal):
    """Grouped heads, ragged lengths (including 0 and lengths below Nq):
    every row equals the training oracle's row evaluation."""
    B, Hq, Hkv, Nq, Nkv, d = 5, 6, 2, 3, 11, 4
    q, k, v = _draw(B, Hq, Hkv, Nq, Nkv, d, seed=2)
    lens = np.array([11, 7, 0, 2, 1])
    o, lse = OD.decode_forward(q, k, v, 0.7, seqlens=lens, causal=causal)
    o_ref, lse_ref = _rows_reference(q, k, v, 0.7, lens, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lse_ref))
    fin = np.isfinite(lse_ref)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_copied_cache_heads():
    """Sharing a cache head among G query heads is the same as giving each
    query head its own copy (numpy's repeat lays the copies out h // G)."""
    B, Hq, Hkv, Nq, Nkv, d = 2, 8, 2, 2, 13, 6
    q, k, v = _draw(B, Hq, Hkv, Nq, Nkv, d, seed=3)
    lens = np.array([13, 5])
    for causal in (False, True):
        o, lse = OD.decode_forward(q, k, v, 0.3, lens, causal)
        o2, lse2 = OD.decode_forward(q, np.repeat(k, Hq // Hkv, axis=1),
                                     np.repeat(v, Hq // Hkv, axis=1), 0.3, lens, causal)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, lse2)


def test_library_softmax():
    """One row against scipy's softmax and logsumexp."""
    q, k, v = _draw(1, 4, 1, 1, 50, 8, seed=4)
    o, lse = OD.decode_forward(q, k, v, 0.25, seqlens=[37])
    for h in range(4):
        s = 0.25 * k[0, 0, :37] @ q[0, h, 0]
        np.testing.assert_allclose(o[0, h, 0], scipy.special.softmax(s) @ v[0, 0, :37],
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h, 0], scipy.special.logsumexp(s), rtol=0, atol=1e-12)


def test_brute_force_scalar_loops():
    """Tiny case, causal, ragged: every output by scalar loops and math.exp."""
    B, Hq, Hkv, Nq, Nkv, d = 2, 4, 2, 3, 6, 3
    q, k, v = _draw(B, Hq, Hkv, Nq, Nkv, d, seed=5)
    lens = [6, 4]
    o, lse = OD.decode_forward(q, k, v, 0.9, lens, causal=True)
    for b in range(B):
        L = lens[b]
        for h in range(Hq):
            c = h // 2
            for i in range(Nq):
                keys = [j for j in range(L) if j <= L - Nq + i]
                sc = [0.9 * sum(q[b, h, i, x] * k[b, c, j, x] for x in range(d)) for j in keys]
                mx = max(sc)
                den = sum(math.exp(t - mx) for t in sc)
                for x in range(d):
                    num = sum(math.exp(t - mx) * v[b, c, j, x] for t, j in zip(sc, keys))
                    assert abs(o[b, h, i, x] - num / den) < 1e-12
                assert abs(lse[b, h, i] - (mx + math.log(den))) < 1e-12


def test_closed_forms():
    q, k, v = _draw(3, 2, 1, 2, 9, 4, seed=6)
    # L = 0: nothing visible
    o, lse = OD.decode_forward(q, k, v, 0.5, seqlens=[0, 1, 9])
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    # L = 1 (not causal): the one key's value row, LSE = its score
    for h in range(2):
        for i in range(2):
            np.testing.assert_allclose(o[1, h, i], v[1, 0, 0], rtol=0, atol=1e-15)
            assert abs(lse[1, h, i] - 0.5 * q[1, h, i] @ k[1, 0, 0]) < 1e-12
    # scale = 0: uniform weights over the visible keys
    o, lse = OD.decode_forward(q, k, v, 0.0, seqlens=[9, 4, 3], causal=True)
    for b, L in enumerate([9, 4, 3]):
        for i in range(2):
            n = L - 2 + i + 1
            np.testing.assert_allclose(o[b, :, i], np.broadcast_to(v[b, 0, :n].mean(0), (2, 4)),
                                       rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, :, i], math.log(n), rtol=0, atol=1e-12)
    # causal with L < Nq: the first Nq - L rows see nothing
    q5, k5, v5 = _draw(1, 1, 1, 4, 6, 3, seed=7)
    o, lse = OD.decode_forward(q5, k5, v5, 0.5, seqlens=[2], causal=True)
    assert np.all(np.isneginf(lse[0, 0, :2])) and np.all(o[0, 0, :2] == 0)
    assert np.all(np.isfinite(lse[0, 0, 2:]))
    np.testing.assert_allclose(o[0, 0, 2], v5[0, 0, 0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", [8, 9, 10])
def test_split_merge_rule(seed):
    """Keys cut into two chunks, each attended separately and merged with the
    pages' two-part rule, give the whole (what a split-KV kernel relies on)."""
    rng = np.random.default_rng(seed)
    q, k, v = _draw(1, 4, 2, 1, 40, 8, seed=seed)
    cut = int(rng.integers(1, 40))
    o, lse = OD.decode_forward(q, k, v, 0.35)
    o1, l1 = OD.decode_forward(q, k[:, :, :cut], v[:, :, :cut], 0.35)
    o2, l2 = OD.decode_forward(q, k[:, :, cut:], v[:, :, cut:], 0.35)
    m, l = online.merge_stats(l1, np.ones_like(l1), l2, np.ones_like(l2))
    w1, w2 = np.exp(l1 - m) / l, np.exp(l2 - m) / l
    np.testing.assert_allclose(w1[..., None] * o1 + w2[..., None] * o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m + np.log(l), lse, rtol=0, atol=1e-12)


def test_planted_mistakes_fail(monkeypatch):
    """Wrong variants planted in the oracle each fail a pin above."""
    B, Hq, Hkv, Nq, Nkv, d = 3, 6, 2, 3, 11, 4
    q, k, v = _draw(B, Hq, Hkv, Nq, Nkv, d, seed=11)
    lens = np.array([11, 8, 5])
    ref = _rows_reference(q, k, v, 0.7, lens, True)

    def differs():
        o, _ = OD.decode_forward(q, k, v, 0.7, seqlens=lens, causal=True)
        return not np.allclose(o, ref[0], atol=1e-9)

    assert not differs()
    with monkeypatch.context() as mp:          # interleaved instead of grouped heads
        mp.setattr(OD, "kv_head", lambda h, Hq_, Hkv_: h % Hkv_)
        assert differs()
    with monkeypatch.context() as mp:          # causal mask aligned to the start
        mp.setattr(OD, "visible_keys",
                   lambda L, n, c: np.arange(L)[None, :] <= np.arange(n)[:, None])
        assert differs()
    with monkeypatch.context() as mp:          # lengths ignored
        real = OD.decode_forward
        mp.setattr(OD, "decode_forward",
                   lambda q_, k_, v_, s_, seqlens=None, causal=False: real(q_, k_, v_, s_, None,
                                                                            causal))
        assert differs()
