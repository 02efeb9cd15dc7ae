"""Pins for the dropout oracle (oracle/dropout.py), CPU only.

The generator is pinned to the published Philox4x32-10 known-answer vectors;
the attention-with-dropout formulas to p = 0 (the plain oracle), finite
differences with the mask held fixed, unbiasedness over seeds and the
softmax-Jacobian identities; planted mistakes must fail a pin.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import dropout as od

HERE = os.path.dirname(os.path.abspath(__file__))


def _inputs(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)) for _ in range(4)]


def test_philox_known_answers():
    kat = json.load(open(os.path.join(HERE, "golden", "philox4x32_10_kat.json")))
    for vec in kat["vectors"]:
        ctr = tuple(np.array([int(c, 16)], dtype=np.uint64) for c in vec["ctr"])
        key = tuple(int(k, 16) for k in vec["key"])
        out = od.philox4x32(ctr, key)
        assert ["%08x" % int(o[0]) for o in out] == vec["out"]


def test_philox_round_count_matters():
    ctr = tuple(np.array([0], dtype=np.uint64) for _ in range(4))
    assert od.philox4x32(ctr, (0, 0), rounds=7) != od.philox4x32(ctr, (0, 0), rounds=10)


def test_threshold_and_keep_fraction():
    assert od.threshold(0.0) == 0
    assert od.threshold(0.5) == 2 ** 15
    assert od.threshold(0.1) == 6553                    # floor(0.1 * 65536)
    assert od.threshold(1.0 - 2.0 ** -20) == 2 ** 16 - 1
    with pytest.raises(ValueError):
        od.threshold(1.0)
    n = 512
    z = od.keep_mask(3, np.arange(n), np.arange(n), 0.3, seed=12345)
    frac = z.mean()
    sigma = math.sqrt(0.3 * 0.7 / z.size)
    assert abs(frac - 0.7) < 5 * sigma
    # rows, columns and the 4-word grouping are not correlated in an obvious way
    assert abs(z[:, 0::4].mean() - z[:, 3::4].mean()) < 10 * sigma * 2
    assert abs(z[0::2].mean() - z[1::2].mean()) < 10 * sigma * 2


def test_keep_mask_element_by_element():
    """Each element against a scalar evaluation of its definition: one
    Philox call per (j // 4, i // 2), word j mod 4, low half for even i,
    high half for odd i."""
    seed, bh, p = 0xDEAD_BEEF_0123, 2, 0.45
    t = od.threshold(p)
    rows, cols = np.arange(6, 11), np.arange(13, 22)
    z = od.keep_mask(bh, rows, cols, p, seed)
    for a, i in enumerate(rows):
        for b, j in enumerate(cols):
            ctr = tuple(np.array([c], dtype=np.uint64) for c in (j // 4, i // 2, bh, 0))
            words = od.philox4x32(ctr, (seed % 2 ** 32, seed // 2 ** 32))
            word = int(words[j % 4][0])
            half = word & 0xFFFF if i % 2 == 0 else word >> 16
            assert z[a, b] == (half >= t), (i, j)


def test_keep_mask_structure():
    rows, cols = np.arange(64), np.arange(96)
    a = od.keep_mask(0, rows, cols, 0.4, seed=7)
    # a sub-block evaluates to the same values as the full matrix
    assert np.array_equal(od.keep_mask(0, rows[10:20], cols[33:70], 0.4, seed=7), a[10:20, 33:70])
    # other head, other seed, other seed word: different masks
    assert not np.array_equal(a, od.keep_mask(1, rows, cols, 0.4, seed=7))
    assert not np.array_equal(a, od.keep_mask(0, rows, cols, 0.4, seed=8))
    assert not np.array_equal(a, od.keep_mask(0, rows, cols, 0.4, seed=7 + (1 << 32)))
    # a larger p drops a superset (same random words, higher threshold)
    b = od.keep_mask(0, rows, cols, 0.6, seed=7)
    assert np.all(b <= a)
    assert np.all(od.keep_mask(0, rows, cols, 0.0, seed=7))


def test_head_outputs_match_whole_tensor():
    """The one-head helper (full-size checks of a few heads) gives each head
    exactly what the whole-tensor routine gives it, mask index included."""
    q, k, v, do = _inputs(2, 3, 20, 4, 8)
    a = od.forward_backward(q, k, v, do, 0.5, 0.3, 77, causal=True)
    for b, h in ((0, 0), (1, 2), (0, 2)):
        r = od.head_outputs(q, k, v, do, 0.5, 0.3, 77, b, h, causal=True)
        for name in ("O", "LSE", "dQ", "dK", "dV"):
            assert np.array_equal(r[name], a[name][b, h]), (name, b, h)


@pytest.mark.parametrize("causal,use_mask", [(False, False), (True, False), (True, True)])
def test_p_zero_is_plain_attention(causal, use_mask):
    q, k, v, do = _inputs(1, 2, 48, 8, 1)
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8) if use_mask else None
    a = od.forward_backward(q, k, v, do, 0.4, 0.0, 99, causal, mask, mask_block=16)
    b = oracle.forward_backward(q, k, v, do, 0.4, causal, mask, mask_block=16)
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        np.testing.assert_allclose(a[name], b[name], rtol=0, atol=1e-13, err_msg=name)


def test_lse_unchanged_and_dk_sums_to_zero():
    q, k, v, do = _inputs(1, 2, 40, 8, 2)
    a = od.forward_backward(q, k, v, do, 0.35, 0.25, 5, causal=True)
    b = oracle.forward_backward(q, k, v, do, 0.35, causal=True)
    np.testing.assert_allclose(a["LSE"], b["LSE"], atol=1e-13)
    np.testing.assert_allclose(a["dK"].sum(axis=2), 0.0, atol=1e-11)


def _loss(q, k, v, do, scale, p, seed, causal):
    return float((od.forward_backward(q, k, v, do, scale, p, seed, causal)["O"] * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences_with_fixed_mask(causal):
    q, k, v, do = _inputs(1, 1, 7, 3, 3)
    scale, p, seed, h = 0.6, 0.3, 11, 1e-6
    g = od.forward_backward(q, k, v, do, scale, p, seed, causal)
    for name, x in (("dQ", q), ("dK", k), ("dV", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"dQ": (xp, k, v), "dK": (q, xp, v), "dV": (q, k, xp)}[name]
            argm = {"dQ": (xm, k, v), "dK": (q, xm, v), "dV": (q, k, xm)}[name]
            num[idx] = (_loss(*args, do, scale, p, seed, causal) -
                        _loss(*argm, do, scale, p, seed, causal)) / (2 * h)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_unbiased_over_seeds():
    q, k, v, do = _inputs(1, 1, 12, 4, 4)
    plain = oracle.forward(q, k, v, 0.5)[0]
    p, n = 0.3, 400
    acc = np.zeros_like(plain)
    sq = np.zeros_like(plain)
    for s in range(n):
        o = od.forward_backward(q, k, v, do, 0.5, p, 1000 + s)["O"]
        acc += o
        sq += o * o
    mean = acc / n
    std = np.sqrt(np.maximum(sq / n - mean ** 2, 1e-30))
    assert np.all(np.abs(mean - plain) < 6 * std / math.sqrt(n) + 1e-12)


def test_planted_mistakes_fail():
    """Two wrong backwards (no 1/(1-p) on dV; the dropped P in dS) and a
    wrong forward (no rescale) each fail a pin above."""
    q, k, v, do = _inputs(1, 1, 7, 3, 5)
    scale, p, seed = 0.6, 0.3, 13
    g = od.forward_backward(q, k, v, do, scale, p, seed)
    idx = np.arange(7)
    z = od.keep_mask(0, idx, idx, p, seed)
    s = scale * q[0, 0] @ k[0, 0].T
    pr = np.exp(s - s.max(1, keepdims=True))
    pr /= pr.sum(1, keepdims=True)
    # (1) dV without the 1/(1-p) factor
    assert not np.allclose((pr * z).T @ do[0, 0], g["dV"][0, 0], atol=1e-6)
    # (2) dS built from the dropped probabilities
    m = z / (1 - p)
    o = (pr * m) @ v[0, 0]
    dp = (do[0, 0] @ v[0, 0].T) * m
    ds_wrong = (pr * m) * (dp - (do[0, 0] * o).sum(1)[:, None])
    assert not np.allclose(scale * ds_wrong @ k[0, 0], g["dQ"][0, 0], atol=1e-6)
    # (3) forward without the rescale is biased: differs from the unbiased O
    assert not np.allclose((pr * z) @ v[0, 0], g["O"][0, 0], atol=1e-6)
