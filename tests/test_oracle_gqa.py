"""Pins of the grouped-head oracle (oracle/gqa.py): it reduces to the plain
oracle (itself pinned in test_oracle.py) when every query head has its own
key/value head, equals the plain oracle on copied key/value heads with the
group's gradients summed, and its shared-head gradients match central finite
differences.  Planted mistakes in it (interleaved head mapping, gradient of a
shared head taken from one query head only) each fail a pin.
"""

import numpy as np
import pytest

import oracle
from oracle import gqa


def _draw(B, Hq, Hkv, N, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, Hq, N, d)))


def test_one_head_per_group_is_plain_attention():
    q, k, v, do = _draw(2, 3, 3, 7, 4, seed=1)
    g = gqa.forward_backward(q, k, v, do, 0.6, causal=True)
    p = oracle.forward_backward(q, k, v, do, 0.6, causal=True)
    for n in ("O", "LSE", "dQ", "dK", "dV"):
        np.testing.assert_array_equal(g[n], p[n])


@pytest.mark.parametrize("Hq,Hkv,causal,masked", [(8, 2, True, False), (6, 3, False, True),
                                                  (4, 1, True, True), (4, 4, False, False)])
def test_copied_heads_and_summed_gradients(Hq, Hkv, causal, masked):
    B, N, d = 2, 9, 5
    q, k, v, do = _draw(B, Hq, Hkv, N, d, seed=Hq + Hkv)
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], np.uint8) if masked else None
    g = gqa.forward_backward(q, k, v, do, 0.4, causal, mask, mask_block=4)
    G = Hq // Hkv
    p = oracle.forward_backward(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), do, 0.4,
                                causal, mask, mask_block=4)
    for n in ("O", "dQ"):
        np.testing.assert_allclose(g[n], p[n], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(g["LSE"]), np.isneginf(p["LSE"]))
    fin = np.isfinite(p["LSE"])
    np.testing.assert_allclose(g["LSE"][fin], p["LSE"][fin], rtol=0, atol=1e-12)
    for n in ("dK", "dV"):
        summed = p[n].reshape(B, Hkv, G, N, d).sum(axis=2)
        np.testing.assert_allclose(g[n], summed, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_shared_head_gradients_by_finite_differences(causal):
    B, Hq, Hkv, N, d = 1, 4, 2, 5, 3
    q, k, v, do = _draw(B, Hq, Hkv, N, d, seed=7)
    g = gqa.forward_backward(q, k, v, do, 0.8, causal)
    eps = 1e-6

    def loss(kk, vv):
        return float((gqa.forward_backward(q, kk, vv, do, 0.8, causal)["O"] * do).sum())

    for name, t in (("dK", k), ("dV", v)):
        num = np.zeros_like(t)
        for idx in np.ndindex(t.shape):
            tp, tm = t.copy(), t.copy()
            tp[idx] += eps
            tm[idx] -= eps
            args_p = (tp, v) if name == "dK" else (k, tp)
            args_m = (tm, v) if name == "dK" else (k, tm)
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=0, atol=1e-7)


def test_row_helpers_match_the_full_result():
    B, Hq, Hkv, N, d = 1, 6, 2, 40, 8
    q, k, v, do = _draw(B, Hq, Hkv, N, d, seed=9)
    full = gqa.forward_backward(q, k, v, do, 0.3, causal=True)
    rows = np.array([0, 7, 39])
    for h in (0, 4, 5):
        r = gqa.query_rows(q[0], k[0], v[0], do[0], 0.3, h, rows, causal=True)
        np.testing.assert_allclose(r["O"], full["O"][0, h, rows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["dQ"], full["dQ"][0, h, rows], rtol=0, atol=1e-12)
    for c in (0, 1):
        r = gqa.key_rows(q[0], k[0], v[0], do[0], 0.3, c, rows, causal=True)
        np.testing.assert_allclose(r["dK"], full["dK"][0, c, rows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["dV"], full["dV"][0, c, rows], rtol=0, atol=1e-12)


def test_planted_mistakes_fail(monkeypatch):
    B, Hq, Hkv, N, d = 1, 4, 2, 6, 3
    q, k, v, do = _draw(B, Hq, Hkv, N, d, seed=11)
    G = Hq // Hkv
    ref = oracle.forward_backward(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), do, 0.5)
    with monkeypatch.context() as mp:          # interleaved heads
        mp.setattr(gqa, "kv_head", lambda h, Hq_, Hkv_: h % Hkv_)
        g = gqa.forward_backward(q, k, v, do, 0.5)
        assert not np.allclose(g["O"], ref["O"], atol=1e-9)
    with monkeypatch.context() as mp:          # shared head keeps one query head's gradient
        def overwrite(grad, head, contribution):
            grad[head] = contribution
        mp.setattr(gqa, "_accumulate", overwrite)
        g = gqa.forward_backward(q, k, v, do, 0.5)
        summed = ref["dK"].reshape(B, Hkv, G, N, d).sum(axis=2)
        assert not np.allclose(g["dK"], summed, atol=1e-9)
        assert np.allclose(g["O"], ref["O"], atol=1e-12)
