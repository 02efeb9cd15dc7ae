"""Pins of the CPU fp64 oracle against facts that do not come from the oracle.

Each test checks the oracle against something fixed independently of it: a
hand-derived worked example, closed forms, a library softmax, scalar
brute force, finite differences, the pages' two-part merge rule, the
block-size invariance of the incremental softmax, and gradient identities.
Pages: [Training-FA] aivaro.ru/en/answers/474; [Week-13]
snula.amonoc.com/course/ru/week-13.html; [FA-guide]
xyznot.com/tr/paper/2205.14135.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import attention as A
from oracle import online

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _qkvdo(B, H, N, d, seed, sigma=1.0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)) * sigma for _ in range(4)]


# --------------------------------------------------------------------------
# Worked example (hand-derived, tests/golden/two_token_worked.json)
# --------------------------------------------------------------------------

def _ev(x):
    return eval(x, {"__builtins__": {}}, {"ln": math.log})  # exact expressions


def _arr(rows):
    return np.array([[_ev(c) for c in r] for r in rows]) if isinstance(rows[0], list) \
        else np.array([_ev(c) for c in rows])


@pytest.mark.parametrize("case", ["dense", "causal"])
def test_worked_two_token_example(case):
    g = json.load(open(os.path.join(GOLDEN, "two_token_worked.json")))
    c = g["cases"][case]
    q, k, v, do = (_arr(g[n])[None, None] for n in ("Q", "K", "V", "dO"))
    r = oracle.forward_backward(q, k, v, do, g["scale"], causal=c["causal"])
    for name in ("O", "dQ", "dK", "dV"):
        np.testing.assert_allclose(r[name][0, 0], _arr(c[name]), atol=1e-15, rtol=1e-14,
                                   err_msg=name)
    np.testing.assert_allclose(r["LSE"][0, 0], _arr(c["LSE"]), atol=1e-15, rtol=1e-14)


# --------------------------------------------------------------------------
# Forward: library special case, scalar brute force, closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("use_mask", [False, True])
def test_forward_matches_scipy_softmax(causal, use_mask):
    q, k, v, _ = _qkvdo(1, 2, 37, 8, seed=3)
    scale = 0.37
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], np.uint8) if use_mask else None
    o, lse = oracle.forward(q, k, v, scale, causal, mask, mask_block=16)
    keep = oracle.keep_matrix(37, 37, causal, mask, mask_block=16)
    for h in range(2):
        s = scale * q[0, h] @ k[0, h].T
        s[~keep] = -np.inf
        p = scipy.special.softmax(s, axis=1)
        np.testing.assert_allclose(o[0, h], p @ v[0, h], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[0, h], scipy.special.logsumexp(s, axis=1),
                                   rtol=1e-13, atol=1e-13)


def test_forward_scalar_brute_force():
    """Pure-Python loops with math.exp on a tiny causal case."""
    q, k, v, _ = _qkvdo(1, 1, 4, 3, seed=11)
    scale = 0.8
    o, lse = oracle.forward(q, k, v, scale, causal=True)
    for i in range(4):
        logits = [scale * sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(3))
                  for j in range(i + 1)]
        w = [math.exp(x) for x in logits]
        z = sum(w)
        assert abs(lse[0, 0, i] - math.log(z)) < 1e-13
        for t in range(3):
            ref = sum(w[j] * v[0, 0, j, t] for j in range(i + 1)) / z
            assert abs(o[0, 0, i, t] - ref) < 1e-13


def test_probability_rows_sum_to_one():
    q, k, v, _ = _qkvdo(1, 1, 50, 16, seed=5)
    keep = oracle.keep_matrix(50, 50, True)
    p, _, _ = A._head_forward(q[0, 0], k[0, 0], v[0, 0], 0.25, keep)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(p[~keep] == 0.0)


@pytest.mark.parametrize("causal,use_mask", [(False, False), (True, False), (False, True),
                                             (True, True)])
def test_scale_zero_is_uniform_average(causal, use_mask):
    """scale = 0 gives uniform weights over the kept keys: O_i is the mean of
    the kept V_j, LSE_i = ln(#kept), dQ = dK = 0 and dV_j sums dO_i / #kept_i
    over the rows that keep j."""
    N, d = 12, 5
    q, k, v, do = _qkvdo(1, 1, N, d, seed=7)
    mask = np.array([[1, 0, 1], [0, 1, 1], [1, 1, 1]], np.uint8) if use_mask else None
    r = oracle.forward_backward(q, k, v, do, 0.0, causal, mask, mask_block=4)
    keep = oracle.keep_matrix(N, N, causal, mask, mask_block=4)
    cnt = keep.sum(axis=1)
    for i in range(N):
        np.testing.assert_allclose(r["O"][0, 0, i], v[0, 0][keep[i]].mean(axis=0), atol=1e-14)
        assert abs(r["LSE"][0, 0, i] - math.log(cnt[i])) < 1e-14
    assert np.abs(r["dQ"]).max() == 0.0 and np.abs(r["dK"]).max() == 0.0
    dv = np.zeros((N, d))
    for i in range(N):
        for j in range(N):
            if keep[i, j]:
                dv[j] += do[0, 0, i] / cnt[i]
    np.testing.assert_allclose(r["dV"][0, 0], dv, atol=1e-14)


def test_single_token():
    """N = 1: O = V, LSE = scale q.k, dQ = dK = 0, dV = dO."""
    q, k, v, do = _qkvdo(2, 3, 1, 8, seed=9)
    for causal in (False, True):
        r = oracle.forward_backward(q, k, v, do, 0.5, causal)
        np.testing.assert_allclose(r["O"], v, atol=1e-15)
        np.testing.assert_allclose(r["LSE"], 0.5 * (q * k).sum(-1), atol=1e-14)
        np.testing.assert_allclose(r["dQ"], 0.0, atol=1e-15)
        np.testing.assert_allclose(r["dK"], 0.0, atol=1e-15)
        np.testing.assert_allclose(r["dV"], do, atol=1e-15)


def test_causal_first_row_and_equal_keys():
    q, k, v, _ = _qkvdo(1, 1, 9, 4, seed=13)
    o, lse = oracle.forward(q, k, v, 1.0, causal=True)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert abs(lse[0, 0, 0] - (q[0, 0, 0] @ k[0, 0, 0])) < 1e-14
    k_eq = np.broadcast_to(k[:, :, :1], k.shape).copy()   # all keys equal
    o2, lse2 = oracle.forward(q, k_eq, v, 1.0, causal=False)
    np.testing.assert_allclose(o2[0, 0], np.broadcast_to(v[0, 0].mean(0), (9, 4)), atol=1e-14)
    np.testing.assert_allclose(lse2[0, 0], q[0, 0] @ k[0, 0, 0] + math.log(9), atol=1e-13)


# --------------------------------------------------------------------------
# Large logits and fully masked rows ([Week-13] "Типичные ошибки")
# --------------------------------------------------------------------------

@pytest.mark.parametrize("gain", [20.0, 1e4])
def test_large_logits_stay_finite(gain):
    q, k, v, do = _qkvdo(1, 1, 40, 16, seed=17)
    k[0, 0, [3, 11, 29]] *= gain
    r = oracle.forward_backward(q, k, v, do, 0.25, causal=False)
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.isfinite(r[name]).all(), name
    s = 0.25 * q[0, 0] @ k[0, 0].T
    np.testing.assert_allclose(r["LSE"][0, 0], scipy.special.logsumexp(s, axis=1),
                               rtol=1e-13)
    if gain == 1e4:
        # Gap between the top logit and the rest is huge: O_i is V_argmax.
        top = np.argmax(s, axis=1)
        srt = np.sort(s, axis=1)
        sure = srt[:, -1] - srt[:, -2] > 50
        assert sure.sum() > 20
        np.testing.assert_allclose(r["O"][0, 0][sure], v[0, 0][top[sure]], atol=1e-12)


def test_fully_masked_rows():
    """A mask that drops a diagonal tile leaves rows with no key: O = 0,
    LSE = -inf, dQ = 0, their dO has no effect on dK/dV, other rows as if the
    mask tile were not special."""
    N, d, mb = 12, 4, 4
    q, k, v, do = _qkvdo(1, 1, N, d, seed=19)
    mask = np.array([[1, 0, 0], [1, 0, 1], [1, 1, 1]], np.uint8)   # tile row 1 under causal: keys 0..3 only
    mask_empty = np.array([[1, 0, 0], [0, 0, 0], [1, 1, 1]], np.uint8)  # tile row 1 keeps nothing
    r = oracle.forward_backward(q, k, v, do, 0.5, True, mask_empty, mask_block=mb)
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        assert not np.isnan(r[name]).any()
    dead = slice(4, 8)
    assert np.all(r["O"][0, 0, dead] == 0.0)
    assert np.all(r["LSE"][0, 0, dead] == -np.inf)
    assert np.all(r["dQ"][0, 0, dead] == 0.0)
    do2 = do.copy()
    do2[0, 0, dead] = 123.0
    r2 = oracle.forward_backward(q, k, v, do2, 0.5, True, mask_empty, mask_block=mb)
    np.testing.assert_array_equal(r2["dK"], r["dK"])
    np.testing.assert_array_equal(r2["dV"], r["dV"])
    # The live rows equal those of a mask whose dead tile row keeps something.
    r3 = oracle.forward_backward(q, k, v, do, 0.5, True, mask, mask_block=mb)
    live = np.r_[0:4, 8:12]
    for name in ("O", "LSE", "dQ"):
        np.testing.assert_allclose(r[name][0, 0, live], r3[name][0, 0, live], atol=1e-14)


# --------------------------------------------------------------------------
# Two-part merge ([FA-guide] "Artımsal Softmax Takibi") and block-size
# invariance of the incremental forward ([FA-guide] "Yöntem" steps 1-4,
# [Week-13] Step 2)
# --------------------------------------------------------------------------

def test_merge_identity_random_cuts():
    rng = np.random.default_rng(23)
    for _ in range(200):
        n = int(rng.integers(2, 60))
        x = rng.standard_normal(n) * rng.choice([1.0, 10.0, 300.0])
        cut = int(rng.integers(1, n))
        a, b = x[:cut], x[cut:]
        m1, m2 = a.max(), b.max()
        l1, l2 = np.exp(a - m1).sum(), np.exp(b - m2).sum()
        m, l = online.merge_stats(m1, l1, m2, l2)
        assert m == x.max()
        assert abs(l - np.exp(x - x.max()).sum()) <= 1e-12 * l
        assert abs((m + math.log(l)) - scipy.special.logsumexp(x)) < 1e-12 * max(1, abs(m))


def test_merge_identity_with_empty_part():
    m, l = online.merge_stats(-np.inf, 0.0, 1.5, 2.0)
    assert m == 1.5 and l == 2.0
    m, l = online.merge_stats(-np.inf, 0.0, -np.inf, 0.0)
    assert m == -np.inf and l == 0.0 and not np.isnan(l)


@pytest.mark.parametrize("routine", ["rescaled", "deferred"])
@pytest.mark.parametrize("bc", [1, 7, 32, 48])
@pytest.mark.parametrize("causal,use_mask", [(False, False), (True, False), (False, True),
                                             (True, True)])
def test_block_size_does_not_matter(routine, bc, causal, use_mask):
    N, d = 48, 8
    q, k, v, _ = _qkvdo(1, 1, N, d, seed=29)
    k[0, 0, 5] *= 30.0     # a large logit so rescaling actually happens
    mask = (np.array([[1, 0, 1, 1], [1, 1, 0, 1], [0, 1, 1, 0], [1, 0, 1, 1]], np.uint8)
            if use_mask else None)
    o_ref, lse_ref = oracle.forward(q, k, v, 0.3, causal, mask, mask_block=12)
    fn = online.tiled_forward_rescaled if routine == "rescaled" else online.tiled_forward_deferred
    for br in (1, 5, 16, N):
        o, m, l = fn(q[0, 0], k[0, 0], v[0, 0], 0.3, br, bc, causal, mask, mask_block=12)
        np.testing.assert_allclose(o, o_ref[0, 0], atol=1e-12, rtol=1e-12)
        with np.errstate(divide="ignore"):
            lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1)), -np.inf)
        np.testing.assert_allclose(lse, lse_ref[0, 0], atol=1e-12, rtol=1e-12)


def test_online_routines_with_fully_masked_blocks_give_no_nan():
    N = 12
    q, k, v, _ = _qkvdo(1, 1, N, 4, seed=31)
    mask = np.array([[1, 0, 0], [0, 0, 0], [1, 1, 1]], np.uint8)
    o_ref, _ = oracle.forward(q, k, v, 1.0, True, mask, mask_block=4)
    for fn in (online.tiled_forward_rescaled, online.tiled_forward_deferred):
        o, m, l = fn(q[0, 0], k[0, 0], v[0, 0], 1.0, 4, 4, True, mask, mask_block=4)
        assert not np.isnan(o).any() and not np.isnan(l).any()
        np.testing.assert_allclose(o, o_ref[0, 0], atol=1e-13)


# --------------------------------------------------------------------------
# Backward: central finite differences and gradient identities
# --------------------------------------------------------------------------

def _loss(q, k, v, do, scale, causal, mask, mb):
    o, _ = oracle.forward(q, k, v, scale, causal, mask, mask_block=mb)
    return float((o * do).sum())


@pytest.mark.parametrize("scale", [0.7, -0.45])
@pytest.mark.parametrize("N,d", [(1, 3), (5, 3), (16, 8)])
@pytest.mark.parametrize("causal,use_mask", [(False, False), (True, False), (False, True),
                                             (True, True)])
def test_gradients_match_finite_differences(N, d, causal, use_mask, scale):
    q, k, v, do = _qkvdo(1, 1, N, d, seed=37 + N + d)
    mb = 4
    t = -(-N // mb)
    mask = None
    if use_mask:
        mask = (np.random.default_rng(41).random((t, t)) < 0.6).astype(np.uint8)
        mask[np.arange(t), np.arange(t)] = 1
    r = oracle.forward_backward(q, k, v, do, scale, causal, mask, mask_block=mb)
    h = 1e-6
    for name, x in (("dQ", q), ("dK", k), ("dV", v)):
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, causal, mask, mb)
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, causal, mask, mb)
            x[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        err = np.abs(g - r[name]).max()
        assert err <= 1e-6 * max(1.0, np.abs(r[name]).max()), (name, err)


def test_gradient_identities():
    q, k, v, do = _qkvdo(2, 2, 30, 8, seed=43)
    for causal in (False, True):
        r = oracle.forward_backward(q, k, v, do, 0.35, causal)
        # sum_j dS_ij = 0 for every row, hence sum_j dK_j = 0.
        np.testing.assert_allclose(r["dK"].sum(axis=2), 0.0, atol=1e-12)
        # Rows of P sum to 1, hence sum_j dV_j = sum_i dO_i.
        np.testing.assert_allclose(r["dV"].sum(axis=2), do.sum(axis=2), atol=1e-12)
        # V -> V + c shifts O by c and leaves dQ, dK unchanged.
        c = np.arange(8.0) * 0.1
        r2 = oracle.forward_backward(q, k, v + c, do, 0.35, causal)
        np.testing.assert_allclose(r2["O"], r["O"] + c, atol=1e-12)
        np.testing.assert_allclose(r2["dQ"], r["dQ"], atol=1e-12)
        np.testing.assert_allclose(r2["dK"], r["dK"], atol=1e-12)
    # K -> K + c (dense) adds q.c to every logit of a row: O unchanged.
    o1, _ = oracle.forward(q, k, v, 0.35, False)
    o2, _ = oracle.forward(q, k + 0.5, v, 0.35, False)
    np.testing.assert_allclose(o2, o1, atol=1e-12)


def test_negative_scale():
    """Any finite scale: a negative one weights the keys by exp of minus the
    dot product (scipy's softmax of the negated scores), and a large negative
    scale picks the key with the smallest score."""
    from scipy.special import logsumexp, softmax
    q, k, v, do = _qkvdo(1, 2, 12, 5, seed=53)
    o, lse = oracle.forward(q, k, v, -0.8, False)
    for h in range(2):
        s_ = -0.8 * q[0, h] @ k[0, h].T
        np.testing.assert_allclose(o[0, h], softmax(s_, axis=1) @ v[0, h], atol=1e-13)
        np.testing.assert_allclose(lse[0, h], logsumexp(s_, axis=1), atol=1e-13)
    o_big, _ = oracle.forward(q, k, v, -1e4, False)
    arg = np.argmin(q[0, 0] @ k[0, 0].T, axis=1)
    np.testing.assert_allclose(o_big[0, 0], v[0, 0][arg], atol=1e-9)
    # -scale with Q equals +scale with -Q (dQ changes sign)
    a = oracle.forward_backward(q, k, v, do, -0.8, True)
    b = oracle.forward_backward(-q, k, v, do, 0.8, True)
    for n in ("O", "LSE", "dK", "dV"):
        np.testing.assert_allclose(a[n], b[n], atol=1e-13)
    np.testing.assert_allclose(a["dQ"], -b["dQ"], atol=1e-13)


def test_scale_is_applied_to_scores():
    """scale * Q K^T: doubling the scale equals doubling Q."""
    q, k, v, do = _qkvdo(1, 1, 10, 4, seed=47)
    a = oracle.forward_backward(q, k, v, do, 0.6, True)
    b = oracle.forward_backward(2 * q, k, v, do, 0.3, True)
    np.testing.assert_allclose(a["O"], b["O"], atol=1e-13)
    np.testing.assert_allclose(a["dQ"], 2 * b["dQ"], atol=1e-12)
    np.testing.assert_allclose(a["dK"], b["dK"], atol=1e-12)


# --------------------------------------------------------------------------
# Row-restricted helpers equal the full evaluation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal,use_mask", [(False, False), (True, False), (False, True),
                                             (True, True)])
def test_row_helpers_equal_full(causal, use_mask):
    N, d = 40, 8
    q, k, v, do = _qkvdo(1, 1, N, d, seed=53)
    mask = None
    if use_mask:
        mask = np.array([[1, 0, 1, 0], [0, 1, 1, 1], [1, 0, 1, 0], [1, 1, 0, 0]], np.uint8)
    mb = 10
    full = oracle.forward_backward(q, k, v, do, 0.4, causal, mask, mask_block=mb)
    rows = np.array([0, 3, 17, 39])
    qr = oracle.query_rows(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.4, rows, causal, mask, mb)
    for name in ("O", "LSE", "dQ"):
        np.testing.assert_allclose(qr[name], full[name][0, 0, rows], atol=1e-13)
    o, lse = oracle.forward_rows(q[0, 0], k[0, 0], v[0, 0], 0.4, rows, causal, mask, mb)
    np.testing.assert_allclose(o, full["O"][0, 0, rows], atol=1e-13)
    cols = np.array([0, 9, 21, 39])
    kr = oracle.key_rows(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.4, cols, causal, mask, mb,
                         row_chunk=7)
    for name in ("dK", "dV"):
        np.testing.assert_allclose(kr[name], full[name][0, 0, cols], atol=1e-13)


def test_kept_pairs_counts():
    assert oracle.kept_pairs(1024, True) == 1024 * 1025 // 2
    assert oracle.kept_pairs(300, False) == 90000
    mask = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], np.uint8)
    # 300 keys: tiles of 128, 128, 44.
    sizes = [128, 128, 44]
    want = sum(sizes[a] * sizes[b] for a in range(3) for b in range(3) if mask[a, b])
    assert oracle.kept_pairs(300, False, mask) == want


# --------------------------------------------------------------------------
# Planted mistakes: each plausible slip in the backward must fail a pin above.
# (The mistake is planted in a copy of the oracle's arithmetic, on the CPU.)
# --------------------------------------------------------------------------

def _bad_backwards():
    def no_D(q, k, v, o, do, p, scale):
        dv = p.T @ do; dp = do @ v.T; ds = p * dp
        return scale * ds @ k, scale * ds.T @ q, dv

    def transposed_dk(q, k, v, o, do, p, scale):
        dv = p.T @ do; dp = do @ v.T; dvec = (do * o).sum(1); ds = p * (dp - dvec[:, None])
        return scale * ds @ k, scale * ds @ q, dv

    def sign_dq(q, k, v, o, do, p, scale):
        dv = p.T @ do; dp = do @ v.T; dvec = (do * o).sum(1); ds = p * (dp - dvec[:, None])
        return -scale * ds @ k, scale * ds.T @ q, dv

    def no_scale(q, k, v, o, do, p, scale):
        dv = p.T @ do; dp = do @ v.T; dvec = (do * o).sum(1); ds = p * (dp - dvec[:, None])
        return ds @ k, ds.T @ q, dv

    def dv_untransposed(q, k, v, o, do, p, scale):
        dv = p @ do; dp = do @ v.T; dvec = (do * o).sum(1); ds = p * (dp - dvec[:, None])
        return scale * ds @ k, scale * ds.T @ q, dv

    def no_p_factor(q, k, v, o, do, p, scale):
        dv = p.T @ do; dp = do @ v.T; dvec = (do * o).sum(1); ds = dp - dvec[:, None]
        return scale * ds @ k, scale * ds.T @ q, dv

    return [no_D, transposed_dk, sign_dq, no_scale, dv_untransposed, no_p_factor]


@pytest.mark.parametrize("bad", _bad_backwards(), ids=lambda f: f.__name__)
def test_planted_backward_mistakes_are_caught(bad, monkeypatch):
    monkeypatch.setattr(A, "_head_backward", bad)
    g = json.load(open(os.path.join(GOLDEN, "two_token_worked.json")))
    c = g["cases"]["dense"]
    q, k, v, do = (_arr(g[n])[None, None] for n in ("Q", "K", "V", "dO"))
    r = oracle.forward_backward(q, k, v, do, g["scale"], causal=False)
    golden_ok = all(np.allclose(r[n][0, 0], _arr(c[n]), atol=1e-12) for n in ("dQ", "dK", "dV"))
    # Finite differences on a small random case.
    qq, kk, vv, dd = _qkvdo(1, 1, 5, 3, seed=59)
    rr = oracle.forward_backward(qq, kk, vv, dd, 0.7, False)
    h = 1e-6
    fd_ok = True
    for name, x in (("dQ", qq), ("dK", kk), ("dV", vv)):
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(qq, kk, vv, dd, 0.7, False, None, 4)
            x[idx] = old - h
            lm = _loss(qq, kk, vv, dd, 0.7, False, None, 4)
            x[idx] = old
            if abs((lp - lm) / (2 * h) - rr[name][idx]) > 1e-6:
                fd_ok = False
    assert not (golden_ok and fd_ok)


def test_planted_forward_mistake_is_caught(monkeypatch):
    """Dropping the max subtraction overflows on large logits; forgetting the
    mask changes the causal worked example."""
    def no_mask(q, k, v, scale, keep):
        s = scale * (q @ k.T)
        p, _, lse = A._softmax_rows(s)
        return p, p @ v, lse
    monkeypatch.setattr(A, "_head_forward", no_mask)
    g = json.load(open(os.path.join(GOLDEN, "two_token_worked.json")))
    c = g["cases"]["causal"]
    q, k, v, do = (_arr(g[n])[None, None] for n in ("Q", "K", "V", "dO"))
    o, _ = oracle.forward(q, k, v, 1.0, causal=True)
    assert not np.allclose(o[0, 0], _arr(c["O"]))
