"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle on
the same seeded inputs, element by element.

Small cases run the full oracle and span several tiles plus a ragged tail;
the five workloads run at full size and are compared on sampled rows, plus
gradient identities that hold at any size.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_09_amd import fa
from io_aware_exact_09_amd import workloads as W
from gpu_util import run_hip, tol_check, upload, upload_mask, device

pytestmark = pytest.mark.gpu

OUTS = ("O", "LSE", "dQ", "dK", "dV")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def check_all(got, ref, dtype, label):
    for n in OUTS:
        if n in got:
            e = tol_check(n, got[n], ref[n], dtype)
            _say(f"  {label} {n}: " + " ".join(f"{k}={v:.3e}" for k, v in e.items()))


# --------------------------------------------------------------------------
# Small shapes: full oracle
# --------------------------------------------------------------------------

SMALL = [
    # (N, d, dtype, causal, mask-kind)
    (1, 64, "bf16", False, None), (1, 128, "fp32", True, None),
    (100, 64, "bf16", True, None), (100, 128, "fp32", False, None),
    (129, 64, "fp32", True, None), (129, 128, "bf16", False, None),
    (300, 64, "bf16", False, "rand"), (300, 128, "bf16", True, "rand"),
    (300, 64, "fp32", True, "rand"), (300, 128, "fp32", False, "rand"),
    (256, 64, "bf16", True, None), (256, 128, "bf16", True, None),
    (384, 128, "bf16", False, None), (384, 64, "fp32", False, None),
    (1000, 64, "bf16", True, "rand"), (1000, 128, "bf16", False, None),
    # bf16 d = 128 without a mask runs the ping-pong forward: ragged and tiny N
    (17, 128, "bf16", True, None), (300, 128, "bf16", True, None),
    (513, 128, "bf16", True, None), (200, 128, "bf16", False, None),
]


@pytest.mark.parametrize("N,d,dtype,causal,mk", SMALL,
                         ids=[f"N{a}-d{b}-{c}-{'causal' if e else 'dense'}-{f or 'nomask'}"
                              for a, b, c, e, f in SMALL])
def test_small_against_full_oracle(N, d, dtype, causal, mk):
    B, H = (1, 2) if N >= 1000 else (2, 3)
    inp = W.random_inputs(B, H, N, d, dtype, seed=N * 7 + d)
    mask = W.random_block_mask(N, 0.6, seed=N + d) if mk == "rand" else None
    scale = 1.0 / math.sqrt(d)
    _say(f"case N={N} d={d} {dtype} causal={causal} mask={mk}")
    got = run_hip(inp, dtype, scale, causal, mask)
    ref = oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, mask)
    check_all(got, ref, dtype, f"N={N}")


def test_fully_masked_rows():
    """A mask that drops a diagonal tile under causal masking leaves query
    rows with no key: O = 0, LSE = -inf, dQ = 0, nothing NaN."""
    N, d = 384, 64
    inp = W.random_inputs(1, 2, N, d, "bf16", seed=5)
    mask = np.array([[1, 0, 0], [0, 0, 1], [1, 1, 1]], np.uint8)   # tile row 1 keeps nothing causal
    got = run_hip(inp, "bf16", 0.125, True, mask)
    ref = oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["do"], 0.125, True, mask)
    assert np.all(got["O"][:, :, 128:256] == 0)
    assert np.all(np.isneginf(got["LSE"][:, :, 128:256]))
    assert np.all(got["dQ"][:, :, 128:256] == 0)
    check_all(got, ref, "bf16", "dead-rows")


def test_scale_zero_uniform():
    N, d = 200, 128
    inp = W.random_inputs(1, 1, N, d, "fp32", seed=9)
    got = run_hip(inp, "fp32", 0.0, True)
    ref = oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["do"], 0.0, True)
    check_all(got, ref, "fp32", "scale0")
    np.testing.assert_allclose(got["LSE"][0, 0], np.log(np.arange(1, N + 1)), atol=1e-5)


def _large_logit_inputs(dtype, frac=0.01):
    """Workload-like large logits: 1% of K rows x20 per head."""
    N, d = 512, 128
    inp = W.random_inputs(1, 2, N, d, "fp32", seed=13)
    rng = np.random.default_rng(14)
    rows = rng.choice(2 * N, size=int(frac * 2 * N), replace=False)
    inp["k"].reshape(2 * N, d)[rows] *= 20.0
    if dtype == "bf16":
        inp = {n: W.bf16_round(t) for n, t in inp.items()}
    return inp, 1 / math.sqrt(d)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_large_logits(dtype):
    """1% of K rows x20 (as in the long-context workload): the literal bar."""
    inp, scale = _large_logit_inputs(dtype)
    got = run_hip(inp, dtype, scale, True)
    ref = oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True)
    check_all(got, ref, dtype, "large-logits")


def _dq_floor_from_bf16_o(inp, scale, causal):
    """dQ error (rel-Frobenius) that storing O in bf16 alone causes: the
    backward's D = rowsum(dO * O) is formed from the stored O.  Test-side
    estimate: exact P and dP, D from the bf16-rounded exact O."""
    q, k, v, do = (np.asarray(inp[n], np.float64) for n in ("q", "k", "v", "do"))
    ref = oracle.forward_backward(q, k, v, do, scale, causal)
    N = q.shape[2]
    keep = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
    err = np.zeros_like(q)
    for h in range(q.shape[1]):
        s = np.where(keep, scale * q[0, h] @ k[0, h].T, -np.inf)
        p = np.exp(s - ref["LSE"][0, h][:, None])
        d_round = (do[0, h] * W.bf16_round(ref["O"][0, h].astype(np.float32))).sum(1)
        d_exact = (do[0, h] * ref["O"][0, h]).sum(1)
        err[0, h] = scale * (p * (d_exact - d_round)[:, None]) @ k[0, h]
    return float(np.linalg.norm(err) / np.linalg.norm(ref["dQ"])), ref


def test_large_logits_dq_tracks_bf16_storage_floor():
    """Few x20 keys per head (3 and 2 of 512): the rows that attend to them
    have dS terms that nearly cancel, and any backward that forms
    D = rowsum(dO * O) from a bf16 O inherits O's rounding there; on this
    input that floor alone is ~1e-2 rel-Frobenius in dQ.  The kernel's dQ
    error must stay within 25% of the floor; every other output meets the
    bar."""
    N, d = 512, 128
    inp = W.random_inputs(1, 2, N, d, "fp32", seed=13)
    inp["k"][0, 0, [3, 77, 300]] *= 20.0
    inp["k"][0, 1, [5, 400]] *= 20.0
    inp = {n: W.bf16_round(t) for n, t in inp.items()}
    scale = 1 / math.sqrt(d)
    floor, ref = _dq_floor_from_bf16_o(inp, scale, True)
    got = run_hip(inp, "bf16", scale, True)
    rel = float(np.linalg.norm(got["dQ"] - ref["dQ"]) / np.linalg.norm(ref["dQ"]))
    _say(f"  dQ rel-Frobenius {rel:.3e}, floor from bf16 O alone {floor:.3e}")
    assert rel <= 1.25 * floor + 1e-3
    for n in ("O", "LSE", "dK", "dV"):
        tol_check(n, got[n], ref[n], "bf16")


def test_extreme_logits_stay_finite():
    """One K row x1000 (logits in the thousands): every output finite and
    close to the oracle (fp32 scores of that size carry ~1e-3 absolute
    rounding, which moves P by ~1e-3 relative)."""
    N, d = 512, 128
    for dtype in ("fp32", "bf16"):
        inp = W.random_inputs(1, 2, N, d, "fp32", seed=17)
        inp["k"][0, 1, 11] *= 1000.0
        if dtype == "bf16":        # both sides get the same bf16 values
            inp = {n: W.bf16_round(t) for n, t in inp.items()}
        got = run_hip(inp, dtype, 1 / math.sqrt(d), True)
        ref = oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["do"], 1 / math.sqrt(d),
                                      True)
        for n in OUTS:
            assert np.isfinite(got[n]).all(), (dtype, n)
        for n in ("O", "dK", "dV"):
            rel = np.linalg.norm(got[n] - ref[n]) / np.linalg.norm(ref[n])
            assert rel <= 1e-2, (dtype, n, rel)
        lse_err = np.abs(got["LSE"] - ref["LSE"]) / np.maximum(1, np.abs(ref["LSE"]))
        assert lse_err.max() <= 1e-4, (dtype, lse_err.max())


@pytest.mark.parametrize("dtype,d,causal", [("fp32", 64, False), ("bf16", 128, True),
                                            ("bf16", 128, False)])
def test_shift_invariances(dtype, d, causal):
    """K -> K + c moves every logit of row i by scale*q_i.c (over whichever
    keys the row keeps), so O, dQ, dK and dV stay put and LSE moves by that
    amount; V -> V + c moves O by c and leaves dQ, dK, dV unchanged (the row
    sums of dS vanish).  K, V and c sit on a grid of multiples of 1/8 so the
    shifted inputs are exact in bf16: any difference comes from the kernels.
    Each pair is compared against the other run within the dtype's bar."""
    N = 300
    inp = W.random_inputs(1, 2, N, d, dtype, seed=61 + d)
    rng = np.random.default_rng(17)
    grid = lambda *shape: (rng.integers(-16, 17, size=shape) / 8.0).astype(np.float32)
    inp["k"], inp["v"] = grid(1, 2, N, d), grid(1, 2, N, d)
    c = (rng.integers(-8, 9, size=d) / 8.0).astype(np.float32)
    scale = 1 / math.sqrt(d)
    base = run_hip(inp, dtype, scale, causal)

    shk = run_hip(dict(inp, k=inp["k"] + c), dtype, scale, causal)
    lse_shift = scale * np.einsum("bhnd,d->bhn", inp["q"].astype(np.float64), c.astype(np.float64))
    tol_check("LSE", shk["LSE"], base["LSE"] + lse_shift, dtype)
    for n in ("O", "dQ", "dK", "dV"):
        e = tol_check(n, shk[n], base[n], dtype)
        _say(f"  K+c {dtype} d={d} causal={causal} {n}: " +
             " ".join(f"{kk}={vv:.3e}" for kk, vv in e.items()))

    shv = run_hip(dict(inp, v=inp["v"] + c), dtype, scale, causal)
    tol_check("O", shv["O"], base["O"] + c.astype(np.float64), dtype)
    tol_check("LSE", shv["LSE"], base["LSE"], dtype)
    for n in ("dQ", "dK", "dV"):
        e = tol_check(n, shv[n], base[n], dtype)
        _say(f"  V+c {dtype} d={d} causal={causal} {n}: " +
             " ".join(f"{kk}={vv:.3e}" for kk, vv in e.items()))


def test_determinism_bitwise():
    """No atomics: two runs give bit-identical outputs."""
    w = W.WORKLOADS["gpt2"].with_shape(B=2, H=4)
    x = W.make_inputs(w)
    q, k, v, do = (upload(x[n], "bf16") for n in ("q", "k", "v", "do"))
    outs = []
    for _ in range(2):
        o, lse = fa.forward(q, k, v, w.scale, True)
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, w.scale, True)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (o, lse, dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a,
                           b.view(torch.uint8) if b.dtype != torch.float32 else b)


def test_stream_argument_is_used():
    """Work enqueued on a side stream is ordered on that stream."""
    inp = W.random_inputs(1, 2, 256, 64, "bf16", seed=21)
    q, k, v = (upload(inp[n], "bf16") for n in ("q", "k", "v"))
    s = torch.cuda.Stream()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fa.fa_fwd(q, k, v, o, lse, 0.125, False, None, stream=s)
    s.synchronize()
    ref_o, ref_l = oracle.forward(inp["q"], inp["k"], inp["v"], 0.125, False)
    tol_check("O", o.float().cpu().numpy(), ref_o, "bf16")
    tol_check("LSE", lse.cpu().numpy(), ref_l, "bf16")


# --------------------------------------------------------------------------
# The five workloads at full size
# --------------------------------------------------------------------------

def _sample_rows(N, rng, n=48):
    fixed = [0, 1, N - 1, N // 2, min(N - 1, 127), min(N - 1, 128)]
    rest = rng.choice(N, size=min(N, n), replace=False)
    return np.unique(np.concatenate([fixed, rest]).astype(np.int64))


def _dev_inputs(x, dtype):
    return [upload(x[n], dtype) for n in ("q", "k", "v", "do")]


def test_long_sequence_query_rows():
    """N = 65536 (four times the longest workload; B*H = 2, so the blocks
    take the ordering for head counts that are not a multiple of 8): sampled
    query rows of O, LSE and dQ against the oracle, and dK, dV through the
    identities sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i."""
    N, d = 65536, 128
    x = W.random_inputs(1, 2, N, d, "bf16", seed=71)
    scale = 1 / math.sqrt(d)
    _say(f"long sequence: B=1 H=2 N={N} d={d} bf16 causal")
    q, k, v, do = _dev_inputs(x, "bf16")
    o, lse = fa.forward(q, k, v, scale, True)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale, True)
    torch.cuda.synchronize()
    got = {"O": o, "LSE": lse, "dQ": dq}
    dk_sum = dk.float().sum(dim=2)
    dk_scale = dk.float().abs().sum(dim=2) + 1e-6
    assert float((dk_sum.abs() / dk_scale).max()) < 2e-2
    rel = float((dv.double().sum(dim=2) - do.double().sum(dim=2)).norm() /
                do.double().sum(dim=2).norm())
    assert rel < 1e-2, rel
    rng = np.random.default_rng(9)
    for h in range(2):
        rows = _sample_rows(N, rng, n=24)
        ref = oracle.query_rows(x["q"][0, h], x["k"][0, h], x["v"][0, h], x["do"][0, h],
                                scale, rows, True)
        for n in ("O", "LSE", "dQ"):
            g = got[n][0, h][torch.from_numpy(rows).to(device())].float().cpu().numpy()
            e = tol_check(n, g, ref[n], "bf16")
            _say(f"  head {h} {n}: " + " ".join(f"{kk}={vv:.3e}" for kk, vv in e.items()))


def test_workload_tiny_full_oracle():
    w = W.WORKLOADS["tiny"]
    x = W.make_inputs(w)
    got = run_hip(x, "fp32", w.scale, w.causal, x["mask"])
    ref = oracle.forward_backward(x["q"], x["k"], x["v"], x["do"], w.scale, w.causal, x["mask"])
    check_all(got, ref, "fp32", "tiny")
    for n in OUTS:       # the literal fp32 bar: max-abs 1e-4 on every output
        assert np.abs(got[n] - ref[n]).max() <= 1e-4, n


@pytest.mark.parametrize("name", ["gpt2", "long", "sparse", "verylong", "long_nc"])
def test_workload_full_size_sampled(name):
    w = W.WORKLOADS[name]
    x = W.make_inputs(w)
    _say(f"workload {name}: B={w.B} H={w.H} N={w.N} d={w.d}")
    q, k, v, do = _dev_inputs(x, w.dtype)
    m = upload_mask(x["mask"])
    o, lse = fa.forward(q, k, v, w.scale, w.causal, m)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, w.scale, w.causal, m)
    torch.cuda.synchronize()
    got = {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}

    # Identities over every head (any size): sum_j dK_j = 0, sum_j dV_j = sum_i dO_i.
    dk_sum = dk.float().sum(dim=2)
    dk_scale = dk.float().abs().sum(dim=2) + 1e-6
    assert float((dk_sum.abs() / dk_scale).max()) < 2e-2
    dv_sum = dv.double().sum(dim=2)
    do_sum = do.double().sum(dim=2)
    rel = float((dv_sum - do_sum).norm() / do_sum.norm())
    _say(f"  identities: max|sum dK|/sum|dK| = {float((dk_sum.abs()/dk_scale).max()):.2e}, "
         f"|sum dV - sum dO|/|sum dO| = {rel:.2e}")
    assert rel < 1e-2

    rng = np.random.default_rng(7)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    for b, h in heads:
        rows = _sample_rows(w.N, rng)
        qr = oracle.query_rows(x["q"][b, h], x["k"][b, h], x["v"][b, h], x["do"][b, h],
                               w.scale, rows, w.causal, x["mask"])
        kr = oracle.key_rows(x["q"][b, h], x["k"][b, h], x["v"][b, h], x["do"][b, h],
                             w.scale, rows, w.causal, x["mask"])
        ref = {**qr, **kr}
        for n in OUTS:
            g = got[n][b, h][torch.from_numpy(rows).to(device())].float().cpu().numpy()
            e = tol_check(n, g, ref[n], w.dtype)
            _say(f"  {name} head ({b},{h}) {n}: " +
                 " ".join(f"{kk}={vv:.3e}" for kk, vv in e.items()))
