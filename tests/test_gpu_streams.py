"""Stream and graph behaviour of the C ABI on the GPU.

* The dK/dV and dQ passes only read what the preprocess wrote, as include/fa.h
  states: enqueued on two side streams that both wait for the preprocess, they
  give bit-identical results to fa_bwd on one stream, whose dQ pass forms D
  itself (so this also pins that D to the preprocess kernel's, bit for bit,
  for each element type and head size).
* The library enqueues kernels only (no memset, allocation or
  synchronisation), so a forward + backward step captured in a HIP graph
  replays to the eager results, replay after replay, with eager work and
  synchronisations in between.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from io_aware_exact_09_amd import fa
from io_aware_exact_09_amd import workloads as W
from gpu_util import upload

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, d, seed, dtype="bf16"):
    x = W.random_inputs(B, H, N, d, dtype, seed=seed)
    return [upload(x[n], dtype) for n in ("q", "k", "v", "do")]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 128), ("fp32", 64)])
def test_dkdv_and_dq_on_two_streams_match_fa_bwd(dtype, d):
    q, k, v, do = _inputs(2, 4, 777, d, seed=31, dtype=dtype)
    scale = d ** -0.5
    o, lse = fa.forward(q, k, v, scale, True)
    dq0, dk0, dv0 = fa.backward(q, k, v, o, do, lse, scale, True)
    torch.cuda.synchronize()

    B, H, N, d = q.shape
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    main = torch.cuda.current_stream()
    fa.fa_bwd_preprocess(o, do, ws, stream=main)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(main)
    s2.wait_stream(main)
    fa.fa_bwd_dkdv(q, k, v, do, lse, dk, dv, scale, True, None, ws, stream=s1)
    fa.fa_bwd_dq(q, k, v, do, lse, dq, scale, True, None, ws, stream=s2)
    main.wait_stream(s1)
    main.wait_stream(s2)
    torch.cuda.synchronize()
    for a, b, n in ((dq, dq0, "dQ"), (dk, dk0, "dK"), (dv, dv0, "dV")):
        assert torch.equal(a, b), n


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 128), ("fp32", 64)])
def test_dq_and_d_writes_the_preprocess_rowterm(dtype, d):
    """fa_bwd_dq_and_d's D equals fa_bwd_preprocess's bit for bit (ragged N,
    so the last row block is partial), and its dQ equals fa_bwd_dq's."""
    q, k, v, do = _inputs(1, 3, 333, d, seed=33, dtype=dtype)
    scale = d ** -0.5
    o, lse = fa.forward(q, k, v, scale, False)
    B, H, N, _ = q.shape
    nb = fa.fa_bwd_workspace_bytes(B, H, N, d)
    ws1 = torch.full((nb,), 0x7F, dtype=torch.uint8, device=q.device)
    ws2 = torch.full((nb,), 0x7F, dtype=torch.uint8, device=q.device)
    dq1, dq2 = torch.empty_like(q), torch.empty_like(q)
    fa.fa_bwd_preprocess(o, do, ws1)
    fa.fa_bwd_dq(q, k, v, do, lse, dq1, scale, False, None, ws1)
    fa.fa_bwd_dq_and_d(q, k, v, o, do, lse, dq2, scale, False, None, ws2)
    torch.cuda.synchronize()
    assert torch.equal(ws1, ws2)
    assert torch.equal(dq1, dq2)


def test_graph_capture_replays_match_eager():
    q, k, v, do = _inputs(1, 4, 640, 64, seed=32)
    scale = 0.125
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)

    def step():
        fa.fa_fwd(q, k, v, o, lse, scale, True, None)
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale, True, None, ws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o, lse, dq, dk, dv)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                    # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan")) if t.dtype == torch.float32 else t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((o, lse, dq, dk, dv), eager):
            assert torch.equal(a, b), f"replay {rep}"
        # eager work between replays
        fa.fa_fwd(q, k, v, torch.empty_like(o), torch.empty_like(lse), scale, False, None)
        torch.cuda.synchronize()
    assert np.isfinite(lse.cpu().numpy()).all()
