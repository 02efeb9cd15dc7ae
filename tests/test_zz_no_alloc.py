"""fa_bwd_static, the backward for callers that cannot allocate, against
fa_bwd through the C ABI: the same kernels, with the row term D in the
library's static device scratch instead of a caller workspace, so the
gradients must be bit-identical.

Two calls in a row, the second with a smaller input (the scratch keeps the
first call's contents, which the second must not see): the largest size the
scratch allows (B*H*N = FA_STATIC_SCRATCH_BYTES / 4 rows), then a small fp32
case with a block mask and a ragged tail.  A size one row over the limit is
rejected before anything is enqueued.
"""

from __future__ import annotations

import math
import sys

import pytest
import torch

from io_aware_exact_09_amd import fa
from io_aware_exact_09_amd import workloads as W
from gpu_util import upload, upload_mask

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _both(B, H, N, d, dtype, causal, mask, seed):
    x = W.random_inputs(B, H, N, d, dtype, seed=seed)
    q, k, v, do = (upload(x[n], dtype) for n in ("q", "k", "v", "do"))
    m = upload_mask(mask)
    scale = 1 / math.sqrt(d)
    o, lse = fa.forward(q, k, v, scale, causal, m)
    ref = fa.backward(q, k, v, o, do, lse, scale, causal, m)
    got = [torch.full_like(t, float("nan")) for t in ref]
    fa.fa_bwd_static(q, k, v, o, do, lse, *got, scale, causal, m)
    torch.cuda.synchronize()
    return ref, got


def test_static_scratch_backward_equals_fa_bwd():
    rows = fa.STATIC_SCRATCH_BYTES // 4
    cases = [
        # (B, H, N, d, dtype, causal, mask): the largest size first, then a smaller one
        (1, 16, rows // 16, 64, "bf16", True, None),
        (2, 3, 300, 128, "fp32", False, W.random_block_mask(300, 0.6, seed=4)),
    ]
    for i, (B, H, N, d, dtype, causal, mask) in enumerate(cases):
        _say(f"call {i}: B={B} H={H} N={N} d={d} {dtype} causal={causal} "
             f"mask={'yes' if mask is not None else 'no'} ({B * H * N} rows of D)")
        ref, got = _both(B, H, N, d, dtype, causal, mask, seed=70 + i)
        for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(a, b), (i, name)


def test_static_scratch_rejects_sizes_over_the_limit():
    rows = fa.STATIC_SCRATCH_BYTES // 4
    q = torch.zeros((1, 1, rows + 1, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, rows + 1), dtype=torch.float32, device="cuda")
    outs = [torch.empty_like(q) for _ in range(3)]
    with pytest.raises(fa.FAError) as e:
        fa.fa_bwd_static(q, q, q, q, q, lse, *outs, 0.125, True)
    assert e.value.status == 10
