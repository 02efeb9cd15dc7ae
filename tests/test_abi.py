"""The C-ABI library loads, exports what include/fa.h declares, and rejects
invalid arguments before launching anything.

These tests make no compute call: every fa_fwd/fa_bwd call below carries at
least one invalid argument, and validation is pure host code that returns
before the HIP runtime is touched.  Pointers are fake, never dereferenced.
"""

import ctypes
import subprocess

import pytest

from io_aware_exact_09_amd import fa

BF16, FP32 = fa.FA_BF16, fa.FA_FP32
A = 0x7f0000000000            # fake, 16-byte aligned, never dereferenced
MB = 1 << 24                   # spacing between fake tensors


def p(i, off=0):
    return ctypes.c_void_p(A + i * MB + off)


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def test_header_symbols_are_exported(lib):
    names = fa.header_functions()
    assert set(names) == {"fa_fwd", "fa_bwd_workspace_bytes", "fa_bwd", "fa_status_str",
                          "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq",
                          "fa_fwd_dropout", "fa_bwd_dropout", "fa_decode", "fa_fwd_gqa",
                          "fa_bwd_gqa", "fa_fwd_fp8", "fa_bwd_gqa_workspace_bytes",
                          "fa_decode_num_splits", "fa_decode_workspace_bytes",
                          "fa_bwd_static", "fa_bwd_dq_and_d", "fa_bwd_splits",
                          "fa_fwd_ws", "fa_fwd_workspace_bytes"}
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None
    # Nothing else leaks out of the library's C ABI namespace.
    assert {e for e in exported if e.startswith("fa_")} == set(names)


def test_status_strings(lib):
    for code, name in fa.STATUS.items():
        s = fa.status_str(code)
        assert s and s != "unknown status", name
    assert fa.status_str(42) == "unknown status"


def test_bwd_splits(lib):
    # enough blocks (B*H*ceil(N/128) >= 256): no split
    assert fa.fa_bwd_splits(2, 16, 16, 4096, 128, "bf16") == (1, 1)
    assert fa.fa_bwd_splits(8, 12, 12, 1024, 64, "bf16") == (1, 1)
    # one head of 16K rows (128 blocks): dK/dV runs of 32 query tiles, dQ runs of 32 key tiles
    assert fa.fa_bwd_splits(1, 1, 1, 16384, 128, "bf16") == (4, 8)
    # d = 64 runs two dK/dV work-groups per compute unit, so it aims at twice as many
    assert fa.fa_bwd_splits(1, 1, 1, 16384, 64, "bf16") == (8, 8)
    # short rows: capped by the tiles per run (4 query tiles, 8 key tiles)
    assert fa.fa_bwd_splits(1, 1, 1, 1024, 128, "bf16") == (2, 2)
    assert fa.fa_bwd_splits(1, 2, 2, 300, 128, "bf16") == (1, 1)
    # fp32 never splits; grouped heads keep their head split for dK/dV
    assert fa.fa_bwd_splits(1, 1, 1, 16384, 128, "fp32") == (1, 1)
    assert fa.fa_bwd_splits(2, 16, 4, 4096, 128, "bf16") == (2, 1)
    with pytest.raises(RuntimeError):
        fa.fa_bwd_splits(1, 6, 4, 100, 64, "bf16")
    st = lib.fa_bwd_splits(1, 1, 1, 128, 64, 0, None, None)
    assert st == 1      # FA_ERR_NULL


def test_fwd_workspace_bytes(lib):
    # one head of 16K rows: 64 blocks of 256 rows -> 8 runs; O, then LSE, in fp32
    rows = 16384
    assert fa.fa_fwd_workspace_bytes(1, 1, 16384, 128) == 8 * rows * 128 * 4 + 8 * rows * 4
    # d = 64 (the four-wave forward, 128-row blocks): 128 blocks -> 8 runs
    assert fa.fa_fwd_workspace_bytes(1, 1, 16384, 64) == 8 * rows * 64 * 4 + 8 * rows * 4
    # enough blocks, or too few key tiles: no split
    assert fa.fa_fwd_workspace_bytes(2, 16, 4096, 128) == 0
    assert fa.fa_fwd_workspace_bytes(4, 8, 8192, 64) == 0
    assert fa.fa_fwd_workspace_bytes(1, 1, 1000, 128) == 2 * 1000 * 128 * 4 + 2 * 1000 * 4
    assert fa.fa_fwd_workspace_bytes(1, 1, 900, 128) == 0
    assert fa.fa_fwd_workspace_bytes(0, 1, 16384, 128) == 0


def test_workspace_bytes(lib):
    # one head of 16K rows: D, then the dK/dV partials (4 runs), then dQ's (8 runs)
    rows = 4 * 16384
    assert fa.fa_bwd_workspace_bytes(1, 1, 16384, 128) == rows + 2 * 4 * 16384 * 128 * 4 \
        + 8 * 16384 * 128 * 4
    assert fa.fa_bwd_workspace_bytes(2, 16, 4096, 128) == 4 * 2 * 16 * 4096
    assert fa.fa_bwd_workspace_bytes(1, 8, 16384, 128) == 4 * 8 * 16384
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 64) == 4
    assert fa.fa_bwd_workspace_bytes(0, 1, 1, 64) == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 96) == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, 1 << 30, 128) == 0     # N*d overflows int32


def fwd(lib, q=p(0), k=p(1), v=p(2), o=p(3), lse=p(4), B=1, H=2, N=128, d=64, scale=0.125,
        causal=0, mask=None, dtype=BF16):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, mask, dtype, None)


def fwd_ws(lib, q=p(0), k=p(1), v=p(2), o=p(3), lse=p(4), B=1, H=2, N=128, d=64, scale=0.125,
           causal=0, mask=None, dtype=BF16, ws=p(9), wsb=1 << 20):
    return lib.fa_fwd_ws(q, k, v, o, lse, B, H, N, d, scale, causal, mask, dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(B=0), 2), (dict(d=96), 3), (dict(dtype=7), 4),
    (dict(o=p(3, 4)), 5), (dict(scale=float("nan")), 8), (dict(o=p(0, 64)), 9),
    (dict(ws=None), 6),            # NULL with a nonzero size
    (dict(ws=p(9, 4)), 6),         # not 16-byte aligned
    (dict(ws=p(3)), 9),            # overlaps O
    (dict(ws=p(1)), 9),            # overlaps K
    (dict(ws=p(4, 256)), 9),       # overlaps LSE
])
def test_fwd_ws_validation(lib, kw, code):
    assert fwd_ws(lib, **kw) == code


def bwd(lib, q=p(0), k=p(1), v=p(2), o=p(3), do=p(4), lse=p(5), dq=p(6), dk=p(7), dv=p(8),
        B=1, H=2, N=128, d=64, scale=0.125, causal=0, mask=None, dtype=BF16, ws=p(9),
        wsb=1 << 20):
    return lib.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, scale, causal, mask, dtype,
                      ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(lse=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(H=-1), 2), (dict(N=0), 2), (dict(N=1 << 30, d=128), 2),
    (dict(d=96), 3), (dict(d=32), 3), (dict(d=256), 3),
    (dict(dtype=7), 4),
    (dict(q=p(0, 8)), 5), (dict(o=p(3, 4)), 5), (dict(lse=p(4, 2)), 5),
    (dict(scale=float("nan")), 8), (dict(scale=float("inf")), 8), (dict(scale=-float("inf")), 8),
    (dict(o=p(0, 64)), 9), (dict(lse=p(2, 16)), 9), (dict(o=p(4)), 9),
    (dict(mask=p(3, 32)), 9),
])
def test_fwd_validation(lib, kw, code):
    assert fwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(do=None), 1), (dict(dv=None), 1), (dict(lse=None), 1),
    (dict(N=0), 2), (dict(d=80), 3), (dict(dtype=-1), 4),
    (dict(dk=p(7, 8)), 5), (dict(lse=p(5, 1)), 5),
    (dict(ws=None), 6), (dict(wsb=4 * 2 * 128 - 1), 6), (dict(ws=p(9, 4)), 6),
    (dict(scale=float("-inf")), 8),
    (dict(dq=p(0, 16)), 9), (dict(dk=p(6, 16)), 9), (dict(ws=p(5)), 9), (dict(dv=p(9)), 9),
    (dict(mask=p(8, 16)), 9),
])
def test_bwd_validation(lib, kw, code):
    assert bwd(lib, **kw) == code


def fwd_drop(lib, pdrop=0.1, seed=7, **kw):
    a = dict(q=p(0), k=p(1), v=p(2), o=p(3), lse=p(4), B=1, H=2, N=128, d=64, scale=0.125,
             causal=0, mask=None, dtype=BF16)
    a.update(kw)
    return lib.fa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                              a["d"], a["scale"], a["causal"], a["mask"], pdrop, seed,
                              a["dtype"], None)


def bwd_drop(lib, pdrop=0.1, seed=7, **kw):
    a = dict(q=p(0), k=p(1), v=p(2), o=p(3), do=p(4), lse=p(5), dq=p(6), dk=p(7), dv=p(8),
             B=1, H=2, N=128, d=64, scale=0.125, causal=0, mask=None, dtype=BF16, ws=p(9),
             wsb=1 << 20)
    a.update(kw)
    return lib.fa_bwd_dropout(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                              a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                              a["causal"], a["mask"], pdrop, seed, a["dtype"], a["ws"], a["wsb"],
                              None)


@pytest.mark.parametrize("pdrop", [-0.1, 1.0, 1.5, float("nan"), float("inf")])
def test_dropout_probability_validation(lib, pdrop):
    assert fwd_drop(lib, pdrop=pdrop) == 8
    assert bwd_drop(lib, pdrop=pdrop) == 8


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(N=0), 2), (dict(d=96), 3), (dict(dtype=7), 4),
    (dict(q=p(0, 8)), 5), (dict(o=p(0, 64)), 9),
])
def test_dropout_entry_points_check_like_the_plain_ones(lib, kw, code):
    assert fwd_drop(lib, **kw) == code
    bkw = {k2: v2 for k2, v2 in kw.items() if k2 != "o"}
    if kw.get("o") is not None and "o" in kw:
        bkw["dq"] = p(0, 64)
    assert bwd_drop(lib, **bkw) == code


def test_gqa_workspace_bytes(lib):
    # long_gqa: 2 x 4 key/value heads x 32 key blocks = 256 work-groups -> split in two
    d_bytes = 4 * 2 * 16 * 4096
    parts = 2 * 2 * 2 * 4 * 4096 * 128 * 4
    assert fa.fa_bwd_gqa_workspace_bytes(2, 16, 4, 4096, 128) == d_bytes + parts
    # one key/value head per query head, or enough work-groups: D only
    assert fa.fa_bwd_gqa_workspace_bytes(2, 16, 16, 4096, 128) == d_bytes
    assert fa.fa_bwd_gqa_workspace_bytes(16, 16, 4, 4096, 128) == 4 * 16 * 16 * 4096
    # split capped at the group size (MQA of 4 heads, one key block)
    assert fa.fa_bwd_gqa_workspace_bytes(1, 4, 1, 100, 64) == 1792 + 2 * 4 * 100 * 64 * 4
    assert fa.fa_bwd_gqa_workspace_bytes(1, 6, 4, 100, 64) == 0


def test_gqa_validation(lib):
    # fwd: (Q, K, V, O, LSE, B, Hq, Hkv, N, d, scale, causal, mask, dtype, stream)
    f = [p(0), p(1), p(2), p(3), p(4), 2, 8, 2, 128, 64, 0.125, 1, None, BF16, None]
    for idx, val, code in ((6, 7, 2), (7, 3, 2), (7, 0, 2), (7, 16, 2), (0, None, 1),
                           (9, 80, 3), (13, 9, 4), (10, float("nan"), 8), (3, p(1, 64), 9)):
        bad = list(f); bad[idx] = val
        assert lib.fa_fwd_gqa(*bad) == code, (idx, val)
    # K spans B * Hkv heads: an output starting inside its last head overlaps it
    kv_bytes = 2 * 2 * 128 * 64 * 2
    bad = list(f); bad[3] = p(1, kv_bytes - 16)
    assert lib.fa_fwd_gqa(*bad) == 9
    # bwd: (Q, K, V, O, dO, LSE, dQ, dK, dV, B, Hq, Hkv, N, d, scale, causal, mask, dtype,
    #       ws, wsb, stream)
    b = [p(0), p(1), p(2), p(3), p(4), p(5), p(6), p(7), p(8), 2, 8, 2, 128, 64, 0.125, 1, None,
         BF16, p(9), 4 << 20, None]
    need = fa.fa_bwd_gqa_workspace_bytes(2, 8, 2, 128, 64)
    for idx, val, code in ((11, 3, 2), (11, 0, 2), (8, None, 1), (18, None, 6),
                           (19, need - 1, 6), (7, p(6, 64), 9), (17, 2, 4)):
        bad = list(b); bad[idx] = val
        assert lib.fa_bwd_gqa(*bad) == code, (idx, val)


def test_fp8_validation(lib):
    # (Q8, K8, Vt8, sq, sk, sv, O, LSE, B, H, N, d, scale, causal, mask, stream)
    f = [p(0), p(1), p(2), p(3), p(4), p(5), p(6), p(7), 2, 4, 256, 128, 0.1, 1, None, None]
    for idx, val, code in ((0, None, 1), (4, None, 1), (7, None, 1), (10, 250, 2), (10, 0, 2),
                           (11, 96, 3), (12, float("nan"), 8), (2, p(2, 4), 5),
                           (3, p(3, 2), 5), (6, p(0, 64), 9), (7, p(5), 9)):
        bad = list(f); bad[idx] = val
        assert lib.fa_fwd_fp8(*bad) == code, (idx, val)


def test_decode_plan(lib):
    # 64 sequences x 8 cache heads: four 2048-key chunks (2048 work-groups)
    assert fa.fa_decode_num_splits(64, 32, 8, 1, 8192, 128) == 4
    assert fa.fa_decode_workspace_bytes(64, 32, 8, 1, 8192, 128) == 64 * 32 * 4 * 129 * 4
    # one long sequence: as many chunks as allowed (128 of 1024 keys)
    assert fa.fa_decode_num_splits(1, 32, 8, 1, 131072, 128) == 128
    # short caches: one chunk, no workspace
    assert fa.fa_decode_num_splits(64, 32, 8, 1, 100, 128) == 1
    assert fa.fa_decode_workspace_bytes(64, 32, 8, 1, 100, 128) == 0
    # explicit counts are an upper bound; chunks are whole 128-key tiles
    assert fa.fa_decode_num_splits(2, 4, 4, 1, 1000, 64, num_splits=7) == 4
    assert fa.fa_decode_num_splits(2, 4, 4, 1, 1000, 64, num_splits=1) == 1
    assert fa.fa_decode_num_splits(2, 4, 4, 1, 1000, 64, num_splits=100) == 8
    assert fa.fa_decode_workspace_bytes(2, 4, 4, 3, 1000, 64, num_splits=100) == 2 * 4 * 3 * 8 * 65 * 4
    # rejected sizes
    assert fa.fa_decode_num_splits(1, 6, 4, 1, 64, 64) == 0          # Hq not a multiple of Hkv
    assert fa.fa_decode_num_splits(1, 4, 4, 1, 64, 96) == 0
    assert fa.fa_decode_num_splits(1, 4, 4, 1, 64, 64, num_splits=1025) == 0
    assert fa.fa_decode_workspace_bytes(0, 4, 4, 1, 64, 64) == 0


def dec(lib, **kw):
    a = dict(q=p(0), k=p(1), v=p(2), sl=None, o=p(3), lse=p(4), B=2, Hq=8, Hkv=2, Nq=1,
             Nkv=4096, d=128, scale=0.1, causal=0, ns=0, dtype=BF16, ws=p(9), wsb=1 << 20)
    a.update(kw)
    return lib.fa_decode(a["q"], a["k"], a["v"], a["sl"], a["o"], a["lse"], a["B"], a["Hq"],
                         a["Hkv"], a["Nq"], a["Nkv"], a["d"], a["scale"], a["causal"], a["ns"],
                         a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(v=None), 1), (dict(lse=None), 1),
    (dict(B=0), 2), (dict(Hkv=3), 2), (dict(Nq=0), 2), (dict(Nkv=0), 2),
    (dict(Nkv=1 << 24), 2), (dict(d=96), 3), (dict(dtype=5), 4),
    (dict(q=p(0, 8)), 5), (dict(sl=p(5, 2)), 5), (dict(lse=p(4, 1)), 5),
    (dict(ws=None), 6), (dict(wsb=100), 6), (dict(ws=p(9, 8)), 6),
    (dict(scale=float("nan")), 8), (dict(ns=-1), 8), (dict(ns=2000), 8),
    (dict(o=p(1, 64)), 9), (dict(lse=p(3, 32)), 9), (dict(ws=p(2, 64)), 9),
    (dict(sl=p(4, 16), ns=1), 9), (dict(o=p(9)), 9),
])
def test_decode_validation(lib, kw, code):
    assert dec(lib, **kw) == code


def test_status_codes_match_header():
    text = open(fa.HEADER_PATH).read()
    for code, name in fa.STATUS.items():
        assert f"{name} = {code}" in text, name


def test_phase_validation(lib):
    # preprocess: (O, dO, B, H, N, d, dtype, ws, wsb, stream)
    assert lib.fa_bwd_preprocess(None, p(1), 1, 2, 128, 64, BF16, p(2), 1 << 20, None) == 1
    assert lib.fa_bwd_preprocess(p(0), p(1), 1, 2, 128, 96, BF16, p(2), 1 << 20, None) == 3
    assert lib.fa_bwd_preprocess(p(0), p(1), 1, 2, 128, 64, BF16, p(2), 1023, None) == 6
    assert lib.fa_bwd_preprocess(p(0), p(1), 1, 2, 128, 64, BF16, p(1, 64), 1 << 20, None) == 9
    # dkdv: (Q, K, V, dO, LSE, dK, dV, B, H, N, d, scale, causal, mask, dtype, ws, wsb, stream)
    args = [p(0), p(1), p(2), p(3), p(4), p(5), p(6), 1, 2, 128, 64, 0.125, 0, None, BF16, p(7),
            1 << 20, None]
    bad = list(args); bad[5] = None
    assert lib.fa_bwd_dkdv(*bad) == 1
    bad = list(args); bad[16] = 4
    assert lib.fa_bwd_dkdv(*bad) == 6
    bad = list(args); bad[6] = p(7)            # dV over the workspace (read by the pass)
    assert lib.fa_bwd_dkdv(*bad) == 9
    bad = list(args); bad[11] = float("inf")
    assert lib.fa_bwd_dkdv(*bad) == 8
    # dq: (Q, K, V, dO, LSE, dQ, B, H, N, d, scale, causal, mask, dtype, ws, wsb, stream)
    args = [p(0), p(1), p(2), p(3), p(4), p(5), 1, 2, 128, 64, 0.125, 1, None, BF16, p(7),
            1 << 20, None]
    bad = list(args); bad[5] = p(0, 16)
    assert lib.fa_bwd_dq(*bad) == 9
    bad = list(args); bad[14] = None
    assert lib.fa_bwd_dq(*bad) == 6
    bad = list(args); bad[13] = 3
    assert lib.fa_bwd_dq(*bad) == 4
    # dq_and_d: (Q, K, V, O, dO, LSE, dQ, B, H, N, d, scale, causal, mask, dtype, ws, wsb,
    # stream); it writes the workspace, so the workspace may overlap no input
    args = [p(0), p(1), p(2), p(3), p(4), p(5), p(6), 1, 2, 128, 64, 0.125, 1, None, BF16, p(7),
            1 << 20, None]
    bad = list(args); bad[3] = None
    assert lib.fa_bwd_dq_and_d(*bad) == 1
    bad = list(args); bad[15] = p(3, 64)       # workspace over O
    assert lib.fa_bwd_dq_and_d(*bad) == 9
    bad = list(args); bad[16] = 1023
    assert lib.fa_bwd_dq_and_d(*bad) == 6
    bad = list(args); bad[10] = 96
    assert lib.fa_bwd_dq_and_d(*bad) == 3


def test_single_hip_runtime_in_process(lib):
    """libfa.so binds to the HIP runtime torch already mapped (one copy)."""
    maps = open("/proc/self/maps").read()
    paths = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(paths) == 1, paths


@pytest.mark.parametrize("scale", [-0.125, -1.0, -0.0, -1e30, 3.4e38])
def test_any_finite_scale_passes_validation(lib, scale):
    """Any finite scale, negative included, passes the argument checks: each
    call below is stopped by the next check in order (a misaligned pointer)."""
    assert fwd(lib, scale=scale, q=p(0, 8)) == 5
    assert bwd(lib, scale=scale, dk=p(7, 8)) == 5
    assert fwd_drop(lib, scale=scale, q=p(0, 8)) == 5
    f = [p(0, 8), p(1), p(2), p(3), p(4), 2, 8, 2, 128, 64, scale, 1, None, BF16, None]
    assert lib.fa_fwd_gqa(*f) == 5
    f8 = [p(0), p(1), p(2, 4), p(3), p(4), p(5), p(6), p(7), 2, 4, 256, 128, scale, 1, None,
          None]
    assert lib.fa_fwd_fp8(*f8) == 5
    assert dec(lib, scale=scale, q=p(0, 8)) == 5


# One head's rows, rounded up to 256, times d times the element size must not
# exceed 2^32 - 1 bytes: the largest accepted N for d = 128 is 2^23 - 256 in
# fp32 and 2^24 - 256 in bf16.
@pytest.mark.parametrize("N,dtype,ok", [
    ((1 << 23) - 256, FP32, True), ((1 << 23) - 255, FP32, False), (1 << 23, FP32, False),
    ((1 << 24) - 256, BF16, True), ((1 << 24) - 255, BF16, False),
])
def test_head_bytes_fit_32_bit_offsets(lib, N, dtype, ok):
    # accepted shapes are stopped by the next check (a misaligned pointer)
    want = 5 if ok else 2
    assert fwd(lib, N=N, d=128, dtype=dtype, B=1, H=1, q=p(0, 8)) == want
    assert bwd(lib, N=N, d=128, dtype=dtype, B=1, H=1, dk=p(7, 8)) == want
    assert lib.fa_bwd_preprocess(p(0), p(1, 8), 1, 1, N, 128, dtype, p(2), 1 << 30,
                                 None) == want
    f8_ok = ok if dtype == BF16 else True        # FP8 codes: the bf16 bound (O is bf16)
    if N % 16 == 0:
        f8 = [p(0), p(1), p(2, 4), p(3), p(4), p(5), p(6), p(7), 1, 1, N, 128, 0.1, 1, None,
              None]
        assert lib.fa_fwd_fp8(*f8) == (5 if f8_ok else 2)


@pytest.mark.parametrize("Nkv,dtype,ok", [
    ((1 << 23) - 256, FP32, True), (1 << 23, FP32, False), ((1 << 24) - 256, BF16, True),
])
def test_decode_cache_head_fits_32_bit_offsets(lib, Nkv, dtype, ok):
    assert dec(lib, Nkv=Nkv, dtype=dtype, ns=1, q=p(0, 8)) == (5 if ok else 2)


def test_static_scratch_entry_point_validation(lib):
    """fa_bwd_static: the checks of fa_bwd, then the static scratch limit
    (4 * B * H * N bytes of D must fit FA_STATIC_SCRATCH_BYTES); every call
    below stops before the device is touched."""
    def call(**kw):
        a = dict(q=p(0), k=p(1), v=p(2), o=p(3), do=p(4), lse=p(5), dq=p(6), dk=p(7), dv=p(8),
                 B=1, H=2, N=128, d=64, scale=0.125, causal=0, mask=None, dtype=BF16)
        a.update(kw)
        return lib.fa_bwd_static(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                                 a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                                 a["causal"], a["mask"], a["dtype"], None)
    assert call(q=None) == 1
    assert call(N=0) == 2
    assert call(d=96) == 3
    assert call(dtype=5) == 4
    assert call(scale=float("nan")) == 8
    rows = fa.STATIC_SCRATCH_BYTES // 4
    assert call(B=1, H=1, N=rows + 1) == 10             # one row more than the scratch holds
    assert call(B=2, H=16, N=rows // 16) == 10
    assert "static scratch" in fa.status_str(10)
    text = open(fa.HEADER_PATH).read()
    assert f"#define FA_STATIC_SCRATCH_BYTES {fa.STATIC_SCRATCH_BYTES}" in text
