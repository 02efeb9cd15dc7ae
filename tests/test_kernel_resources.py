"""Register, scratch and occupancy budget of every kernel (CPU: compiler remarks).

A kernel that spills registers to scratch memory inside its tile loop runs
several times slower without any change in its results (the non-causal bf16
dQ pass once did: 1183 vs 358 us on a 2x16x4096x128 shape), so the parity
tests cannot see it.  This test compiles each HIP source for gfx950 with the
compiler's resource-usage remarks and checks, for every instantiated kernel:
no scratch memory (except the list below), LDS within the 160 KiB of a CU, and
the waves per SIMD the hot kernels are designed for.
"""

from __future__ import annotations

import concurrent.futures as cf
import re

import pytest

from io_aware_exact_09_amd import build as B

SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_fwd_fp8.hip"]

# Kernels are named by (function, template arguments) with bf16 as "bf16",
# float as "f32", integers and bools as Python values.
#
# Known to spill: the dK/dV pass with dropout and a block mask, bf16,
# d = 128, without the causal mask.  At one wave per SIMD it uses all 512
# registers (256 VGPRs, 256 AGPRs); 4 VGPRs more go to spill slots in the
# accumulation registers (no scratch memory).  The other dropout kernels fit.
SCRATCH_ALLOWED = {
    ("fa_bwd_dkdv_kernel", ("bf16", 128, False, True, True)),
}

# Waves per SIMD the kernels are laid out for (bf16, d = 128, no dropout).
OCCUPANCY = {
    ("fa_fwd_pp_kernel", ("bf16", 128, True)): 2,
    ("fa_fwd_pp_kernel", ("bf16", 128, False)): 2,
    ("fa_bwd_dkdv_kernel", ("bf16", 128, True, False, False)): 1,
    ("fa_bwd_dkdv_kernel", ("bf16", 128, False, False, False)): 1,
    ("fa_bwd_dq_kernel", ("bf16", 128, True, False, False)): 2,
    ("fa_bwd_dq_kernel", ("bf16", 128, False, False, False)): 2,
    # d = 64: two waves per SIMD (two work-groups per compute unit)
    ("fa_bwd_dkdv_kernel", ("bf16", 64, True, False, False)): 2,
    ("fa_bwd_dkdv_kernel", ("bf16", 64, False, True, False)): 2,
    # d = 64 forward and dQ pass: three waves per SIMD
    ("fa_fwd_kernel", ("bf16", 64, True, False, False)): 3,
    ("fa_fwd_kernel", ("bf16", 64, False, True, False)): 3,
    ("fa_bwd_dq_kernel", ("bf16", 64, True, False, False)): 3,
    ("fa_bwd_dq_kernel", ("bf16", 64, False, True, False)): 3,
}

LDS_BYTES = 160 * 1024

_ARG = re.compile(r"DF16b|f|Li(\d+)E|Lb([01])E")


def kernel_key(mangled: str):
    """(name, template arguments) of a mangled fa:: kernel template
    (the system demangler does not know the bf16 type code)."""
    m = re.match(r"_ZN2fa(\d+)", mangled)
    assert m, mangled
    n = int(m.group(1))
    name = mangled[m.end():m.end() + n]
    rest = mangled[m.end() + n:]
    assert rest.startswith("I"), mangled
    args, pos = [], 1
    while not rest.startswith("E", pos):
        a = _ARG.match(rest, pos)
        assert a, mangled
        tok = a.group(0)
        args.append("bf16" if tok == "DF16b" else "f32" if tok == "f" else
                    int(a.group(1)) if a.group(1) is not None else a.group(2) == "1")
        pos = a.end()
    return name, tuple(args)


def test_kernel_key_parses_the_mangled_forms():
    assert kernel_key("_ZN2fa16fa_fwd_pp_kernelIDF16bLi128ELb1EEEvPKT_S3_S3_PS1_Pfiiif") == \
        ("fa_fwd_pp_kernel", ("bf16", 128, True))
    assert kernel_key("_ZN2fa16fa_bwd_dq_kernelIfLi64ELb0ELb1ELb0EEEvPKT_S3_") == \
        ("fa_bwd_dq_kernel", ("f32", 64, False, True, False))


@pytest.fixture(scope="module")
def usage():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        per_src = list(ex.map(B.resource_usage, SOURCES))
    return {kernel_key(n): u for per in per_src for n, u in per.items()}


def test_every_source_reports_its_kernels(usage):
    kinds = ("fa_fwd_kernel", "fa_fwd_pp_kernel", "fa_bwd_delta_kernel", "fa_bwd_dkdv_kernel",
             "fa_bwd_dq_kernel", "fa_decode_split_kernel", "fa_decode_combine_kernel",
             "fa_fwd_fp8_kernel")
    for k in kinds:
        assert any(n == k for n, _ in usage), k
    for n in list(SCRATCH_ALLOWED) + list(OCCUPANCY):
        assert n in usage, n


def test_no_scratch_outside_the_known_list(usage):
    bad = {n: (u.get("ScratchSize"), u.get("VGPRs Spill")) for n, u in usage.items()
           if (u.get("ScratchSize", 0) or u.get("VGPRs Spill", 0)) and n not in SCRATCH_ALLOWED}
    assert not bad, bad


def test_lds_fits_a_cu(usage):
    big = {n: u["LDS Size"] for n, u in usage.items() if u.get("LDS Size", 0) > LDS_BYTES}
    assert not big, big


def test_hot_kernels_keep_their_waves_per_simd(usage):
    got = {n: usage[n].get("Occupancy") for n in OCCUPANCY}
    assert got == OCCUPANCY
