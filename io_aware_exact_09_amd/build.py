"""Build libfa.so in-tree with hipcc for gfx950.

    python -m io_aware_exact_09_amd.build        (or build() from Python)

Every HIP translation unit is compiled in parallel, then linked into
``io_aware_exact_09_amd/libfa.so``.  The packed-fp32 target feature is turned
off for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_fwd_fp8.hip",
           "fa_static.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results and accumulators in VGPRs (operands may still come
        # from AGPRs): the accumulators the VALU works on (S, dP) then need
        # no copies out of AGPRs, which otherwise cost about one VALU
        # instruction per accumulator register per tile in the dK/dV pass.
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I", os.path.join(ROOT, "include"),
    ]


def _compile(src: str, extra: list[str]) -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + common_flags() + extra
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


_REMARK = re.compile(r"remark: +(Function Name|TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|SGPRs Spill|VGPRs Spill|"
                     r"LDS Size \[bytes/block\]): (\S+)")


def resource_usage(src: str) -> dict[str, dict[str, int]]:
    """Per-kernel register, scratch, occupancy and LDS figures of one source
    file, from a device-only compile with the compiler's resource-usage
    remarks: {mangled kernel name: {"VGPRs": .., "AGPRs": .., "ScratchSize":
    .., "Occupancy": .., "VGPRs Spill": .., "SGPRs Spill": .., "LDS Size": ..}}."""
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", os.devnull, "--cuda-device-only",
           "-Rpass-analysis=kernel-resource-usage"] + common_flags()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    out: dict[str, dict[str, int]] = {}
    cur = None
    for m in _REMARK.finditer(r.stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val)
    return out


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


PROBE_SRC = os.path.join(ROOT, "tests", "gpu_probe", "mfma_rounding_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "gpu_probe", "libfa_probe.so")


def build_test_probe(verbose: bool = False) -> str:
    """Test support, not part of libfa.so: the one-wave matrix-instruction
    probe the GPU tests use to check the accumulation model of the FP8 and
    bf16 instructions (tests/gpu_probe)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), "-shared", PROBE_SRC, "-o", tmp] + common_flags()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
    build_test_probe(verbose=True)
