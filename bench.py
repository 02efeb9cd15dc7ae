"""Benchmark: exact-attention forward + training backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]

A step is one pass of the whole hot path over one batch: fa_fwd, then the
two kernels of fa_bwd (the dQ pass, which also forms the row term D, then the
dK/dV pass) through its phase entry points fa_bwd_dq_and_d and fa_bwd_dkdv,
on torch's current stream, inputs resident in HBM.  W untimed warm-up steps;
then the secondary measurements (K steps without cache eviction, "warm", and
the two-stream steps); then exactly K timed steps bracketed by
torch.cuda.synchronize(), the headline.  Before each of those (outside its
HIP events) a read of a 512 MiB device buffer evicts L2 and the 256 MB
Infinity Cache, so every timed step starts with its inputs in HBM only.  The
eviction reads rather than writes: a write would leave hundreds of MB of
dirty lines in the caches, whose write-back the timed step would then pay
for.  Each kernel of the step is bracketed by HIP events on the same stream,
created without the system-scope fence (HipEvent), so that recording them
does not flush the caches between the kernels.  The headline is the median
step time of those K steps, taken last because the GPU's clocks need a few
tens of steps of sustained work to settle.
Prints ONE JSON line.

Workloads are seeded synthetic inputs with the shapes of the FlashAttention
reading guide's training workloads (io_aware_exact_09_amd/workloads.py); the
default, "long" (B=2, H=16, N=4096, d=128, bf16, causal), is the N >= 4096,
d = 128 shape the throughput target is stated for.

Throughput uses algorithmic FLOPs (4 d per kept pair forward, 10 d backward;
causal and block-sparse skipping excluded, the dQ pass's recomputation not
counted).  The roofline object is for the kernel with the largest share of the
step, with its average launch time over the K timed steps; peak is the
published MI355X dense bf16 MFMA rate, 2.5 PFLOP/s (fp32 MFMA 157.3 TFLOP/s
for fp32 workloads).

The cpu_baseline leg times the CPU fp64 oracle on a bounded sample of the same
workload (whole heads, about 10-30 s) on this host's cores.  Secondary fields:
warm (the steps without the eviction) and two_stream_step (the staged phases:
the D preprocess, then the dK/dV and dQ passes on two streams; the headline
step is fa_bwd's single stream).

Decode workloads (--workload decode | decode_mix | decode_spec): a step is one
fa_decode call over the whole batch (64 sequences, 8K cache, 32 query heads
over 8 cache heads); value and roofline are algorithmic HBM bytes (visible
cache rows of K and V once, Q, O, LSE) per second against 8 TB/s, with the HIP
event pair around the call (its chunk kernel and the merge kernel).  FP8
(--workload long_fp8): a step is one fa_fwd_fp8 call.  Both use the same
protocol (evicted caches, median headline, warm secondary).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; 200 for the short gpt2 and tiny steps)")
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target duration of the CPU oracle sample")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="time fa_fwd_dropout + fa_bwd_dropout with this dropout probability "
                         "(the headline line is the dropout-free step)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain device copy of FA_COPY_PROBE_BYTES (512 MiB) first, "
                         "to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--no-two-stream", action="store_true",
                    help="skip the two-stream secondary (its staged phases launch the D "
                         "preprocess and a dQ pass that reads D; counter runs leave it out so "
                         "that every dQ launch is the headline's)")
    args = ap.parse_args()
    if args.steps is None:   # at least 200 repetitions where a step takes ~0.1 ms
        args.steps = 200 if args.workload in ("gpt2", "tiny") else 50
    return args


def recorded_traffic(workload, kernel):
    """Calibrated HBM bytes per launch of `kernel` from profiles/, if they
    were measured on the current kernel sources (else None)."""
    from io_aware_exact_09_amd import profiles
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != profiles.source_hash(profiles.family(workload)) or kernel not in rec:
        return None
    k = rec[kernel]
    if "read_bytes" not in k or "write_bytes" not in k:
        return None
    return k["read_bytes"] + k["write_bytes"]


def copy_probe(args, dev):
    """With --copy-probe: one torch.neg over FA_COPY_PROBE_BYTES (512 MiB) of
    bf16, reading n bytes and writing n bytes, to calibrate the rocprofv3
    FETCH_SIZE / WRITE_SIZE counters (the probe is found by its kernel name)."""
    if not args.copy_probe:
        return
    import torch
    n = int(os.environ.get("FA_COPY_PROBE_BYTES", 512 << 20))
    src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


FLUSH_BYTES = 512 << 20


class HipEvent:
    """A HIP timing event on torch's current stream, created with
    hipEventDisableSystemFence.  Recording a default event ends with a
    system-scope release, which writes back and invalidates the GPU caches
    and so slows the kernel launched after it (measured: a step with events
    between its kernels ran up to 8% longer on the 1K-token workload); this
    event only takes the timestamp.  The timed steps end with
    torch.cuda.synchronize(), which orders the host's reads of the times."""

    _hip = None
    FLAGS = 0x20000000       # hipEventDisableSystemFence

    @classmethod
    def runtime(cls):
        # The HIP runtime torch has already mapped (one copy per process).
        if cls._hip is None:
            import ctypes
            maps = open("/proc/self/maps").read()
            paths = sorted({ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln})
            if not paths:
                raise RuntimeError("no HIP runtime mapped (import torch and touch the GPU first)")
            hip = ctypes.CDLL(paths[0])
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        st = self.runtime().hipEventCreateWithFlags(ctypes.byref(self.h), self.FLAGS)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self):
        import torch
        st = self._hip.hipEventRecord(self.h, self._ct.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = self._ct.c_float()
        st = self._hip.hipEventElapsedTime(self._ct.byref(ms), self.h, end.h)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)


def eviction_buffer(dev):
    """FLUSH_BYTES of device memory, written once and settled, whose read
    (evict()) replaces the contents of L2 and the Infinity Cache."""
    import torch
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    evict(buf)
    torch.cuda.synchronize()
    return buf


def evict(buf):
    """Read the whole eviction buffer: one fp32 reduction kernel, which leaves
    clean lines (an int32 sum would first widen the buffer to int64 in a
    temporary, writing 1 GiB)."""
    return buf.sum()


def timed_steps(step, steps, nev, flush=None):
    """Run `steps` steps, step(events) recording `nev` HIP events on the
    current stream; with `flush` (an eviction_buffer), read it before each
    step, outside the step's events.  Bracketed by torch.cuda.synchronize().
    Returns (per-step event lists, wall seconds)."""
    import torch
    evs = [[HipEvent() for _ in range(nev)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            evict(flush)
        step(evs[i])
    torch.cuda.synchronize()
    return evs, time.perf_counter() - t0


def step_stats(ms):
    """median (headline), p50, p95 and mean with its 95% Student-t half-width."""
    s = sorted(ms)
    n = len(s)
    mean = statistics.mean(s)
    sd = statistics.stdev(s) if n > 1 else 0.0
    tcrit = {2: 12.706, 3: 4.303, 4: 3.182, 5: 2.776, 6: 2.571, 8: 2.365, 10: 2.262,
             15: 2.145, 20: 2.093, 30: 2.045}.get(n, 1.96 if n > 30 else 2.1)
    return {"median": statistics.median(s), "p50": s[n // 2],
            "p95": s[min(n - 1, int(0.95 * n))], "mean": mean,
            "ci95_half_width": tcrit * sd / math.sqrt(n) if n > 1 else None}


def cpu_model():
    """The host CPU's model name (lscpu's "Model name")."""
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ln.strip().startswith("Model name"):
                return ln.split(":", 1)[1].strip()
    except Exception:  # pragma: no cover
        pass
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def cpu_baseline(w, x, budget_s):
    """Time the fp64 oracle (fwd + bwd, whole heads) on a bounded sample."""
    import oracle
    from io_aware_exact_09_amd import accounting
    try:
        import threadpoolctl
        threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()),
                      default=os.cpu_count())
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        c = h // (w.H // w.kv_heads)                       # its key/value head
        kv = (slice(b, b + 1), slice(c, c + 1))
        oracle.forward_backward(x["q"][sl], x["k"][kv], x["v"][kv], x["do"][sl], w.scale,
                                w.causal, x["mask"])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    f = accounting.flops(1, done, w.N, w.d, w.causal, x["mask"])
    return {
        "value": (f["fwd"] + f["bwd"]) / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} heads (fwd+bwd, fp64 NumPy, S and P materialised), "
                  f"{el:.1f} s",
        "cpu_model": cpu_model(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(heads are independent, so several GPUs would each run this same "
              "single-GPU step on their share).", file=sys.stderr)
        sys.exit(2)

    import torch
    from io_aware_exact_09_amd import accounting, fa
    from io_aware_exact_09_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload in W.DECODE_WORKLOADS:
        return bench_decode(args)
    w = W.WORKLOADS[args.workload]
    if w.dtype == "fp8":
        return bench_fp8(args, w)
    x = W.make_inputs(w)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v, do = (torch.from_numpy(x[n]).to(dev).to(tdt).contiguous()
                   for n in ("q", "k", "v", "do"))
    mask = None if x["mask"] is None else torch.from_numpy(x["mask"]).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_gqa_workspace_bytes(w.B, w.H, w.kv_heads, w.N, w.d),
                     dtype=torch.uint8, device=dev)
    sc, cz = w.scale, w.causal
    copy_probe(args, dev)

    drop = args.dropout
    grouped = w.Hkv is not None and w.Hkv != w.H
    if grouped and drop > 0:
        print("--dropout is not offered for grouped key/value heads", file=sys.stderr)
        sys.exit(2)
    # Shapes whose blocks fill few compute units run the backward split (runs
    # of tiles with fp32 partials), which only the whole entry points do.
    split = (not grouped and drop == 0 and w.dtype == "bf16"
             and fa.fa_bwd_splits(w.B, w.H, w.H, w.N, w.d, w.dtype) != (1, 1))
    phases = ["fwd", "bwd"] if (drop > 0 or grouped or split) else ["fwd", "dq", "dkdv"]
    # ... and the forward in runs of key tiles, with a workspace
    fwd_ws_bytes = fa.fa_fwd_workspace_bytes(w.B, w.H, w.N, w.d) \
        if (split and mask is None) else 0
    fws = torch.empty(fwd_ws_bytes, dtype=torch.uint8, device=dev) if fwd_ws_bytes else None

    def step(ev=None):
        if split:
            # fa_fwd_ws (its kernels), then fa_bwd (its kernels in one entry point)
            if ev: ev[0].record()
            if fws is not None:
                fa.fa_fwd_ws(q, k, v, o, lse, sc, cz, mask, fws)
            else:
                fa.fa_fwd(q, k, v, o, lse, sc, cz, mask)
            if ev: ev[1].record()
            fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, sc, cz, mask, ws)
            if ev: ev[2].record()
            return
        if grouped:
            # fa_fwd_gqa, then fa_bwd_gqa (its kernels in one entry point)
            if ev: ev[0].record()
            fa.fa_fwd_gqa(q, k, v, o, lse, sc, cz, mask)
            if ev: ev[1].record()
            fa.fa_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, sc, cz, mask, ws)
            if ev: ev[2].record()
            return
        if drop > 0:
            # the backward's kernels run inside one entry point here
            if ev: ev[0].record()
            fa.fa_fwd_dropout(q, k, v, o, lse, sc, drop, 1234, cz, mask)
            if ev: ev[1].record()
            fa.fa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, sc, drop, 1234, cz, mask, ws)
            if ev: ev[2].record()
            return
        if ev: ev[0].record()
        fa.fa_fwd(q, k, v, o, lse, sc, cz, mask)
        if ev: ev[1].record()
        fa.fa_bwd_dq_and_d(q, k, v, o, do, lse, dq, sc, cz, mask, ws)
        if ev: ev[2].record()
        fa.fa_bwd_dkdv(q, k, v, do, lse, dk, dv, sc, cz, mask, ws)
        if ev: ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The secondary measurements first (K warm steps, then the two-stream
    # steps), then the headline: K timed steps, each after a cache eviction.
    # The GPU's clocks take a few tens of steps of sustained work to settle
    # (a trace of five warm-up steps followed by the timed ones shows the
    # dK/dV pass falling from ~375 to ~277 us over its first ~40 launches), so
    # the headline comes last, at the clocks a training loop runs at.
    nev = len(phases) + 1
    warm_evs, _ = timed_steps(step, args.steps, nev)
    two = two_stream_steps(args, step_parts=(q, k, v, o, lse, do, dq, dk, dv, sc, cz, mask, ws)) \
        if "dkdv" in phases and not args.no_two_stream else None
    flush = eviction_buffer(dev)
    evs, wall = timed_steps(step, args.steps, nev, flush)
    del flush

    per = {p: [e[i].elapsed_time(e[i + 1]) for e in evs] for i, p in enumerate(phases)}
    steps_ms = [e[0].elapsed_time(e[nev - 1]) for e in evs]
    warm_ms = [e[0].elapsed_time(e[nev - 1]) for e in warm_evs]
    st = step_stats(steps_ms)
    ms_step = st["median"]
    fl = accounting.flops(w.B, w.H, w.N, w.d, w.causal, x["mask"])
    peak = PEAK_TFLOPS[w.dtype]
    total = fl["fwd"] + fl["bwd"]
    value = total / (ms_step * 1e-3) / 1e12

    avg = {p: statistics.mean(per[p]) for p in phases}
    med = {p: statistics.median(per[p]) for p in phases}
    kflops = {"fwd": fl["fwd_kernel"], "dkdv": fl["dkdv_kernel"], "dq": fl["dq_kernel"],
              "bwd": fl["bwd"]}
    # The library runs bf16, d = 128 without a block mask on the ping-pong
    # forward kernel, everything else on the four-wave one.
    fwd_name = ("fa_fwd_pp_kernel" if w.dtype == "bf16" and w.d == 128 and w.mask_density is None
                and drop == 0 else "fa_fwd_kernel")
    if fws is not None:
        fwd_name = "fa_fwd_ws (all its kernels)"
    names = {"fwd": fwd_name, "dkdv": "fa_bwd_dkdv_kernel", "dq": "fa_bwd_dq_kernel",
             "bwd": ("fa_bwd_gqa" if grouped else "fa_bwd" if split else "fa_bwd_dropout")
             + " (all its kernels)"}
    dom = max(phases, key=lambda p: avg[p])
    ach = kflops[dom] / (avg[dom] * 1e-3) / 1e12
    roof = {"kernel": names[dom], "bound": "mfma", "achieved": ach, "peak": peak,
            "unit": "TFLOP/s", "frac": ach / peak,
            "traffic": recorded_traffic(w.name, names[dom]),
            "algorithmic_flops_per_launch": kflops[dom], "avg_launch_ms": avg[dom],
            "launches_averaged": args.steps}

    kernels = {}
    for p in phases:
        kernels[names[p]] = {"avg_ms": avg[p], "median_ms": med[p],
                             "tflops": kflops[p] / (avg[p] * 1e-3) / 1e12}

    fwd_ms = med["fwd"]
    bwd_ms = med["bwd"] if "bwd" in med else \
        statistics.median([a + b for a, b in zip(per["dq"], per["dkdv"])])

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, x, args.cpu_seconds)

    out = {
        "metric": "attention fwd+bwd TFLOP/s (bf16, 1 MI355X) and % of MFMA peak",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded iid normal Q, K, V, dO)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.kv_heads, "N": w.N,
                   "d": w.d,
                   "causal": w.causal, "block_sparse": x["mask"] is not None,
                   "dropout": drop,
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)"},
        "pct_of_peak": 100.0 * value / peak,
        "fwd_tflops": fl["fwd"] / (fwd_ms * 1e-3) / 1e12,
        "bwd_tflops": fl["bwd"] / (bwd_ms * 1e-3) / 1e12,
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "step_ms_stats": st,
        "timing": f"median of {args.steps} steps, each after a read of a {FLUSH_BYTES >> 20} MiB "
                  "device buffer outside its HIP events (caches evicted); per-kernel HIP events "
                  f"(no system-scope fence) on the launch stream; order: {args.warmup} warm-up "
                  f"steps, {args.steps} warm steps "
                  "(secondary), the two-stream steps (secondary), then these steps",
        "wall_s_timed": wall,
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": cpu,
        "warm": {"ms_per_step_median": statistics.median(warm_ms),
                 "value": total / (statistics.median(warm_ms) * 1e-3) / 1e12,
                 "steps": len(warm_ms)},
        "peak_tflops": peak,
    }
    if two is not None:
        out["two_stream_step"] = {**two, "value": total / (two["ms_per_step"] * 1e-3) / 1e12}
    print(json.dumps(out))


def two_stream_steps(args, step_parts):
    """Secondary timing: the same step with the dK/dV pass on the calling
    stream and the dQ pass on a second stream (default priority).  The two
    passes are independent, so a caller of the phase entry points can
    overlap them; each ends with CUs idle while its last work-groups finish.
    Every step ends with the calling stream waiting for the second one (the
    next forward rewrites O and LSE, which the dQ pass reads)."""
    import torch
    from io_aware_exact_09_amd import fa
    q, k, v, o, lse, do, dq, dk, dv, sc, cz, mask, ws = step_parts
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def step2():
        fa.fa_fwd(q, k, v, o, lse, sc, cz, mask)
        fa.fa_bwd_preprocess(o, do, ws)
        side.wait_stream(main)
        fa.fa_bwd_dkdv(q, k, v, do, lse, dk, dv, sc, cz, mask, ws)
        fa.fa_bwd_dq(q, k, v, do, lse, dq, sc, cz, mask, ws, stream=side)
        main.wait_stream(side)

    for _ in range(5):
        step2()
    e0, e1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step2()
    e1.record()
    torch.cuda.synchronize()
    return {"ms_per_step": e0.elapsed_time(e1) / args.steps, "steps": args.steps,
            "schedule": "fa_fwd, fa_bwd_preprocess, then fa_bwd_dkdv on the calling stream "
                        "and fa_bwd_dq on a second stream"}


def cpu_baseline_decode(w, x, budget_s):
    """Time the fp64 decode oracle on whole sequences (all heads) for about
    budget_s seconds."""
    import oracle
    from io_aware_exact_09_amd import accounting
    try:
        import threadpoolctl
        threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()),
                      default=os.cpu_count())
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    done = []
    t0 = time.perf_counter()
    for b in range(w.B):
        sl = slice(b, b + 1)
        oracle.decode.decode_forward(x["q"][sl], x["k"][sl], x["v"][sl], w.scale,
                                     x["seqlens"][sl], w.causal)
        done.append(b)
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    elem = 2 if w.dtype == "bf16" else 4
    by = accounting.decode_bytes(len(done), w.Hq, w.Hkv, w.Nq, w.d, elem, x["seqlens"][done])
    return {
        "value": by["total"] / el / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(done)} of {w.B} sequences (all heads, fp64 NumPy), {el:.1f} s",
        "cpu_model": cpu_model(),
    }


def bench_fp8(args, w):
    """FP8 forward: one step is one fa_fwd_fp8 call over the whole batch
    (inputs quantized to E4M3 on the host before timing)."""
    import torch
    from io_aware_exact_09_amd import accounting, fa
    from io_aware_exact_09_amd import workloads as W

    x = W.make_inputs(w)
    qz = W.quantize_fp8(x["q"], x["k"], x["v"])
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(np.ascontiguousarray(qz[n])).to(dev)
         for n in ("q8", "k8", "vt8", "sq", "sk", "sv")}
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    copy_probe(args, dev)

    def step(ev=None):
        if ev: ev[0].record()
        fa.fa_fwd_fp8(t["q8"], t["k8"], t["vt8"], t["sq"], t["sk"], t["sv"], o, lse, w.scale,
                      w.causal)
        if ev: ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    warm_evs, _ = timed_steps(step, args.steps, 2)          # secondary first (clocks settle)
    flush = eviction_buffer(dev)
    evs, wall = timed_steps(step, args.steps, 2, flush)
    del flush
    per = [e[0].elapsed_time(e[1]) for e in evs]
    st = step_stats(per)
    ms_step = st["median"]
    fl = accounting.flops(w.B, w.H, w.N, w.d, w.causal, None)
    peak = 5000.0                                   # dense FP8 MFMA, TFLOP/s
    value = fl["fwd"] / (ms_step * 1e-3) / 1e12
    avg = statistics.mean(per)
    ach = fl["fwd_kernel"] / (avg * 1e-3) / 1e12
    warm_ms = statistics.median([e[0].elapsed_time(e[1]) for e in warm_evs])
    out = {
        "metric": "attention FP8 (E4M3) forward TFLOP/s (1 MI355X) and % of FP8 MFMA peak",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded iid normal Q, K, V quantized to E4M3 per block)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "parallelism": "none (1 GPU)"},
        "pct_of_peak": 100.0 * value / peak,
        "step_ms_stats": st,
        "timing": f"median of {args.steps} calls, each after a read of a {FLUSH_BYTES >> 20} MiB "
                  "device buffer outside its HIP events (caches evicted), after the warm "
                  "secondary",
        "wall_s_timed": wall,
        "roofline": {"kernel": "fa_fwd_fp8_kernel", "bound": "mfma", "achieved": ach,
                     "peak": peak, "unit": "TFLOP/s", "frac": ach / peak,
                     "traffic": recorded_traffic(w.name, "fa_fwd_fp8_kernel"),
                     "algorithmic_flops_per_launch": fl["fwd_kernel"], "avg_launch_ms": avg},
        "cpu_baseline": None,
        "warm": {"ms_per_step_median": warm_ms,
                 "value": fl["fwd"] / (warm_ms * 1e-3) / 1e12},
    }
    print(json.dumps(out))


def decode_traffic(workload, S):
    """Calibrated HBM bytes of one fa_decode call (its one or two kernels)."""
    a = recorded_traffic(workload, "fa_decode_split_kernel")
    if a is None or S == 1:
        return a
    b = recorded_traffic(workload, "fa_decode_combine_kernel")
    return None if b is None else a + b


def bench_decode(args):
    """Split-KV decode: one step is one fa_decode call (its chunk kernel and,
    with several chunks, the merge kernel) over the whole batch."""
    import torch
    from io_aware_exact_09_amd import accounting, fa
    from io_aware_exact_09_amd import workloads as W

    w = W.DECODE_WORKLOADS[args.workload]
    x = W.make_decode_inputs(w)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(tdt).contiguous() for n in ("q", "k", "v"))
    sl = torch.from_numpy(x["seqlens"]).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    S = fa.fa_decode_num_splits(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.d)
    nws = fa.fa_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.d)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
    copy_probe(args, dev)

    def step(ev=None):
        if ev: ev[0].record()
        fa.fa_decode(q, k, v, o, lse, w.scale, sl, w.causal, 0, ws)
        if ev: ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    warm_evs, _ = timed_steps(step, args.steps, 2)          # secondary first (clocks settle)
    flush = eviction_buffer(dev)
    evs, wall = timed_steps(step, args.steps, 2, flush)
    del flush
    per = [e[0].elapsed_time(e[1]) for e in evs]
    st = step_stats(per)
    ms_step = st["median"]
    warm_ms = statistics.median([e[0].elapsed_time(e[1]) for e in warm_evs])
    elem = 2 if w.dtype == "bf16" else 4
    by = accounting.decode_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.d, elem, x["seqlens"])
    value = by["total"] / (ms_step * 1e-3) / 1e9
    avg = statistics.mean(per)
    ach = by["total"] / (avg * 1e-3) / 1e9
    name = "fa_decode_split_kernel" + (" + fa_decode_combine_kernel" if S > 1 else "")
    roof = {"kernel": name, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
            "traffic": decode_traffic(w.name, S),
            "algorithmic_bytes_per_launch": by["total"], "avg_launch_ms": avg}
    cpu = None if args.no_cpu else cpu_baseline_decode(w, x, args.cpu_seconds)
    out = {
        "metric": "decode attention HBM GB/s (bf16, 1 MI355X) and % of 8 TB/s",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded iid normal Q and key/value cache)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq,
                   "Nkv": w.Nkv, "d": w.d, "causal": w.causal, "lengths": w.lengths,
                   "cache_tokens": int(np.asarray(x["seqlens"]).sum()), "chunks": S,
                   "parallelism": "none (1 GPU)"},
        "pct_of_peak": 100.0 * value / HBM_PEAK_GBS,
        "tflops": by["flops"] / (ms_step * 1e-3) / 1e12,
        "step_ms_stats": st,
        "timing": f"median of {args.steps} calls, each after a read of a {FLUSH_BYTES >> 20} MiB "
                  "device buffer outside its HIP events (caches evicted), after the warm "
                  "secondary",
        "wall_s_timed": wall,
        "roofline": roof,
        "cpu_baseline": cpu,
        "warm": {"ms_per_step_median": warm_ms, "value": by["total"] / (warm_ms * 1e-3) / 1e9},
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
