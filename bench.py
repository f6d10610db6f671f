"""Benchmark: FP32 SGEMM GFLOPS on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3_4096]
                    [--prewarm-s S] [--variant mfma|valu] [--no-cpu-baseline]
                    [--no-per-config] [--lowp all|bf16|f16|fp8|fp8e4m3|fp8e5m2|none]
                    [--lowp-only] [--lowp-k K] [--operand-fill draws|zeros]

A step is one SGEMM call, C = alpha*A*B + beta*C, on the headline workload
(M = N = K = 4096, alpha = 1.5, beta = 0.5, uniform [-1, 1) inputs, C
prefilled), with every operand already resident in device memory.  The same
call first runs back to back for S seconds (the pre-warm: a GPU that has
just come out of idle runs its first launches at a lower shader clock; each
other workload gets min(S, 0.2) seconds before its graph timing), then
W untimed steps, then exactly K timed steps bracketed by device
synchronisations.  The shader clock is measured right before and right after
the timed region.  The work count is 2*M*N*K per step ("GEMM 优化之路",
problem statement; the alpha/beta update is not counted).

Output: one JSON line with the throughput, the kernel's roofline position
(HIP events around every launch on the stream the kernel runs on), the CPU
oracle timed on a bounded sample of the same workload, and per-workload
GFLOPS for the other problem shapes and for decode-like products (1, 16 or 4
rows of A against B stored N x K, and one row against B as stored, with B's
stream rate); then the same
problems with bfloat16, binary16, E4M3 or E5M2 A and B and FP32 C (the
"lowp" object: per format,
the headline problem's roofline against the dense matrix-core peak of that
format, and the other shapes).  --lowp-only --lowp-k K times only the 16/8-bit
headline problem with K in place of 4096: two such runs under a cycle counter
give the kernels' cost per K step apart from their fixed cost.
--operand-fill zeros times the same calls on all-zero A and B: the 16/8-bit
kernels then run faster (the chip holds a higher clock when fewer operand
bits toggle), the FP32 kernel does not.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SGEMM GFLOPS and % of MI355X FP32 peak at M=N=K=4096 (1 GPU)"
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.json")
# Seconds of back-to-back launches before each per-workload graph timing, so
# that every shape is timed at the clock the GPU holds under load rather than
# after the host-side set-up between shapes (1024^3: ~19.5 against ~20.6 us).
PER_CONFIG_PREWARM_S = 0.2
# Decode-like products timed beside the five workloads: (workload, rows of A)
# with B stored N x K -- 1 x 4096 x 4096 (the headline's draws), 16 x 4096 x
# 4096, and 4 x 11008 x 4096 (the MLP shape's draws).
SMALL_M_CASES = (("c3_4096", 1), ("c3_4096", 16), ("c5_mlp", 4))


# the kernel code, the tile order and the tile shapes of each family
KERNEL_SOURCES = {"mfma": ("mfma_sgemm.hpp", "tile_map.hpp", "tiles.hpp"),
                  "valu": ("valu_sgemm.hpp", "tile_map.hpp", "tiles.hpp"),
                  "lp": ("lowp_gemm.hpp", "mfma_sgemm.hpp", "tile_map.hpp")}


def code_lines(text: str) -> str:
    """The source without // comments and blank lines: what the compiler sees
    of these headers (they hold no // inside string literals)."""
    out = []
    for line in text.splitlines():
        line = line.split("//", 1)[0].rstrip()
        if line:
            out.append(line)
    return "\n".join(out)


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code that defines a kernel family and its tile order
    (comments excluded, so documentation edits keep traffic records valid)."""
    csrc = os.path.join(ROOT, "fp32_gemm_major_amd", "csrc")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel.split("_")[0]]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + code_lines(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter runs, if they were
    taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    for e in data.get("entries", []):
        if (e.get("workload") == workload and e.get("kernel") == kernel
                and e.get("source_hash") == kernel_source_hash(kernel)):
            return e.get("hbm_bytes_per_launch")
    return None


def prewarm(launch, seconds, torch):
    """Run `launch` back to back, ten at a time, until `seconds` have passed;
    returns (launches, seconds taken)."""
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            launch()
        n += 10
        torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def time_launches(launch, steps, warmup, torch, before_timed=None):
    """Run `launch` warmup + steps times; return (total_ms, per-launch ms list).
    ``before_timed`` runs after the warmup, outside the timed region."""
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    if before_timed is not None:
        before_timed()
        torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record()
        launch()
        ends[i].record()
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    total = starts[0].elapsed_time(ends[-1])
    return total, per


def time_back_to_back(launch, steps, warmup, torch):
    """Mean ms per launch of `steps` launches queued back to back, timed by
    one event before the first and one after the last (same stream)."""
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        launch()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def time_graph(launch, reps, torch):
    """Mean time of one launch, from `reps` launches captured in a HIP graph and
    replayed back to back, so host launch overhead is not in the figure."""
    launch()  # compile-free warm start outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            launch()
    g.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        best = ms if best is None else min(best, ms)
    del g
    return best


def time_oracle(ops, target_s: float, threads: int):
    """Time the CPU oracle (FP64 triple loop, no error-bound pass) on the first
    rows of a problem with `threads` threads, growing the row count until one
    run takes about `target_s` seconds; when the whole problem takes less, it
    is repeated until the repetitions take about `target_s`.  Returns
    (GFLOPS, rows, repetitions, seconds)."""
    import oracle

    M, N, K = ops.M, ops.N, ops.K

    def run(rows, reps=1):
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.gemm(rows, N, K, ops.alpha, ops.A, ops.lda, ops.B, ops.ldb, ops.beta,
                        ops.C, ops.ldc, with_t=False, nthreads=threads)
        return time.perf_counter() - t0

    rows = min(threads, M)
    t = run(rows)
    for _ in range(3):  # grow the sample until it takes about target_s
        if t >= 0.6 * target_s or rows >= M:
            break
        want = int(rows * target_s / max(t, 1e-6))
        rows = max(rows + threads, min(M, (want // threads) * threads))
        rows = min(rows, M)
        t = run(rows)
    reps = 1
    if rows >= M and t < 0.6 * target_s:
        reps = max(2, int(round(target_s / max(t, 1e-6))))
        t = run(rows, reps)
    return 2.0 * rows * N * K * reps / t / 1e9, rows, reps, t


def cpu_baseline(ops, target_s: float):
    """The oracle on the host cores: all of them on a row slab of the timed
    problem, and one core on the small workloads (whole or a row slab)."""
    import oracle
    from fp32_gemm_major_amd import workloads as wl

    cores = oracle.default_threads()
    gf, rows, reps, t = time_oracle(ops, target_s, cores)
    single = {}
    for name in ("c1_128", "c2_1024", "c4_edge"):
        w = wl.WORKLOADS[name]
        g1, r1, n1, t1 = time_oracle(wl.operands(w), 1.5, 1)
        single[name] = {"gflops": round(g1, 3), "rows": r1, "of_rows": w.M,
                        "repetitions": n1, "seconds": round(t1, 2)}
    return {
        "value": round(gf, 3),
        "unit": "GFLOPS",
        "cores": cores,
        "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of the {ops.M}x{ops.N}x{ops.K} problem ({rows}x{ops.N} "
                  f"outputs, full K){f' x {reps} repetitions' if reps > 1 else ''}, "
                  f"FP64 accumulation, {t:.1f} s",
        "single_core": single,
    }


def lowp_section(args, sg, rf, wl, torch):
    """The products with 16-bit A and B (bfloat16 / binary16) or 8-bit A and
    B (E4M3 / E5M2) and FP32 C: the headline problem timed back to back on
    the launch stream, as its own roofline against the dense matrix-core
    peak of its input format, and the other workloads and the headline
    problem in the other storages from replayed HIP graphs.  The 8-bit
    headline and workloads store A as M x K and B as N x K (both
    K-contiguous), the 16-bit ones A as M x K and B as K x N."""
    formats = {"all": ("bf16", "f16", "fp8e4m3", "fp8e5m2"), "bf16": ("bf16",),
               "f16": ("f16",), "fp8": ("fp8e4m3", "fp8e5m2"),
               "fp8e4m3": ("fp8e4m3",), "fp8e5m2": ("fp8e5m2",), "none": ()}[args.lowp]
    if not formats:
        return None
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16,
           "fp8e4m3": torch.float8_e4m3fn, "fp8e5m2": torch.float8_e5m2}
    codes = {"bf16": sg.SGEMM_DTYPE_BF16, "f16": sg.SGEMM_DTYPE_F16,
             "fp8e4m3": sg.SGEMM_DTYPE_FP8_E4M3, "fp8e5m2": sg.SGEMM_DTYPE_FP8_E5M2}
    peaks = {"bf16": rf.PEAK_BF16_FLOPS, "f16": rf.PEAK_F16_FLOPS,
             "fp8e4m3": rf.PEAK_FP8_FLOPS, "fp8e5m2": rf.PEAK_FP8_FLOPS}
    h = sg.Handle()  # with a workspace, as the FP32 section: the library's default plans
    out = {}

    def prepare(name, dt, ta=False, tb=False, k=0, M=None):
        w = wl.WORKLOADS[name]
        if k > 0:  # the same problem at another K (--lowp-k)
            w = dataclasses.replace(w, K=k)
        if M is not None:  # decode-like: fewer rows of A
            w = dataclasses.replace(w, M=M)
        ops = wl.operands16(w, dt, ta=ta, tb=tb)
        raw = "uint8" if dt in wl.FORMATS8 else "int16"
        A = torch.from_numpy(ops.A.view(raw)).cuda().view(tdt[dt])
        B = torch.from_numpy(ops.B.view(raw)).cuda().view(tdt[dt])
        C = torch.from_numpy(ops.C).cuda()
        if args.operand_fill == "zeros":
            A.view(torch.uint8).zero_()
            B.view(torch.uint8).zero_()
        kid, _ = sg.sgemm_lowp_plan_handle(
            h.h, codes[dt], int(ta), int(tb), w.M, w.N, w.K, A.data_ptr(), ops.lda,
            B.data_ptr(), ops.ldb, C.data_ptr(), ops.ldc)

        def launch():
            h.gemm_lowp(A, B, C, w.alpha, w.beta, M=w.M, N=w.N, K=w.K, lda=ops.lda,
                        ldb=ops.ldb, ldc=ops.ldc, transa=ta, transb=tb)
        return w, (A, B, C), kid, launch

    for dt in formats:
        peak = peaks[dt]
        fp8 = dt in wl.FORMATS8
        w, dev, kid, launch = prepare(args.workload, dt, tb=fp8, k=args.lowp_k)
        steps = max(args.steps // 2, 10)
        # A change of workload restarts the GPU's clock ramp (tens of
        # milliseconds): the same pre-warm as the FP32 call, shorter.
        if args.prewarm_s > 0:
            prewarm(launch, min(args.prewarm_s, 0.3), torch)
        # Back-to-back launches between two events on the launch stream: a
        # ~130 us kernel bracketed by its own events measured ~5 us longer
        # than the profiler's duration for it.
        kms = time_back_to_back(launch, steps, max(args.warmup, 5), torch)
        achieved = rf.flops(w.M, w.N, w.K) / (kms * 1e-3)
        sec = {"roofline": {
            "bound": "mfma",
            "achieved": round(achieved / 1e12, 2),
            "peak": peak / 1e12,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(w.label + "_" + dt, sg.sgemm_lowp_kernel_name(kid)),
            "kernel": sg.sgemm_lowp_kernel_name(kid),
            "kernel_ms_mean": round(kms, 5),
            "alg_bytes": rf.alg_bytes(w.M, w.N, w.K, w.beta, ab_bytes=1 if fp8 else 2),
            "flops_per_launch": rf.flops(w.M, w.N, w.K),
            "launches": steps,
            # sustained rate of this format's MFMA chain with no memory traffic
            "mfma_chain_tflops": round(sg.mfma_chain_tflops(
                iterations=256 if fp8 else 1024, dtype=codes[dt]), 1),
        }}
        if fp8:
            sec["storage"] = "A M x K, B N x K"
        del dev
        per_config = {}
        if not args.no_per_config and args.lowp_k <= 0:
            cases = [("c1_128", False, fp8, 200), ("c2_1024", False, fp8, 200),
                     ("c4_edge", False, fp8, 100), ("c5_mlp", False, fp8, 20)]
            # the headline problem in the other three storages
            cases += [(args.workload, ta, tb, 20) for ta, tb in
                      ((False, False), (False, True), (True, False), (True, True))
                      if (ta, tb) != (False, fp8)]
            for name, ta, tb, reps in cases:
                w2, dev2, kid2, launch2 = prepare(name, dt, ta, tb)
                if args.prewarm_s > 0:
                    prewarm(launch2, min(args.prewarm_s, PER_CONFIG_PREWARM_S), torch)
                ms = time_graph(launch2, reps, torch)
                gf = rf.flops(w2.M, w2.N, w2.K) / (ms * 1e-3) / 1e9
                suffix = {(False, False): "_nn", (False, True): "_nt",
                          (True, False): "_tn", (True, True): "_tt"}[(ta, tb)]
                tag = name + (suffix if name == args.workload else "")
                per_config[tag] = {"gflops": round(gf, 1),
                                   "frac_of_peak": round(gf * 1e9 / peak, 4),
                                   "kernel_ms": round(ms, 5),
                                   "kernel": sg.sgemm_lowp_kernel_name(kid2)}
                del dev2
            # decode-like products, B stored N x K (as for FP32)
            for name, M in SMALL_M_CASES:
                w2, dev2, kid2, launch2 = prepare(name, dt, tb=True, M=M)
                if args.prewarm_s > 0:
                    prewarm(launch2, min(args.prewarm_s, PER_CONFIG_PREWARM_S), torch)
                ms = time_graph(launch2, 100, torch)
                gf = rf.flops(w2.M, w2.N, w2.K) / (ms * 1e-3) / 1e9
                per_config[f"{name}_m{M}_nt"] = {
                    "gflops": round(gf, 1), "kernel_ms": round(ms, 5),
                    "b_tbps": round((1 if fp8 else 2) * w2.N * w2.K / (ms * 1e-3) / 1e12, 3),
                    "kernel": sg.sgemm_lowp_kernel_name(kid2)}
                del dev2
        sec["per_config"] = per_config
        out[dt] = sec
    h.close()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3_4096")
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="seconds of back-to-back launches before the warmup steps")
    ap.add_argument("--variant", choices=["mfma", "valu"], default="mfma")
    ap.add_argument("--kernel", type=int, default=-1, help="force a kernel id")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--lowp", choices=["all", "bf16", "f16", "fp8", "fp8e4m3", "fp8e5m2",
                                       "none"], default="all",
                    help="which 16-bit- or 8-bit-input products to time after the FP32 ones")
    ap.add_argument("--lowp-k", type=int, default=0,
                    help="time the 16/8-bit headline problem at this K instead (two "
                         "runs at different K separate a kernel's cost per K step from "
                         "its fixed cost); the other workloads are then skipped")
    ap.add_argument("--lowp-only", action="store_true",
                    help="time only the 16-bit- and 8-bit-input products (for profiler "
                         "runs)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed region, run one plain device copy of this "
                         "many bytes (a reference dispatch for HBM byte counters)")
    ap.add_argument("--operand-fill", choices=["draws", "zeros"], default="draws",
                    help="zeros: time every product on all-zero A and B instead of the "
                         "workloads' draws (the 16/8-bit kernels' time depends on the "
                         "operand bits through the clock the chip holds; results are "
                         "not meaningful then)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this SGEMM library runs on one GPU; multi-GPU runs are not "
              "supported (--gpus must be 1)", file=sys.stderr)
        return 2

    import numpy as np  # noqa: F401
    import torch

    import fp32_gemm_major_amd as sg
    from fp32_gemm_major_amd import roofline as rf
    from fp32_gemm_major_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    variant = sg.SGEMM_VARIANT_MFMA if args.variant == "mfma" else sg.SGEMM_VARIANT_VALU
    h = sg.Handle(variant=variant, kernel=args.kernel)

    launches = {}  # launches per call of each prepared problem

    def prepare(name, ta=False, tb=False, M=None):
        w = wl.WORKLOADS[name]
        if M is not None:  # the same draws with fewer rows of A (decode-like)
            w = dataclasses.replace(w, M=M)
        ops = wl.operands(w, ta=ta, tb=tb)
        dev = [torch.from_numpy(x).cuda() for x in (ops.A, ops.B, ops.C)]
        if args.operand_fill == "zeros":
            dev[0].zero_()
            dev[1].zero_()
        plan = [(args.kernel, 0, w.N)] if args.kernel >= 0 else h.plan(
            w.M, w.N, w.K, dev[0].data_ptr(), ops.lda, dev[1].data_ptr(), ops.ldb,
            dev[2].data_ptr(), ops.ldc, transa=ta, transb=tb)
        kid = plan[0][0]
        launches[(name if not (ta or tb) else f"{name}_{int(ta)}{int(tb)}")
                 + ("" if M is None else f"_m{M}")] = len(plan)

        def launch():
            h.gemm(dev[0], dev[1], dev[2], w.alpha, w.beta, M=w.M, N=w.N, K=w.K,
                   lda=ops.lda, ldb=ops.ldb, ldc=ops.ldc, transa=ta, transb=tb)
        return w, ops, dev, kid, launch

    def reference_copy():
        # one plain device copy of known size: the scale for HBM byte counters
        if args.copy_bytes > 0:
            n = args.copy_bytes // 4
            src = torch.ones(n, device="cuda")
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst

    if args.lowp_only:
        lowp = lowp_section(args, sg, rf, wl, torch)
        h.close()
        reference_copy()
        print(json.dumps({"lowp": lowp}), flush=True)
        return 0

    w, ops, dev, kid, launch = prepare(args.workload)
    kname = sg.sgemm_kernel_name(kid)
    clock = {}
    # The shader clock as this call runs it: the same call with the kernel's
    # own clock stamps, twice right before the timed region and twice right
    # after it, launched without waiting (an idle gap, or any other work,
    # restarts the GPU's clock ramp) and read back after the timed region.
    # Their buffers are allocated first: from the pre-warm to the end of the
    # timed region nothing but this call runs on the GPU.
    clocked = launches[args.workload] == 1 and \
        sg.sgemm_kernel_schedule(kid) == sg.SGEMM_SCHEDULE_TILES and \
        sg.sgemm_kernel_info(kid)["variant"] == sg.SGEMM_VARIANT_MFMA
    stamp_bufs = [torch.zeros(4 * 65536, dtype=torch.int64, device="cuda")
                  for _ in range(4)] if clocked else []
    stamped = []
    torch.cuda.synchronize()
    pw_launches, pw_s = prewarm(launch, args.prewarm_s, torch) if args.prewarm_s > 0 \
        else (0, 0.0)

    def stamp(bufs):
        for b in bufs:
            stamped.append((b, h.gemm_stamped(dev[0], dev[1], dev[2], b, w.alpha, w.beta,
                                              M=w.M, N=w.N, K=w.K, lda=ops.lda,
                                              ldb=ops.ldb, ldc=ops.ldc)))

    total_ms, per = time_launches(launch, args.steps, args.warmup, torch,
                                  before_timed=lambda: stamp(stamp_bufs[:2]))
    stamp(stamp_bufs[2:])
    torch.cuda.synchronize()
    if stamped:
        khz = sg.sgemm_diag_wall_clock_khz()
        reads = [sg.clock_from_stamps(b[: 4 * n].cpu(), n, khz) for b, n in stamped]
        for when, part in (("before", reads[:2]), ("after", reads[2:])):
            clock[when + "_ghz"] = statistics.mean(g for g, _ in part)
            clock[when + "_span_us"] = statistics.mean(u for _, u in part)
    del stamp_bufs, stamped
    flops = rf.flops(w.M, w.N, w.K)
    ms_per_step = total_ms / args.steps
    kernel_ms = sum(per) / len(per)
    value = flops / (ms_per_step * 1e-3) / 1e9
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    peak = rf.PEAK_FP32_FLOPS / 1e12
    head = min(5, len(per))
    clock["spec_ghz"] = rf.CLOCK_HZ / 1e9
    if "before_ghz" in clock:
        observed_ghz = (clock["before_ghz"] + clock["after_ghz"]) / 2
        peak_at_clock = rf.CUS * rf.FP32_FLOPS_PER_CU_CLOCK * observed_ghz * 1e9
        clock["peak_tflops_at_observed"] = round(peak_at_clock / 1e12, 2)
        clock["pct_of_peak_at_observed"] = round(100.0 * value * 1e9 / peak_at_clock, 2)
    trend = {"first5_ms": round(sum(per[:head]) / head, 5),
             "last5_ms": round(sum(per[-head:]) / head, 5)}
    roof = {
        "bound": "mfma" if variant == sg.SGEMM_VARIANT_MFMA else "alu",
        "achieved": round(achieved, 3),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": measured_traffic(w.label, kname),
        "kernel": kname,
        "kernel_ms_mean": round(kernel_ms, 5),
        "kernel_ms_min": round(min(per), 5),
        "kernel_ms_median": round(statistics.median(per), 5),
        "alg_bytes": rf.alg_bytes(w.M, w.N, w.K, w.beta),
        "flops_per_launch": flops,
        # sustained rate of an MFMA chain with no memory traffic, measured now
        "mfma_chain_tflops": round(sg.mfma_chain_tflops(), 2),
    }
    del dev
    reference_copy()

    per_config = None
    if not args.no_per_config:
        # Each workload's launches are captured in a HIP graph and replayed, so
        # the small problems are timed without host launch overhead.
        per_config = {}

        def entry(w2, kid2, ms, peak=rf.PEAK_FP32_FLOPS):
            gf = rf.flops(w2.M, w2.N, w2.K) / (ms * 1e-3) / 1e9
            return {"gflops": round(gf, 1), "frac_of_peak": round(gf * 1e9 / peak, 4),
                    "kernel_ms": round(ms, 5), "kernel": sg.sgemm_kernel_name(kid2)}

        def timed(launch2, n):
            if args.prewarm_s > 0:
                prewarm(launch2, min(args.prewarm_s, PER_CONFIG_PREWARM_S), torch)
            return time_graph(launch2, n, torch)

        reps = {"c1_128": 200, "c2_1024": 200, "c4_edge": 100, "c5_mlp": 20}
        for name, n in reps.items():
            w2, _, dev2, kid2, launch2 = prepare(name)
            per_config[name] = entry(w2, kid2, timed(launch2, n))
            del dev2
        per_config[args.workload] = {"gflops": round(achieved * 1e3, 1),
                                     "frac_of_peak": roof["frac"],
                                     "kernel_ms": roof["kernel_ms_mean"],
                                     "kernel": kname}
        if variant == sg.SGEMM_VARIANT_MFMA:
            # the headline problem with transposed operand storage
            for ta, tb, tag in ((False, True, "nt"), (True, False, "tn"),
                                (True, True, "tt")):
                w3, _, dev3, kid3, launch3 = prepare(args.workload, ta, tb)
                per_config[f"{args.workload}_{tag}"] = entry(
                    w3, kid3, timed(launch3, 20))
                del dev3
            h.set_variant(sg.SGEMM_VARIANT_VALU)
            w3, _, dev3, _, launch3 = prepare(args.workload)
            kid3 = sg.sgemm_select_kernel(sg.SGEMM_VARIANT_VALU, w3.M, w3.N, w3.K,
                                          dev3[0].data_ptr(), w3.K, dev3[1].data_ptr(),
                                          w3.N, dev3[2].data_ptr(), w3.N)
            per_config[args.workload + "_valu"] = entry(w3, kid3, timed(launch3, 10))
            h.set_variant(variant)
            del dev3
            # decode-like products: a few rows of A against B stored N x K
            # (a Linear layer's weight), and one row against B as stored,
            # bound by reading B once; the
            # library's default plan, which picks between the matrix-core
            # split-K kernels and the one-pass vector-ALU ones
            h.set_variant(sg.SGEMM_VARIANT_AUTO)
            for name, M, tb in [c + (True,) for c in SMALL_M_CASES] + [("c3_4096", 1, False)]:
                w3, _, dev3, kid3, launch3 = prepare(name, tb=tb, M=M)
                e = entry(w3, kid3, timed(launch3, 100))
                e["b_tbps"] = round(4.0 * w3.N * w3.K / (e["kernel_ms"] * 1e-3) / 1e12, 3)
                per_config[f"{name}_m{M}" + ("_nt" if tb else "")] = e
                del dev3
            h.set_variant(variant)
    h.close()
    lowp = lowp_section(args, sg, rf, wl, torch)

    cpu = None if args.no_cpu_baseline else cpu_baseline(ops, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "operand_fill": args.operand_fill,
        "pct_of_fp32_peak": round(100.0 * value * 1e9 / rf.PEAK_FP32_FLOPS, 2),
        "prewarm": {"seconds": round(pw_s, 2), "launches": pw_launches},
        "clock": {k: round(v, 3) if isinstance(v, float) else v for k, v in clock.items()},
        "launch_trend": trend,
        "config": {"workload": w.label, "M": w.M, "N": w.N, "K": w.K,
                   "alpha": w.alpha, "beta": w.beta, "kernel": kname,
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_config": per_config,
        "lowp": lowp,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
