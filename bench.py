"""Benchmark: one ZeRO rank's fused reduce + AdamW + bf16 re-cast step on one GPU.

A step is one call of the library on the whole workload (default: the
70B-parameter model's 1/64 shard, 1,093,750,000 parameters, 64 replica
gradient chunks, warm state at step 5000, weight decay 0.1).  Inputs are
seeded synthetic draws generated in device memory before timing.

Prints one JSON line.  `value` is parameters updated per second; the roofline
object prices the kernel's algorithmic bytes, (2N + 26) per parameter, against
MI355X's 8 TB/s HBM peak.  The CPU oracle's throughput on a bounded sample of
the same workload is reported beside it as `cpu_baseline`.  Parity at these
sizes, in the same launch configuration, is checked by tests/test_gpu_fullsize.py.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "params/s and achieved HBM GB/s (% of peak) for fused reduce+Adam shard step"
HBM_PEAK_GBPS = 8000.0
KERNEL_SRCS = [os.path.join(ROOT, "sharded_mixed_precision_rank_amd", "csrc", f)
               for f in ("zs_kernels.hip", "zs_twopass.hip", "zs_device.h", "zs_phased.h", "zs_internal.h",
                         "zs_twopass.h")]
PROFILES = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# bench.py --workload NAME
WORKLOADS = {
    "flat-1m": lambda W: W.FLAT_1M_N2,                             # 2^20 params, N=2, cold, step 1
    "flat-124m": lambda W: W.FLAT_124M_N8,                         # 124M params, N=8, warm, step 100
    "list-llama7b": lambda W: W.list_llama7b_dp8_n8(),             # 288 tensors, 809.5M params, N=8
    "flat-70b": lambda W: W.FLAT_70B_DP64_N64,                     # 70B/64 shard, N=64, step 5000, wd 0.1
    "list-llama70b": lambda W: W.list_llama70b_dp64_n64(),         # the 70B/64 shard as 720 per-layer tensors
    "list-ragged": lambda W: W.list_ragged_20000_n16(1),           # 20,000 ragged tensors, N=16, cold
    "list-ragged-warm": lambda W: W.list_ragged_20000_n16(10000),  # the same, warm, step 10000
}


def workload(name: str):
    from synth import workloads as W

    return WORKLOADS[name](W)


def kernel_hash() -> str:
    """Hash of the sources the step kernels are built from, comments and blank space left out (an
    edit to a comment does not make a counter summary stale)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def counter_traffic(w, kernel: str):
    """HBM bytes per step of `kernel` (its name without template arguments; one launch, or the sum over a
    step's consecutive launches) from the committed rocprofv3 counter summary for this workload, if it
    was taken on the current kernel source; else None.  The per-kernel summary
    (zs_kernel_<workload>_counters.txt) gives the read+write total; the per-workload one
    (zs_kernels_<workload>.txt) gives read and write bytes under each kernel's line."""
    tag = w.name.replace("/", "-")
    path = os.path.join(PROFILES, f"zs_kernel_{tag}_counters.txt")
    multi = os.path.join(PROFILES, f"zs_kernels_{tag}.txt")
    if os.path.exists(path):
        txt = open(path, encoding="utf-8").read()
        m_name = re.search(r"^# rocprofv3 counter summary: (\w+),", txt, flags=re.M)
        m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
        if not m_name or m_name.group(1) != kernel or not m_bytes:
            return None
        total = float(m_bytes.group(1))
    elif os.path.exists(multi):
        txt = open(multi, encoding="utf-8").read()
        m = re.search(rf"^{re.escape(kernel)}: .* per step.*\n\s+hbm read\s+([0-9.eE+]+) B/step.*\n"
                      rf"\s+hbm write\s+([0-9.eE+]+) B/step", txt, flags=re.M)
        if not m:
            return None
        total = float(m.group(1)) + float(m.group(2))
    else:
        return None
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    if not m_hash or m_hash.group(1) != kernel_hash():
        return None
    return total


def pattern_ceiling(w, d, window=(0, 0), reps: int = 5, phased: bool = False):
    """What the memory system delivers for the step's own access pattern on this machine: the measurement
    probe (bench_probe/libzshard_probe.so) replays the fused kernel's loads and stores, tile layout and
    non-temporal hints included, with the AdamW arithmetic taken out, on the same buffers.  Reported as
    GB/s of the pattern's own bytes for the read streams alone ((2N+12) B/param), for the full
    read+write mix ((2N+26) B/param) with each tile's writes issued as soon as it is done, when the
    step groups its writes in device-clock windows (`window` = (period, open) ticks) for the same mix
    with the same windows, and when the step runs the phased schedule, for its super-chunk loop (the
    library's own code, zs_phased.h) over the shard's whole super-chunks.  It overwrites the state: run
    it after the timed steps."""
    import ctypes

    import torch

    import bench_probe

    lib = bench_probe.load()
    N, n = w.N, d["arena_len"]
    full = n // 512 * 512   # the probe covers whole 512-parameter tiles
    tab = (ctypes.c_void_p * N)(*[g.data_ptr() for g in d["G"]])
    stream = torch.cuda.current_stream()
    out = {}
    modes = [(0, 2 * N + 12, "read"), (1, 2 * N + 26, "read_write")]
    if window[0]:
        modes.append((2, 2 * N + 26, "read_write_windowed"))
    if phased:
        modes.append((3, 2 * N + 26, "read_write_phased"))
    covered = torch.zeros(1, dtype=torch.int64, device="cuda")
    for write, bpp, name in modes:
        def call():
            ptrs = (tab, N, n, d["P"].data_ptr(), d["M"].data_ptr(), d["V"].data_ptr(), d["B"].data_ptr())
            if write == 3:
                return lib.zs_probe_pattern_phased(*ptrs, covered.data_ptr(), stream.cuda_stream)
            if write == 2:
                return lib.zs_probe_pattern_windowed(*ptrs, window[0], window[1], stream.cuda_stream)
            return lib.zs_probe_pattern(*ptrs, write, stream.cuda_stream)
        if call() != 0:
            if write == 3:
                continue  # the phased probe covers N = 64 only
            return None  # a replica count or alignment the probe does not cover
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        params = int(covered.item()) if write == 3 else full
        out[f"{name}_GBps"] = bpp * params * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    return out


def copy_ceiling(gbytes: float = 8.0, reps: int = 5) -> float:
    """Read+write GB/s of the probe's copy kernel (built as the step's kernels are: one-wave
    512-element tiles, whole-line lane layout, non-temporal loads and stores, launches of at most
    3 GB) over `gbytes` in all, half read and half written: the box's rate for an even mix."""
    import torch

    import bench_probe

    lib = bench_probe.load()
    n = int(gbytes * 1e9) // 8
    src = torch.empty(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    stream = torch.cuda.current_stream()
    def call():
        if lib.zs_probe_copy(src.data_ptr(), dst.data_ptr(), n, stream.cuda_stream) != 0:
            raise RuntimeError("zs_probe_copy failed")
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 8 * n / t / 1e9


def cpu_baseline(w, target_s: float) -> dict:
    """The CPU oracle, as it stands, timed on this host's cores over a bounded
    slice of the workload (the first `n` parameters), repeated until about
    `target_s` seconds of compute have run."""
    import numpy as np

    import oracle
    from synth import workloads as W

    cores = len(os.sched_getaffinity(0))
    threads = min(cores, 16)
    n = 2_000_000 if w.N >= 32 else 8_000_000
    h = W.host_inputs(w, 0, n)
    o = oracle.load()
    P, M, V = h["P"].copy(), h["M"].copy(), h["V"].copy()
    B = np.empty(n, dtype=np.uint16)
    def timed(nthreads: int, budget: float):
        reps, spent = 0, 0.0
        while spent < budget or reps == 0:
            t0 = time.perf_counter()
            o.step_inplace(h["G"], P, M, V, B, w.hp(), w.step + reps, threads=nthreads)
            spent += time.perf_counter() - t0
            reps += 1
        return reps, spent

    reps, spent = timed(threads, target_s)
    reps1, spent1 = timed(1, min(3.0, target_s / 3))  # the same oracle on one core
    pps = n * reps / spent
    return dict(value=pps, unit="params/s", cores=threads, kind="oracle",
                gbps=pps * (2 * w.N + 26) / 1e9, single_thread_value=n * reps1 / spent1,
                sample=f"first {n} params of {w.name} (N={w.N}), {reps} oracle steps in {spent:.1f} s on "
                       f"{threads} threads of {cores} cores; {reps1} steps in {spent1:.1f} s on one thread")


def offload_breakdown(zs, torch, d, w, n, chunk) -> dict:
    """Rates of the offload step's parts, each timed alone: the host AdamW over the whole shard (it reads
    the fp32 mean gradient, master, m, v and writes master, m, v and the bf16 copy: 30 B/param of host
    memory traffic) and one chunk's fp32 gradient copy to pinned memory and bf16 copy back."""
    threads = min(16, len(os.sched_getaffinity(0)))
    n = d["P"].numel()
    g = torch.full((n,), 1e-3, dtype=torch.float32)
    b = torch.empty(n, dtype=torch.int16)
    t0 = time.perf_counter()
    zs.cpu_adam(g, d["P"], d["M"], d["V"], b, w.hp(), w.step + 10_000, threads)
    host_s = time.perf_counter() - t0
    del g, b
    k = min(chunk, n)
    dg = torch.empty(k, dtype=torch.float32, device="cuda")
    db = torch.empty(k, dtype=torch.int16, device="cuda")
    hg = torch.empty(k, dtype=torch.float32).pin_memory()
    hb = torch.empty(k, dtype=torch.int16).pin_memory()
    rates = {}
    for name, dst, src in (("d2h", hg, dg), ("h2d", db, hb)):
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        rates[name] = 10 * src.numel() * src.element_size() / (e0.elapsed_time(e1) / 1e3) / 1e9
    del dg, db, hg, hb
    return {"host_adam_params_per_s": n / host_s, "host_adam_GBps": 30 * n / host_s / 1e9, "host_threads": threads,
            "host_add_GBps": host_add_ceiling(torch, threads),
            "d2h_GBps": rates["d2h"], "h2d_GBps": rates["h2d"],
            "pcie_bytes_per_param": 6, "chunk_elems": k}


def host_add_ceiling(torch, threads: int, elems: int = 1 << 28, reps: int = 5) -> float:
    """Host memory ceiling for the host AdamW: torch's threaded c = a + b over 1 GiB fp32 arrays,
    counted as 12 B per element (two reads, one write), best of ``reps``."""
    prev = torch.get_num_threads()
    torch.set_num_threads(threads)
    try:
        a = torch.rand(elems)
        b = torch.rand(elems)
        c = torch.empty(elems)
        best = float("inf")
        for _ in range(reps):
            t0 = time.perf_counter()
            torch.add(a, b, out=c)
            best = min(best, time.perf_counter() - t0)
        return 12 * elems / best / 1e9
    finally:
        torch.set_num_threads(prev)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="flat-70b", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle baseline budget (0 = skip)")
    ap.add_argument("--no-copy", action="store_true", help="skip the copy-kernel and access-pattern ceilings")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the step itself: no other schedules, per-pass times, flat reference or "
                         "window-less rerun (for profiler runs that count launches per step)")
    ap.add_argument("--blocks", type=int, default=0, help="workgroups per launch (0 = library default)")
    ap.add_argument("--path", default="fused", choices=["fused", "clip", "fp16", "offload"],
                    help="fused: the one-pass step; clip: two-pass with global-norm clipping (max_norm 1); "
                         "fp16: two-pass with fp16 replicas, loss scale 2^16, clipping and an fp16 working copy; "
                         "offload: fp32 state in host memory, AdamW on the CPU, reduction on the GPU")
    ap.add_argument("--offload-chunk", type=int, default=1 << 26, help="parameters per offload pipeline chunk")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library runs one rank's shard step on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import sharded_mixed_precision_rank_amd as zs
    from synth import workloads as W

    w = workload(args.workload)
    zs.set_grid_blocks(args.blocks)
    log(f"workload {w.name}: {w.n_params} params, N={w.N}, step={w.step}, wd={w.weight_decay}")
    t0 = time.perf_counter()
    d = W.device_inputs(w)
    torch.cuda.synchronize()
    log(f"inputs drawn in device memory in {time.perf_counter() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 1e9:.1f} GB)")

    two_pass = args.path in ("clip", "fp16")
    offload = None
    if args.path == "offload":
        if w.is_list:
            print("the offload path runs on flat shards", file=sys.stderr)
            return 2
        threads = min(16, len(os.sched_getaffinity(0)))
        for k in "PMV":   # the fp32 state moves to pinned host memory
            d[k] = d[k].cpu().pin_memory()
        torch.cuda.empty_cache()
        offload = zs.Offload(args.offload_chunk, threads)
        log(f"offload: host state {3 * 4 * d['arena_len'] / 1e9:.1f} GB pinned, {threads} CPU threads, "
            f"chunk {args.offload_chunk}")
    if two_pass and w.is_list:
        print("the two-pass paths run on flat shards", file=sys.stderr)
        return 2
    loss_scale = 2.0 ** 16 if args.path == "fp16" else 1.0
    gfmt = "fp16" if args.path == "fp16" else "bf16"
    if args.path == "fp16":
        # fp16 replicas: the same seeded draws times the loss scale, rounded to fp16 (input preparation)
        import synth

        k = w.keys()
        tmp = torch.empty(d["arena_len"], dtype=torch.float32, device="cuda")
        for r in range(w.N):
            synth.dev_fill_normal_f32(tmp, k["G"][r], 0, w.g_sigma * loss_scale)
            d["G"][r] = tmp.half()
        del tmp
        d["B"] = torch.zeros(d["arena_len"], dtype=torch.float16, device="cuda")
    ws = sqn = None
    if two_pass:
        ws = torch.empty(zs.two_pass_workspace_bytes(d["arena_len"]), dtype=torch.uint8, device="cuda")
        sqn = torch.empty(1, dtype=torch.float64, device="cuda")

    plan = None
    if w.is_list:
        offs, _ = w.layout()
        plan = zs.ListPlan.from_arenas(w.sizes, offs, d["G"], d["P"], d["M"], d["V"], d["B"])

    def step(t):
        if plan is not None:
            plan.step(w.hp(), t)
        elif offload is not None:
            offload.step(d["G"], d["P"], d["M"], d["V"], d["B"], w.hp(), t)
        elif two_pass:
            zs.clipped_step_flat(d["G"], d["P"], d["M"], d["V"], d["B"], w.hp(), t, max_norm=1.0,
                                 loss_scale=loss_scale, grad_format=gfmt, param_format=gfmt, workspace=ws, sqnorm=sqn)
        else:
            zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], w.hp(), t)

    for k in range(args.warmup):
        step(w.step + k)
    torch.cuda.synchronize()
    # one event between consecutive steps: the K-step total gives the mean, the gaps the median and minimum
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record()
    for k in range(args.steps):
        step(w.step + args.warmup + k)
        ev[k + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps))
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    ms_min = per_step[0]
    cold_ms = None
    footprint = sum(t.numel() * t.element_size() for t in (*d["G"], d["P"], d["M"], d["V"], d["B"]) if t.is_cuda)
    if offload is None and footprint < (1 << 30):
        # the workload fits in the 256 MB Infinity Cache: also time each step after a 1 GB scratch write
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cold = []
        for k in range(10):
            scratch.fill_(k)
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            step(w.step + args.warmup + args.steps + k)
            c1.record()
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1))
        del scratch
        cold_ms = sorted(cold)[len(cold) // 2]
        log(f"cold (after a 1 GB scratch write): {cold_ms:.4f} ms/step, median of 10")
    n = w.n_params
    bpp = 2 * w.N + (34 if two_pass else 26)   # offload: the same algorithmic bytes as the fused step
    bytes_per_step = bpp * n
    achieved = bytes_per_step / (ms / 1e3) / 1e9
    log(f"{ms:.3f} ms/step, {n / (ms / 1e3) / 1e9:.2f} G params/s, {achieved:.0f} GB/s "
        f"(per step: median {ms_median:.3f} ms, min {ms_min:.3f} ms)")

    # the flat step's schedule and the write window the step took (0, 0: none), and so the kernel that ran;
    # a list plan takes the flat step's windows, by its total parameter count
    flat_fused = offload is None and not two_pass and not w.is_list
    sched = zs.flat_schedule(w.N, n) if flat_fused else None
    window = (0, 0) if offload is not None else zs.write_window(
        "reduce" if two_pass else "list" if w.is_list else "flat", w.N, n)

    def median_ms_of(fn, t0: int, k: int = 5) -> float:
        fn(t0)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
        e[0].record()
        for j in range(k):
            fn(t0 + 1 + j)
            e[j + 1].record()
        torch.cuda.synchronize()
        return sorted(e[j].elapsed_time(e[j + 1]) for j in range(k))[k // 2]

    def median_ms(k: int = 5) -> float:
        return median_ms_of(step, w.step, k)

    unwindowed = None
    other_schedules = None
    passes = None
    flat_reference = None
    if two_pass and offload is None and not args.no_extras:
        # each pass on its own, in this process: pass 1 (2N read, 4 written per parameter, and the norm) and
        # pass 2 (16 read, 14 written), against the algorithmic bytes of each
        gfmt_ = "fp16" if args.path == "fp16" else "bf16"

        def pass_ms(fn, k: int = 5) -> float:
            fn()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
            e[0].record()
            for j in range(k):
                fn()
                e[j + 1].record()
            torch.cuda.synchronize()
            return sorted(e[j].elapsed_time(e[j + 1]) for j in range(k))[k // 2]

        p1 = pass_ms(lambda: zs.reduce_grads_flat(d["G"], ws, sqn, loss_scale, gfmt_))
        p2 = pass_ms(lambda: zs.adam_from_grads_flat(ws, n, d["P"], d["M"], d["V"], d["B"], w.hp(), w.step, sqn,
                                                     1.0, gfmt_))
        passes = {"pass1_ms": p1, "pass1_GBps": (2 * w.N + 4) * n / (p1 / 1e3) / 1e9,
                  "pass2_ms": p2, "pass2_GBps": 30 * n / (p2 / 1e3) / 1e9,
                  "pass1_schedule": zs.reduce_schedule(w.N, n)}
        log(f"pass 1 ({passes['pass1_schedule']}): {p1:.3f} ms, {passes['pass1_GBps']:.0f} GB/s; "
            f"pass 2: {p2:.3f} ms, {passes['pass2_GBps']:.0f} GB/s (medians of 5)")
    if w.is_list and plan is not None and not args.no_extras:
        # one flat call over the list's whole arena (its gaps included), in this process: what the list's
        # per-tensor structure costs
        L = d["P"].numel()
        fm = median_ms_of(lambda t: zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], w.hp(), t), w.step)
        flat_reference = {"ms_per_step_median": fm, "arena_params": L, "list_over_flat": ms_median / (fm * n / L)}
        log(f"one flat call over the arena: {fm:.3f} ms ({fm * n / L:.3f} ms for the list's parameters); "
            f"the list takes {100 * (flat_reference['list_over_flat'] - 1):+.2f}%")
    if flat_fused and not args.no_extras:
        # the same steps on the flat step's other schedules, in this process: what the schedule is worth
        other_schedules = {}
        for other in ("phased", "windowed", "stream"):
            if other == sched:
                continue
            zs.set_flat_schedule(other)
            if zs.flat_schedule(w.N, n) == other:
                other_schedules[other] = {"ms_per_step_median": median_ms(), "steps": 5}
                log(f"{other} schedule: {other_schedules[other]['ms_per_step_median']:.3f} ms/step (median of 5)")
        zs.set_flat_schedule("auto")
    elif window[0] and not args.no_extras:
        # the same steps with the windows switched off, in this process: the windows' own effect
        zs.set_write_window(1)
        unwindowed = {"ms_per_step_median": median_ms(), "steps": 5}
        zs.set_write_window(0)
        log(f"without write windows: {unwindowed['ms_per_step_median']:.3f} ms/step (median of 5)")
    tn = f"<{w.N}>" if w.N in (1, 2, 4, 8, 16, 32, 64) else "<0>"
    if w.is_list:
        lsched = zs.flat_schedule(w.N, n)   # a list plan takes the schedule of a flat shard of its size
        kernel = ("list_phased_kernel" + (tn if w.N == 64 else "<0>") if lsched == "phased" else
                  ("list_window_kernel" if window[0] else "list_kernel") + tn)
    elif two_pass:
        p1s = zs.reduce_schedule(w.N, n)
        kernel = ("reduce_phased_kernel" + (tn if w.N == 64 else "<0>") if p1s == "phased" else
                  ("reduce_window_kernel" if window[0] else "reduce_kernel") + tn) + " + gbar_kernel"
    elif sched == "phased":
        kernel = "flat_phased_kernel" + (tn if w.N == 64 else "<0>")
    else:
        kernel = ("flat_window_kernel" if window[0] else "flat_kernel") + tn
    pattern = None
    if args.path == "fused" and not w.is_list and not args.no_copy and footprint >= (1 << 30):
        pattern = pattern_ceiling(w, d, window, phased=sched == "phased")
        if pattern:
            own = ("read_write_phased_GBps" if sched == "phased" and "read_write_phased_GBps" in pattern else
                   "read_write_windowed_GBps" if window[0] else "read_write_GBps")
            same = pattern[own]
            pattern["kernel_frac_of_read_write"] = achieved / same
            pattern["kernel_pattern"] = own[:-5]
            log(f"access-pattern ceiling without arithmetic: reads alone {pattern['read_GBps']:.0f} GB/s, "
                f"reads+writes stored per tile {pattern['read_write_GBps']:.0f} GB/s"
                + (f", with the step's write windows {same:.0f} GB/s" if window[0] else "")
                + (f", on the step's phased schedule {same:.0f} GB/s" if own == "read_write_phased_GBps" else "")
                + f"; the step reaches {100 * pattern['kernel_frac_of_read_write']:.1f}% of the pattern with "
                  f"its own schedule")
    offload_parts = None
    if offload is not None:
        offload.close()
        offload_parts = offload_breakdown(zs, torch, d, w, n, args.offload_chunk)
        log(f"offload parts: {offload_parts}")
    del d, plan
    torch.cuda.empty_cache()
    ceiling = None if args.no_copy else copy_ceiling()
    if ceiling:
        log(f"copy-kernel ceiling {ceiling:.0f} GB/s")
    traffic = counter_traffic(w, kernel.split("<")[0]) if args.path == "fused" else None
    base = cpu_baseline(w, args.cpu_seconds) if args.cpu_seconds > 0 else None
    if base:
        log(f"cpu baseline {base['value'] / 1e6:.1f} M params/s ({base['sample']})")

    rec = {
        "metric": METRIC, "value": n / (ms / 1e3), "unit": "params/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "ms_per_step_median": ms_median, "ms_per_step_min": ms_min,
        "cold_ms_per_step": cold_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "n_params": n, "replicas": w.N, "adam_step": w.step,
                   "weight_decay": w.weight_decay, "path": args.path,
                   "schedule": sched if not w.is_list else zs.flat_schedule(w.N, n),
                   "write_window_ticks": list(window) if window[0] else None,
                   "max_bytes_per_launch": zs.launch_bytes(),
                   "storage": ("fp16" if args.path == "fp16" else "bf16") + " grads and working copy, fp32 master/m/v"},
        "hbm_GBps": achieved, "hbm_frac_of_peak": achieved / HBM_PEAK_GBPS,
        "copy_ceiling_GBps": ceiling,
        "pattern_ceiling": pattern,
        "without_write_windows": unwindowed,
        "other_schedules": other_schedules,
        "passes": passes,
        "flat_reference": flat_reference,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic if args.path == "fused" else None,
                     "bytes_per_param": bpp, "kernel": kernel},
        "cpu_baseline": base,
    }
    if offload_parts:
        # the offload step is bound by the host AdamW's memory traffic, not by HBM
        host_gbps = 30 * n / (ms / 1e3) / 1e9
        rec["roofline"] = {"bound": "host-memory", "achieved": host_gbps, "peak": offload_parts["host_add_GBps"],
                           "unit": "GB/s", "frac": host_gbps / offload_parts["host_add_GBps"], "traffic": None,
                           "bytes_per_param": 30, "kernel": "host AdamW (AVX2)"}
        rec["offload"] = offload_parts
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
