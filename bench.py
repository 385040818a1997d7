#!/usr/bin/env python3
"""Benchmark: FP32 GEMM C = A·B on one MI355X through the C ABI.

A step is one product over the workload (default: M = N = K = 4096,
row-major, A and B uniform on [-1, 1) from seed 2) with A, B and C resident in
HBM.  For the skinny workload, whose operands would fit in the 256 MiB
last-level cache, the steps rotate over three operand sets (``--buffers``).

Untimed launches first: a clock ramp of at least --warmup-seconds (0.3 s)
of launches, since an idle GPU needs tens of milliseconds of work to reach
its full clock, then the W counted warm-up steps (--warmup, default 10).
Then K timed steps bracketed by device synchronisation.  Every
--event-every-th launch of the timed steps, and more often when K is small
(at least min(10, K) of them), is also bracketed by a pair of HIP events on
the stream it is enqueued on (each pair adds a few microseconds between
kernels, so they are not put around every launch).  Right after the timed
steps a fixed-work FP32 matrix-core kernel (libsgemm_probe.so) reads the
clock the matrix pipes run at.  Prints one JSON line.

  value            2MNK * K / wall time of the K steps, TFLOP/s
  roofline         the GEMM kernel against the FP32 matrix peak (157.3
                   TFLOP/s): achieved = 2MNK / mean event-timed launch
  roofline.traffic HBM bytes per launch from the rocprofv3 FETCH_SIZE and
                   WRITE_SIZE counters recorded under profiles/, each scaled
                   by the factor a plain copy of known size gives, or null
                   when the kernel sources changed since they were taken
  config.clock     the probe's rate and the clock it implies (its matrix
                   instructions hold each SIMD's pipe a known number of
                   cycles), and the shader clock read from its counters
  cpu_baseline     the CPU oracle on a bounded row sample of the same product,
                   repeated for about --cpu-seconds; the same leg first
                   checks the GPU's C on those rows against the oracle
                   (max |C - Cref| / (|A|.|B|) <= 1e-5, else exit status 3)
                   and times the whole 256cube and ragged products on one
                   core

``--ladder`` runs every step of the ablation ladder (``sgemm_ladder``) on the
workload instead, one JSON line per step.

``--op sgemm_ws`` times ``sgemm_ws`` (K split across workgroups through a
workspace of ``sgemm_workspace_bytes``) on the workload, with the plain
``sgemm`` of the same shape beside it; the events bracket both of its kernels.

``--op vendor`` times ``sgemm`` and the vendor FP32 GEMM (``torch.matmul``,
hipBLASLt) side by side on a fixed list of shapes, as context: one JSON line
per shape, both under the same warm-up and operand rotation.

``--op kscan`` runs the product on the workload's M x N for each K of
``--ks`` (0 included: C = 0, the launch and the stores alone), --steps
launches each, one JSON line per K with the plan and the event-timed median:
with a kernel trace over it (bench_profile.py kscan) it separates a launch's
fixed cost from its cost per K slab.

``--copy-calibration`` instead runs a device-to-device copy of known size (for
the counter scale factors) and prints its size.  ``--op transpose`` measures
the tiled transpose instead (``--layout``; HBM-bound, GB/s against 8 TB/s,
rotating over ``--buffers`` input/output pairs so that no launch is served
from the last-level cache, with a plain copy of the same bytes beside it).
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

METRIC = "SGEMM TFLOP/s at M=N=K=4096 fp32 (1 GPU) and % of MI355X FP32 peak"
PEAK_FP32_TFLOPS = 157.3     # 256 CU x 2.4 GHz x 256 FP32 flop/clk (dense)
PEAK_HBM_GBS = 8000.0

WORKLOADS = {
    "4096cube": (4096, 4096, 4096, "uniform", 2),
    "256cube": (256, 256, 256, "uniform", 1),
    "ragged": (1000, 1500, 777, "uniform", 3),
    "skinny": (65536, 128, 256, "normal", 4),
    "8192cube": (8192, 8192, 8192, "normal", 5),
    # under-filled grids with a long K, for --op sgemm_ws (split K)
    "256x256x8192": (256, 256, 8192, "uniform", 6),
    "512x512x16384": (512, 512, 16384, "normal", 7),
    "1024x1024x8192": (1024, 1024, 8192, "uniform", 8),
    # one GPU's share of 4096^3 sharded eight ways along M
    "512x4096x4096": (512, 4096, 4096, "uniform", 9),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{kernel}_{workload}.txt")


def kernel_source_hash() -> str:
    """Digest of the code of the product GEMM kernels (device code only; not
    the transpose, not the ablation ladder's own kernels; comments and
    whitespace left out): the counters recorded under profiles/ stay valid
    while it is unchanged."""
    from tiled_fp32_gemm_amd import build
    h = hashlib.sha256()
    for p in build.sources():
        name = os.path.basename(p)
        if name == "common.hpp" or (name.startswith("kernel_")
                                    and "transpose" not in name
                                    and "ladder" not in name):
            text = open(p).read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(name.encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, src_hash: str):
    """Calibrated HBM bytes per launch from profiles/, if still current."""
    path = TRAFFIC_FILE.format(kernel=kernel, workload=workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_]+)\s*[:=]\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("source_hash") != src_hash or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


TOLERANCE = 1e-5   # |C - Cref| <= TOLERANCE * (|A|.|B|), elementwise


def cpu_baseline(A, B, M, N, K, rows: int, seconds: float, gpu_rows) -> tuple:
    """The CPU leg: the oracle on rows 0..rows-1 of the product.  Its first,
    untimed, run (with the magnitude sums |A|.|B|) is the reference that
    gpu_rows(rows) -- the GPU's C, rows 0..rows-1 -- is checked against; then
    the C-only run is repeated until `seconds` of CPU time have passed (at
    least once, at most 50 times) for the baseline figure.  Also times the
    whole 256cube and ragged products on one core.  Returns (baseline dict,
    check dict)."""
    import numpy as np

    import oracle
    import seedgen
    rows = min(rows, M)
    sub = A[:rows]
    Cref, T = oracle.gemm(sub, B, with_t=True)
    C = gpu_rows(rows).astype(np.float64)
    err = np.abs(C - Cref)
    with np.errstate(divide="ignore", invalid="ignore"):
        norm = np.where(T > 0, err / T, np.where(err > 0, np.inf, 0.0))
    worst = float(norm.max()) if norm.size else 0.0
    ok = bool(np.all(np.isfinite(C)) and worst <= TOLERANCE)
    check = {"rows": f"0..{rows - 1}", "elements": int(C.size),
             "max_err_norm": worst, "tolerance": TOLERANCE, "ok": ok}
    del Cref, T, C, err, norm
    reps, total = 0, 0.0
    while reps < 50 and (reps == 0 or total < seconds):
        t0 = time.perf_counter()
        oracle.gemm(sub, B, with_t=False)
        total += time.perf_counter() - t0
        reps += 1
    one_core = {}
    for name in ("256cube", "ragged"):
        m, n, k, dist, seed = WORKLOADS[name]
        a, b = seedgen.gemm_inputs(m, n, k, dist, seed)
        t0 = time.perf_counter()
        oracle.gemm(a, b, with_t=False, threads=1)
        dt = time.perf_counter() - t0
        one_core[name] = {"seconds": round(dt, 4),
                          "gflops": round(2.0 * m * n * k / dt / 1e9, 3)}
    base = {"value": round(2.0 * rows * N * K * reps / total / 1e12, 6),
            "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the {M}x{N}x{K} product "
                      f"(C only, fp64 accumulation), {reps} run(s) in "
                      f"{total:.2f} s",
            "one_core": one_core}
    return base, check


def clock_probe(stream, repeats: int = 5, iters: int = 2048) -> dict:
    """Runs the matrix-core clock probe `repeats` times between HIP events.
    Each SIMD's matrix pipe is busy for iters * MFMA_PER_ITER * (WAVES / 4) *
    MFMA_CYCLES cycles per launch, so cycles / median duration is the clock
    the matrix pipes ran at; the probe's own counters (clock64 against the
    constant-rate wall_clock64) give a second reading."""
    import numpy as np
    import torch

    from tiled_fp32_gemm_amd import probe
    words = probe.STAMP_WORDS * probe.WORKGROUPS
    stamps = torch.zeros(words, dtype=torch.int64, device="cuda:0")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(repeats)]
    for a, b in evs:
        a.record(stream)
        st = probe.mfma_clock(stream.cuda_stream, iters, stamps.data_ptr())
        b.record(stream)
        if st != 0:
            raise RuntimeError(f"clock probe launch failed (status {st})")
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    cycles = iters * probe.MFMA_PER_ITER * (probe.WAVES // 4) * probe.MFMA_CYCLES
    flops = (probe.WORKGROUPS * probe.WAVES * iters * probe.MFMA_PER_ITER
             * 32 * 32 * 2 * 2)
    v = probe.versions()
    st = stamps.view(probe.WORKGROUPS, probe.STAMP_WORDS).cpu().numpy().astype(np.float64)
    dw = st[:, 3] - st[:, 1]
    counter_mhz = (float(np.median((st[:, 2] - st[:, 0]) / dw)) * v["wall_clock_khz"] / 1e3
                   if np.all(dw > 0) else None)
    return {"probe_ms": round(ms, 5),
            "probe_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_clock_ghz": round(cycles / (ms * 1e-3) / 1e9, 4),
            "clock64_mhz": None if counter_mhz is None else round(counter_mhz, 1),
            "wall_clock_khz": v["wall_clock_khz"]}


def versions() -> dict:
    """ROCm, HIP runtime and driver, and torch versions of this run."""
    import torch

    from tiled_fp32_gemm_amd import probe
    out = {"torch": torch.__version__, "torch_hip": torch.version.hip}
    try:
        out["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        out["rocm"] = None
    v = probe.versions()
    out["hip_runtime"] = v["hip_runtime"]
    out["hip_driver"] = v["hip_driver"]
    try:
        out["amdgpu_module"] = open("/sys/module/amdgpu/version").read().strip()
    except OSError:
        out["amdgpu_module"] = None
    return out


def copy_calibration(nbytes: int) -> None:
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0")
    src.uniform_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}), flush=True)


def bench_transpose(args) -> int:
    """out = in^T on a rows x cols matrix: bytes moved = 2 * 4 * rows * cols."""
    import numpy as np
    import torch

    import tiled_fp32_gemm_amd as sg
    sg.load()
    rows, cols = args.rows, args.cols
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    # Launch i uses buffer pair i mod n: with n pairs spanning more than the
    # 256 MiB last-level cache, every launch reads and writes HBM.
    n = max(1, 4 if args.buffers is None else args.buffers)
    tins = [torch.rand((rows, cols), device=dev, generator=g) for _ in range(n)]
    touts = [torch.empty((cols, rows), device=dev) for _ in range(n)]
    stream = torch.cuda.current_stream(dev)
    code = sg.TRANSPOSE_LAYOUTS[args.layout]

    def step(i):
        st = sg.sgemm_transpose_ex(rows, cols, tins[i % n].data_ptr(), cols,
                                   touts[i % n].data_ptr(), rows,
                                   stream.cuda_stream, code)
        if st != sg.OK:
            raise sg.SgemmError(st, "sgemm_transpose_ex")

    def timed(fn):
        timed.nwarm = warm_up(fn, args)[0]
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            starts[i].record(stream)
            fn(i)
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])

    wall, ev_ms = timed(step)
    nwarm = timed.nwarm
    # Context: a device-to-device copy of the same bytes over the same buffers.
    _, copy_ms = timed(lambda i: touts[i % n].view(-1).copy_(tins[i % n].view(-1)))
    nbytes = 2.0 * 4 * rows * cols
    achieved = nbytes / (float(ev_ms.mean()) / 1e3) / 1e9
    copy_gbs = nbytes / (float(copy_ms.mean()) / 1e3) / 1e9
    print(json.dumps({
        "metric": "tiled transpose GB/s (fp32, 1 GPU)",
        "value": round(nbytes * args.steps / wall / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": nwarm,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"transpose {rows}x{cols} fp32, layout {args.layout}",
                   "buffer_pairs": n,
                   "kernel_ms_median": round(float(np.median(ev_ms)), 5),
                   "copy_same_bytes_gbs": round(copy_gbs, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None},
        "cpu_baseline": None}), flush=True)
    return 0


def warm_up(fn, args) -> tuple:
    """Untimed launches fn(0), fn(1), ...: first a clock ramp, in synchronised
    batches of 10, of at least 20 launches and at least --warmup-seconds (an
    idle GPU takes tens of milliseconds of work to reach its full clock),
    then the counted warm-up steps, --warmup of them (default 10).  Returns
    (counted steps, ramp seconds, ramp launches)."""
    import torch
    ramp, t0 = 0, time.perf_counter()
    while ramp < 20 or time.perf_counter() - t0 < args.warmup_seconds:
        for _ in range(10):
            fn(ramp)
            ramp += 1
        torch.cuda.synchronize()
    ramp_s = time.perf_counter() - t0
    w = 10 if args.warmup is None else args.warmup
    for i in range(w):
        fn(ramp + i)
    torch.cuda.synchronize()
    return w, ramp_s, ramp


def event_stride(steps: int, every: int) -> int:
    """Every how many timed steps one is event-timed: --event-every, lowered
    so that at least min(10, steps) launches are."""
    return max(1, min(every, steps // 10))


def timed_steps(step, args, stream):
    """Warms up (warm_up), then runs --steps timed steps between two device
    synchronisations, every event_stride()-th also between two HIP events on
    stream.  Returns (wall seconds, event-timed milliseconds of the sampled
    steps, warm_up's result)."""
    import numpy as np
    import torch
    warm = warm_up(lambda i: step(), args)
    steps = args.steps
    every = event_stride(steps, args.event_every)
    timed = [i for i in range(steps) if i % every == every // 2] or [0]
    starts = {i: torch.cuda.Event(enable_timing=True) for i in timed}
    ends = {i: torch.cuda.Event(enable_timing=True) for i in timed}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i in starts:
            starts[i].record(stream)
            step()
            ends[i].record(stream)
        else:
            step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, np.array([starts[i].elapsed_time(ends[i]) for i in timed]), warm


def bench_ws(args) -> int:
    """sgemm_ws on the workload (two kernels per step: the partial products of
    the K splits, then their fixed-order sum), with plain sgemm beside it."""
    import numpy as np
    import torch

    import seedgen
    import tiled_fp32_gemm_amd as sg
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    sg.load()
    M, N, K, dist, seed = WORKLOADS[args.workload]
    A, B = seedgen.gemm_inputs(M, N, K, dist, seed)
    dev = torch.device("cuda:0")
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    tC = torch.empty((M, N), dtype=torch.float32, device=dev)
    need = sg.sgemm_workspace_bytes(M, N, K)
    ws = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=dev)
    st, plan = sg.sgemm_plan_query_ws(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N,
                                      tC.data_ptr(), N, need)
    if st != sg.OK:
        raise sg.SgemmError(st, "sgemm_plan_query_ws")
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def step_ws():
        st = sg.sgemm_ws(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N, tC.data_ptr(),
                         N, sh, ws.data_ptr(), need)
        if st != sg.OK:
            raise sg.SgemmError(st, "sgemm_ws")

    def step_plain():
        st = sg.sgemm(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N, tC.data_ptr(), N, sh)
        if st != sg.OK:
            raise sg.SgemmError(st, "sgemm")

    wall, ev_ms, warm = timed_steps(step_ws, args, stream)
    nwarm = warm[0]
    wall_p, ev_p, _ = timed_steps(step_plain, args, stream)
    flops = 2.0 * M * N * K
    achieved = flops / (float(ev_ms.mean()) / 1e3) / 1e12
    print(json.dumps({
        "metric": "SGEMM TFLOP/s with K split across workgroups (fp32, 1 GPU)",
        "value": round(flops * args.steps / wall / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": nwarm,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"sgemm_ws {args.workload}: C=A·B, M={M} N={N} "
                               f"K={K}, row-major fp32, A,B {dist} seed {seed}",
                   "M": M, "N": N, "K": K, "kernel": plan.kernel.decode(),
                   "splits": plan.splits, "workspace_bytes": plan.workspace_bytes,
                   "workgroups": plan.workgroups, "threads": plan.threads,
                   "device": torch.cuda.get_device_name(dev),
                   "source_hash": kernel_source_hash(),
                   "event_timed_launches": len(ev_ms),
                   "call_ms_median": round(float(np.median(ev_ms)), 5),
                   "sgemm_same_shape_tflops": round(flops * args.steps / wall_p / 1e12, 3),
                   "sgemm_same_shape_ms_median": round(float(np.median(ev_p)), 5)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                     "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP32_TFLOPS, 4), "traffic": None},
        "cpu_baseline": None}), flush=True)
    return 0


# Shapes for --op vendor: the five workloads, squares, tall, wide, short-K,
# long-K and ragged shapes.
VENDOR_SHAPES = [(256, 256, 256), (512, 512, 512), (1024, 1024, 1024),
                 (2048, 2048, 2048), (3072, 3072, 3072), (4096, 4096, 4096),
                 (6144, 6144, 6144), (8192, 8192, 8192), (1000, 1500, 777),
                 (65536, 128, 256), (16384, 256, 1024), (128, 16384, 1024),
                 (32768, 512, 512), (4096, 4096, 128), (8192, 8192, 256),
                 (256, 256, 16384), (512, 512, 8192), (1024, 1024, 8192),
                 (512, 4096, 4096), (4096, 512, 4096), (3000, 2000, 1111),
                 (777, 777, 777), (5000, 5000, 300), (12288, 12288, 1024)]


def bench_vendor(args) -> int:
    """sgemm against torch.matmul (the vendor library) on VENDOR_SHAPES."""
    import numpy as np
    import torch

    import tiled_fp32_gemm_amd as sg
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    sg.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    shapes = VENDOR_SHAPES
    if args.shapes:
        shapes = [tuple(int(v) for v in sh.split("x")) for sh in args.shapes.split(",")]
    for M, N, K in shapes:
        # operand sets enough to exceed the 256 MiB last-level cache twice
        nbytes = 4 * (M * K + K * N + M * N)
        nsets = max(1, min(64, -(-(512 << 20) // nbytes)))
        sets = [(torch.rand((M, K), device=dev, generator=g) * 2 - 1,
                 torch.rand((K, N), device=dev, generator=g) * 2 - 1,
                 torch.empty((M, N), device=dev)) for _ in range(nsets)]
        ptrs = [(a.data_ptr(), b.data_ptr(), c.data_ptr()) for a, b, c in sets]
        cnt = [0, 0]

        def ours():
            pa, pb, pc = ptrs[cnt[0] % nsets]
            cnt[0] += 1
            st = sg.sgemm(M, N, K, pa, K, pb, N, pc, N, sh)
            if st != sg.OK:
                raise sg.SgemmError(st, "sgemm")

        def vendor():
            a, b, c = sets[cnt[1] % nsets]
            cnt[1] += 1
            torch.matmul(a, b, out=c)

        need = sg.sgemm_workspace_bytes(M, N, K)
        ws = torch.empty(max(need // 4, 1), device=dev)

        def ours_ws():
            pa, pb, pc = ptrs[cnt[0] % nsets]
            cnt[0] += 1
            st = sg.sgemm_ws(M, N, K, pa, K, pb, N, pc, N, sh, ws.data_ptr(), need)
            if st != sg.OK:
                raise sg.SgemmError(st, "sgemm_ws")

        flops = 2.0 * M * N * K
        wall, ev, _ = timed_steps(ours, args, stream)
        wall_v, ev_v, _ = timed_steps(vendor, args, stream)
        # sgemm_ws is sgemm itself where the planner takes no split
        wall_w = timed_steps(ours_ws, args, stream)[0] if need > 0 else wall
        st, plan = sg.sgemm_plan_query(M, N, K, ptrs[0][0], K, ptrs[0][1], N,
                                       ptrs[0][2], N, 0)
        print(json.dumps({
            "metric": "SGEMM TFLOP/s against the vendor library (fp32, 1 GPU)",
            "M": M, "N": N, "K": K, "operand_sets": nsets,
            "kernel": plan.kernel.decode(), "steps": args.steps,
            "sgemm_tflops": round(flops * args.steps / wall / 1e12, 2),
            "vendor_tflops": round(flops * args.steps / wall_v / 1e12, 2),
            "sgemm_ws_tflops": round(flops * args.steps / wall_w / 1e12, 2),
            "ws_splits": sg.sgemm_plan_query_ws(M, N, K, ptrs[0][0], K, ptrs[0][1], N,
                                                ptrs[0][2], N, need)[1].splits,
            "sgemm_event_ms_median": round(float(np.median(ev)), 5),
            "vendor_event_ms_median": round(float(np.median(ev_v)), 5)}),
            flush=True)
        del sets, ws
    return 0


def bench_ladder(args) -> int:
    """Every ablation ladder step (sgemm_ladder) on the workload: one JSON
    line per step, in ladder order."""
    import numpy as np
    import torch

    import seedgen
    import tiled_fp32_gemm_amd as sg
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    sg.load()
    M, N, K, dist, seed = WORKLOADS[args.workload]
    A, B = seedgen.gemm_inputs(M, N, K, dist, seed)
    dev = torch.device("cuda:0")
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    tC = torch.empty((M, N), dtype=torch.float32, device=dev)
    ref = torch.empty_like(tC)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    st = sg.sgemm(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N, ref.data_ptr(), N, sh)
    if st != sg.OK:
        raise sg.SgemmError(st, "sgemm")
    flops = 2.0 * M * N * K
    for step, name in enumerate(sg.ladder_steps()):
        def run():
            st = sg.sgemm_ladder(step, M, N, K, tA.data_ptr(), K, tB.data_ptr(), N,
                                 tC.data_ptr(), N, sh)
            if st != sg.OK:
                raise sg.SgemmError(st, "sgemm_ladder")
        nwarm, _, ramp_n = warm_up(lambda i: run(), args)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            starts[i].record(stream)
            run()
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev_ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
        # every step computes the same product: compare with the product path
        rel = float((tC - ref).abs().max() / ref.abs().max())
        achieved = flops / (float(ev_ms.mean()) / 1e3) / 1e12
        print(json.dumps({
            "metric": "ablation ladder step TFLOP/s (fp32, 1 GPU)",
            "value": round(flops * args.steps / wall / 1e12, 3), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": nwarm,
            "ms_per_step": round(wall / args.steps * 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"sgemm {args.workload}: M={M} N={N} K={K}",
                       "ladder_step": step, "name": name,
                       "clock_ramp_launches": ramp_n,
                       "kernel_ms_median": round(float(np.median(ev_ms)), 5),
                       "max_rel_diff_vs_sgemm": rel},
            "roofline": {"bound": "mfma" if name.startswith("mfma") else "alu",
                         "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS,
                         "unit": "TFLOP/s",
                         "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
                         "traffic": None},
            "cpu_baseline": None}), flush=True)
    return 0


def bench_kscan(args) -> int:
    """The product kernel on the workload's M x N at each K of --ks."""
    import numpy as np
    import torch

    import seedgen
    import tiled_fp32_gemm_amd as sg
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    sg.load()
    M, N, K0, dist, seed = WORKLOADS[args.workload]
    # By default K0 +- multiples of 32 (same partial last slab, so the planner
    # keeps the workload's tile), and 0.
    ks = [int(k) for k in args.ks.split(",")] if args.ks else sorted(
        {0} | {k for k in (K0 + 32 * j for j in range(-64, 48, 4)) if 0 < k <= 2 * K0 + 512})
    kmax = max(max(ks), 1)
    A, B = seedgen.gemm_inputs(M, N, kmax, dist, seed)
    dev = torch.device("cuda:0")
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    tC = torch.empty((M, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for K in ks:
        def step():
            st = sg.sgemm(M, N, K, tA.data_ptr(), kmax, tB.data_ptr(), N, tC.data_ptr(), N,
                          stream.cuda_stream)
            if st != sg.OK:
                raise sg.SgemmError(st, "sgemm")
        wall, ev_ms, warm = timed_steps(step, args, stream)
        st, plan = sg.sgemm_plan_query(M, N, K, tA.data_ptr(), kmax, tB.data_ptr(), N,
                                       tC.data_ptr(), N, 0)
        print(json.dumps({"metric": "kscan", "M": M, "N": N, "K": K,
                          "kernel": plan.kernel.decode(), "tile_k": plan.tile_k,
                          "workgroups": plan.workgroups, "steps": args.steps,
                          "warmup": warm[0], "clock_ramp_launches": warm[2],
                          "event_ms_median": round(float(np.median(ev_ms)), 5)}),
              flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=None,
                    help="counted untimed steps after the clock ramp (default 10)")
    ap.add_argument("--warmup-seconds", type=float, default=0.3,
                    help="clock ramp before the warm-up steps: launches for at "
                         "least this long (and at least 20)")
    ap.add_argument("--workload", default="4096cube", choices=sorted(WORKLOADS))
    ap.add_argument("--algo", default="auto", choices=["auto", "mfma", "fma", "simple"])
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows of the product the CPU oracle computes")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle sample until this much time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=10, metavar="N",
                    help="time every N-th launch of the timed steps with HIP "
                         "events (lowered so that at least min(10, steps) are)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--shapes", default=None,
                    help="--op vendor: comma-separated MxNxK list instead of the built-in one")
    ap.add_argument("--op", default="sgemm",
                    choices=["sgemm", "sgemm_ws", "transpose", "vendor", "kscan"])
    ap.add_argument("--ks", default=None,
                    help="--op kscan: comma-separated K values (default: 0 to 2048 "
                         "around the workload's K)")
    ap.add_argument("--ladder", action="store_true",
                    help="run every ablation ladder step on the workload")
    ap.add_argument("--layout", default="auto",
                    choices=["auto", "naive", "padded", "swizzled"])
    ap.add_argument("--buffers", type=int, default=None,
                    help="operand sets the launches rotate over (transpose: "
                         "4 pairs; sgemm: 3 for skinny, whose set is smaller "
                         "than the 256 MiB last-level cache, else 1)")
    ap.add_argument("--rows", type=int, default=8192)
    ap.add_argument("--cols", type=int, default=8192)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the benchmark "
              "runs the kernel on one GPU (one GPU's share of a sharded "
              "product is the same kernel at a smaller shape)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import seedgen
    import tiled_fp32_gemm_amd as sg

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return 0
    if args.op == "transpose":
        return bench_transpose(args)
    if args.op == "sgemm_ws":
        return bench_ws(args)
    if args.op == "vendor":
        return bench_vendor(args)
    if args.op == "kscan":
        return bench_kscan(args)
    if args.ladder:
        return bench_ladder(args)

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    sg.load()   # raises if the HIP library is missing: there is no fallback

    M, N, K, dist, seed = WORKLOADS[args.workload]
    A, B = seedgen.gemm_inputs(M, N, K, dist, seed)
    dev = torch.device("cuda:0")
    # Step i uses operand set i mod n.  Set 0 holds the seeded inputs; the
    # others are copies at other addresses, so that with n sets spanning more
    # than the last-level cache no launch finds its operands there.
    nsets = args.buffers if args.buffers is not None else (
        3 if args.workload == "skinny" else 1)
    nsets = max(1, nsets)
    tA = torch.from_numpy(A).to(dev)
    tB = torch.from_numpy(B).to(dev)
    sets = [(tA, tB, torch.empty((M, N), dtype=torch.float32, device=dev))]
    for _ in range(nsets - 1):
        sets.append((tA.clone(), tB.clone(), torch.empty_like(sets[0][2])))
    tC = sets[0][2]
    algo = sg.ALGOS[args.algo]
    plan = sg.plan(tA, tB, tC, algo)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    ptrs = [(a.data_ptr(), b.data_ptr(), c.data_ptr()) for a, b, c in sets]
    counter = [0]

    def step():
        pa, pb, pc = ptrs[counter[0] % nsets]
        counter[0] += 1
        st = sg.sgemm_ex(M, N, K, pa, K, pb, N, pc, N, sh, algo)
        if st != sg.OK:
            raise sg.SgemmError(st, "sgemm_ex")

    wall, ev_ms, (nwarm, ramp_s, ramp_n) = timed_steps(step, args, stream)
    clock = clock_probe(stream)

    flops = 2.0 * M * N * K
    value = flops * args.steps / wall / 1e12
    kern_s = float(ev_ms.mean()) / 1e3
    achieved = flops / kern_s / 1e12
    src_hash = kernel_source_hash()
    traffic = read_traffic(plan["kernel"], args.workload, src_hash)
    compulsory = 4.0 * (M * K + K * N + M * N)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"sgemm {args.workload}: C=A·B, M={M} N={N} K={K}, "
                        f"row-major fp32, A,B {dist} seed {seed}",
            "M": M, "N": N, "K": K, "algo": args.algo,
            "kernel": plan["kernel"], "tile": [plan["tile_m"], plan["tile_n"],
                                                plan["tile_k"]],
            "workgroups": plan["workgroups"],
            "operand_sets": nsets,
            "pct_of_fp32_peak": round(100.0 * value / PEAK_FP32_TFLOPS, 2),
            "compulsory_hbm_gbs": round(compulsory / kern_s / 1e9, 1),
            "compulsory_pct_of_hbm_peak": round(100.0 * compulsory / kern_s / 1e9
                                                / PEAK_HBM_GBS, 2),
            # the counted HBM bytes (roofline.traffic) over the same time
            "traffic_hbm_gbs": (round(traffic / kern_s / 1e9, 1)
                                if traffic is not None else None),
            "traffic_pct_of_hbm_peak": (round(100.0 * traffic / kern_s / 1e9
                                              / PEAK_HBM_GBS, 2)
                                        if traffic is not None else None),
            "event_timed_launches": len(ev_ms),
            "kernel_ms_median": round(float(np.median(ev_ms)), 5),
            "kernel_ms_p10_p90": [round(float(np.percentile(ev_ms, 10)), 5),
                                  round(float(np.percentile(ev_ms, 90)), 5)],
            "source_hash": src_hash,
            "device": torch.cuda.get_device_name(dev),
            "arch": torch.cuda.get_device_properties(dev).gcnArchName,
            "clock_ramp_s": round(ramp_s, 3),
            "clock_ramp_launches": ramp_n,
            "clock": clock,
            "inputs_sha256": seedgen.sha256_of(A, B),
            "versions": versions(),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    status = 0
    if not args.no_cpu_baseline:
        out["cpu_baseline"], check = cpu_baseline(
            A, B, M, N, K, args.cpu_rows, args.cpu_seconds,
            lambda r: tC[:r].cpu().numpy())
        out["config"]["max_err_norm"] = check["max_err_norm"]
        out["config"]["check"] = check
        if not check["ok"]:
            status = 3
            print(f"bench.py: the GPU product is out of tolerance against the "
                  f"oracle: {check}", file=sys.stderr)
    print(json.dumps(out), flush=True)
    return status


if __name__ == "__main__":
    sys.exit(main())
