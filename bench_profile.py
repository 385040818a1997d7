#!/usr/bin/env python3
"""rocprofv3 passes over bench.py, reduced to the short summaries kept under
profiles/.

Every pass is a child process of its own,

  timeout -s KILL <seconds> rocprofv3 <pass options> -f csv -T -d <raw>/<pass>
      -o <name> -- python3 <repo>/bench.py <bench options>

with the program straight after ``--``, run from /tmp with TMPDIR=/tmp.  A
kernel-trace pass (``--kernel-trace --stats``) gives per-dispatch durations;
each counter pass (``--pmc``) collects one group of counters in a run of its
own (FETCH_SIZE, then WRITE_SIZE, then the LDS and matrix-core group), since
counter passes serialise the dispatches and their durations are not used.
HBM bytes are FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by the
factor each counter reads on a plain 256 MiB device copy.

  python3 bench_profile.py gemm --workload 4096cube   ktrace_, traffic_, lds_<kernel>_<workload>.txt
  python3 bench_profile.py split --workload 256x256x8192    split_<kernel>_<workload>.txt
  python3 bench_profile.py ladder                     ladder_4096cube.txt
  python3 bench_profile.py transpose                  transpose_layouts_8192x8192.txt
  python3 bench_profile.py kscan --workload ragged     kscan_<kernel>_<workload>.txt
  python3 bench_profile.py all                        all of the above, every workload

--out sets where the summaries go (default: profiles/ of this checkout),
--raw where rocprofv3 writes its raw output (default: sgemm_prof_raw under
the system's temporary directory).  The pages ask for a
fixed, repeatable measurement: warm up, repeat, keep the median and spread,
read the bank-conflict counter, and check the result before comparing times
("Memory-bank mechanism and accelerated compute", section on turning
derivations into measurements); this tool is that harness for the GPU's
counters.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

COPY_BYTES = 256 << 20
LDS_COUNTERS = ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAVES",
                "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES",
                "SQ_INSTS_VALU_MFMA_MOPS_F32", "GRBM_GUI_ACTIVE"]
GEMM_WORKLOADS = ["4096cube", "8192cube", "skinny", "ragged", "256cube"]
SPLIT_WORKLOADS = ["256x256x8192", "512x512x16384", "1024x1024x8192", "512x4096x4096"]
TRANSPOSE_LAYOUTS = ["naive", "padded", "swizzled"]
# kernel function names (as rocprofv3 -T prints them) of each plan family
FAMILY_KERNEL = [("mfma_lds_", "sgemm_mfma_direct_kernel"), ("mfma_", "sgemm_mfma_kernel"),
                 ("fma_", "sgemm_fma_kernel"), ("simple_", "sgemm_simple_kernel")]
REDUCE_KERNEL = "sgemm_split_reduce_kernel"
BENCH = "python3 <repo>/bench.py"


def say(*a):
    print("[bench_profile]", *a, flush=True)


def kernel_function(plan_name: str) -> str:
    for prefix, fn in FAMILY_KERNEL:
        if plan_name.startswith(prefix):
            return fn
    raise ValueError(plan_name)


# -- running passes -----------------------------------------------------------

def rocprof(raw: str, tag: str, prof_args: list, bench_args: list,
            timeout: int = 300) -> tuple:
    """One rocprofv3 pass over bench.py; returns (output dir, bench stdout,
    the command as printed in summaries).  Raises on a non-zero exit."""
    out = os.path.join(raw, tag)
    os.makedirs(out, exist_ok=True)
    cmd = (["timeout", "-s", "KILL", str(timeout), "rocprofv3", *prof_args, "-f", "csv",
            "-T", "-d", out, "-o", "run", "--", sys.executable,
            os.path.join(ROOT, "bench.py"), *bench_args])
    shown = (f"cd /tmp && TMPDIR=/tmp rocprofv3 {' '.join(prof_args)} -f csv -T "
             f"-d <raw>/{tag} -o run -- {BENCH} {' '.join(bench_args)}").rstrip()
    say(f"pass {tag}: {' '.join(prof_args)} -- bench.py {' '.join(bench_args)}")
    env = dict(os.environ, TMPDIR="/tmp")
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True)
    with open(os.path.join(out, "bench_stdout.txt"), "w") as f:
        f.write(r.stdout)
    with open(os.path.join(out, "bench_stderr.txt"), "w") as f:
        f.write(r.stderr)
    # rocprofv3 may end with a segmentation fault of its own after the program
    # has finished and its files are whole; accept that only when the bench
    # printed its last line.
    finished = '"metric"' in r.stdout or '"copy_bytes"' in r.stdout
    if r.returncode != 0 and not (r.returncode in (139, -11) and finished):
        raise RuntimeError(f"pass {tag} failed with status {r.returncode}:\n"
                           f"{r.stderr[-2000:]}")
    say(f"pass {tag}: done")
    return out, r.stdout, shown


def bench_lines(stdout: str) -> list:
    return [json.loads(l) for l in stdout.splitlines() if l.startswith("{")]


def read_csv(out: str, kind: str) -> list:
    path = os.path.join(out, f"run_{kind}.csv")
    with open(path) as f:
        return list(csv.DictReader(f))


def counters(out: str, grid=None) -> dict:
    """{(kernel name, counter): [value per dispatch]}, of the dispatches of
    `grid` work-items only when given."""
    agg = collections.defaultdict(list)
    for r in read_csv(out, "counter_collection"):
        if grid is None or int(r["Grid_Size"]) == grid:
            agg[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return agg


def per_dispatch(agg: dict, kernel: str, counter: str) -> tuple:
    xs = [x for (k, c), v in agg.items() if c == counter and k.startswith(kernel)
          for x in v]
    if not xs:
        raise KeyError(f"no {counter} for {kernel}")
    return sum(xs) / len(xs), min(xs), max(xs), len(xs)


def durations(out: str, kernel: str, grid=None) -> list:
    """Dispatch durations (ns) of kernel (of `grid` work-items only, when
    given), in dispatch order."""
    rows = [r for r in read_csv(out, "kernel_trace") if r["Kernel_Name"].startswith(kernel)
            and (grid is None or int(r["Grid_Size_X"]) == grid)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]


def stats_row(out: str, kernel: str) -> dict:
    for r in read_csv(out, "kernel_stats"):
        if r["Name"].startswith(kernel):
            return r
    raise KeyError(kernel)


_copy_scale = None


def copy_scale(raw: str) -> tuple:
    """(fetch scale, write scale, commands): bytes per KiB-count of the two
    counters on a plain device copy of COPY_BYTES."""
    global _copy_scale
    if _copy_scale is None:
        scales, shown = [], []
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            out, _, cmd = rocprof(raw, f"copy_{c}", ["--pmc", c],
                                  ["--copy-calibration", str(COPY_BYTES)], 120)
            # the device copy's dispatches (the runtime's buffer-copy kernel),
            # not the fill that made the source
            vals = [x for (k, cc), v in counters(out).items()
                    if cc == c and "copyBuffer" in k for x in v]
            mean = sum(vals) / len(vals)
            scales.append(COPY_BYTES / 1024 / mean)
            shown.append(cmd)
        _copy_scale = (scales[0], scales[1], shown)
    return _copy_scale


def traffic_pass(raw: str, tag: str, bench_args: list, grid=None) -> tuple:
    """({kernel: {counter: (KiB per dispatch, dispatches)}}, commands), of
    the dispatches of `grid` work-items only when given."""
    res, shown = {}, []
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        out, _, cmd = rocprof(raw, f"{tag}_{c}", ["--pmc", c], bench_args, 180)
        shown.append(cmd)
        for (k, cc), v in counters(out, grid).items():
            if cc == c:
                res.setdefault(k, {})[c] = (sum(v) / len(v), len(v))
    return res, shown


def kib(res: dict, kernel: str, counter: str) -> tuple:
    for k, d in res.items():
        if k.startswith(kernel) and counter in d:
            return d[counter]
    raise KeyError((kernel, counter))


# -- summaries ----------------------------------------------------------------

def header_cmd(argv_note: str) -> str:
    return f"made by: python3 bench_profile.py {argv_note}"


def profile_gemm(workload: str, raw: str, dest: str) -> list:
    import bench
    from tiled_fp32_gemm_amd import build
    build.ensure_built()
    wl = ["--workload", workload] if workload != "4096cube" else []
    made = header_cmd(f"gemm --workload {workload}")
    # 1. kernel trace of the bench command itself
    out, stdout, cmd_t = rocprof(raw, f"ktrace_{workload}", ["--kernel-trace", "--stats"],
                                 wl, 600)
    b = bench_lines(stdout)[-1]
    cfg = b["config"]
    plan, M, N, K = cfg["kernel"], cfg["M"], cfg["N"], cfg["K"]
    fn = kernel_function(plan)
    flops = 2.0 * M * N * K
    st = stats_row(out, fn)
    durs = durations(out, fn)
    timed = durs[-b["steps"]:]
    t_avg = sum(timed) / len(timed)
    ev_ms = flops / (b["roofline"]["achieved"] * 1e12) * 1e3
    agree = 100.0 * (t_avg / 1e6 - ev_ms) / ev_ms
    src = cfg["source_hash"]
    lines = [f"# rocprofv3 kernel trace: {plan}, workload {workload} (M={M} N={N} K={K})",
             made,
             f"command: {cmd_t}",
             f"device: {cfg.get('device')} ({cfg.get('arch')}), 1 GPU; source_hash: {src}",
             f"versions: {json.dumps(cfg.get('versions'))}",
             "",
             "kernel_stats (rocprofv3 --stats, all dispatches incl. the clock ramp and warm-up):",
             f"  name: {st['Name']}", f"  calls: {st['Calls']}",
             f"  average_ns: {float(st['AverageNs']):.0f}", f"  min_ns: {st['MinNs']}",
             f"  max_ns: {st['MaxNs']}", f"  stddev_ns: {float(st['StdDev']):.0f}",
             f"timed_dispatches_average_ns: {t_avg:.0f}  (last {len(timed)} dispatches = "
             f"the timed steps)",
             f"timed_dispatches_median_ns: {sorted(timed)[len(timed) // 2]:.0f}",
             f"tflops_from_trace_average: {flops / t_avg / 1e3:.2f}",
             f"frac_of_157.3_from_trace: {flops / t_avg / 1e3 / 157.3:.4f}",
             "",
             "bench.py line of the same run:",
             f"  value_tflops: {b['value']}",
             f"  roofline_achieved_tflops: {b['roofline']['achieved']}",
             f"  roofline_frac: {b['roofline']['frac']}",
             f"  event_timed_launches: {cfg['event_timed_launches']}",
             f"  hip_event_average_ms: {ev_ms:.5f}",
             f"  agreement_trace_vs_events: {agree:+.2f}%",
             f"  clock: {json.dumps(cfg.get('clock'))}",
             f"  clock_ramp_s: {cfg.get('clock_ramp_s')}, warmup steps: {b['warmup']}"]
    if cfg.get("check"):
        lines.append(f"  check: {json.dumps(cfg['check'])}")
    if abs(agree) > 2.0:
        lines += ["  note: for a kernel this short each launch's HIP event pair also spans",
                  "        the host's time to enqueue it (Python and ctypes), so the events",
                  "        read long; the trace figure is the kernel's own duration"]
    written = [_write(dest, f"ktrace_{plan}_{workload}.txt", lines)]
    # 2. HBM traffic
    short = wl + ["--steps", "5", "--warmup", "1", "--warmup-seconds", "0", "--no-cpu-baseline"]
    res, cmds = traffic_pass(raw, f"traffic_{workload}", short)
    fs, ws, ccmds = copy_scale(raw)
    fk, nf = kib(res, fn, "FETCH_SIZE")
    wk, nw = kib(res, fn, "WRITE_SIZE")
    hbm = (fk * fs + wk * ws) * 1024
    alg = 4.0 * (M * K + K * N + M * N)
    lines = [f"# HBM traffic per launch: {plan}, workload {workload} (M={M} N={N} K={K})",
             made,
             f"command_fetch: {cmds[0]}", f"command_write: {cmds[1]}",
             f"command_copy_calibration: {ccmds[0]}   (and WRITE_SIZE)",
             f"fetch_kib_per_dispatch: {fk:.1f}   (mean of {nf} dispatches)",
             f"write_kib_per_dispatch: {wk:.1f}   (mean of {nw} dispatches)",
             f"copy_256MiB_fetch_scale: {fs:.4f}",
             f"copy_256MiB_write_scale: {ws:.4f}",
             f"hbm_bytes_per_launch: {hbm:.0f}",
             f"algorithmic_bytes_per_launch: {alg:.0f}   (4*(MK+KN+MN))",
             f"ratio_hbm_to_algorithmic: {hbm / alg:.3f}",
             f"source_hash: {src}"]
    written.append(_write(dest, f"traffic_{plan}_{workload}.txt", lines))
    # 3. LDS and matrix-core counters
    out, _, cmd_l = rocprof(raw, f"lds_{workload}", ["--pmc", *LDS_COUNTERS], short, 180)
    agg = counters(out)
    lines = [f"# LDS and matrix-core counters: {plan}, workload {workload} "
             f"(M={M} N={N} K={K})", made, f"command: {cmd_l}",
             "per dispatch (mean over dispatches of the GEMM kernel):"]
    for c in sorted(LDS_COUNTERS):
        mean, lo, hi, n = per_dispatch(agg, fn, c)
        lines.append(f"  {c}: {mean:.0f}   (n={n}, min={lo:.0f}, max={hi:.0f})")
    mops = per_dispatch(agg, fn, "SQ_INSTS_VALU_MFMA_MOPS_F32")[0]
    lines.append(f"mfma_flops_per_dispatch: {mops * 512:.4g}   (MOPS_F32 x 512; "
                 f"algorithmic 2MNK = {flops:.4g}, ratio {mops * 512 / flops:.4f})")
    grbm = per_dispatch(agg, fn, "GRBM_GUI_ACTIVE")[0]
    if t_avg > 100e3:
        lines.append(f"effective_clock_ghz: {grbm / 8 / t_avg:.3f}   (GRBM_GUI_ACTIVE per "
                     f"dispatch / 8 XCDs / the kernel-trace average duration)")
    else:
        lines.append("effective_clock_ghz: n/a (the kernel is too short for GRBM_GUI_ACTIVE "
                     "to measure it)")
    lines.append(f"source_hash: {src}")
    written.append(_write(dest, f"lds_{plan}_{workload}.txt", lines))
    return written


def _split_roles(rows: list, ts_key: str) -> tuple:
    """Classify the product-kernel rows of an --op sgemm_ws run, given in
    dispatch order: a partial-product dispatch is one directly followed by
    the reduce kernel; plain sgemm's dispatches all follow the last reduce.
    Returns (split rows, plain rows, reduce rows)."""
    split, plain, red = [], [], []
    last_red = max((i for i, r in enumerate(rows) if REDUCE_KERNEL in r["Kernel_Name"]),
                   default=-1)
    for i, r in enumerate(rows):
        if REDUCE_KERNEL in r["Kernel_Name"]:
            red.append(r)
        elif i > last_red:
            plain.append(r)
        elif i + 1 < len(rows) and REDUCE_KERNEL in rows[i + 1]["Kernel_Name"]:
            split.append(r)
    return split, plain, red


def profile_split(workload: str, raw: str, dest: str) -> list:
    made = header_cmd(f"split --workload {workload}")
    args = ["--op", "sgemm_ws", "--workload", workload]
    out, stdout, cmd_t = rocprof(raw, f"ktrace_ws_{workload}", ["--kernel-trace", "--stats"],
                                 args, 600)
    b = bench_lines(stdout)[-1]
    cfg = b["config"]
    M, N, K, S = cfg["M"], cfg["N"], cfg["K"], cfg["splits"]
    flops = 2.0 * M * N * K
    fn = "sgemm_mfma_direct_kernel"
    steps = b["steps"]
    rows = [r for r in read_csv(out, "kernel_trace")
            if r["Kernel_Name"].startswith(fn) or REDUCE_KERNEL in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    sp_rows, pl_rows, rd_rows = _split_roles(rows, "Start_Timestamp")
    dur = lambda rs: [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rs]
    split_part, plain, red_t = dur(sp_rows)[-steps:], dur(pl_rows)[-steps:], dur(rd_rows)[-steps:]
    plain_wgs = int(pl_rows[-1]["Grid_Size_X"]) // int(pl_rows[-1]["Workgroup_Size_X"])
    avg = lambda xs: sum(xs) / len(xs)
    short = args + ["--steps", "5", "--warmup", "1", "--warmup-seconds", "0"]
    fs, ws, _ = copy_scale(raw)
    per, cmds = {}, []
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        outc, _, cmd = rocprof(raw, f"traffic_ws_{workload}_{c}", ["--pmc", c], short, 180)
        cmds.append(cmd)
        crow = [r for r in read_csv(outc, "counter_collection") if r["Counter_Name"] == c and
                (r["Kernel_Name"].startswith(fn) or REDUCE_KERNEL in r["Kernel_Name"])]
        crow.sort(key=lambda r: int(r["Dispatch_Id"]))
        for role, rs in zip(("split", "plain", "reduce"), _split_roles(crow, "Dispatch_Id")):
            vals = [float(r["Counter_Value"]) for r in rs]
            per.setdefault(role, {})[c] = sum(vals) / len(vals)

    def hbm(role):
        f, w = per[role]["FETCH_SIZE"], per[role]["WRITE_SIZE"]
        return (f * fs + w * ws) * 1024, f, w

    hs, hp, hr = hbm("split"), hbm("plain"), hbm("reduce")
    call = avg(split_part) + avg(red_t)
    lines = [f"# K split across workgroups (sgemm_ws): {cfg['kernel']}, M={M} N={N} K={K}, "
             f"{S} splits", made,
             f"command_trace: {cmd_t}",
             f"command_counters: {cmds[0]}   (then WRITE_SIZE, each in a run of its own; "
             f"scale factors from the 256 MiB copy calibration: fetch {fs:.4f}, write "
             f"{ws:.4f}); a partial-product dispatch is the one followed by the sum kernel, "
             f"plain sgemm's follow the last sum",
             f"device: {cfg.get('device')}, 1 GPU; source_hash: {cfg.get('source_hash')}", "",
             f"per kernel, trace average over the {steps} timed dispatches:",
             f"  partial products (split kernel): {fn}, {cfg['workgroups']} workgroups",
             f"    average_ns: {avg(split_part):.0f}",
             f"    tflops: {flops / avg(split_part) / 1e3:.2f}",
             f"    hbm_bytes_per_launch: {hs[0]:.0f}   (fetch {hs[1]:.1f} KiB, write "
             f"{hs[2]:.1f} KiB per dispatch)",
             f"    algorithmic_bytes_per_launch: {4 * (M * K + K * N + S * M * N)}",
             f"  fixed-order sum (reduce kernel): {REDUCE_KERNEL}",
             f"    average_ns: {avg(red_t):.0f}",
             f"    hbm_bytes_per_launch: {hr[0]:.0f}   (fetch {hr[1]:.1f} KiB, write "
             f"{hr[2]:.1f} KiB per dispatch)",
             f"    algorithmic_bytes_per_launch: {(S + 1) * M * N * 4}",
             f"    gbs_algorithmic: {(S + 1) * M * N * 4 / avg(red_t):.1f}",
             f"  plain sgemm, same shape: {fn}, {plain_wgs} workgroups",
             f"    average_ns: {avg(plain):.0f}",
             f"    tflops: {flops / avg(plain) / 1e3:.2f}",
             f"    hbm_bytes_per_launch: {hp[0]:.0f}",
             f"    algorithmic_bytes_per_launch: {4 * (M * K + K * N + M * N)}", "",
             f"split call = partial + sum kernels: {call:.0f} ns -> "
             f"{flops / call / 1e3:.2f} TFLOP/s; plain sgemm {avg(plain):.0f} ns -> gain "
             f"{avg(plain) / call:.2f}x",
             "", "bench.py line of the same run:",
             f"  value_tflops: {b['value']}",
             f"  roofline_achieved_tflops: {b['roofline']['achieved']}",
             f"  call_ms_median (events): {cfg['call_ms_median']}",
             f"  sgemm_same_shape_tflops: {cfg['sgemm_same_shape_tflops']}"]
    return [_write(dest, f"split_{cfg['kernel']}_{workload}.txt", lines)]


def _step_segments(blines: list, dispatches: list) -> list:
    """Split a ladder run's GEMM dispatches (after the one reference sgemm
    the bench computes first) into the steps' own: per step, its clock ramp,
    warm-up and timed launches, as its bench line counts them."""
    segs, pos = [], 1
    for d in blines:
        n = d["config"]["clock_ramp_launches"] + d["warmup"] + d["steps"]
        segs.append(dispatches[pos:pos + n])
        pos += n
    if pos != len(dispatches):
        raise RuntimeError(f"ladder: {len(dispatches)} dispatches, expected {pos}")
    return segs


def profile_ladder(raw: str, dest: str) -> list:
    made = header_cmd("ladder")
    args = ["--ladder", "--steps", "5", "--warmup", "1"]
    out, stdout, cmd_t = rocprof(raw, "ktrace_ladder", ["--kernel-trace", "--stats"], args, 900)
    blines = bench_lines(stdout)
    trace = [r for r in read_csv(out, "kernel_trace") if r["Kernel_Name"].startswith("sgemm_")]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    tsegs = _step_segments(blines, [(r["Kernel_Name"], int(r["End_Timestamp"]) -
                                     int(r["Start_Timestamp"])) for r in trace])
    cargs = ["--ladder", "--steps", "1", "--warmup", "0", "--warmup-seconds", "0"]
    cnt = ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAVES",
           "SQ_INSTS_VALU"]
    outc, stdc, cmd_c = rocprof(raw, "pmc_ladder", ["--pmc", *cnt], cargs, 900)
    disp = {}
    for r in read_csv(outc, "counter_collection"):
        if r["Kernel_Name"].startswith("sgemm_"):
            disp.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = \
                float(r["Counter_Value"])
    csegs = _step_segments(bench_lines(stdc), [disp[k] for k in sorted(disp)])
    flops = 2.0 * 4096 ** 3
    lines = ["# Ablation ladder (sgemm_ladder), workload 4096cube: M = N = K = 4096, fp32, "
             "A,B uniform seed 2, MI355X", made,
             f"command_trace: {cmd_t}", f"command_counters: {cmd_c}",
             "each step changes one thing against the step before; TFLOP/s = 2MNK / mean of "
             "the 5 timed dispatches in the trace; counters from the step's last dispatch", "",
             f"{'step':>4}  {'name':38s} {'TFLOP/s':>8} {'kernel':28s} {'SQ_INSTS_LDS':>13}"
             f"  {'SQ_LDS_IDX_ACTIVE':>17}  {'SQ_LDS_BANK_CONFLICT':>20}"]
    for d, ts, cs in zip(blines, tsegs, csegs):
        c = d["config"]
        timed = [x for _, x in ts[-d["steps"]:]]
        cd = cs[-1]
        lines.append(f"{c['ladder_step']:>4}  {c['name']:38s} "
                     f"{flops / (sum(timed) / len(timed)) / 1e3:8.2f} {ts[-1][0][:28]:28s} "
                     f"{cd['SQ_INSTS_LDS']:13.0f}  {cd['SQ_LDS_IDX_ACTIVE']:17.0f}  "
                     f"{cd['SQ_LDS_BANK_CONFLICT']:20.0f}")
    lines += ["", "bench.py lines (HIP-event kernel time):"]
    for d in blines:
        c = d["config"]
        lines.append(f"  {c['ladder_step']:>2} {c['name']:38s} achieved "
                     f"{d['roofline']['achieved']:8.3f} TFLOP/s, max rel diff vs sgemm "
                     f"{c['max_rel_diff_vs_sgemm']:.1e}")
    return [_write(dest, "ladder_4096cube.txt", lines)]


def profile_transpose(raw: str, dest: str) -> list:
    made = header_cmd("transpose")
    rows = cols = 8192
    nbytes = 2 * 4 * rows * cols
    table, blines, cmds = [], [], {}
    cnt = ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAVES",
           "GRBM_GUI_ACTIVE"]
    for lay in TRANSPOSE_LAYOUTS:
        args = ["--op", "transpose", "--layout", lay, "--steps", "100", "--warmup", "10"]
        out, stdout, cmd_t = rocprof(raw, f"ktrace_t_{lay}", ["--kernel-trace", "--stats"],
                                     args, 300)
        d = bench_lines(stdout)[-1]
        dur = durations(out, "sgemm_transpose_kernel")[-100:]
        avg = sum(dur) / len(dur)
        outc, _, cmd_c = rocprof(raw, f"pmc_t_{lay}", ["--pmc", *cnt],
                                 ["--op", "transpose", "--layout", lay, "--steps", "3",
                                  "--warmup", "1", "--warmup-seconds", "0"], 300)
        agg = counters(outc)
        cv = {c: per_dispatch(agg, "sgemm_transpose_kernel", c)[0] for c in cnt}
        cmds = {"trace": cmd_t.replace(lay, "<layout>"), "pmc": cmd_c.replace(lay, "<layout>")}
        table.append(f"{lay:9s} {avg / 1e3:13.2f} {nbytes / avg:12.1f} "
                     f"{nbytes / avg / 8000:14.3f} {d['config']['copy_same_bytes_gbs']:21.1f} "
                     f"{cv['SQ_LDS_BANK_CONFLICT']:21.0f} {cv['SQ_LDS_IDX_ACTIVE']:18.0f} "
                     f"{cv['SQ_INSTS_LDS']:13.0f} {cv['SQ_WAVES']:9.0f}")
        blines.append(f"  {lay}: value {d['value']} GB/s (wall), roofline.achieved "
                      f"{d['roofline']['achieved']} GB/s, kernel median "
                      f"{d['config']['kernel_ms_median']} ms, copy "
                      f"{d['config']['copy_same_bytes_gbs']} GB/s")
    lines = [f"# Tiled transpose {rows} x {cols} fp32 (in 256 MiB, out 256 MiB): LDS layouts "
             f"on MI355X", made,
             f"command_trace: {cmds['trace']}", f"command_counters: {cmds['pmc']}",
             "tile: 64 input rows x 128 input columns, 256 threads; launches rotate over 4 "
             "input/output buffer pairs (2 GiB, past the 256 MiB last-level cache)",
             f"bytes per launch: 2 * 4 * {rows} * {cols} = {nbytes} (algorithmic: read once, "
             "write once)", "",
             "layout    trace_avg_us  GB/s(trace)  frac_of_8TB/s  copy_same_bytes_GB/s  "
             "SQ_LDS_BANK_CONFLICT  SQ_LDS_IDX_ACTIVE  SQ_INSTS_LDS  SQ_WAVES", *table, "",
             "bench.py lines (event-timed launches, 100 steps; copy = a device copy of the "
             "same bytes over the same buffers):", *blines]
    return [_write(dest, f"transpose_layouts_{rows}x{cols}.txt", lines)]


def profile_kscan(workload: str, raw: str, dest: str) -> list:
    """Trace durations of the product kernel over K at the workload's M x N:
    the fixed cost of a launch (K = 0: the launch and the C stores) and the
    cost per K slab (a least-squares line over the K of the workload's own
    plan), against the slab's compute at the matrix peak."""
    made = header_cmd(f"kscan --workload {workload}")
    args = ["--op", "kscan", "--workload", workload, "--steps", "50", "--warmup", "5"]
    out, stdout, cmd = rocprof(raw, f"kscan_{workload}", ["--kernel-trace"], args, 600)
    lines_b = bench_lines(stdout)
    rows = [r for r in read_csv(out, "kernel_trace") if "sgemm" in r["Kernel_Name"]
            and "probe" not in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    table, pos, pts = [], 0, []
    M, N = lines_b[0]["M"], lines_b[0]["N"]
    import bench
    K0 = bench.WORKLOADS[workload][2]
    plan0 = [d for d in lines_b if d["K"] == K0][0]["kernel"]
    for d in lines_b:
        n = d["clock_ramp_launches"] + d["warmup"] + d["steps"]
        seg = rows[pos:pos + n][-d["steps"]:]
        pos += n
        dur = sorted(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in seg)
        med = dur[len(dur) // 2] / 1e3
        slabs = -(-d["K"] // d["tile_k"]) if d["K"] else 0
        table.append(f"  K={d['K']:6d}  slabs={slabs:4d}  trace_median_us={med:9.3f}  "
                     f"kernel={d['kernel']}")
        if d["kernel"][:-5] == plan0[:-5] and d["K"] > 0:   # any load form
            pts.append((slabs, med))
    if pos != len(rows):
        raise RuntimeError(f"kscan: {len(rows)} dispatches, expected {pos}")
    n = len(pts)
    sx, sy = sum(p[0] for p in pts), sum(p[1] for p in pts)
    sxx, sxy = sum(p[0] ** 2 for p in pts), sum(p[0] * p[1] for p in pts)
    slope = (n * sxy - sx * sy) / (n * sxx - sx * sx)
    icpt = (sy - slope * sx) / n
    wl = [d for d in lines_b if d["K"] == K0][0]
    tk, wgs = wl["tile_k"], wl["workgroups"]
    m = plan0.split("_")[2].split("x")
    bm, bn = int(m[0]), int(m[1])
    per_cu = -(-wgs // 256)   # tiles per CU
    slab_peak_us = per_cu * 2.0 * bm * bn * tk / (157.3e12 / 256) * 1e6
    slabs0 = -(-K0 // tk)
    floor = [d for d in lines_b if d["K"] == 0]
    k0_us = None
    if floor:
        i0 = lines_b.index(floor[0])
        k0_us = float(table[i0].split("trace_median_us=")[1].split()[0])
    lines = [f"# Launch cost against K: {plan0}, M={M} N={N} (workload {workload}, "
             f"K={K0}), MI355X", made, f"command: {cmd}", "",
             "per K (trace median of the 50 timed launches):", *table, "",
             f"fit over the {n} points with the workload's kernel: duration = "
             f"{icpt:.3f} us + {slope:.4f} us x slabs",
             f"slab at the FP32 matrix peak: {per_cu} tiles per CU x 2 x {bm} x {bn} x {tk} "
             f"flop / 614.5 GFLOP/s = {slab_peak_us:.4f} us -> steady slabs run at "
             f"{slab_peak_us / slope:.3f} of peak",
             f"K = 0 (launch + C stores only): {k0_us} us",
             f"workload: {slabs0} slabs -> fit {icpt + slope * slabs0:.3f} us; at the peak "
             f"per slab with the measured fixed cost: {icpt + slab_peak_us * slabs0:.3f} us "
             f"= {2.0 * M * N * K0 / ((icpt + slab_peak_us * slabs0) * 1e-6) / 1e12:.1f} "
             f"TFLOP/s"]
    return [_write(dest, f"kscan_{plan0}_{workload}.txt", lines)]


def lds_conflicts(workload: str, raw: str) -> tuple:
    """(plan name, SQ_LDS_BANK_CONFLICT per dispatch of the product kernel)
    for a short bench run of the workload: the pages' bank-conflict reading
    on the production kernel."""
    args = ["--workload", workload, "--steps", "1", "--warmup", "0", "--warmup-seconds", "0",
            "--no-cpu-baseline"]
    out, stdout, _ = rocprof(raw, f"conflicts_{workload}",
                             ["--pmc", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS"], args, 240)
    plan = bench_lines(stdout)[-1]["config"]["kernel"]
    agg = counters(out)
    fn = kernel_function(plan)
    vals = [x for (k, c), v in agg.items() if c == "SQ_LDS_BANK_CONFLICT" and k.startswith(fn)
            for x in v]
    return plan, vals


def _write(dest: str, name: str, lines: list) -> str:
    os.makedirs(dest, exist_ok=True)
    path = os.path.join(dest, name)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    say(f"wrote {path}")
    return path


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("what", choices=["gemm", "split", "ladder", "transpose", "kscan", "all"])
    ap.add_argument("--workload", default=None)
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--raw", default=os.path.join(tempfile.gettempdir(), "sgemm_prof_raw"))
    args = ap.parse_args()
    raw, dest = os.path.abspath(args.raw), os.path.abspath(args.out)
    done = []
    if args.what in ("gemm", "all"):
        for w in [args.workload] if args.workload else GEMM_WORKLOADS:
            done += profile_gemm(w, raw, dest)
    if args.what in ("split", "all"):
        for w in [args.workload] if args.workload and args.what == "split" else SPLIT_WORKLOADS:
            done += profile_split(w, raw, dest)
    if args.what in ("ladder", "all"):
        done += profile_ladder(raw, dest)
    if args.what in ("transpose", "all"):
        done += profile_transpose(raw, dest)
    if args.what in ("kscan", "all"):
        for w in [args.workload] if args.workload and args.what == "kscan" else ["ragged",
                                                                               "skinny"]:
            done += profile_kscan(w, raw, dest)
    say(f"{len(done)} summaries written")
    return 0


if __name__ == "__main__":
    sys.exit(main())
