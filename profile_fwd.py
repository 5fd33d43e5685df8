"""rocprofv3 evidence for the forward kernel at the bench workload.

Run on a GPU machine from the repository root:

    python3 profile_fwd.py            # kernel trace, FETCH_SIZE / WRITE_SIZE, SQ counter passes

Writes its summaries under gpurun_out/profile_fwd/profiles/ (the GPU machine
keeps only gpurun_out/); `python3 profile_fwd.py --summarize` rebuilds them
from the returned CSVs, under profiles/:
  fwd_d128_c3_kernel_trace.md  per-kernel durations of `bench.py --no-cpu --no-others`
  fwd_d128_c3_traffic.md       HBM bytes per launch of the forward kernel
  fwd_d128_c3_traffic.json     the same figure, keyed by a hash of the kernel
                               sources (bench.py reports it only while the
                               hash still matches)
  fwd_d128_c3_counters.md      shader clock, MFMA busy, VALU/LDS activity, LDS
                               bank conflicts and the instruction mix
  kernels_all_workloads.md     kernel durations of the full `bench.py --no-cpu`
                               (every workload: c2, c3, c4, c5 forward and c5
                               backward), per workload and kernel

The TCC FETCH_SIZE / WRITE_SIZE counters are calibrated against a plain
device copy of known size: the factor (bytes moved / counter bytes) for each
counter is applied to the forward kernel's counter value.  Each counter is
collected in its own rocprofv3 pass (counter-block limits).

`python3 profile_fwd.py --copy BYTES` is the calibration workload: it copies a
BYTES-long device buffer three times (run under rocprofv3 by the main mode).

`python3 profile_fwd.py --kernels` takes the same two SQ passes for the other
kernels on their workloads (`--run NAME` is the workload each pass profiles:
c2 and c5 forward, the c5 backward's two kernels, the causal backward at the
c3 shape) and the HBM traffic of the c4 forward, and writes
  kernel_counters.md            one section per kernel: clock, MFMA busy, VALU
                                and transcendental issue, LDS, scratch/registers
  fwd_d128_c4_traffic.md        FETCH_SIZE / WRITE_SIZE of the c4 forward
"""

from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(ROOT, "gpurun_out", "profile_fwd")
PROFILES = os.path.join(ROOT, "profiles")
FWD_KERNEL = "fwd_d128_kernel"
COPY_BYTES = 1 << 30
BENCH = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "30", "--warmup", "5", "--no-cpu", "--no-others"]
# SQ counter passes (at most 8 SQ and 2 GRBM counters each)
SQ_PASSES = {
    "sq1": ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
            "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_VALU_MFMA_COEXEC_CYCLES", "GRBM_GUI_ACTIVE"],
    "sq2": ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
            "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_SALU", "SQ_WAVES", "GRBM_GUI_ACTIVE"],
    "tcc": ["TCC_HIT_sum", "TCC_MISS_sum", "GRBM_GUI_ACTIVE"],
}
PASSES = ["ktrace", "traffic", *SQ_PASSES, "ktrace_all"]
BENCH_ALL = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "10", "--warmup", "3", "--no-cpu"]
FLOP_C3 = 4 * 8192 * 8192 * 128 * 2 * 16 // 2
# 256-row query block t (of 32 per head) visits key tiles 0 .. 4t+3 of 64 keys
EXP_C3 = 2 * 16 * sum(256 * 64 * (4 * t + 4) for t in range(8192 // 256))


# --kernels: (name, workload run, kernel-name regex, source, instance, flop per launch)
def _flop(name):
    sys.path.insert(0, ROOT)
    from fa_inputs import WORKLOADS

    w = WORKLOADS[name]
    return w


# (the kernel regex is a plain name: each workload runs one instance of it)
KERNEL_SETS = [
    ("c2 forward, D=64 (B=4 H=16 N=2048)", "c2_fwd", "fwd_d64_kernel", "fa_fwd_d64.hip",
     "fwd_d64_kernelILb0E", lambda: _flop("c2").fwd_flop()),
    ("c5 forward, D=256 (B=1 H=4 N=4096)", "c5_fwd", "fwd_d256_kernel", "fa_fwd_d256.hip",
     "fwd_d256_kernel", lambda: _flop("c5").fwd_flop()),
    ("c5 backward dQ, D=256", "c5_bwd", "bwd_dq_kernel", "fa_bwd.hip", "bwd_dq_kernelILi256ELb0E",
     lambda: 6 * 4096 * 4096 * 256 * 4),
    ("c5 backward dK/dV, D=256", "c5_bwd", "bwd_dkdv_d256_kernel", "fa_bwd_dkdv_d256.hip",
     "bwd_dkdv_d256_kernelILi256ELb0E", lambda: 8 * 4096 * 4096 * 256 * 4),
    ("causal backward dQ at the c3 shape, D=128 (B=2 H=16 N=8192)", "c3_bwd", "bwd_dq_kernel", "fa_bwd.hip",
     "bwd_dq_kernelILi128ELb1E", lambda: 3 * 8192 * 8192 * 128 * 32),
    ("causal backward dK/dV at the c3 shape, D=128", "c3_bwd", "bwd_dkdv_kernel", "fa_bwd.hip",
     "bwd_dkdv_kernelILi128ELb1E", lambda: 4 * 8192 * 8192 * 128 * 32),
]
RUN_REPS = 12


def run_workload(name: str, reps: int) -> None:
    """One workload, `reps` launches (the profiled program of --kernels)."""
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import exact_attention_51_amd as fa
    from fa_inputs import WORKLOADS, make_inputs

    key, kind = name.split("_")
    w = WORKLOADS[key]
    if key == "c3" and kind == "bwd":
        w = w.with_(backward=True, seed=13)
    x = make_inputs(w, with_do=kind == "bwd")

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    q, k, v = bf(x.q_bits), bf(x.k_bits), bf(x.v_bits)
    o, lse = fa.fwd(q, k, v, w.scale, w.causal)
    if kind == "bwd":
        do = bf(x.do_bits)
        for _ in range(reps):
            fa.bwd(q, k, v, o, do, lse, w.scale, w.causal)
    else:
        for _ in range(reps):
            fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)
    torch.cuda.synchronize()
    print(f"copied {name} x{reps}", flush=True)  # the line run() looks for


def copy_workload(nbytes: int) -> None:
    import torch

    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(f"copied {nbytes} bytes 3 times", flush=True)


def run(cmd: list[str], timeout: int) -> None:
    """Run a rocprofv3 pass.  rocprofv3 may end with SIGSEGV after the
    profiled program has finished and its results are written: exit code
    139 (or -11) is accepted only when the profiled program's own last line
    was printed (bench.py's JSON record, or the copy workload's "copied"
    line), never for a crash of the program itself; the summary step then
    also needs the result files."""
    print("+ " + " ".join(cmd), flush=True)
    env = dict(os.environ, TMPDIR="/tmp")
    res = subprocess.run(cmd, timeout=timeout, env=env, cwd="/tmp", stdout=subprocess.PIPE, text=True)
    sys.stdout.write(res.stdout)
    sys.stdout.flush()
    rc = res.returncode
    if rc == 0:
        return
    finished = any(line.startswith('{"metric"') or line.startswith("copied ") for line in res.stdout.splitlines())
    if rc in (139, -11) and finished:
        print(f"rocprofv3 ended with {rc} after the program finished; results kept", flush=True)
        return
    raise SystemExit(f"rocprofv3 failed with exit code {rc}")


def counter_rows(outdir: str) -> list[dict]:
    (path,) = glob.glob(os.path.join(outdir, "**", "*counter_collection.csv"), recursive=True)
    with open(path) as f:
        return list(csv.DictReader(f))


def per_dispatch(rows: list[dict], name_filter) -> list[float]:
    vals: dict[int, float] = {}
    for r in rows:
        if name_filter(r["Kernel_Name"]):
            d = int(r["Dispatch_Id"])
            vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
    return [vals[d] for d in sorted(vals)]


def kernel_source_hash() -> str:
    sys.path.insert(0, ROOT)
    import bench

    return bench.kernel_source_hash()


def collected_source_hash(out: str) -> str:
    """The kernel source hash recorded when the traffic counters were taken
    (not the hash of the sources at summary time, which may be newer)."""
    try:
        with open(os.path.join(out, "traffic_source_hash.txt")) as f:
            return f.read().strip()
    except OSError:
        return "unknown"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--copy", type=int, default=0, help="calibration workload: copy this many bytes")
    ap.add_argument("--summarize", action="store_true",
                    help="only rebuild profiles/ from the CSVs already under gpurun_out/profile_fwd")
    ap.add_argument("--passes", default=",".join(PASSES), help=f"comma-separated subset of {','.join(PASSES)}")
    ap.add_argument("--kernels", action="store_true", help="SQ passes of the other kernels, c4 traffic")
    ap.add_argument("--run", default="", help="profiled workload of --kernels (c2_fwd, c5_fwd, c5_bwd, c3_bwd, c4_fwd)")
    args = ap.parse_args()
    passes = args.passes.split(",")
    if args.copy:
        copy_workload(args.copy)
        return 0
    if args.run:
        run_workload(args.run, RUN_REPS)
        return 0
    if args.kernels:
        out = os.path.join(ROOT, "gpurun_out", "profile_kernels")
        if not args.summarize:
            os.makedirs(out, exist_ok=True)
            me = [sys.executable, os.path.abspath(__file__)]
            for i, (label, run_name, regex, _, _, _) in enumerate(KERNEL_SETS):
                for pname, ctrs in SQ_PASSES.items():
                    if pname == "tcc":
                        continue
                    run(["rocprofv3", "--pmc", *ctrs, "--kernel-include-regex", regex, "--output-format", "csv", "-d",
                         os.path.join(out, f"k{i}_{pname}"), "-o", "run", "--", *me, "--run", run_name], 300)
            for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
                run(["rocprofv3", "--pmc", ctr, "--kernel-include-regex", FWD_KERNEL, "--output-format", "csv", "-d",
                     os.path.join(out, f"c4_{ctr}"), "-o", "run", "--", *me, "--run", "c4_fwd"], 300)
                run(["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d", os.path.join(out, f"copy_{ctr}"), "-o",
                     "run", "--", *me, "--copy", str(COPY_BYTES)], 300)
        summarize_kernels(out, PROFILES if args.summarize else os.path.join(out, "profiles"))
        return 0

    if not args.summarize:
        os.makedirs(OUT, exist_ok=True)
        me = [sys.executable, os.path.abspath(__file__)]
        if "ktrace" in passes:
            run(cmd_kernel_trace(), 600)  # 1. kernel trace with per-kernel statistics
        if "traffic" in passes:
            with open(os.path.join(OUT, "traffic_source_hash.txt"), "w") as f:
                f.write(kernel_source_hash() + "\n")
        for ctr in ("FETCH_SIZE", "WRITE_SIZE") if "traffic" in passes else ():  # 2. forward, then copy
            run(["rocprofv3", "--pmc", ctr, "--kernel-include-regex", FWD_KERNEL, "--output-format", "csv", "-d",
                 os.path.join(OUT, f"fwd_{ctr}"), "-o", "run", "--", *BENCH], 300)
            run(["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d", os.path.join(OUT, f"copy_{ctr}"), "-o",
                 "run", "--", *me, "--copy", str(COPY_BYTES)], 300)
        if "ktrace_all" in passes:  # 4. kernel trace of every workload
            run(["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
                 os.path.join(OUT, "ktrace_all"), "-o", "run", "--", *BENCH_ALL], 600)
        for name, ctrs in SQ_PASSES.items():  # 3. SQ / TCC counters of the forward kernel
            if name not in passes:
                continue
            run(["rocprofv3", "--pmc", *ctrs, "--kernel-include-regex", FWD_KERNEL, "--output-format", "csv", "-d",
                 os.path.join(OUT, name), "-o", "run", "--", *BENCH], 300)
    if not args.summarize and set(passes) != set(PASSES):
        print("partial run: rebuild the summaries with --summarize once every pass has results", flush=True)
        return 0
    summarize(OUT, PROFILES if args.summarize else os.path.join(OUT, "profiles"))
    return 0


def cmd_kernel_trace() -> list[str]:
    return ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", os.path.join(OUT, "ktrace"),
            "-o", "run", "--", *BENCH]


def summarize(out: str, dest: str) -> None:
    """Turn the rocprofv3 CSVs under `out` into the summaries under `dest`."""
    os.makedirs(dest, exist_ok=True)
    (stats,) = glob.glob(os.path.join(out, "ktrace", "**", "*kernel_stats.csv"), recursive=True)
    with open(stats) as f:
        krows = list(csv.DictReader(f))
    counters = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        fwd = per_dispatch(counter_rows(os.path.join(out, f"fwd_{ctr}")), lambda n: FWD_KERNEL in n)
        cp = per_dispatch(counter_rows(os.path.join(out, f"copy_{ctr}")), lambda n: True)
        cp = sorted(cp)[-3:]  # the three copies are the largest dispatches
        counters[ctr] = {"fwd_kib": fwd, "copy_kib": cp}
    fetch_f = (COPY_BYTES / 1024) / statistics.median(counters["FETCH_SIZE"]["copy_kib"])
    write_f = (COPY_BYTES / 1024) / statistics.median(counters["WRITE_SIZE"]["copy_kib"])
    fetch_b = statistics.median(counters["FETCH_SIZE"]["fwd_kib"][1:]) * 1024 * fetch_f
    write_b = statistics.median(counters["WRITE_SIZE"]["fwd_kib"][1:]) * 1024 * write_f
    total = fetch_b + write_b
    rec = {
        "kernel": FWD_KERNEL,
        "workload": "causal forward B=2 H=16 N=8192 D=128 bf16",
        "kernel_source_hash": collected_source_hash(out),
        "bytes_per_launch": round(total),
        "fetch_bytes": round(fetch_b),
        "write_bytes": round(write_b),
        "copy_scale_fetch": fetch_f,
        "copy_scale_write": write_f,
        "raw": {ctr: {k: {"n": len(v), "median": statistics.median(v), "min": min(v), "max": max(v)} for k, v in d.items()}
                for ctr, d in counters.items()},  # KiB per dispatch (forward) and per copy
        "command": "python3 profile_fwd.py",
    }
    with open(os.path.join(dest, "fwd_d128_c3_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)

    lines = ["# Forward kernel, causal B=2 H=16 N=8192 D=128 bf16: kernel trace", "",
             "Command (repository root, GPU box): `python3 profile_fwd.py`, which runs", "",
             "    " + " ".join(cmd_kernel_trace()).replace(ROOT + "/", "").replace(sys.executable, "python3"), "",
             "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in krows:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    with open(os.path.join(dest, "fwd_d128_c3_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    algo = 2 * 16 * 8192 * 128 * 2 * 4 + 2 * 16 * 8192 * 4  # Q, K, V read + O written, L written
    lines = ["# Forward kernel, causal B=2 H=16 N=8192 D=128 bf16: HBM traffic per launch", "",
             "Command (repository root, GPU box): `python3 profile_fwd.py` (one rocprofv3 `--pmc` pass per counter,",
             "forward kernel filtered by name; calibration = 1 GiB device copy, `python3 profile_fwd.py --copy 1073741824`).", "",
             f"- FETCH_SIZE scale (copy bytes / counter bytes): {fetch_f:.4f}",
             f"- WRITE_SIZE scale: {write_f:.4f}",
             f"- forward fetch: {fetch_b / 2**20:.1f} MiB, write: {write_b / 2**20:.1f} MiB, total {total / 2**20:.1f} MiB per launch",
             f"- algorithmic bytes (Q, K, V read once; O, L written once): {algo / 2**20:.1f} MiB",
             f"- ratio measured / algorithmic: {total / algo:.2f}",
             f"- kernel source hash: {rec['kernel_source_hash']}"]
    with open(os.path.join(dest, "fwd_d128_c3_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if all(os.path.isdir(os.path.join(out, n)) for n in ("sq1", "sq2")):
        summarize_counters(out, dest)
    if os.path.isdir(os.path.join(out, "ktrace_all")):
        summarize_all_workloads(out, dest)
    print("\n".join(lines), flush=True)


def per_dispatch_counters(outdir: str) -> tuple[dict, dict]:
    """Counter totals and (start, end) timestamps per dispatch of the forward kernel."""
    vals: dict[int, dict] = {}
    span: dict[int, tuple] = {}
    for r in counter_rows(outdir):
        if FWD_KERNEL not in r["Kernel_Name"]:
            continue
        d = int(r["Dispatch_Id"])
        v = vals.setdefault(d, {})
        v[r["Counter_Name"]] = v.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            span[d] = (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
    return vals, span


def summarize_all_workloads(out: str, dest: str) -> None:
    """Per-dispatch kernel trace of the full bench run, split by workload.

    bench.py runs c3, then c2, c4, c5 forward and c5 backward (whose setup
    runs one c5 forward), then the pages' shape B=2 H=4 N=2048 D=128 in both
    masking modes, the causal backward at the c3 shape (whose setup runs one
    c3-shape forward), the head dims 32, 96 and 160 on the c2, c3 and c5
    shapes, then fa_fwd_sparse at the c3 shape with a window of
    16 key blocks and with a random half of the blocks (the same kernel
    instance: the first half of its launches is the window run), then
    fa_fwd_kv on the pages' shape in both masking
    modes and on two decode shapes (one row per head: 1x8 heads over 32768
    keys, split 32 ways, then 8x16 heads over 8192 keys, split 2 ways); runs
    of one kernel instance are told apart by that order, and a merge kernel
    belongs to the kernel launched just before it.  Medians skip each run's
    first launch."""
    sys.path.insert(0, ROOT)
    from fa_inputs import WORKLOADS

    (path,) = glob.glob(os.path.join(out, "ktrace_all", "**", "*kernel_trace.csv"), recursive=True)
    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    families = [r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0] for r in rows]

    def targs(family):  # template arguments of a forward kernel instance
        return family[family.index("<") + 1 : family.rindex(">")].split(", ") if "<" in family else []

    def is_kv(family):
        return "fwd_bf16_kernel" in family and len(targs(family)) >= 6 and targs(family)[5] == "true"

    def is_sparse(family):
        return "fwd_bf16_kernel" in family and len(targs(family)) >= 7 and targs(family)[6] == "true"

    n_sparse = sum(is_sparse(f) for f in families)
    seen_c2, seen_c5, seen_c3_bwd, runs, last, i_sparse = False, False, False, {}, None, 0
    for i, (r, family) in enumerate(zip(rows, families)):
        if is_sparse(family):
            label = "c3 sparse window16" if i_sparse < n_sparse // 2 else "c3 sparse random50"
            i_sparse += 1
        elif "merge" in family:
            label = last
        elif "decode_kernel" in family:
            # the run's own merge (next launch) tells the two decode shapes apart
            nxt = families[i + 1] if i + 1 < len(families) else ""
            label = "decode 1x8x32768 kv" if "merge_wide" in nxt else "decode 8x16x8192 kv"
        elif is_kv(family):  # the fa_fwd_kv instances
            label = "p1 causal fwd kv" if "<128, true" in family else "p1 fwd kv"
        elif "bwd_" in family:
            if "<256" in family or "d256" in family:
                label, seen_c5 = "c5 bwd", True
            else:
                label, seen_c3_bwd = "c3 bwd", True
        elif any(f"fwd_bf16_kernel<{d}," in family for d in (32, 96, 160)):
            label = next(f"d{d} fwd" for d in (32, 96, 160) if f"fwd_bf16_kernel<{d}," in family)
        elif "fwd_bf16_kernel<64" in family or "fwd_d64_kernel" in family:
            label, seen_c2 = "c2 fwd", True
        elif "fwd_bf16_kernel<256" in family or "fwd_d256_kernel" in family:
            label, seen_c5 = "c5 fwd", True
        elif "fwd_d128_kernel" in family or "fwd_bf16_kernel<128" in family:
            # bench order: c3, c2, c4, c5, the pages' shape, c3-shape bwd
            causal = "<true>" in family or "<128, true" in family
            if seen_c5:
                label = "p1 causal fwd" if causal else "p1 fwd"
                if i + 1 < len(families) and "bwd_dq" in families[i + 1]:
                    label = "c3 bwd setup fwd"
            else:
                label = "c4 fwd" if seen_c2 else "c3 fwd"
        else:
            continue
        last = label
        runs.setdefault((label, family), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    p1 = WORKLOADS["c3"].with_(B=2, H=4, N=2048, D=128)
    flop = {"c2 fwd": WORKLOADS["c2"].fwd_flop(), "c3 fwd": WORKLOADS["c3"].fwd_flop(),
            "c4 fwd": WORKLOADS["c4"].fwd_flop(), "c5 fwd": WORKLOADS["c5"].fwd_flop(),
            "p1 fwd": p1.with_(causal=False).fwd_flop(), "p1 causal fwd": p1.with_(causal=True).fwd_flop()}
    flop["p1 fwd kv"], flop["p1 causal fwd kv"] = flop["p1 fwd"], flop["p1 causal fwd"]
    flop["d32 fwd"] = WORKLOADS["c2"].with_(D=32).fwd_flop()
    flop["d96 fwd"] = WORKLOADS["c3"].with_(D=96).fwd_flop()
    flop["d160 fwd"] = WORKLOADS["c5"].with_(D=160).fwd_flop()
    import bench
    import numpy as np

    w3 = WORKLOADS["c3"]
    nb3 = w3.N // 64
    for lab, m in (("c3 sparse window16", bench.sparse_band_mask(nb3)),
                   ("c3 sparse random50", (np.random.default_rng(8).random((nb3, nb3)) < 0.5).astype(np.uint8))):
        flop[lab] = 4 * w3.D * w3.B * w3.H * bench.sparse_visible_pairs(m, w3.N, True)
    kv_bytes = {"decode 1x8x32768 kv": 2 * 8 * 32768 * 128 * 2, "decode 8x16x8192 kv": 2 * 128 * 8192 * 128 * 2}
    w5, w3 = WORKLOADS["c5"], WORKLOADS["c3"]
    per_bwd = {"bwd_dq": 6 * w5.N * w5.N * w5.D * w5.B * w5.H, "bwd_dkdv": 8 * w5.N * w5.N * w5.D * w5.B * w5.H}
    per_bwd3 = {"bwd_dq": 3 * w3.N * w3.N * w3.D * w3.B * w3.H, "bwd_dkdv": 4 * w3.N * w3.N * w3.D * w3.B * w3.H}
    lines = ["# Kernel durations of every bench workload", "",
             "Command (repository root, GPU box): `python3 profile_fwd.py`; pass `ktrace_all` =",
             f"`rocprofv3 --kernel-trace --stats -- {' '.join(['python3', 'bench.py'] + BENCH_ALL[2:])}`.",
             "Median and minimum over the launches of each run after its first; TFLOPS from the median, with",
             "4N²D·B·H (halved under causal) for the forward, 6N²D·B·H for dQ and 8N²D·B·H for dK/dV (halved",
             "for the causal c3-shape backward), and for the block-sparse rows 4D per (query, key) pair the",
             "block and causal masks leave.  Decode rows give the K/V read rate of the decode kernel",
             "(2·B·H·Nk·D·2 bytes per launch) instead; a merge kernel is listed under the run it serves.", "",
             "| workload | kernel | launches | median µs | min µs | TFLOPS or K/V GB/s |", "|---|---|---|---|---|---|"]
    for (label, kname), ts in runs.items():
        body = ts[1:] if len(ts) > 1 else ts
        med = statistics.median(body)
        if label == "c5 bwd":
            f = next((v for k, v in per_bwd.items() if k in kname), None)
        elif label == "c3 bwd":
            f = next((v for k, v in per_bwd3.items() if k in kname), None)
        elif "merge" in kname:
            f = None
        else:
            f = flop.get(label)
        tf = f"{f / (med * 1e-6) / 1e12:.0f}" if f else ""
        if label in kv_bytes and "decode_kernel" in kname:
            tf = f"{kv_bytes[label] / (med * 1e-6) / 1e9:.0f} GB/s"
        short = kname.replace("void ", "").replace("fa::", "")
        lines.append(f"| {label} | `{short}` | {len(ts)} | {med:.1f} | {min(body):.1f} | {tf} |")
    with open(os.path.join(dest, "kernels_all_workloads.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def tcc_lines(med: dict) -> list[str]:
    if ("tcc", "TCC_HIT_sum") not in med:
        return []
    hit, miss = med[("tcc", "TCC_HIT_sum")], med[("tcc", "TCC_MISS_sum")]
    return [f"- L2 (TCC) requests: {hit:.4g} hits, {miss:.4g} misses; hit rate {100 * hit / (hit + miss):.1f}%"]


def build_metadata_lines() -> list[str]:
    """Register, scratch and LDS use of the forward kernel instance the bench
    line times, from the compiler's resource-usage remarks on our own build."""
    sys.path.insert(0, ROOT)
    from exact_attention_51_amd import build

    src = os.path.join(ROOT, "exact_attention_51_amd", "csrc", "fa_fwd_d128.hip")
    cmd = [build.hipcc(), *build.COMMON_FLAGS, *build.source_flags("fa_fwd_d128.hip"), "--offload-device-only",
           "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", os.devnull]
    try:
        err = subprocess.run(cmd, capture_output=True, text=True, timeout=600).stderr.splitlines()
    except (OSError, subprocess.TimeoutExpired):
        return []
    want = ("VGPRs:", "AGPRs:", "ScratchSize [bytes/lane]:", "Occupancy [waves/SIMD]:", "LDS Size [bytes/block]:")
    for i, line in enumerate(err):
        if "Function Name:" in line and "fwd_d128_kernelILb1EE" in line:
            got = []
            for rest in err[i + 1:i + 16]:
                if "Function Name:" in rest:
                    break
                body = rest.split("remark: ")[-1].split(" [-Rpass")[0].strip()
                if body.startswith(want):
                    got.append(body)
            return ["- compiler resource usage of this instance (D=128, causal, 4 waves of 64 rows; hipcc"
                    " -Rpass-analysis=kernel-resource-usage): " + "; ".join(got)]
    return []


def summarize_counters(out: str, dest: str) -> None:
    """Medians over the dispatches of each SQ pass (the first one skipped).

    GRBM_GUI_ACTIVE comes back summed over the 8 XCDs, so one XCD's busy
    cycles are a eighth of it; with the dispatch duration that gives the
    shader clock.  SQ_VALU_MFMA_BUSY_CYCLES is normalised by those cycles
    times the 1024 SIMDs (the same normalisation matches the MFMA share
    implied by the achieved TFLOPS at the measured clock, printed beside)."""
    med = {}
    clocks = []
    for name in SQ_PASSES:
        if not os.path.isdir(os.path.join(out, name)):
            continue
        vals, span = per_dispatch_counters(os.path.join(out, name))
        ids = sorted(vals)[1:]
        for k in {k for d in ids for k in vals[d]}:
            med[(name, k)] = statistics.median(vals[d][k] for d in ids)
        for d in ids:
            if d in span and span[d][1] > span[d][0]:
                clocks.append((vals[d]["GRBM_GUI_ACTIVE"] / 8 / (span[d][1] - span[d][0]), span[d][1] - span[d][0]))
    gui = med[("sq1", "GRBM_GUI_ACTIVE")] / 8
    ghz = statistics.median(c for c, _ in clocks) if clocks else float("nan")
    ns = statistics.median(t for _, t in clocks) if clocks else float("nan")
    mfma = med[("sq1", "SQ_VALU_MFMA_BUSY_CYCLES")] / (gui * 1024)
    coexec = med[("sq1", "SQ_VALU_MFMA_COEXEC_CYCLES")] / max(med[("sq1", "SQ_VALU_MFMA_BUSY_CYCLES")], 1)
    implied = (FLOP_C3 / (ns * 1e-9)) / (1024 * 1024 * ghz * 1e9) if clocks else float("nan")
    bank = med[("sq2", "SQ_LDS_BANK_CONFLICT")] / max(med[("sq2", "SQ_LDS_IDX_ACTIVE")], 1)
    lds_active = med[("sq2", "SQ_LDS_IDX_ACTIVE")] / (gui * 256)
    n_mfma = med[("sq2", "SQ_INSTS_MFMA")]
    valu_busy = 4 * med[("sq1", "SQ_ACTIVE_INST_VALU")] / (gui * 1024)  # quad-cycles, summed over waves
    n_exp = 64 * med[("sq2", "SQ_INSTS_VALU_TRANS_F32")]
    mix = {k: med[("sq2", k)] / n_mfma for k in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_INSTS_SALU")}
    lines = ["# Forward kernel, causal B=2 H=16 N=8192 D=128 bf16: SQ counters", "",
             "Command (repository root, GPU box): `python3 profile_fwd.py`; two `rocprofv3 --pmc` passes over",
             "`bench.py --steps 30 --warmup 5 --no-cpu --no-others`, kernel filtered by name, medians over the",
             "dispatches after the first:", ""]
    for name, ctrs in SQ_PASSES.items():
        lines.append(f"- pass {name}: `{' '.join(ctrs)}`")
    lines += ["",
              f"- dispatch duration (median): {ns / 1e3:.1f} us; cycles per XCD (GRBM_GUI_ACTIVE / 8): {gui:.0f};"
              f" shader clock {ghz:.2f} GHz",
              f"- MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs) = {100 * mfma:.1f}%;"
              f" MFMA share implied by the TFLOPS at that clock (1024 FLOP/clk/SIMD): {100 * implied:.1f}%",
              f"- MFMA cycles co-executing VALU work: {100 * coexec:.1f}%",
              f"- VALU issue (SQ_ACTIVE_INST_VALU, quad-cycles summed over waves, x 4 / (cycles x 1024 SIMDs),"
              f" MFMA issue included): {100 * valu_busy:.1f}%",
              f"- transcendental lane-operations (SQ_INSTS_VALU_TRANS_F32 x 64): {n_exp / 1e9:.4f} G, against one"
              f" exp2 per score of every key tile a 256-row query block visits (diagonal tiles included,"
              f" masked scores too): {EXP_C3 / 1e9:.4f} G",
              f"- LDS: SQ_LDS_IDX_ACTIVE / (cycles x 256 CUs) = {100 * lds_active:.1f}%;"
              f" bank-conflict cycles / LDS active cycles = {100 * bank:.2f}%",
              f"- instructions per MFMA: VALU (MFMA included) {mix['SQ_INSTS_VALU']:.2f}, of them transcendental"
              f" {mix['SQ_INSTS_VALU_TRANS_F32']:.2f}; LDS {mix['SQ_INSTS_LDS']:.2f}; SALU {mix['SQ_INSTS_SALU']:.2f}",
              f"- waves per dispatch: {med[('sq2', 'SQ_WAVES')]:.0f}",
              *tcc_lines(med),
              *build_metadata_lines(),
              f"- kernel source hash: {collected_source_hash(out)}"]
    with open(os.path.join(dest, "fwd_d128_c3_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def resource_usage(src_name: str, instance: str) -> str:
    """Register, scratch and LDS use of one kernel instance from the
    compiler's resource-usage remarks on our own build."""
    sys.path.insert(0, ROOT)
    from exact_attention_51_amd import build

    src = os.path.join(ROOT, "exact_attention_51_amd", "csrc", src_name)
    cmd = [build.hipcc(), *build.COMMON_FLAGS, *build.source_flags(src_name), "--offload-device-only",
           "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", os.devnull]
    try:
        err = subprocess.run(cmd, capture_output=True, text=True, timeout=600).stderr.splitlines()
    except (OSError, subprocess.TimeoutExpired):
        return ""
    want = ("VGPRs:", "AGPRs:", "ScratchSize [bytes/lane]:", "Occupancy [waves/SIMD]:", "LDS Size [bytes/block]:")
    for i, line in enumerate(err):
        if "Function Name:" in line and instance in line:
            got = []
            for rest in err[i + 1:i + 16]:
                if "Function Name:" in rest:
                    break
                body = rest.split("remark: ")[-1].split(" [-Rpass")[0].strip()
                if body.startswith(want):
                    got.append(body)
            return "; ".join(got)
    return ""


def kernel_medians(outdir: str, regex_plain: str) -> tuple[dict, list]:
    vals: dict[int, dict] = {}
    span: dict[int, tuple] = {}
    for r in counter_rows(outdir):
        name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
        if regex_plain not in name:
            continue
        d = int(r["Dispatch_Id"])
        v = vals.setdefault(d, {})
        v[r["Counter_Name"]] = v.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            span[d] = (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
    ids = sorted(vals)[1:] or sorted(vals)
    med = {k: statistics.median(vals[d][k] for d in ids if k in vals[d]) for k in {k for d in ids for k in vals[d]}}
    spans = [(vals[d]["GRBM_GUI_ACTIVE"] / 8 / (span[d][1] - span[d][0]), span[d][1] - span[d][0]) for d in ids
             if d in span and span[d][1] > span[d][0]]
    return med, spans


def summarize_kernels(out: str, dest: str) -> None:
    """kernel_counters.md and fwd_d128_c4_traffic.md from the --kernels CSVs."""
    os.makedirs(dest, exist_ok=True)
    lines = ["# SQ counters of the other kernels", "",
             "Command (repository root, GPU box): `python3 profile_fwd.py --kernels`: per kernel, two",
             "`rocprofv3 --pmc` passes (the counter sets below) over `python3 profile_fwd.py --run WORKLOAD`",
             f"({RUN_REPS} launches of the workload on seeded synthetic inputs), kernel filtered by name, medians",
             "over the dispatches after the first.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024",
             "SIMDs); TFLOPS from the median dispatch duration and the workload's FLOP count (4N²D per head",
             "for the forward, 6N²D for dQ, 8N²D for dK/dV, halved under causal masking).", ""]
    for name, ctrs in SQ_PASSES.items():
        if name != "tcc":
            lines.append(f"- pass {name}: `{' '.join(ctrs)}`")
    for i, (label, run_name, regex, src, instance, flop) in enumerate(KERNEL_SETS):
        plain = regex
        if not all(os.path.isdir(os.path.join(out, f"k{i}_{p}")) for p in ("sq1", "sq2")):
            continue
        m1, sp = kernel_medians(os.path.join(out, f"k{i}_sq1"), plain)
        m2, _ = kernel_medians(os.path.join(out, f"k{i}_sq2"), plain)
        if not m1 or not m2:
            continue
        gui = m1["GRBM_GUI_ACTIVE"] / 8
        ghz = statistics.median(c for c, _ in sp) if sp else float("nan")
        ns = statistics.median(t for _, t in sp) if sp else float("nan")
        tf = flop() / (ns * 1e-9) / 1e12 if sp else float("nan")
        n_mfma = max(m2["SQ_INSTS_MFMA"], 1)
        lines += ["", f"## {label}: `{regex}`", "",
                  f"- dispatch duration (median): {ns / 1e3:.1f} us -> {tf:.0f} TFLOPS ({100 * tf / 2500:.1f}% of the"
                  f" bf16 dense peak); shader clock {ghz:.2f} GHz",
                  f"- MFMA busy: {100 * m1['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * 1024):.1f}%; MFMA cycles co-executing"
                  f" VALU: {100 * m1['SQ_VALU_MFMA_COEXEC_CYCLES'] / max(m1['SQ_VALU_MFMA_BUSY_CYCLES'], 1):.1f}%",
                  f"- VALU issue (x 4 / (cycles x 1024 SIMDs), MFMA issue included):"
                  f" {100 * 4 * m1['SQ_ACTIVE_INST_VALU'] / (gui * 1024):.1f}%; LDS instruction wait / wave cycles:"
                  f" {100 * m1['SQ_WAIT_INST_LDS'] / max(m1['SQ_WAVE_CYCLES'], 1):.1f}%",
                  f"- instructions per MFMA: VALU (MFMA included) {m2['SQ_INSTS_VALU'] / n_mfma:.2f}, of them"
                  f" transcendental {m2['SQ_INSTS_VALU_TRANS_F32'] / n_mfma:.2f}; LDS {m2['SQ_INSTS_LDS'] / n_mfma:.2f};"
                  f" SALU {m2['SQ_INSTS_SALU'] / n_mfma:.2f}",
                  f"- LDS: SQ_LDS_IDX_ACTIVE / (cycles x 256 CUs) = {100 * m2['SQ_LDS_IDX_ACTIVE'] / (gui * 256):.1f}%;"
                  f" bank-conflict cycles / LDS active = {100 * m2['SQ_LDS_BANK_CONFLICT'] / max(m2['SQ_LDS_IDX_ACTIVE'], 1):.2f}%",
                  f"- waves per dispatch: {m2['SQ_WAVES']:.0f}",
                  f"- compiler resource usage (`{instance}`): {resource_usage(src, instance)}"]
    with open(os.path.join(dest, "kernel_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)
    # c4 traffic
    try:
        fwd = {c: per_dispatch(counter_rows(os.path.join(out, f"c4_{c}")), lambda n: FWD_KERNEL in n)
               for c in ("FETCH_SIZE", "WRITE_SIZE")}
        cp = {c: sorted(per_dispatch(counter_rows(os.path.join(out, f"copy_{c}")), lambda n: True))[-3:]
              for c in ("FETCH_SIZE", "WRITE_SIZE")}
    except (ValueError, OSError):
        return
    fetch_f = (COPY_BYTES / 1024) / statistics.median(cp["FETCH_SIZE"])
    write_f = (COPY_BYTES / 1024) / statistics.median(cp["WRITE_SIZE"])
    fetch_b = statistics.median(fwd["FETCH_SIZE"][1:]) * 1024 * fetch_f
    write_b = statistics.median(fwd["WRITE_SIZE"][1:]) * 1024 * write_f
    algo = 1 * 8 * 32768 * 128 * 2 * 4 + 1 * 8 * 32768 * 4
    tl = ["# Forward kernel, causal B=1 H=8 N=32768 D=128 bf16 (Q x3): HBM traffic per launch", "",
          "Command (repository root, GPU box): `python3 profile_fwd.py --kernels` (one rocprofv3 `--pmc` pass per",
          "counter over `python3 profile_fwd.py --run c4_fwd`, forward kernel filtered by name; calibration = 1 GiB",
          "device copy).", "",
          f"- FETCH_SIZE scale (copy bytes / counter bytes): {fetch_f:.4f}; WRITE_SIZE scale: {write_f:.4f}",
          f"- forward fetch: {fetch_b / 2**20:.1f} MiB, write: {write_b / 2**20:.1f} MiB, total"
          f" {(fetch_b + write_b) / 2**20:.1f} MiB per launch",
          f"- algorithmic bytes (Q, K, V read once; O, L written once): {algo / 2**20:.1f} MiB",
          f"- ratio measured / algorithmic: {(fetch_b + write_b) / algo:.2f}"]
    with open(os.path.join(dest, "fwd_d128_c4_traffic.md"), "w") as f:
        f.write("\n".join(tl) + "\n")
    print("\n".join(tl), flush=True)


if __name__ == "__main__":
    sys.exit(main())
