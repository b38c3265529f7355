#!/usr/bin/env python3
"""Benchmark of OUT_PROD through a resident Q4_K weight on one MI355X.

One step = the whole hot path on the two Q4_K shapes of a 4096-wide model
with a 14336-wide MLP:
  large-T  W = 14336 x 4096 (N x K), G = 4096 x 14336, dst = 4096 x 4096
           -> the tiled fused dequant + F32-MFMA kernel (producer/consumer waves)
  skinny   W = 4096 x 14336, G = 16 x 4096, dst = 16 x 14336
           -> the one-pass small-T kernel
Inputs are seeded synthetic data (workloads.py) resident in HBM before the
timed region. value = whole-step F32 TFLOP/s (2*T*N*K per call).

Prints ONE JSON line. --gpus N > 1 is refused: the path runs on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

PEAK_F32_TFLOPS = 157.3  # MI355X dense MFMA F32
PEAK_HBM_GBS = 8000.0    # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
LARGE = "q4_k_n14336_k4096_t4096"
SKINNY = "q4_k_n4096_k14336_t16"
PROFILES = os.path.join(REPO, "profiles")
KERNEL_SOURCES = ["quantized_weight_backward_amd/csrc/retro_kernels.h",
                  "quantized_weight_backward_amd/csrc/retro_split_kernel.h",
                  "quantized_weight_backward_amd/csrc/retro_unit.hip",
                  "quantized_weight_backward_amd/csrc/retro_host.h",
                  "quantized_weight_backward_amd/csrc/retro_ws_kernel.h",
                  "quantized_weight_backward_amd/csrc/retro_decode.h",
                  "quantized_weight_backward_amd/csrc/retro_api.hip"]


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and whitespace removed, so
    that an edit of a comment does not void the recorded counters."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(REPO, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(tag: str):
    """HBM bytes per launch from a committed counter summary, or None when
    the summary is missing or the kernels changed since it was taken."""
    path = os.path.join(PROFILES, f"{tag}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"source_sha256:\s*(\w+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d {out}/prof_trace -o run -- "
             "python3 bench.py --steps 20 --warmup 3 --no-cpu-baseline",
    "FETCH_SIZE": "rocprofv3 --pmc FETCH_SIZE -f csv -d {out}/pmc_FETCH_SIZE -o run -- "
                  "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline",
    "WRITE_SIZE": "rocprofv3 --pmc WRITE_SIZE -f csv -d {out}/pmc_WRITE_SIZE -o run -- "
                  "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline",
    "mfma": "rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES "
            "GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS -f csv "
            "-d {out}/pmc_mfma -o run -- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline",
    "copy_FETCH_SIZE": "rocprofv3 --pmc FETCH_SIZE -f csv -d {out}/pmc_copy_FETCH_SIZE -o run -- "
                       "python3 bench.py --copy-probe-mib 1024",
    "copy_WRITE_SIZE": "rocprofv3 --pmc WRITE_SIZE -f csv -d {out}/pmc_copy_WRITE_SIZE -o run -- "
                       "python3 bench.py --copy-probe-mib 1024",
}
KERNELS = {  # summary tag -> (kernel-name prefix in rocprofv3 output, workload, variant)
    f"ws_{LARGE}": ("void retro::out_prod_ws_kernel<12, 2, 4, 2, 1, false>", LARGE, "ws_128x256"),
    f"skinny_{SKINNY}": ("void retro::out_prod_skinny_kernel<12, 16, true>", SKINNY, "skinny"),
    f"split_{LARGE}": ("void retro::out_prod_split_kernel<12>", LARGE, "split_128x256"),
}
LARGE_TAG, SKINNY_TAG = f"ws_{LARGE}", f"skinny_{SKINNY}"
# Kernel traces of single cases outside the benchmark step (opt-in variants,
# the forward), each from its own run of `bench.py --profile-case`:
# summary tag -> (workload, dense weight type or "", op, variant, kernel-name prefix)
CASE_TRACES = {
    "split128_mxfp4_n17408_k5120_t2048": ("mxfp4_n17408_k5120_t2048", "", "out_prod", "split_128x128",
                                          "void retro::out_prod_split_kernel<39>"),
    "split128_q4_0_n17408_k5120_t2048": ("q4_0_n17408_k5120_t2048", "", "out_prod", "split_128x128",
                                         "void retro::out_prod_split_kernel<2>"),
    "split128_bf16_n4096_k4096_t512": ("dense_n4096_k4096_t512", "bf16", "out_prod", "split_128x128",
                                       "void retro::out_prod_split_kernel<30>"),
    "mulmat_skinny_q4_k_n4096_k14336_t16": ("q4_k_n4096_k14336_t16", "", "mul_mat", "skinny",
                                            "void retro::mul_mat_skinny_kernel<12>"),
}


def case_trace_command(tag: str, run_dir: str) -> str:
    workload, wtype, op, variant, _ = CASE_TRACES[tag]
    out = os.path.relpath(run_dir, REPO).rstrip("/")
    dense = f" --wtype {wtype}" if wtype else ""
    return (f"rocprofv3 --kernel-trace --stats -f csv -d {out}/trace_{tag} -o run -- python3 bench.py "
            f"--profile-case {workload}{dense} --op {op} --variant {variant} --launches 10")


def _mean_counter(path: str, prefix: str) -> tuple[float, int]:
    import csv

    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if r["Kernel_Name"].startswith(prefix)]
    return (sum(vals) / len(vals) if vals else float("nan")), len(vals)


def profile_command(name: str, run_dir: str) -> str:
    """The rocprofv3 command of PROFILE_COMMANDS[name] writing under run_dir."""
    return PROFILE_COMMANDS[name].format(out=os.path.relpath(run_dir, REPO).rstrip("/"))


def summarize(run_dir: str) -> None:
    """Write profiles/<tag>_trace.md, <tag>_traffic.md and <tag>_counters.md
    from rocprofv3 output under run_dir (the commands in PROFILE_COMMANDS with
    {out} = run_dir, run from the repository root)."""
    import csv

    os.makedirs(PROFILES, exist_ok=True)
    stats = list(csv.DictReader(open(os.path.join(run_dir, "prof_trace", "run_kernel_stats.csv"))))
    copy_bytes = 1024 << 20
    f_copy, _ = _mean_counter(os.path.join(run_dir, "pmc_copy_FETCH_SIZE", "run_counter_collection.csv"),
                              "__amd_rocclr_copyBuffer")
    w_copy, _ = _mean_counter(os.path.join(run_dir, "pmc_copy_WRITE_SIZE", "run_counter_collection.csv"),
                              "__amd_rocclr_copyBuffer")
    f_scale = copy_bytes / (f_copy * 1024)
    w_scale = copy_bytes / (w_copy * 1024)
    src = kernel_source_hash()
    for tag, (workload, wtype, op, variant, prefix) in CASE_TRACES.items():
        path = os.path.join(run_dir, f"trace_{tag}", "run_kernel_stats.csv")
        if not os.path.exists(path):
            continue
        row = next(r for r in csv.DictReader(open(path)) if r["Name"].startswith(prefix))
        lines = [f"# {tag}: rocprofv3 kernel trace", "",
                 f"Command (repository root): `{case_trace_command(tag, run_dir)}`", "",
                 f"Kernel: `{row['Name']}` ({op}, workload {workload}{' ' + wtype if wtype else ''}, "
                 f"variant {variant})", "",
                 "| calls | average (us) | min (us) | max (us) |", "|---|---|---|---|",
                 f"| {row['Calls']} | {float(row['AverageNs']) / 1e3:.2f} | {float(row['MinNs']) / 1e3:.2f} | "
                 f"{float(row['MaxNs']) / 1e3:.2f} |", "",
                 f"kernel source_sha256: {src}", ""]
        open(os.path.join(PROFILES, f"{tag}_trace.md"), "w").write("\n".join(lines))
        print(f"{tag}: avg {float(row['AverageNs']) / 1e3:.2f} us")
    for tag, (prefix, workload, _) in KERNELS.items():
        row = next(r for r in stats if r["Name"].startswith(prefix))
        lines = [f"# {tag}: rocprofv3 kernel trace", "",
                 f"Command (repository root): `{profile_command('trace', run_dir)}`", "",
                 f"Kernel: `{row['Name']}` (workload {workload})", "",
                 "| calls | average (us) | min (us) | max (us) | share of GPU time |",
                 "|---|---|---|---|---|",
                 f"| {row['Calls']} | {float(row['AverageNs']) / 1e3:.2f} | {float(row['MinNs']) / 1e3:.2f} | "
                 f"{float(row['MaxNs']) / 1e3:.2f} | {float(row['Percentage']):.2f}% |", "",
                 f"kernel source_sha256: {src}", ""]
        open(os.path.join(PROFILES, f"{tag}_trace.md"), "w").write("\n".join(lines))
        fetch, nf = _mean_counter(os.path.join(run_dir, "pmc_FETCH_SIZE", "run_counter_collection.csv"), prefix)
        write, nw = _mean_counter(os.path.join(run_dir, "pmc_WRITE_SIZE", "run_counter_collection.csv"), prefix)
        hbm = fetch * 1024 * f_scale + write * 1024 * w_scale
        lines = [f"# {tag}: HBM traffic per launch (rocprofv3 counters)", "",
                 "Commands (repository root):", "",
                 *[f"- `{profile_command(k, run_dir)}`" for k in ("FETCH_SIZE", "WRITE_SIZE", "copy_FETCH_SIZE",
                                                           "copy_WRITE_SIZE")], "",
                 "Calibration: a 1 GiB device-to-device copy reads and writes 1073741824 bytes; the counters "
                 f"read FETCH_SIZE = {f_copy:.1f} KiB and WRITE_SIZE = {w_copy:.1f} KiB per copy launch, so "
                 f"FETCH_SIZE is scaled by {f_scale:.4f} and WRITE_SIZE by {w_scale:.4f}.", "",
                 "| counter | KiB per launch (mean) | launches | scaled bytes |", "|---|---|---|---|",
                 f"| FETCH_SIZE | {fetch:.1f} | {nf} | {fetch * 1024 * f_scale:.4g} |",
                 f"| WRITE_SIZE | {write:.1f} | {nw} | {write * 1024 * w_scale:.4g} |", "",
                 f"hbm_bytes_per_launch: {hbm:.6g}",
                 f"source_sha256: {src}", ""]
        open(os.path.join(PROFILES, f"{tag}_traffic.md"), "w").write("\n".join(lines))
        mfma_csv = os.path.join(run_dir, "pmc_mfma", "run_counter_collection.csv")
        if os.path.exists(mfma_csv):
            write_counter_summary(tag, prefix, workload, mfma_csv, src, profile_command("mfma", run_dir))
        print(f"{tag}: avg {float(row['AverageNs']) / 1e3:.2f} us, traffic {hbm / 1e6:.1f} MB per launch")


def write_counter_summary(tag: str, prefix: str, workload: str, path: str, src: str, command: str) -> None:
    """profiles/<tag>_counters.md: per-launch means of the MFMA pass, with
    the checks of the F32 MFMA work against 2*T*N*K (one MOP = 512 FLOPs)."""
    import csv

    import workloads as wl

    per = {}
    for r in csv.DictReader(open(path)):
        if r["Kernel_Name"].startswith(prefix):
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    mean = {k: sum(v) / len(v) for k, v in per.items()}
    case = wl.WORKLOADS[workload]
    flops = 2.0 * case["T"] * case["N"] * case["K"]
    lines = [f"# {tag}: MFMA and LDS counters per launch (rocprofv3)", "",
             f"Command (repository root): `{command}`", "",
             "| counter | mean per launch |", "|---|---|",
             *[f"| {k} | {v:.6g} |" for k, v in sorted(mean.items())], ""]
    mops = mean.get("SQ_INSTS_VALU_MFMA_MOPS_F32")
    if mops:
        lines += [f"F32 MFMA FLOPs counted: {mops * 512:.6g} (512 per MOP); 2*T*N*K = {flops:.6g}; "
                  f"ratio {mops * 512 / flops:.4f} (above 1 by the tile padding of the last t and k tiles).", ""]
    busy, cu = mean.get("SQ_VALU_MFMA_BUSY_CYCLES"), mean.get("SQ_BUSY_CU_CYCLES")
    if busy and cu:
        # MFMA busy cycles are summed over the 4 SIMDs of each CU, busy CU
        # cycles over the CUs
        lines += [f"MFMA busy fraction per SIMD = SQ_VALU_MFMA_BUSY_CYCLES / (4 * SQ_BUSY_CU_CYCLES) = "
                  f"{busy / (4 * cu):.4f}", ""]
    valu = mean.get("SQ_INSTS_VALU")
    if valu and cu:
        lines += [f"VALU instructions per SIMD per busy cycle = SQ_INSTS_VALU / (4 * SQ_BUSY_CU_CYCLES) = "
                  f"{valu / (4 * cu):.4f} (a wave64 VALU instruction occupies a SIMD for about 4 cycles)", ""]
    lines += [f"source_sha256: {src}", ""]
    open(os.path.join(PROFILES, f"{tag}_counters.md"), "w").write("\n".join(lines))


def cpu_baseline(case: dict, target_s: float = 20.0) -> dict:
    """The CPU oracle (double accumulation, as it stands) on sampled t rows of
    the large-T workload, all host cores; FLOPs counted as 2*N*K per row."""
    import numpy as np

    import oracle

    cores = max(1, min(16, os.cpu_count() or 1))  # a one-GPU share of the host
    N, K = case["N"], case["K"]
    rows = np.arange(8 * cores) % case["T"]
    t0 = time.perf_counter()
    oracle.out_prod(case["type"], case["W"], case["G"], K, rows=rows, nthreads=cores)
    first = time.perf_counter() - t0
    nrows = int(len(rows) * max(1.0, target_s / max(first, 1e-3)))
    nrows = max(len(rows), min(nrows, case["T"]))
    rows = np.arange(nrows)
    t0 = time.perf_counter()
    oracle.out_prod(case["type"], case["W"], case["G"], K, rows=rows, nthreads=cores)
    secs = time.perf_counter() - t0
    flops = 2.0 * N * K * nrows
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "host_cpu": model, "host_threads": os.cpu_count(),
            "sample": f"{nrows} of {case['T']} t rows of {LARGE} (full decode of W included), "
                      f"{secs:.1f} s"}


def cpu_baseline_skinny(case: dict) -> dict:
    """The CPU oracle on one host thread over the whole T = 16 workload (all
    16 t rows, full decode of W)."""
    import oracle

    t0 = time.perf_counter()
    oracle.out_prod(case["type"], case["W"], case["G"], case["K"], nthreads=1)
    secs = time.perf_counter() - t0
    flops = 2.0 * case["T"] * case["N"] * case["K"]
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"all {case['T']} t rows of {SKINNY} (full decode of W included), {secs:.2f} s"}


def kernel_family(variant: str) -> str:
    return {"ws": "out_prod_ws_kernel", "tile": "out_prod_tile_kernel"}.get(variant.split("_")[0].rstrip("2"),
                                                                         "out_prod_skinny_kernel")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device-to-device copy of this size (counter calibration)")
    ap.add_argument("--profile-case", metavar="WORKLOAD", default=None,
                    help="only run one workload LAUNCHES times (for a kernel trace) and exit")
    ap.add_argument("--wtype", default="", help="with --profile-case: f32, f16 or bf16 for the dense workload")
    ap.add_argument("--op", choices=("out_prod", "mul_mat"), default="out_prod")
    ap.add_argument("--variant", default="auto", help="with --profile-case: a variant name, or auto")
    ap.add_argument("--launches", type=int, default=10)
    ap.add_argument("--summarize", metavar="RUN_DIR", default=None,
                    help="write profiles/*.md from rocprofv3 output under RUN_DIR and exit (no GPU)")
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize)
        return 0

    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(a sharded job would run this kernel on each GPU's own rows of G)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import quantized_weight_backward_amd as q
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs cuda:0"
    dev = torch.device("cuda:0")

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}))
        return 0

    if args.profile_case:
        wtype = {"f32": q.F32, "f16": q.F16, "bf16": q.BF16}.get(args.wtype) if args.wtype else None
        c = wl.workload(args.profile_case, wtype)
        vid = 0 if args.variant == "auto" else {v: k for k, v in q.VARIANT_NAMES.items()}[args.variant]
        W = torch.from_numpy(c["W"]).to(dev)
        if args.op == "out_prod":
            G = torch.from_numpy(c["G"]).to(dev)
            out = torch.empty((c["T"], c["K"]), dtype=torch.float32, device=dev)
            call = lambda: q.out_prod(c["type"], W, G, c["K"], out=out, variant=vid)
        else:
            X = torch.randn((c["T"], c["K"]), device=dev)
            out = torch.empty((c["T"], c["N"]), dtype=torch.float32, device=dev)
            call = lambda: q.mul_mat(c["type"], W, X, out=out, variant=vid)
        for _ in range(2):
            call()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.launches)]
        for e in ev:
            e[0].record()
            call()
            e[1].record()
        torch.cuda.synchronize()
        ms = [e[0].elapsed_time(e[1]) for e in ev]
        print(json.dumps({"profile_case": args.profile_case, "wtype": args.wtype, "op": args.op,
                          "variant": args.variant, "launches": args.launches,
                          "median_us": round(float(np.median(ms)) * 1e3, 2)}))
        return 0

    print("bench: generating inputs", file=sys.stderr, flush=True)
    large = wl.workload(LARGE)
    skinny = wl.workload(SKINNY)
    Wl = torch.from_numpy(large["W"]).to(dev)
    Gl = torch.from_numpy(large["G"]).to(dev)
    Dl = torch.empty((large["T"], large["K"]), dtype=torch.float32, device=dev)
    # several copies of the skinny W (33 MB each) so that consecutive calls
    # cannot be served from the 256 MB Infinity Cache
    n_rot = 12
    Ws = [torch.from_numpy(skinny["W"]).to(dev) for _ in range(n_rot)]
    Gs = torch.from_numpy(skinny["G"]).to(dev)
    Ds = torch.empty((skinny["T"], skinny["K"]), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    v_large = q.choice(q.Q4_K, large["K"], large["N"], large["T"])
    v_skinny = q.choice(q.Q4_K, skinny["K"], skinny["N"], skinny["T"])

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        q.out_prod(q.Q4_K, Wl, Gl, large["K"], out=Dl)
        if ev is not None:
            ev[1].record(stream)
        q.out_prod(q.Q4_K, Ws[i % n_rot], Gs, skinny["K"], out=Ds)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t_large = np.array([e[0].elapsed_time(e[1]) for e in events]) * 1e-3  # seconds
    t_skinny = np.array([e[1].elapsed_time(e[2]) for e in events]) * 1e-3

    fl_large = 2.0 * large["T"] * large["N"] * large["K"]
    fl_skinny = 2.0 * skinny["T"] * skinny["N"] * skinny["K"]
    wbytes = float(skinny["W"].nbytes)
    avg_large = float(t_large.mean())
    avg_skinny = float(t_skinny.mean())
    achieved = fl_large / avg_large / 1e12
    traffic = read_traffic(LARGE_TAG) if q.VARIANT_NAMES[v_large] == KERNELS[LARGE_TAG][2] else None
    ms_per_step = wall / args.steps * 1e3
    value = (fl_large + fl_skinny) / (wall / args.steps) / 1e12

    # The exact-split variant (bf16 MFMA on exact operand parts; opt-in, never
    # chosen automatically) on the large workload, timed after the step loop.
    split = None
    if q.variant_applies(q.VARIANT_SPLIT_128x256, q.Q4_K, large["K"], large["N"], large["T"]):
        for _ in range(2):
            q.out_prod(q.Q4_K, Wl, Gl, large["K"], out=Dl, variant=q.VARIANT_SPLIT_128x256)
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in sev:
            e[0].record(stream)
            q.out_prod(q.Q4_K, Wl, Gl, large["K"], out=Dl, variant=q.VARIANT_SPLIT_128x256)
            e[1].record(stream)
        torch.cuda.synchronize()
        t_split = np.array([e[0].elapsed_time(e[1]) for e in sev]) * 1e-3
        # MFMA work issued per launch: per 128 x 256 tile and 32-row chunk,
        # 384 bf16 32x32x16 products (32768 FLOP each) and 24 16x16x32 ones
        # (16384 FLOP) for the min term
        tiles = -(-large["T"] // 128) * -(-large["K"] // 256)
        chunks = -(-large["N"] // 32)
        issued = tiles * chunks * (384 * 32768 + 24 * 16384)
        avg_split = float(t_split.mean())
        split = {"kernel": "out_prod_split_kernel (split_128x256)", "traffic": read_traffic(f"split_{LARGE}"),
                 "avg_launch_ms": round(avg_split * 1e3, 4),
                 "min_launch_ms": round(float(t_split.min()) * 1e3, 4),
                 "tflops": round(fl_large / avg_split / 1e12, 3),
                 "f32_mfma_roof_frac": round(fl_large / avg_split / 1e12 / PEAK_F32_TFLOPS, 4),
                 "bf16_flops_issued_per_launch": issued,
                 "bf16_mfma_frac": round(issued / avg_split / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "speedup_vs_f32_kernel": round(avg_large / avg_split, 3)}

    # Measured ceilings on this GPU, timed after the rest: MFMA-only loops
    # (no memory traffic) for the F32-input and bf16 instructions, and a
    # 16-byte device copy of 1 GiB (2 GiB over HBM).
    def timed(launch, reps=5):
        launch()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in ev:
            e[0].record(stream)
            launch()
            e[1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3

    sink = q.probe_sink(dev)
    f32_fl = q.probe_mfma(q.PROBE_MFMA_F32, sink, 4096)
    mfma_f32 = f32_fl / timed(lambda: q.probe_mfma(q.PROBE_MFMA_F32, sink, 4096)) / 1e12
    bf16_fl = q.probe_mfma(q.PROBE_MFMA_BF16, sink, 4096)
    mfma_bf16 = bf16_fl / timed(lambda: q.probe_mfma(q.PROBE_MFMA_BF16, sink, 4096)) / 1e12
    csrc = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    cdst = torch.empty_like(csrc)
    copy_gbs = 2.0 * csrc.numel() * 4 / timed(lambda: q.probe_copy(csrc, cdst)) / 1e9
    del csrc, cdst, sink
    ceilings = {"kind": "measured on this GPU: MFMA-only loops (no memory), 16-byte copy of 1 GiB",
                "mfma_f32_tflops": round(mfma_f32, 2), "mfma_bf16_tflops": round(mfma_bf16, 1),
                "copy_gbs": round(copy_gbs, 1),
                "mfma_f32_clock_ghz": round(mfma_f32 / PEAK_F32_TFLOPS * 2.4, 3)}
    if split is not None:
        split["bf16_mfma_frac_of_measured"] = round(split["bf16_flops_issued_per_launch"] / avg_split / 1e12 / mfma_bf16, 4)

    skinny_tflops = fl_skinny / avg_skinny / 1e12
    skinny_gbs = wbytes / avg_skinny / 1e9
    t_roof = max(wbytes / (PEAK_HBM_GBS * 1e9), fl_skinny / (PEAK_F32_TFLOPS * 1e12))

    out = {
        "metric": "OUT_PROD TFLOP/s and weight GB/s vs roofline, Q4_K 4096x14336 T=4096 and T=16",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Q4_K blocks and N(0,1) F32 gradients)",
        "config": {"workload": f"{LARGE} + {SKINNY}", "weight_type": "q4_k",
                   "large_t": {"N": large["N"], "K": large["K"], "T": large["T"],
                               "kernel": q.VARIANT_NAMES[v_large]},
                   "skinny": {"N": skinny["N"], "K": skinny["K"], "T": skinny["T"],
                              "kernel": q.VARIANT_NAMES[v_skinny], "w_copies_rotated": n_rot}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_F32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_F32_TFLOPS, 4),
                     "frac_of_measured": round(achieved / mfma_f32, 4),
                     "traffic": traffic,
                     "kernel": f"{kernel_family(q.VARIANT_NAMES[v_large])} ({q.VARIANT_NAMES[v_large]})",
                     "avg_launch_ms": round(avg_large * 1e3, 4), "min_launch_ms": round(float(t_large.min()) * 1e3, 4),
                     "flops_per_launch": fl_large},
        "skinny": {"kernel": "out_prod_skinny_kernel", "traffic": read_traffic(SKINNY_TAG),
                   "avg_launch_us": round(avg_skinny * 1e6, 3),
                   "min_launch_us": round(float(t_skinny.min()) * 1e6, 3),
                   "tflops": round(skinny_tflops, 3), "weight_gbs": round(skinny_gbs, 1),
                   "hbm_frac": round(skinny_gbs / PEAK_HBM_GBS, 4),
                   "f32_mfma_frac": round(skinny_tflops / PEAK_F32_TFLOPS, 4),
                   "f32_mfma_frac_of_measured": round(skinny_tflops / mfma_f32, 4),
                   "hbm_frac_of_measured_copy": round(skinny_gbs / copy_gbs, 4),
                   "binding_roof_frac": round(t_roof / avg_skinny, 4),
                   "weight_bytes": wbytes},
        "exact_split": split,
        "ceilings": ceilings,
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(large)
        out["cpu_baseline_skinny"] = cpu_baseline_skinny(skinny)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
