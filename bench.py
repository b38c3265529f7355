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

After the step loop the same process times every benchmarked workload at
the kernel retro_out_prod chooses for it (the tiny Q8_0 case, the dense
4096 x 4096 weight in F32, F16 and BF16, Q4_0 17408 x 5120, and the two
Q4_K shapes), each as back-to-back launches between two HIP events, and
reports them under "workloads".

Prints ONE JSON line. --gpus N > 1 is refused: the path runs on one GPU.
"""

from __future__ import annotations

import argparse
import csv
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
# T = 16 through the other matrix of the MLP: 64 slabs of dst (the workspace
# call's n-split kernel against the skinny kernel, reported beside the step)
SKINNY_FEW = "q4_k_n14336_k4096_t16"
# Every benchmarked workload: (workload, dense storage type or "").
WORKLOADS = [
    ("q8_0_n128_k256_t64", ""),
    ("dense_n4096_k4096_t512", "f32"),
    ("dense_n4096_k4096_t512", "f16"),
    ("dense_n4096_k4096_t512", "bf16"),
    ("q4_0_n17408_k5120_t2048", ""),
    (LARGE, ""),
    (SKINNY, ""),
]
# W copies rotated between launches of a workload whose weight could stay
# in the 256 MB Infinity Cache across launches and is read at the HBM rate
# (the small-T shape; the others are bound by the matrix rate)
ROTATE = {SKINNY: 12}
PROFILES = os.path.join(REPO, "profiles")
KERNEL_SOURCES = ["quantized_weight_backward_amd/csrc/retro_kernels.h",
                  "quantized_weight_backward_amd/csrc/retro_split_kernel.h",
                  "quantized_weight_backward_amd/csrc/retro_unit.hip",
                  "quantized_weight_backward_amd/csrc/retro_host.h",
                  "quantized_weight_backward_amd/csrc/retro_ws_kernel.h",
                  "quantized_weight_backward_amd/csrc/retro_decode.h",
                  "quantized_weight_backward_amd/csrc/retro_api.hip"]
TYPE_IDS = {"q8_0": 8, "q4_0": 2, "q4_k": 12, "f32": 0, "f16": 1, "bf16": 30, "mxfp4": 39}


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


def workload_tag(workload: str, dense: str) -> str:
    """dense_n4096_k4096_t512 + f16 -> f16_n4096_k4096_t512; others unchanged."""
    return workload.replace("dense", dense) if dense else workload


def kernel_family(variant: str) -> str:
    head = variant.split("_")[0]
    return {"ws": "out_prod_ws_kernel", "ws2": "out_prod_ws_kernel", "tile": "out_prod_tile_kernel",
            "split": "out_prod_split_kernel"}.get(head, "out_prod_skinny_kernel")


# Template arguments (WA, WB, CT, NG, NC) of the producer/consumer kernel of
# each variant, as the launches instantiate it (G stored by rows).
WS_ARGS = {"ws_256x256": "4, 2, 2, 1, 8", "ws_128x256": "2, 4, 2, 1, 4", "ws_64x256": "1, 4, 2, 1, 4",
           "ws_32x256": "1, 2, 1, 1, 4", "ws_128x128": "2, 2, 2, 1, 4", "ws_64x128": "1, 2, 2, 1, 4",
           "ws2_64x128": "1, 2, 2, 2, 4", "ws_32x128": "1, 1, 1, 1, 4"}


def kernel_prefix(variant: str, wtype: int) -> str:
    """Start of the demangled kernel name rocprofv3 reports for a variant
    and weight type: the producer/consumer kernel's full template argument
    list, so that the two launches of a plan are told apart."""
    if variant in WS_ARGS:
        return f"void retro::out_prod_ws_kernel<{wtype}, {WS_ARGS[variant]}, false>"
    return f"void retro::{kernel_family(variant)}<{wtype},"


def launch_plan(q, wtype: int, K: int, N: int, T: int) -> list[tuple[str, int, int]]:
    """The launches out_prod makes: [(variant name, first column, end column)]."""
    v0, ks, v1 = q.plan(wtype, K, N, T)
    parts = [(q.VARIANT_NAMES[v0], 0, ks)]
    if ks < K:
        parts.append((q.VARIANT_NAMES[v1], ks, K))
    return parts


def plan_label(parts) -> str:
    """ws_64x128, or ws_128x256[0:4096]+ws2_64x128[4096:5120]."""
    if len(parts) == 1:
        return parts[0][0]
    return "+".join(f"{v}[{a}:{b}]" for v, a, b in parts)


def plan_tag(parts) -> str:
    """File-name part of a plan: ws_64x128, or ws_128x256+ws2_64x128."""
    return "+".join(v for v, _, _ in parts)


def call_durations(trace_csv: str, prefixes: list[str], drop: int) -> tuple[list[str], list[list[float]], list[float]]:
    """Per-launch durations of each launch of a call (one kernel per prefix,
    distinct), and their per-call sums."""
    names, per = [], []
    for prefix in prefixes:
        name, durs = steady_dispatches(trace_csv, prefix, drop)
        names.append(name)
        per.append(durs)
    n = min(len(d) for d in per)
    return names, per, [sum(d[i] for d in per) for i in range(n)]


def read_profile_value(tag: str, key: str):
    """A value recorded in profiles/<tag>_traffic.md, or None when the
    summary is missing or the kernels changed since it was taken."""
    path = os.path.join(PROFILES, f"{tag}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"source_sha256:\s*(\w+)", text)
    val = re.search(key + r":\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


def read_traffic(tag: str):
    return read_profile_value(tag, "hbm_bytes_per_launch")


# The default step loop. The profiled runs leave out the few-slab comparison,
# whose skinny launches (another shape of the same kernel) would mix into the
# step kernel's figures; its two kernels have traces of their own (CASE_TRACES).
BENCH_PROFILE_ARGS = "--steps 20 --warmup 5 --reps 20 --no-cpu-baseline --no-few-slab"
COUNTER_ARGS = "--steps 3 --warmup 1 --reps 3 --min-ms 0 --no-cpu-baseline --no-few-slab"
PROFILE_WARMUP = 5  # launches of each kernel dropped from a trace summary (the bench's warm-up steps)
PROFILE_STEPS = 20  # the timed steps that follow them
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d {out}/prof_trace -o run -- "
             f"python3 bench.py {BENCH_PROFILE_ARGS}",
    "FETCH_SIZE": "rocprofv3 --pmc FETCH_SIZE -f csv -d {out}/pmc_FETCH_SIZE -o run -- "
                  f"python3 bench.py {COUNTER_ARGS}",
    "WRITE_SIZE": "rocprofv3 --pmc WRITE_SIZE -f csv -d {out}/pmc_WRITE_SIZE -o run -- "
                  f"python3 bench.py {COUNTER_ARGS}",
    "mfma": "rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES "
            "GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS -f csv "
            f"-d {{out}}/pmc_mfma -o run -- python3 bench.py {COUNTER_ARGS}",
    "waits": "rocprofv3 --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_INSTS_SALU "
             f"SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_MISC -f csv -d {{out}}/pmc_waits -o run -- python3 bench.py "
             f"{COUNTER_ARGS}",
    "tcc_req": "rocprofv3 --pmc TCC_EA0_RDREQ TCC_EA0_RDREQ_32B TCC_EA0_RDREQ_64B TCC_EA0_RDREQ_128B -f csv "
               f"-d {{out}}/pmc_tcc_req -o run -- python3 bench.py {COUNTER_ARGS}",
    "tcc_hit": "rocprofv3 --pmc TCC_HIT TCC_MISS TCC_EA0_RDREQ_DRAM -f csv "
               f"-d {{out}}/pmc_tcc_hit -o run -- python3 bench.py {COUNTER_ARGS}",
    "copy_FETCH_SIZE": "rocprofv3 --pmc FETCH_SIZE -f csv -d {out}/pmc_copy_FETCH_SIZE -o run -- "
                       "python3 bench.py --copy-probe-mib 1024",
    "copy_WRITE_SIZE": "rocprofv3 --pmc WRITE_SIZE -f csv -d {out}/pmc_copy_WRITE_SIZE -o run -- "
                       "python3 bench.py --copy-probe-mib 1024",
}
# Counter passes summarised per kernel (each a rocprofv3 run of its own).
COUNTER_PASSES = ("mfma", "waits", "tcc_req", "tcc_hit")
# Kernel traces of single cases outside the benchmark run (opt-in variants,
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
                                            "void retro::mul_mat_skinny_kernel<12,"),
    # T = 16 with 64 slabs of dst: the skinny kernel, then the workspace
    # call's n-split form
    "skinny_q4_k_n14336_k4096_t16": (SKINNY_FEW, "", "out_prod", "skinny",
                                     "void retro::out_prod_skinny_kernel<12, 8, true, 1>"),
    "skinny_split_q4_k_n14336_k4096_t16": (SKINNY_FEW, "", "out_prod_ws", "skinny_split",
                                           "void retro::out_prod_skinny_split_kernel<12, 8, 1>"),
}
CASE_WARMUP = 2  # launches --profile-case makes before its timed ones


def case_trace_command(tag: str, run_dir: str) -> str:
    workload, wtype, op, variant, _ = CASE_TRACES[tag]
    out = os.path.relpath(run_dir, REPO).rstrip("/")
    dense = f" --wtype {wtype}" if wtype else ""
    return (f"rocprofv3 --kernel-trace --stats -f csv -d {out}/trace_{tag} -o run -- python3 bench.py "
            f"--profile-case {workload}{dense} --op {op} --variant {variant} --launches 10")


def profile_command(name: str, run_dir: str) -> str:
    """The rocprofv3 command of PROFILE_COMMANDS[name] writing under run_dir."""
    return PROFILE_COMMANDS[name].format(out=os.path.relpath(run_dir, REPO).rstrip("/"))


def _find_csv(run_dir: str, sub: str, suffix: str) -> str | None:
    """rocprofv3 writes <out>/<host>/<pid>_... or <out>/run_<suffix>; find it."""
    base = os.path.join(run_dir, sub)
    for root, _, files in os.walk(base):
        for f in sorted(files):
            if f.endswith(suffix):
                return os.path.join(root, f)
    return None


def steady_dispatches(trace_csv: str, prefix: str, drop: int) -> tuple[str, list[float]]:
    """Durations (ns) of the dispatches of the one kernel whose name starts
    with prefix, in launch order, without the first `drop` (warm-up)."""
    rows = [r for r in csv.DictReader(open(trace_csv)) if r["Kernel_Name"].startswith(prefix)]
    names = {r["Kernel_Name"] for r in rows}
    if len(names) != 1:
        raise RuntimeError(f"{prefix}: expected one kernel, found {sorted(names)}")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]
    return names.pop(), durs[drop:]


def _counter_means(path: str, prefix: str, drop: int = 1) -> dict:
    """Per-dispatch counter values of one kernel (the first `drop`
    dispatches, warm-up, excluded), averaged per counter."""
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Kernel_Name"].startswith(prefix):
            per.setdefault(r["Counter_Name"], {}).setdefault(int(r["Dispatch_Id"]), 0.0)
            per[r["Counter_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    out = {}
    for name, by_dispatch in per.items():
        vals = [by_dispatch[d] for d in sorted(by_dispatch)][drop:] or list(by_dispatch.values())
        out[name] = (sum(vals) / len(vals), len(vals))
    return out


def _copy_scale(run_dir: str, sub: str, counter: str) -> tuple[float, float]:
    path = _find_csv(run_dir, sub, "counter_collection.csv")
    vals = _counter_means(path, "__amd_rocclr_copyBuffer", drop=0)
    kib = vals[counter][0]
    return kib, (1024 << 20) / (kib * 1024)


def _stats_row(name: str, durs: list[float], steps: int = 0) -> list[str]:
    """Table of launch durations (ns in, us out). With steps > 0 the first
    `steps` durations are the benchmark's timed step loop, given a row of
    their own."""
    def row(label, part):
        us = [d / 1e3 for d in part]
        return (f"| {label} | {len(us)} | {sum(us) / len(us):.2f} | {sorted(us)[len(us) // 2]:.2f} | {min(us):.2f} | "
                f"{max(us):.2f} |")
    rows = [row("timed steps", durs[:steps])] if steps else []
    return [f"Kernel: `{name}`", "",
            "| launches | count | mean (us) | median (us) | min (us) | max (us) |", "|---|---|---|---|---|---|",
            *rows, row("all after warm-up", durs), ""]


def summarize(run_dir: str) -> None:
    """Write profiles/<tag>_trace.md, <tag>_traffic.md and <tag>_counters.md
    for every benchmarked workload's kernel, from rocprofv3 output under
    run_dir (the commands in PROFILE_COMMANDS with {out} = run_dir, run from
    the repository root). Trace figures are over steady-state dispatches only
    (each kernel's first PROFILE_WARMUP launches dropped)."""
    import quantized_weight_backward_amd as q
    import workloads as wl

    os.makedirs(PROFILES, exist_ok=True)
    src = kernel_source_hash()
    trace_csv = _find_csv(run_dir, "prof_trace", "kernel_trace.csv")
    f_copy, f_scale = _copy_scale(run_dir, "pmc_copy_FETCH_SIZE", "FETCH_SIZE")
    w_copy, w_scale = _copy_scale(run_dir, "pmc_copy_WRITE_SIZE", "WRITE_SIZE")
    fetch_csv = _find_csv(run_dir, "pmc_FETCH_SIZE", "counter_collection.csv")
    write_csv = _find_csv(run_dir, "pmc_WRITE_SIZE", "counter_collection.csv")
    for workload, dense in WORKLOADS:
        c = wl.WORKLOADS[workload]
        wtype = TYPE_IDS[dense] if dense else c["type"]
        parts = launch_plan(q, wtype, c["K"], c["N"], c["T"])
        prefixes = [kernel_prefix(v, wtype) for v, _, _ in parts]
        variant = plan_label(parts)
        tag = f"{plan_tag(parts)}_{workload_tag(workload, dense)}"
        names, per, durs = call_durations(trace_csv, prefixes, PROFILE_WARMUP)
        flops = 2.0 * c["T"] * c["N"] * c["K"]
        # the two step kernels: their first PROFILE_STEPS launches after the
        # warm-up are the timed step loop, the bench's own figure
        steps = PROFILE_STEPS if workload in (LARGE, SKINNY) else 0
        head = durs[:steps] if steps else durs
        mean_s = sum(head) / len(head) / 1e9
        part_rows = []
        if len(parts) > 1:
            for (v, a, b), n, d in zip(parts, names, per):
                part_rows += [f"Launch over dst columns [{a}, {b}) ({v}):", "", *_stats_row(n, d)]
            part_rows += ["Per call (the two launches summed):", ""]
        lines = [f"# {tag}: rocprofv3 kernel trace", "",
                 f"Command (repository root): `{profile_command('trace', run_dir)}`", "",
                 f"Workload {workload_tag(workload, dense)}, the launches retro_out_prod makes ({variant}). "
                 f"The first {PROFILE_WARMUP} launches of each kernel (the benchmark's warm-up) are left out"
                 + (f"; the next {steps} are the timed step loop." if steps else "."), "",
                 *part_rows,
                 *(_stats_row(names[0], durs, steps) if len(parts) == 1 else
                   _stats_row(" + ".join(names), durs, steps)),
                 "Figures below at the mean of the " + ("timed steps." if steps else "launches after warm-up."), "",
                 f"F32 TFLOP/s at the mean: {flops / mean_s / 1e12:.2f} "
                 f"(2*T*N*K = {flops:.6g}); fraction of the 157.3 TFLOP/s F32 peak: "
                 f"{flops / mean_s / 1e12 / PEAK_F32_TFLOPS:.4f}", ""]
        if workload == SKINNY:
            wbytes = c["N"] * wl.row_bytes(wtype, c["K"])
            t_roof = max(wbytes / (PEAK_HBM_GBS * 1e9), flops / (PEAK_F32_TFLOPS * 1e12))
            lines += [f"Weight GB/s at the mean: {wbytes / mean_s / 1e9:.1f}; fraction of the binding roof "
                      f"(max of weight bytes / 8 TB/s and FLOPs / 157.3 TFLOP/s = {t_roof * 1e6:.2f} us): "
                      f"{t_roof / mean_s:.4f}", ""]
        lines += [f"kernel source_sha256: {src}", ""]
        open(os.path.join(PROFILES, f"{tag}_trace.md"), "w").write("\n".join(lines))
        # per call: the launches' per-dispatch means added
        fetch = [sum(_counter_means(fetch_csv, p)["FETCH_SIZE"][0] for p in prefixes),
                 min(_counter_means(fetch_csv, p)["FETCH_SIZE"][1] for p in prefixes)]
        write = [sum(_counter_means(write_csv, p)["WRITE_SIZE"][0] for p in prefixes),
                 min(_counter_means(write_csv, p)["WRITE_SIZE"][1] for p in prefixes)]
        hbm = fetch[0] * 1024 * f_scale + write[0] * 1024 * w_scale
        lines = [f"# {tag}: HBM traffic per call (rocprofv3 counters)", "",
                 "Commands (repository root):", "",
                 *[f"- `{profile_command(k, run_dir)}`" for k in ("FETCH_SIZE", "WRITE_SIZE", "copy_FETCH_SIZE",
                                                           "copy_WRITE_SIZE")], "",
                 "Calibration: a 1 GiB device-to-device copy reads and writes 1073741824 bytes; the counters "
                 f"read FETCH_SIZE = {f_copy:.1f} KiB and WRITE_SIZE = {w_copy:.1f} KiB per copy launch, so "
                 f"FETCH_SIZE is scaled by {f_scale:.4f} and WRITE_SIZE by {w_scale:.4f}.", "",
                 *([f"The call makes {len(parts)} launches ({variant}); each counter is the sum of their "
                     "per-dispatch means.", ""] if len(parts) > 1 else []),
                 "| counter | KiB per call (mean) | calls | scaled bytes |", "|---|---|---|---|",
                 f"| FETCH_SIZE | {fetch[0]:.1f} | {fetch[1]} | {fetch[0] * 1024 * f_scale:.4g} |",
                 f"| WRITE_SIZE | {write[0]:.1f} | {write[1]} | {write[0] * 1024 * w_scale:.4g} |", "",
                 f"hbm_bytes_per_launch: {hbm:.6g}",
                 f"source_sha256: {src}", ""]
        open(os.path.join(PROFILES, f"{tag}_traffic.md"), "w").write("\n".join(lines))
        write_counter_summary(tag, prefixes, c, run_dir, src)
        print(f"{tag}: mean {sum(durs) / len(durs) / 1e3:.2f} us over {len(durs)}, traffic {hbm / 1e6:.1f} MB")
    # the opt-in exact split, timed after the step loop on the large workload
    c = wl.WORKLOADS[LARGE]
    prefix, tag = "void retro::out_prod_split_kernel<12>", f"split_128x256_{LARGE}"
    name, durs = steady_dispatches(trace_csv, prefix, 2)
    flops = 2.0 * c["T"] * c["N"] * c["K"]
    mean_s = sum(durs) / len(durs) / 1e9
    lines = [f"# {tag}: rocprofv3 kernel trace", "",
             f"Command (repository root): `{profile_command('trace', run_dir)}`", "",
             f"Workload {LARGE}, the opt-in exact split (split_128x256); its first 2 launches (warm-up) are left "
             "out.", "", *_stats_row(name, durs),
             f"Algorithmic F32-equivalent TFLOP/s at the mean: {flops / mean_s / 1e12:.2f} "
             f"({flops / mean_s / 1e12 / PEAK_F32_TFLOPS:.4f} of the F32 peak)", "",
             f"kernel source_sha256: {src}", ""]
    open(os.path.join(PROFILES, f"{tag}_trace.md"), "w").write("\n".join(lines))
    fetch = _counter_means(fetch_csv, prefix)["FETCH_SIZE"]
    write = _counter_means(write_csv, prefix)["WRITE_SIZE"]
    hbm = fetch[0] * 1024 * f_scale + write[0] * 1024 * w_scale
    lines = [f"# {tag}: HBM traffic per launch (rocprofv3 counters)", "", "Commands (repository root):", "",
             *[f"- `{profile_command(k, run_dir)}`" for k in ("FETCH_SIZE", "WRITE_SIZE", "copy_FETCH_SIZE",
                                                       "copy_WRITE_SIZE")], "",
             f"FETCH_SIZE scaled by {f_scale:.4f} and WRITE_SIZE by {w_scale:.4f} (1 GiB copy calibration).", "",
             "| counter | KiB per launch (mean) | launches | scaled bytes |", "|---|---|---|---|",
             f"| FETCH_SIZE | {fetch[0]:.1f} | {fetch[1]} | {fetch[0] * 1024 * f_scale:.4g} |",
             f"| WRITE_SIZE | {write[0]:.1f} | {write[1]} | {write[0] * 1024 * w_scale:.4g} |", "",
             f"hbm_bytes_per_launch: {hbm:.6g}", f"source_sha256: {src}", ""]
    open(os.path.join(PROFILES, f"{tag}_traffic.md"), "w").write("\n".join(lines))
    write_counter_summary(tag, [prefix], c, run_dir, src)
    print(f"{tag}: mean {sum(durs) / len(durs) / 1e3:.2f} us, traffic {hbm / 1e6:.1f} MB")
    for tag, (workload, dense, op, variant, prefix) in CASE_TRACES.items():
        path = _find_csv(run_dir, f"trace_{tag}", "kernel_trace.csv")
        if not path:
            continue
        name, durs = steady_dispatches(path, prefix, CASE_WARMUP)
        lines = [f"# {tag}: rocprofv3 kernel trace", "",
                 f"Command (repository root): `{case_trace_command(tag, run_dir)}`", "",
                 f"{op}, workload {workload_tag(workload, dense)}, variant {variant}; the first {CASE_WARMUP} "
                 "launches (warm-up) are left out.", "",
                 *_stats_row(name, durs), f"kernel source_sha256: {src}", ""]
        open(os.path.join(PROFILES, f"{tag}_trace.md"), "w").write("\n".join(lines))
        print(f"{tag}: mean {sum(durs) / len(durs) / 1e3:.2f} us")


def write_counter_summary(tag: str, prefixes: list[str], case: dict, run_dir: str, src: str) -> None:
    """profiles/<tag>_counters.md: per-call means of the counter passes (the
    per-dispatch means of a call's launches added), with the F32 MFMA work
    checked against 2*T*N*K (one MOP = 512 FLOPs)."""
    mean, commands = {}, []
    for p in COUNTER_PASSES:
        path = _find_csv(run_dir, f"pmc_{p}", "counter_collection.csv")
        if path:
            for prefix in prefixes:
                for k, v in _counter_means(path, prefix).items():
                    mean[k] = mean.get(k, 0.0) + v[0]
            commands.append(profile_command(p, run_dir))
    if not mean:
        return
    flops = 2.0 * case["T"] * case["N"] * case["K"]
    lines = [f"# {tag}: counters per call (rocprofv3)", "", "Commands (repository root), one pass each:", "",
             *[f"- `{c}`" for c in commands], "",
             *([f"The call makes {len(prefixes)} launches; each counter is the sum of their per-dispatch means.", ""]
               if len(prefixes) > 1 else []),
             "| counter | mean per call |", "|---|---|",
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
    wcyc, wany = mean.get("SQ_WAVE_CYCLES"), mean.get("SQ_WAIT_ANY")
    if wcyc and wany:
        lines += [f"Waves waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES) = {wany / wcyc:.4f}", ""]
    req = mean.get("TCC_EA0_RDREQ_sum") or mean.get("TCC_EA0_RDREQ")
    if req:
        b32 = mean.get("TCC_EA0_RDREQ_32B_sum") or mean.get("TCC_EA0_RDREQ_32B") or 0.0
        b64 = mean.get("TCC_EA0_RDREQ_64B_sum") or mean.get("TCC_EA0_RDREQ_64B") or 0.0
        b128 = mean.get("TCC_EA0_RDREQ_128B_sum") or mean.get("TCC_EA0_RDREQ_128B") or 0.0
        lines += [f"L2-to-memory read requests: {req:.6g} (32 B: {b32:.6g}, 64 B: {b64:.6g}, 128 B: {b128:.6g}); "
                  f"bytes by size {32 * b32 + 64 * b64 + 128 * b128:.6g}", ""]
    hit, miss = mean.get("TCC_HIT_sum") or mean.get("TCC_HIT"), mean.get("TCC_MISS_sum") or mean.get("TCC_MISS")
    if hit is not None and miss:
        lines += [f"L2 hit rate TCC_HIT / (TCC_HIT + TCC_MISS) = {hit / (hit + miss):.4f}", ""]
    lines += [f"source_sha256: {src}", ""]
    open(os.path.join(PROFILES, f"{tag}_counters.md"), "w").write("\n".join(lines))


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            return next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        return ""


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
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "host_cpu": host_cpu(), "host_threads": os.cpu_count(),
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


def oracle_timing(case: dict) -> dict:
    """The CPU oracle beside a workload's GPU figure: single-threaded, median of
    3 calls (100 for shapes under 10 MFLOP), on all t rows or, for the larger
    shapes, a bounded sample of them (threaded over t rows on up to 16 host
    threads when even the sample is large)."""
    import numpy as np

    import oracle

    T, N, K = case["T"], case["N"], case["K"]
    full = 2.0 * T * N * K
    threads, rows = 1, T
    if full > 1e11:  # hundreds of GFLOP: threaded over a sample of t rows
        threads = max(1, min(16, os.cpu_count() or 1))
        rows = min(T, 16 * threads)
    elif full > 1e10:  # tens of GFLOP: one thread on a sample of t rows
        rows = min(T, 16)
    sel = np.arange(rows)
    repeats = 100 if full < 1e7 else 3
    secs = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        oracle.out_prod(case["type"], case["W"], case["G"], K, rows=sel, nthreads=threads)
        secs.append(time.perf_counter() - t0)
    med = float(np.median(secs))
    return {"value": 2.0 * N * K * rows / med / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {T} t rows (full decode of W included), median of {repeats}: {med:.4f} s"}


def smi_under_load(enqueue) -> dict:
    """Graphics clocks and socket power that amd-smi reports while about 4 s
    of queued GPU work run (enqueue() queues them before the query, so the
    query lands inside them)."""
    import subprocess

    import torch

    enqueue()
    res = {"source": "amd-smi metric -c -p --json"}
    try:
        time.sleep(0.5)
        txt = subprocess.run(["amd-smi", "metric", "-c", "-p", "--json"], capture_output=True, text=True,
                             timeout=20).stdout
        gpu = json.loads(txt)["gpu_data"][0]
        clk = gpu["clock"]
        gfx = sorted(k for k in clk if k.startswith("gfx_"))
        res["gfx_mhz"] = [clk[k]["clk"]["value"] for k in gfx]
        res["max_mhz"] = clk[gfx[0]]["max_clk"]["value"]
        res["socket_power_w"] = gpu.get("power", {}).get("socket_power", {}).get("value")
    except Exception as exc:  # the tool may be absent or print something else
        res["error"] = f"{type(exc).__name__}: {exc}"[:200]
    torch.cuda.synchronize()
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=20, help="launches per workload timed after the steps (at least)")
    ap.add_argument("--min-ms", type=float, default=100.0,
                    help="each back-to-back batch covers at least this many ms of launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-few-slab", action="store_true",
                    help="leave out the T = 16, 64-slab comparison of retro_out_prod and retro_out_prod_ws")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device-to-device copy of this size (counter calibration)")
    ap.add_argument("--profile-case", metavar="WORKLOAD", default=None,
                    help="only run one workload LAUNCHES times (for a kernel trace) and exit")
    ap.add_argument("--wtype", default="", help="with --profile-case: f32, f16 or bf16 for the dense workload")
    ap.add_argument("--op", choices=("out_prod", "out_prod_ws", "mul_mat"), default="out_prod")
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
    ids = {v: k for k, v in q.VARIANT_NAMES.items()}

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
        vid = 0 if args.variant == "auto" else ids[args.variant]
        W = torch.from_numpy(c["W"]).to(dev)
        if args.op == "out_prod":
            G = torch.from_numpy(c["G"]).to(dev)
            out = torch.empty((c["T"], c["K"]), dtype=torch.float32, device=dev)
            call = lambda: q.out_prod(c["type"], W, G, c["K"], out=out, variant=vid)
        elif args.op == "out_prod_ws":
            G = torch.from_numpy(c["G"]).to(dev)
            out = torch.empty((c["T"], c["K"]), dtype=torch.float32, device=dev)
            wsp = q.new_workspace(dev)
            call = lambda: q.out_prod_ws(c["type"], W, G, c["K"], wsp, out=out, variant=vid)
        else:
            X = torch.randn((c["T"], c["K"]), device=dev)
            out = torch.empty((c["T"], c["N"]), dtype=torch.float32, device=dev)
            call = lambda: q.mul_mat(c["type"], W, X, out=out, variant=vid)
        for _ in range(CASE_WARMUP):
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
    n_rot = ROTATE[SKINNY]
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

    print("bench: timing the step", file=sys.stderr, flush=True)
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
    achieved = fl_large / avg_large / 1e12
    ms_per_step = wall / args.steps * 1e3
    value = (fl_large + fl_skinny) / (wall / args.steps) / 1e12
    large_tag = f"{q.VARIANT_NAMES[v_large]}_{LARGE}"
    skinny_tag = f"{q.VARIANT_NAMES[v_skinny]}_{SKINNY}"

    def back_to_back(call, reps):
        """Mean launch time (s) of `reps` launches enqueued back to back
        between two HIP events on the launch stream. One launch of the
        large-T kernel (about 3.6 ms of matrix work) goes first, so that the
        host has queued every timed launch before the first event completes:
        host launch overhead cannot leave the GPU idle between them, and the
        GPU clock is at its loaded level (an idle spin lets it drop)."""
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q.out_prod(q.Q4_K, Wl, Gl, large["K"], out=Dl)
        b0.record(stream)
        for i in range(reps):
            call(i)
        b1.record(stream)
        torch.cuda.synchronize()
        return b0.elapsed_time(b1) * 1e-3 / reps

    # The small-T kernel on its own: launch pairs inside the step include the
    # events' own overhead (a few us against a ~25 us kernel), so its figures
    # come from launches back to back on rotated W copies.
    def batch_reps(est_s):
        """Launches in a back-to-back batch: at least --reps and two rounds of
        the rotated copies, and enough to cover --min-ms (at most 5000)."""
        return max(args.reps, 2 * n_rot, min(5000, int(np.ceil(args.min_ms * 1e-3 / max(est_s, 1e-7)))))

    call_skinny = lambda i: q.out_prod(q.Q4_K, Ws[i % n_rot], Gs, skinny["K"], out=Ds)  # noqa: E731
    skinny_reps = batch_reps(float(np.median(t_skinny)))
    avg_skinny = back_to_back(call_skinny, skinny_reps)

    # Every benchmarked workload at the kernel retro_out_prod chooses.
    print("bench: timing every workload", file=sys.stderr, flush=True)
    per_workload = []
    oracle_cases = []  # (entry, case) timed on the CPU after all GPU work
    for workload, dense in WORKLOADS:
        if workload == LARGE:
            c, W_list, G, D = large, [Wl], Gl, Dl
        elif workload == SKINNY:
            c, W_list, G, D = skinny, Ws, Gs, Ds
        else:
            c = wl.workload(workload, TYPE_IDS[dense] if dense else None)
            W_list = [torch.from_numpy(c["W"]).to(dev) for _ in range(ROTATE.get(workload, 1))]
            G = torch.from_numpy(c["G"]).to(dev)
            D = torch.empty((c["T"], c["K"]), dtype=torch.float32, device=dev)
        wtype, K, N, T = c["type"], c["K"], c["N"], c["T"]
        parts = launch_plan(q, wtype, K, N, T)
        variant = plan_label(parts)
        call = lambda i: q.out_prod(wtype, W_list[i % len(W_list)], G, K, out=D)  # noqa: E731
        for i in range(5):
            call(i)
        torch.cuda.synchronize()
        # The mean launch time from one back-to-back batch of at least
        # --min-ms (sized from 5 launches timed together); then per-launch
        # event pairs (median, min), with the clock at its loaded level.
        npairs = max(args.reps, 2 * len(W_list))
        est = back_to_back(call, 5)
        reps = max(npairs, min(5000, int(np.ceil(args.min_ms * 1e-3 / est))))
        sec = back_to_back(call, reps)
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(npairs)]
        for i, e in enumerate(pev):
            e[0].record(stream)
            call(i)
            e[1].record(stream)
        torch.cuda.synchronize()
        pairs = np.array([e[0].elapsed_time(e[1]) for e in pev]) * 1e-3
        flops = 2.0 * T * N * K
        wb = float(c["W"].nbytes)
        t_roof = max(wb / (PEAK_HBM_GBS * 1e9), flops / (PEAK_F32_TFLOPS * 1e12))
        tag = f"{plan_tag(parts)}_{workload_tag(workload, dense)}"
        per_workload.append({
            "workload": workload_tag(workload, dense), "weight_type": wl.TYPE_NAMES[wtype], "kernel": variant,
            "launches": reps, "launches_per_call": len(parts), "avg_launch_us": round(sec * 1e6, 3),
            "event_pairs": {"launches": npairs, "median_us": round(float(np.median(pairs)) * 1e6, 3),
                            "min_us": round(float(pairs.min()) * 1e6, 3)},
            "tflops": round(flops / sec / 1e12, 3),
            "f32_mfma_frac": round(flops / sec / 1e12 / PEAK_F32_TFLOPS, 4),
            "weight_gbs": round(wb / sec / 1e9, 1), "hbm_frac_weights": round(wb / sec / 1e9 / PEAK_HBM_GBS, 4),
            "binding_roof": "f32_mfma" if flops / (PEAK_F32_TFLOPS * 1e12) >= wb / (PEAK_HBM_GBS * 1e9) else "hbm",
            "binding_roof_frac": round(t_roof / sec, 4), "traffic": read_traffic(tag),
            "w_copies_rotated": len(W_list)})
        if workload not in (LARGE, SKINNY):
            oracle_cases.append((per_workload[-1], c))
            del W_list, G, D
            torch.cuda.empty_cache()

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
        split = {"kernel": "out_prod_split_kernel (split_128x256)",
                 "traffic": read_traffic(f"split_128x256_{LARGE}"),
                 "avg_launch_ms": round(avg_split * 1e3, 4),
                 "min_launch_ms": round(float(t_split.min()) * 1e3, 4),
                 "tflops": round(fl_large / avg_split / 1e12, 3),
                 "f32_mfma_roof_frac": round(fl_large / avg_split / 1e12 / PEAK_F32_TFLOPS, 4),
                 "bf16_flops_issued_per_launch": issued,
                 "bf16_mfma_frac": round(issued / avg_split / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "speedup_vs_f32_kernel": round(avg_large / avg_split, 3)}

    # T = 16 with few slabs of dst (64 for K = 4096): retro_out_prod's skinny
    # kernel against retro_out_prod_ws, whose n-split kernel spreads the rows
    # of W over every CU; rotated W copies, back-to-back batches.
    skinny_split = None
    few = None if args.no_few_slab else wl.workload(SKINNY_FEW)
    if few is not None:
        few_W = [torch.from_numpy(few["W"]).to(dev) for _ in range(ROTATE[SKINNY])]
        few_G = torch.from_numpy(few["G"]).to(dev)
        few_D = torch.empty((few["T"], few["K"]), dtype=torch.float32, device=dev)
        few_ws = q.new_workspace(dev)
        few_calls = {
            "skinny": lambda i: q.out_prod(q.Q4_K, few_W[i % len(few_W)], few_G, few["K"], out=few_D),
            "workspace": lambda i: q.out_prod_ws(q.Q4_K, few_W[i % len(few_W)], few_G, few["K"], few_ws, out=few_D),
        }
        few_fl = 2.0 * few["T"] * few["N"] * few["K"]
        few_t = {}
        for name, call in few_calls.items():
            for i in range(5):
                call(i)
            torch.cuda.synchronize()
            few_t[name] = back_to_back(call, batch_reps(back_to_back(call, 5)))
        few_roof = max(float(few["W"].nbytes) / (PEAK_HBM_GBS * 1e9), few_fl / (PEAK_F32_TFLOPS * 1e12))
        skinny_split = {
            "workload": SKINNY_FEW, "slabs_of_dst": -(-few["K"] // 64),
            "workspace_bytes": q.workspace_size(q.Q4_K, few["K"], few["N"], few["T"]),
            "skinny": {"kernel": "out_prod_skinny_kernel (retro_out_prod)", "avg_launch_us": round(few_t["skinny"] * 1e6, 3),
                       "f32_mfma_frac": round(few_fl / few_t["skinny"] / 1e12 / PEAK_F32_TFLOPS, 4),
                       "binding_roof_frac": round(few_roof / few_t["skinny"], 4)},
            "workspace": {"kernel": "out_prod_skinny_split_kernel (retro_out_prod_ws)",
                          "avg_launch_us": round(few_t["workspace"] * 1e6, 3),
                          "f32_mfma_frac": round(few_fl / few_t["workspace"] / 1e12 / PEAK_F32_TFLOPS, 4),
                          "binding_roof_frac": round(few_roof / few_t["workspace"], 4)},
            "speedup": round(few_t["skinny"] / few_t["workspace"], 3),
        }
        del few_W, few_G, few_D, few_ws

    # Between the skinny step (T = 16) and the large-T step: the skinny
    # workload's W at T = 32 and 64 through retro_out_prod (the skinny kernel
    # with two and four blocks of 16 rows of G), back-to-back batches on the
    # rotated W copies.
    mid_t = []
    if not args.no_few_slab:
        g_mid = torch.randn((64, skinny["N"]), device=dev)
        for T_mid in (32, 64):
            G_mid = g_mid[:T_mid].contiguous()
            D_mid = torch.empty((T_mid, skinny["K"]), dtype=torch.float32, device=dev)
            call = lambda i, G_mid=G_mid, D_mid=D_mid: q.out_prod(q.Q4_K, Ws[i % n_rot], G_mid, skinny["K"], out=D_mid)  # noqa: E731
            for i in range(5):
                call(i)
            torch.cuda.synchronize()
            sec = back_to_back(call, batch_reps(back_to_back(call, 5)))
            fl = 2.0 * T_mid * skinny["N"] * skinny["K"]
            mid_t.append({"workload": f"q4_k_n{skinny['N']}_k{skinny['K']}_t{T_mid}",
                          "kernel": q.plan_names(q.Q4_K, skinny["K"], skinny["N"], T_mid),
                          "avg_launch_us": round(sec * 1e6, 3), "tflops": round(fl / sec / 1e12, 3),
                          "f32_mfma_frac": round(fl / sec / 1e12 / PEAK_F32_TFLOPS, 4)})
        del g_mid

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
    # F32 MFMA waves beside FMA waves on the same SIMDs: each alone, then
    # together. serial_frac = (both - larger) / smaller: 0 when the two run
    # side by side, 1 when they take turns.
    mix = {name: timed(lambda m=m, v=v: q.probe_mfma_valu(sink, m, v)) * 1e3
           for name, m, v in (("mfma_only_ms", 4096, 0), ("valu_only_ms", 0, 8192), ("both_ms", 4096, 8192))}
    lo, hi = sorted((mix["mfma_only_ms"], mix["valu_only_ms"]))
    mix = {k: round(x, 4) for k, x in mix.items()}
    mix["serial_frac"] = round((mix["both_ms"] - hi) / lo, 3)
    csrc = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    cdst = torch.empty_like(csrc)
    copy_gbs = 2.0 * csrc.numel() * 4 / timed(lambda: q.probe_copy(csrc, cdst)) / 1e9
    del csrc, cdst
    clock = clock_large = None
    if not args.no_cpu_baseline:
        # about 4 s each: the F32 matrix-core probe, then the large-T kernel
        clock = smi_under_load(lambda: [q.probe_mfma(q.PROBE_MFMA_F32, sink, 4096) for _ in range(1100)])
        n_large = max(1, int(4.0 / avg_large))
        clock_large = smi_under_load(
            lambda: [q.out_prod(q.Q4_K, Wl, Gl, large["K"], out=Dl) for _ in range(n_large)])
    ceilings = {"kind": "measured on this GPU: MFMA-only loops (no memory), 16-byte copy of 1 GiB",
                "mfma_f32_tflops": round(mfma_f32, 2), "mfma_bf16_tflops": round(mfma_bf16, 1),
                "copy_gbs": round(copy_gbs, 1),
                "mfma_f32_beside_valu": mix,
                "smi_clock_under_mfma_load": clock,
                "smi_under_large_kernel": clock_large,
                "mfma_f32_clock_ghz": round(mfma_f32 / PEAK_F32_TFLOPS * 2.4, 3)}
    if split is not None:
        split["bf16_mfma_frac_of_measured"] = round(split["bf16_flops_issued_per_launch"] / avg_split / 1e12 / mfma_bf16, 4)
    for entry in per_workload:
        entry["f32_mfma_frac_of_measured"] = round(entry["tflops"] / mfma_f32, 4)

    skinny_tflops = fl_skinny / avg_skinny / 1e12
    skinny_gbs = wbytes / avg_skinny / 1e9
    t_roof = max(wbytes / (PEAK_HBM_GBS * 1e9), fl_skinny / (PEAK_F32_TFLOPS * 1e12))

    out = {
        "metric": "OUT_PROD TFLOP/s and weight GB/s vs roofline, Q4_K 4096\u00d714336 T=4096 and T=16",
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
                     "traffic": read_traffic(large_tag),
                     "kernel": f"{kernel_family(q.VARIANT_NAMES[v_large])} ({q.VARIANT_NAMES[v_large]})",
                     "avg_launch_ms": round(avg_large * 1e3, 4), "min_launch_ms": round(float(t_large.min()) * 1e3, 4),
                     "flops_per_launch": fl_large},
        "skinny": {"kernel": f"{kernel_family(q.VARIANT_NAMES[v_skinny])} ({q.VARIANT_NAMES[v_skinny]})",
                   "traffic": read_traffic(skinny_tag),
                   "avg_launch_us": round(avg_skinny * 1e6, 3),
                   "avg_launch_us_event_pairs": round(float(t_skinny.mean()) * 1e6, 3),
                   "tflops": round(skinny_tflops, 3), "weight_gbs": round(skinny_gbs, 1),
                   "hbm_frac": round(skinny_gbs / PEAK_HBM_GBS, 4),
                   "f32_mfma_frac": round(skinny_tflops / PEAK_F32_TFLOPS, 4),
                   "f32_mfma_frac_of_measured": round(skinny_tflops / mfma_f32, 4),
                   "hbm_frac_of_measured_copy": round(skinny_gbs / copy_gbs, 4),
                   "binding_roof_frac": round(t_roof / avg_skinny, 4),
                   "weight_bytes": wbytes},
        "workloads": per_workload,
        "exact_split": split,
        "skinny_split": skinny_split,
        "mid_t": mid_t,
        "ceilings": ceilings,
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(large)
        out["cpu_baseline_skinny"] = cpu_baseline_skinny(skinny)
        for entry, c in oracle_cases:
            entry["oracle"] = oracle_timing(c)
        for entry in per_workload:
            if entry["workload"] == LARGE:
                entry["oracle"] = {k: out["cpu_baseline"][k] for k in ("value", "unit", "cores", "sample")}
            elif entry["workload"] == SKINNY:
                entry["oracle"] = {k: out["cpu_baseline_skinny"][k] for k in ("value", "unit", "cores", "sample")}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
