#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X: attention forward + row online softmax.

One step = one attention forward over the batched causal workload (B=8, H=32,
N=8192, d=128, bf16, K rows scaled by U(0.5, 2)) followed by one row softmax
over the 4096 x 32768 fp32 workload, inputs already resident in device memory.

Prints ONE JSON line:
  value       attention TFLOP/s = 4*N^2*d*B*H/2 (causal) / mean attention
              kernel time, from HIP events on the stream the kernels run on;
  softmax     GB/s = 8 bytes per element (one read of X, one write of Y) /
              mean softmax kernel time;
  roofline    the attention kernel against the dense bf16 MFMA peak, with
              HBM traffic from the committed rocprofv3 counter summary when
              it was taken on the current kernel source;
  cpu_baseline  the fp64 oracle timed on this host's cores over a bounded
              sample of query rows of the same workload.
  After the timed steps, beside them: the backward (fa_bwd) on the same
  inputs, the forward with a sliding window over packed documents
  (fa_fwd_local, FLOP over visible pairs), the forward under a block-sparse
  pattern (fa_fwd_blocksparse, FLOP over visible pairs), one GPU's share of
  the causal workload split 8 ways by heads (B8 H4), the split-row softmax over
  4 rows of 2^24 columns (GB/s at 8 bytes per element; it moves 12), and the
  split-KV decode of one query per head against 32768 cached keys (GB/s of
  K, V, Q, O and LSE moved once), the fp8 forward on the B8 H32 N8192 d128
  causal shape (TFLOP/s against the dense fp8 peak), and the two head-dim-64
  workloads (one head of 4096 keys, one causal head of 131072).  Beside the
  softmax: a hand-written non-temporal 16-byte device copy of 512 MiB
  (fa_stream_copy), the practical HBM ceiling, timed in the same run.  Beside
  the attention: a stream of bf16 MFMAs on N(0,1) operands (fa_mfma_stream),
  the rate the matrix units hold on such data with nothing else running.

Other modes:
  --ingest-counters DIR_FETCH DIR_WRITE   turn two rocprofv3 --pmc runs
        (FETCH_SIZE, then WRITE_SIZE) of this script into the traffic
        summary under profiles/.
  --ingest-trace DIR   turn a rocprofv3 --kernel-trace --stats run of this
        script into the kernel-duration summary under profiles/.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s at B=8,H=32,N=8192,d=128 bf16 + % MFMA peak; softmax GB/s"
ATTN_WORKLOAD = "attn_bf16_b8h32n8192_causal"
SOFTMAX_WORKLOAD = "softmax_4096x32768"
SPLIT_WORKLOAD = "softmax_split_4x16777216"
DECODE_WORKLOAD = "decode_bf16_b8h32_q1_kv32768_d128"
FP8_WORKLOAD = "attn_fp8_b8h32n8192_causal"
D64_WORKLOADS = ["attn_bf16_n4096", "attn_bf16_n131072_causal"]
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published
COPY_BYTES = 512 << 20         # probe copy (fa_stream_copy): 512 MiB read + 512 MiB written
MFMA_STREAM_BLOCKS = 2048      # matrix-unit probe (fa_mfma_stream): 8 workgroups per CU,
MFMA_STREAM_ITERS = 512        # 4096 MFMAs per wave, ~1 ms per launch
MFMA_STREAM_SEED = 97100
TRAFFIC_FILE = os.path.join(ROOT, "profiles", f"traffic_{ATTN_WORKLOAD}+{SOFTMAX_WORKLOAD}.md")
_SHARED = ["online_softmax_04_amd/csrc/common.h", "online_softmax_04_amd/csrc/mfma_tile.h",
           "online_softmax_04_amd/csrc/kernels.h"]
KERNEL_SOURCES = {
    "attn": ["online_softmax_04_amd/csrc/attn_fwd.hip", *_SHARED],
    "softmax": ["online_softmax_04_amd/csrc/softmax.hip", *_SHARED],
    "fp8": ["online_softmax_04_amd/csrc/attn_fwd_fp8.hip", *_SHARED],
}
# name parts that pick each kernel out of a profile of this script (the attention entry is
# the mangled dense causal bf16 d=128 instance, not the sliding-window one); the probe
# copy is fa_stream_copy (reads and writes COPY_BYTES)
KERNEL_NAME_PART = {"attn": "attn_fwd_mfmaIDF16bLi128ELb1ELi0E", "softmax": "softmax_persist",
                    "copy": "stream_copy"}


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# traffic summary (rocprofv3 counters)
# ---------------------------------------------------------------------------
def _counter_rows(d):
    """Per-dispatch counter rows of a rocprofv3 --pmc run: its CSV output, or the
    counters_collection view of its rocpd database."""
    import csv
    import sqlite3
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        for f in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
            con = sqlite3.connect(f)
            for did, name, cname, val in con.execute(
                    "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
                rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": cname,
                             "Counter_Value": val})
    if not rows:
        raise SystemExit(f"no counter rows under {d}")
    return rows


def attn_workgroups(B: int, H: int, N: int, causal: bool) -> int:
    """Workgroups of a 16-bit or fp8 forward launch: one per 256-query block, or,
    causal, one per pair of blocks (mt, n - 1 - mt) of a head."""
    blocks = -(-N // 256)
    return B * H * (-(-blocks // 2) if causal else blocks)


def _attn_grid() -> int:
    """Threads of the headline attention launch (the benchmark also launches the same
    kernel at other shapes; its dispatches are told apart by grid size)."""
    import workloads
    w = workloads.ATTN[ATTN_WORKLOAD]
    return attn_workgroups(w.B, w.H, w.N, w.causal) * 512


def _is_attn_dispatch(r) -> bool:
    grid = r.get("Grid_Size") or r.get("Grid_Size_X")
    return KERNEL_NAME_PART["attn"] in r.get("Kernel_Name", "") and grid is not None and int(grid) == _attn_grid()


def _per_kernel(rows, counter):
    """Mean counter value per dispatch for each kernel family (attn, softmax, copy)."""
    per_dispatch = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        name = r.get("Kernel_Name", "")
        for kind, part in KERNEL_NAME_PART.items():
            if kind == "attn" and not _is_attn_dispatch(r):
                continue
            if part in name:
                key = (kind, r.get("Dispatch_Id"))
                per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (kind, _), val in per_dispatch.items():
        out.setdefault(kind, []).append(val)
    return {k: sum(v) / len(v) for k, v in out.items()}


def ingest_counters(dir_fetch: str, dir_write: str):
    fetch = _per_kernel(_counter_rows(dir_fetch), "FETCH_SIZE")
    write = _per_kernel(_counter_rows(dir_write), "WRITE_SIZE")
    for need in ("attn", "softmax", "copy"):
        if need not in fetch or need not in write:
            raise SystemExit(f"counters for {need} missing (fetch {sorted(fetch)}, write {sorted(write)})")
    # FETCH_SIZE / WRITE_SIZE are in KiB per dispatch; scale each by what it
    # reads for the probe copy of known size
    f_scale = COPY_BYTES / (fetch["copy"] * 1024.0)
    w_scale = COPY_BYTES / (write["copy"] * 1024.0)
    out = {"fetch_scale": f_scale, "write_scale": w_scale, "copy_bytes": COPY_BYTES, "kernels": {}}
    for kind in ("attn", "softmax"):
        out["kernels"][kind] = {
            "source_sha": source_hash(kind),
            "fetch_kib_raw": fetch[kind], "write_kib_raw": write[kind],
            "fetch_bytes": fetch[kind] * 1024.0 * f_scale,
            "write_bytes": write[kind] * 1024.0 * w_scale,
        }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("# HBM traffic per dispatch (rocprofv3 counters)\n\n")
        fh.write("Commands (run from the repository root on one MI355X):\n\n")
        fh.write("    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run -- "
                 "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline\n")
        fh.write("    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run -- "
                 "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline\n")
        fh.write("    python3 bench.py --ingest-counters gpurun_out/pmc_fetch gpurun_out/pmc_write\n\n")
        fh.write("FETCH_SIZE and WRITE_SIZE are KiB per dispatch summed over the TCC "
                 "channels; each is scaled by the ratio of known bytes to the counter's "
                 f"reading for a plain {COPY_BYTES >> 20} MiB device copy in the same run "
                 f"(fetch x{f_scale:.4f}, write x{w_scale:.4f}).\n\n")
        fh.write("| kernel | source sha | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | written bytes |\n")
        fh.write("|---|---|---|---|---|---|\n")
        for kind, k in out["kernels"].items():
            fh.write(f"| {kind} | {k['source_sha']} | {k['fetch_kib_raw']:.0f} | {k['write_kib_raw']:.0f} "
                     f"| {k['fetch_bytes']:.4g} | {k['write_bytes']:.4g} |\n")
        fh.write("\n```json\n" + json.dumps(out, indent=1) + "\n```\n")
    print(json.dumps(out))


MFMA_FILE = os.path.join(ROOT, "profiles", f"mfma_{ATTN_WORKLOAD}.md")
MFMA_PASS_A = "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE"
MFMA_PASS_B = ("SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
               "SQ_INSTS_VMEM SQ_INSTS_SALU SQ_INSTS_VALU_TRANS_F32")


def kernel_mfma_count(w) -> tuple[int, int]:
    """MFMAs one attn_fwd_mfma launch issues on workload w (d = 128), as (32x32x16 MFMAs,
    16x16x32 MFMAs): every wave runs QK and PV (D/16 + D/16 32x32x16 MFMAs per 32-key
    block, two blocks per 64-key tile) and the row sum (one 16x16x32 MFMA per 16 keys) on
    each key tile up to the last one holding a key visible to one of its 32 queries."""
    bm, bn = 256, 64
    n_mt = -(-w.N // bm)
    nk_all = -(-w.N // bn)
    tiles = 0
    for mt in range(n_mt):
        i0 = mt * bm
        n_kt = min(nk_all, (i0 + bm - 1) // bn + 1) if w.causal else nk_all
        for wave in range(8):
            qw0 = i0 + 32 * (2 * (wave & 3) + (wave >> 2))
            n_w = min(n_kt, (qw0 + 31) // bn + 1) if w.causal else n_kt
            tiles += n_w
    return tiles * 2 * (w.d // 16) * 2 * w.B * w.H, tiles * (bn // 16) * w.B * w.H


def ingest_mfma_fp8(dir_a: str, dir_b: str):
    """Matrix-pipe and instruction counters of the fp8 forward on its workload, from the
    same two --pmc passes (the fp8 MFMA op count is not among them; busy cycles are)."""
    import csv
    import workloads
    w = workloads.ATTN[FP8_WORKLOAD]
    vals = {}
    for d in (dir_a, dir_b):
        for r in _counter_rows(d):
            name = r.get("Kernel_Name", "")
            if "attn_fwd_fp8_d128" not in name or int(r.get("Grid_Size") or 0) != _attn_grid():
                continue
            key = (d, r["Dispatch_Id"])
            vals.setdefault(key, {})
            vals[key][r["Counter_Name"]] = vals[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not vals:
        print("no fp8 dispatches in the counter runs")
        return
    mean = {}
    for cs in vals.values():
        for name, v in cs.items():
            mean.setdefault(name, []).append(v)
    mean = {k: sum(v) / len(v) for k, v in mean.items()}
    cu, simd, xcc = 256, 4, 8
    for f in glob.glob(os.path.join(dir_a, "**", "*agent_info.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Agent_Type") == "GPU":
                cu, simd = int(r["Cu_Count"]), int(r["Simd_Per_Cu"])
                xcc = int(r.get("Num_Xcc") or xcc)
    busy = mean.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan"))
    active = mean.get("GRBM_GUI_ACTIVE", float("nan")) / xcc
    n_mfma = mean.get("SQ_INSTS_MFMA", float("nan"))
    lines = [
        f"# MFMA utilisation: attn_fwd_fp8_d128<causal> on {w.name}\n",
        "Commands (run from the repository root on one MI355X): the two --pmc passes of "
        f"`profiles/mfma_{ATTN_WORKLOAD}.md`, then\n",
        "    python3 bench.py --ingest-mfma gpurun_out/pmc_mfma_a gpurun_out/pmc_mfma_b\n",
        f"Kernel source sha {source_hash('fp8')}; means over {len(vals)} profiled dispatch records "
        f"of the {_attn_grid()}-thread launch.\n",
        "| quantity | value |", "|---|---|",
        f"| SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) | {busy:.4g} |",
        f"| fp8 MFMA instructions (SQ_INSTS_MFMA) | {n_mfma:.4g} |",
        f"| busy cycles per 32x32x64 fp8 MFMA | {busy / n_mfma:.2f} |",
        f"| GRBM_GUI_ACTIVE per XCD | {active:.4g} |",
        f"| **MFMA pipe utilisation = busy / (active x {cu} CUs x {simd} SIMDs)** | **{busy / (active * cu * simd):.1%}** |",
        "",
        "| counter | value | per MFMA |", "|---|---|---|",
    ]
    for name in MFMA_PASS_B.split():
        v = mean.get(name, float("nan"))
        lines.append(f"| {name} | {v:.4g} | {v / n_mfma:.3f} |")
    lines.append("")
    path = os.path.join(ROOT, "profiles", f"mfma_{FP8_WORKLOAD}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(open(path).read())


def ingest_mfma(dir_a: str, dir_b: str):
    """Write the MFMA-utilisation summary of the attention kernel from two rocprofv3 --pmc
    passes of the benchmark (MFMA_PASS_A, then MFMA_PASS_B)."""
    import csv
    import workloads
    w = workloads.ATTN[ATTN_WORKLOAD]
    vals, durs = {}, {}
    for d in (dir_a, dir_b):
        for r in _counter_rows(d):
            if not _is_attn_dispatch(r):
                continue
            key = (d, r["Dispatch_Id"])
            vals.setdefault(key, {})
            vals[key][r["Counter_Name"]] = vals[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if "Start_Timestamp" in r:
                durs[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    if not vals:
        raise SystemExit("no attention dispatches in the counter runs")
    mean = {}
    for key, cs in vals.items():
        for name, v in cs.items():
            mean.setdefault(name, []).append(v)
    mean = {k: sum(v) / len(v) for k, v in mean.items()}
    dur = sum(durs.values()) / len(durs) if durs else float("nan")
    cu, simd, xcc = 256, 4, 8
    for f in glob.glob(os.path.join(dir_a, "**", "*agent_info.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Agent_Type") == "GPU":
                cu, simd = int(r["Cu_Count"]), int(r["Simd_Per_Cu"])
                xcc = int(r.get("Num_Xcc") or xcc)
    n_big, n_small = kernel_mfma_count(w)
    mfma_flop = n_big * 32 * 32 * 16 * 2 + n_small * 16 * 16 * 32 * 2
    n_mfma = mfma_flop / (32 * 32 * 16 * 2)  # in 32x32x16 equivalents (32 busy cycles each)
    counted_flop = mean.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", float("nan")) * 512
    busy = mean.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan"))
    active = mean.get("GRBM_GUI_ACTIVE", float("nan")) / xcc  # the counter sums the XCDs
    util = busy / (active * cu * simd)
    clock = active / dur / 1e9
    lines = [
        f"# MFMA utilisation: attn_fwd_mfma<bf16,128,causal> on {ATTN_WORKLOAD}\n",
        "Commands (run from the repository root on one MI355X):\n",
        f"    rocprofv3 --pmc {MFMA_PASS_A} --output-format csv -d gpurun_out/pmc_mfma_a -o run -- "
        "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline",
        f"    rocprofv3 --pmc {MFMA_PASS_B} --output-format csv -d gpurun_out/pmc_mfma_b -o run -- "
        "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline",
        "    python3 bench.py --ingest-mfma gpurun_out/pmc_mfma_a gpurun_out/pmc_mfma_b\n",
        f"Kernel source sha {source_hash('attn')}; means over {len(vals)} profiled dispatches "
        f"(mean duration under the profiler {dur * 1e3:.3f} ms).\n",
        "| quantity | value |", "|---|---|",
        f"| algorithmic FLOP (4 N^2 d B H / 2) | {w.flops:.4g} |",
        f"| MFMA FLOP the tile schedule issues ({n_big} 32x32x16 MFMAs for QK and PV, {n_small} "
        f"16x16x32 MFMAs for the row sums) | {mfma_flop:.4g} |",
        f"| MFMA FLOP counted (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) | {counted_flop:.4g} |",
        f"| SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) | {busy:.4g} |",
        f"| busy cycles per 32x32x16-equivalent MFMA | {busy / n_mfma:.2f} |",
        f"| GRBM_GUI_ACTIVE per XCD (GPU cycles; the counter sums {xcc} XCDs) | {active:.4g} |",
        f"| mean shader clock = GRBM_GUI_ACTIVE / duration | {clock:.3f} GHz |",
        f"| **MFMA pipe utilisation = busy / (active x {cu} CUs x {simd} SIMDs)** | **{util:.1%}** |",
        f"| achieved algorithmic rate under the profiler | {w.flops / dur / 1e12:.1f} TFLOP/s |",
        f"| same, as a fraction of the clock-for-clock peak ({cu * simd} SIMDs x 1024 FLOP/clk at "
        f"{clock:.2f} GHz) | {w.flops / dur / (cu * simd * 1024 * clock * 1e9):.1%} |",
        f"| same, as a fraction of the published 2.5 PFLOP/s | {w.flops / dur / 2.5e15:.1%} |",
        "",
        "Instruction mix per dispatch (second pass):\n",
        "| counter | value | per 32x32x16-equivalent MFMA |", "|---|---|---|",
    ]
    for name in MFMA_PASS_B.split():
        v = mean.get(name, float("nan"))
        lines.append(f"| {name} | {v:.4g} | {v / n_mfma:.3f} |")
    lines.append("")
    os.makedirs(os.path.dirname(MFMA_FILE), exist_ok=True)
    with open(MFMA_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(open(MFMA_FILE).read())


def ingest_trace(d: str, warmup: int):
    """Write the per-kernel duration summary of a rocprofv3 --kernel-trace --stats run of the
    default benchmark.  Besides rocprofv3's own statistics over every call, the summary gives
    the mean over the timed calls only (each kernel's calls after the first `warmup`), which is
    what the benchmark's HIP events measure."""
    import csv
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    traces = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not stats or not traces:
        raise SystemExit(f"no kernel_stats.csv / kernel_trace.csv under {d}")
    share = {r["Name"]: float(r["Percentage"]) for r in csv.DictReader(open(stats[0]))}
    total_ns = sum(float(r["TotalDurationNs"]) for r in csv.DictReader(open(stats[0])))
    # calls grouped by kernel and grid size: the benchmark runs some kernels at two shapes
    per_call = {}
    for r in csv.DictReader(open(traces[0])):
        per_call.setdefault((r["Kernel_Name"], int(r["Grid_Size_X"])), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    grids = {}
    for name, grid in per_call:
        grids.setdefault(name, []).append(grid)
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{ATTN_WORKLOAD}+{SOFTMAX_WORKLOAD}.md")
    with open(path, "w") as fh:
        fh.write(f"# Kernel durations: {ATTN_WORKLOAD} + {SOFTMAX_WORKLOAD}\n\n")
        fh.write("Command (run from the repository root on one MI355X):\n\n")
        fh.write("    rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_trace "
                 "-o run -- python3 bench.py --no-cpu-baseline\n")
        fh.write(f"    python3 bench.py --ingest-trace gpurun_out/prof_trace --warmup {warmup}\n\n")
        fh.write(f"Kernel sources: attention sha {source_hash('attn')}, softmax sha "
                 f"{source_hash('softmax')}.\n\n")
        fh.write(f"\"timed mean\" skips each kernel's first {warmup} calls (the benchmark's untimed "
                 "warm-up steps, while the clock ramps up).\n\n")
        fh.write("Rows are per kernel and grid size (threads); the headline attention launch is "
                 f"the one with {_attn_grid()} threads.\n\n")
        fh.write("| kernel | grid | calls | timed mean (us) | mean of all calls (us) | min (us) | max (us) | share |\n"
                 "|---|---|---|---|---|---|---|---|\n")
        for (name, grid), calls in sorted(per_call.items(), key=lambda kv: -sum(kv[1])):
            short = name if len(name) < 90 else name[:87] + "..."
            timed = calls[warmup:] if len(calls) > warmup else []
            tm = f"{sum(timed) / len(timed):.2f}" if timed else "-"
            sh = (f"{share[name]:.2f}%" if len(grids[name]) == 1 and name in share
                  else f"{sum(calls) * 1e3 / total_ns * 100:.2f}%")
            fh.write(f"| `{short}` | {grid} | {len(calls)} | {tm} | {sum(calls) / len(calls):.2f} | "
                     f"{min(calls):.2f} | {max(calls):.2f} | {sh} |\n")
    print(open(path).read())


def load_traffic(kind: str):
    """Scaled HBM bytes per dispatch of `kind`, or None if absent or stale."""
    try:
        text = open(TRAFFIC_FILE).read()
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        k = blob["kernels"][kind]
    except (OSError, IndexError, KeyError, ValueError):
        return None
    if k.get("source_sha") != source_hash(kind):
        return None
    return k["fetch_bytes"] + k["write_bytes"]


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the attention workload
# ---------------------------------------------------------------------------
def cpu_baseline(w, q, k, v, target_s: float = 15.0):
    import numpy as np
    import oracle
    import workloads

    orc = oracle.load()
    threads = oracle.default_threads()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def run(rows_per_head):
        flops, t0 = 0.0, time.perf_counter()
        for b, h in heads:
            rows = workloads.attn_sample_rows(w, b, h, count=rows_per_head)
            orc.attention_head(q[b, h], k[b, h], v[b, h], w.sm_scale, w.causal, rows,
                               dtype=w.dtype, threads=threads)
            vis = (rows + 1) if w.causal else np.full(rows.shape, w.N)
            flops += float(np.sum(4.0 * vis * w.d))
        return flops, time.perf_counter() - t0

    # Grow the sample until one timing costs at least 2/3 of target_s.  Each step aims at
    # target_s by linear extrapolation; a per-head fixed cost makes small samples look slow,
    # so the extrapolation undershoots and the loop repeats.
    rows = 16
    flops, secs = run(rows)
    while secs < target_s * 2 / 3 and rows < 2048:
        rows = int(min(2048, rows * min(8.0, max(1.5, target_s / max(secs, 1e-3)))))
        flops, secs = run(rows)
    # the single-thread rate on a small sample of the same rows (a few seconds)
    t1_flops, t1 = 0.0, time.perf_counter()
    for b, h in heads[:: max(1, len(heads) // 16)]:
        r1 = workloads.attn_sample_rows(w, b, h, count=16)
        orc.attention_head(q[b, h], k[b, h], v[b, h], w.sm_scale, w.causal, r1, dtype=w.dtype,
                           threads=1)
        vis = (r1 + 1) if w.causal else np.full(r1.shape, w.N)
        t1_flops += float(np.sum(4.0 * vis * w.d))
    t1 = time.perf_counter() - t1
    return {
        "value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "one_thread_value": t1_flops / t1 / 1e12,
        "sample": f"{rows} seeded query rows in each of the {len(heads)} heads "
                  f"({flops:.3g} FLOP counted as 4*visible_keys*d per row) in {secs:.1f} s; "
                  "fp64 three-pass definition, one materialised score row at a time",
        "extrapolated_full_s": w.flops / (flops / secs),
    }


# ---------------------------------------------------------------------------
# main benchmark
# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--ingest-trace", metavar="TRACE_DIR")
    ap.add_argument("--ingest-mfma", nargs=2, metavar=("PASS_A_DIR", "PASS_B_DIR"))
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.ingest_trace:
        ingest_trace(args.ingest_trace, args.warmup)
        return
    if args.ingest_mfma:
        ingest_mfma(*args.ingest_mfma)
        ingest_mfma_fp8(*args.ingest_mfma)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is "
              "built and measured on a single MI355X", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import online_softmax_04_amd as fa
    import workloads

    dev = torch.device("cuda:0")
    w = workloads.ATTN[ATTN_WORKLOAD]
    sw = workloads.SOFTMAX[SOFTMAX_WORKLOAD]
    print(f"[bench] generating {w.name} and {sw.name}", file=sys.stderr, flush=True)
    q, k, v = workloads.attn_full(w, threads=16)
    x = workloads.softmax_input(sw, threads=16)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    qd, kd, vd = to(q), to(k), to(v)
    od = torch.empty_like(qd)
    lsed = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    xd = torch.from_numpy(x).to(dev)
    yd = torch.empty_like(xd)
    cs = torch.randn(COPY_BYTES // 4, device=dev)
    cd = torch.empty_like(cs)
    # the d = 64 workloads: one head of 4096 keys, and one causal head of 131072
    d64 = {}
    for name in D64_WORKLOADS:
        wd = workloads.ATTN[name]
        hq, hk, hv = workloads.attn_full(wd, threads=16)
        d64[name] = (wd, to(hq), to(hk), to(hv), torch.empty((wd.B, wd.H, wd.N, wd.d),
                     dtype=torch.bfloat16, device=dev),
                     torch.empty((wd.B, wd.H, wd.N), dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream()
    print("[bench] inputs resident; warming up", file=sys.stderr, flush=True)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fa_fwd(qd, kd, vd, od, lsed, w.B, w.H, w.N, w.d, w.sm_scale, 1, stream)
        if ev is not None:
            ev[1].record(stream)
        fa.online_softmax_rows(xd, yd, sw.rows, sw.cols, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    # probe copy (non-temporal 16-byte loads and stores): the practical HBM ceiling
    # beside the softmax, and the known-size kernel that scales the byte counters
    for _ in range(3):
        fa.fa_stream_copy(cs, cd, COPY_BYTES, stream)
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(10)]
    for e in cev:
        e[0].record(stream)
        fa.fa_stream_copy(cs, cd, COPY_BYTES, stream)
        e[1].record(stream)
    torch.cuda.synchronize()
    copy_each = sorted(e[0].elapsed_time(e[1]) for e in cev)
    copy_ms = sum(copy_each) / len(copy_each)
    # matrix-unit probe: bf16 MFMAs on N(0,1) operands (drawn like the attention inputs),
    # the rate a dense contraction can hold on this data when nothing else runs
    g = torch.Generator(device=dev).manual_seed(MFMA_STREAM_SEED)
    mops = torch.randn(fa.MFMA_STREAM_OPERAND_BYTES // 2, device=dev, generator=g).to(torch.bfloat16)
    mout = torch.empty(MFMA_STREAM_BLOCKS * 512, dtype=torch.float32, device=dev)
    for _ in range(2):
        fa.fa_mfma_stream(mops, mout, MFMA_STREAM_BLOCKS, MFMA_STREAM_ITERS, stream)
    mev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
    for e in mev:
        e[0].record(stream)
        fa.fa_mfma_stream(mops, mout, MFMA_STREAM_BLOCKS, MFMA_STREAM_ITERS, stream)
        e[1].record(stream)
    torch.cuda.synchronize()
    mfma_ms = sum(e[0].elapsed_time(e[1]) for e in mev) / len(mev)
    mfma_ceiling = MFMA_STREAM_BLOCKS * 8 * MFMA_STREAM_ITERS * 8 * 32768 / (mfma_ms * 1e-3) / 1e12
    print(f"[bench] matrix-unit probe {mfma_ceiling:.1f} TFLOP/s on N(0,1) bf16 operands", file=sys.stderr,
          flush=True)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_each = sorted(e[0].elapsed_time(e[1]) for e in events)
    sm_each = sorted(e[1].elapsed_time(e[2]) for e in events)
    attn_ms = sum(attn_each) / args.steps
    sm_ms = sum(sm_each) / args.steps
    print(f"[bench] timed {args.steps} steps: attention {attn_ms:.3f} ms, softmax {sm_ms * 1e3:.1f} us",
          file=sys.stderr, flush=True)

    def timed(fn, steps):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return sorted(e[0].elapsed_time(e[1]) for e in ev)

    # The backward pass (fa_bwd) on the same inputs, after the timed steps: the
    # forward's O and logsumexp, a synthetic upstream gradient.  Reported beside
    # the step, not inside it.
    gen = torch.Generator(device=dev).manual_seed(97700)
    dod = torch.randn(qd.shape, device=dev, generator=gen).to(torch.bfloat16)
    dqd, dkd, dvd = (torch.empty_like(qd) for _ in range(3))
    wsd = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N) // 4, dtype=torch.float32, device=dev)

    def bwd():
        fa.fa_bwd(qd, kd, vd, od, dod, lsed, dqd, dkd, dvd, wsd, w.B, w.H, w.N, w.d, w.sm_scale, 1,
                  stream)

    for _ in range(args.warmup):
        bwd()
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        bev[i][0].record(stream)
        bwd()
        bev[i][1].record(stream)
    torch.cuda.synchronize()
    bwd_each = sorted(e[0].elapsed_time(e[1]) for e in bev)
    bwd_ms = sum(bwd_each) / args.steps
    bwd_flop = 2.5 * w.flops  # dV, dP, dQ, dK and the recomputed S: 5 products vs 2
    bwd_tflops = bwd_flop / (bwd_ms * 1e-3) / 1e12
    print(f"[bench] backward {bwd_ms:.3f} ms", file=sys.stderr, flush=True)

    # Structured masks (sliding window over packed documents) on the same inputs;
    # FLOP counted over the visible query-key pairs only.
    lw = workloads.LOCAL_WORKLOAD
    doc = workloads.packed_doc_starts(w.B, w.N, lw["doc_seed"], lw["doc_min"], lw["doc_max"])
    pairs = 0
    for b in range(w.B):
        lo, hi = workloads.local_ranges(doc[b], lw["window"])
        pairs += int(np.sum(hi - lo + 1))
    loc_flop = 4.0 * w.d * w.H * pairs
    docd = torch.from_numpy(doc).to(dev)
    lod = torch.empty_like(qd)

    def local():
        fa.fa_fwd_local(qd, kd, vd, lod, lsed, docd, lw["window"], w.B, w.H, w.N, w.d, w.sm_scale,
                        stream)

    for _ in range(args.warmup):
        local()
    lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        lev[i][0].record(stream)
        local()
        lev[i][1].record(stream)
    torch.cuda.synchronize()
    loc_each = sorted(e[0].elapsed_time(e[1]) for e in lev)
    loc_ms = sum(loc_each) / args.steps
    loc_tflops = loc_flop / (loc_ms * 1e-3) / 1e12
    print(f"[bench] local {loc_ms:.3f} ms", file=sys.stderr, flush=True)

    # Block-sparse pattern (sink block, diagonal band, 10 % random blocks) on the
    # same inputs; FLOP counted over the visible query-key pairs only.
    bw = workloads.BLOCKSPARSE_WORKLOAD
    bs_ptr, bs_idx = workloads.block_sparse_pattern(w.N, bw["pattern_seed"], band=bw["band"],
                                                    sinks=bw["sinks"], p_random=bw["p_random"],
                                                    causal=w.causal)
    bs_pairs = workloads.block_sparse_pairs(w.N, bs_ptr, bs_idx, w.causal)
    bs_flop = 4.0 * w.d * w.B * w.H * bs_pairs
    bs_ptr_d = torch.from_numpy(bs_ptr).to(dev)
    bs_idx_d = torch.from_numpy(bs_idx).to(dev)

    def blocksparse():
        fa.fa_fwd_blocksparse(qd, kd, vd, lod, lsed, bs_ptr_d, bs_idx_d, bs_idx.size, w.B, w.H,
                              w.N, w.d, w.sm_scale, int(w.causal), stream)

    for _ in range(args.warmup):
        blocksparse()
    bs_each = timed(blocksparse, args.steps)
    bs_ms = sum(bs_each) / args.steps
    bs_tflops = bs_flop / (bs_ms * 1e-3) / 1e12
    print(f"[bench] blocksparse {bs_ms:.3f} ms", file=sys.stderr, flush=True)

    # One GPU's share of the same workload split over 8 GPUs by heads (4 of the 32
    # heads of every batch row): the kernel at the shape it would run at there.
    sh_h = w.H // 8
    sq, sk, sv = (t[:, :sh_h].contiguous() for t in (qd, kd, vd))
    so = torch.empty_like(sq)
    sl = torch.empty((w.B, sh_h, w.N), dtype=torch.float32, device=dev)

    def shard():
        fa.fa_fwd(sq, sk, sv, so, sl, w.B, sh_h, w.N, w.d, w.sm_scale, int(w.causal), stream)

    for _ in range(args.warmup):
        shard()
    sh_each = timed(shard, args.steps)
    sh_ms = sum(sh_each) / args.steps
    sh_flop = w.flops / 8
    sh_tflops = sh_flop / (sh_ms * 1e-3) / 1e12
    del sq, sk, sv, so, sl
    print(f"[bench] 8-way head shard {sh_ms:.3f} ms", file=sys.stderr, flush=True)

    # Split-row softmax on few very long rows (several workgroups per row), and
    # the one-workgroup-per-row path on the same input for comparison.
    spw = workloads.SOFTMAX[SPLIT_WORKLOAD]
    spx = torch.from_numpy(workloads.softmax_input(spw, threads=4)).to(dev)
    spy = torch.empty_like(spx)
    sp_wsb = fa.online_softmax_split_workspace_bytes(spw.rows, spw.cols)
    sp_ws = torch.empty(sp_wsb // 4, dtype=torch.float32, device=dev)

    def split():
        fa.online_softmax_rows_split(spx, spy, spw.rows, spw.cols, sp_ws, sp_wsb, stream)

    for _ in range(args.warmup):
        split()
    sp_each = timed(split, args.steps)
    sp_ms = sum(sp_each) / args.steps
    sp_gbps = spw.algorithmic_bytes / (sp_ms * 1e-3) / 1e9
    unsplit_each = timed(lambda: fa.online_softmax_rows(spx, spy, spw.rows, spw.cols, stream), 2)
    unsplit_gbps = spw.algorithmic_bytes / (unsplit_each[0] * 1e-3) / 1e9
    del spx, spy
    print(f"[bench] split softmax {sp_ms * 1e3:.1f} us", file=sys.stderr, flush=True)

    # fp8 forward on the same shape (E4M3 Q/K/V with per-tensor descales, bf16 O)
    fw = workloads.ATTN[FP8_WORKLOAD]
    f8 = workloads.attn_full(fw, threads=16)
    f8q, f8k, f8v = (torch.from_numpy(t).to(dev) for t in f8)
    del f8
    f8o = torch.empty(f8q.shape, dtype=torch.bfloat16, device=dev)
    f8l = torch.empty((fw.B, fw.H, fw.N), dtype=torch.float32, device=dev)

    def fp8():
        fa.fa_fwd_fp8(f8q, f8k, f8v, f8o, f8l, fw.B, fw.H, fw.N, fw.d, fw.sm_scale, *fw.descales,
                      int(fw.causal), stream)

    for _ in range(args.warmup):
        fp8()
    f8_each = timed(fp8, args.steps)
    f8_ms = sum(f8_each) / args.steps
    f8_tflops = fw.flops / (f8_ms * 1e-3) / 1e12
    del f8q, f8k, f8v, f8o
    print(f"[bench] fp8 forward {f8_ms:.3f} ms", file=sys.stderr, flush=True)

    # Split-KV decode: one query per head against a 32768-key cache (HBM-bound: K and
    # V are read once).
    dw = workloads.DECODE[DECODE_WORKLOAD]
    dq_h, dk_h, dv_h = workloads.decode_full(dw, threads=16)
    dqd, dkd, dvd = (torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).to(dev)
                     for t in (dq_h, dk_h, dv_h))
    del dq_h, dk_h, dv_h
    dod = torch.empty_like(dqd)
    dlse = torch.empty((dw.B, dw.H, dw.Nq), dtype=torch.float32, device=dev)
    dec_wsb = fa.fa_decode_workspace_bytes(dw.B, dw.H, dw.Nq, dw.Nk, dw.d)
    dec_ws = torch.empty(dec_wsb // 4, dtype=torch.float32, device=dev)

    def decode():
        fa.fa_decode(dqd, dkd, dvd, dod, dlse, dec_ws, dec_wsb, dw.B, dw.H, dw.Nq, dw.Nk, dw.d,
                     dw.sm_scale, int(dw.causal), stream)

    for _ in range(args.warmup):
        decode()
    dec_each = timed(decode, args.steps)
    dec_ms = sum(dec_each) / args.steps
    dec_gbps = dw.algorithmic_bytes / (dec_ms * 1e-3) / 1e9
    del dqd, dkd, dvd
    print(f"[bench] decode {dec_ms * 1e3:.1f} us", file=sys.stderr, flush=True)

    # the d = 64 workloads (one head each): TFLOP/s against the same bf16 peak
    d64_out = {}
    for name, (wd, hq, hk, hv, ho, hl) in d64.items():
        def fwd64(wd=wd, hq=hq, hk=hk, hv=hv, ho=ho, hl=hl):
            fa.fa_fwd(hq, hk, hv, ho, hl, wd.B, wd.H, wd.N, wd.d, wd.sm_scale, int(wd.causal), stream)

        for _ in range(args.warmup):
            fwd64()
        each = timed(fwd64, args.steps)
        ms = sum(each) / args.steps
        tf = wd.flops / (ms * 1e-3) / 1e12
        d64_out[name] = {
            "value": round(tf, 2), "unit": "TFLOP/s", "flop_per_launch": wd.flops,
            "B": wd.B, "H": wd.H, "N": wd.N, "d": wd.d, "causal": wd.causal,
            "avg_launch_ms": round(ms, 5), "median_launch_ms": round(each[len(each) // 2], 5),
            "min_launch_ms": round(each[0], 5),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "kernel": f"attn_fwd_mfma<bf16,64,{'causal' if wd.causal else 'dense'}>",
                         "workgroups": attn_workgroups(wd.B, wd.H, wd.N, wd.causal)}}
        print(f"[bench] {name} {ms:.3f} ms", file=sys.stderr, flush=True)
    del d64

    tflops = w.flops / (attn_ms * 1e-3) / 1e12
    sm_bytes = sw.algorithmic_bytes
    sm_gbps = sm_bytes / (sm_ms * 1e-3) / 1e9
    attrs = fa.kernel_attributes(fa.OP_FA_FWD, w.d, True)
    sm_attrs = fa.kernel_attributes(fa.OP_SOFTMAX, sw.cols)
    attn_traffic = load_traffic("attn")
    sm_traffic = load_traffic("softmax")
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} + {sw.name}", "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": True, "softmax_rows": sw.rows, "softmax_cols": sw.cols},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": attn_traffic, "kernel": "attn_fwd_mfma<bf16,128,causal>",
                     "flop_per_launch": w.flops, "avg_launch_ms": round(attn_ms, 5),
                     "median_launch_ms": round(attn_each[len(attn_each) // 2], 5),
                     "min_launch_ms": round(attn_each[0], 5),
                     "mfma_ceiling_tflops": round(mfma_ceiling, 1),
                     "mfma_ceiling_kernel": "mfma_stream (fa_mfma_stream: 32x32x16 bf16 MFMAs from "
                                            "registers, N(0,1) operands, 2 waves per SIMD, "
                                            f"{MFMA_STREAM_BLOCKS} workgroups)",
                     "frac_of_mfma_ceiling": round(tflops / mfma_ceiling, 4)},
        "softmax": {"value": round(sm_gbps, 1), "unit": "GB/s",
                    "roofline": {"bound": "hbm", "achieved": round(sm_gbps, 1),
                                 "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                 "frac": round(sm_gbps / PEAK_HBM_GBPS, 4), "traffic": sm_traffic,
                                 "kernel": "softmax_persist<1024,8>",
                                 "bytes_per_launch": sm_bytes, "avg_launch_us": round(sm_ms * 1e3, 2),
                                 "median_launch_us": round(sm_each[len(sm_each) // 2] * 1e3, 2),
                                 "min_launch_us": round(sm_each[0] * 1e3, 2)},
                    "copy_gbps": round(2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9, 1),
                    "copy_kernel": "stream_copy (fa_stream_copy, 16-byte non-temporal, "
                                   f"{COPY_BYTES >> 20} MiB read + {COPY_BYTES >> 20} MiB written)",
                    "frac_of_copy": round(sm_gbps / (2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9), 4)},
        "backward": {"value": round(bwd_tflops, 2), "unit": "TFLOP/s",
                     "flop_per_launch": bwd_flop,
                     "mfma_flop_issued_per_launch": 3.5 * w.flops,
                     "avg_launch_ms": round(bwd_ms, 5),
                     "median_launch_ms": round(bwd_each[len(bwd_each) // 2], 5),
                     "roofline": {"bound": "mfma", "achieved": round(bwd_tflops, 2),
                                  "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
                                  "kernels": ["attn_bwd_dq<bf16,128,causal>",
                                              "attn_bwd_dkdv<bf16,128,causal>"]}},
        "local": {"workload": lw["name"], "value": round(loc_tflops, 2), "unit": "TFLOP/s",
                  "visible_pairs": pairs, "flop_per_launch": loc_flop,
                  "avg_launch_ms": round(loc_ms, 5),
                  "median_launch_ms": round(loc_each[len(loc_each) // 2], 5),
                  "roofline": {"bound": "mfma", "achieved": round(loc_tflops, 2),
                               "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(loc_tflops / PEAK_BF16_TFLOPS, 4),
                               "kernel": "attn_fwd_mfma<bf16,128,causal,local>"}},
        "blocksparse": {"workload": bw["name"], "value": round(bs_tflops, 2), "unit": "TFLOP/s",
                        "visible_pairs_per_head": bs_pairs, "listed_blocks": int(bs_idx.size),
                        "flop_per_launch": bs_flop, "avg_launch_ms": round(bs_ms, 5),
                        "median_launch_ms": round(bs_each[len(bs_each) // 2], 5),
                        "roofline": {"bound": "mfma", "achieved": round(bs_tflops, 2),
                                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                     "frac": round(bs_tflops / PEAK_BF16_TFLOPS, 4),
                                     "kernel": "attn_fwd_mfma<bf16,128,causal,blocksparse>"}},
        "shard_8way_heads": {"workload": f"attn_bf16_b{w.B}h{sh_h}n{w.N}_causal (heads 0-{sh_h - 1} of each batch row)",
                             "value": round(sh_tflops, 2), "unit": "TFLOP/s",
                             "flop_per_launch": sh_flop, "avg_launch_ms": round(sh_ms, 5),
                             "median_launch_ms": round(sh_each[len(sh_each) // 2], 5),
                             "roofline": {"bound": "mfma", "achieved": round(sh_tflops, 2),
                                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                          "frac": round(sh_tflops / PEAK_BF16_TFLOPS, 4),
                                          "kernel": "attn_fwd_mfma<bf16,128,causal>"}},
        "softmax_split": {"workload": spw.name, "value": round(sp_gbps, 1), "unit": "GB/s",
                          "bytes_per_launch": spw.algorithmic_bytes,
                          "bytes_moved_per_launch": 12 * spw.rows * spw.cols,
                          "avg_launch_us": round(sp_ms * 1e3, 2),
                          "median_launch_us": round(sp_each[len(sp_each) // 2] * 1e3, 2),
                          "one_workgroup_per_row_gbps": round(unsplit_gbps, 1),
                          "roofline": {"bound": "hbm", "achieved": round(sp_gbps, 1),
                                       "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                       "frac": round(sp_gbps / PEAK_HBM_GBPS, 4),
                                       "kernels": ["softmax_split_partials<512,true>",
                                                   "softmax_split_normalise<512,true>"]}},
        "fp8": {"workload": fw.name, "value": round(f8_tflops, 2), "unit": "TFLOP/s",
                "flop_per_launch": fw.flops, "avg_launch_ms": round(f8_ms, 5),
                "median_launch_ms": round(f8_each[len(f8_each) // 2], 5),
                "roofline": {"bound": "mfma", "achieved": round(f8_tflops, 2),
                             "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(f8_tflops / PEAK_FP8_TFLOPS, 4),
                             "kernel": "attn_fwd_fp8_d128<causal>"}},
        "decode": {"workload": dw.name, "value": round(dec_gbps, 1), "unit": "GB/s",
                   "bytes_per_launch": dw.algorithmic_bytes, "workspace_bytes": dec_wsb,
                   "avg_launch_us": round(dec_ms * 1e3, 2),
                   "median_launch_us": round(dec_each[len(dec_each) // 2] * 1e3, 2),
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1),
                                "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                                "kernels": ["attn_decode_partial<bf16,128,causal>",
                                            "attn_decode_merge<bf16,128>"]}},
        "d64": d64_out,
        "kernel_resources": {"attention": attrs, "softmax": sm_attrs,
                             "decode": fa.kernel_attributes(fa.OP_FA_DECODE, dw.d, dw.causal),
                             "backward_dq": fa.kernel_attributes(fa.OP_FA_BWD_DQ, w.d, True),
                             "backward_dkdv": fa.kernel_attributes(fa.OP_FA_BWD_DKDV, w.d, True)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, q, k, v)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
