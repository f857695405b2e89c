#!/usr/bin/env python3
"""Benchmark of the fused HSTU attention forward on one MI355X.

One step = the whole hot path over one batch of synthetic input already
resident in HBM: the tile scheduler (hstu_*_plan) and the fused forward
kernel (hstu_*_run), both through the C ABI. Prints ONE JSON line:
effective TFLOP/s = 4 * head_dim * (visible query/key pairs summed over
query heads) / time per step, with the dominant kernel's roofline (achieved
vs MI355X's dense MFMA peak, or vs HBM bandwidth for the workloads that
stream rab, a user mask or a KV cache) and the float64 CPU oracle timed on
the host as a baseline.

Timing is cold by default: before every timed step a 1 GiB device buffer is
read (outside the timed events), which evicts the inputs from the L2 caches
and the 256 MB Infinity Cache, so every step reads them from HBM, and leaves
no dirty lines whose write-back would compete with the step.
Steps are timed with HIP events on the launch stream. Back-to-back (warm)
steps are reported as secondary keys.

Default workload: fp16 GQA jagged causal, batch 16, lengths lognormal
(median 1500, clipped to [128, 4096]), 8 query heads sharing 2 kv heads,
head_dim 128 -- the largest configuration that fits one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3, "fp8": 5000.0}  # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0
ELEM = {"bf16": 2, "f16": 2, "f32": 4, "fp8": 1}
OUT_ELEM = {"fp8": 2}  # the FP8 cast writes bf16
FLUSH_BYTES = 1 << 30  # read before each cold step: > 256 MB Infinity Cache + 8 x 4 MB L2

# The roof that binds each workload's forward kernel (algorithmic flops and
# bytes per launch at MI355X's dense MFMA and HBM peaks): MFMA for the
# causal and GQA workloads, HBM for the ones that stream rab, a user mask
# or a KV cache. The tiny fp32 workload is launch-bound; its line is
# priced against the fp32 MFMA peak.
BOUND = {"tiny_fp32_bidirectional": "mfma", "bf16_mha_causal": "mfma", "fp16_gqa_causal": "mfma",
         "bf16_rab_target": "hbm", "bf16_paged_target": "hbm", "bf16_custom_mask": "hbm", "bf16_delta_qk": "hbm",
         "fp8_gqa_causal": "mfma", "fp16_gqa_local": "mfma"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fp16_gqa_causal")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all", action="store_true", help="one JSON line per workload (extra lines for analysis)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only plain 1 GiB device copies (the reference point for the HBM byte counters)")
    ap.add_argument("--counter-summary", nargs="+", metavar=("WORKLOAD", "DIR"),
                    help="CPU only: turn rocprofv3 --pmc output folders (the passes of COUNTER_PASSES) into "
                         "profiles/counters_<WORKLOAD>.txt")
    ap.add_argument("--stats-summary", nargs=3, metavar=("WORKLOAD", "TRACE_DIR", "BENCH_OUT"),
                    help="CPU only: turn a rocprofv3 --kernel-trace --stats output folder of this script on "
                         "WORKLOAD (and the JSON line that run printed, saved in BENCH_OUT) into "
                         "profiles/kernels_<WORKLOAD>_stats.txt")
    ap.add_argument("--default-command", action="store_true",
                    help="with --stats-summary: the traced run was the default command (no flags); the summary "
                         "goes to profiles/fwd_kernel_<WORKLOAD>_stats.txt")
    ap.add_argument("--traffic-record", nargs=5, metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                          "COPY_WRITE_DIR"),
                    help="CPU only: turn the four rocprofv3 --pmc output folders (FETCH_SIZE / WRITE_SIZE of this "
                         "workload and of --copy-calibration) into profiles/fwd_kernel_<WORKLOAD>_traffic.{json,txt}")
    return ap.parse_args()


KERNEL_SOURCE = os.path.join(ROOT, "hstu_jagged_attention_amd", "csrc", "hstu_kernels.hip")
COPY_BYTES = 1 << 30


def kernel_source_sha256():
    """sha256 of the kernel source with // comments and blank lines removed
    (a comment edit does not change the kernel the counters describe)."""
    import hashlib
    import re
    with open(KERNEL_SOURCE) as f:
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in f]
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()


def measured_traffic(name):
    """HBM bytes per launch of the forward kernel on this workload, as read
    by the FETCH_SIZE and WRITE_SIZE counters and scaled by what the same
    counters read for a plain copy of known size. The record names the
    sha256 of the kernel source it was taken on; a record taken on other
    source gives None (the figure no longer describes the kernel)."""
    path = os.path.join(ROOT, "profiles", f"fwd_kernel_{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return rec.get("traffic_bytes_per_launch")


def is_fwd(kernel_name):
    """The forward kernel's dispatches (16-bit / fp32 fwd_kernel or the FP8 fwd_fp8_kernel)."""
    return "fwd_kernel" in kernel_name or "fwd_fp8_kernel" in kernel_name


def is_flush(kernel_name):
    """The cache flush's dispatch: torch's reduction over the 1 GiB buffer."""
    return "at::native" in kernel_name and "reduce_kernel" in kernel_name


def _counter_rows(folder, counter):
    """(kernel name, value) of every dispatch in the rocprofv3 counter CSVs under folder."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {folder}")
    return rows


def traffic_record(name, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Writes the HBM traffic record of the forward kernel on one workload:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch, from two separate
    rocprofv3 --pmc runs of this script on the workload), each scaled by
    what the same counter reads for the plain 1 GiB copies of
    --copy-calibration, against the algorithmic bytes of one launch."""
    import statistics
    copy_kib = COPY_BYTES / 1024.0
    cf = [v for k, v in _counter_rows(copy_fetch_dir, "FETCH_SIZE") if "copyBuffer" in k]
    cw = [v for k, v in _counter_rows(copy_write_dir, "WRITE_SIZE") if "copyBuffer" in k]
    fetch_factor = copy_kib / statistics.mean(cf)
    write_factor = copy_kib / statistics.mean(cw)
    fk = [v for k, v in _counter_rows(fetch_dir, "FETCH_SIZE") if is_fwd(k)]
    wk = [v for k, v in _counter_rows(write_dir, "WRITE_SIZE") if is_fwd(k)]
    fetch, write = statistics.mean(fk), statistics.mean(wk)
    traffic = (fetch * fetch_factor + write * write_factor) * 1024.0
    from hstu_jagged_attention_amd import workloads as wl
    _, alg_bytes, _ = workload_work(name, wl.WORKLOADS[name]())
    fwd_name = "fwd_fp8_kernel" if name.startswith("fp8") else "fwd_kernel"
    rec = {"workload": name, "kernel": fwd_name, "kernel_source_sha256": kernel_source_sha256(),
           "fetch_kib_per_dispatch": round(fetch, 3), "write_kib_per_dispatch": round(write, 3),
           "fetch_factor": round(fetch_factor, 5), "write_factor": round(write_factor, 5),
           "traffic_bytes_per_launch": int(round(traffic)), "algorithmic_bytes_per_launch": int(round(alg_bytes)),
           "dispatches": len(fk)}
    base = os.path.join(ROOT, "profiles", f"fwd_kernel_{name}_traffic")
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
    run = "python3 REPO/bench.py"
    lines = [
        f"fwd_kernel HBM traffic on workload {name} (rocprofv3 --pmc, one counter per run)", "",
        "Commands (each run from /tmp with TMPDIR=/tmp; REPO = repository root, OUT = any output folder):",
        f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/{name}_FETCH_SIZE -o p -- "
        f"{run} --workload {name} --steps 10 --warmup 2 --no-cpu-baseline",
        f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/{name}_WRITE_SIZE -o p -- "
        f"{run} --workload {name} --steps 10 --warmup 2 --no-cpu-baseline",
        f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/copy_FETCH_SIZE -o p -- "
        f"{run} --copy-calibration",
        f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/copy_WRITE_SIZE -o p -- "
        f"{run} --copy-calibration",
        f"  {run} --traffic-record {name} <the four -d folders above>   (this summary)", "",
        f"Copy calibration (__amd_rocclr_copyBuffer, 1 GiB read + 1 GiB written = {copy_kib:.0f} KiB each):",
        f"  FETCH_SIZE reads {statistics.mean(cf):.1f} KiB -> fetch factor {fetch_factor:.5f}",
        f"  WRITE_SIZE reads {statistics.mean(cw):.1f} KiB -> write factor {write_factor:.5f}", "",
        f"fwd_kernel, per dispatch ({len(fk)} dispatches):",
        f"  FETCH_SIZE mean {fetch:.1f} KiB (min {min(fk):.1f}, max {max(fk):.1f})",
        f"  WRITE_SIZE mean {write:.1f} KiB (min {min(wk):.1f}, max {max(wk):.1f})",
        f"  traffic = (FETCH*{fetch_factor:.4f} + WRITE*{write_factor:.4f}) KiB = {traffic / 1e6:.2f} MB per launch",
        f"  algorithmic bytes per launch = {alg_bytes / 1e6:.2f} MB; traffic / algorithmic = {traffic / alg_bytes:.2f}",
        f"kernel source sha256 {kernel_source_sha256()}", ""]
    with open(base + ".txt", "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


# Counter passes of --counter-summary, each within one run's hardware limits
# (at most 8 SQ, 4 TCC and 2 GRBM counters; derived counters count their
# inputs).
COUNTER_PASSES = {
    "util": "MfmaUtil VALUBusy SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_BF16",
    "insts": "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_SALU "
             "SQ_WAIT_INST_LDS SQ_WAVE_CYCLES",
    "l2": "TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
}


def counter_summary(name, folders):
    """Writes profiles/counters_<name>.txt from rocprofv3 --pmc CSV folders
    (one folder per pass of COUNTER_PASSES, each a run of this script on the
    workload): per-dispatch means of every counter over the forward kernel's
    dispatches, and the ratios read from them."""
    import csv
    import glob
    import statistics
    from hstu_jagged_attention_amd import workloads as wl
    vals, kernels = {}, set()
    for folder in folders:
        for f in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if not is_fwd(r["Kernel_Name"]):
                        continue
                    kernels.add(r["Kernel_Name"].split("(")[0][:120])
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no fwd_kernel counter rows under {folders}")
    m = {k: statistics.mean(v) for k, v in vals.items()}
    flops, alg_bytes, _ = workload_work(name, wl.WORKLOADS[name]())
    lines = [f"fwd_kernel hardware counters on workload {name} (rocprofv3 --pmc, per-dispatch means)", "",
             "Commands (each run from /tmp with TMPDIR=/tmp; REPO = repository root, OUT = any output folder):"]
    for pas, ctrs in COUNTER_PASSES.items():
        lines.append(f"  timeout -s KILL 120 rocprofv3 --pmc {ctrs} --output-format csv -d OUT/{name}_{pas} -o p -- "
                     f"python3 REPO/bench.py --workload {name} --steps 3 --warmup 1 --no-cpu-baseline")
    lines.append(f"  python3 REPO/bench.py --counter-summary {name} " +
                 " ".join(f"OUT/{name}_{p}" for p in COUNTER_PASSES) + "   (this summary)")
    lines += ["", "Kernel: " + ", ".join(sorted(kernels)), "", "Counters (mean per dispatch):"]
    for k in sorted(m):
        lines.append(f"  {k:32s} {m[k]:16.1f}   ({len(vals[k])} dispatches)")
    lines += ["", "Read from them:"]
    mops = m.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
    if "MfmaUtil" in m:
        lines.append(f"  MFMA busy (MfmaUtil)                      {m['MfmaUtil']:.1f} % of SIMD-cycles")
    if "VALUBusy" in m:
        lines.append(f"  VALU busy (VALUBusy)                      {m['VALUBusy']:.1f} %")
    if mops:
        lines.append(f"  MFMA flops executed / effective           {mops * 512 / flops:.3f}  "
                     f"(executed {mops * 512 / 1e9:.2f} GFLOP, effective {flops / 1e9:.2f} GFLOP)")
    if m.get("SQ_INSTS_MFMA"):
        mf = m["SQ_INSTS_MFMA"]
        lines.append(f"  VALU instructions per MFMA                {m.get('SQ_INSTS_VALU', 0.0) / mf:.2f}  "
                     "(SQ_INSTS_VALU counts the MFMAs too)")
        lines.append(f"  fp32 transcendentals per MFMA             {m.get('SQ_INSTS_VALU_TRANS_F32', 0.0) / mf:.2f}")
        lines.append(f"  LDS instructions per MFMA                 {m.get('SQ_INSTS_LDS', 0.0) / mf:.2f}")
        lines.append(f"  SALU instructions per MFMA                {m.get('SQ_INSTS_SALU', 0.0) / mf:.2f}")
    if m.get("SQ_INSTS_LDS"):
        lines.append(f"  LDS bank-conflict cycles per LDS instr.   {m.get('SQ_LDS_BANK_CONFLICT', 0.0) / m['SQ_INSTS_LDS']:.3f}")
    if m.get("SQ_WAVE_CYCLES"):
        lines.append(f"  LDS-issue wait / wave cycles              {m.get('SQ_WAIT_INST_LDS', 0.0) / m['SQ_WAVE_CYCLES']:.3f}")
    if "TCC_HIT_sum" in m:
        hm = m["TCC_HIT_sum"] + m.get("TCC_MISS_sum", 0.0)
        lines.append(f"  L2 (TCC) hit rate                         {m['TCC_HIT_sum'] / hm:.3f}  ({hm:.0f} requests)")
    lines.append("")
    out = os.path.join(ROOT, "profiles", f"counters_{name}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def stats_summary(name, trace_dir, bench_out, default_command=False):
    """Writes the kernel-trace summary of one bench run: rocprofv3's
    per-kernel statistics, and the forward kernel's mean duration over its
    cold dispatches (those that follow the cache flush, directly or after
    the plan kernel, as in the timed steps and the run-phase timing) and over
    the others (warm), to set beside the bench line's launch_ms_mean and
    launch_ms_mean_warm."""
    import csv
    import glob
    import statistics

    def one(pattern):
        files = sorted(glob.glob(os.path.join(trace_dir, "**", pattern), recursive=True))
        if not files:
            raise SystemExit(f"no {pattern} under {trace_dir}")
        return files[0]
    with open(one("*kernel_stats.csv")) as f:
        stats = list(csv.DictReader(f))
    with open(one("*kernel_trace.csv")) as f:
        trace = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    with open(bench_out) as f:
        line = next(json.loads(x) for x in f if x.startswith("{") and '"metric"' in x)
    cold, warm, prev = [], [], []
    for r in trace:
        kn = r["Kernel_Name"]
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if is_fwd(kn):
            after_flush = prev and (is_flush(prev[-1]) or ("plan_kernel" in prev[-1] and len(prev) > 1
                                                          and is_flush(prev[-2])))
            (cold if after_flush else warm).append(dur)
        prev.append(kn)
    total = sum(float(r["TotalDurationNs"]) for r in stats)

    def short(kn):
        kn = kn.replace("(anonymous namespace)::", "")
        return (kn[:84] + "...") if len(kn) > 87 else kn
    cmd = "python3 REPO/bench.py" + ("" if default_command else f" --workload {name} --steps 30 --warmup 5 "
                                                                "--no-cpu-baseline")
    r = line["roofline"]
    lines = [f"Kernels of workload {name}: rocprofv3 kernel-trace statistics of "
             + ("the default bench command" if default_command else "one bench run"), "",
             "Command (run from /tmp with TMPDIR=/tmp; REPO = repository root, OUT = any output folder):",
             f"  rocprofv3 --kernel-trace --stats --output-format csv -d OUT/stats_{name} -o run -- {cmd} "
             "> OUT/bench_{name}.out".replace("{name}", name),
             f"  python3 REPO/bench.py --stats-summary {name} OUT/stats_{name} OUT/bench_{name}.out"
             + (" --default-command" if default_command else "") + "   (this summary)",
             "(the run does warmup + steps cold plan/run pairs, each after a 1 GiB read that flushes the caches, "
             "then cold run-only launches, then warm back-to-back steps, runs and plans; durations in microseconds)",
             "",
             f"{'kernel':90s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for row in sorted(stats, key=lambda x: -float(x["TotalDurationNs"])):
        lines.append(f"{short(row['Name']):90s} {int(row['Calls']):6d} {float(row['AverageNs']) / 1e3:9.3f} "
                     f"{float(row['MinNs']) / 1e3:9.3f} {float(row['MaxNs']) / 1e3:9.3f} "
                     f"{100 * float(row['TotalDurationNs']) / total:6.2f}")
    lines += ["", "fwd_kernel dispatches by cache state (from the per-dispatch trace):",
              f"  cold (after the flush): {len(cold):4d} dispatches, mean {statistics.mean(cold):9.3f} us"
              if cold else "  cold: none",
              f"  warm:                   {len(warm):4d} dispatches, mean {statistics.mean(warm):9.3f} us"
              if warm else "  warm: none", "",
              "bench.py line printed by the same run:",
              f"  value {line['value']} {line['unit']}, ms_per_step {line['ms_per_step']} (cold), "
              f"warm_ms_per_step {line.get('warm_ms_per_step')}",
              f"  roofline: bound {r['bound']}, achieved {r['achieved']} {r['unit']}, frac {r['frac']}, "
              f"launch_ms_mean {r['launch_ms_mean']} (cold run phase: {r['kernel']}), "
              f"launch_ms_mean_warm {r.get('launch_ms_mean_warm')}, plan {r.get('plan_kernel_ms_mean_warm')} ms"]
    if "cpu_baseline" in line:
        cb = line["cpu_baseline"]
        lines.append(f"  cpu_baseline {cb['value']} {cb['unit']} ({cb['kind']}, {cb['cores']} threads; {cb['sample']})")
    lines.append("")
    fname = f"fwd_kernel_{name}_stats.txt" if default_command else f"kernels_{name}_stats.txt"
    with open(os.path.join(ROOT, "profiles", fname), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def copy_calibration(dev):
    """Plain device-to-device copies of COPY_BYTES each (read COPY_BYTES, write
    COPY_BYTES): the reference kernel for scaling the byte counters."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize(dev)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "copies": 5}), flush=True)


def workload_work(name, c):
    """Effective flops, algorithmic HBM bytes per launch and the config
    description of a workload (host-side accounting, no GPU)."""
    from hstu_jagged_attention_amd import metrics
    E = ELEM[c.dtype]
    if name == "bf16_paged_target":
        pairs = metrics.pairs_paged(c.history_lengths, c.new_lengths, c.num_context, c.num_targets,
                                    c.target_group_size, c.mask_type, c.local_window)
        Tq = int(c.seq_offsets_q[-1])
        alg_bytes = metrics.algorithmic_bytes_paged(Tq, int(c.history_lengths.sum()), c.num_heads_q, c.num_heads_kv,
                                                    c.head_dim, E)
        desc = dict(batch=c.batch, history="U{512..4096}", new_tokens="U{1..64}", page_size=c.page_size,
                    total_new_tokens=Tq, total_history_tokens=int(c.history_lengths.sum()))
    else:
        T, Tk = int(c.seq_offsets[-1]), int(c.key_lengths.sum())
        if c.mask is not None:
            m = c.mask.float().numpy()
            total, rab_entries = metrics.user_mask_counts(m, c.lengths, c.num_heads_q,
                                                          0 if c.rab is None else int(c.rab.shape[1]))
            pairs = total / c.num_heads_q
            in_seq = float(sum(int(L) ** 2 for L in c.lengths)) * m.shape[1]
            alg_bytes = metrics.algorithmic_bytes_jagged(T, c.num_heads_q, c.num_heads_kv, c.head_dim, E,
                                                         extra_bytes=(in_seq + rab_entries) * E)
        else:
            if c.seq_offsets_k is None:
                pairs = metrics.pairs_jagged(c.seq_offsets, c.num_context, c.num_targets, c.target_group_size,
                                             c.mask_type, c.local_window)
            else:
                pairs = metrics.pairs_delta(c.key_lengths, c.lengths, c.num_context, c.num_targets,
                                            c.target_group_size, c.mask_type, c.local_window)
            alg_bytes = metrics.algorithmic_bytes_jagged(T, c.num_heads_q, c.num_heads_kv, c.head_dim, E,
                                                         pairs if c.rab is not None else 0, Tk=Tk,
                                                         out_bytes=OUT_ELEM.get(c.dtype))
        desc = dict(batch=c.batch, total_tokens=T, max_seq_len=c.max_seq_len, lengths_min=int(c.lengths.min()),
                    lengths_max=int(c.lengths.max()))
        if c.seq_offsets_k is not None:
            desc.update(total_key_tokens=Tk, key_lengths_min=int(c.key_lengths.min()),
                        key_lengths_max=int(c.key_lengths.max()))
        if c.mask is not None:
            desc.update(user_mask_heads=int(c.mask.shape[1]), rab_heads=0 if c.rab is None else int(c.rab.shape[1]))
    flops = metrics.effective_flops(pairs, c.num_heads_q, c.head_dim)
    desc.update(num_heads_q=c.num_heads_q, num_heads_kv=c.num_heads_kv, head_dim=c.head_dim,
                mask={0: "causal", 2: "bidirectional", 3: "user mask"}[c.mask_type],
                rab=bool(getattr(c, "rab", None) is not None), visible_pairs_per_head=pairs)
    if c.local_window:
        desc.update(local_window=c.local_window)
    return flops, alg_bytes, desc


def build_step(name, dev):
    import torch
    import hstu_jagged_attention_amd as hj
    from hstu_jagged_attention_amd import workloads as wl
    c = wl.WORKLOADS[name]()
    if name == "bf16_paged_target":
        prep = hj.prepare_fwd_paged(c.q.to(dev), c.k_new.to(dev), c.v_new.to(dev), c.kv_cache.to(dev),
                                    torch.as_tensor(c.seq_offsets_q), torch.as_tensor(c.page_offsets),
                                    torch.as_tensor(c.page_ids), torch.as_tensor(c.last_page_len),
                                    num_context=c.num_context, num_targets=c.num_targets, max_seq_len=c.max_seq_len,
                                    mask_type=c.mask_type, target_group_size=c.target_group_size,
                                    local_window=c.local_window, alpha=c.alpha, out_scale=c.out_scale)
    else:
        prep = hj.prepare_fwd(c.q.to(dev), c.k.to(dev), c.v.to(dev), torch.as_tensor(c.seq_offsets),
                              rab=None if c.rab is None else c.rab.to(dev),
                              mask=None if c.mask is None else c.mask.to(dev),
                              seq_offsets_k=None if c.seq_offsets_k is None else torch.as_tensor(c.seq_offsets_k),
                              num_context=c.num_context, num_targets=c.num_targets, max_seq_len=c.max_seq_len,
                              mask_type=c.mask_type, target_group_size=c.target_group_size,
                              local_window=c.local_window, alpha=c.alpha, out_scale=c.out_scale)
    flops, alg_bytes, desc = workload_work(name, c)
    return c, prep, flops, alg_bytes, desc


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_sample(c, name, flops_full, stride):
    """(run, flops, description) of one oracle pass over the workload: the
    whole of it (stride 1) or every stride-th query row of every sequence,
    all heads."""
    import numpy as np
    import oracle
    from hstu_jagged_attention_amd import metrics

    def f64(t):
        return t.double().numpy()

    if name == "bf16_paged_target":
        q, kn, vn, kv = f64(c.q), f64(c.k_new), f64(c.v_new), f64(c.kv_cache)
        if stride == 1:
            rows, fl, desc = None, flops_full, "whole workload"
        else:
            rows, pairs = [], 0
            for b in range(c.batch):
                q0, q1 = int(c.seq_offsets_q[b]), int(c.seq_offsets_q[b + 1])
                Lh = int(c.history_lengths[b])
                nc = 0 if c.num_context is None else int(c.num_context[b])
                nt = 0 if c.num_targets is None else int(c.num_targets[b])
                per_row = metrics.visible_per_row(Lh + q1 - q0, nc, nt, c.target_group_size, c.mask_type,
                                                  c.local_window)
                for t in range(q0, q1, stride):
                    rows += [(t, h) for h in range(c.num_heads_q)]
                    pairs += int(per_row[Lh + t - q0]) * c.num_heads_q
            fl, desc = 4.0 * c.head_dim * pairs, f"every {stride}th new token of every request, all heads"
        run = lambda: oracle.hstu_fwd_paged(q, kn, vn, kv, c.seq_offsets_q, c.page_offsets, c.page_ids,
                                            c.last_page_len, num_context=c.num_context, num_targets=c.num_targets,
                                            mask_type=c.mask_type, target_group_size=c.target_group_size,
                                            alpha=c.alpha, out_scale=c.out_scale, rows=rows,
                                            local_window=c.local_window)
        return run, fl, desc
    q, k, v = f64(c.q), f64(c.k), f64(c.v)
    rab = None if c.rab is None else f64(c.rab)
    mask = None if c.mask is None else f64(c.mask)
    if stride == 1:
        rows, fl, desc = None, flops_full, "whole workload"
    else:
        rows, frac = [], 0.0
        for b in range(c.batch):
            s0, L = int(c.seq_offsets[b]), int(c.lengths[b])
            for i in range(0, L, stride):
                rows += [(s0 + i, h) for h in range(c.num_heads_q)]
        # Flops of the sample: the visible pairs of the sampled rows (query i
        # of a sequence sits at key position Lk - Lq + i).
        pairs = 0
        m = None if c.mask is None else c.mask.float().numpy()
        for b in range(c.batch):
            Lq, Lk = int(c.lengths[b]), int(c.key_lengths[b])
            pos = np.arange(0, Lq, stride) + (Lk - Lq)
            if m is not None:
                blk = np.nan_to_num(m[b, :, pos, :Lk], nan=0.0)
                pairs += int(np.count_nonzero(blk)) * (c.num_heads_q // m.shape[1])
            else:
                nc = 0 if c.num_context is None else int(c.num_context[b])
                nt = 0 if c.num_targets is None else int(c.num_targets[b])
                per_row = metrics.visible_per_row(Lk, nc, nt, c.target_group_size, c.mask_type, c.local_window)
                pairs += int(per_row[pos].sum()) * c.num_heads_q
        fl = 4.0 * c.head_dim * pairs
        desc = f"every {stride}th query row of every sequence, all heads"
    run = lambda: oracle.hstu_fwd(q, k, v, c.seq_offsets, rab=rab, mask=mask, seq_offsets_k=c.seq_offsets_k,
                                  num_context=c.num_context, num_targets=c.num_targets, max_seq_len=c.max_seq_len,
                                  mask_type=c.mask_type, target_group_size=c.target_group_size, alpha=c.alpha,
                                  out_scale=c.out_scale, rows=rows, p_fp8=c.dtype == "fp8",
                                  local_window=c.local_window)
    return run, fl, desc


def _time_for(run, seconds):
    runs, total = 0, 0.0
    while runs == 0 or total < seconds:
        t0 = time.perf_counter()
        run()
        total += time.perf_counter() - t0
        runs += 1
    return runs, total


# Row strides of the oracle samples: (all host threads, one thread). The
# whole small workloads take well under a second per pass; the large ones
# are sampled so that each figure takes about 10 s (all threads) and 5 s
# (one thread) of CPU time.
ORACLE_STRIDES = {"tiny_fp32_bidirectional": (1, 1), "bf16_mha_causal": (1, 8), "bf16_rab_target": (16, 128),
                  "fp16_gqa_causal": (16, 128), "bf16_paged_target": (1, 8), "bf16_custom_mask": (1, 8),
                  "bf16_delta_qk": (1, 8), "fp8_gqa_causal": (16, 128), "fp16_gqa_local": (4, 32)}


def cpu_baseline(c, name, flops_full):
    """The float64 oracle (as it stands) on the host's cores over the same
    inputs, then on one thread over a smaller sample."""
    import oracle
    s_all, s_one = ORACLE_STRIDES[name]
    threads = oracle.num_threads()
    run, fl, desc = oracle_sample(c, name, flops_full, s_all)
    runs, total = _time_for(run, 10.0)
    res = {"value": fl * runs / total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{desc}; {runs} runs in {total:.2f} s on {threads} threads", "cpu_model": cpu_model()}
    run1, fl1, desc1 = oracle_sample(c, name, flops_full, s_one)
    oracle.set_num_threads(1)
    try:
        runs1, total1 = _time_for(run1, 5.0)
    finally:
        oracle.set_num_threads(threads)
    res["single_thread"] = {"value": fl1 * runs1 / total1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                            "sample": f"{desc1}; {runs1} runs in {total1:.2f} s"}
    return res


def split_keys(c):
    """True when the library splits long items over the key range (paged
    calls and jagged calls with their own key offsets, 16-bit dtypes): the
    run phase then also launches the ordered reduction kernel."""
    return c.dtype != "f32" and (hasattr(c, "kv_cache") or getattr(c, "seq_offsets_k", None) is not None)


def measure(name, args, dev):
    import statistics
    import torch
    c, prep, flops, alg_bytes, desc = build_step(name, dev)
    stream = torch.cuda.current_stream(dev)
    flush_buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device=dev).view(4096, -1)

    def flush():
        # A read of the whole buffer (one row maximum per output, one
        # reduction kernel) evicts the inputs from every L2 and from the
        # Infinity Cache and leaves no dirty line behind. A write flush would
        # leave up to the caches' size of dirty lines whose write-back then
        # competes with the timed kernel's reads: a plain 302 MB read runs at
        # about 3.2 TB/s after a 1 GiB fill and 6.1 TB/s after a 1 GiB read.
        flush_buf.amax(dim=1)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    for _ in range(args.warmup):
        flush()
        prep.plan()
        prep.run()
    torch.cuda.synchronize(dev)

    # Timed region: exactly K cold steps. Each step is bracketed by HIP
    # events on the launch stream; the cache flush before it is not.
    marks = [(ev(), ev()) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in marks:
        flush()
        e0.record(stream)
        prep.plan()
        prep.run()
        e1.record(stream)
    torch.cuda.synchronize(dev)
    region_wall_ms = (time.perf_counter() - t0) * 1e3
    step_ms = [e0.elapsed_time(e1) for e0, e1 in marks]
    ms_per_step = statistics.mean(step_ms)

    # The run phase alone (the forward kernel, plus the ordered reduction of
    # split items), cold: plan, flush, then events around the run.
    rmarks = [(ev(), ev()) for _ in range(args.steps)]
    for e0, e1 in rmarks:
        prep.plan()
        flush()
        e0.record(stream)
        prep.run()
        e1.record(stream)
    torch.cuda.synchronize(dev)
    run_ms = statistics.mean(e0.elapsed_time(e1) for e0, e1 in rmarks)

    # Warm (secondary): K back-to-back steps, then K back-to-back runs and
    # plans, each group between two events (their latency amortised over K).
    def warm(fn):
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / args.steps

    warm_step_ms = warm(lambda: (prep.plan(), prep.run()))
    prep.plan()
    warm_run_ms = warm(prep.run)
    plan_ms = warm(prep.plan)

    dtype = c.dtype
    peak_f = PEAK_TFLOPS[dtype]
    mfma_tflops = flops / (run_ms * 1e-3) / 1e12
    hbm_gbs = alg_bytes / (run_ms * 1e-3) / 1e9
    bound = BOUND[name]
    if bound == "mfma":
        achieved, peak, unit = mfma_tflops, peak_f, "TFLOP/s"
    else:
        achieved, peak, unit = hbm_gbs, PEAK_HBM_GBS, "GB/s"
    roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(name),
                "kernel": ("fwd_fp8_kernel" if c.dtype == "fp8" else "fwd_kernel") +
                          ("+reduce_kernel" if split_keys(c) else ""),
                "launch_ms_mean": round(run_ms, 5), "launch_ms_mean_warm": round(warm_run_ms, 5),
                "plan_kernel_ms_mean_warm": round(plan_ms, 5), "algorithmic_flops": flops,
                "algorithmic_bytes": alg_bytes, "mfma_tflops": round(mfma_tflops, 3),
                "mfma_frac": round(mfma_tflops / peak_f, 4), "algorithmic_hbm_GBps": round(hbm_gbs, 1),
                "hbm_frac": round(hbm_gbs / PEAK_HBM_GBS, 4)}
    value = flops / (ms_per_step * 1e-3) / 1e12
    res = {"metric": "HSTU fwd effective TFLOP/s (unmasked pairs) + % of bf16 MFMA peak, 1 GPU",
           "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": dtype, "data": "synthetic (seeded numpy draws, rounded to dtype)",
           "config": dict(workload=name, **desc),
           # the metric's percentage: of the dense bf16 peak (of the fp32 peak for the fp32 workload)
           "pct_of_mfma_peak": round(100 * value / (peak_f if dtype == "f32" else PEAK_TFLOPS["bf16"]), 2),
           "timing": "cold: a 1 GiB device read before each step (outside the events) evicts L2 and Infinity "
                     "Cache; per-step HIP events on the launch stream",
           "ms_per_step_median": round(statistics.median(step_ms), 5),
           "timed_region_wall_ms": round(region_wall_ms, 3),
           "warm_ms_per_step": round(warm_step_ms, 5),
           "warm_value": round(flops / (warm_step_ms * 1e-3) / 1e12, 3),
           "roofline": roofline}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(c, name, flops)
    return res


def main():
    args = parse()
    if args.traffic_record:
        traffic_record(*args.traffic_record)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary[0], args.counter_summary[1:])
        return
    if args.stats_summary:
        stats_summary(*args.stats_summary, default_command=args.default_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the library has no multi-GPU "
              "path; see the sharding note in the design document)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import hstu_jagged_attention_amd as hj
    hj.load_library()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
        return
    names = ["tiny_fp32_bidirectional", "bf16_mha_causal", "bf16_rab_target", "fp16_gqa_causal",
             "bf16_paged_target", "bf16_custom_mask", "bf16_delta_qk", "fp8_gqa_causal", "fp16_gqa_local"] \
        if args.all \
        else [args.workload]
    for name in names:
        print(f"[bench] {name}: building inputs", file=sys.stderr, flush=True)
        res = measure(name, args, dev)
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
