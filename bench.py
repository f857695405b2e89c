#!/usr/bin/env python3
"""Benchmark of the fused HSTU attention forward on one MI355X.

One step = the whole hot path over one batch of synthetic input already
resident in HBM: the tile scheduler (hstu_*_plan) and the fused forward
kernel (hstu_*_run), both through the C ABI. Prints ONE JSON line:
effective TFLOP/s = 4 * head_dim * (visible query/key pairs summed over
query heads) / wall time per step, with the dominant kernel's roofline
(achieved vs MI355X's dense MFMA peak, per-launch time from HIP events on
the launch stream) and the float64 CPU oracle timed on the host as a
baseline.

Default workload: bf16 MHA jagged causal, batch 8, lengths ~ U{256..1024},
4 heads, head_dim 128.
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

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}  # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0
ELEM = {"bf16": 2, "f16": 2, "f32": 4}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bf16_mha_causal")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all", action="store_true", help="one JSON line per workload (extra lines for analysis)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only plain 1 GiB device copies (the reference point for the HBM byte counters)")
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
    fk = [v for k, v in _counter_rows(fetch_dir, "FETCH_SIZE") if "fwd_kernel" in k]
    wk = [v for k, v in _counter_rows(write_dir, "WRITE_SIZE") if "fwd_kernel" in k]
    fetch, write = statistics.mean(fk), statistics.mean(wk)
    traffic = (fetch * fetch_factor + write * write_factor) * 1024.0
    from hstu_jagged_attention_amd import workloads as wl
    _, alg_bytes, _ = workload_work(name, wl.WORKLOADS[name]())
    rec = {"workload": name, "kernel": "fwd_kernel", "kernel_source_sha256": kernel_source_sha256(),
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
                                    c.target_group_size, c.mask_type)
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
                                             c.mask_type)
            else:
                pairs = metrics.pairs_delta(c.key_lengths, c.lengths, c.num_context, c.num_targets,
                                            c.target_group_size, c.mask_type)
            alg_bytes = metrics.algorithmic_bytes_jagged(T, c.num_heads_q, c.num_heads_kv, c.head_dim, E,
                                                         pairs if c.rab is not None else 0, Tk=Tk)
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
                                    mask_type=c.mask_type, target_group_size=c.target_group_size, alpha=c.alpha,
                                    out_scale=c.out_scale)
    else:
        prep = hj.prepare_fwd(c.q.to(dev), c.k.to(dev), c.v.to(dev), torch.as_tensor(c.seq_offsets),
                              rab=None if c.rab is None else c.rab.to(dev),
                              mask=None if c.mask is None else c.mask.to(dev),
                              seq_offsets_k=None if c.seq_offsets_k is None else torch.as_tensor(c.seq_offsets_k),
                              num_context=c.num_context, num_targets=c.num_targets, max_seq_len=c.max_seq_len,
                              mask_type=c.mask_type, target_group_size=c.target_group_size, alpha=c.alpha,
                              out_scale=c.out_scale)
    flops, alg_bytes, desc = workload_work(name, c)
    return c, prep, flops, alg_bytes, desc


def cpu_baseline(c, name, flops_full):
    """The float64 oracle on the host cores over the same inputs (whole
    workload when that is a few seconds of CPU work, else a row sample)."""
    import numpy as np
    import oracle
    from hstu_jagged_attention_amd import metrics

    def f64(t):
        return t.double().numpy()

    if name == "bf16_paged_target":
        run = lambda: oracle.hstu_fwd_paged(f64(c.q), f64(c.k_new), f64(c.v_new), f64(c.kv_cache), c.seq_offsets_q,
                                            c.page_offsets, c.page_ids, c.last_page_len, num_context=c.num_context,
                                            num_targets=c.num_targets, mask_type=c.mask_type,
                                            target_group_size=c.target_group_size, alpha=c.alpha,
                                            out_scale=c.out_scale)
        sample, fl = "whole workload", flops_full
    elif name in ("bf16_mha_causal", "tiny_fp32_bidirectional", "bf16_custom_mask", "bf16_delta_qk"):
        q, k, v = f64(c.q), f64(c.k), f64(c.v)
        rab = None if c.rab is None else f64(c.rab)
        mask = None if c.mask is None else f64(c.mask)
        run = lambda: oracle.hstu_fwd(q, k, v, c.seq_offsets, rab=rab, mask=mask, seq_offsets_k=c.seq_offsets_k,
                                      num_context=c.num_context, num_targets=c.num_targets,
                                      max_seq_len=c.max_seq_len, mask_type=c.mask_type,
                                      target_group_size=c.target_group_size, alpha=c.alpha, out_scale=c.out_scale)
        sample, fl = "whole workload", flops_full
    else:
        # Row sample: every 16th token of every sequence, all heads.
        q, k, v = f64(c.q), f64(c.k), f64(c.v)
        rows, pairs = [], 0
        for b in range(c.batch):
            s0, L = int(c.seq_offsets[b]), int(c.lengths[b])
            nc = 0 if c.num_context is None else int(c.num_context[b])
            nt = 0 if c.num_targets is None else int(c.num_targets[b])
            per_row = metrics.visible_per_row(L, nc, nt, c.target_group_size, c.mask_type)
            for i in range(0, L, 16):
                rows += [(s0 + i, h) for h in range(c.num_heads_q)]
                pairs += int(per_row[i]) * c.num_heads_q
        rab = None if c.rab is None else f64(c.rab)
        run = lambda: oracle.hstu_fwd(q, k, v, c.seq_offsets, rab=rab, num_context=c.num_context,
                                      num_targets=c.num_targets, max_seq_len=c.max_seq_len, mask_type=c.mask_type,
                                      target_group_size=c.target_group_size, alpha=c.alpha, out_scale=c.out_scale,
                                      rows=rows)
        sample, fl = "every 16th query row of every sequence, all heads", 4.0 * c.head_dim * pairs
    # Repeat the sample until about 10 s of CPU work has been timed.
    runs, total = 0, 0.0
    while runs == 0 or total < 10.0:
        t0 = time.perf_counter()
        run()
        total += time.perf_counter() - t0
        runs += 1
    return {"value": fl * runs / total / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{sample}; {runs} runs in {total:.2f} s"}


def measure(name, args, dev):
    import torch
    c, prep, flops, alg_bytes, desc = build_step(name, dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        prep.plan()
        prep.run()
    torch.cuda.synchronize(dev)
    # Timed region: exactly K steps.
    t0 = time.perf_counter()
    for _ in range(args.steps):
        prep.plan()
        prep.run()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # Per-kernel launch durations with HIP events on the launch stream: K
    # back-to-back launches of one phase between two events, so the event
    # markers' own latency is amortised over K launches (a plan stays valid
    # for any number of runs: the run kernel rewinds its queue counters).
    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / n

    n_ev = max(args.steps, 10)
    plan_ms = timed(prep.plan, n_ev)
    prep.plan()
    run_ms = timed(prep.run, n_ev)
    achieved_tflops = flops / (run_ms * 1e-3) / 1e12
    dtype = c.dtype
    peak = PEAK_TFLOPS[dtype]
    hbm_gbs = alg_bytes / (run_ms * 1e-3) / 1e9
    roofline = {"bound": "mfma", "achieved": round(achieved_tflops, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved_tflops / peak, 4), "traffic": measured_traffic(name),
                "kernel": "fwd_kernel" + ("+reduce_kernel" if name == "bf16_paged_target" else ""),
                "launch_ms_mean": round(run_ms, 5),
                "plan_kernel_ms_mean": round(plan_ms, 5), "algorithmic_flops": flops, "algorithmic_bytes": alg_bytes,
                "algorithmic_hbm_GBps": round(hbm_gbs, 1), "hbm_frac": round(hbm_gbs / PEAK_HBM_GBS, 4)}
    value = flops / (ms_per_step * 1e-3) / 1e12
    res = {"metric": "HSTU fwd effective TFLOP/s (unmasked pairs) + % of bf16 MFMA peak, 1 GPU",
           "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": dtype, "data": "synthetic (seeded numpy draws, rounded to dtype)",
           "config": dict(workload=name, **desc), "pct_of_mfma_peak": round(100 * value / peak, 2),
           "roofline": roofline}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(c, name, flops)
    return res


def main():
    args = parse()
    if args.traffic_record:
        traffic_record(*args.traffic_record)
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
             "bf16_paged_target", "bf16_custom_mask", "bf16_delta_qk"] if args.all else [args.workload]
    for name in names:
        print(f"[bench] {name}: building inputs", file=sys.stderr, flush=True)
        res = measure(name, args, dev)
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
