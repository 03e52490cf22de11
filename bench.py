#!/usr/bin/env python3
"""Benchmark of absorbed-path MLA decode on one MI355X.

One step = one ``mla_decode_run`` call (Q quantisation, split-KV attention,
LSE merge when the plan splits) over the workload's synthetic inputs, which
are resident in HBM before the timed region starts. Prints ONE JSON line.

Default workload: bs=256, kv_len=8192 per sequence, FP8 E4M3FN latent cache
(2,097,152 cache rows, 1.21 GB), absmax Q scale. The cache is 4.7x the
MI355X's 256 MB last-level cache, so back-to-back steps read it from HBM.

Roofline: the dominant kernel is the stage-1 attention; its algorithmic bytes
per launch (576 B per cache row, 9,216 B of Q codes per work item, and the
output or partial written per item) over its average duration, timed with
HIP events on the stream the library launches on, against the 8 TB/s HBM
peak. ``traffic`` is the measured HBM bytes of that kernel from the committed
rocprofv3 counter summary, scaled by the counters of a plain copy of known
size, or null when the kernel source has changed since it was taken.

cpu_baseline: the CPU oracle (fp64) timed on a bounded sample of the same
workload on this host's cores, scaled to one call.
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

HBM_PEAK_GBPS = 8000.0
METRIC = "MLA decode µs/call + achieved HBM GB/s (% peak), bs=256 kv=8192 fp8"
STAGE1_SOURCES = ["mla_latent_kv_bf16_amd/csrc/stage1_fp8.hip",
                  "mla_latent_kv_bf16_amd/csrc/device_common.h"]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "stage1_fp8_bs256_kv8192_counters.md")


def stage1_source_hash() -> str:
    h = hashlib.sha256()
    for p in STAGE1_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per stage-1 launch from the committed counter summary, or
    None if absent or taken on a different kernel source."""
    if not os.path.exists(PMC_SUMMARY):
        return None, "no counter summary"
    text = open(PMC_SUMMARY).read()
    m = re.search(r"<!--\s*traffic-json:\s*(\{.*?\})\s*-->", text, re.S)
    if not m:
        return None, "counter summary has no traffic line"
    d = json.loads(m.group(1))
    if d.get("stage1_source_hash") != stage1_source_hash():
        return None, "kernel changed since the counters were taken"
    return float(d["hbm_bytes_per_launch"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def cpu_baseline(w, q, kv, nsample: int):
    import numpy as np

    import oracle
    import workloads
    qo, kvp = workloads.indptrs([w.kv_len] * w.batch)
    nsample = min(nsample, w.batch)
    seqs = list(range(0, w.batch, max(1, w.batch // nsample)))[:nsample]
    # cache encoding is input preparation (untimed, as on the GPU side)
    rows = np.concatenate([np.arange(kvp[b], kvp[b + 1]) for b in seqs])
    sub_kv = kv[rows]
    sub_kvp = np.zeros(len(seqs) + 1, dtype=np.int32)
    sub_kvp[1:] = np.cumsum([kvp[b + 1] - kvp[b] for b in seqs])
    if w.kv_format == "fp8":
        ks = oracle.fp8_absmax_scale(kv)
        codes, scales = oracle.fp8_quantize(sub_kv, ks), None
    else:
        ks = 0.0
        codes, scales = oracle.mxfp4_encode(sub_kv)
    t0 = time.perf_counter()
    qs = (oracle.fp8_static_scale() if w.q_scale_mode == "static"
          else oracle.fp8_absmax_scale(q))
    q8 = oracle.fp8_quantize(q, qs)
    t1 = time.perf_counter()
    sub_qo = np.arange(len(seqs) + 1, dtype=np.int32)
    oracle.mla_decode(q8[seqs], qs, codes, ks, sub_qo, sub_kvp, workloads.SM_SCALE,
                      kv_format=0 if w.kv_format == "fp8" else 1, kv_scales=scales)
    t2 = time.perf_counter()
    per_call_s = (t1 - t0) + (t2 - t1) * w.batch / len(seqs)
    return {
        "value": per_call_s * 1e6,
        "unit": "us/call",
        "cores": min(oracle.num_threads(), len(seqs)),
        "kind": "oracle",
        "sample": (f"{len(seqs)} of {w.batch} sequences (all 16 heads, fp64 attention on "
                   f"dequantised codes) plus Q quantisation of the whole batch, scaled by "
                   f"{w.batch}/{len(seqs)}; cache encoding excluded as input preparation; "
                   f"measured {t2 - t0:.2f} s wall"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bs256_kv8192_fp8")
    ap.add_argument("--q-scale", choices=["absmax", "static"], default=None)
    ap.add_argument("--max-splits", type=int, default=0)
    ap.add_argument("--num-cus", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=128)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import mla_latent_kv_bf16_amd as mla
    import workloads

    w = workloads.BY_NAME[args.workload]
    if args.q_scale:
        import dataclasses
        w = dataclasses.replace(w, q_scale_mode=args.q_scale)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs (host, seeded) -> HBM; cache encoded by the library (untimed)
    q = workloads.make_q(w.batch, w.seed_q)
    kv = workloads.make_kv([w.kv_len] * w.batch, w.seed_kv)
    qo, kvp = workloads.indptrs([w.kv_len] * w.batch)
    qd = q.to(dev)
    kvd = kv.to(dev)
    fmt = mla.MLA_KV_FP8_E4M3FN if w.kv_format == "fp8" else mla.MLA_KV_MXFP4
    if w.kv_format == "fp8":
        cache = torch.empty(kvd.shape, dtype=torch.uint8, device=dev)
        kv_scale = torch.empty(1, dtype=torch.float32, device=dev)
        qws = torch.empty(mla.mla_quant_fp8_workspace_size(kvd.numel()), dtype=torch.uint8,
                          device=dev)
        mla.mla_quant_fp8(kvd, cache, kv_scale, mla.MLA_Q_SCALE_ABSMAX, qws)
        block_scales = None
        kv_row_bytes = 576
    else:
        cache = torch.empty((kvd.shape[0], 288), dtype=torch.uint8, device=dev)
        block_scales = torch.empty((kvd.shape[0], 18), dtype=torch.uint8, device=dev)
        mla.mla_encode_mxfp4(kvd, cache, block_scales)
        kv_scale = None
        kv_row_bytes = 288 + 18
    torch.cuda.synchronize()
    del kvd

    plan = mla.mla_decode_plan(qo, kvp, fmt, num_cus=args.num_cus, max_splits=args.max_splits)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    q8 = torch.empty(qd.shape, dtype=torch.uint8, device=dev)
    q_scale = torch.empty(1, dtype=torch.float32, device=dev)
    out = torch.empty((w.batch, 16, 512), dtype=torch.bfloat16, device=dev)
    static = w.q_scale_mode == "static"
    if static:
        q_scale.fill_(6.0 / 448.0)
    mode = mla.MLA_Q_SCALE_STATIC if static else mla.MLA_Q_SCALE_ABSMAX

    def step(m=mode):
        mla.mla_decode_run(plan, qd, q8, q_scale, cache, out, kv_scale=kv_scale,
                           kv_block_scales=block_scales, q_scale_mode=m, workspace=ws)

    # ---- headline: K steps back to back, bracketed by synchronisation
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {w.name} {w.q_scale_mode}: {ms_per_step * 1e3:.1f} us/step "
          f"(host wall {wall / args.steps * 1e6:.1f} us/step)", file=sys.stderr, flush=True)

    # ---- the other Q-scale mode, same plan and cache (reported beside)
    other = mla.MLA_Q_SCALE_ABSMAX if static else mla.MLA_Q_SCALE_STATIC
    if not static:
        q_scale.fill_(6.0 / 448.0)
    for _ in range(3):
        step(other)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step(other)
    e1.record()
    torch.cuda.synchronize()
    other_ms = e0.elapsed_time(e1) / args.steps
    if not static:
        step()  # restore the absmax scale in q_scale
    torch.cuda.synchronize()

    # ---- dominant kernel alone: stage-1 launches, each between two events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for _ in range(3):
        mla.mla_decode_stage1(plan, q8, q_scale, cache, out, kv_scale=kv_scale,
                              kv_block_scales=block_scales, workspace=ws)
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        mla.mla_decode_stage1(plan, q8, q_scale, cache, out, kv_scale=kv_scale,
                              kv_block_scales=block_scales, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    s1_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # ---- bytes
    total_kv = int(kvp[-1])
    nq = w.batch * 16 * 576
    n_items = plan.num_items
    partial_bytes = 16 * 512 * 4 + 16 * 4
    kv_bytes = total_kv * kv_row_bytes
    out_bytes = w.batch * 16 * 512 * 2
    metric_bytes = (kv_bytes + nq * 2 * (1 if static else 2) + nq * 2 + out_bytes
                    + plan.num_slots * partial_bytes * 2)
    stage1_bytes = (kv_bytes + n_items * 16 * 576
                    + (n_items - plan.num_slots) * 16 * 512 * 2 + plan.num_slots * partial_bytes)
    us = ms_per_step * 1e3
    gbps = metric_bytes / (ms_per_step * 1e-3) / 1e9
    s1_gbps = stage1_bytes / (s1_ms * 1e-3) / 1e9
    if w.name == "bs256_kv8192_fp8" and w.kv_format == "fp8":
        traffic, traffic_note = read_traffic()
    else:
        traffic, traffic_note = None, "counters were taken on bs256_kv8192_fp8 only"

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    result = {
        "metric": METRIC,
        "value": round(us, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if w.kv_format == "fp8" else "fp8xfp4",
        "data": "synthetic (seeded N(0,1) bf16 Q and latent cache, cache encoded on the GPU)",
        "config": {
            "workload": w.name, "batch": w.batch, "kv_len": w.kv_len, "q_heads": 16,
            "kv_heads": 1, "qk_dim": 576, "v_dim": 512, "kv_format": w.kv_format,
            "q_scale": w.q_scale_mode, "work_items": n_items, "split_slots": plan.num_slots,
            "parallelism": "single GPU",
        },
        "hbm_gbps": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "metric_bytes_per_call": metric_bytes,
        "other_q_scale_us": {("absmax" if static else "static"): round(other_ms * 1e3, 2)},
        "stage1_us": round(s1_ms * 1e3, 2),
        "host_wall_us_per_step": round(wall / args.steps * 1e6, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(s1_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(s1_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_note": traffic_note,
            "kernel": "stage1_fp8_kernel" if w.kv_format == "fp8" else "stage1_mxfp4_kernel",
            "algorithmic_bytes_per_launch": stage1_bytes,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, q, kv, args.cpu_sample_seqs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
