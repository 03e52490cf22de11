#!/usr/bin/env python3
"""Benchmark of absorbed-path MLA decode on one MI355X.

One step = one ``mla_decode_run_fused`` call (Q quantisation inside the
split-KV attention kernel, LSE merge by the last workgroup of each split
sequence; with an absmax Q scale one small reduction launch runs first) over
the workload's synthetic inputs, which are resident in HBM before the timed
region starts. Its outputs equal those of the three-launch ``mla_decode_run``
bit for bit; both paths are timed in both Q-scale modes. Prints ONE JSON line.

Default workload: bs=256, kv_len=8192 per sequence, FP8 E4M3FN latent cache
(2,097,152 cache rows, 1.21 GB), absmax Q scale. The cache is 4.7x the
MI355X's 256 MB last-level cache, so back-to-back steps read it from HBM.

Roofline: the dominant kernel is the fused stage-1 attention kernel (the only
launch of a static-scale step). Its algorithmic bytes per launch (576 B per
cache row, each work item's 18,432 B of bf16 Q, the Q codes written once per
sequence, the output, and split partials written and read back) over its
average duration in a run of back-to-back launches (HIP events around the
run, on the stream the library launches on), against the 8 TB/s HBM peak.
Single launches between two events are also reported, hot and after a
512 MiB read that evicts the 256 MB last-level cache ("cold"); for the
default workload, whose cache is far larger than that cache, the two agree. ``traffic`` is
that kernel's measured HBM bytes from the committed rocprofv3 counter
summary, scaled by the counters of a plain copy of known size, or null when
the kernel source has changed since it was taken.

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
_CSRC = "mla_latent_kv_bf16_amd/csrc/"
# Counter summaries of the dominant kernel per cache format, and the sources
# whose hash they record: a summary taken on an older kernel reads as null.
COUNTERS = {
    "fp8": ("stage1_fp8_fused_bs256_kv8192_counters.md",
            ["stage1_fp8.hip", "stage1_fp8_tile.h", "device_common.h", "stage_common.h",
             "../build.py"]),
    "bf16": ("stage1_bf16_bs256_kv8192_counters.md",
             ["stage1_bf16.hip", "device_common.h", "stage_common.h", "../build.py"]),
    "mxfp4": ("stage1_mxfp4_bs256_kv1024_counters.md",
              ["stage1_mxfp4.hip", "device_common.h", "stage_common.h", "../build.py"]),
    "rows": (None, ["stage1_fp8_rows.hip", "stage1_fp8_tile.h", "device_common.h",
                    "stage_common.h", "../build.py"]),
}
MFMA_SUMMARY = os.path.join(ROOT, "profiles", "stage1_mfma_busy_bs256.md")
# traffic of the fused static-scale FP8 launch at the smaller FP8 workloads
SMALL_COUNTERS = "stage1_fp8_fused_small_batches_counters.md"
# (batch, kv_len) of the workload each format's counter summary was taken on
COUNTER_SHAPES = {"fp8": (256, 8192), "bf16": (256, 8192), "mxfp4": (256, 1024)}


def _code_only(text: str) -> str:
    """Source text without comments and blank space, so that a comment edit
    does not count as a kernel change."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def stage1_source_hash(fmt: str = "fp8") -> str:
    h = hashlib.sha256()
    for p in COUNTERS[fmt][1]:
        with open(os.path.join(ROOT, _CSRC + p)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(fmt: str):
    """HBM bytes per launch of the format's dominant kernel from the committed
    counter summary, or None if absent or taken on a different kernel source."""
    if COUNTERS.get(fmt, (None,))[0] is None:
        return None, f"no counters are kept for the {fmt} cache"
    path = os.path.join(ROOT, "profiles", COUNTERS[fmt][0])
    if not os.path.exists(path):
        return None, "no counter summary"
    text = open(path).read()
    m = re.search(r"<!--\s*traffic-json:\s*(\{.*?\})\s*-->", text, re.S)
    if not m:
        return None, "counter summary has no traffic line"
    d = json.loads(m.group(1))
    if d.get("stage1_source_hash") != stage1_source_hash(fmt):
        return None, "kernel changed since the counters were taken"
    return float(d["hbm_bytes_per_launch"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def read_workload_traffic(name: str):
    """HBM bytes per fused static-scale launch of one of the smaller FP8
    workloads, from the committed counter summary, or None if absent or
    taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", SMALL_COUNTERS)
    if not os.path.exists(path):
        return None
    m = re.search(r"<!--\s*traffic-map-json:\s*(\{.*?\})\s*-->", open(path).read(), re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("stage1_source_hash") != stage1_source_hash("fp8"):
        return None
    e = d["workloads"].get(name)
    return float(e["hbm_bytes_per_launch"]) if e else None


def workload_traffic(w):
    """Measured HBM bytes per fused static-scale launch of a one-row workload
    from whichever committed summary covers it, else None."""
    if COUNTER_SHAPES.get(w.kv_format) == (w.batch, w.kv_len):
        return read_traffic(w.kv_format)[0]
    return read_workload_traffic(w.name) if w.kv_format == "fp8" else None


def read_mfma_busy(key: str):
    """MfmaUtil (%) of a stage-1 kernel from the committed summary, or None if
    absent or taken on a different kernel source (keys: fp8, bf16, mxfp4,
    rows4 = the FP8 cache with 4 query rows)."""
    if not os.path.exists(MFMA_SUMMARY):
        return None
    m = re.search(r"<!--\s*mfma-json:\s*(\{.*?\})\s*-->", open(MFMA_SUMMARY).read(), re.S)
    d = json.loads(m.group(1)).get(key) if m else None
    if not d:
        return None
    fmt = "rows" if key == "rows4" else key
    if d.get("source_hash") != stage1_source_hash(fmt):
        return None
    return d["mfma_util_pct"]


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
    if w.kv_format == "bf16":
        pass
    elif w.kv_format == "fp8":
        ks = oracle.fp8_absmax_scale(kv)
        codes, scales = oracle.fp8_quantize(sub_kv, ks), None
    else:
        ks = 0.0
        codes, scales = oracle.mxfp4_encode(sub_kv)
    if w.kv_format == "bf16":  # the oracle reads the bf16 rows as they are
        t0 = time.perf_counter()
        oracle.mla_decode_bf16(q, kv, np.arange(w.batch + 1, dtype=np.int32), kvp,
                               workloads.SM_SCALE, seqs=seqs)
        t2 = time.perf_counter()
        return {
            "value": (t2 - t0) * w.batch / len(seqs) * 1e6,
            "unit": "us/call",
            "cores": min(oracle.num_threads(), len(seqs)),
            "kind": "oracle",
            "sample": (f"{len(seqs)} of {w.batch} sequences (all 16 heads, fp64 attention on "
                       f"the bf16 rows), scaled by {w.batch}/{len(seqs)}; measured "
                       f"{t2 - t0:.2f} s wall"),
        }
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


class Case:
    """One workload resident in HBM: inputs, encoded cache, plan, buffers."""

    def __init__(self, w, args, dev):
        import torch

        import mla_latent_kv_bf16_amd as mla
        import workloads
        self.w = w
        self.R = getattr(args, "q_len", 1) or 1  # query rows per sequence
        self.rows = w.batch * self.R
        self.q = workloads.make_q(self.rows, w.seed_q)
        self.kv_host = workloads.make_kv([w.kv_len] * w.batch, w.seed_kv)
        self.qo, self.kvp = workloads.indptrs([w.kv_len] * w.batch, [self.R] * w.batch)
        self.qd = self.q.to(dev)
        kvd = self.kv_host.to(dev)
        fmt = {"fp8": mla.MLA_KV_FP8_E4M3FN, "mxfp4": mla.MLA_KV_MXFP4,
               "bf16": mla.MLA_KV_BF16}[w.kv_format]
        self.bf16 = w.kv_format == "bf16"
        if self.bf16:
            self.cache = kvd.clone()  # the bf16 latent rows themselves
            self.kv_scale = None
            self.block_scales = None
            self.kv_row_bytes = 576 * 2
        elif w.kv_format == "fp8":
            self.cache = torch.empty(kvd.shape, dtype=torch.uint8, device=dev)
            self.kv_scale = torch.empty(1, dtype=torch.float32, device=dev)
            qws = torch.empty(mla.mla_quant_fp8_workspace_size(kvd.numel()), dtype=torch.uint8,
                              device=dev)
            mla.mla_quant_fp8(kvd, self.cache, self.kv_scale, mla.MLA_Q_SCALE_ABSMAX, qws)
            self.block_scales = None
            self.kv_row_bytes = 576
        else:
            self.cache = torch.empty((kvd.shape[0], 288), dtype=torch.uint8, device=dev)
            self.block_scales = torch.empty((kvd.shape[0], 18), dtype=torch.uint8, device=dev)
            mla.mla_encode_mxfp4(kvd, self.cache, self.block_scales)
            self.kv_scale = None
            self.kv_row_bytes = 288 + 18
        torch.cuda.synchronize()
        del kvd
        # hashed here, as encoded and before any scatter into pages: copying
        # the cache to the host later would sit between a paged pool's
        # warm-up and the timed steps
        self.input_hashes = input_hashes(self)
        self.page_size = getattr(args, "page_size", 0) or 0
        if self.page_size:
            # the cache's rows scattered over a pool of pages in a seeded order
            (pi, ids, last, self.num_pages,
             rows) = workloads.make_page_table([w.kv_len] * w.batch, self.page_size, w.seed_kv)
            pool = torch.zeros((self.num_pages * self.page_size, self.cache.shape[1]),
                               dtype=self.cache.dtype, device=dev)
            rows_d = torch.from_numpy(rows).to(dev)
            pool[rows_d] = self.cache
            self.cache = pool
            if self.block_scales is not None:
                spool = torch.zeros((self.num_pages * self.page_size, 18), dtype=torch.uint8,
                                    device=dev)
                spool[rows_d] = self.block_scales
                self.block_scales = spool
            self.page_ids = torch.from_numpy(ids).to(dev)
            self.plan = mla.mla_decode_plan_paged(self.qo, pi, last, self.page_size, fmt,
                                                  num_cus=args.num_cus,
                                                  max_splits=args.max_splits)
        else:
            self.plan = mla.mla_decode_plan(self.qo, self.kvp, fmt, num_cus=args.num_cus,
                                            max_splits=args.max_splits)
        # the library's choice for query rows (1-4 per sequence): the FP8
        # cache always shares each tile between them, the MXFP4 cache when
        # the per-row schedule would need more than one round of workgroups
        self.shared_rows = False
        if 1 < self.R <= 4 and fmt != mla.MLA_KV_BF16:
            per_row = mla.mla_decode_plan_host(self.qo, self.kvp, fmt, num_cus=args.num_cus,
                                               max_splits=args.max_splits)[0].shape[0]
            cus = args.num_cus or torch.cuda.get_device_properties(dev).multi_processor_count
            self.shared_rows = fmt == mla.MLA_KV_FP8_E4M3FN or per_row > cus
        self.ws = torch.empty(max(self.plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
        mla.mla_decode_workspace_init(self.plan, self.ws)
        self.q8 = torch.empty(self.qd.shape, dtype=torch.uint8, device=dev)
        self.q_scale = torch.empty(1, dtype=torch.float32, device=dev)
        self.out = torch.empty((self.rows, 16, 512), dtype=torch.bfloat16, device=dev)
        self.checked = False  # the binding's buffer checks ran once on these buffers
        if self.page_size:
            # A freshly scattered pool runs slower for its first few dozen
            # passes (measured: bs256 kv8192 FP8 at one row per page, 250 us
            # per step over the first 60 and 215 us after, static or absmax
            # alike), so its preparation ends with PAGED_POOL_WARMUP untimed
            # static-scale steps.
            self.q_scale.fill_(STATIC_Q_SCALE)
            for _ in range(PAGED_POOL_WARMUP):
                self.step(True, True)
            torch.cuda.synchronize()

    def step(self, fused: bool, static: bool):
        import mla_latent_kv_bf16_amd as mla
        # the first call checks the buffers against the plan; the timed loops
        # then skip those host-side checks (same buffers every step)
        check, self.checked = not self.checked, True
        if self.bf16 and self.page_size:  # one path: no Q quantisation, single launch
            mla.mla_decode_run_bf16_paged(self.plan, self.qd, self.cache, self.page_ids,
                                          self.num_pages, self.out, workspace=self.ws,
                                          check=check)
            return
        if self.bf16:
            mla.mla_decode_run_bf16(self.plan, self.qd, self.cache, self.out, workspace=self.ws,
                                    check=check)
            return
        if self.page_size:
            fn = mla.mla_decode_run_fused_paged if fused else mla.mla_decode_run_paged
            fn(self.plan, self.qd, self.q8, self.q_scale, self.cache, self.page_ids,
               self.num_pages, self.out, kv_scale=self.kv_scale,
               kv_block_scales=self.block_scales,
               q_scale_mode=mla.MLA_Q_SCALE_STATIC if static else mla.MLA_Q_SCALE_ABSMAX,
               workspace=self.ws, check=check)
            return
        fn = mla.mla_decode_run_fused if fused else mla.mla_decode_run
        fn(self.plan, self.qd, self.q8, self.q_scale, self.cache, self.out,
           kv_scale=self.kv_scale, kv_block_scales=self.block_scales,
           q_scale_mode=mla.MLA_Q_SCALE_STATIC if static else mla.MLA_Q_SCALE_ABSMAX,
           workspace=self.ws, check=check)

    def time_steps(self, fused: bool, static: bool, steps: int, warmup: int):
        """Mean ms per step over `steps` back-to-back steps (events around the
        whole run, synchronised on both sides) and the host wall time."""
        import torch
        if static:
            self.q_scale.fill_(STATIC_Q_SCALE)
        for _ in range(warmup):
            self.step(fused, static)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self.step(fused, static)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall / steps

    def per_launch_ms(self, launch, steps: int, between=None, samples=False):
        """Mean duration of single calls, each between two events (with
        `between` run outside the events before each call); with samples=True
        also the list of durations."""
        import numpy as np
        import torch
        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            if between is not None:
                between()
            a.record()
            launch()
            b.record()
        torch.cuda.synchronize()
        d = [a.elapsed_time(b) for a, b in evs]
        return (float(np.mean(d)), d) if samples else float(np.mean(d))

    def stage1_ms(self, steps: int):
        import mla_latent_kv_bf16_amd as mla
        if self.page_size or self.bf16:
            return float("nan")  # the plain stage-1 entry point takes no page table
        return self.per_launch_ms(
            lambda: mla.mla_decode_stage1(self.plan, self.q8, self.q_scale, self.cache, self.out,
                                          kv_scale=self.kv_scale,
                                          kv_block_scales=self.block_scales, workspace=self.ws,
                                          check=not self.checked),
            steps)

    def metric_bytes(self, static: bool) -> int:
        """B: bytes a decode step moves by the method's definition: latent
        cache + bf16 Q (read twice with an absmax scale) + Q codes (written and
        read) + bf16 O + split partials (written and read)."""
        w = self.w
        nq = self.rows * 16 * 576
        partial_bytes = 16 * 512 * 4 + 16 * 4
        if self.bf16:  # bf16 Q read once, no codes
            return (int(self.kvp[-1]) * self.kv_row_bytes + nq * 2 + self.rows * 16 * 512 * 2
                    + self.plan.num_slots * partial_bytes * 2)
        return (int(self.kvp[-1]) * self.kv_row_bytes + nq * 2 * (1 if static else 2) + 2 * nq
                + self.rows * 16 * 512 * 2 + self.plan.num_slots * partial_bytes * 2)

    def min_bytes(self) -> int:
        """B_min: latent cache + bf16 Q + bf16 O, which no schedule avoids (a
        time-based fraction of it cannot be raised by choosing more splits)."""
        w = self.w
        return (int(self.kvp[-1]) * self.kv_row_bytes + self.rows * 16 * 576 * 2
                + self.rows * 16 * 512 * 2)

    def fused_bytes(self, static: bool) -> int:
        """Algorithmic bytes of one fused stage-1 launch: cache rows, each
        item's bf16 Q rows (and absmax partials), Q codes written once per
        sequence, the output, and split partials written and read back."""
        w = self.w
        n_items = self.plan.num_items
        partial_bytes = 16 * 512 * 4 + 16 * 4
        nb = 0 if (static or self.bf16) else 4 * min(1024, -(-self.rows * 16 * 576 // (8 * 256)))
        codes = 0 if self.bf16 else self.rows * 16 * 576
        return (int(self.kvp[-1]) * self.kv_row_bytes + n_items * (16 * 576 * 2 + nb)
                + codes + self.rows * 16 * 512 * 2
                + self.plan.num_slots * partial_bytes * 2)

    def stage1_bytes(self) -> int:
        """Algorithmic bytes of one plain stage-1 launch: cache rows, each
        item's Q codes, and the output or partial it writes."""
        n_items = self.plan.num_items
        partial_bytes = 16 * 512 * 4 + 16 * 4
        return (int(self.kvp[-1]) * self.kv_row_bytes + n_items * 16 * 576
                + (n_items - self.plan.num_slots) * 16 * 512 * 2
                + self.plan.num_slots * partial_bytes)


STATIC_Q_SCALE = 6.0 / 448.0
PAGED_POOL_WARMUP = 64  # untimed steps after a paged pool is built
FLUSH_BYTES = 512 << 20   # cold-cache mode: a 512 MiB read between calls (MALL is 256 MB)


NT_CACHE_BYTES = 512 << 20  # the library streams caches this large with non-temporal loads


def kernel_name(w, args, cache_bytes: int, shared_rows: bool = False) -> str:
    """The stage-1 kernel instance the roofline times (fused, static scale)."""
    # the MXFP4 kernel's page form: 0 contiguous, 1 one page per tile, 2 pages of 8 or 16
    # rows, 3 pages of 1, 2 or 4 rows
    mx_pg = (0 if not args.page_size else 1 if args.page_size >= 32
             else 2 if args.page_size >= 8 else 3)
    if shared_rows and w.kv_format == "fp8":
        paged = "true" if args.page_size else "false"
        return (f"stage1_fp8_rows_kernel<true, {paged}> (fused, static Q scale; "
                "1-4 rows per sequence)")
    if shared_rows:
        return (f"stage1_mxfp4_rows_kernel<true, {mx_pg}> (fused, static Q scale; "
                "1-4 rows per sequence)")
    nt = "true" if cache_bytes >= NT_CACHE_BYTES else "false"
    return {"fp8": f"stage1_fp8_kernel<true, {'true' if args.page_size else 'false'}, {nt}>"
                   " (fused, static Q scale)",
            "mxfp4": f"stage1_mxfp4_kernel<true, {nt}, {mx_pg}>"
                     " (fused, static Q scale)",
            "bf16": f"stage1_bf16_kernel<true, {nt}, {'true' if args.page_size else 'false'}>"
            }[w.kv_format]


def input_hashes(c) -> dict:
    """SHA-256 of the headline workload's inputs: the seeded bf16 Q and latent
    cache, and the cache as the library encoded it (codes and scales, in
    sequence order before any scatter into pages)."""
    import torch

    def sha(t):
        t = t.detach().contiguous().cpu()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        return hashlib.sha256(t.numpy().tobytes()).hexdigest()
    torch.cuda.synchronize()
    out = {"q_bf16": sha(c.q), "kv_bf16": sha(c.kv_host), "kv_encoded": sha(c.cache)}
    if c.kv_scale is not None:
        out["kv_scale"] = sha(c.kv_scale)
    if c.block_scales is not None:
        out["kv_block_scales"] = sha(c.block_scales)
    return out


def pct(d, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(d) * 1e3, q)), 2)


_probe = None


def read_probe(nt: bool = False):
    """libmla_hbm_probe.so's streaming read (cached loads, or non-temporal)."""
    return _probe_lib()[1 if nt else 0]


def _probe_lib():
    global _probe
    if _probe is None:
        import ctypes
        lib = ctypes.CDLL(os.path.join(ROOT, "mla_latent_kv_bf16_amd", "libmla_hbm_probe.so"))
        for fn in (lib.mla_hbm_read_probe, lib.mla_hbm_read_probe_nt):
            fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                           ctypes.c_void_p]
            fn.restype = ctypes.c_int
        lib.mla_hbm_read_probe_lds_nt.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                                  ctypes.c_void_p]
        lib.mla_hbm_read_probe_lds_nt.restype = ctypes.c_int
        _probe = (lib.mla_hbm_read_probe, lib.mla_hbm_read_probe_nt,
                  lib.mla_hbm_read_probe_lds_nt)
    return _probe


class Flush:
    """Reads 512 MiB between calls so that none of the call's inputs is left
    in the 256 MB last-level cache (a read leaves no dirty lines whose
    write-back would compete with the timed call)."""

    def __init__(self, dev):
        import torch
        self.buf = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def __call__(self):
        import torch
        rc = read_probe()(self.buf.data_ptr(), FLUSH_BYTES, self.sink.data_ptr(), 2048,
                          torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(f"mla_hbm_read_probe failed ({rc})")


def measured_read_peak(dev, reps: int = 10):
    """Best HBM read bandwidth of a streaming read over 2 GiB
    (libmla_hbm_probe.so): 16-byte loads into registers, cached or
    non-temporal, or non-temporal buffer->LDS copies (the decode kernels'
    form), over a few grids; in GB/s, with the kind and grid that reached it."""
    import torch
    nbytes = 2 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    best = (0.0, "")
    kinds = {0: "cached loads", 1: "non-temporal loads", 2: "non-temporal buffer->LDS copies"}
    runs = [(k, grid) for k in (0, 1) for grid in (1024, 2048, 4096, 8192)]
    runs += [(2, grid) for grid in (256, 512, 1024)]
    for kind, grid in runs:
        probe = _probe_lib()[kind]

        def go():
            if kind == 2:
                rc = probe(buf.data_ptr(), nbytes, grid, stream)
            else:
                rc = probe(buf.data_ptr(), nbytes, sink.data_ptr(), grid, stream)
            if rc:
                raise RuntimeError(f"mla_hbm_read_probe failed ({rc})")
        go()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            go()
        e1.record()
        torch.cuda.synchronize()
        gbps = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        best = max(best, (gbps, f"{kinds[kind]}, grid {grid}"))
    del buf
    torch.cuda.empty_cache()
    return round(best[0], 1), best[1]


def measure_paths(c: Case, steps: int, warmup: int) -> dict:
    """us/call of the four library paths: {run, run_fused} x {absmax, static}
    (the bf16 cache has one path)."""
    if c.bf16:
        ms, _ = c.time_steps(True, True, steps, warmup)
        return {"run_bf16": round(ms * 1e3, 2)}
    res = {}
    for fused in (False, True):
        for static in (False, True):
            ms, _ = c.time_steps(fused, static, steps, warmup)
            res[f"{'run_fused' if fused else 'run'}_{'static' if static else 'absmax'}"] = (
                round(ms * 1e3, 2))
    return res


def graph_step_us(c: Case, static: bool, nsteps: int = 20, reps: int = 10) -> float:
    """us per step of the fused path with nsteps steps captured in one HIP
    graph and the graph replayed reps times between two events (the launch
    gaps of a captured decode loop)."""
    import torch
    if static:
        c.q_scale.fill_(STATIC_Q_SCALE)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        c.step(True, static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(nsteps):
            c.step(True, static)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (reps * nsteps)


def measure_case(c: Case, args, static: bool, flush) -> dict:
    """Per-call time distribution of the fused path (each call between two
    events), back to back ("hot") and after a 512 MiB read that evicts the
    256 MB last-level cache ("cold"), and the per-step time of a captured
    loop; empty in headline-only runs."""
    if flush is None:
        return {}
    if static:
        c.q_scale.fill_(STATIC_Q_SCALE)
    _, hot = c.per_launch_ms(lambda: c.step(True, static), args.steps, samples=True)
    _, cold = c.per_launch_ms(lambda: c.step(True, static), args.steps,
                              between=flush, samples=True)
    return {"per_call_us_p10_p50_p90": [pct(hot, 10), pct(hot, 50), pct(hot, 90)],
            "cold_per_call_us_p10_p50_p90": [pct(cold, 10), pct(cold, 50), pct(cold, 90)],
            "graph_us_per_step": round(graph_step_us(c, static), 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bs256_kv8192_fp8")
    ap.add_argument("--q-scale", choices=["absmax", "static"], default=None)
    ap.add_argument("--max-splits", type=int, default=0)
    ap.add_argument("--page-size", type=int, default=0,
                    help="paged cache with pages of this many rows (a power of two; MXFP4: at "
                         "least 8), the pages in a seeded random order; 0 = contiguous cache")
    ap.add_argument("--kv-format", choices=["fp8", "mxfp4", "bf16"], default=None,
                    help="override the workload's cache format (bf16: the unquantised path)")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query rows per sequence (multi-token prediction; causal within the "
                         "sequence)")
    ap.add_argument("--num-cus", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the per-workload summary of the other four shapes")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the fused path (headline and single launches); for profiler runs")
    ap.add_argument("--cpu-sample-seqs", type=int, default=128)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the decode runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import workloads

    w = workloads.BY_NAME[args.workload]
    if args.q_scale or args.kv_format:
        import dataclasses
        w = dataclasses.replace(w, q_scale_mode=args.q_scale or w.q_scale_mode,
                                kv_format=args.kv_format or w.kv_format)
        w = dataclasses.replace(w, name=f"bs{w.batch}_kv{w.kv_len}_{w.kv_format}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    static = w.q_scale_mode == "static"
    bf16 = w.kv_format == "bf16"

    # the read ceiling is probed before the first workload and after the
    # last (sustained streaming lowers it by a few per cent); the best counts
    peak0 = None if args.headline_only else measured_read_peak(dev)
    c = Case(w, args, dev)
    q_host, kv_host = c.q, c.kv_host
    c_items, c_slots = c.plan.num_items, c.plan.num_slots
    c_cache_bytes = int(c.kvp[-1]) * c.kv_row_bytes
    c_shared_rows = c.shared_rows
    inputs_sha256 = c.input_hashes
    flush = None if args.headline_only else Flush(dev)
    # ---- the four library paths (also warms the GPU up), unless only the
    # headline is wanted (profiler runs)
    paths = {} if args.headline_only else measure_paths(c, args.steps, 3)
    if paths:
        print(f"[bench] paths {paths}", file=sys.stderr, flush=True)
    # ---- headline: the single-launch path in the workload's Q-scale mode
    ms_per_step, wall = c.time_steps(True, static, args.steps, args.warmup)
    print(f"[bench] {w.name} {w.q_scale_mode} fused: {ms_per_step * 1e3:.1f} us/step",
          file=sys.stderr, flush=True)
    head = measure_case(c, args, static, flush)

    # ---- the fused kernel alone (a static-scale fused run is one launch) and
    # the plain stage-1 kernel alone, each launch between two events
    c.q_scale.fill_(STATIC_Q_SCALE)
    fused_ms, _ = c.time_steps(True, True, args.steps, args.warmup)
    fused_1_ms = c.per_launch_ms(lambda: c.step(True, True), args.steps)
    cold_none = flush is None
    fused_cold_ms = (float("nan") if cold_none else
                     c.per_launch_ms(lambda: c.step(True, True), args.steps, between=flush))
    if args.headline_only:
        s1_ms = float("nan")
    else:
        c.time_steps(False, static, 1, 0)  # codes and scale in q8 / q_scale for stage 1
        s1_ms = c.stage1_ms(args.steps)
    us = ms_per_step * 1e3
    mbytes = c.metric_bytes(static)
    gbps = mbytes / (ms_per_step * 1e-3) / 1e9
    bmin = c.min_bytes()
    s1_bytes = c.stage1_bytes()
    s1_gbps = s1_bytes / (s1_ms * 1e-3) / 1e9
    f_bytes = c.fused_bytes(True)
    f_gbps = f_bytes / (fused_ms * 1e-3) / 1e9
    cshape = COUNTER_SHAPES.get(w.kv_format)
    if (w.batch, w.kv_len) == cshape and not args.page_size and args.q_len == 1:
        traffic, traffic_note = read_traffic(w.kv_format)
    elif cshape:
        traffic, traffic_note = None, f"counters were taken on bs{cshape[0]}_kv{cshape[1]} only"
    else:
        traffic, traffic_note = None, f"no counters are kept for the {w.kv_format} cache"
    mfma_key = {(256, 8192, "fp8", 1): "fp8", (256, 8192, "bf16", 1): "bf16",
                (256, 1024, "mxfp4", 1): "mxfp4", (256, 8192, "fp8", 4): "rows4"}.get(
        (w.batch, w.kv_len, w.kv_format, args.q_len))
    mfma_busy = read_mfma_busy(mfma_key) if mfma_key and not args.page_size else None

    others = {}
    if not (args.no_other_workloads or args.headline_only or args.page_size or args.kv_format):
        for ow in workloads.WORKLOADS:
            if ow.name == w.name:
                continue
            del c
            torch.cuda.empty_cache()
            c = Case(ow, args, dev)
            ostatic = ow.q_scale_mode == "static"
            # the four paths first: they also warm the freshly allocated case up
            # (its first steps run slower while its pages are first touched)
            opaths = measure_paths(c, args.steps, 3)
            ms, _ = c.time_steps(True, ostatic, args.steps, args.warmup)
            ob = c.metric_bytes(ostatic)
            o_s1 = c.stage1_ms(args.steps)
            c.q_scale.fill_(STATIC_Q_SCALE)
            o_f, _ = c.time_steps(True, True, args.steps, args.warmup)
            o_f1 = c.per_launch_ms(lambda: c.step(True, True), args.steps)
            o_fc = c.per_launch_ms(lambda: c.step(True, True), args.steps, between=flush)
            ofb = c.fused_bytes(True)
            others[ow.name] = {
                "us_per_call": round(ms * 1e3, 2),
                "hbm_gbps": round(ob / (ms * 1e-3) / 1e9, 1),
                "hbm_frac_of_peak": round(ob / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "bmin_frac_of_peak": round(c.min_bytes() / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "q_scale": ow.q_scale_mode,
                **measure_case(c, args, ostatic, flush),
                "fused_kernel_us": round(o_f * 1e3, 2),
                "fused_kernel_frac_of_peak": round(ofb / (o_f * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "fused_kernel_single_launch_us_hot_cold": [round(o_f1 * 1e3, 2),
                                                           round(o_fc * 1e3, 2)],
                "fused_kernel_cold_frac_of_peak": round(
                    ofb / (o_fc * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "cache_bytes": int(c.kvp[-1]) * c.kv_row_bytes,
                "fused_kernel_algorithmic_bytes": ofb,
                "fused_kernel_traffic_bytes": workload_traffic(ow),
                "plain_stage1_us": round(o_s1 * 1e3, 2),
                "plain_stage1_frac_of_peak": round(
                    c.stage1_bytes() / (o_s1 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "paths_us": opaths,
            }
            print(f"[bench] {ow.name}: {others[ow.name]}", file=sys.stderr, flush=True)
        del c
        torch.cuda.empty_cache()
    del flush
    torch.cuda.empty_cache()
    peak1 = None if args.headline_only else measured_read_peak(dev)
    read_peak, read_grid = max(peak0, peak1) if peak0 else (None, None)

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
        "dtype": {"fp8": "fp8", "mxfp4": "fp8xfp4", "bf16": "bf16"}[w.kv_format],
        "data": "synthetic (seeded N(0,1) bf16 Q and latent cache, cache encoded on the GPU)",
        "config": {
            "workload": w.name, "batch": w.batch, "kv_len": w.kv_len, "q_len": args.q_len,
            "page_size": args.page_size or None,
            "q_heads": 16,
            "kv_heads": 1, "qk_dim": 576, "v_dim": 512, "kv_format": w.kv_format,
            "q_scale": None if bf16 else w.q_scale_mode,
            "entry_point": "mla_decode_run_bf16" if bf16 else "mla_decode_run_fused",
            "work_items": c_items, "split_slots": c_slots, "parallelism": "single GPU",
        },
        "inputs_sha256": inputs_sha256,
        "hbm_gbps": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "metric_bytes_per_call": mbytes,
        "bmin_bytes_per_call": bmin,
        "bmin_frac_of_peak": round(bmin / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "measured_read_peak_gbps": read_peak,
        "measured_read_peak_probe": read_grid,
        "measured_read_peak_first_last_gbps": [peak0[0], peak1[0]] if peak0 else None,
        **head,
        "paths_us": paths,
        "plain_stage1": None if (args.headline_only or args.page_size or bf16) else {
            "us": round(s1_ms * 1e3, 2), "gbps": round(s1_gbps, 1),
            "frac": round(s1_gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes_per_launch": s1_bytes},
        "host_wall_us_per_step": round(wall * 1e6, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(f_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(f_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_note": traffic_note,
            "kernel": kernel_name(w, args, c_cache_bytes, c_shared_rows),
            "kernel_us": round(fused_ms * 1e3, 2),
            "kernel_us_note": "mean of back-to-back static-scale fused launches",
            "single_launch_us_hot_cold": [round(fused_1_ms * 1e3, 2),
                                          None if cold_none else round(fused_cold_ms * 1e3, 2)],
            "frac_cold": None if cold_none else round(
                f_bytes / (fused_cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "cache_state": (f"cache {c_cache_bytes / 1e9:.2f} GB against the 256 MB last-level "
                            "cache: " + ("streamed from HBM every step" if
                                         c_cache_bytes > (512 << 20) else
                                         "resident in it between hot steps; frac_cold is "
                                         "the single launch after a 512 MiB read")),
            "algorithmic_bytes_per_launch": f_bytes,
            "frac_of_measured_read_peak": round(f_gbps / read_peak, 4) if read_peak else None,
            "mfma_busy_pct": mfma_busy,
            "mfma_busy_note": ("rocprofv3 MfmaUtil, profiles/stage1_mfma_busy_bs256.md"
                               if mfma_busy is not None else
                               "no MfmaUtil summary for this kernel source and workload"),
        },
        "other_workloads": others,
    }
    if not args.no_cpu_baseline and args.q_len == 1:
        result["cpu_baseline"] = cpu_baseline(w, q_host, kv_host, args.cpu_sample_seqs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
