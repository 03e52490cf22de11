"""Helpers for the GPU parity tests: build one decode case on both sides.

GPU side: bf16 inputs uploaded, the KV cache quantised by the library's own
encoder, the decode run through the C ABI. Oracle side: the same bf16 inputs
quantised and decoded by the CPU oracle. Inputs come only from workloads.py.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import mla_latent_kv_bf16_amd as mla
import oracle
import workloads

DEV = torch.device("cuda:0")
TOL_ABS, TOL_REL = 1e-2, 2e-2
LSE_TOL = 2e-3


def announce(msg: str):
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


class GpuCache:
    """Device-resident quantised latent cache."""

    def __init__(self, kv_bf16_host: torch.Tensor, fmt: str):
        self.fmt = fmt
        kvd = kv_bf16_host.to(DEV)
        if fmt == "fp8":
            self.kv = torch.empty(kvd.shape, dtype=torch.uint8, device=DEV)
            self.kv_scale = torch.empty(1, dtype=torch.float32, device=DEV)
            ws = torch.empty(max(mla.mla_quant_fp8_workspace_size(kvd.numel()), 256),
                             dtype=torch.uint8, device=DEV)
            mla.mla_quant_fp8(kvd, self.kv, self.kv_scale, mla.MLA_Q_SCALE_ABSMAX, ws)
            self.block_scales = None
        else:
            rows = kvd.shape[0]
            self.kv = torch.empty((rows, 288), dtype=torch.uint8, device=DEV)
            self.block_scales = torch.empty((rows, 18), dtype=torch.uint8, device=DEV)
            mla.mla_encode_mxfp4(kvd, self.kv, self.block_scales)
            self.kv_scale = None
        torch.cuda.synchronize()
        del kvd


class GpuDecode:
    """Plan + buffers for one shape; run() returns (out bf16, lse, q8, q_scale)."""

    def __init__(self, qo, kvp, fmt: str, max_splits: int = 0, num_cus: int = 0):
        self.fmt = fmt
        self.batch = len(qo) - 1
        self.plan = mla.mla_decode_plan(qo, kvp, 0 if fmt == "fp8" else 1, num_cus=num_cus,
                                        max_splits=max_splits)
        self.ws = torch.zeros(max(self.plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
        self.rows = self.plan.rows  # query rows (= sequences at qseqlen 1)
        b = max(self.rows, 1)
        self.q8 = torch.empty((b, 16, 576), dtype=torch.uint8, device=DEV)
        self.q_scale = torch.empty(1, dtype=torch.float32, device=DEV)
        self.out = torch.empty((b, 16, 512), dtype=torch.bfloat16, device=DEV)
        self.lse = torch.empty((b, 16), dtype=torch.float32, device=DEV)

    def run(self, q_dev, cache: GpuCache, q_mode: str = "absmax", static_scale=None,
            with_lse=True, logit_cap=0.0):
        if q_mode == "static":
            self.q_scale.fill_(float(static_scale))
        mla.mla_decode_run(self.plan, q_dev, self.q8, self.q_scale, cache.kv, self.out,
                           kv_scale=cache.kv_scale, kv_block_scales=cache.block_scales,
                           q_scale_mode=(mla.MLA_Q_SCALE_STATIC if q_mode == "static"
                                         else mla.MLA_Q_SCALE_ABSMAX), logit_cap=logit_cap,
                           workspace=self.ws, lse_out=self.lse if with_lse else None)
        torch.cuda.synchronize()
        return (self.out.float().cpu().numpy(), self.lse.cpu().numpy(),
                self.q8.cpu().numpy(), np.float32(self.q_scale.item()))

    def run_fused(self, q_dev, cache: GpuCache, q_mode: str = "absmax", static_scale=None,
                  with_lse=True, init=False, logit_cap=0.0):
        """The same step through mla_decode_run_fused (init: prepare the
        workspace's counters first)."""
        if init:
            mla.mla_decode_workspace_init(self.plan, self.ws)
        if q_mode == "static":
            self.q_scale.fill_(float(static_scale))
        mla.mla_decode_run_fused(self.plan, q_dev, self.q8, self.q_scale, cache.kv, self.out,
                                 kv_scale=cache.kv_scale, kv_block_scales=cache.block_scales,
                                 q_scale_mode=(mla.MLA_Q_SCALE_STATIC if q_mode == "static"
                                               else mla.MLA_Q_SCALE_ABSMAX), logit_cap=logit_cap,
                                 workspace=self.ws, lse_out=self.lse if with_lse else None)
        torch.cuda.synchronize()
        return (self.out.float().cpu().numpy(), self.lse.cpu().numpy(),
                self.q8.cpu().numpy(), np.float32(self.q_scale.item()))


class OracleSide:
    """The same case computed by the CPU oracle."""

    def __init__(self, q_host, kv_host, fmt: str, q_mode: str = "absmax"):
        self.fmt = fmt
        self.q_scale = (oracle.fp8_static_scale() if q_mode == "static"
                        else oracle.fp8_absmax_scale(q_host))
        self.q8 = oracle.fp8_quantize(q_host, self.q_scale)
        self.kv_host = kv_host
        if fmt == "fp8":
            self.kv_scale = oracle.fp8_absmax_scale(kv_host)
        else:
            self.kv_scale = 0.0

    def kv_codes(self, rows: slice | None = None):
        x = self.kv_host if rows is None else self.kv_host[rows]
        if self.fmt == "fp8":
            return oracle.fp8_quantize(x, self.kv_scale), None
        return oracle.mxfp4_encode(x)

    def decode(self, qo, kvp, seqs=None, logit_cap=0.0):
        """fp64 reference for the selected sequences (all if None). Only the
        cache rows of those sequences are quantised."""
        if seqs is None:
            codes, scales = self.kv_codes()
            return oracle.mla_decode(self.q8, self.q_scale, codes, self.kv_scale, qo, kvp,
                                     workloads.SM_SCALE, kv_format=0 if self.fmt == "fp8" else 1,
                                     kv_scales=scales, logit_cap=logit_cap)
        outs, lses = [], []
        for b in seqs:
            lo, hi = int(kvp[b]), int(kvp[b + 1])
            codes, scales = self.kv_codes(slice(lo, hi))
            qo1 = np.array([0, 1], dtype=np.int32)
            kv1 = np.array([0, hi - lo], dtype=np.int32)
            o, l = oracle.mla_decode(self.q8[b:b + 1], self.q_scale, codes, self.kv_scale, qo1,
                                     kv1, workloads.SM_SCALE,
                                     kv_format=0 if self.fmt == "fp8" else 1, kv_scales=scales)
            outs.append(o[0])
            lses.append(l[0])
        return np.stack(outs), np.stack(lses)


def assert_close(got, ref, what=""):
    """|got - ref| <= 1e-2 + 2e-2 |ref| elementwise."""
    got = np.asarray(got, dtype=np.float64)
    excess = np.abs(got - ref) - (TOL_ABS + TOL_REL * np.abs(ref))
    worst = float(excess.max()) if excess.size else -1.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert worst <= 0, (f"{what}: outside tolerance by {worst:.3g} at "
                        f"{np.unravel_index(int(np.argmax(excess)), excess.shape)}")


def assert_lse_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: LSE finiteness differs"
    if fin.any():
        d = np.abs(got[fin] - ref[fin]).max()
        assert d <= LSE_TOL, f"{what}: LSE differs by {d:.3g}"
