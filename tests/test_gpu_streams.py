"""Concurrent decodes on two streams, each with its own plan and workspace:
every output equals the same decode run alone, bit for bit (a plan is
immutable and a run touches only its own workspace and outputs)."""
import numpy as np
import pytest
import torch

import mla_latent_kv_bf16_amd as mla
import workloads
from gpu_cases import DEV, GpuCache, announce

pytestmark = pytest.mark.gpu


class _Job:
    def __init__(self, kv_lens, seed, fmt):
        qo, kvp = workloads.indptrs(kv_lens)
        rows = len(kv_lens)
        self.cache = GpuCache(workloads.make_kv(kv_lens, seed), fmt)
        self.plan = mla.mla_decode_plan(qo, kvp, 0 if fmt == "fp8" else 1)
        self.ws = torch.zeros(max(self.plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
        mla.mla_decode_workspace_init(self.plan, self.ws)
        self.q = workloads.make_q(rows, seed + 1).to(DEV)
        self.q8 = torch.empty((rows, 16, 576), dtype=torch.uint8, device=DEV)
        self.q_scale = torch.empty(1, dtype=torch.float32, device=DEV)
        self.out = torch.empty((rows, 16, 512), dtype=torch.bfloat16, device=DEV)
        self.lse = torch.empty((rows, 16), dtype=torch.float32, device=DEV)

    def run(self, fused, stream=None):
        fn = mla.mla_decode_run_fused if fused else mla.mla_decode_run
        fn(self.plan, self.q, self.q8, self.q_scale, self.cache.kv, self.out,
           kv_scale=self.cache.kv_scale, kv_block_scales=self.cache.block_scales,
           q_scale_mode=mla.MLA_Q_SCALE_ABSMAX, workspace=self.ws, lse_out=self.lse,
           stream=stream)

    def snapshot(self):
        return [t.contiguous().view(torch.uint8).cpu().numpy().copy()
                for t in (self.out, self.lse, self.q8, self.q_scale)]


@pytest.mark.parametrize("fused", [True, False])
def test_two_streams_equal_serial(fused):
    announce(f"two streams fused={fused}")
    a = _Job([3000, 17, 4096, 900], 800, "fp8")
    b = _Job([5000, 1, 2048], 810, "mxfp4")
    a.run(fused)
    b.run(fused)
    torch.cuda.synchronize()
    ref_a, ref_b = a.snapshot(), b.snapshot()
    for t in (a.out, b.out):
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(5):  # interleaved launches on both streams
        a.run(fused, stream=sa)
        b.run(fused, stream=sb)
    torch.cuda.synchronize()
    for got, ref, name in ((a.snapshot(), ref_a, "a"), (b.snapshot(), ref_b, "b")):
        for x, y, what in zip(got, ref, ("out", "lse", "q8", "q_scale")):
            assert np.array_equal(x, y), f"job {name}: {what} differs from its serial run"
