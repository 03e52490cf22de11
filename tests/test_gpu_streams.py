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


def test_plan_does_not_wait_for_other_streams():
    """mla_decode_plan copies its work lists on the stream it is given and
    waits for that stream only: built on stream B while stream A still has
    milliseconds of decodes queued, it returns before A has drained, and the
    plan then decodes correctly on B."""
    announce("plan on one stream while another decodes")
    # stream A: decodes over a 604 MB cache of finite random codes (~0.1 ms each)
    lens_a = [8192] * 128
    qo_a, kvp_a = workloads.indptrs(lens_a)
    kv8 = torch.randint(0, 0x7E, (int(kvp_a[-1]), 576), dtype=torch.uint8, device=DEV)
    ks = torch.full((1,), 0.01, dtype=torch.float32, device=DEV)
    plan_a = mla.mla_decode_plan(qo_a, kvp_a)
    ws_a = torch.zeros(max(plan_a.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    mla.mla_decode_workspace_init(plan_a, ws_a)
    qa = torch.randn((128, 16, 576), device=DEV).bfloat16()
    q8a = torch.empty((128, 16, 576), dtype=torch.uint8, device=DEV)
    qsa = torch.empty(1, dtype=torch.float32, device=DEV)
    outa = torch.empty((128, 16, 512), dtype=torch.bfloat16, device=DEV)
    # stream B: a small case checked against the oracle
    job = _Job([700, 33, 1500], 820, "fp8")
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(200):
        mla.mla_decode_run_fused(plan_a, qa, q8a, qsa, kv8, outa, kv_scale=ks, workspace=ws_a,
                                 stream=sa, check=False)
    qo_b, kvp_b = workloads.indptrs([700, 33, 1500])
    plan_b = mla.mla_decode_plan(qo_b, kvp_b, stream=sb)
    a_busy = not sa.query()
    job.plan = plan_b
    job.ws = torch.zeros(max(plan_b.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    with torch.cuda.stream(sb):
        job.run(False, stream=sb)
    torch.cuda.synchronize()
    assert a_busy, "mla_decode_plan returned only after the other stream had drained"
    from gpu_cases import OracleSide, assert_close, assert_lse_close
    orc = OracleSide(workloads.make_q(3, 821), workloads.make_kv([700, 33, 1500], 820), "fp8")
    ref, ref_lse = orc.decode(qo_b, kvp_b)
    assert np.array_equal(job.q8.cpu().numpy(), orc.q8)
    assert_close(job.out.float().cpu().numpy(), ref, "plan built beside a busy stream")
    assert_lse_close(job.lse.cpu().numpy(), ref_lse, "plan built beside a busy stream")


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
