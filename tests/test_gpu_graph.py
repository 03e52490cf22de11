"""The decode captured in a HIP graph (torch.cuda.CUDAGraph): every replay,
with eager work and new Q values between replays, equals the eager run on the
same inputs bit for bit. The single-launch path keeps per-row arrival counters
that its last workgroup resets, so replays must find them at zero again; the
three-launch path is captured too. Both Q-scale modes, split and unsplit;
the FP8 and MXFP4 caches, one query row per sequence and several sharing each
tile (the MXFP4 plans with rows made for 8 compute units, so that they take
the shared-row kernel)."""
import numpy as np
import pytest
import torch

import mla_latent_kv_bf16_amd as mla
import workloads
from gpu_cases import DEV, GpuCache, announce

pytestmark = pytest.mark.gpu

# (kv lengths, max_splits, query rows per sequence, cache format, compute units)
CASES = [([1000, 333, 1, 64, 2048, 0], 0, None, "fp8", 0), ([4096] * 8, -4, None, "fp8", 0),
         ([300, 7000], 0, None, "fp8", 0), ([3000, 65, 900], -3, None, "mxfp4", 0),
         ([2000, 40, 700], -2, [2, 4, 3], "fp8", 0),
         ([2000, 40, 700], -2, [2, 4, 3], "mxfp4", 8)]


def _bits(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("q_mode", ["absmax", "static"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[3]}_{len(c[0])}seq_s{c[1]}"
                         f"{'_rows' if c[2] else ''}")
def test_graph_replays_equal_eager(case, q_mode, fused):
    kv_lens, max_splits, q_lens, fmt, cus = case
    announce(f"graph fused={fused} {q_mode} {fmt} {kv_lens} rows {q_lens} splits {max_splits}")
    qo, kvp = workloads.indptrs(kv_lens, q_lens)
    rows = int(qo[-1])
    cache = GpuCache(workloads.make_kv(kv_lens, 700 + rows), fmt)
    plan = mla.mla_decode_plan(qo, kvp, 0 if fmt == "fp8" else 1, max_splits=max_splits,
                               num_cus=cus)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    mla.mla_decode_workspace_init(plan, ws)
    q = torch.empty((rows, 16, 576), dtype=torch.bfloat16, device=DEV)
    q8 = torch.empty((rows, 16, 576), dtype=torch.uint8, device=DEV)
    q_scale = torch.full((1,), 6.0 / 448.0, dtype=torch.float32, device=DEV)
    out = torch.empty((rows, 16, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((rows, 16), dtype=torch.float32, device=DEV)
    mode = mla.MLA_Q_SCALE_ABSMAX if q_mode == "absmax" else mla.MLA_Q_SCALE_STATIC
    fn = mla.mla_decode_run_fused if fused else mla.mla_decode_run

    def step():
        fn(plan, q, q8, q_scale, cache.kv, out, kv_scale=cache.kv_scale,
           kv_block_scales=cache.block_scales, q_scale_mode=mode, workspace=ws, lse_out=lse)

    def eager(seed):
        q.copy_(workloads.make_q(rows, seed).to(DEV))
        step()
        torch.cuda.synchronize()
        return [_bits(t) for t in (out, lse, q8, q_scale)]

    refs = {s: eager(s) for s in (710, 711)}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # settle the stream before capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i, seed in enumerate([710, 711, 710, 711]):
        q.copy_(workloads.make_q(rows, seed).to(DEV))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        q8.fill_(0x55)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [_bits(t) for t in (out, lse, q8, q_scale)]
        for a, b, name in zip(got, refs[seed], ("out", "lse", "q8", "q_scale")):
            assert np.array_equal(a, b), f"replay {i} (Q seed {seed}): {name} differs from eager"
        # eager work between replays on the same buffers
        assert eager(seed)[0].tobytes() == refs[seed][0].tobytes()
    del g
