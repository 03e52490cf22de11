"""GPU parity of the bf16 path (bf16 Q and cache, no quantisation) and of the
logit soft-cap, through mla_decode_run_bf16, against the oracle element by
element (|gpu - ref| <= 1e-2 + 2e-2 |ref|, LSE within 2e-3)."""
import numpy as np
import pytest
import torch

import mla_latent_kv_bf16_amd as mla
import oracle
import workloads
from gpu_cases import DEV, announce, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu
SM = workloads.SM_SCALE


def _run(kv_lens, q_lens, seed, cap=0.0, max_splits=0, reps=1):
    qo, kvp = workloads.indptrs(kv_lens, q_lens)
    rows = int(qo[-1])
    q = workloads.make_q(rows, seed)
    kv = workloads.make_kv(kv_lens, seed + 1)
    plan = mla.mla_decode_plan(qo, kvp, mla.MLA_KV_BF16, max_splits=max_splits)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    mla.mla_decode_workspace_init(plan, ws)
    r = max(rows, 1)
    out = torch.empty((r, 16, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((r, 16), dtype=torch.float32, device=DEV)
    qd, kvd = q.to(DEV), kv.to(DEV) if kv.shape[0] else torch.zeros((1, 576), dtype=torch.bfloat16, device=DEV)
    res = []
    for _ in range(reps):
        mla.mla_decode_run_bf16(plan, qd, kvd, out, sm_scale=SM, logit_cap=cap, workspace=ws,
                                lse_out=lse)
        torch.cuda.synchronize()
        res.append((out.float().cpu().numpy()[:rows], lse.cpu().numpy()[:rows]))
    ref, ref_lse = oracle.mla_decode_bf16(q, kv, qo, kvp, SM, cap)
    return res, ref, ref_lse


CASES = [
    ([1], None, 0), ([16], None, 0), ([17], None, 0), ([33, 64, 65], None, 0),
    ([1000, 0, 4097], None, 0), ([1, 2, 3, 5, 8, 13, 21, 34, 55, 89], None, 0),
    ([1000, 333, 1, 64, 2048], None, -5), ([700, 31, 32, 33], [1, 2, 3, 4], 0),
]


@pytest.mark.parametrize("cap", [0.0, 2.0, 30.0])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{'-'.join(map(str, c[0]))[:30]}_s{c[2]}"
                         f"{'_rows' if c[1] else ''}")
def test_bf16_against_oracle(case, cap):
    kv_lens, q_lens, max_splits = case
    announce(f"bf16 {kv_lens} rows {q_lens} splits {max_splits} cap {cap}")
    res, ref, ref_lse = _run(kv_lens, q_lens, 900 + len(kv_lens), cap, max_splits)
    assert_close(res[0][0], ref, f"bf16 {kv_lens}")
    assert_lse_close(res[0][1], ref_lse, f"bf16 {kv_lens}")


def test_bf16_repeated_runs_identical():
    """Split sequences merged by their last workgroup, five runs in a row on
    one workspace: identical bits (the counters return to zero)."""
    announce("bf16 repeated")
    res, ref, _ = _run([3000, 129, 2048], None, 950, 0.0, -4, reps=5)
    for o, l in res[1:]:
        assert np.array_equal(o.view(np.uint32), res[0][0].view(np.uint32))
        assert np.array_equal(l.view(np.uint32), res[0][1].view(np.uint32))
    assert_close(res[0][0], ref, "bf16 repeated")


def test_bf16_bs64_kv1024_sampled():
    """A bigger batch: all rows against the oracle."""
    announce("bf16 bs64 kv1024")
    res, ref, ref_lse = _run([1024] * 64, None, 960)
    assert_close(res[0][0], ref, "bf16 bs64")
    assert_lse_close(res[0][1], ref_lse, "bf16 bs64")


def test_bf16_argument_errors():
    announce("bf16 argument errors")
    qo, kvp = workloads.indptrs([10])
    plan8 = mla.mla_decode_plan(qo, kvp)
    plan16 = mla.mla_decode_plan(qo, kvp, mla.MLA_KV_BF16)
    ws = torch.zeros(max(plan16.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    q = torch.zeros((1, 16, 576), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((10, 576), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((1, 16, 512), dtype=torch.bfloat16, device=DEV)
    for plan, cap in ((plan8, 0.0), (plan16, -1.0), (plan16, float("nan"))):
        with pytest.raises(mla.MLADecodeError) as e:
            mla.mla_decode_run_bf16(plan, q, kv, out, logit_cap=cap, workspace=ws)
        assert e.value.status == 1
    q8 = torch.empty((1, 16, 576), dtype=torch.uint8, device=DEV)
    qs = torch.ones(1, dtype=torch.float32, device=DEV)
    with pytest.raises(mla.MLADecodeError) as e:   # the FP8 entry points reject a bf16 plan
        mla.mla_decode_run(plan16, q, q8, qs, kv, out, kv_scale=qs, workspace=ws)
    assert e.value.status == 1
