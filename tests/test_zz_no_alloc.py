"""The entry point that allocates nothing (mla_decode_run_fused_noalloc),
called through the C ABI, against mla_decode_run_fused with its own
workspace on the same inputs: outputs identical bit for bit, over several
calls in a row whose plans differ in size (the library's fixed scratch
keeps the last call's contents), and a plan beyond the scratch's limits
rejected before any launch."""
import numpy as np
import pytest
import torch

import mla_latent_kv_bf16_amd as mla
import workloads
from gpu_cases import DEV, GpuCache, announce

pytestmark = pytest.mark.gpu


class _Case:
    def __init__(self, kv_lens, seed, fmt, max_splits=0, q_lens=None, num_cus=0):
        qo, kvp = workloads.indptrs(kv_lens, q_lens)
        self.rows = int(qo[-1])
        self.cache = GpuCache(workloads.make_kv(kv_lens, seed), fmt)
        self.plan = mla.mla_decode_plan(qo, kvp, 0 if fmt == "fp8" else 1, max_splits=max_splits,
                                        num_cus=num_cus)
        self.ws = torch.zeros(max(self.plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
        mla.mla_decode_workspace_init(self.plan, self.ws)
        self.q = workloads.make_q(self.rows, seed + 1).to(DEV)

    def _buffers(self):
        return (torch.full((self.rows, 16, 576), 0xAA, dtype=torch.uint8, device=DEV),
                torch.full((1,), 0.01, dtype=torch.float32, device=DEV),
                torch.full((self.rows, 16, 512), float("nan"), dtype=torch.bfloat16, device=DEV),
                torch.full((self.rows, 16), float("nan"), dtype=torch.float32, device=DEV))

    def run(self, noalloc: bool, mode: str, cap: float = 0.0):
        q8, qs, out, lse = self._buffers()
        qs.fill_(6.0 / 448.0)
        kw = dict(kv_scale=self.cache.kv_scale, kv_block_scales=self.cache.block_scales,
                  q_scale_mode=(mla.MLA_Q_SCALE_STATIC if mode == "static"
                                else mla.MLA_Q_SCALE_ABSMAX), logit_cap=cap, lse_out=lse)
        if noalloc:
            mla.mla_decode_run_fused_noalloc(self.plan, self.q, q8, qs, self.cache.kv, out, **kw)
        else:
            mla.mla_decode_run_fused(self.plan, self.q, q8, qs, self.cache.kv, out,
                                     workspace=self.ws, **kw)
        torch.cuda.synchronize()
        return [t.contiguous().view(torch.uint8).cpu().numpy().copy() for t in (out, lse, q8, qs)]


def _assert_same(got, ref, what):
    for x, y, name in zip(got, ref, ("out", "lse", "q8", "q_scale")):
        assert np.array_equal(x, y), f"{what}: {name} differs from mla_decode_run_fused"


def test_noalloc_equals_fused_on_calls_in_a_row():
    """A split FP8 plan (its partials and counters in the scratch), then
    smaller plans: MXFP4 with splits, 3 rows (absmax reduced in the kernel),
    one row; then the first plan again, and the MXFP4 plan with a logit
    soft-cap; then sequences with several query rows sharing each tile
    (MXFP4 planned for 8 compute units, and FP8), split."""
    cases = [
        ("fp8 6 rows, 8 splits", _Case([3000, 17, 4096, 900, 2500, 64], 900, "fp8", -8), "absmax"),
        ("mxfp4 2 rows, 3 splits", _Case([700, 33], 910, "mxfp4", -3), "static"),
        ("fp8 3 rows, 4 splits", _Case([1500, 0, 260], 920, "fp8", -4), "absmax"),
        ("fp8 1 row, unsplit", _Case([77], 930, "fp8"), "static"),
        ("mxfp4 shared rows 2-4-3, 2 splits",
         _Case([900, 40, 1200], 940, "mxfp4", -2, q_lens=[2, 4, 3], num_cus=8), "absmax"),
        ("fp8 shared rows 3-1, 3 splits",
         _Case([2000, 300], 950, "fp8", -3, q_lens=[3, 1]), "static"),
    ]
    order = [(0, 0.0), (1, 0.0), (2, 0.0), (3, 0.0), (0, 0.0), (3, 0.0), (1, 2.0), (4, 0.0),
             (5, 0.0), (4, 0.0)]
    for i, cap in order:
        what, case, mode = cases[i]
        announce(f"no-alloc call: {what} ({mode}, cap {cap})")
        assert case.plan.num_slots <= 500
        ref = case.run(False, mode, cap)
        got = case.run(True, mode, cap)
        _assert_same(got, ref, what)


def test_noalloc_rejects_a_plan_beyond_its_scratch():
    announce("no-alloc: plan with 1024 partial slots is rejected")
    case = _Case([4096] * 16, 940, "fp8", -64)
    assert case.plan.num_slots == 1024
    q8, qs, out, lse = case._buffers()
    with pytest.raises(mla.MLADecodeError) as e:
        mla.mla_decode_run_fused_noalloc(case.plan, case.q, q8, qs, case.cache.kv, out,
                                         kv_scale=case.cache.kv_scale, lse_out=lse)
    assert e.value.status == 4  # MLA_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and (q8 == 0xAA).all()  # nothing was launched
    # a plan within the limits still runs afterwards
    small = _Case([300, 5], 950, "fp8", -2)
    _assert_same(small.run(True, "absmax"), small.run(False, "absmax"), "after a rejected call")
