"""GPU parity of the logit soft-cap on the quantised paths: each scaled logit
s becomes cap * tanh(s / cap) before the softmax (the `logit_cap` argument
of the pages' FP8 decode calls, 0 on every page). The FP8 and MXFP4 caches,
the three-launch, fused, shared-row and paged kernels, through the C ABI
against the oracle's capped decode, element by element; a cap of 0 leaves
every output bit unchanged."""
import numpy as np
import pytest

import workloads
from gpu_cases import DEV, GpuCache, GpuDecode, OracleSide, announce, assert_close, assert_lse_close
from test_gpu_paged import PagedCase

pytestmark = pytest.mark.gpu

# the scaled logits of N(0,1) data are of order 1: 0.5 and 2 bend them hard,
# 30 barely
CAPS = [0.5, 2.0, 30.0]


@pytest.mark.parametrize("fused", [False, True], ids=["three_launch", "fused"])
@pytest.mark.parametrize("cap", CAPS)
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
# (rows_shared is planned for 8 compute units, so that MXFP4 takes its
# shared-row kernel too)
@pytest.mark.parametrize("case", [([700, 33, 1500, 0, 64], None, -3, 0),
                                  ([300, 129, 1024], [2, 4, 1], 0, 8),
                                  ([40, 2, 9, 600], [5, 2, 1, 6], 0, 0)],
                         ids=["ragged_split", "rows_shared", "rows_per_row"])
def test_cap_against_oracle(case, fmt, cap, fused):
    kv_lens, q_lens, max_splits, cus = case
    announce(f"cap {cap} {fmt} fused={fused} kv {kv_lens} q {q_lens}")
    qo, kvp = workloads.indptrs(kv_lens, q_lens)
    rows = int(qo[-1])
    q = workloads.make_q(rows, 500 + rows)
    kv = workloads.make_kv(kv_lens, 501 + rows)
    cache = GpuCache(kv, fmt)
    dec = GpuDecode(qo, kvp, fmt, max_splits=max_splits, num_cus=cus)
    orc = OracleSide(q, kv, fmt)
    ref, ref_lse = orc.decode(qo, kvp, logit_cap=cap)
    if fused:
        got, lse, q8, _ = dec.run_fused(q.to(DEV), cache, init=True, logit_cap=cap)
    else:
        got, lse, q8, _ = dec.run(q.to(DEV), cache, logit_cap=cap)
    assert np.array_equal(q8[:rows], orc.q8)
    assert_close(got[:rows], ref, f"cap {cap} {fmt}")
    assert_lse_close(lse[:rows], ref_lse, f"cap {cap} {fmt}")


@pytest.mark.parametrize("fused", [False, True], ids=["three_launch", "fused"])
@pytest.mark.parametrize("fmt,page_size", [("fp8", 16), ("fp8", 64), ("mxfp4", 2), ("mxfp4", 64)])
def test_cap_paged_against_oracle(fmt, page_size, fused):
    announce(f"cap 2.0 paged {fmt} P={page_size} fused={fused}")
    c = PagedCase([300, 1, 700, 64], None, page_size, 510, max_splits=-2, fmt=fmt)
    got, lse, _, _ = c.run(fused, logit_cap=2.0)
    ref, ref_lse, _, _, _, _ = c.oracle(logit_cap=2.0)
    assert_close(got, ref, f"paged P={page_size} cap 2")
    assert_lse_close(lse, ref_lse, f"paged P={page_size} cap 2")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_cap_zero_changes_nothing(fmt):
    """logit_cap = 0 is the uncapped decode bit for bit."""
    announce(f"cap 0 bit-identical {fmt}")
    kv_lens = [900, 17, 2048]
    qo, kvp = workloads.indptrs(kv_lens)
    q = workloads.make_q(3, 520)
    cache = GpuCache(workloads.make_kv(kv_lens, 521), fmt)
    dec = GpuDecode(qo, kvp, fmt, max_splits=-2)
    a = dec.run_fused(q.to(DEV), cache, init=True)
    a = [np.array(x, copy=True) for x in a]
    b = dec.run_fused(q.to(DEV), cache, logit_cap=0.0)
    for x, y in zip(a, b):
        assert np.array_equal(np.ascontiguousarray(x).view(np.uint8),
                              np.ascontiguousarray(y).view(np.uint8))
