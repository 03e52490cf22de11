"""GPU parity with several query rows per sequence (multi-token prediction or
speculative rows): row i of a sequence with R rows attends causally to the
first kv_len - (R - 1 - i) cache rows; with 1-4 rows in every sequence the
rows share each cache tile (the FP8 and MXFP4 shared-row kernels). Both cache formats, both Q-scale modes,
the three-launch and the fused path, against the CPU oracle element by
element; the fused path also against the three-launch one bit for bit."""
import numpy as np
import pytest

import workloads
from gpu_cases import DEV, GpuCache, GpuDecode, OracleSide, announce, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu

CASES = [
    ([40, 3, 1, 0, 65, 9], [4, 4, 2, 3, 1, 3], 0),
    ([1000, 5000, 257], [2, 4, 3], 0),
    ([1000, 333, 2048], [2, 3, 4], -3),
    ([700, 31, 32, 33], [1, 2, 3, 4], 0),
    ([300, 40, 2], [5, 2, 6], 0),   # more than 4 rows: every row on its own range
]


def _same(a, b, what):
    for x, y, name in zip(a, b, ("out", "lse", "q8", "q_scale")):
        x = np.ascontiguousarray(x).reshape(-1)
        y = np.ascontiguousarray(y).reshape(-1)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{what}: {name} differs"


# (MXFP4 shares tiles between rows only when the per-row schedule would need
# more than one round of workgroups: "mxfp4_shared" plans for 8 compute
# units, which these batches exceed)
@pytest.mark.parametrize("q_mode", ["absmax", "static"])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "mxfp4_shared"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{'-'.join(map(str, c[1]))}_s{c[2]}")
def test_query_rows_against_oracle(case, fmt, q_mode):
    kv_lens, q_lens, max_splits = case
    announce(f"rows {fmt} {q_mode} kv {kv_lens} q {q_lens} splits {max_splits}")
    cus = 8 if fmt == "mxfp4_shared" else 0
    fmt = fmt.split("_")[0]
    qo, kvp = workloads.indptrs(kv_lens, q_lens)
    rows = int(qo[-1])
    q = workloads.make_q(rows, 400 + rows)
    kv = workloads.make_kv(kv_lens, 401 + rows)
    cache = GpuCache(kv, fmt)
    dec = GpuDecode(qo, kvp, fmt, max_splits=max_splits, num_cus=cus)
    assert dec.rows == rows
    orc = OracleSide(q, kv, fmt, q_mode)
    qd = q.to(DEV)
    plain = dec.run(qd, cache, q_mode, orc.q_scale)
    assert np.array_equal(plain[2][:rows], orc.q8)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(plain[0][:rows], ref, f"rows {q_lens}")
    assert_lse_close(plain[1][:rows], ref_lse, f"rows {q_lens}")
    fused = dec.run_fused(qd, cache, q_mode, orc.q_scale, init=True)
    _same(plain, fused, f"rows {q_lens} fused")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("R", [2, 3, 4])
def test_query_rows_bs64_kv2048(R, fmt):
    """A bigger batch at uniform R: every row against the oracle."""
    bs, n = 64, 2048
    announce(f"rows {fmt} bs{bs} kv{n} R{R}")
    qo, kvp = workloads.indptrs([n] * bs, [R] * bs)
    rows = bs * R
    q = workloads.make_q(rows, 450 + R)
    kv = workloads.make_kv([n] * bs, 451 + R)
    cache = GpuCache(kv, fmt)
    # planned for 64 compute units: both formats take the shared-row
    # schedule, one item per sequence
    dec = GpuDecode(qo, kvp, fmt, num_cus=64)
    assert dec.plan.num_items == bs
    orc = OracleSide(q, kv, fmt, "absmax")
    got = dec.run_fused(q.to(DEV), cache, "absmax", init=True)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(got[0][:rows], ref, f"bs{bs} R{R}")
    assert_lse_close(got[1][:rows], ref_lse, f"bs{bs} R{R}")


def test_mxfp4_rows_schedule_choice():
    """MXFP4 rows share tiles only when per-row items would take more than one
    round of workgroups (256 compute units here)."""
    announce("mxfp4 rows schedule choice")
    qo, kvp = workloads.indptrs([2048] * 64, [2] * 64)      # 128 rows: one round per row
    assert GpuDecode(qo, kvp, "mxfp4", num_cus=256).plan.num_items >= 128
    qo, kvp = workloads.indptrs([1024] * 256, [2] * 256)    # 512 rows: shared, 256 items
    assert GpuDecode(qo, kvp, "mxfp4", num_cus=256).plan.num_items == 256
    assert GpuDecode(qo, kvp, "fp8", num_cus=256).plan.num_items == 256
