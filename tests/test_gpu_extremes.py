"""GPU parity at the size limits of the decode: one very long sequence
(split across most of the chip, and at the 64-split cap), thousands of
short ragged sequences, and long sequences with several query rows. Each
case runs the three-launch path against the CPU oracle element by element
and the fused path against the three-launch one bit for bit."""
import numpy as np
import pytest

import workloads
from gpu_cases import DEV, GpuCache, GpuDecode, OracleSide, announce, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu

SPLIT_CAP = 64  # the plan's cap on one query row's splits (ranges below 64 x 2^22 rows)


def _same(a, b, what):
    for x, y, name in zip(a, b, ("out", "lse", "q8", "q_scale")):
        x = np.ascontiguousarray(x).reshape(-1)
        y = np.ascontiguousarray(y).reshape(-1)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{what}: {name} differs"


def _check(kv_lens, fmt, seed, q_lens=None, max_splits=0, q_mode="absmax"):
    qo, kvp = workloads.indptrs(kv_lens, q_lens)
    rows = int(qo[-1])
    q = workloads.make_q(rows, seed)
    kv = workloads.make_kv(kv_lens, seed + 1)
    cache = GpuCache(kv, fmt)
    dec = GpuDecode(qo, kvp, fmt, max_splits=max_splits)
    orc = OracleSide(q, kv, fmt, q_mode)
    qd = q.to(DEV)
    plain = dec.run(qd, cache, q_mode, orc.q_scale)
    assert np.array_equal(plain[2][:rows], orc.q8)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(plain[0][:rows], ref, f"{fmt} {len(kv_lens)} seqs")
    assert_lse_close(plain[1][:rows], ref_lse, f"{fmt} {len(kv_lens)} seqs")
    fused = dec.run_fused(qd, cache, q_mode, orc.q_scale, init=True)
    _same(plain, fused, f"{fmt} {len(kv_lens)} seqs fused")
    return dec


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_one_long_sequence_policy_splits(fmt):
    """262,144 cache rows in one sequence: the policy would spread it over
    all CUs and stops at the split cap."""
    announce(f"extreme {fmt} one sequence of 262144 rows, policy splits")
    dec = _check([262144], fmt, 610)
    assert dec.plan.num_slots == SPLIT_CAP


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_split_cap(fmt):
    """Asking for more splits than the cap: the plan clips to it and the result
    is still right."""
    announce(f"extreme {fmt} 131072 rows, 2000 splits asked")
    dec = _check([131072], fmt, 620, max_splits=-2000)
    assert dec.plan.num_slots == SPLIT_CAP


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_thousands_of_short_sequences(fmt):
    """4096 ragged sequences of 0..64 rows (a few hundred of them empty)."""
    rng = np.random.default_rng(630)
    kv_lens = [int(x) for x in rng.integers(0, 65, size=4096)]
    announce(f"extreme {fmt} 4096 short sequences")
    _check(kv_lens, fmt, 631)


@pytest.mark.parametrize("q_len", [2, 4])
def test_long_sequences_with_query_rows(q_len):
    """Two 65,536-row sequences with several causal query rows each (FP8:
    the rows share every cache tile)."""
    announce(f"extreme fp8 2 x 65536 rows, {q_len} query rows")
    _check([65536, 65536], "fp8", 640 + q_len, q_lens=[q_len, q_len])
