"""GPU parity on seeded random shapes: ragged batches of up to 24 sequences
with 0 to 6000 cache rows and 1 to 4 query rows each, a random split policy,
both cache formats and both Q-scale modes. The three-launch path against
the CPU oracle element by element, and the fused path against the
three-launch one bit for bit (outputs, LSE, codes and scale). "mxfp4_cus8"
plans for 8 compute units, so that batches with query rows take the MXFP4
shared-row kernel."""
import numpy as np
import pytest

import workloads
from gpu_cases import DEV, GpuCache, GpuDecode, OracleSide, announce, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu


def _shape(seed):
    """The seed's batch: lengths skewed towards short sequences, some empty,
    some one row long, query rows 1-4, and a split policy."""
    rng = np.random.default_rng(seed)
    batch = int(rng.integers(1, 25))
    kv_lens = []
    for _ in range(batch):
        kind = rng.random()
        if kind < 0.1:
            kv_lens.append(0)
        elif kind < 0.2:
            kv_lens.append(int(rng.integers(1, 33)))
        else:
            kv_lens.append(int(rng.integers(1, 6001)))
    q_lens = [int(rng.integers(1, 5)) for _ in range(batch)] if rng.random() < 0.5 else None
    max_splits = int(rng.choice([0, 0, 1, 2, -2, -5]))
    return kv_lens, q_lens, max_splits


@pytest.mark.parametrize("q_mode", ["absmax", "static"])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "mxfp4_cus8"])
@pytest.mark.parametrize("seed", range(6))
def test_random_shape_against_oracle(seed, fmt, q_mode):
    cus = 8 if fmt == "mxfp4_cus8" else 0
    fmt = fmt.split("_")[0]
    kv_lens, q_lens, max_splits = _shape(1000 + seed)
    announce(f"random shape seed {seed} {fmt} {q_mode}: kv {kv_lens} q {q_lens} "
             f"splits {max_splits}")
    qo, kvp = workloads.indptrs(kv_lens, q_lens)
    rows = int(qo[-1])
    q = workloads.make_q(rows, 2000 + seed)
    kv = workloads.make_kv(kv_lens, 3000 + seed)
    cache = GpuCache(kv, fmt)
    dec = GpuDecode(qo, kvp, fmt, max_splits=max_splits, num_cus=cus)
    orc = OracleSide(q, kv, fmt, q_mode)
    qd = q.to(DEV)
    plain = dec.run(qd, cache, q_mode, orc.q_scale)
    assert np.array_equal(plain[2][:rows], orc.q8)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(plain[0][:rows], ref, f"random {seed}")
    assert_lse_close(plain[1][:rows], ref_lse, f"random {seed}")
    plain = [np.array(x, copy=True) for x in plain]
    fused = dec.run_fused(qd, cache, q_mode, orc.q_scale, init=True)
    for x, y, name in zip(plain, fused, ("out", "lse", "q8", "q_scale")):
        x = np.ascontiguousarray(x).reshape(-1)
        y = np.ascontiguousarray(y).reshape(-1)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"random {seed}: fused {name}"


_PAGE_SIZES = {"fp8": [1, 2, 4, 8, 16, 32, 64, 256], "mxfp4": [1, 2, 4, 8, 16, 32, 64, 512],
               "bf16": [1, 4, 16, 64]}


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "bf16"])
@pytest.mark.parametrize("seed", range(6))
def test_random_paged_shape_against_oracle(seed, fmt):
    """The same random batches on a paged cache with a random page size of
    the format's range: against the oracle on the gathered rows, and the
    fused path against the three-launch one bit for bit."""
    from test_gpu_paged import PagedCase

    kv_lens, q_lens, max_splits = _shape(1100 + seed)
    rng = np.random.default_rng(1200 + 10 * seed + ["fp8", "mxfp4", "bf16"].index(fmt))
    P = int(rng.choice(_PAGE_SIZES[fmt]))
    q_mode = "absmax" if seed % 2 == 0 else "static"
    announce(f"random paged seed {seed} {fmt} P{P} {q_mode}: kv {kv_lens} q {q_lens} "
             f"splits {max_splits}")
    c = PagedCase(kv_lens, q_lens, P, 1300 + seed, q_mode, max_splits=max_splits, fmt=fmt)
    ref, ref_lse, q8_ref, _, _, _ = c.oracle()
    plain = c.run(False)
    assert_close(plain[0], ref, f"random paged {seed}")
    assert_lse_close(plain[1], ref_lse, f"random paged {seed}")
    if fmt == "bf16":
        return  # one entry point, no Q codes
    assert np.array_equal(plain[2], q8_ref)
    plain = [np.array(x, copy=True) for x in plain]
    fused = c.run(True)
    for x, y, name in zip(plain, fused, ("out", "lse", "q8", "q_scale")):
        x = np.ascontiguousarray(x).reshape(-1)
        y = np.ascontiguousarray(y).reshape(-1)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"random paged {seed}: {name}"
