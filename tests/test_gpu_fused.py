"""GPU tests of the single-launch decode (mla_decode_run_fused): Q quantised
inside the attention kernel and split sequences merged by their last
workgroup. Its outputs must equal those of the three-launch mla_decode_run
bit for bit (that path is checked against the oracle in test_gpu_decode.py),
and small cases are also compared with the oracle directly."""
import numpy as np
import pytest
import torch

import mla_latent_kv_bf16_amd as mla
import workloads
from gpu_cases import (DEV, GpuCache, GpuDecode, OracleSide, announce, assert_close,
                       assert_lse_close)

pytestmark = pytest.mark.gpu


def _assert_same(a, b, what):
    """Outputs of the two paths: identical bits (out as float32 of bf16, lse, q8, q_scale)."""
    for x, y, name in zip(a, b, ("out", "lse", "q8", "q_scale")):
        x = np.ascontiguousarray(x).reshape(-1)
        y = np.ascontiguousarray(y).reshape(-1)
        assert x.shape == y.shape, f"{what}: {name} shape"
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{what}: {name} differs"


CASES = [
    ([1], 0), ([33], 0), ([127, 128, 129], 0), ([1000, 0, 4097], 0), ([0], 0), ([0, 0, 5], 0),
    ([1, 2, 3, 5, 8, 13, 21, 34, 55, 89], 0), ([257, 513, 1025, 96, 97, 95], 0),
    ([1000, 333, 1, 64, 2048], -3), ([1000, 333, 1, 64, 2048], -31), ([3000, 5], 7),
    # 8 and 9 rows
    ([64, 1, 300, 0, 2, 1024, 7, 31], 0), ([64, 1, 300, 0, 2, 1024, 7, 31, 5], 0),
    # 4 and 5 rows: the largest Q whose absmax each FP8 workgroup reduces itself, and the next
    ([5, 900, 0, 2048], -2), ([5, 900, 0, 2048, 77], -2),
]


@pytest.mark.parametrize("q_mode", ["static", "absmax"])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{'-'.join(map(str, c[0]))[:30]}_s{c[1]}")
def test_fused_equals_plain_and_oracle(case, fmt, q_mode):
    kv_lens, max_splits = case
    announce(f"fused {fmt} {q_mode} {kv_lens} splits {max_splits}")
    qo, kvp = workloads.indptrs(kv_lens)
    seed = 300 + len(kv_lens)
    q = workloads.make_q(len(kv_lens), seed)
    kv = workloads.make_kv(kv_lens, seed + 1)
    cache = GpuCache(kv, fmt)
    dec = GpuDecode(qo, kvp, fmt, max_splits=max_splits)
    orc = OracleSide(q, kv, fmt, q_mode)
    qd = q.to(DEV)
    plain = dec.run(qd, cache, q_mode, orc.q_scale)
    dec.out.fill_(float("nan"))
    dec.lse.fill_(float("nan"))
    dec.q8.fill_(0x55)
    fused = dec.run_fused(qd, cache, q_mode, orc.q_scale, init=True)
    _assert_same(plain, fused, f"{fmt} {q_mode} {kv_lens}")
    nb = len(kv_lens)
    assert np.array_equal(fused[2][:nb], orc.q8)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(fused[0][:nb], ref, f"fused {kv_lens}")
    assert_lse_close(fused[1][:nb], ref_lse, f"fused {kv_lens}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_fused_counters_reset_between_runs(fmt):
    """Five fused runs in a row on one workspace, each with new Q values,
    each equal to the plain path: the per-sequence counters return to zero."""
    kv_lens = [1500, 4000, 129, 0, 640]
    announce(f"fused repeated {fmt} {kv_lens}")
    qo, kvp = workloads.indptrs(kv_lens)
    kv = workloads.make_kv(kv_lens, 91)
    cache = GpuCache(kv, fmt)
    dec = GpuDecode(qo, kvp, fmt, max_splits=-4)
    dec.ws.fill_(0xFF)  # garbage everywhere, then the init call
    mla.mla_decode_workspace_init(dec.plan, dec.ws)
    for r in range(5):
        qd = workloads.make_q(len(kv_lens), 500 + r).to(DEV)
        plain = dec.run(qd, cache, "absmax")
        fused = dec.run_fused(qd, cache, "absmax")
        _assert_same(plain, fused, f"run {r}")


@pytest.mark.parametrize("name", ["bs4_kv1024_fp8", "bs32_kv1024_fp8", "bs64_kv8192_fp8",
                                  "bs256_kv8192_fp8", "bs256_kv1024_mxfp4"])
@pytest.mark.parametrize("q_mode", ["static", "absmax"])
def test_fused_workloads_equal_plain(name, q_mode):
    """Every benchmark workload at full size: fused == plain bit for bit."""
    w = workloads.BY_NAME[name]
    announce(f"fused workload {name} {q_mode}")
    qo, kvp = workloads.indptrs([w.kv_len] * w.batch)
    q = workloads.make_q(w.batch, w.seed_q)
    kv = workloads.make_kv([w.kv_len] * w.batch, w.seed_kv)
    cache = GpuCache(kv, w.kv_format)
    del kv
    dec = GpuDecode(qo, kvp, w.kv_format)
    qd = q.to(DEV)
    static = 6.0 / 448.0
    plain = dec.run(qd, cache, q_mode, static)
    fused = dec.run_fused(qd, cache, q_mode, static, init=True)
    _assert_same(plain, fused, name)
    fused2 = dec.run_fused(qd, cache, q_mode, static)
    _assert_same(plain, fused2, name + " second run")


def test_fused_argument_errors():
    announce("fused argument errors")
    kv_lens = [0, 0]
    qo, kvp = workloads.indptrs(kv_lens)
    dec = GpuDecode(qo, kvp, "fp8")
    q = torch.zeros((2, 16, 576), dtype=torch.bfloat16, device=DEV)
    dec.q_scale.fill_(0.01)
    # the FP8 cache scale is read by every fused workgroup, even with no rows
    with pytest.raises(mla.MLADecodeError) as e:
        mla.mla_decode_run_fused(dec.plan, q, dec.q8, dec.q_scale, None, dec.out,
                                 kv_scale=None, q_scale_mode=mla.MLA_Q_SCALE_STATIC,
                                 workspace=dec.ws)
    assert e.value.status == 1
    with pytest.raises(mla.MLADecodeError) as e:
        mla.mla_decode_workspace_init(dec.plan, dec.ws[:0] if dec.plan.workspace_bytes else None)
    assert e.value.status in (1, 4)
    # all-empty batch: O = 0, LSE = -inf, Q codes written
    ks = torch.ones(1, dtype=torch.float32, device=DEV)
    mla.mla_decode_workspace_init(dec.plan, dec.ws)
    mla.mla_decode_run_fused(dec.plan, q, dec.q8, dec.q_scale, None, dec.out, kv_scale=ks,
                             q_scale_mode=mla.MLA_Q_SCALE_STATIC, workspace=dec.ws,
                             lse_out=dec.lse)
    torch.cuda.synchronize()
    assert torch.all(dec.out[:2] == 0)
    assert torch.all(torch.isneginf(dec.lse[:2]))
    assert torch.all(dec.q8[:2] == 0)


@pytest.mark.parametrize("where", ["first", "last", "middle"])
@pytest.mark.parametrize("rows", [1, 3, 4, 5])
def test_fused_absmax_sees_all_of_q(rows, where):
    """The absmax scale covers every row of Q, also when each workgroup
    reduces it itself (FP8, at most 4 rows): one outlier in the first, the
    last or a middle element of Q sets the scale and every code."""
    announce(f"fused fp8 absmax outlier {where} of {rows} rows")
    kv_lens = [700, 65, 1500, 33, 260][:rows]
    qo, kvp = workloads.indptrs(kv_lens)
    q = workloads.make_q(rows, 950 + rows).float()
    flat = q.view(-1)
    idx = {"first": 0, "last": flat.numel() - 1, "middle": flat.numel() // 2 + 123}[where]
    flat[idx] = -37.5
    q = q.to(torch.bfloat16)
    kv = workloads.make_kv(kv_lens, 960 + rows)
    cache = GpuCache(kv, "fp8")
    dec = GpuDecode(qo, kvp, "fp8", max_splits=-2)
    orc = OracleSide(q, kv, "fp8", "absmax")
    assert orc.q_scale == np.float32(37.5) / np.float32(448.0)
    qd = q.to(DEV)
    plain = dec.run(qd, cache, "absmax")
    fused = dec.run_fused(qd, cache, "absmax", init=True)
    _assert_same(plain, fused, f"outlier {where} {rows} rows")
    assert fused[3].view(np.uint32) == np.float32(orc.q_scale).view(np.uint32)
    assert np.array_equal(fused[2][:rows], orc.q8)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(fused[0][:rows], ref, f"outlier {where}")
    assert_lse_close(fused[1][:rows], ref_lse, f"outlier {where}")
