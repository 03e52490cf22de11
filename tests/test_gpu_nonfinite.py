"""GPU parity for non-finite input. The reading (the oracle's, after torch's
amax in the pages' quantisers, kernelindex.com amd-mixed-mla 722089
`quantize_fp8` / 738050 `_quantize_fp8`): NaN propagates.

- Absmax scale: NaN if any element is NaN, +inf if one is infinite.
- Codes: x / scale clamped to +-448 and rounded; a NaN quotient is 0x7F.
- MXFP4: a block holding a NaN or an infinity gets the e8m0 NaN scale 0xFF
  and zero element bytes.
- Attention: a NaN input poisons exactly the outputs the oracle's fp64
  arithmetic makes NaN; every other output meets the usual tolerance.

Codes and scales are compared bit for bit (a NaN scale as NaN), outputs by
their NaN pattern and, where finite, within 1e-2 + 2e-2 |ref|.
"""
import math

import numpy as np
import pytest
import torch

import mla_latent_kv_bf16_amd as mla
import oracle
import workloads
from gpu_cases import DEV, GpuDecode, announce, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu

VALUES = [math.nan, math.inf, -math.inf]


def _planted(x: torch.Tensor, where: dict) -> torch.Tensor:
    x = x.clone()
    flat = x.view(-1)
    for i, v in where.items():
        flat[i] = v
    return x


def _same_scale(got, ref):
    got, ref = np.float32(got), np.float32(ref)
    if np.isnan(ref):
        assert np.isnan(got), f"scale {got}, NaN expected"
    else:
        assert got.view(np.uint32) == ref.view(np.uint32), f"scale {got} != {ref}"


def _gpu_quant(x_host, mode, static_scale):
    xd = x_host.contiguous().to(DEV)
    out = torch.empty(xd.shape, dtype=torch.uint8, device=DEV)
    sc = torch.empty(1, dtype=torch.float32, device=DEV)
    if mode == "static":
        sc.fill_(float(static_scale))
    ws = torch.empty(max(mla.mla_quant_fp8_workspace_size(xd.numel()), 256), dtype=torch.uint8,
                     device=DEV)
    mla.mla_quant_fp8(xd, out, sc, mla.MLA_Q_SCALE_STATIC if mode == "static"
                      else mla.MLA_Q_SCALE_ABSMAX, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), np.float32(sc.item())


@pytest.mark.parametrize("mode", ["absmax", "static"])
@pytest.mark.parametrize("value", VALUES, ids=["nan", "inf", "-inf"])
@pytest.mark.parametrize("n", [3 * 16 * 576, 3 * 16 * 576 - 5])
def test_quantiser_nonfinite(n, value, mode):
    """The standalone quantiser, on a size with and without a scalar tail; the
    planted values sit in the vector part and (n % 8 != 0) in the tail."""
    announce(f"quantiser non-finite n={n} {value} {mode}")
    x = workloads.randn_bf16((3 * 16 * 576,), 61)[:n].contiguous()
    x = _planted(x, {1000: value, n - 2: value})
    s_ref = oracle.fp8_static_scale() if mode == "static" else oracle.fp8_absmax_scale(x)
    codes, s = _gpu_quant(x, mode, s_ref)
    _same_scale(s, s_ref)
    assert np.array_equal(codes, oracle.fp8_quantize(x, s_ref))


def _decode_case(kv_lens, seed, q_where, mode, fused, fmt="fp8", max_splits=0):
    qo, kvp = workloads.indptrs(kv_lens)
    q = _planted(workloads.make_q(len(kv_lens), seed), q_where)
    kv = workloads.make_kv(kv_lens, seed + 1)
    dec = GpuDecode(qo, kvp, fmt, max_splits=max_splits)
    s_ref = oracle.fp8_static_scale() if mode == "static" else oracle.fp8_absmax_scale(q)
    q8_ref = oracle.fp8_quantize(q, s_ref)
    kvd = kv.to(DEV)
    if fmt == "fp8":
        k8 = torch.empty(kvd.shape, dtype=torch.uint8, device=DEV)
        ks = torch.empty(1, dtype=torch.float32, device=DEV)
        ws = torch.empty(max(mla.mla_quant_fp8_workspace_size(kvd.numel()), 256),
                         dtype=torch.uint8, device=DEV)
        mla.mla_quant_fp8(kvd, k8, ks, mla.MLA_Q_SCALE_ABSMAX, ws)
        cache = type("C", (), {"kv": k8, "kv_scale": ks, "block_scales": None})
        kscale = oracle.fp8_absmax_scale(kv)
        ref = oracle.mla_decode(q8_ref, s_ref, oracle.fp8_quantize(kv, kscale), kscale, qo, kvp,
                                workloads.SM_SCALE)
    else:
        rows = kvd.shape[0]
        pk = torch.empty((rows, 288), dtype=torch.uint8, device=DEV)
        bs = torch.empty((rows, 18), dtype=torch.uint8, device=DEV)
        mla.mla_encode_mxfp4(kvd, pk, bs)
        cache = type("C", (), {"kv": pk, "kv_scale": None, "block_scales": bs})
        opk, obs = oracle.mxfp4_encode(kv)
        ref = oracle.mla_decode(q8_ref, s_ref, opk, 0.0, qo, kvp, workloads.SM_SCALE,
                                kv_format=1, kv_scales=obs)
    run = dec.run_fused if fused else dec.run
    kw = {"init": True} if fused else {}
    got, lse, q8, qs = run(q.to(DEV), cache, mode, s_ref, **kw)
    b = len(kv_lens)
    return got[:b], lse[:b], q8[:b], qs, q8_ref, s_ref, ref


def _compare_with_nan(got, lse, ref, ref_lse, what):
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), f"{what}: NaN pattern of the output differs"
    lnan = np.isnan(ref_lse)
    assert np.array_equal(np.isnan(lse), lnan), f"{what}: NaN pattern of the LSE differs"
    if (~nan).any():
        assert_close(got[~nan], ref[~nan], what)
    if (~lnan).any():
        assert_lse_close(lse[~lnan], ref_lse[~lnan], what)


# 3 sequences: every FP8 workgroup reduces the absmax of Q itself; 9: a
# separate partial-maxima launch first. Forced splits exercise the merges.
ROW_CASES = [([700, 33, 1500], -3), ([64, 1, 300, 0, 2, 1024, 7, 31, 5], -2)]


@pytest.mark.parametrize("fused", [False, True], ids=["three_launch", "fused"])
@pytest.mark.parametrize("mode", ["absmax", "static"])
@pytest.mark.parametrize("value", VALUES, ids=["nan", "inf", "-inf"])
@pytest.mark.parametrize("case", ROW_CASES, ids=["3rows", "9rows"])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_decode_nonfinite_q(fmt, case, value, mode, fused):
    """A non-finite Q element (sequence 1, head 3, dim 200)."""
    kv_lens, splits = case
    announce(f"decode non-finite Q {fmt} {kv_lens} {value} {mode} fused={fused}")
    where = {(1 * 16 + 3) * 576 + 200: value}
    got, lse, q8, qs, q8_ref, s_ref, (ref, ref_lse) = _decode_case(
        kv_lens, 71, where, mode, fused, fmt, splits)
    _same_scale(qs, s_ref)
    assert np.array_equal(q8, q8_ref)
    _compare_with_nan(got, lse, ref, ref_lse, f"{fmt} {value} {mode} fused={fused}")
    live = np.array(kv_lens) > 0            # an empty sequence stays O = 0, LSE = -inf
    if mode == "absmax":
        assert np.isnan(ref[live]).all()    # every code NaN, or every product 0 * inf
        assert not ref[~live].any()
    elif math.isnan(value):
        assert np.isnan(ref[1, 3]).all() and np.isnan(ref).sum() == 512
    else:
        assert np.isfinite(ref).all()       # an infinity saturates to +-448


@pytest.mark.parametrize("value", VALUES, ids=["nan", "inf", "-inf"])
def test_mxfp4_encoder_nonfinite_block(value):
    announce(f"MXFP4 encoder non-finite {value}")
    kv = _planted(workloads.make_kv([40, 9], 81), {5 * 576 + 100: value, 45 * 576 + 575: value})
    kvd = kv.to(DEV)
    pk = torch.empty((49, 288), dtype=torch.uint8, device=DEV)
    bs = torch.empty((49, 18), dtype=torch.uint8, device=DEV)
    mla.mla_encode_mxfp4(kvd, pk, bs)
    torch.cuda.synchronize()
    opk, obs = oracle.mxfp4_encode(kv)
    assert obs[5, 3] == 0xFF and obs[45, 17] == 0xFF
    assert np.array_equal(pk.cpu().numpy(), opk) and np.array_equal(bs.cpu().numpy(), obs)


@pytest.mark.parametrize("fused", [False, True], ids=["three_launch", "fused"])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("dim", [100, 570], ids=["v_dim", "rope_dim"])
def test_decode_nan_in_cache(dim, fmt, fused):
    """A NaN in sequence 1's cache row 5: the FP8 cache's absmax scale turns
    every code NaN (all outputs NaN); the MXFP4 block scale poisons only that
    sequence."""
    kv_lens = [40, 300, 17]
    announce(f"decode NaN in cache {fmt} dim {dim} fused={fused}")
    qo, kvp = workloads.indptrs(kv_lens)
    q = workloads.make_q(3, 91)
    kv = _planted(workloads.make_kv(kv_lens, 92), {(40 + 5) * 576 + dim: math.nan})
    dec = GpuDecode(qo, kvp, fmt, max_splits=-2)
    s_ref = oracle.fp8_absmax_scale(q)
    q8_ref = oracle.fp8_quantize(q, s_ref)
    kvd = kv.to(DEV)
    if fmt == "fp8":
        k8 = torch.empty(kvd.shape, dtype=torch.uint8, device=DEV)
        ks = torch.empty(1, dtype=torch.float32, device=DEV)
        ws = torch.empty(max(mla.mla_quant_fp8_workspace_size(kvd.numel()), 256),
                         dtype=torch.uint8, device=DEV)
        mla.mla_quant_fp8(kvd, k8, ks, mla.MLA_Q_SCALE_ABSMAX, ws)
        cache = type("C", (), {"kv": k8, "kv_scale": ks, "block_scales": None})
        kscale = oracle.fp8_absmax_scale(kv)
        assert math.isnan(kscale)
        ref, ref_lse = oracle.mla_decode(q8_ref, s_ref, oracle.fp8_quantize(kv, kscale), kscale,
                                         qo, kvp, workloads.SM_SCALE)
    else:
        pk = torch.empty((kvd.shape[0], 288), dtype=torch.uint8, device=DEV)
        bs = torch.empty((kvd.shape[0], 18), dtype=torch.uint8, device=DEV)
        mla.mla_encode_mxfp4(kvd, pk, bs)
        cache = type("C", (), {"kv": pk, "kv_scale": None, "block_scales": bs})
        opk, obs = oracle.mxfp4_encode(kv)
        ref, ref_lse = oracle.mla_decode(q8_ref, s_ref, opk, 0.0, qo, kvp, workloads.SM_SCALE,
                                         kv_format=1, kv_scales=obs)
        assert np.isnan(ref[1]).all() and np.isfinite(ref[[0, 2]]).all()
    run = dec.run_fused if fused else dec.run
    kw = {"init": True} if fused else {}
    got, lse, _, _ = run(q.to(DEV), cache, "absmax", s_ref, **kw)
    _compare_with_nan(got[:3], lse[:3], ref, ref_lse, f"NaN cache {fmt} dim {dim}")


@pytest.mark.parametrize("fused", [False, True], ids=["three_launch", "fused"])
def test_mxfp4_shared_rows_nan_in_cache(fused):
    """The MXFP4 shared-row kernel (planned for 8 compute units) with a NaN in
    sequence 1's cache row 5, which all three of its query rows see: those
    rows are NaN, the other sequences' rows are finite."""
    kv_lens, q_lens = [40, 300, 17], [2, 3, 1]
    announce(f"MXFP4 shared rows, NaN in cache, fused={fused}")
    qo, kvp = workloads.indptrs(kv_lens, q_lens)
    rows = int(qo[-1])
    q = workloads.make_q(rows, 93)
    kv = _planted(workloads.make_kv(kv_lens, 94), {(40 + 5) * 576 + 100: math.nan})
    dec = GpuDecode(qo, kvp, "mxfp4", max_splits=-2, num_cus=8)
    s_ref = oracle.fp8_absmax_scale(q)
    q8_ref = oracle.fp8_quantize(q, s_ref)
    kvd = kv.to(DEV)
    pk = torch.empty((kvd.shape[0], 288), dtype=torch.uint8, device=DEV)
    bs = torch.empty((kvd.shape[0], 18), dtype=torch.uint8, device=DEV)
    mla.mla_encode_mxfp4(kvd, pk, bs)
    cache = type("C", (), {"kv": pk, "kv_scale": None, "block_scales": bs})
    opk, obs = oracle.mxfp4_encode(kv)
    ref, ref_lse = oracle.mla_decode(q8_ref, s_ref, opk, 0.0, qo, kvp, workloads.SM_SCALE,
                                     kv_format=1, kv_scales=obs)
    assert np.isnan(ref[2:5]).all() and np.isfinite(ref[[0, 1, 5]]).all()
    run = dec.run_fused if fused else dec.run
    kw = {"init": True} if fused else {}
    got, lse, _, _ = run(q.to(DEV), cache, "absmax", s_ref, **kw)
    _compare_with_nan(got[:rows], lse[:rows], ref, ref_lse, "NaN cache, MXFP4 shared rows")
