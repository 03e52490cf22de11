"""The Q quantisers divide by the per-tensor scale through a reciprocal and
one fused-multiply-add correction when the scale lies in [2^-100, 2^100],
and by plain IEEE division outside it. Both sides of both ends of that range,
through every kernel that converts Q: the standalone quantiser over every
bf16 value, and the fused FP8, MXFP4 and shared-row kernels (Q codes equal to
the oracle's bit for bit, outputs equal to the three-launch path bit for bit
and to the oracle within the tolerance)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_cases import LSE_TOL, DEV, GpuCache, GpuDecode, announce, assert_close
from test_gpu_quant import _all_bf16, _gpu_quant

pytestmark = pytest.mark.gpu

EDGE_SCALES = [2.0 ** -120, 2.0 ** -101, 2.0 ** -100, 2.0 ** 100, 2.0 ** 101, 2.0 ** 120]


@pytest.mark.parametrize("scale", EDGE_SCALES + [1e-40, 3.0e38],
                         ids=lambda s: f"{s:.3g}")
def test_quantiser_every_bf16_value_at_range_edges(scale):
    announce(f"exhaustive bf16 quant at edge scale {scale:.3g}")
    x = _all_bf16()
    s = np.float32(scale)
    codes, _ = _gpu_quant(x, "static", s)
    assert np.array_equal(codes, oracle.fp8_quantize(x, s))


def _scaled_q(rows, seed, scale):
    # N(0,1) times 16 scale (a power of two, so exact in bf16): codes spread
    # over e4m3's range without saturating
    q = workloads.make_q(rows, seed).float() * np.float32(16.0 * scale)
    return q.to(torch.bfloat16)


@pytest.mark.parametrize("kind", ["fp8", "mxfp4", "fp8_rows"])
@pytest.mark.parametrize("scale", EDGE_SCALES, ids=lambda s: f"{s:.3g}")
def test_fused_kernels_at_range_edges(scale, kind):
    fmt = "mxfp4" if kind == "mxfp4" else "fp8"
    kv_lens = [300, 77, 1000]
    q_lens = [2, 2, 2] if kind == "fp8_rows" else None
    announce(f"fused {kind} static scale {scale:.3g}")
    qo, kvp = workloads.indptrs(kv_lens, q_lens)
    rows = int(qo[-1])
    q = _scaled_q(rows, 900, scale)
    kv = workloads.make_kv(kv_lens, 901)
    cache = GpuCache(kv, fmt)
    dec = GpuDecode(qo, kvp, fmt, max_splits=-3)
    qd = q.to(DEV)
    s = np.float32(scale)
    plain = dec.run(qd, cache, "static", s)
    ref_codes = oracle.fp8_quantize(q, s)
    assert np.array_equal(plain[2][:rows], ref_codes)
    fused = dec.run_fused(qd, cache, "static", s, init=True)
    for x, y, name in zip(plain, fused, ("out", "lse", "q8")):
        assert np.array_equal(np.ascontiguousarray(x).view(np.uint8),
                              np.ascontiguousarray(y).view(np.uint8)), f"fused {name} differs"
    if fmt == "fp8":
        kv_scale = oracle.fp8_absmax_scale(kv)
        kv_codes, kv_blocks = oracle.fp8_quantize(kv, kv_scale), None
    else:
        kv_scale = 0.0
        kv_codes, kv_blocks = oracle.mxfp4_encode(kv)
    ref, ref_lse = oracle.mla_decode(ref_codes, s, kv_codes, kv_scale, qo, kvp,
                                     workloads.SM_SCALE, kv_format=0 if fmt == "fp8" else 1,
                                     kv_scales=kv_blocks)
    assert_close(plain[0][:rows], ref, f"{kind} scale {scale:.3g}")
    # At scales near 2^100 the logits are of order 1e31, where fp32 values are
    # spaced about 1e25 apart: the LSE bar gets a relative term (a few fp32
    # roundings of the logit scale and of the log-sum) besides the usual one.
    got = plain[1][:rows].astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.all(np.abs(got[fin] - ref_lse[fin]) <= LSE_TOL + 3e-5 * np.abs(ref_lse[fin]))
