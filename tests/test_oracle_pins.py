"""Pins for the CPU oracle: each test ties it to something other than itself.

- FP8 E4M3FN codec and the per-tensor quantiser: torch's float8_e4m3fn cast
  (a library routine) and torch fp32 arithmetic, over every bf16 input, every
  rounding boundary and a large random sample of fp32 inputs.
- e2m1 / e8m0: closed forms and a brute-force nearest-code search.
- MXFP4 blocks: hand-worked blocks with known codes.
- Attention: torch's scaled_dot_product_attention in fp64 (a library routine)
  on the dequantised inputs, torch.logsumexp for the LSE, and closed-form
  special cases (kv_len 1, identical keys, empty range), plus the split-merge
  identity.
The constants are checked against tests/golden/page_constants.json.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")
SM = 1.0 / 24.0


def _torch_e4m3fn(x_f32: np.ndarray) -> np.ndarray:
    """torch's fp32 -> float8_e4m3fn cast after clamping to +-448."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# --------------------------------------------------------------------------
# constants from the pages
# --------------------------------------------------------------------------

def test_golden_constants():
    g = json.load(open(GOLDEN))
    assert g["num_heads"]["value"] == workloads.HEADS == oracle.HEADS
    assert g["qk_head_dim"]["value"] == workloads.DQK == oracle.DQK
    assert g["kv_lora_rank"]["value"] + g["qk_rope_head_dim"]["value"] == workloads.DQK
    assert g["v_head_dim"]["value"] == workloads.DV == oracle.DV
    assert g["sm_scale"]["value"] == pytest.approx(workloads.SM_SCALE, rel=0, abs=1e-17)
    assert g["sm_scale"]["value"] == 1.0 / math.sqrt(576)
    assert g["sm_scale_log2"]["value"] == pytest.approx(workloads.SM_SCALE * math.log2(math.e),
                                                        rel=1e-12)
    assert g["mxfp4_block"]["value"] == oracle.MX_BLOCK
    # one 576-d row encodes to 288 packed bytes and 18 e8m0 scales
    p, s = oracle.mxfp4_encode(np.zeros((3, 576), dtype=np.uint16))
    assert p.shape == (3, g["mxfp4_packed_bytes_per_row"]["value"])
    assert s.shape == (3, g["mxfp4_blocks_per_row"]["value"])
    # the static scale maps +-6 sigma onto the format's max, for both flavours
    assert g["static_q_scale_page_fnuz"]["value"] == pytest.approx(6.0 / 240.0)
    assert float(oracle.fp8_static_scale()) == np.float32(6.0) / np.float32(448.0)
    assert g["static_q_scale_ocp"]["value"] == pytest.approx(float(oracle.fp8_static_scale()),
                                                            rel=1e-7)
    # the page's clip-rate figure is the two-sided N(0,1) tail beyond 6 sigma
    assert math.erfc(6 / math.sqrt(2)) == pytest.approx(g["static_scale_clip_rate"]["value"],
                                                        rel=0.05)
    # benchmark shapes used by the workloads are among the pages' shapes
    shapes = {tuple(x) for x in g["benchmark_shapes"]["value"]}
    for w in workloads.WORKLOADS:
        assert (w.batch, w.kv_len) in shapes


# --------------------------------------------------------------------------
# FP8 E4M3FN
# --------------------------------------------------------------------------

def test_e4m3fn_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3fn_decode(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3fn_decode_closed_forms():
    assert oracle.e4m3fn_decode(0x7E) == 448.0
    assert oracle.e4m3fn_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3fn_decode(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3fn_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3fn_decode(0x38) == 1.0
    assert oracle.e4m3fn_decode(0xB8) == -1.0
    assert oracle.e4m3fn_decode(0x80) == 0.0 and math.copysign(1, oracle.e4m3fn_decode(0x80)) < 0


def test_e4m3fn_roundtrip_every_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3fn_encode(oracle.e4m3fn_decode(c)) == c


def test_e4m3fn_encode_spot_values():
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 2.0 ** -10 * (1 + 1e-4), 448.0, 464.0, 470.0,
                  1e30, -1e-20, -0.0, 0.0, float("inf"), -float("inf")], dtype=np.float32)
    got = oracle.e4m3fn_encode_array(x)
    assert got.tolist() == [0x38, 0x3A, 0x00, 0x01, 0x7E, 0x7E, 0x7E, 0x7E, 0x80, 0x80, 0x00,
                            0x7E, 0xFE]
    assert oracle.e4m3fn_encode(float("nan")) == 0x7F


def test_e4m3fn_encode_every_bf16_vs_torch():
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[~np.isnan(x)]
    assert np.array_equal(oracle.e4m3fn_encode_array(x), _torch_e4m3fn(x))


def test_e4m3fn_encode_rounding_boundaries_vs_torch():
    vals = np.array(sorted({oracle.e4m3fn_decode(c) for c in range(0, 0x7F)}), dtype=np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0
    pts = np.concatenate([vals, mids]).astype(np.float32)
    near = []
    for k in (-3, -2, -1, 0, 1, 2, 3):
        near.append((pts.view(np.int32) + k).view(np.float32))
    x = np.concatenate(near)
    x = x[np.isfinite(x) & (x >= 0)]
    x = np.concatenate([x, -x])
    assert np.array_equal(oracle.e4m3fn_encode_array(x), _torch_e4m3fn(x))


def test_e4m3fn_encode_random_fp32_vs_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(oracle.e4m3fn_encode_array(x), _torch_e4m3fn(x))


# --------------------------------------------------------------------------
# e2m1 and e8m0
# --------------------------------------------------------------------------

E2M1_MAG = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_closed_form():
    for c in range(16):
        v = E2M1_MAG[c & 7]
        assert oracle.e2m1_decode(c) == (-v if c & 8 else v)


def _brute_e2m1(x: np.ndarray) -> np.ndarray:
    """Nearest of the 8 magnitudes by exhaustive search; ties to the even code."""
    mag = np.array(E2M1_MAG)
    a = np.abs(x)[:, None]
    err = np.abs(a - mag[None, :])
    best = err.min(axis=1, keepdims=True)
    cand = err == best
    # among tied candidates prefer an even code
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (pick | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def test_e2m1_encode_ties_table():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 6.0: 7, 7.9: 7}
    for x, c in ties.items():
        assert oracle.e2m1_encode(x) == c
        assert oracle.e2m1_encode(-x) == c | 8


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-8, 8, 200_000), rng.normal(0, 1, 100_000)])
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    around = np.concatenate([np.nextafter(ties, 0), ties, np.nextafter(ties, 10)])
    x = np.concatenate([x, around, -around, [0.0, -0.0]])
    assert np.array_equal(oracle.e2m1_encode_array(x), _brute_e2m1(x))


def test_e8m0_decode():
    for b in range(255):
        assert oracle.e8m0_decode(b) == math.ldexp(1.0, b - 127)
    assert math.isnan(oracle.e8m0_decode(255))
    ref = torch.arange(255, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64)
    got = torch.tensor([oracle.e8m0_decode(b) for b in range(255)], dtype=torch.float64)
    assert torch.equal(ref, got)


# --------------------------------------------------------------------------
# per-tensor quantiser vs torch fp32 arithmetic + torch's cast
# --------------------------------------------------------------------------

def _torch_quant(x_bf16: torch.Tensor, static: bool):
    xf = x_bf16.float()
    if static:
        scale = torch.tensor(6.0, dtype=torch.float32) / torch.tensor(448.0, dtype=torch.float32)
    else:
        scale = xf.abs().amax().clamp(min=torch.tensor(1e-12, dtype=torch.float32)) / 448.0
    codes = (xf / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return np.float32(scale.item()), codes.numpy()


@pytest.mark.parametrize("static", [False, True])
@pytest.mark.parametrize("shape,mult", [((3, 16, 576), 1.0), ((5, 16, 576), 1e-3),
                                        ((2, 16, 576), 300.0), ((7, 576), 1e-30)])
def test_fp8_quantiser_vs_torch(static, shape, mult):
    g = torch.Generator().manual_seed(11)
    x = (torch.randn(shape, generator=g) * mult).to(torch.bfloat16)
    s_ref, c_ref = _torch_quant(x, static)
    s = oracle.fp8_static_scale() if static else oracle.fp8_absmax_scale(x)
    assert np.float32(s).view(np.uint32) == s_ref.view(np.uint32)
    assert np.array_equal(oracle.fp8_quantize(x, s), c_ref)


def test_fp8_absmax_zero_tensor():
    x = torch.zeros((4, 576), dtype=torch.bfloat16)
    assert oracle.fp8_absmax_scale(x) == np.float32(1e-12) / np.float32(448.0)
    assert not oracle.fp8_quantize(x, oracle.fp8_absmax_scale(x)).any()


def test_fp8_quantiser_amax_maps_to_max_code():
    x = workloads.randn_bf16((8, 16, 576), 5)
    s = oracle.fp8_absmax_scale(x)
    c = oracle.fp8_quantize(x, s)
    # the element of largest magnitude lands on +-448 (0x7E / 0xFE)
    i = int(np.argmax(np.abs(x.float().numpy()).reshape(-1)))
    assert c.reshape(-1)[i] & 0x7F == 0x7E


# --------------------------------------------------------------------------
# MXFP4 blocks
# --------------------------------------------------------------------------

def _bf16(vals) -> np.ndarray:
    return workloads.bf16_bits(torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16))


def test_mxfp4_hand_blocks():
    row = np.zeros((1, 64), dtype=np.float32)
    row[0, :32] = 1.0                      # amax 1 -> e = -2, x*4 = 4 -> code 6
    row[0, 32] = 7.0                       # amax 7 -> e = 0; 7 saturates to 6 (code 7)
    row[0, 33] = -0.75                     # 0.75 is a tie -> even code 2 (1.0), sign bit
    row[0, 34] = 1.25                      # tie -> code 2
    row[0, 35] = 2.9                       # -> 3.0, code 5
    p, s = oracle.mxfp4_encode(_bf16(row))
    assert s.tolist() == [[127 - 2, 127 + 0]]
    assert p[0, :16].tolist() == [0x66] * 16
    assert p[0, 16] == (0x7 | (0xA << 4))  # element 32 low nibble, element 33 high nibble
    assert p[0, 17] == (0x2 | (0x5 << 4))
    assert not p[0, 18:].any()


def test_mxfp4_zero_and_power_of_two_blocks():
    row = np.zeros((2, 32), dtype=np.float32)
    row[1, 5] = 2.0 ** -20                  # amax a power of two: byte 127 + (-20) - 2
    p, s = oracle.mxfp4_encode(_bf16(row))
    assert s[0, 0] == 0 and not p[0].any()  # zero block -> exponent -127
    assert s[1, 0] == 127 - 22
    assert (p[1, 2] & 0xF0) >> 4 == 6       # 2^-20 / 2^-22 = 4 -> code 6, element 5 high nibble


def test_mxfp4_roundtrip_error_bound():
    x = workloads.randn_bf16((64, 576), 9)
    p, s = oracle.mxfp4_encode(x)
    dq = oracle.mxfp4_dequant(p, s)
    xf = x.double().numpy()
    scale = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    # every value is the nearest e2m1 grid point of x/scale (saturating at 6)
    y = np.clip(np.abs(xf) / scale, 0, 6)
    grid = np.array(E2M1_MAG)
    nearest = np.abs(y[..., None] - grid).min(axis=-1)
    assert np.allclose(np.abs(np.abs(dq) / scale - y), nearest, atol=0, rtol=0)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def _small_case(kv_lens, seed, fmt="fp8"):
    qo, kvp = workloads.indptrs(kv_lens)
    q = workloads.make_q(len(kv_lens), seed)
    kv = workloads.make_kv(kv_lens, seed + 1)
    qs = oracle.fp8_absmax_scale(q)
    q8 = oracle.fp8_quantize(q, qs)
    if fmt == "fp8":
        ks = oracle.fp8_absmax_scale(kv)
        k8 = oracle.fp8_quantize(kv, ks)
        kd = oracle.fp8_dequant(k8, ks)
        out, lse = oracle.mla_decode(q8, qs, k8, ks, qo, kvp, SM)
    else:
        pk, sc = oracle.mxfp4_encode(kv)
        kd = oracle.mxfp4_dequant(pk, sc)
        out, lse = oracle.mla_decode(q8, qs, pk, 0.0, qo, kvp, SM, kv_format=1, kv_scales=sc)
    qd = oracle.fp8_dequant(q8, qs)
    return qo, kvp, qd, kd, out, lse


def _sdpa(qd_row, kd_rows):
    """torch SDPA, fp64, 16 heads against one shared latent head."""
    q = torch.from_numpy(qd_row)[None, :, None, :]                # (1, 16, 1, 576)
    k = torch.from_numpy(kd_rows)[None, None].expand(1, 16, -1, -1).contiguous()
    v = torch.from_numpy(kd_rows[:, :512].copy())[None, None].expand(1, 16, -1, -1).contiguous()
    o = F.scaled_dot_product_attention(q, k, v, scale=SM)[0, :, 0, :]
    s = (q[0, :, 0, :] @ k[0, 0].T) * SM
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_attention_vs_sdpa(fmt):
    kv_lens = [1, 7, 33, 100, 300]
    qo, kvp, qd, kd, out, lse = _small_case(kv_lens, 21, fmt)
    for b in range(len(kv_lens)):
        o_ref, l_ref = _sdpa(qd[b], kd[kvp[b]:kvp[b + 1]])
        np.testing.assert_allclose(out[b], o_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b], l_ref, rtol=1e-12, atol=1e-12)


def test_attention_kv_len_one_returns_v_row():
    qo, kvp, qd, kd, out, lse = _small_case([1, 1, 1], 31)
    for b in range(3):
        for h in range(16):
            assert np.array_equal(out[b, h], kd[b, :512])
            assert lse[b, h] == pytest.approx(float(qd[b, h] @ kd[b]) * SM, rel=1e-14)


def test_attention_identical_keys_give_mean_of_v():
    # all keys identical in their 576 QK dims would make V identical too, so
    # make the scores identical instead: Q is nonzero only on dims 512..575 and
    # every key shares those dims, while the V dims (0..511) differ.
    rng = np.random.default_rng(5)
    n = 37
    kd = rng.normal(size=(n, 576))
    kd[:, 512:] = kd[0, 512:]
    q = np.zeros(576)
    q[512:] = rng.normal(size=64)
    o, lse = oracle.attend(q, kd, SM)
    np.testing.assert_allclose(o, kd[:, :512].mean(axis=0), rtol=1e-12, atol=1e-14)
    assert lse == pytest.approx(float(q @ kd[0]) * SM + math.log(n), rel=1e-13)


def test_attention_rope_tail_matters():
    # scores driven only by dims 512..575: the result must still match the
    # library reference, and differ from one that drops those dims.
    rng = np.random.default_rng(6)
    kd = rng.normal(size=(50, 576)) * 3
    q = np.zeros((16, 576))
    q[:, 512:] = rng.normal(size=(16, 64)) * 3
    out = np.stack([oracle.attend(q[h], kd, SM)[0] for h in range(16)])
    o_ref, _ = _sdpa(q, kd)
    np.testing.assert_allclose(out, o_ref, rtol=1e-12, atol=1e-13)
    o_drop, _ = _sdpa(np.ascontiguousarray(q[:, :512]), np.ascontiguousarray(kd[:, :512]))
    assert np.abs(out - o_drop).max() > 0.1


def test_attention_empty_range():
    o, lse = oracle.attend(np.ones(576), np.zeros((0, 576)), SM)
    assert not o.any() and lse == -math.inf
    o, lse = oracle.lse_merge(np.zeros((3, 512)), np.full(3, -np.inf))
    assert not o.any() and lse == -math.inf


def test_split_then_merge_equals_unsplit():
    kv_lens = [257, 1000, 64]
    qo, kvp, qd, kd, out, lse = _small_case(kv_lens, 41)
    rng = np.random.default_rng(2)
    # rebuild the codes the same way _small_case did
    q = workloads.make_q(len(kv_lens), 41)
    kv = workloads.make_kv(kv_lens, 42)
    qs, ks = oracle.fp8_absmax_scale(q), oracle.fp8_absmax_scale(kv)
    q8, k8 = oracle.fp8_quantize(q, qs), oracle.fp8_quantize(kv, ks)
    for b, n in enumerate(kv_lens):
        cuts = np.sort(rng.choice(np.arange(1, n), size=4, replace=False))
        lo = np.concatenate([[0], cuts]).astype(np.int32)
        hi = np.concatenate([cuts, [n]]).astype(np.int32)
        seqs = np.full(lo.size, b, dtype=np.int32)
        o_s, l_s = oracle.mla_decode(q8, qs, k8, ks, qo, kvp, SM, seqs=seqs, kv_lo=lo, kv_hi=hi)
        for h in range(16):
            o_m, l_m = oracle.lse_merge(o_s[:, h], l_s[:, h])
            np.testing.assert_allclose(o_m, out[b, h], rtol=1e-12, atol=1e-14)
            assert l_m == pytest.approx(lse[b, h], rel=1e-13)


def test_selected_sequences_match_full_run():
    kv_lens = [10, 0, 50, 3]
    qo, kvp, qd, kd, out, lse = _small_case(kv_lens, 51)
    assert not out[1].any() and np.all(lse[1] == -np.inf)
    q = workloads.make_q(4, 51)
    kv = workloads.make_kv(kv_lens, 52)
    qs, ks = oracle.fp8_absmax_scale(q), oracle.fp8_absmax_scale(kv)
    o2, l2 = oracle.mla_decode(oracle.fp8_quantize(q, qs), qs, oracle.fp8_quantize(kv, ks), ks,
                               qo, kvp, SM, seqs=[3, 0])
    assert np.array_equal(o2[0], out[3]) and np.array_equal(o2[1], out[0])
    assert np.array_equal(l2, lse[[3, 0]])


# --------------------------------------------------------------------------
# several query rows per sequence (causal, bottom-right aligned)
# --------------------------------------------------------------------------

def _mtp_case(kv_lens, q_lens, seed, fmt="fp8"):
    qo, kvp = workloads.indptrs(kv_lens, q_lens)
    q = workloads.make_q(int(qo[-1]), seed)
    kv = workloads.make_kv(kv_lens, seed + 1)
    qs = oracle.fp8_absmax_scale(q)
    q8 = oracle.fp8_quantize(q, qs)
    if fmt == "fp8":
        ks = oracle.fp8_absmax_scale(kv)
        k8 = oracle.fp8_quantize(kv, ks)
        kd = oracle.fp8_dequant(k8, ks)
        out, lse = oracle.mla_decode(q8, qs, k8, ks, qo, kvp, SM)
    else:
        pk, sc = oracle.mxfp4_encode(kv)
        kd = oracle.mxfp4_dequant(pk, sc)
        out, lse = oracle.mla_decode(q8, qs, pk, 0.0, qo, kvp, SM, kv_format=1, kv_scales=sc)
    return qo, kvp, oracle.fp8_dequant(q8, qs), kd, out, lse


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_query_rows_vs_torch_lower_right_causal_bias(fmt):
    """Rows of one sequence against torch SDPA with torch's own bottom-right
    causal bias (torch.nn.attention.bias.causal_lower_right); rows that see no
    cache row give O = 0 and LSE = -inf (torch returns NaN there)."""
    import warnings

    from torch.nn.attention.bias import causal_lower_right
    kv_lens = [40, 3, 1, 0, 65, 9]
    q_lens = [4, 4, 2, 3, 1, 3]
    qo, kvp, qd, kd, out, lse = _mtp_case(kv_lens, q_lens, 61, fmt)
    for b in range(len(kv_lens)):
        r0, r1 = int(qo[b]), int(qo[b + 1])
        R, n = r1 - r0, int(kvp[b + 1] - kvp[b])
        kb = kd[kvp[b]:kvp[b + 1]]
        visible = [n - (R - 1 - i) for i in range(R)]
        for i in range(R):
            if visible[i] <= 0:
                assert not out[r0 + i].any() and np.all(lse[r0 + i] == -np.inf)
        if n == 0:
            continue
        q = torch.from_numpy(qd[r0:r1]).permute(1, 0, 2)[None]           # (1, 16, R, 576)
        k = torch.from_numpy(kb)[None, None].expand(1, 16, -1, -1).contiguous()
        v = torch.from_numpy(kb[:, :512].copy())[None, None].expand(1, 16, -1, -1).contiguous()
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            bias = causal_lower_right(R, n)
            o_ref = F.scaled_dot_product_attention(q, k, v, attn_mask=bias, scale=SM)[0]
            mask = bias._materialize(device="cpu")
        s = (q[0] @ k[0].transpose(-1, -2)) * SM                             # (16, R, n)
        s = s.masked_fill(~mask, -math.inf)
        l_ref = torch.logsumexp(s, dim=-1)                                   # (16, R)
        for i in range(R):
            if visible[i] <= 0:
                continue
            np.testing.assert_allclose(out[r0 + i], o_ref[:, i].numpy(), rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[r0 + i], l_ref[:, i].numpy(), rtol=1e-12, atol=1e-12)


def test_query_rows_last_row_sees_the_whole_cache():
    """The last query row of a sequence equals the single-row decode over the
    whole sequence; row i equals it over the first n - (R - 1 - i) rows."""
    kv_lens, q_lens = [50, 7], [3, 2]
    qo, kvp, qd, kd, out, lse = _mtp_case(kv_lens, q_lens, 71)
    for b in range(2):
        R, n = q_lens[b], kv_lens[b]
        kb = kd[kvp[b]:kvp[b + 1]]
        for i in range(R):
            for h in (0, 9):
                o1, l1 = oracle.attend(qd[qo[b] + i, h], kb[:n - (R - 1 - i)], SM)
                np.testing.assert_allclose(out[qo[b] + i, h], o1, rtol=1e-13, atol=1e-15)
                assert lse[qo[b] + i, h] == pytest.approx(l1, rel=1e-14)


def test_query_rows_split_then_merge_equals_unsplit():
    kv_lens, q_lens = [300, 70], [4, 3]
    qo, kvp, qd, kd, out, lse = _mtp_case(kv_lens, q_lens, 81)
    q = workloads.make_q(int(qo[-1]), 81)
    kv = workloads.make_kv(kv_lens, 82)
    qs, ks = oracle.fp8_absmax_scale(q), oracle.fp8_absmax_scale(kv)
    q8, k8 = oracle.fp8_quantize(q, qs), oracle.fp8_quantize(kv, ks)
    for b, n in enumerate(kv_lens):
        # the last cut sits inside the causal tail, so a split sees part of it
        lo = np.array([0, n // 3, n - 2], dtype=np.int32)
        hi = np.array([n // 3, n - 2, n], dtype=np.int32)
        seqs = np.full(3, b, dtype=np.int32)
        o_s, l_s = oracle.mla_decode(q8, qs, k8, ks, qo, kvp, SM, seqs=seqs, kv_lo=lo, kv_hi=hi)
        R = q_lens[b]
        for i in range(R):
            for h in range(0, 16, 5):
                parts_o = o_s[[s * R + i for s in range(3)], h]
                parts_l = l_s[[s * R + i for s in range(3)], h]
                o_m, l_m = oracle.lse_merge(parts_o, parts_l)
                np.testing.assert_allclose(o_m, out[qo[b] + i, h], rtol=1e-12, atol=1e-14)
                assert l_m == pytest.approx(lse[qo[b] + i, h], rel=1e-13)


# --------------------------------------------------------------------------
# bf16 cache (no quantisation) and the logit soft-cap
# --------------------------------------------------------------------------

def _bf16_to_f64(t):
    return t.to(torch.float64).numpy()


def test_bf16_decode_vs_sdpa():
    """bf16 Q and cache decoded exactly, against torch SDPA in fp64, with
    causal query rows."""
    import warnings

    from torch.nn.attention.bias import causal_lower_right
    kv_lens, q_lens = [1, 40, 0, 300], [1, 3, 2, 2]
    qo, kvp = workloads.indptrs(kv_lens, q_lens)
    q = workloads.make_q(int(qo[-1]), 91)
    kv = workloads.make_kv(kv_lens, 92)
    out, lse = oracle.mla_decode_bf16(q, kv, qo, kvp, SM)
    qd, kd = _bf16_to_f64(q), _bf16_to_f64(kv)
    for b in range(len(kv_lens)):
        r0, r1 = int(qo[b]), int(qo[b + 1])
        n = int(kvp[b + 1] - kvp[b])
        if n == 0:
            assert not out[r0:r1].any() and np.all(lse[r0:r1] == -np.inf)
            continue
        kb = kd[kvp[b]:kvp[b + 1]]
        qq = torch.from_numpy(qd[r0:r1]).permute(1, 0, 2)[None]
        k = torch.from_numpy(kb)[None, None].expand(1, 16, -1, -1).contiguous()
        v = torch.from_numpy(kb[:, :512].copy())[None, None].expand(1, 16, -1, -1).contiguous()
        R = r1 - r0
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            bias = causal_lower_right(R, n)
            o_ref = F.scaled_dot_product_attention(qq, k, v, attn_mask=bias, scale=SM)[0]
        for i in range(R):
            if n - (R - 1 - i) <= 0:
                assert not out[r0 + i].any()
                continue
            np.testing.assert_allclose(out[r0 + i], o_ref[:, i].numpy(), rtol=1e-12, atol=1e-13)


def test_logit_cap_limits():
    """The soft-cap: a huge cap changes nothing; a tiny cap flattens every
    logit to about 0, so the output tends to the mean of V (closed forms)."""
    rng = np.random.default_rng(12)
    kd = rng.normal(size=(50, 576)) * 2
    q = rng.normal(size=576) * 2
    o0, l0 = oracle.attend(q, kd, SM)
    o1, l1 = oracle.attend_cap(q, kd, SM, 1e12)
    np.testing.assert_allclose(o1, o0, rtol=1e-10, atol=1e-12)
    assert l1 == pytest.approx(l0, rel=1e-10)
    cap = 1e-7
    o2, l2 = oracle.attend_cap(q, kd, SM, cap)
    np.testing.assert_allclose(o2, kd[:, :512].mean(axis=0), rtol=1e-6, atol=1e-6)
    assert l2 == pytest.approx(math.log(50), abs=1e-6)


def test_logit_cap_vs_torch():
    """Capped logits cap * tanh(s / cap) through torch's tanh, softmax and
    logsumexp, against the oracle, on scores large enough to saturate."""
    rng = np.random.default_rng(13)
    kd = rng.normal(size=(80, 576)) * 4
    for cap in (1.0, 5.0, 30.0):
        for h in range(3):
            q = rng.normal(size=576) * 4
            o, l = oracle.attend_cap(q, kd, SM, cap)
            s = torch.from_numpy(kd) @ torch.from_numpy(q) * SM
            s = cap * torch.tanh(s / cap)
            p = torch.softmax(s, dim=0)
            np.testing.assert_allclose(o, (p @ torch.from_numpy(kd[:, :512])).numpy(),
                                       rtol=1e-12, atol=1e-13)
            assert l == pytest.approx(float(torch.logsumexp(s, dim=0)), rel=1e-13)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_quantised_decode_with_logit_cap_vs_torch(fmt):
    """The FP8 / MXFP4 decode with a soft-cap, against torch on the
    dequantised inputs: scores (q . k) * sm_scale, capped to
    cap * tanh(s / cap), then softmax, P V and logsumexp, in fp64; ragged
    sequences, one query row each."""
    kv_lens = [1, 7, 40, 150]
    qo, kvp, qd, kd, out0, lse0 = _small_case(kv_lens, 51, fmt)
    q = workloads.make_q(len(kv_lens), 51)
    kv = workloads.make_kv(kv_lens, 52)
    qs = oracle.fp8_absmax_scale(q)
    q8 = oracle.fp8_quantize(q, qs)
    if fmt == "fp8":
        ks = oracle.fp8_absmax_scale(kv)
        codes, scales = oracle.fp8_quantize(kv, ks), None
    else:
        ks = 0.0
        codes, scales = oracle.mxfp4_encode(kv)
    # scores here are O(1): caps of 0.5 and 2 bend them, 1e30 leaves them alone
    for cap in (0.5, 2.0, 1e30):
        out, lse = oracle.mla_decode(q8, qs, codes, ks, qo, kvp, SM, kv_format=0 if fmt == "fp8" else 1,
                                     kv_scales=scales, logit_cap=cap)
        if cap == 1e30:
            np.testing.assert_allclose(out, out0, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse, lse0, rtol=1e-12, atol=1e-13)
            continue
        for b in range(len(kv_lens)):
            rows = kd[kvp[b]:kvp[b + 1]]
            s = (torch.from_numpy(qd[b]) @ torch.from_numpy(rows).T) * SM    # (16, n)
            s = cap * torch.tanh(s / cap)
            p = torch.softmax(s, dim=-1)
            ref = p @ torch.from_numpy(rows[:, :512].copy())
            np.testing.assert_allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[b], torch.logsumexp(s, dim=-1).numpy(), rtol=1e-13,
                                       atol=1e-13)
            # every capped logit lies below the cap, so LSE < cap + log(n)
            assert np.all(lse[b] < cap + math.log(kv_lens[b]))


# --------------------------------------------------------------------------
# non-finite input: NaN propagates, as torch's amax in the pages' quantisers
# (kernelindex.com amd-mixed-mla 722089 `quantize_fp8`, 738050 `_quantize_fp8`)
# --------------------------------------------------------------------------

def _e4m3_is_nan(codes) -> np.ndarray:
    """E4M3FN has two NaN codes, 0x7F and 0xFF."""
    return (np.asarray(codes, dtype=np.uint8) & 0x7F) == 0x7F


def _planted(shape, seed, where: dict) -> torch.Tensor:
    x = workloads.randn_bf16(shape, seed).clone()
    flat = x.view(-1)
    for i, v in where.items():
        flat[i] = v
    return x


@pytest.mark.parametrize("value", [math.nan, math.inf, -math.inf])
def test_fp8_absmax_nonfinite_vs_torch(value):
    x = _planted((3, 16, 576), 12, {1000: value})
    s = oracle.fp8_absmax_scale(x)
    ref = x.float().abs().amax().clamp(min=torch.tensor(1e-12)) / 448.0
    if math.isnan(value):
        assert math.isnan(s) and math.isnan(ref.item())
    else:
        assert s == np.float32(np.inf) and ref.item() == math.inf
    codes = oracle.fp8_quantize(x, s)
    rc = (x.float() / ref).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan = _e4m3_is_nan(codes)
    # the same elements are NaN (torch keeps a NaN's sign bit, the oracle writes 0x7F)
    assert np.array_equal(nan, _e4m3_is_nan(rc))
    assert np.all(codes[nan] == 0x7F)
    assert np.array_equal(codes[~nan], rc[~nan])
    if math.isnan(value):
        assert nan.all()                      # x / NaN
    else:
        assert nan.reshape(-1)[1000] and nan.sum() == 1   # inf / inf; finite / inf = +-0
        assert np.all((codes[~nan] & 0x7F) == 0)


def test_fp8_static_scale_nonfinite_elements_vs_torch():
    x = _planted((2, 16, 576), 13, {5: math.nan, 77: math.inf, 900: -math.inf})
    s = oracle.fp8_static_scale()
    codes = oracle.fp8_quantize(x, s).reshape(-1)
    _, rc = _torch_quant(x, static=True)
    rc = rc.reshape(-1)
    assert codes[5] == 0x7F and _e4m3_is_nan(rc[5])
    assert codes[77] == 0x7E and codes[900] == 0xFE      # infinities saturate to +-448
    keep = np.ones(codes.size, dtype=bool)
    keep[5] = False
    assert np.array_equal(codes[keep], rc[keep])


@pytest.mark.parametrize("value", [math.nan, math.inf, -math.inf])
def test_mxfp4_nonfinite_block(value):
    x = _planted((4, 576), 14, {2 * 576 + 100: value})   # row 2, block 3
    p, s = oracle.mxfp4_encode(x)
    clean = x.clone()
    clean.view(-1)[2 * 576 + 100] = 0.0
    p0, s0 = oracle.mxfp4_encode(clean)
    assert s[2, 3] == 0xFF and not p[2, 48:64].any()
    s_other, p_other = s.copy(), p.copy()
    s_other[2, 3], p_other[2, 48:64] = s0[2, 3], p0[2, 48:64]
    assert np.array_equal(s_other, s0) and np.array_equal(p_other, p0)
    # 0xFF is e8m0's NaN code (torch's float8_e8m0fnu agrees), so the block
    # dequantises to NaN and nothing else does
    assert torch.tensor([0xFF], dtype=torch.uint8).view(torch.float8_e8m0fnu).float().isnan().all()
    dq = oracle.mxfp4_dequant(p, s)
    bad = np.zeros(dq.shape, dtype=bool)
    bad[2, 96:128] = True
    assert np.isnan(dq[bad]).all() and np.isfinite(dq[~bad]).all()


def test_attention_nan_code_poisons_its_head_only():
    """A NaN Q code makes its (row, head) NaN and nothing else; torch SDPA on
    the dequantised inputs agrees."""
    kv_lens = [40, 9]
    qo, kvp, qd, kd, out, lse = _small_case(kv_lens, 41)
    q = workloads.make_q(2, 41)
    qs = oracle.fp8_absmax_scale(q)
    q8 = oracle.fp8_quantize(q, qs)
    q8[1, 3, 200] = 0x7F
    kv = workloads.make_kv(kv_lens, 42)
    ks = oracle.fp8_absmax_scale(kv)
    k8 = oracle.fp8_quantize(kv, ks)
    o2, l2 = oracle.mla_decode(q8, qs, k8, ks, qo, kvp, SM)
    bad = np.zeros(o2.shape[:2], dtype=bool)
    bad[1, 3] = True
    assert np.isnan(o2[bad]).all() and np.isnan(l2[bad]).all()
    assert np.array_equal(o2[~bad], out[~bad]) and np.array_equal(l2[~bad], lse[~bad])
    qd2 = oracle.fp8_dequant(q8, qs)
    ref, _ = _sdpa(qd2[1], kd[40:49])
    assert np.isnan(ref[3]).all()
    np.testing.assert_allclose(o2[1, [h for h in range(16) if h != 3]],
                               ref[[h for h in range(16) if h != 3]], rtol=1e-12, atol=1e-14)


def test_attention_nan_cache_row_poisons_its_sequence_only():
    kv_lens = [40, 9, 17]
    qo, kvp, qd, kd, out, lse = _small_case(kv_lens, 43)
    q = workloads.make_q(3, 43)
    qs = oracle.fp8_absmax_scale(q)
    q8 = oracle.fp8_quantize(q, qs)
    kv = workloads.make_kv(kv_lens, 44)
    ks = oracle.fp8_absmax_scale(kv)
    k8 = oracle.fp8_quantize(kv, ks)
    k8[45, 570] = 0x7F                        # a rope-tail dim of sequence 1's row 5
    o2, l2 = oracle.mla_decode(q8, qs, k8, ks, qo, kvp, SM)
    assert np.isnan(o2[1]).all() and np.isnan(l2[1]).all()
    assert np.array_equal(o2[[0, 2]], out[[0, 2]]) and np.array_equal(l2[[0, 2]], lse[[0, 2]])


def test_lse_merge_nan_and_empty_partials():
    rng = np.random.default_rng(3)
    o_s = rng.standard_normal((3, 512))
    o, l = oracle.lse_merge(o_s, np.array([0.5, np.nan, 1.0]))
    assert np.isnan(o).all() and math.isnan(l)
    o, l = oracle.lse_merge(o_s, np.array([-np.inf, np.nan, -np.inf]))
    assert np.isnan(o).all() and math.isnan(l)
    o, l = oracle.lse_merge(o_s, np.array([-np.inf, -np.inf, -np.inf]))
    assert not o.any() and l == -math.inf
    # an empty split carries no weight
    o, l = oracle.lse_merge(o_s, np.array([0.25, -np.inf, 0.25]))
    np.testing.assert_allclose(o, (o_s[0] + o_s[2]) / 2, rtol=1e-15)
    assert l == pytest.approx(0.25 + math.log(2.0), rel=1e-15)
