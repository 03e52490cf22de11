"""GPU parity of the quantisers: the library's FP8 and MXFP4 codes must equal
the oracle's bit for bit (same bytes, same fp32 scale)."""
import numpy as np
import pytest
import torch

import mla_latent_kv_bf16_amd as mla
import oracle
import workloads
from gpu_cases import DEV, announce

pytestmark = pytest.mark.gpu


def _gpu_quant(x_host: torch.Tensor, mode: str, scale=None):
    xd = x_host.contiguous().to(DEV)
    out = torch.empty(xd.shape, dtype=torch.uint8, device=DEV)
    sc = torch.empty(1, dtype=torch.float32, device=DEV)
    if mode == "static":
        sc.fill_(float(scale))
    ws = torch.empty(max(mla.mla_quant_fp8_workspace_size(xd.numel()), 256), dtype=torch.uint8,
                     device=DEV)
    mla.mla_quant_fp8(xd, out, sc, mla.MLA_Q_SCALE_STATIC if mode == "static"
                      else mla.MLA_Q_SCALE_ABSMAX, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), np.float32(sc.item())


@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["absmax", "static"])
def test_q_codes_match_oracle(w, mode):
    announce(f"q quant {w.name} {mode}")
    q = workloads.make_q(w.batch, w.seed_q)
    s_ref = oracle.fp8_static_scale() if mode == "static" else oracle.fp8_absmax_scale(q)
    codes, s = _gpu_quant(q, mode, s_ref)
    assert s.view(np.uint32) == np.float32(s_ref).view(np.uint32)
    assert np.array_equal(codes, oracle.fp8_quantize(q, s_ref))


def _all_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    keep = np.isfinite(f)
    u = (bits[keep]).astype(np.uint16)
    pad = (-u.size) % 8
    u = np.concatenate([u, np.zeros(pad, dtype=np.uint16)])
    return torch.from_numpy(u.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("scale", [1.0, 0.5, 6.0 / 448.0, 3.0e-3, 1.7e-5, 2.0 ** -20, 1e30])
def test_every_bf16_value_static_scale(scale):
    announce(f"exhaustive bf16 quant, scale {scale}")
    x = _all_bf16()
    s = np.float32(scale)
    codes, _ = _gpu_quant(x, "static", s)
    assert np.array_equal(codes, oracle.fp8_quantize(x, s))


def test_every_bf16_value_absmax():
    announce("exhaustive bf16 quant, absmax")
    x = _all_bf16()
    codes, s = _gpu_quant(x, "absmax")
    s_ref = oracle.fp8_absmax_scale(x)
    assert s.view(np.uint32) == s_ref.view(np.uint32)
    assert np.array_equal(codes, oracle.fp8_quantize(x, s_ref))


@pytest.mark.parametrize("n", [1, 7, 9, 4095, 1000003])
def test_quant_ragged_lengths(n):
    announce(f"quant ragged n={n}")
    x = workloads.randn_bf16((n,), 1234 + n) * 3
    for mode in ("absmax", "static"):
        s_ref = oracle.fp8_absmax_scale(x) if mode == "absmax" else np.float32(0.01)
        codes, s = _gpu_quant(x, mode, s_ref)
        assert s.view(np.uint32) == np.float32(s_ref).view(np.uint32)
        assert np.array_equal(codes, oracle.fp8_quantize(x, s_ref))


def test_quant_zero_and_empty():
    announce("quant zeros / empty")
    x = torch.zeros(64, dtype=torch.bfloat16)
    codes, s = _gpu_quant(x, "absmax")
    assert s == np.float32(1e-12) / np.float32(448.0) and not codes.any()
    xe = torch.zeros(8, dtype=torch.bfloat16)[:0]
    _, s = _gpu_quant(xe, "absmax")
    assert s == np.float32(1e-12) / np.float32(448.0)


@pytest.mark.parametrize("w", workloads.WORKLOADS[:4], ids=lambda w: w.name)
def test_kv_codes_match_oracle(w):
    announce(f"kv quant {w.name}")
    kv = workloads.make_kv([w.kv_len] * w.batch, w.seed_kv)
    codes, s = _gpu_quant(kv, "absmax")
    s_ref = oracle.fp8_absmax_scale(kv)
    assert s.view(np.uint32) == s_ref.view(np.uint32)
    if kv.shape[0] <= 600_000:
        assert np.array_equal(codes, oracle.fp8_quantize(kv, s_ref))
    else:
        rng = np.random.default_rng(0)
        for r0 in rng.integers(0, kv.shape[0] - 4096, size=16):
            sl = slice(int(r0), int(r0) + 4096)
            assert np.array_equal(codes[sl], oracle.fp8_quantize(kv[sl], s_ref))


def _special_mx_rows():
    rows = np.zeros((8, 576), dtype=np.float32)
    rows[1, :] = 1.0
    rows[2, ::3] = -0.75
    rows[3, :32] = np.array([2.0 ** -130] * 16 + [2.0 ** -128] * 16)   # bf16 subnormals
    rows[4, :] = 3.0e38
    rows[4, 1::2] = -1.0e-38
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    rows[5, :] = np.tile(np.concatenate([ties, -ties, ties * 2, -ties / 2]), 18)
    rows[6, :] = np.linspace(-7, 7, 576)
    rows[7, 100] = 1e-20
    return torch.from_numpy(rows).to(torch.bfloat16)


@pytest.mark.parametrize("which", ["random", "special", "bs256_kv1024"])
def test_mxfp4_encoder_matches_oracle(which):
    announce(f"mxfp4 encode {which}")
    if which == "random":
        x = workloads.randn_bf16((1031, 576), 77) * 5
    elif which == "special":
        x = _special_mx_rows()
    else:
        w = workloads.BY_NAME["bs256_kv1024_mxfp4"]
        x = workloads.make_kv([w.kv_len] * w.batch, w.seed_kv)
    xd = x.to(DEV)
    packed = torch.empty((x.shape[0], 288), dtype=torch.uint8, device=DEV)
    scales = torch.empty((x.shape[0], 18), dtype=torch.uint8, device=DEV)
    mla.mla_encode_mxfp4(xd, packed, scales)
    torch.cuda.synchronize()
    p_ref, s_ref = oracle.mxfp4_encode(x)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
