"""CPU reference oracle for absorbed-path MLA decode -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library in
``mla_latent_kv_bf16_amd`` and its binding) never imports it, and the two
share no code. Every function here is a thin ctypes/numpy wrapper around
``mla_oracle.c``, which holds all of the arithmetic and cites the passages of
the kernelindex.com "amd-mixed-mla" pages it follows.

Parity status: every function is pinned by the CPU test suite
(``tests/test_oracle_pins.py``) against torch's float8 casts and fp32 ops,
brute-force nearest-code search, closed forms and torch's fp64
scaled_dot_product_attention; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

HEADS = 16
DQK = 576
DV = 512
MX_BLOCK = 32


def build(force: bool = True) -> str:
    """Compile mla_oracle.c into liboracle.so next to it (gcc, OpenMP, fp64)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
             "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i32p = ctypes.POINTER(ctypes.c_int32)
        f64p = ctypes.POINTER(ctypes.c_double)
        L.orc_e4m3fn_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3fn_decode.restype = ctypes.c_double
        L.orc_e4m3fn_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3fn_encode.restype = ctypes.c_uint8
        L.orc_e4m3fn_encode_f32.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_size_t, u8p]
        L.orc_e4m3fn_encode_f32.restype = None
        L.orc_e2m1_encode_f64.argtypes = [f64p, ctypes.c_size_t, u8p]
        L.orc_e2m1_encode_f64.restype = None
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e2m1_encode.argtypes = [ctypes.c_double]
        L.orc_e2m1_encode.restype = ctypes.c_uint8
        L.orc_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_decode.restype = ctypes.c_double
        L.orc_fp8_absmax_scale.argtypes = [u16p, ctypes.c_size_t]
        L.orc_fp8_absmax_scale.restype = ctypes.c_float
        L.orc_fp8_static_scale.argtypes = []
        L.orc_fp8_static_scale.restype = ctypes.c_float
        L.orc_fp8_quantize.argtypes = [u16p, ctypes.c_size_t, ctypes.c_float, u8p]
        L.orc_fp8_quantize.restype = None
        L.orc_mxfp4_encode_rows.argtypes = [u16p, ctypes.c_size_t, ctypes.c_size_t, u8p, u8p]
        L.orc_mxfp4_encode_rows.restype = None
        L.orc_mxfp4_dequant_rows.argtypes = [u8p, u8p, ctypes.c_size_t, ctypes.c_size_t, f64p]
        L.orc_mxfp4_dequant_rows.restype = None
        L.orc_attend.argtypes = [f64p, f64p, ctypes.c_int, ctypes.c_double, f64p, f64p]
        L.orc_attend.restype = None
        L.orc_lse_merge.argtypes = [ctypes.c_int, f64p, f64p, f64p, f64p]
        L.orc_lse_merge.restype = None
        L.orc_mla_decode.argtypes = [
            ctypes.c_int, u8p, ctypes.c_float, u8p, u8p, ctypes.c_float, i32p, i32p,
            ctypes.c_int, i32p, ctypes.c_int, i32p, i32p, ctypes.c_double, f64p, f64p]
        L.orc_mla_decode.restype = ctypes.c_longlong
        L.orc_mla_decode_cap.argtypes = [
            ctypes.c_int, u8p, ctypes.c_float, u8p, u8p, ctypes.c_float, i32p, i32p,
            ctypes.c_int, i32p, ctypes.c_int, i32p, i32p, ctypes.c_double, ctypes.c_double, f64p,
            f64p]
        L.orc_mla_decode_cap.restype = ctypes.c_longlong
        L.orc_attend_cap.argtypes = [f64p, f64p, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                     f64p, f64p]
        L.orc_attend_cap.restype = None
        L.orc_mla_decode_bf16.argtypes = [
            u16p, u16p, i32p, i32p, ctypes.c_int, i32p, ctypes.c_int, i32p, i32p,
            ctypes.c_double, ctypes.c_double, f64p, f64p]
        L.orc_mla_decode_bf16.restype = ctypes.c_longlong
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(x) -> np.ndarray:
    """bf16 payload as uint16 (accepts a torch bf16 tensor or a uint16 array)."""
    if hasattr(x, "view") and hasattr(x, "dtype") and "bfloat16" in str(x.dtype):
        import torch
        x = x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return np.ascontiguousarray(x, dtype=np.uint16)


# -- scalar codecs ---------------------------------------------------------

def e4m3fn_decode(code: int) -> float:
    return lib().orc_e4m3fn_decode(code)


def e4m3fn_encode(x: float) -> int:
    return lib().orc_e4m3fn_encode(x)


def e4m3fn_encode_array(x: np.ndarray) -> np.ndarray:
    """orc_e4m3fn_encode applied to every element of an fp32 array."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_e4m3fn_encode_f32(_ptr(x, ctypes.c_float), x.size, _ptr(out, ctypes.c_uint8))
    return out


def e2m1_encode_array(x: np.ndarray) -> np.ndarray:
    """orc_e2m1_encode applied to every element of an fp64 array."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_e2m1_encode_f64(_ptr(x, ctypes.c_double), x.size, _ptr(out, ctypes.c_uint8))
    return out


def e2m1_decode(nib: int) -> float:
    return lib().orc_e2m1_decode(nib)


def e2m1_encode(x: float) -> int:
    return lib().orc_e2m1_encode(x)


def e8m0_decode(b: int) -> float:
    return lib().orc_e8m0_decode(b)


# -- tensor quantisers -------------------------------------------------------

def fp8_absmax_scale(x_bf16) -> np.float32:
    x = _u16(x_bf16).reshape(-1)
    return np.float32(lib().orc_fp8_absmax_scale(_ptr(x, ctypes.c_uint16), x.size))


def fp8_static_scale() -> np.float32:
    return np.float32(lib().orc_fp8_static_scale())


def fp8_quantize(x_bf16, scale: float) -> np.ndarray:
    """e4m3fn codes of fp32(x)/scale, same shape as x."""
    x = _u16(x_bf16)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_fp8_quantize(_ptr(x, ctypes.c_uint16), x.size, ctypes.c_float(scale),
                           _ptr(out, ctypes.c_uint8))
    return out


def mxfp4_encode(x_bf16) -> tuple[np.ndarray, np.ndarray]:
    """Rows of 576 (any multiple of 32) -> (packed rows x cols/2, scales rows x cols/32)."""
    x = _u16(x_bf16)
    cols = x.shape[-1]
    assert cols % MX_BLOCK == 0
    rows = x.size // cols
    packed = np.empty(x.shape[:-1] + (cols // 2,), dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (cols // MX_BLOCK,), dtype=np.uint8)
    lib().orc_mxfp4_encode_rows(_ptr(x, ctypes.c_uint16), rows, cols,
                                _ptr(packed, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8))
    return packed, scales


def mxfp4_dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    cols = packed.shape[-1] * 2
    rows = packed.size // packed.shape[-1]
    out = np.empty(packed.shape[:-1] + (cols,), dtype=np.float64)
    lib().orc_mxfp4_dequant_rows(_ptr(packed, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                                 rows, cols, _ptr(out, ctypes.c_double))
    return out


def fp8_dequant(codes: np.ndarray, scale: float) -> np.ndarray:
    table = np.array([e4m3fn_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)] * float(scale)


# -- attention ---------------------------------------------------------------

def attend(q: np.ndarray, kd: np.ndarray, sm_scale: float):
    """One head: q (576,), kd (n, 576) fp64 -> (o (512,), lse natural)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    kd = np.ascontiguousarray(kd, dtype=np.float64).reshape(-1, DQK)
    o = np.empty(DV, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    lib().orc_attend(_ptr(q, ctypes.c_double), _ptr(kd, ctypes.c_double), kd.shape[0],
                     sm_scale, _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    return o, float(lse[0])


def attend_cap(q: np.ndarray, kd: np.ndarray, sm_scale: float, cap: float):
    """attend() with the logit soft-cap cap * tanh(s / cap) (cap > 0)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    kd = np.ascontiguousarray(kd, dtype=np.float64).reshape(-1, DQK)
    o = np.empty(DV, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    lib().orc_attend_cap(_ptr(q, ctypes.c_double), _ptr(kd, ctypes.c_double), kd.shape[0],
                         sm_scale, cap, _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    return o, float(lse[0])


def mla_decode_bf16(q_bf16, kv_bf16, qo_indptr, kv_indptr, sm_scale: float,
                    logit_cap: float = 0.0, seqs=None, kv_lo=None, kv_hi=None):
    """fp64 decode of the bf16 path: q (rows, 16, 576) and kv (total_kv, 576)
    as bf16 tensors or uint16 bit arrays. Returns (out (rows, 16, 512), lse)."""
    import torch

    def bits(x):
        if isinstance(x, torch.Tensor):
            return x.contiguous().view(torch.int16).numpy().view(np.uint16)
        return np.ascontiguousarray(x, dtype=np.uint16)
    q = bits(q_bf16)
    kv = bits(kv_bf16)
    qo = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    kvp = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    batch = qo.size - 1
    if seqs is None:
        sel, nsel, rows = None, batch, int(qo[-1] - qo[0])
    else:
        sel = np.ascontiguousarray(seqs, dtype=np.int32)
        nsel = sel.size
        rows = int(sum(int(qo[b + 1] - qo[b]) for b in sel))
    out = np.empty((rows, HEADS, DV), dtype=np.float64)
    lse = np.empty((rows, HEADS), dtype=np.float64)
    lo = hi = None
    if kv_lo is not None:
        lo = np.ascontiguousarray(kv_lo, dtype=np.int32)
        hi = np.ascontiguousarray(kv_hi, dtype=np.int32)
    if kv.size == 0:
        kv = np.zeros(DQK, dtype=np.uint16)
    n = lib().orc_mla_decode_bf16(
        _ptr(q, ctypes.c_uint16), _ptr(kv, ctypes.c_uint16), _ptr(qo, ctypes.c_int32),
        _ptr(kvp, ctypes.c_int32), batch, _ptr(sel, ctypes.c_int32) if sel is not None else None,
        nsel, _ptr(lo, ctypes.c_int32) if lo is not None else None,
        _ptr(hi, ctypes.c_int32) if hi is not None else None, sm_scale, logit_cap,
        _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if n < 0:
        raise ValueError("oracle rejected its arguments")
    return out, lse


def lse_merge(o_s: np.ndarray, lse_s: np.ndarray):
    o_s = np.ascontiguousarray(o_s, dtype=np.float64).reshape(-1, DV)
    lse_s = np.ascontiguousarray(lse_s, dtype=np.float64).reshape(-1)
    o = np.empty(DV, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    lib().orc_lse_merge(lse_s.size, _ptr(o_s, ctypes.c_double), _ptr(lse_s, ctypes.c_double),
                        _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    return o, float(lse[0])


def mla_decode(q8: np.ndarray, q_scale: float, kv: np.ndarray, kv_scale: float,
               qo_indptr, kv_indptr, sm_scale: float, kv_format: int = 0,
               kv_scales: np.ndarray | None = None, seqs=None, kv_lo=None, kv_hi=None,
               logit_cap: float = 0.0):
    """fp64 decode. kv_format 0: kv = (total_kv, 576) e4m3fn codes with kv_scale;
    1: kv = (total_kv, 288) packed e2m1 with kv_scales (total_kv, 18) e8m0;
    logit_cap > 0 soft-caps each scaled logit to cap * tanh(s / cap).
    Returns (out (rows, 16, 512), lse (rows, 16)) for the selected sequences."""
    q8 = np.ascontiguousarray(q8, dtype=np.uint8)
    kv = np.ascontiguousarray(kv, dtype=np.uint8)
    qo = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    kvp = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    batch = qo.size - 1
    if seqs is None:
        sel = None
        nsel = batch
        rows = int(qo[-1] - qo[0])
    else:
        sel = np.ascontiguousarray(seqs, dtype=np.int32)
        nsel = sel.size
        rows = int(sum(int(qo[b + 1] - qo[b]) for b in sel))
    out = np.empty((rows, HEADS, DV), dtype=np.float64)
    lse = np.empty((rows, HEADS), dtype=np.float64)
    ks = None
    if kv_format == 1:
        ks = np.ascontiguousarray(kv_scales, dtype=np.uint8)
    lo = hi = None
    if kv_lo is not None:
        lo = np.ascontiguousarray(kv_lo, dtype=np.int32)
        hi = np.ascontiguousarray(kv_hi, dtype=np.int32)
    n = lib().orc_mla_decode_cap(
        kv_format, _ptr(q8, ctypes.c_uint8), ctypes.c_float(q_scale), _ptr(kv, ctypes.c_uint8),
        _ptr(ks, ctypes.c_uint8) if ks is not None else None, ctypes.c_float(kv_scale),
        _ptr(qo, ctypes.c_int32), _ptr(kvp, ctypes.c_int32), batch,
        _ptr(sel, ctypes.c_int32) if sel is not None else None, nsel,
        _ptr(lo, ctypes.c_int32) if lo is not None else None,
        _ptr(hi, ctypes.c_int32) if hi is not None else None,
        sm_scale, float(logit_cap), _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if n < 0:
        raise ValueError("oracle rejected its arguments")
    assert n == rows
    return out, lse


def num_threads() -> int:
    return lib().orc_num_threads()
