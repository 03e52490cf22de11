"""Thin ctypes binding of libmla_decode.so (include/mla_decode.h).

Every function here has the name of the C entry point it wraps and does
argument marshalling only: torch tensors become ``data_ptr()`` values, the
current torch stream becomes the HIP stream, and a non-zero status becomes an
``MLADecodeError``. All computation happens in the library's HIP kernels.
PyTorch provides device memory and streams.

If the library has not been built, loading fails with an error that says so;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_decode.so")

MLA_OK = 0
MLA_KV_FP8_E4M3FN = 0
MLA_KV_MXFP4 = 1
MLA_KV_BF16 = 2
MLA_Q_SCALE_STATIC = 0
MLA_Q_SCALE_ABSMAX = 1
NUM_HEADS = 16
QK_DIM = 576
V_DIM = 512
MX_BLOCK = 32


class MLADecodeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {mla_status_string(status)} (status {status})")


_lib = None
_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                f"g.build()'` (or mla_latent_kv_bf16_amd/build.py)")
        # torch first: it loads its own HIP runtime, and the library's
        # libamdhip64 dependency must resolve to that same, already loaded
        # copy (the one that owns the streams and memory passed in). Loaded
        # first, the library would pull in the system's runtime and the
        # process would hold two, whose device calls then fail.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.mla_status_string.argtypes = [ctypes.c_int]
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_decode_plan.argtypes = [_i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp,
                                      ctypes.POINTER(_vp)]
        L.mla_decode_plan.restype = ctypes.c_int
        L.mla_decode_plan_host.argtypes = [_i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _i32p,
                                           ctypes.c_int32, _i32p, ctypes.c_int32, _i32p]
        L.mla_decode_plan_host.restype = ctypes.c_int
        L.mla_decode_plan_counts.argtypes = [_vp, _i32p]
        L.mla_decode_plan_counts.restype = ctypes.c_int
        L.mla_decode_plan_destroy.argtypes = [_vp]
        L.mla_decode_plan_destroy.restype = None
        L.mla_decode_workspace_size.argtypes = [_vp, ctypes.POINTER(ctypes.c_size_t)]
        L.mla_decode_workspace_size.restype = ctypes.c_int
        L.mla_decode_run.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp,
                                     ctypes.c_float, ctypes.c_float, _vp, ctypes.c_size_t, _vp,
                                     _vp, _vp]
        L.mla_decode_run.restype = ctypes.c_int
        L.mla_decode_run_fused.argtypes = L.mla_decode_run.argtypes
        L.mla_decode_run_fused.restype = ctypes.c_int
        L.mla_decode_run_fused_noalloc.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp,
                                                   _vp, ctypes.c_float, ctypes.c_float, _vp, _vp,
                                                   _vp]
        L.mla_decode_run_fused_noalloc.restype = ctypes.c_int
        L.mla_decode_run_bf16.argtypes = [_vp, _vp, _vp, ctypes.c_float, ctypes.c_float, _vp,
                                          ctypes.c_size_t, _vp, _vp, _vp]
        L.mla_decode_run_bf16.restype = ctypes.c_int
        L.mla_decode_run_bf16_paged.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_float,
                                                ctypes.c_float, _vp, ctypes.c_size_t, _vp, _vp,
                                                _vp]
        L.mla_decode_run_bf16_paged.restype = ctypes.c_int
        L.mla_decode_plan_paged.argtypes = [_i32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, _vp, ctypes.POINTER(_vp)]
        L.mla_decode_plan_paged.restype = ctypes.c_int
        for name in ("mla_decode_run_paged", "mla_decode_run_fused_paged"):
            f = getattr(L, name)
            f.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp,
                          ctypes.c_int32, ctypes.c_float, ctypes.c_float, _vp, ctypes.c_size_t,
                          _vp, _vp, _vp]
            f.restype = ctypes.c_int
        L.mla_decode_workspace_init.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
        L.mla_decode_workspace_init.restype = ctypes.c_int
        for name in ("mla_decode_attend", "mla_decode_stage1"):
            f = getattr(L, name)
            f.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, ctypes.c_float, _vp,
                          ctypes.c_size_t, _vp, _vp, _vp]
            f.restype = ctypes.c_int
        for name in ("mla_decode_attend_paged", "mla_decode_stage1_paged"):
            f = getattr(L, name)
            f.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_float,
                          ctypes.c_float, _vp, ctypes.c_size_t, _vp, _vp, _vp]
            f.restype = ctypes.c_int
        L.mla_decode_merge.argtypes = [_vp, _vp, ctypes.c_size_t, _vp, _vp, _vp]
        L.mla_decode_merge.restype = ctypes.c_int
        L.mla_quant_fp8_workspace_size.argtypes = [ctypes.c_size_t,
                                                   ctypes.POINTER(ctypes.c_size_t)]
        L.mla_quant_fp8_workspace_size.restype = ctypes.c_int
        L.mla_quant_fp8.argtypes = [_vp, ctypes.c_size_t, ctypes.c_int32, _vp, _vp, _vp,
                                    ctypes.c_size_t, _vp]
        L.mla_quant_fp8.restype = ctypes.c_int
        L.mla_encode_mxfp4.argtypes = [_vp, ctypes.c_size_t, _vp, _vp, _vp]
        L.mla_encode_mxfp4.restype = ctypes.c_int
        _lib = L
    return _lib


def mla_status_string(status: int) -> str:
    return lib().mla_status_string(status).decode()


def _check(status: int, what: str):
    if status != MLA_OK:
        raise MLADecodeError(status, what)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _host_i32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


MLA_INVALID_ARGUMENT = 1
# bytes per cache row by format (MXFP4: packed e2m1 pairs; the 18 e8m0
# block scales per row are a separate array)
_ROW_BYTES = {MLA_KV_FP8_E4M3FN: QK_DIM, MLA_KV_MXFP4: QK_DIM // 2, MLA_KV_BF16: 2 * QK_DIM}


def _buf(t, what: str, elem_bytes: int, numel: int, optional: bool = False):
    """Checks that t is a contiguous GPU tensor of at least numel elements of
    elem_bytes bytes each (the C ABI receives only its address), raising
    MLADecodeError(MLA_INVALID_ARGUMENT) otherwise; None passes if optional
    or if nothing is needed."""
    if t is None:
        if optional or numel == 0:
            return
        raise MLADecodeError(MLA_INVALID_ARGUMENT, f"{what} is missing")
    if not getattr(t, "is_cuda", False):
        raise MLADecodeError(MLA_INVALID_ARGUMENT, f"{what} is not a GPU tensor")
    if t.element_size() != elem_bytes:
        raise MLADecodeError(MLA_INVALID_ARGUMENT,
                             f"{what} has {t.element_size()}-byte elements, {elem_bytes} expected")
    if not t.is_contiguous():
        raise MLADecodeError(MLA_INVALID_ARGUMENT, f"{what} is not contiguous")
    if t.numel() < numel:
        raise MLADecodeError(MLA_INVALID_ARGUMENT,
                             f"{what} holds {t.numel()} elements, {numel} needed")


class Plan:
    """Owns an mla_plan_t; destroyed with the object (or by destroy()).

    Besides the counts it keeps what the run wrappers need to check buffer
    sizes: the cache format, the cache rows the plan reads (contiguous
    plans) and, for a paged plan, its page size and page-table length."""

    def __init__(self, handle: int, counts, kv_format: int = MLA_KV_FP8_E4M3FN,
                 total_kv: int = 0, page_size: int = 0, total_pages: int = 0):
        self.handle = handle
        # rows: query rows decoded (= sequences when every sequence has one)
        self.num_items, self.num_merges, self.num_slots, self.rows = (int(c) for c in counts)
        self.batch = self.rows
        self.kv_format = int(kv_format)
        self.total_kv = int(total_kv)
        self.page_size = int(page_size)
        self.total_pages = int(total_pages)
        size = ctypes.c_size_t()
        _check(lib().mla_decode_workspace_size(handle, ctypes.byref(size)),
               "mla_decode_workspace_size")
        self.workspace_bytes = size.value

    def destroy(self):
        if self.handle:
            lib().mla_decode_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def mla_decode_plan(qo_indptr, kv_indptr, kv_format: int = MLA_KV_FP8_E4M3FN,
                    num_heads: int = NUM_HEADS, num_cus: int = 0, max_splits: int = 0,
                    stream=None) -> Plan:
    """Host int32 CSR pointers (numpy / CPU tensor / list) -> Plan. The work
    lists are copied on `stream` (default: torch's current stream), which the
    call then waits for."""
    qo = _host_i32(qo_indptr)
    kv = _host_i32(kv_indptr)
    batch = qo.size - 1
    if kv.size != qo.size:
        raise ValueError("qo_indptr and kv_indptr must have the same length")
    h = _vp()
    _check(lib().mla_decode_plan(qo.ctypes.data_as(_i32p), kv.ctypes.data_as(_i32p), batch,
                                 num_heads, kv_format, num_cus, max_splits, _stream(stream),
                                 ctypes.byref(h)),
           "mla_decode_plan")
    counts = (ctypes.c_int32 * 4)()
    _check(lib().mla_decode_plan_counts(h, counts), "mla_decode_plan_counts")
    return Plan(h.value, list(counts), kv_format, total_kv=int(kv[-1]))


def mla_decode_plan_paged(qo_indptr, kv_page_indptr, kv_last_page_len, page_size: int,
                          kv_format: int = MLA_KV_FP8_E4M3FN, num_heads: int = NUM_HEADS,
                          num_cus: int = 0, max_splits: int = 0, stream=None) -> Plan:
    """Plan for a paged cache: host int32 query-row and page row pointers and
    the rows of each sequence's last page -> Plan."""
    qo = _host_i32(qo_indptr)
    pi = _host_i32(kv_page_indptr)
    last = _host_i32(kv_last_page_len)
    batch = qo.size - 1
    if pi.size != qo.size or last.size != batch:
        raise ValueError("qo_indptr / kv_page_indptr / kv_last_page_len sizes disagree")
    h = _vp()
    _check(lib().mla_decode_plan_paged(qo.ctypes.data_as(_i32p), pi.ctypes.data_as(_i32p),
                                       last.ctypes.data_as(_i32p), batch, page_size, num_heads,
                                       kv_format, num_cus, max_splits, _stream(stream),
                                       ctypes.byref(h)),
           "mla_decode_plan_paged")
    counts = (ctypes.c_int32 * 4)()
    _check(lib().mla_decode_plan_counts(h, counts), "mla_decode_plan_counts")
    return Plan(h.value, list(counts), kv_format, page_size=page_size, total_pages=int(pi[-1]))


def mla_decode_plan_host(qo_indptr, kv_indptr, kv_format: int = MLA_KV_FP8_E4M3FN,
                         num_heads: int = NUM_HEADS, num_cus: int = 0, max_splits: int = 0):
    """Host-only scheduler: returns (items (n, 4), merges (m, 4), num_slots)."""
    qo = _host_i32(qo_indptr)
    kv = _host_i32(kv_indptr)
    batch = qo.size - 1
    counts = np.zeros(3, dtype=np.int32)
    args = (qo.ctypes.data_as(_i32p), kv.ctypes.data_as(_i32p), batch, num_heads, kv_format,
            num_cus, max_splits)
    _check(lib().mla_decode_plan_host(*args, None, 0, None, 0, counts.ctypes.data_as(_i32p)),
           "mla_decode_plan_host")
    items = np.zeros((max(int(counts[0]), 1), 4), dtype=np.int32)
    merges = np.zeros((max(int(counts[1]), 1), 4), dtype=np.int32)
    _check(lib().mla_decode_plan_host(*args, items.ctypes.data_as(_i32p), items.shape[0],
                                      merges.ctypes.data_as(_i32p), merges.shape[0],
                                      counts.ctypes.data_as(_i32p)), "mla_decode_plan_host")
    return items[:counts[0]], merges[:counts[1]], int(counts[2])


def mla_decode_plan_destroy(plan: Plan):
    plan.destroy()


def mla_decode_workspace_size(plan: Plan) -> int:
    return plan.workspace_bytes


def _check_step(plan: Plan, q_bf16, q_fp8, q_scale, kv, kv_block_scales, kv_scale, out_bf16,
                lse_out, num_pages: int | None = None, kv_page_ids=None):
    """Buffer checks of one decode step against the plan (the workspace size
    is checked by the library, which is passed it)."""
    if plan.rows == 0:
        return
    nq = plan.rows * NUM_HEADS
    if q_bf16 is not None or q_fp8 is None:
        _buf(q_bf16, "q_bf16", 2, nq * QK_DIM)
    _buf(q_fp8, "q_fp8", 1, nq * QK_DIM, optional=plan.kv_format == MLA_KV_BF16)
    _buf(q_scale, "q_scale", 4, 1, optional=plan.kv_format == MLA_KV_BF16)
    if num_pages is None:
        _buf(kv, "kv", 2 if plan.kv_format == MLA_KV_BF16 else 1,
             plan.total_kv * _ROW_BYTES[plan.kv_format] // (2 if plan.kv_format == MLA_KV_BF16 else 1))
        if plan.kv_format == MLA_KV_MXFP4:
            _buf(kv_block_scales, "kv_block_scales", 1, plan.total_kv * (QK_DIM // MX_BLOCK))
    else:
        pool_rows = int(num_pages) * plan.page_size
        if plan.kv_format == MLA_KV_BF16:
            _buf(kv, "kv_pool", 2, pool_rows * QK_DIM)
        else:
            _buf(kv, "kv_pool", 1, pool_rows * _ROW_BYTES[plan.kv_format])
        if plan.kv_format == MLA_KV_MXFP4:
            _buf(kv_block_scales, "kv_block_scales", 1, pool_rows * (QK_DIM // MX_BLOCK))
        _buf(kv_page_ids, "kv_page_ids", 4, plan.total_pages)
    _buf(kv_scale, "kv_scale", 4, 1, optional=True)
    _buf(out_bf16, "out_bf16", 2, nq * V_DIM)
    _buf(lse_out, "lse_out", 4, nq, optional=True)


def mla_decode_run(plan: Plan, q_bf16, q_fp8, q_scale, kv, out_bf16, *, kv_scale=None,
                   kv_block_scales=None, q_scale_mode: int = MLA_Q_SCALE_ABSMAX,
                   sm_scale: float = 1.0 / 24.0, logit_cap: float = 0.0, workspace=None,
                   lse_out=None, stream=None, check: bool = True):
    """check=False skips the buffer checks (for a loop over buffers already
    checked once)."""
    if check:
        _check_step(plan, q_bf16, q_fp8, q_scale, kv, kv_block_scales, kv_scale, out_bf16,
                    lse_out)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_decode_run(plan.handle, _ptr(q_bf16), _ptr(q_fp8), _ptr(q_scale),
                                q_scale_mode, _ptr(kv), _ptr(kv_block_scales), _ptr(kv_scale),
                                sm_scale, logit_cap, _ptr(workspace), ws_bytes, _ptr(out_bf16),
                                _ptr(lse_out), _stream(stream)), "mla_decode_run")


def mla_decode_run_fused(plan: Plan, q_bf16, q_fp8, q_scale, kv, out_bf16, *, kv_scale=None,
                         kv_block_scales=None, q_scale_mode: int = MLA_Q_SCALE_ABSMAX,
                         sm_scale: float = 1.0 / 24.0, logit_cap: float = 0.0, workspace=None,
                         lse_out=None, stream=None, check: bool = True):
    if check:
        _check_step(plan, q_bf16, q_fp8, q_scale, kv, kv_block_scales, kv_scale, out_bf16,
                    lse_out)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_decode_run_fused(plan.handle, _ptr(q_bf16), _ptr(q_fp8), _ptr(q_scale),
                                      q_scale_mode, _ptr(kv), _ptr(kv_block_scales),
                                      _ptr(kv_scale), sm_scale, logit_cap, _ptr(workspace),
                                      ws_bytes, _ptr(out_bf16), _ptr(lse_out), _stream(stream)),
           "mla_decode_run_fused")


def mla_decode_run_fused_noalloc(plan: Plan, q_bf16, q_fp8, q_scale, kv, out_bf16, *,
                                 kv_scale=None, kv_block_scales=None,
                                 q_scale_mode: int = MLA_Q_SCALE_ABSMAX,
                                 sm_scale: float = 1.0 / 24.0, logit_cap: float = 0.0,
                                 lse_out=None, stream=None, check: bool = True):
    """mla_decode_run_fused with the library's fixed per-device scratch as
    its workspace (no workspace argument, nothing allocated)."""
    if check:
        _check_step(plan, q_bf16, q_fp8, q_scale, kv, kv_block_scales, kv_scale, out_bf16,
                    lse_out)
    _check(lib().mla_decode_run_fused_noalloc(plan.handle, _ptr(q_bf16), _ptr(q_fp8),
                                              _ptr(q_scale), q_scale_mode, _ptr(kv),
                                              _ptr(kv_block_scales), _ptr(kv_scale), sm_scale,
                                              logit_cap, _ptr(out_bf16), _ptr(lse_out),
                                              _stream(stream)),
           "mla_decode_run_fused_noalloc")


def _run_paged(name, plan, q_bf16, q_fp8, q_scale, kv_pool, kv_page_ids, num_pages, out_bf16,
               kv_scale, q_scale_mode, sm_scale, workspace, lse_out, stream, check=True,
               logit_cap=0.0, kv_block_scales=None):
    if check:
        _check_step(plan, q_bf16, q_fp8, q_scale, kv_pool, kv_block_scales, kv_scale, out_bf16,
                    lse_out, num_pages=max(int(num_pages), 0), kv_page_ids=kv_page_ids)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(getattr(lib(), name)(plan.handle, _ptr(q_bf16), _ptr(q_fp8), _ptr(q_scale),
                                q_scale_mode, _ptr(kv_pool), _ptr(kv_block_scales),
                                _ptr(kv_scale), _ptr(kv_page_ids),
                                num_pages, sm_scale, logit_cap, _ptr(workspace), ws_bytes,
                                _ptr(out_bf16), _ptr(lse_out), _stream(stream)), name)


def mla_decode_run_paged(plan: Plan, q_bf16, q_fp8, q_scale, kv_pool, kv_page_ids,
                         num_pages: int, out_bf16, *, kv_scale=None, kv_block_scales=None,
                         q_scale_mode: int = MLA_Q_SCALE_ABSMAX, sm_scale: float = 1.0 / 24.0,
                         logit_cap: float = 0.0, workspace=None, lse_out=None, stream=None,
                         check: bool = True):
    """kv_block_scales: the MXFP4 pool's (rows, 18) E8M0 scales (None for FP8)."""
    _run_paged("mla_decode_run_paged", plan, q_bf16, q_fp8, q_scale, kv_pool, kv_page_ids,
               num_pages, out_bf16, kv_scale, q_scale_mode, sm_scale, workspace, lse_out, stream,
               check, logit_cap, kv_block_scales)


def mla_decode_run_fused_paged(plan: Plan, q_bf16, q_fp8, q_scale, kv_pool, kv_page_ids,
                               num_pages: int, out_bf16, *, kv_scale=None, kv_block_scales=None,
                               q_scale_mode: int = MLA_Q_SCALE_ABSMAX,
                               sm_scale: float = 1.0 / 24.0, logit_cap: float = 0.0,
                               workspace=None, lse_out=None, stream=None, check: bool = True):
    _run_paged("mla_decode_run_fused_paged", plan, q_bf16, q_fp8, q_scale, kv_pool, kv_page_ids,
               num_pages, out_bf16, kv_scale, q_scale_mode, sm_scale, workspace, lse_out, stream,
               check, logit_cap, kv_block_scales)


def mla_decode_run_bf16(plan: Plan, q_bf16, kv_bf16, out_bf16, *, sm_scale: float = 1.0 / 24.0,
                        logit_cap: float = 0.0, workspace=None, lse_out=None, stream=None,
                        check: bool = True):
    if check:
        _check_step(plan, q_bf16, None, None, kv_bf16, None, None, out_bf16, lse_out)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_decode_run_bf16(plan.handle, _ptr(q_bf16), _ptr(kv_bf16), sm_scale,
                                     logit_cap, _ptr(workspace), ws_bytes, _ptr(out_bf16),
                                     _ptr(lse_out), _stream(stream)), "mla_decode_run_bf16")


def mla_decode_run_bf16_paged(plan: Plan, q_bf16, kv_pool, kv_page_ids, num_pages: int,
                              out_bf16, *, sm_scale: float = 1.0 / 24.0, logit_cap: float = 0.0,
                              workspace=None, lse_out=None, stream=None, check: bool = True):
    """mla_decode_run_bf16 on a paged bf16 pool: kv_pool (num_pages * page_size,
    576) bf16, kv_page_ids device int32 indexed by the plan's page row pointers."""
    if check:
        _check_step(plan, q_bf16, None, None, kv_pool, None, None, out_bf16, lse_out,
                    num_pages=max(int(num_pages), 0), kv_page_ids=kv_page_ids)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_decode_run_bf16_paged(plan.handle, _ptr(q_bf16), _ptr(kv_pool),
                                           _ptr(kv_page_ids), num_pages, sm_scale, logit_cap,
                                           _ptr(workspace), ws_bytes, _ptr(out_bf16),
                                           _ptr(lse_out), _stream(stream)),
           "mla_decode_run_bf16_paged")


def mla_decode_workspace_init(plan: Plan, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_decode_workspace_init(plan.handle, _ptr(workspace), ws_bytes,
                                           _stream(stream)), "mla_decode_workspace_init")


def _attend_like(name, plan, q_fp8, q_scale, kv, out_bf16, kv_scale, kv_block_scales,
                 sm_scale, workspace, lse_out, stream, check=True, logit_cap=0.0):
    if check:
        _check_step(plan, None, q_fp8, q_scale, kv, kv_block_scales, kv_scale, out_bf16, lse_out)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(getattr(lib(), name)(plan.handle, _ptr(q_fp8), _ptr(q_scale), _ptr(kv),
                                _ptr(kv_block_scales), _ptr(kv_scale), sm_scale, logit_cap,
                                _ptr(workspace), ws_bytes, _ptr(out_bf16), _ptr(lse_out),
                                _stream(stream)), name)


def mla_decode_attend(plan: Plan, q_fp8, q_scale, kv, out_bf16, *, kv_scale=None,
                      kv_block_scales=None, sm_scale: float = 1.0 / 24.0, logit_cap: float = 0.0,
                      workspace=None, lse_out=None, stream=None, check: bool = True):
    _attend_like("mla_decode_attend", plan, q_fp8, q_scale, kv, out_bf16, kv_scale,
                 kv_block_scales, sm_scale, workspace, lse_out, stream, check, logit_cap)


def mla_decode_stage1(plan: Plan, q_fp8, q_scale, kv, out_bf16, *, kv_scale=None,
                      kv_block_scales=None, sm_scale: float = 1.0 / 24.0, logit_cap: float = 0.0,
                      workspace=None, lse_out=None, stream=None, check: bool = True):
    _attend_like("mla_decode_stage1", plan, q_fp8, q_scale, kv, out_bf16, kv_scale,
                 kv_block_scales, sm_scale, workspace, lse_out, stream, check, logit_cap)


def _attend_like_paged(name, plan, q_fp8, q_scale, kv_pool, kv_page_ids, num_pages, out_bf16,
                       kv_scale, kv_block_scales, sm_scale, logit_cap, workspace, lse_out, stream,
                       check):
    if check:
        _check_step(plan, None, q_fp8, q_scale, kv_pool, kv_block_scales, kv_scale, out_bf16,
                    lse_out, num_pages=max(int(num_pages), 0), kv_page_ids=kv_page_ids)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(getattr(lib(), name)(plan.handle, _ptr(q_fp8), _ptr(q_scale), _ptr(kv_pool),
                                _ptr(kv_block_scales), _ptr(kv_scale), _ptr(kv_page_ids),
                                num_pages, sm_scale, logit_cap, _ptr(workspace), ws_bytes,
                                _ptr(out_bf16), _ptr(lse_out), _stream(stream)), name)


def mla_decode_attend_paged(plan: Plan, q_fp8, q_scale, kv_pool, kv_page_ids, num_pages: int,
                            out_bf16, *, kv_scale=None, kv_block_scales=None,
                            sm_scale: float = 1.0 / 24.0, logit_cap: float = 0.0,
                            workspace=None, lse_out=None, stream=None, check: bool = True):
    """mla_decode_attend on a paged pool (arguments as mla_decode_run_paged)."""
    _attend_like_paged("mla_decode_attend_paged", plan, q_fp8, q_scale, kv_pool, kv_page_ids,
                       num_pages, out_bf16, kv_scale, kv_block_scales, sm_scale, logit_cap,
                       workspace, lse_out, stream, check)


def mla_decode_stage1_paged(plan: Plan, q_fp8, q_scale, kv_pool, kv_page_ids, num_pages: int,
                            out_bf16, *, kv_scale=None, kv_block_scales=None,
                            sm_scale: float = 1.0 / 24.0, logit_cap: float = 0.0,
                            workspace=None, lse_out=None, stream=None, check: bool = True):
    """mla_decode_stage1 on a paged pool (arguments as mla_decode_run_paged)."""
    _attend_like_paged("mla_decode_stage1_paged", plan, q_fp8, q_scale, kv_pool, kv_page_ids,
                       num_pages, out_bf16, kv_scale, kv_block_scales, sm_scale, logit_cap,
                       workspace, lse_out, stream, check)


def mla_decode_merge(plan: Plan, workspace, out_bf16, lse_out=None, stream=None):
    if plan.rows:
        _buf(out_bf16, "out_bf16", 2, plan.rows * NUM_HEADS * V_DIM)
        _buf(lse_out, "lse_out", 4, plan.rows * NUM_HEADS, optional=True)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_decode_merge(plan.handle, _ptr(workspace), ws_bytes, _ptr(out_bf16),
                                  _ptr(lse_out), _stream(stream)), "mla_decode_merge")


def mla_quant_fp8_workspace_size(n: int) -> int:
    size = ctypes.c_size_t()
    _check(lib().mla_quant_fp8_workspace_size(n, ctypes.byref(size)),
           "mla_quant_fp8_workspace_size")
    return size.value


def mla_quant_fp8(x_bf16, out_fp8, scale, scale_mode: int = MLA_Q_SCALE_ABSMAX, workspace=None,
                  stream=None):
    if x_bf16.numel():
        _buf(x_bf16, "x_bf16", 2, x_bf16.numel())
        _buf(out_fp8, "out_fp8", 1, x_bf16.numel())
    _buf(scale, "scale", 4, 1)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_quant_fp8(_ptr(x_bf16), x_bf16.numel(), scale_mode, _ptr(scale),
                               _ptr(out_fp8), _ptr(workspace), ws_bytes, _stream(stream)),
           "mla_quant_fp8")


def mla_encode_mxfp4(x_bf16, packed, block_scales, stream=None):
    if x_bf16.numel() % QK_DIM:
        raise MLADecodeError(MLA_INVALID_ARGUMENT, "x_bf16 is not a whole number of 576-dim rows")
    rows = x_bf16.numel() // QK_DIM
    if rows:
        _buf(x_bf16, "x_bf16", 2, rows * QK_DIM)
        _buf(packed, "packed", 1, rows * (QK_DIM // 2))
        _buf(block_scales, "block_scales", 1, rows * (QK_DIM // MX_BLOCK))
    _check(lib().mla_encode_mxfp4(_ptr(x_bf16), rows, _ptr(packed), _ptr(block_scales),
                                  _stream(stream)), "mla_encode_mxfp4")
