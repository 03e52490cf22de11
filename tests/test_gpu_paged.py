"""GPU parity of the paged FP8, MXFP4 and bf16 caches: sequences' rows
scattered over a pool of pages in a seeded random order. The paged path is checked against the
oracle on the gathered rows, and (one query row per sequence) bit for bit
against the contiguous path run on the same codes gathered in order."""
import numpy as np
import pytest
import torch

import mla_latent_kv_bf16_amd as mla
import oracle
import workloads
from gpu_cases import DEV, announce, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu
SM = workloads.SM_SCALE


class PagedCase:
    def __init__(self, kv_lens, q_lens, page_size, seed, q_mode="absmax", max_splits=0,
                 fmt="fp8", num_cus=0):
        self.kv_lens, self.page_size, self.fmt = kv_lens, page_size, fmt
        self.qo, self.kvp = workloads.indptrs(kv_lens, q_lens)
        self.rows = int(self.qo[-1])
        (self.pi, self.ids, self.last, self.num_pages,
         self.row_of_token) = workloads.make_page_table(kv_lens, page_size, seed)
        self.q = workloads.make_q(self.rows, seed + 1)
        kv = workloads.make_kv(kv_lens, seed + 2)
        pool = workloads.randn_bf16((self.num_pages * page_size, 576), seed + 3)
        if kv.shape[0]:
            pool[torch.from_numpy(self.row_of_token)] = kv
        self.pool = pool
        self.q_mode = q_mode
        self.kv_format = {"fp8": mla.MLA_KV_FP8_E4M3FN, "mxfp4": mla.MLA_KV_MXFP4,
                          "bf16": mla.MLA_KV_BF16}[fmt]
        self.plan = mla.mla_decode_plan_paged(self.qo, self.pi, self.last, page_size,
                                              kv_format=self.kv_format, max_splits=max_splits,
                                              num_cus=num_cus)
        assert self.plan.rows == self.rows

    def run(self, fused, ids=None, logit_cap=0.0):
        poold = self.pool.to(DEV)
        if self.fmt == "bf16":
            codes, ks, bs = poold, None, None
        elif self.fmt == "fp8":
            codes = torch.empty(poold.shape, dtype=torch.uint8, device=DEV)
            ks = torch.empty(1, dtype=torch.float32, device=DEV)
            qws = torch.empty(mla.mla_quant_fp8_workspace_size(poold.numel()),
                              dtype=torch.uint8, device=DEV)
            mla.mla_quant_fp8(poold, codes, ks, mla.MLA_Q_SCALE_ABSMAX, qws)
            bs = None
        else:
            codes = torch.empty((poold.shape[0], 288), dtype=torch.uint8, device=DEV)
            bs = torch.empty((poold.shape[0], 18), dtype=torch.uint8, device=DEV)
            mla.mla_encode_mxfp4(poold, codes, bs)
            ks = None
        self.codes, self.kv_scale, self.block_scales = codes, ks, bs
        ws = torch.zeros(max(self.plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
        mla.mla_decode_workspace_init(self.plan, ws)
        r = max(self.rows, 1)
        q8 = torch.empty((r, 16, 576), dtype=torch.uint8, device=DEV)
        qs = torch.full((1,), 6.0 / 448.0, dtype=torch.float32, device=DEV)
        out = torch.empty((r, 16, 512), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((r, 16), dtype=torch.float32, device=DEV)
        idsd = torch.from_numpy(self.ids if ids is None else ids).to(DEV)
        mode = mla.MLA_Q_SCALE_STATIC if self.q_mode == "static" else mla.MLA_Q_SCALE_ABSMAX
        if self.fmt == "bf16":  # one launch, no Q codes
            mla.mla_decode_run_bf16_paged(self.plan, self.q.to(DEV), codes, idsd, self.num_pages,
                                          out, sm_scale=SM, logit_cap=logit_cap, workspace=ws,
                                          lse_out=lse)
        else:
            fn = mla.mla_decode_run_fused_paged if fused else mla.mla_decode_run_paged
            fn(self.plan, self.q.to(DEV), q8, qs, codes, idsd, self.num_pages, out, kv_scale=ks,
               kv_block_scales=bs, q_scale_mode=mode, logit_cap=logit_cap, workspace=ws,
               lse_out=lse)
        torch.cuda.synchronize()
        return (out.float().cpu().numpy()[:self.rows], lse.cpu().numpy()[:self.rows],
                q8.cpu().numpy()[:self.rows], float(qs.item()))

    def oracle(self, ids=None, logit_cap=0.0):
        """The oracle on the sequences' rows gathered from the pool (rows of a
        page id outside the pool are zero codes, and zero scale bytes in the
        MXFP4 cache). Returns (out, lse, q8, gathered codes, gathered block
        scales or None, kv scale)."""
        rows = self.row_of_token if ids is None else self._rows_for(ids)
        if self.fmt == "bf16":
            ok = (rows >= 0) & (rows < self.pool.shape[0])
            gathered = torch.zeros((rows.size, 576), dtype=torch.bfloat16)
            if ok.any():
                dst = torch.from_numpy(np.nonzero(ok)[0])
                gathered[dst] = self.pool[torch.from_numpy(rows[ok])]
            out, lse = oracle.mla_decode_bf16(self.q, gathered, self.qo, self.kvp, SM, logit_cap)
            return out, lse, None, gathered, None, None
        qs = (oracle.fp8_static_scale() if self.q_mode == "static"
              else oracle.fp8_absmax_scale(self.q))
        q8 = oracle.fp8_quantize(self.q, qs)
        if self.fmt == "fp8":
            ks = oracle.fp8_absmax_scale(self.pool)
            pool_codes, pool_scales = oracle.fp8_quantize(self.pool, ks), None
        else:
            ks = 0.0
            pool_codes, pool_scales = oracle.mxfp4_encode(self.pool)
        ok = (rows >= 0) & (rows < pool_codes.shape[0])
        gathered = np.zeros((rows.size, pool_codes.shape[1]), dtype=np.uint8)
        gathered[ok] = pool_codes[rows[ok]]
        gscales = None
        if pool_scales is not None:
            gscales = np.zeros((rows.size, pool_scales.shape[1]), dtype=np.uint8)
            gscales[ok] = pool_scales[rows[ok]]
        out, lse = oracle.mla_decode(q8, qs, gathered, ks, self.qo, self.kvp, SM,
                                     kv_format=0 if self.fmt == "fp8" else 1,
                                     kv_scales=gscales, logit_cap=logit_cap)
        return out, lse, q8, gathered, gscales, ks

    def _rows_for(self, ids):
        P = self.page_size
        rows = []
        for b, n in enumerate(self.kv_lens):
            t = np.arange(n, dtype=np.int64)
            rows.append(ids[self.pi[b] + t // P].astype(np.int64) * P + t % P)
        return np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)


CASES = [
    ([1000, 0, 37, 513], None, 1),
    ([1000, 0, 37, 513], None, 16),
    ([1000, 0, 37, 513], None, 32),
    ([1000, 0, 37, 513], None, 64),
    ([3000, 5, 64, 65], None, 256),
    ([700, 31, 32, 33], [1, 2, 3, 4], 16),
    ([700, 31, 32, 33], [2, 1, 4, 3], 128),
]


@pytest.mark.parametrize("fused", [False, True], ids=["three_launches", "fused"])
@pytest.mark.parametrize("q_mode", ["absmax", "static"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"P{c[2]}_{'-'.join(map(str, c[0]))}"
                         f"{'_rows' if c[1] else ''}")
def test_paged_against_oracle(case, q_mode, fused):
    kv_lens, q_lens, P = case
    announce(f"paged P{P} {kv_lens} rows {q_lens} {q_mode} fused={fused}")
    c = PagedCase(kv_lens, q_lens, P, 600 + P, q_mode)
    got, lse, q8, _ = c.run(fused)
    ref, ref_lse, q8_ref, _, _, _ = c.oracle()
    assert np.array_equal(q8, q8_ref)
    assert_close(got, ref, f"paged P{P}")
    assert_lse_close(lse, ref_lse, f"paged P{P}")


# FP8 pages with 1-4 query rows per sequence: the rows share each cache tile
# (the shared-row kernel on a paged cache; below 32 rows per page a tile
# gathers its rows page by page)
ROWS_CASES = [
    ([700, 31, 32, 33], [2, 1, 4, 3], 32),
    ([1000, 0, 37, 513], [4, 4, 1, 2], 64),
    ([2048, 96], [3, 3], 256),
    ([700, 31, 32, 33], [2, 1, 4, 3], 1),
    ([1000, 0, 37, 513], [4, 4, 1, 2], 4),
    ([2048, 96, 5], [3, 2, 4], 16),
]


@pytest.mark.parametrize("fused", [False, True], ids=["three_launches", "fused"])
@pytest.mark.parametrize("q_mode", ["absmax", "static"])
@pytest.mark.parametrize("case", ROWS_CASES, ids=lambda c: f"P{c[2]}_{'-'.join(map(str, c[0]))}")
def test_paged_shared_rows_against_oracle(case, q_mode, fused):
    kv_lens, q_lens, P = case
    announce(f"paged shared rows P{P} {kv_lens} rows {q_lens} {q_mode} fused={fused}")
    c = PagedCase(kv_lens, q_lens, P, 680 + P, q_mode)
    got, lse, q8, _ = c.run(fused)
    ref, ref_lse, q8_ref, _, _, _ = c.oracle()
    assert np.array_equal(q8, q8_ref)
    assert_close(got, ref, f"paged rows P{P}")
    assert_lse_close(lse, ref_lse, f"paged rows P{P}")


@pytest.mark.parametrize("fmt,P", [("fp8", 1), ("fp8", 8), ("fp8", 32), ("fp8", 128),
                                   ("mxfp4", 2), ("mxfp4", 8), ("mxfp4", 16), ("mxfp4", 32),
                                   ("mxfp4", 128)])
def test_paged_shared_rows_equal_contiguous_bitwise(fmt, P):
    """The paged plan takes the shared-row schedule of the contiguous plan
    (same items) and its outputs equal the contiguous run's bit for bit (both
    planned for 8 compute units, so that MXFP4 takes the shared rows too)."""
    kv_lens, q_lens = [2000, 1, 300, 4097], [2, 4, 1, 3]
    announce(f"paged shared rows vs contiguous {fmt} P{P}")
    c = PagedCase(kv_lens, q_lens, P, 740 + P, "static", max_splits=-3, fmt=fmt, num_cus=8)
    got = c.run(True)
    _, _, _, gathered, gscales, _ = c.oracle()
    plan = mla.mla_decode_plan(c.qo, c.kvp, c.kv_format, max_splits=-3, num_cus=8)
    shared = mla.mla_decode_plan(c.qo, c.kvp, mla.MLA_KV_FP8_E4M3FN, max_splits=-3, num_cus=8)
    assert plan.num_items == shared.num_items  # the shared-row schedule
    assert (plan.num_items, plan.num_merges, plan.num_slots) == (
        c.plan.num_items, c.plan.num_merges, c.plan.num_slots)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    mla.mla_decode_workspace_init(plan, ws)
    q8 = torch.empty((c.rows, 16, 576), dtype=torch.uint8, device=DEV)
    qs = torch.full((1,), 6.0 / 448.0, dtype=torch.float32, device=DEV)
    out = torch.empty((c.rows, 16, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((c.rows, 16), dtype=torch.float32, device=DEV)
    mla.mla_decode_run_fused(plan, c.q.to(DEV), q8, qs, torch.from_numpy(gathered).to(DEV), out,
                             kv_scale=c.kv_scale,
                             kv_block_scales=None if gscales is None
                             else torch.from_numpy(gscales).to(DEV),
                             q_scale_mode=mla.MLA_Q_SCALE_STATIC, workspace=ws, lse_out=lse)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy().view(np.uint32), got[0].view(np.uint32))
    assert np.array_equal(lse.cpu().numpy().view(np.uint32), got[1].view(np.uint32))


# MXFP4 pages of any size (below 32 rows gathered page by page; below 8 each
# row's 18 scale bytes come in as 5 dwords)
MX_CASES = [
    ([1000, 0, 37, 513], None, 1),
    ([700, 31, 32, 33], [1, 2, 3, 4], 2),
    ([3000, 5, 64, 65], None, 4),
    ([1000, 0, 37, 513], None, 8),
    ([700, 31, 32, 33], [1, 2, 3, 4], 16),
    ([1000, 0, 37, 513], None, 32),
    ([1000, 0, 37, 513], None, 64),
    ([3000, 5, 64, 65], None, 256),
    ([700, 31, 32, 33], [2, 1, 4, 3], 128),
]


@pytest.mark.parametrize("fused", [False, True], ids=["three_launches", "fused"])
@pytest.mark.parametrize("q_mode", ["absmax", "static"])
@pytest.mark.parametrize("case", MX_CASES, ids=lambda c: f"P{c[2]}_{'-'.join(map(str, c[0]))}"
                         f"{'_rows' if c[1] else ''}")
def test_paged_mxfp4_against_oracle(case, q_mode, fused):
    kv_lens, q_lens, P = case
    announce(f"paged mxfp4 P{P} {kv_lens} rows {q_lens} {q_mode} fused={fused}")
    c = PagedCase(kv_lens, q_lens, P, 650 + P, q_mode, fmt="mxfp4")
    got, lse, q8, _ = c.run(fused)
    ref, ref_lse, q8_ref, _, _, _ = c.oracle()
    assert np.array_equal(q8, q8_ref)
    assert_close(got, ref, f"paged mxfp4 P{P}")
    assert_lse_close(lse, ref_lse, f"paged mxfp4 P{P}")


# MXFP4 shared rows on pages (planned for 8 compute units: the per-row
# schedule would then take several rounds, so the rows share each tile)
MX_ROWS_CASES = [
    ([700, 31, 32, 33], [2, 1, 4, 3], 1),
    ([700, 31, 32, 33], [2, 1, 4, 3], 8),
    ([1000, 0, 37, 513], [4, 4, 1, 2], 16),
    ([2048, 96, 5], [3, 2, 4], 64),
]


@pytest.mark.parametrize("fused", [False, True], ids=["three_launches", "fused"])
@pytest.mark.parametrize("q_mode", ["absmax", "static"])
@pytest.mark.parametrize("case", MX_ROWS_CASES, ids=lambda c: f"P{c[2]}_{'-'.join(map(str, c[0]))}")
def test_paged_mxfp4_shared_rows_against_oracle(case, q_mode, fused):
    kv_lens, q_lens, P = case
    announce(f"paged mxfp4 shared rows P{P} {kv_lens} rows {q_lens} {q_mode} fused={fused}")
    c = PagedCase(kv_lens, q_lens, P, 760 + P, q_mode, fmt="mxfp4", num_cus=8)
    got, lse, q8, _ = c.run(fused)
    ref, ref_lse, q8_ref, _, _, _ = c.oracle()
    assert np.array_equal(q8, q8_ref)
    assert_close(got, ref, f"paged mxfp4 rows P{P}")
    assert_lse_close(lse, ref_lse, f"paged mxfp4 rows P{P}")


# bf16 pages of any size: below 16 rows a tile gathers its rows page by page
BF_CASES = [
    ([1000, 0, 37, 513], None, 1),
    ([1000, 0, 37, 513], None, 8),
    ([1000, 0, 37, 513], None, 16),
    ([3000, 5, 64, 65], None, 64),
    ([700, 31, 32, 33], [2, 1, 4, 3], 4),
]


@pytest.mark.parametrize("cap", [0.0, 2.0])
@pytest.mark.parametrize("case", BF_CASES, ids=lambda c: f"P{c[2]}_{'-'.join(map(str, c[0]))}"
                         f"{'_rows' if c[1] else ''}")
def test_paged_bf16_against_oracle(case, cap):
    kv_lens, q_lens, P = case
    announce(f"paged bf16 P{P} {kv_lens} rows {q_lens} cap {cap}")
    c = PagedCase(kv_lens, q_lens, P, 670 + P, fmt="bf16")
    got, lse, _, _ = c.run(True, logit_cap=cap)
    ref, ref_lse, _, _, _, _ = c.oracle(logit_cap=cap)
    assert_close(got, ref, f"paged bf16 P{P}")
    assert_lse_close(lse, ref_lse, f"paged bf16 P{P}")


@pytest.mark.parametrize("P", [1, 4, 16, 256])
def test_paged_bf16_equals_contiguous_bitwise(P):
    kv_lens = [2000, 1, 300, 4097]
    announce(f"paged bf16 vs contiguous P{P}")
    c = PagedCase(kv_lens, None, P, 720 + P, max_splits=-3, fmt="bf16")
    got = c.run(True)
    _, _, _, gathered, _, _ = c.oracle()
    plan = mla.mla_decode_plan(c.qo, c.kvp, mla.MLA_KV_BF16, max_splits=-3)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    mla.mla_decode_workspace_init(plan, ws)
    out = torch.empty((c.rows, 16, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((c.rows, 16), dtype=torch.float32, device=DEV)
    mla.mla_decode_run_bf16(plan, c.q.to(DEV), gathered.to(DEV), out, sm_scale=SM, workspace=ws,
                            lse_out=lse)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy().view(np.uint32), got[0].view(np.uint32))
    assert np.array_equal(lse.cpu().numpy().view(np.uint32), got[1].view(np.uint32))


@pytest.mark.parametrize("fmt,P", [("fp8", 1), ("fp8", 8), ("fp8", 32), ("fp8", 128),
                                   ("mxfp4", 1), ("mxfp4", 2), ("mxfp4", 4), ("mxfp4", 8),
                                   ("mxfp4", 16), ("mxfp4", 32), ("mxfp4", 512)])
def test_paged_equals_contiguous_bitwise(fmt, P):
    """One query row per sequence: the paged kernel reads the same bytes in
    the same order as the contiguous one on the gathered cache."""
    kv_lens = [2000, 1, 300, 4097]
    announce(f"paged vs contiguous {fmt} P{P}")
    c = PagedCase(kv_lens, None, P, 700 + P, "static", max_splits=-3, fmt=fmt)
    got = c.run(True)
    _, _, _, gathered, gscales, _ = c.oracle()
    plan = mla.mla_decode_plan(c.qo, c.kvp, c.kv_format, max_splits=-3)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    mla.mla_decode_workspace_init(plan, ws)
    kvd = torch.from_numpy(gathered).to(DEV)
    bsd = None if gscales is None else torch.from_numpy(gscales).to(DEV)
    q8 = torch.empty((c.rows, 16, 576), dtype=torch.uint8, device=DEV)
    qs = torch.full((1,), 6.0 / 448.0, dtype=torch.float32, device=DEV)
    out = torch.empty((c.rows, 16, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((c.rows, 16), dtype=torch.float32, device=DEV)
    mla.mla_decode_run_fused(plan, c.q.to(DEV), q8, qs, kvd, out, kv_scale=c.kv_scale,
                             kv_block_scales=bsd, q_scale_mode=mla.MLA_Q_SCALE_STATIC,
                             workspace=ws, lse_out=lse)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy().view(np.uint32), got[0].view(np.uint32))
    assert np.array_equal(lse.cpu().numpy().view(np.uint32), got[1].view(np.uint32))


@pytest.mark.parametrize("fmt,P", [("fp8", 4), ("fp8", 64), ("mxfp4", 1), ("mxfp4", 4),
                                   ("mxfp4", 16), ("mxfp4", 64), ("bf16", 2), ("bf16", 32)])
def test_paged_ids_outside_the_pool_read_zeros(fmt, P):
    """Page ids past the pool (or negative) read as zero codes, no fault."""
    kv_lens = [300, 90]
    announce(f"paged bad ids {fmt} P{P}")
    c = PagedCase(kv_lens, None, P, 800 + P, "static", fmt=fmt)
    ids = c.ids.copy()
    ids[1] = c.num_pages + 5
    ids[-1] = -7
    got = c.run(False, ids=ids)
    ref, ref_lse, _, _, _, _ = c.oracle(ids=ids)
    assert_close(got[0], ref, "bad ids")
    assert_lse_close(got[1], ref_lse, "bad ids")


def test_paged_argument_errors():
    announce("paged argument errors")
    qo, pi = np.array([0, 1], np.int32), np.array([0, 2], np.int32)
    with pytest.raises(mla.MLADecodeError) as e:          # no such cache format
        mla.mla_decode_plan_paged(qo, pi, np.array([3], np.int32), 4, kv_format=7)
    assert e.value.status == 1
    bfp = mla.mla_decode_plan_paged(qo, pi, np.array([3], np.int32), 32,
                                    kv_format=mla.MLA_KV_BF16)
    bws = torch.zeros(max(bfp.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    bq = torch.zeros((1, 16, 576), dtype=torch.bfloat16, device=DEV)
    bkv = torch.zeros((64, 576), dtype=torch.bfloat16, device=DEV)
    bout = torch.empty((1, 16, 512), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mla.MLADecodeError) as e:          # a paged bf16 plan needs its own run
        mla.mla_decode_run_bf16(bfp, bq, bkv, bout, workspace=bws)
    assert e.value.status == 1
    bids = torch.zeros(2, dtype=torch.int32, device=DEV)
    bflat = mla.mla_decode_plan(qo, np.array([0, 20], np.int32), mla.MLA_KV_BF16)
    with pytest.raises(mla.MLADecodeError) as e:          # ... which takes no contiguous plan
        mla.mla_decode_run_bf16_paged(bflat, bq, bkv, bids, 2, bout, workspace=bws)
    assert e.value.status == 1
    for last in (0, 17):                                   # last page length out of range
        with pytest.raises(mla.MLADecodeError) as e:
            mla.mla_decode_plan_paged(qo, pi, np.array([last], np.int32), 16)
        assert e.value.status == 1
    with pytest.raises(mla.MLADecodeError) as e:           # page size not a power of two
        mla.mla_decode_plan_paged(qo, pi, np.array([3], np.int32), 24)
    assert e.value.status == 1
    plan = mla.mla_decode_plan_paged(qo, pi, np.array([3], np.int32), 16)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    q = torch.zeros((1, 16, 576), dtype=torch.bfloat16, device=DEV)
    q8 = torch.empty((1, 16, 576), dtype=torch.uint8, device=DEV)
    qs = torch.ones(1, dtype=torch.float32, device=DEV)
    out = torch.empty((1, 16, 512), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((32, 576), dtype=torch.uint8, device=DEV)
    with pytest.raises(mla.MLADecodeError) as e:           # a paged plan needs the paged run
        mla.mla_decode_run(plan, q, q8, qs, kv, out, kv_scale=qs, workspace=ws)
    assert e.value.status == 1
    ids = torch.zeros(2, dtype=torch.int32, device=DEV)
    with pytest.raises(mla.MLADecodeError) as e:           # no pages in the pool
        mla.mla_decode_run_paged(plan, q, q8, qs, kv, ids, 0, out, kv_scale=qs, workspace=ws)
    assert e.value.status == 1
    flat = mla.mla_decode_plan(qo, np.array([0, 20], np.int32))
    with pytest.raises(mla.MLADecodeError) as e:           # a contiguous plan has no pages
        mla.mla_decode_run_paged(flat, q, q8, qs, kv, ids, 2, out, kv_scale=qs, workspace=ws)
    assert e.value.status == 1


# Steps (2) and (3) from given Q codes on a paged pool: attend, and stage 1
# followed by the merge, against the three-launch run of the same step
ATTEND_CASES = [
    ("fp8", [1000, 0, 37, 513], None, 1, 0),
    ("fp8", [3000, 5, 64, 65], None, 64, 3),
    ("fp8", [700, 31, 32, 33], [2, 1, 4, 3], 16, 0),
    ("mxfp4", [1000, 0, 37, 513], None, 8, 0),
    ("mxfp4", [3000, 5, 64, 65], None, 64, 3),
    ("mxfp4", [700, 31, 32, 33], [1, 2, 3, 4], 32, 0),
]


@pytest.mark.parametrize("case", ATTEND_CASES,
                         ids=lambda c: f"{c[0]}_P{c[3]}_{'-'.join(map(str, c[1]))}"
                         f"{'_rows' if c[2] else ''}_s{c[4]}")
def test_paged_attend_and_stage1_equal_run(case):
    fmt, kv_lens, q_lens, P, max_splits = case
    announce(f"paged attend/stage1 {fmt} P{P} {kv_lens} rows {q_lens} splits {max_splits}")
    c = PagedCase(kv_lens, q_lens, P, 720 + P, "absmax", max_splits=max_splits, fmt=fmt)
    got, lse, q8, qs = c.run(False)
    ref, ref_lse, q8_ref, _, _, _ = c.oracle()
    assert np.array_equal(q8, q8_ref)
    assert_close(got, ref, f"paged run {fmt} P{P}")
    q8d = torch.from_numpy(q8).to(DEV)
    qsd = torch.tensor([qs], dtype=torch.float32, device=DEV)
    idsd = torch.from_numpy(c.ids).to(DEV)
    for fn in ("attend", "stage1"):
        ws = torch.zeros(max(c.plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
        out = torch.empty((c.rows, 16, 512), dtype=torch.bfloat16, device=DEV)
        lse2 = torch.empty((c.rows, 16), dtype=torch.float32, device=DEV)
        kw = dict(kv_scale=c.kv_scale, kv_block_scales=c.block_scales, sm_scale=SM,
                  workspace=ws, lse_out=lse2)
        if fn == "attend":
            mla.mla_decode_attend_paged(c.plan, q8d, qsd, c.codes, idsd, c.num_pages, out, **kw)
        else:
            mla.mla_decode_stage1_paged(c.plan, q8d, qsd, c.codes, idsd, c.num_pages, out, **kw)
            mla.mla_decode_merge(c.plan, ws, out, lse2)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy()
        assert np.array_equal(o.view(np.uint32), got.view(np.uint32)), fn
        assert np.array_equal(lse2.cpu().numpy().view(np.uint32), lse.view(np.uint32)), fn


def test_paged_attend_argument_errors():
    announce("paged attend/stage1 argument errors")
    qo, pi = np.array([0, 1], np.int32), np.array([0, 2], np.int32)
    plan = mla.mla_decode_plan_paged(qo, pi, np.array([3], np.int32), 16)
    flat = mla.mla_decode_plan(qo, np.array([0, 20], np.int32))
    ws = torch.zeros(max(plan.workspace_bytes, flat.workspace_bytes, 256), dtype=torch.uint8,
                     device=DEV)
    q8 = torch.zeros((1, 16, 576), dtype=torch.uint8, device=DEV)
    qs = torch.ones(1, dtype=torch.float32, device=DEV)
    out = torch.empty((1, 16, 512), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((32, 576), dtype=torch.uint8, device=DEV)
    ids = torch.zeros(2, dtype=torch.int32, device=DEV)
    for fn in (mla.mla_decode_attend, mla.mla_decode_stage1):   # a paged plan needs the page table
        with pytest.raises(mla.MLADecodeError) as e:
            fn(plan, q8, qs, kv, out, kv_scale=qs, workspace=ws)
        assert e.value.status == 1
    for fn in (mla.mla_decode_attend_paged, mla.mla_decode_stage1_paged):
        with pytest.raises(mla.MLADecodeError) as e:             # ... a contiguous plan none
            fn(flat, q8, qs, kv, ids, 2, out, kv_scale=qs, workspace=ws)
        assert e.value.status == 1
        with pytest.raises(mla.MLADecodeError) as e:             # no pages in the pool
            fn(plan, q8, qs, kv, ids, 0, out, kv_scale=qs, workspace=ws)
        assert e.value.status == 1
    bfp = mla.mla_decode_plan_paged(qo, pi, np.array([3], np.int32), 16,
                                    kv_format=mla.MLA_KV_BF16)
    bkv = torch.zeros((32, 576), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mla.MLADecodeError) as e:                 # a bf16 plan has no Q codes
        mla.mla_decode_attend_paged(bfp, q8, qs, bkv, ids, 2, out, workspace=ws)
    assert e.value.status == 1
