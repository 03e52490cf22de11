"""The binding's buffer checks (CPU): every run wrapper checks device,
element size, contiguity and size of the tensors it passes to the C ABI
against the plan, and raises MLADecodeError(MLA_INVALID_ARGUMENT) before any
call into the library. A stand-in object plays the tensors here."""
from types import SimpleNamespace

import pytest

import mla_latent_kv_bf16_amd as mla
from mla_latent_kv_bf16_amd import binding


class FakeTensor:
    def __init__(self, numel, elem, cuda=True, contiguous=True):
        self._n, self._e, self.is_cuda, self._c = numel, elem, cuda, contiguous

    def numel(self):
        return self._n

    def element_size(self):
        return self._e

    def is_contiguous(self):
        return self._c


def plan(rows=3, fmt=mla.MLA_KV_FP8_E4M3FN, total_kv=100, page_size=0, total_pages=0):
    return SimpleNamespace(rows=rows, kv_format=fmt, total_kv=total_kv, page_size=page_size,
                           total_pages=total_pages)


def good(p):
    nq = p.rows * 16
    kv_elems = {mla.MLA_KV_FP8_E4M3FN: (576, 1), mla.MLA_KV_MXFP4: (288, 1),
                mla.MLA_KV_BF16: (576, 2)}[p.kv_format]
    return dict(q_bf16=FakeTensor(nq * 576, 2), q_fp8=FakeTensor(nq * 576, 1),
                q_scale=FakeTensor(1, 4), kv=FakeTensor(p.total_kv * kv_elems[0], kv_elems[1]),
                kv_block_scales=FakeTensor(p.total_kv * 18, 1) if p.kv_format == mla.MLA_KV_MXFP4
                else None,
                kv_scale=FakeTensor(1, 4), out_bf16=FakeTensor(nq * 512, 2),
                lse_out=FakeTensor(nq, 4))


def check(p, **kw):
    args = good(p)
    args.update(kw)
    binding._check_step(p, args["q_bf16"], args["q_fp8"], args["q_scale"], args["kv"],
                        args["kv_block_scales"], args["kv_scale"], args["out_bf16"],
                        args["lse_out"])


@pytest.mark.parametrize("fmt", [mla.MLA_KV_FP8_E4M3FN, mla.MLA_KV_MXFP4, mla.MLA_KV_BF16])
def test_matching_buffers_pass(fmt):
    check(plan(fmt=fmt))
    check(plan(fmt=fmt), lse_out=None, kv_scale=None)


@pytest.mark.parametrize("name,bad", [
    ("q_bf16", FakeTensor(3 * 16 * 576 - 1, 2)),          # one element short
    ("q_bf16", FakeTensor(3 * 16 * 576, 4)),              # float32 instead of bf16
    ("q_bf16", FakeTensor(3 * 16 * 576, 2, cuda=False)),  # host tensor
    ("q_fp8", FakeTensor(3 * 16 * 576, 1, contiguous=False)),
    ("q_scale", FakeTensor(0, 4)),
    ("kv", FakeTensor(100 * 576 - 16, 1)),
    ("kv", None),
    ("out_bf16", FakeTensor(3 * 16 * 512 - 1, 2)),
    ("lse_out", FakeTensor(3 * 16 - 1, 4)),
    ("kv_scale", FakeTensor(1, 2)),
])
def test_wrong_buffers_raise_invalid_argument(name, bad):
    with pytest.raises(mla.MLADecodeError) as e:
        check(plan(), **{name: bad})
    assert e.value.status == binding.MLA_INVALID_ARGUMENT
    assert name.split("_")[0] in str(e.value)


def test_mxfp4_needs_block_scales():
    p = plan(fmt=mla.MLA_KV_MXFP4)
    with pytest.raises(mla.MLADecodeError):
        check(p, kv_block_scales=None)
    with pytest.raises(mla.MLADecodeError):
        check(p, kv_block_scales=FakeTensor(100 * 18 - 1, 1))
    with pytest.raises(mla.MLADecodeError):  # the packed cache is 288 B per row
        check(p, kv=FakeTensor(100 * 288 - 1, 1))


def test_empty_needs_nothing():
    check(plan(rows=0), q_bf16=None, kv=None, out_bf16=None)   # no rows: the library decides
    check(plan(total_kv=0), kv=None)                           # no cache rows: kv may be absent


def test_paged_pool_and_page_table():
    p = plan(total_kv=0, page_size=16, total_pages=5)
    args = good(p)
    ok = dict(args, kv=FakeTensor(7 * 16 * 576, 1))

    def run(**kw):
        a = dict(ok)
        a.update(kw)
        binding._check_step(p, a["q_bf16"], a["q_fp8"], a["q_scale"], a["kv"], None,
                            a["kv_scale"], a["out_bf16"], a["lse_out"], num_pages=7,
                            kv_page_ids=a.get("ids", FakeTensor(5, 4)))
    run()
    with pytest.raises(mla.MLADecodeError):
        run(kv=FakeTensor(7 * 16 * 576 - 1, 1))
    with pytest.raises(mla.MLADecodeError):
        run(ids=FakeTensor(4, 4))
    with pytest.raises(mla.MLADecodeError):
        run(ids=FakeTensor(5, 8))
