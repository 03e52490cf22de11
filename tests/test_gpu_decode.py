"""GPU parity of the decode: the HIP path through the C ABI against the CPU
oracle, element by element, within |gpu - ref| <= 1e-2 + 2e-2 |ref| for the
bf16 output and 2e-3 for the natural-log LSE."""
import functools
import os

import numpy as np
import pytest
import torch

import mla_latent_kv_bf16_amd as mla
import oracle
import workloads
from gpu_cases import (DEV, GpuCache, GpuDecode, OracleSide, announce, assert_close,
                       assert_lse_close)

pytestmark = pytest.mark.gpu


def _need_fmt(fmt):
    assert fmt in ("fp8", "mxfp4")


def _case(kv_lens, seed, fmt="fp8", q_mode="absmax", max_splits=0, q=None, kv=None):
    qo, kvp = workloads.indptrs(kv_lens)
    q = workloads.make_q(len(kv_lens), seed) if q is None else q
    kv = workloads.make_kv(kv_lens, seed + 1) if kv is None else kv
    cache = GpuCache(kv, fmt)
    dec = GpuDecode(qo, kvp, fmt, max_splits=max_splits)
    orc = OracleSide(q, kv, fmt, q_mode)
    got, lse, q8, qs = dec.run(q.to(DEV), cache, q_mode, orc.q_scale)
    assert np.array_equal(q8[:len(kv_lens)], orc.q8)
    assert qs.view(np.uint32) == np.float32(orc.q_scale).view(np.uint32)
    return qo, kvp, got[:len(kv_lens)], lse[:len(kv_lens)], orc, cache, dec


RAGGED = [
    [1], [2], [31], [32], [33], [127, 128, 129], [1, 2, 3, 5, 8, 13, 21, 34, 55, 89],
    [1000, 0, 4097], [0], [257, 513, 1025, 96, 97, 95],
]


@pytest.mark.parametrize("kv_lens", RAGGED, ids=lambda l: "-".join(map(str, l))[:40])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_ragged_against_oracle(kv_lens, fmt):
    _need_fmt(fmt)
    announce(f"ragged {fmt} {kv_lens}")
    qo, kvp, got, lse, orc, _, _ = _case(kv_lens, 11 + len(kv_lens), fmt)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(got, ref, f"ragged {kv_lens}")
    assert_lse_close(lse, ref_lse, f"ragged {kv_lens}")


@pytest.mark.parametrize("max_splits", [1, -2, -5])
def test_mxfp4_long_items_against_oracle(max_splits):
    """MXFP4 items of 23 to 129 tiles of 32 rows, with ragged last tiles: from
    24 tiles on, the kernel gives an item's last two rounds of eight tiles to
    its first four waves only."""
    kv_lens = [736, 737, 767, 768, 769, 800, 1023, 1024, 1025, 2047, 4097]
    announce(f"mxfp4 long items, max_splits {max_splits}")
    qo, kvp, got, lse, orc, _, _ = _case(kv_lens, 77, "mxfp4", max_splits=max_splits)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(got, ref, f"mxfp4 long items {max_splits}")
    assert_lse_close(lse, ref_lse, f"mxfp4 long items {max_splits}")


@pytest.mark.parametrize("max_splits", [-1, -2, -3, -7, -31, 2, 5])
def test_split_counts_against_oracle(max_splits):
    kv_lens = [1000, 333, 1, 64, 2048]
    announce(f"forced splits {max_splits}")
    qo, kvp, got, lse, orc, _, _ = _case(kv_lens, 5, max_splits=max_splits)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(got, ref, f"max_splits {max_splits}")
    assert_lse_close(lse, ref_lse, f"max_splits {max_splits}")


@pytest.mark.parametrize("q_mode", ["absmax", "static"])
def test_static_and_absmax_scale(q_mode):
    announce(f"q mode {q_mode}")
    kv_lens = [700, 1500, 3]
    qo, kvp, got, lse, orc, _, _ = _case(kv_lens, 17, q_mode=q_mode)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(got, ref, q_mode)
    assert_lse_close(lse, ref_lse, q_mode)


@functools.lru_cache(maxsize=1)
def _big_inputs(name):
    w = workloads.BY_NAME[name]
    q = workloads.make_q(w.batch, w.seed_q)
    kv = workloads.make_kv([w.kv_len] * w.batch, w.seed_kv)
    return w, q, kv


@pytest.mark.parametrize("name", ["bs4_kv1024_fp8", "bs32_kv1024_fp8"])
def test_small_workloads_full(name):
    announce(f"workload {name} (full oracle)")
    w, q, kv = _big_inputs(name)
    qo, kvp, got, lse, orc, _, _ = _case([w.kv_len] * w.batch, 0, w.kv_format, q=q, kv=kv)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(got, ref, name)
    assert_lse_close(lse, ref_lse, name)


@pytest.mark.parametrize("name,q_mode", [("bs64_kv8192_fp8", "absmax"),
                                         ("bs64_kv8192_fp8", "static"),
                                         ("bs256_kv8192_fp8", "absmax"),
                                         ("bs256_kv8192_fp8", "static"),
                                         ("bs256_kv1024_mxfp4", "absmax"),
                                         ("bs256_kv1024_mxfp4", "static")])
def test_large_workloads_full(name, q_mode):
    """Full-size inputs in the benchmark's launch configuration (default plan),
    every sequence compared with the oracle, through both the three-launch and
    the single-launch entry points."""
    _need_fmt(workloads.BY_NAME[name].kv_format)
    w, q, kv = _big_inputs(name)
    announce(f"workload {name} {q_mode} (full oracle, three-launch path)")
    qo, kvp, got, lse, orc, cache, dec = _case([w.kv_len] * w.batch, 0, w.kv_format, q_mode,
                                               q=q, kv=kv)
    announce(f"workload {name} {q_mode}: oracle over all {w.batch} sequences")
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(got, ref, f"{name} {q_mode} three-launch")
    assert_lse_close(lse, ref_lse, f"{name} {q_mode} three-launch")
    announce(f"workload {name} {q_mode} (full oracle, fused path)")
    fgot, flse, fq8, fqs = dec.run_fused(q.to(DEV), cache, q_mode, orc.q_scale, init=True)
    assert np.array_equal(fq8[:w.batch], orc.q8)
    assert fqs.view(np.uint32) == np.float32(orc.q_scale).view(np.uint32)
    assert_close(fgot[:w.batch], ref, f"{name} {q_mode} fused")
    assert_lse_close(flse[:w.batch], ref_lse, f"{name} {q_mode} fused")


def test_kv_len_one_returns_v_row_exactly():
    announce("kv_len 1 returns V row")
    kv_lens = [1, 1, 1, 1]
    qo, kvp, got, lse, orc, cache, _ = _case(kv_lens, 23)
    codes, _ = orc.kv_codes()
    v = oracle.fp8_dequant(codes[:, :512], orc.kv_scale)
    expect = torch.from_numpy(v).float().bfloat16().float().numpy()
    for b in range(4):
        for h in range(16):
            assert np.array_equal(got[b, h], expect[b])


def test_identical_scores_give_mean_of_v():
    announce("identical scores -> mean of V")
    n = 300
    q = workloads.make_q(1, 31)
    q[:, :, :512] = 0
    kv = workloads.make_kv([n], 32)
    kv[:, 512:] = kv[0, 512:]
    qo, kvp, got, lse, orc, _, _ = _case([n], 0, q=q, kv=kv)
    codes, _ = orc.kv_codes()
    mean = oracle.fp8_dequant(codes[:, :512], orc.kv_scale).mean(axis=0)
    for h in range(16):
        np.testing.assert_allclose(got[0, h], mean, rtol=2 ** -8, atol=1e-6)


def test_rope_tail_drives_scores():
    announce("scores only from latent dims 512..575")
    n = 200
    q = workloads.make_q(2, 41)
    q[:, :, :512] = 0
    q = (q.float() * 3).bfloat16()
    kv = workloads.make_kv([n, n], 42)
    qo, kvp, got, lse, orc, _, _ = _case([n, n], 0, q=q, kv=kv)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(got, ref, "rope tail")
    assert_lse_close(lse, ref_lse, "rope tail")
    codes, _ = orc.kv_codes()
    v = oracle.fp8_dequant(codes[:, :512], orc.kv_scale)
    mean0 = v[:n].mean(axis=0)
    assert np.abs(ref[0] - mean0).max() > 0.1   # the tail really moves the weights


def test_partials_against_oracle_split_mode():
    announce("stage-1 partials vs oracle split ranges")
    kv_lens = [1000, 64, 333]
    qo, kvp, got, lse, orc, cache, dec = _case(kv_lens, 51, max_splits=-3)
    items, merges, nslots = mla.mla_decode_plan_host(qo, kvp, max_splits=-3)
    assert nslots > 0
    ws = dec.ws.cpu().numpy()
    part_o = ws[:nslots * 16 * 512 * 4].view(np.float32).reshape(nslots, 16, 512)
    off = ((nslots * 16 * 512 * 4 + 255) // 256) * 256
    part_lse = ws[off:off + nslots * 16 * 4].view(np.float32).reshape(nslots, 16)
    codes, _ = orc.kv_codes()
    for b, lo, hi, slot in items:
        if slot < 0:
            continue
        o, l = oracle.mla_decode(orc.q8, orc.q_scale, codes, orc.kv_scale, qo, kvp,
                                 workloads.SM_SCALE, seqs=[b], kv_lo=[lo - kvp[b]],
                                 kv_hi=[hi - kvp[b]])
        assert_close(part_o[slot], o[0], f"partial slot {slot}")
        assert np.abs(part_lse[slot] * np.log(2) - l[0]).max() <= 2e-3


def test_merge_alone_on_oracle_partials():
    announce("merge kernel on oracle partials")
    kv_lens = [900, 0, 450, 1300]
    qo, kvp = workloads.indptrs(kv_lens)
    q = workloads.make_q(4, 61)
    kv = workloads.make_kv(kv_lens, 62)
    orc = OracleSide(q, kv, "fp8")
    codes, _ = orc.kv_codes()
    dec = GpuDecode(qo, kvp, "fp8", max_splits=-4)
    items, merges, nslots = mla.mla_decode_plan_host(qo, kvp, max_splits=-4)
    part_o = np.zeros((nslots, 16, 512), dtype=np.float32)
    part_lse = np.zeros((nslots, 16), dtype=np.float32)
    for b, lo, hi, slot in items:
        o, l = oracle.mla_decode(orc.q8, orc.q_scale, codes, orc.kv_scale, qo, kvp,
                                 workloads.SM_SCALE, seqs=[b], kv_lo=[lo - kvp[b]],
                                 kv_hi=[hi - kvp[b]])
        part_o[slot] = o[0]
        part_lse[slot] = l[0] / np.log(2)
    ws = np.zeros(dec.ws.numel(), dtype=np.uint8)
    ws[:part_o.nbytes] = part_o.view(np.uint8).reshape(-1)
    off = ((part_o.nbytes + 255) // 256) * 256
    ws[off:off + part_lse.nbytes] = part_lse.view(np.uint8).reshape(-1)
    dec.ws.copy_(torch.from_numpy(ws))
    out = torch.full((4, 16, 512), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((4, 16), dtype=torch.float32, device=DEV)
    mla.mla_decode_merge(dec.plan, dec.ws, out, lse)
    torch.cuda.synchronize()
    ref, ref_lse = orc.decode(qo, kvp)
    got = out.float().cpu().numpy()
    for m in merges:
        b = int(m[0])
        assert_close(got[b], ref[b], f"merge b={b}")
        assert_lse_close(lse.cpu().numpy()[b], ref_lse[b], f"merge b={b}")
    assert not got[1].any() and np.all(np.isneginf(lse.cpu().numpy()[1]))


def test_run_is_deterministic():
    announce("bitwise determinism")
    kv_lens = [3000, 17, 4096]
    qo, kvp = workloads.indptrs(kv_lens)
    q = workloads.make_q(3, 71)
    kv = workloads.make_kv(kv_lens, 72)
    cache = GpuCache(kv, "fp8")
    dec = GpuDecode(qo, kvp, "fp8", max_splits=-5)
    qd = q.to(DEV)
    a = dec.run(qd, cache)
    b = dec.run(qd, cache)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_empty_batch():
    announce("empty batch")
    dec = GpuDecode(np.array([0], np.int32), np.array([0], np.int32), "fp8")
    kv = torch.zeros((1, 576), dtype=torch.uint8, device=DEV)
    ks = torch.ones(1, dtype=torch.float32, device=DEV)
    q = torch.zeros((1, 16, 576), dtype=torch.bfloat16, device=DEV)
    mla.mla_decode_run(dec.plan, q, dec.q8, dec.q_scale, kv, dec.out, kv_scale=ks,
                       workspace=dec.ws)
    torch.cuda.synchronize()
    assert dec.q_scale.item() == np.float32(1e-12) / np.float32(448.0)


def test_binding_rejects_wrong_buffers():
    """Tensors that do not match the plan (short, wrong element size, host,
    strided) are refused by the binding before any launch: the output keeps
    its contents, and the matching call afterwards runs."""
    announce("binding buffer checks")
    qo, kvp = workloads.indptrs([100, 200])
    dec = GpuDecode(qo, kvp, "fp8")
    kv = torch.zeros((300, 576), dtype=torch.uint8, device=DEV)
    ks = torch.ones(1, dtype=torch.float32, device=DEV)
    q = torch.zeros((2, 16, 576), dtype=torch.bfloat16, device=DEV)
    dec.out.fill_(7.0)
    torch.cuda.synchronize()
    for fused in (False, True):
        run = mla.mla_decode_run_fused if fused else mla.mla_decode_run
        for bad in (dict(q=q[:1]), dict(q=q.float()), dict(q=q.cpu()),
                    dict(q=q.transpose(1, 2)), dict(kv=kv[:299]), dict(out=dec.out[:1]),
                    dict(q8=dec.q8.view(torch.int16))):
            args = dict(q=q, q8=dec.q8, kv=kv, out=dec.out)
            args.update(bad)
            with pytest.raises(mla.MLADecodeError) as e:
                run(dec.plan, args["q"], args["q8"], dec.q_scale, args["kv"], args["out"],
                    kv_scale=ks, workspace=dec.ws)
            assert e.value.status == 1
    torch.cuda.synchronize()
    assert torch.all(dec.out == 7.0)
    mla.mla_decode_run(dec.plan, q, dec.q8, dec.q_scale, kv, dec.out, kv_scale=ks,
                       workspace=dec.ws)
    torch.cuda.synchronize()
    assert torch.all(dec.out == 0)   # zero Q and cache: every output row is the mean of zeros


def test_package_imported_before_torch():
    """A process that imports this package before torch still runs a decode:
    the library binds to torch's HIP runtime (regression test; a second
    runtime used to fail every device call of the library)."""
    import subprocess
    import sys
    announce("package imported before torch (subprocess)")
    code = (
        "import mla_latent_kv_bf16_amd as mla\n"
        "import numpy as np, torch\n"
        "qo, kvp = np.array([0, 1], np.int32), np.array([0, 40], np.int32)\n"
        "plan = mla.mla_decode_plan(qo, kvp)\n"
        "d = 'cuda'\n"
        "ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=d)\n"
        "q = torch.zeros((1, 16, 576), dtype=torch.bfloat16, device=d)\n"
        "kv = torch.zeros((40, 576), dtype=torch.uint8, device=d)\n"
        "ks = torch.ones(1, dtype=torch.float32, device=d)\n"
        "q8 = torch.empty((1, 16, 576), dtype=torch.uint8, device=d)\n"
        "qs = torch.empty(1, dtype=torch.float32, device=d)\n"
        "out = torch.full((1, 16, 512), 7.0, dtype=torch.bfloat16, device=d)\n"
        "mla.mla_decode_run(plan, q, q8, qs, kv, out, kv_scale=ks, workspace=ws)\n"
        "torch.cuda.synchronize()\n"
        "assert torch.all(out == 0), 'decode did not run'\n"
        "print('ok')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=110,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def test_argument_errors():
    announce("argument errors")
    qo, kvp = workloads.indptrs([100, 200])
    dec = GpuDecode(qo, kvp, "fp8", max_splits=-2)
    kv = torch.zeros((300, 576), dtype=torch.uint8, device=DEV)
    ks = torch.ones(1, dtype=torch.float32, device=DEV)
    q = torch.zeros((2, 16, 576), dtype=torch.bfloat16, device=DEV)
    ok = dict(kv_scale=ks, workspace=dec.ws)

    def status(**kw):
        args = dict(ok)
        args.update(kw)
        try:
            mla.mla_decode_run(dec.plan, args.pop("q", q), dec.q8, dec.q_scale,
                               args.pop("kv", kv), args.pop("out", dec.out), **args)
        except mla.MLADecodeError as e:
            return e.status
        return 0

    assert status() == 0
    assert status(workspace=dec.ws[:16]) == 4
    assert status(kv_block_scales=kv) == 1
    assert status(kv_scale=None) == 1
    assert status(sm_scale=float("nan")) == 1
    assert status(sm_scale=-1.0) == 1
    assert status(q_scale_mode=5) == 1
    assert status(out=dec.out.view(-1)[1:]) == 1     # misaligned output
    torch.cuda.synchronize()


def _sink_and_tail(kv_lens, sinks, seed):
    """Q and cache where each sequence's scores come from the rope dims only:
    one key (the sink, V = 0) lies 16-17 log2 units above a long tail of keys
    whose V ~ N(1, 1). The tail then holds about 8 % of the softmax mass, at
    weights of 2^-17 .. 2^-16 of the sink's."""
    rows = sum(kv_lens)
    g = torch.Generator().manual_seed(seed)
    kv = torch.randn((rows, 576), generator=g).add_(1.0).clamp_(-6.0, 6.0)
    # tail rope values U(0.08, 0.34): logits 16-17 log2 units below the sink's
    kv[:, 512:] = torch.rand((rows, 1), generator=g) * 0.26 + 0.08
    starts = np.concatenate([[0], np.cumsum(kv_lens)[:-1]])
    for b, pos in enumerate(sinks):
        if pos is not None:
            r = int(starts[b]) + pos
            kv[r, :512] = 0.0
            kv[r, 512:] = 4.5            # exact in e4m3 at the cache scale 1/64
    kv[1, 0] = 7.0                       # the cache's largest magnitude: scale 7/448 = 1/64
    q = torch.zeros((len(kv_lens), 16, 576))
    q[:, :, 512:] = 1.0
    return q.to(torch.bfloat16), kv.to(torch.bfloat16)


@pytest.mark.parametrize("max_splits", [1, 0], ids=["unsplit", "policy"])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_long_low_tail_after_a_dominant_key(fmt, max_splits):
    """Weights far below the maximum still count in P.V: a dominant key with
    V = 0 (first tile, a middle tile, the last tile, none) and 8191 keys
    whose weights lie 2^-14 .. 2^-18 below it."""
    kv_lens = [8192] * 4
    announce(f"dominant key + long low tail {fmt} max_splits {max_splits}")
    q, kv = _sink_and_tail(kv_lens, [0, 5000, 8191, None], 97)
    qo, kvp, got, lse, orc, cache, dec = _case(kv_lens, 0, fmt, "absmax", max_splits, q=q, kv=kv)
    ref, ref_lse = orc.decode(qo, kvp)
    # the construction: the tail holds a few per cent of the mass of sequences
    # 0-2 (about 8 % with the FP8 cache; the MXFP4 cache's coarser rope
    # values leave a smaller gap and about 25 %)
    assert 0.02 < np.abs(ref[:3]).mean() < 0.3
    assert_close(got, ref, f"sink + tail {fmt} three-launch")
    assert_lse_close(lse, ref_lse, f"sink + tail {fmt} three-launch")
    fgot, flse, _, _ = dec.run_fused(q.to(DEV), cache, "absmax", None, init=True)
    assert_close(fgot[:4], ref, f"sink + tail {fmt} fused")
    assert_lse_close(flse[:4], ref_lse, f"sink + tail {fmt} fused")
