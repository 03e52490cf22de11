"""CPU tests of the host side of libmla_decode.so: the library loads and
exports every entry point its header declares, and the scheduler's work
items and merge map are valid for the benchmark shapes and ragged inputs.
No kernel is launched."""
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import mla_latent_kv_bf16_amd as mla
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    pat = r"^\s*(?:MLA_\w*API\s+)?(?:const\s+)?\w+\*?\s+\**(mla_\w+)\s*\("
    return sorted(set(re.findall(pat, text, flags=re.M)))


def test_header_entry_points_are_exported():
    names = _declared_functions()
    assert "mla_decode_plan" in names and "mla_decode_run" in names
    assert len(names) >= 10
    assert "mla_decode_run_fused" in names and "mla_decode_workspace_init" in names
    L = mla.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in the header but not exported"


def test_only_the_c_abi_is_exported():
    """Every dynamic symbol the library defines is an entry point of the header."""
    import subprocess
    lib_path = os.path.join(ROOT, "mla_latent_kv_bf16_amd", "libmla_decode.so")
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True,
                         text=True, check=True).stdout
    text_syms = {ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3
                 and ln.split()[1] == "T"}
    assert text_syms == set(_declared_functions())


def test_hbm_probe_library_exports_its_header():
    """The measurement helper library loads (no GPU call) and exports exactly
    what include/mla_hbm_probe.h declares."""
    import ctypes
    import subprocess
    lib_path = os.path.join(ROOT, "mla_latent_kv_bf16_amd", "libmla_hbm_probe.so")
    names = _declared_functions(os.path.join(ROOT, "include", "mla_hbm_probe.h"))
    assert names == ["mla_hbm_read_probe", "mla_hbm_read_probe_lds_nt", "mla_hbm_read_probe_nt"]
    L = ctypes.CDLL(lib_path)
    for n in names:
        assert hasattr(L, n)
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True,
                         text=True, check=True).stdout
    text_syms = {ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3
                 and ln.split()[1] == "T"}
    assert text_syms == set(names)


def test_status_strings():
    assert mla.mla_status_string(0) == "ok"
    for s in range(1, 6):
        assert mla.mla_status_string(s) not in ("ok", "unknown status")
    assert mla.mla_status_string(99) == "unknown status"


def _check_schedule(kv_lens, items, merges, nslots):
    qo, kvp = workloads.indptrs(kv_lens)
    covered = np.zeros(int(kvp[-1]), dtype=np.int32)
    per_seq_slots = {}
    for b, lo, hi, slot in items:
        assert hi > lo, "empty work item"
        assert kvp[b] <= lo and hi <= kvp[b + 1]
        covered[lo:hi] += 1
        per_seq_slots.setdefault(int(b), []).append(int(slot))
    assert np.all(covered == 1), "every cache row belongs to exactly one item"
    seen_slots = []
    merged = {int(m[0]): m for m in merges}
    for b, n in enumerate(kv_lens):
        slots = per_seq_slots.get(b, [])
        if n == 0:
            assert not slots and b in merged and merged[b][2] == 0
        elif len(slots) == 1:
            assert slots == [-1] and b not in merged
        else:
            m = merged[b]
            assert m[2] == len(slots)
            assert sorted(slots) == list(range(m[1], m[1] + m[2]))
            seen_slots += slots
    assert sorted(seen_slots) == list(range(nslots))


@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=lambda w: w.name)
def test_schedule_benchmark_shapes(w):
    lens = [w.kv_len] * w.batch
    qo, kvp = workloads.indptrs(lens)
    fmt = 0 if w.kv_format == "fp8" else 1
    items, merges, nslots = mla.mla_decode_plan_host(qo, kvp, kv_format=fmt, num_cus=256)
    _check_schedule(lens, items, merges, nslots)
    # about one item per compute unit, never below two 32-token tiles per wave
    assert len(items) <= 2 * 256 or w.batch > 256
    assert min(hi - lo for _, lo, hi, _ in items) >= min(256, w.kv_len)


def test_schedule_policy_values():
    def splits(bs, kv):
        qo, kvp = workloads.indptrs([kv] * bs)
        items, _, _ = mla.mla_decode_plan_host(qo, kvp, num_cus=256)
        return len(items) // bs
    assert splits(4, 1024) == 4
    assert splits(32, 1024) == 4
    assert splits(64, 8192) == 4
    assert splits(256, 8192) == 1
    assert splits(256, 1024) == 1


@pytest.mark.parametrize("kv_lens", [[1], [0], [0, 0], [5, 0, 1, 33, 32, 31, 64, 1000],
                                     [100000], [7] * 300, [4096, 1, 1, 1]])
@pytest.mark.parametrize("max_splits", [0, 1, 3, -2, -7, -64])
def test_schedule_ragged(kv_lens, max_splits):
    qo, kvp = workloads.indptrs(kv_lens)
    items, merges, nslots = mla.mla_decode_plan_host(qo, kvp, num_cus=256, max_splits=max_splits)
    _check_schedule(kv_lens, items, merges, nslots)
    if max_splits > 0:
        for b in range(len(kv_lens)):
            assert sum(1 for it in items if it[0] == b) <= max_splits


@pytest.mark.parametrize("max_splits", [0, -64, -65, -2000])
def test_schedule_split_cap(max_splits):
    """A query row gets at most 64 splits, whatever the request (the header's
    max_splits contract), and forced splits below the cap are honoured."""
    qo, kvp = workloads.indptrs([131072, 40960])
    items, merges, nslots = mla.mla_decode_plan_host(qo, kvp, num_cus=256, max_splits=max_splits)
    _check_schedule([131072, 40960], items, merges, nslots)
    per_seq = [sum(1 for it in items if it[0] == b) for b in range(2)]
    assert max(per_seq) <= 64
    if max_splits < 0:
        assert per_seq == [64, 64]


# bytes per cache row the kernels address with 32-bit offsets within an item
_ITEM_ROW_BYTES = {mla.MLA_KV_FP8_E4M3FN: 576, mla.MLA_KV_MXFP4: 288 + 18, mla.MLA_KV_BF16: 1152}


@pytest.mark.parametrize("fmt", [mla.MLA_KV_FP8_E4M3FN, mla.MLA_KV_MXFP4, mla.MLA_KV_BF16])
@pytest.mark.parametrize("num_cus,max_splits", [(1, 0), (256, 1), (256, 0), (7, -3), (1, 2)])
def test_schedule_item_bytes_stay_below_2_32(fmt, num_cus, max_splits):
    """Whatever the CU count or split request, no item's bytes reach 2^32
    (items cap at 2^22 rows, 2^21 for the bf16 cache)."""
    lens = [4_000_000, 9_000_001, 33]
    qo, kvp = workloads.indptrs(lens)
    items, merges, nslots = mla.mla_decode_plan_host(qo, kvp, kv_format=fmt, num_cus=num_cus,
                                                     max_splits=max_splits)
    _check_schedule(lens, items, merges, nslots)
    rows = items[:, 2].astype(np.int64) - items[:, 1]
    assert rows.max() * _ITEM_ROW_BYTES[fmt] < 2 ** 32
    assert rows.max() <= (2 ** 21 if fmt == mla.MLA_KV_BF16 else 2 ** 22)


def test_schedule_bf16_range_beyond_2_30_rows_unsupported():
    """A bf16 row range needing more than 512 items of 2^21 rows cannot be
    merged (the merge holds at most 512 partials per row): UNSUPPORTED, while
    the same range with the FP8 cache fits."""
    qo, kvp = workloads.indptrs([2 ** 30 + 1])
    with pytest.raises(mla.MLADecodeError) as e:
        mla.mla_decode_plan_host(qo, kvp, kv_format=mla.MLA_KV_BF16)
    assert e.value.status == 2
    items, _, _ = mla.mla_decode_plan_host(qo, kvp, kv_format=mla.MLA_KV_FP8_E4M3FN, max_splits=1)
    assert len(items) == 257 and (items[:, 2] - items[:, 1]).max() <= 2 ** 22
    qo, kvp = workloads.indptrs([2 ** 30])
    items, _, _ = mla.mla_decode_plan_host(qo, kvp, kv_format=mla.MLA_KV_BF16, max_splits=1)
    assert len(items) == 512


def _xcd_reference_order(items, seq_of_row=None):
    """The item order written out from its description: items longest first
    (stable over the items' creation order), sequences take the residues mod 8 in turn, index 8 j + r holds
    the j-th item of residue r's list, or the next item of the list with the
    most left once r's list has run out. Items name their query row; rows of
    one sequence count as that sequence."""
    # creation order is by query row, then split; a stable sort keeps it
    by_len = sorted(items.tolist(), key=lambda it: (-(it[2] - it[1]), it[0], it[1]))
    lists, res = [[] for _ in range(8)], {}
    for it in by_len:
        key = it[0] if seq_of_row is None else int(seq_of_row[it[0]])
        if key not in res:
            res[key] = len(res) % 8
        lists[res[key]].append(it)
    pos, out = [0] * 8, []
    while len(out) < len(by_len):
        for r in range(8):
            if len(out) == len(by_len):
                break
            src = r
            if pos[r] == len(lists[r]):
                left = [len(lists[q]) - pos[q] for q in range(8)]
                src = int(np.argmax(left))
            out.append(lists[src][pos[src]])
            pos[src] += 1
    return np.array(out, dtype=np.int32).reshape(-1, 4)


@pytest.mark.parametrize("lens", [[5, 9000, 40, 700, 0, 3000], [1024] * 4, [1024] * 32,
                                  [8192] * 64, [8192] * 256, [3000, 17, 2048, 5000, 1, 900, 64]])
def test_schedule_deterministic_and_xcd_grouped(lens):
    qo, kvp = workloads.indptrs(lens)
    a = mla.mla_decode_plan_host(qo, kvp, num_cus=64)
    b = mla.mla_decode_plan_host(qo, kvp, num_cus=64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    items = a[0]
    assert np.array_equal(items, _xcd_reference_order(items))
    # each XCD (index mod 8) still takes its items longest first
    for r in range(8):
        sizes = items[r::8, 2] - items[r::8, 1]
        if len(lens) >= 8 and len(set(lens)) == 1:
            assert np.all(np.diff(sizes) <= 0)


def test_schedule_groups_a_sequence_on_one_xcd():
    # bs32 and bs64 split four ways: every sequence's items share one residue
    for lens in ([1024] * 32, [8192] * 64):
        qo, kvp = workloads.indptrs(lens)
        items, _, _ = mla.mla_decode_plan_host(qo, kvp)
        assert len(items) == 4 * len(lens)
        for b in range(len(lens)):
            idx = np.nonzero(items[:, 0] == b)[0]
            assert len(idx) == 4 and len(set(idx % 8)) == 1
    # unsplit sequences keep their order
    qo, kvp = workloads.indptrs([8192] * 256)
    items, _, _ = mla.mla_decode_plan_host(qo, kvp)
    assert np.array_equal(items[:, 0], np.arange(256))


def test_schedule_empty_batch():
    items, merges, nslots = mla.mla_decode_plan_host([0], [0])
    assert len(items) == 0 and len(merges) == 0 and nslots == 0


@pytest.mark.parametrize("qo,kv,heads,fmt,status", [
    ([0, 1, 2], [0, 5, 3], 16, 0, 1),     # kv_indptr decreases
    ([0, 1, 2], [1, 5, 9], 16, 0, 1),     # kv_indptr does not start at 0
    ([1, 2, 3], [0, 5, 9], 16, 0, 1),     # qo_indptr does not start at 0
    ([0, 2, 1], [0, 5, 9], 16, 0, 1),     # qo_indptr decreases
    ([0, 1, 2], [0, 5, 9], 8, 0, 2),      # head count other than 16
    ([0, 1, 2], [0, 5, 9], 16, 3, 2),     # unknown cache format
])
def test_schedule_rejects(qo, kv, heads, fmt, status):
    with pytest.raises(mla.MLADecodeError) as e:
        mla.mla_decode_plan_host(qo, kv, kv_format=fmt, num_heads=heads)
    assert e.value.status == status


def test_schedule_small_output_arrays_rejected():
    qo, kvp = workloads.indptrs([1000, 1000])
    L = mla.lib()
    import ctypes
    i32p = ctypes.POINTER(ctypes.c_int32)
    counts = np.zeros(3, dtype=np.int32)
    items = np.zeros(4, dtype=np.int32)
    st = L.mla_decode_plan_host(qo.ctypes.data_as(i32p), kvp.ctypes.data_as(i32p), 2, 16, 0, 256,
                                -4, items.ctypes.data_as(i32p), 1, None, 0,
                                counts.ctypes.data_as(i32p))
    assert st == 1


@pytest.mark.parametrize("kv_lens,q_lens,max_splits", [
    ([40, 3, 1, 0, 65, 9], [4, 4, 2, 3, 1, 3], 0),
    ([1000, 5000, 257], [2, 4, 3], 0),
    ([1000, 5000, 257], [2, 4, 3], -5),
    ([8192] * 8, [2] * 8, 0),
])
def test_schedule_query_rows(kv_lens, q_lens, max_splits):
    """Several query rows per sequence: row i of R covers exactly the first
    kv_len - (R - 1 - i) cache rows of its sequence (causal), each row has its
    own items, slots and merge entry, and the items index the query row."""
    qo, kvp = workloads.indptrs(kv_lens, q_lens)
    items, merges, nslots = mla.mla_decode_plan_host(qo, kvp, num_cus=256,
                                                     max_splits=max_splits)
    rows = int(qo[-1])
    ends = []
    for b, (n, R) in enumerate(zip(kv_lens, q_lens)):
        for i in range(R):
            ends.append((int(kvp[b]), int(kvp[b]) + max(0, n - (R - 1 - i))))
    assert len(ends) == rows
    per_row = {}
    for r, lo, hi, slot in items:
        assert 0 <= r < rows and hi > lo
        per_row.setdefault(int(r), []).append((int(lo), int(hi), int(slot)))
    merged = {int(m[0]): m for m in merges}
    seen = []
    for r, (beg, end) in enumerate(ends):
        parts = sorted(per_row.get(r, []))
        if end == beg:
            assert not parts and merged[r][2] == 0
            continue
        assert parts[0][0] == beg and parts[-1][1] == end
        assert all(parts[k][1] == parts[k + 1][0] for k in range(len(parts) - 1))
        if len(parts) == 1:
            assert parts[0][2] == -1 and r not in merged
        else:
            m = merged[r]
            assert sorted(p[2] for p in parts) == list(range(m[1], m[1] + m[2]))
            seen += [p[2] for p in parts]
    assert sorted(seen) == list(range(nslots))


_ROW_BYTES = {mla.MLA_KV_FP8_E4M3FN: 576, mla.MLA_KV_MXFP4: 306, mla.MLA_KV_BF16: 1152}


@settings(max_examples=300, deadline=None)
@given(data=st.data(), fmt=st.sampled_from(sorted(_ROW_BYTES)),
       num_cus=st.sampled_from([0, 1, 7, 64, 256, 304]),
       max_splits=st.sampled_from([0, 1, 2, 5, -1, -3, -64]))
def test_schedule_properties_on_random_shapes(data, fmt, num_cus, max_splits):
    """Random ragged batches with 1-4 query rows per sequence: every query
    row's causal range is covered exactly once by its items, slots and merge
    entries match, items stay below 2^32 bytes, the order is the XCD order
    written out from its description, and the result is deterministic."""
    kv = data.draw(st.lists(st.integers(0, 6000), min_size=0, max_size=24), label="kv_lens")
    q_lens = data.draw(st.lists(st.integers(1, 4), min_size=len(kv), max_size=len(kv)),
                       label="q_lens")
    qo, kvp = workloads.indptrs(kv, q_lens)
    a = mla.mla_decode_plan_host(qo, kvp, kv_format=fmt, num_cus=num_cus, max_splits=max_splits)
    b = mla.mla_decode_plan_host(qo, kvp, kv_format=fmt, num_cus=num_cus, max_splits=max_splits)
    assert all(np.array_equal(x, y) for x, y in zip(a[:2], b[:2])) and a[2] == b[2]
    items, merges, nslots = a
    seq_of_row = np.repeat(np.arange(len(kv)), q_lens)
    ends = []
    for bq, (n, R) in enumerate(zip(kv, q_lens)):
        for i in range(R):
            ends.append((int(kvp[bq]), int(kvp[bq]) + max(0, n - (R - 1 - i))))
    per_row = {}
    for r, lo, hi, slot in items:
        assert hi > lo and (hi - lo) * _ROW_BYTES[fmt] < 2 ** 32
        per_row.setdefault(int(r), []).append((int(lo), int(hi), int(slot)))
    merged = {int(m[0]): m for m in merges}
    seen = []
    for r, (beg, end) in enumerate(ends):
        parts = sorted(per_row.get(r, []))
        if end == beg:
            assert not parts and merged[r][2] == 0
            continue
        assert parts[0][0] == beg and parts[-1][1] == end
        assert all(parts[k][1] == parts[k + 1][0] for k in range(len(parts) - 1))
        if len(parts) == 1:
            assert parts[0][2] == -1 and r not in merged
        else:
            m = merged[r]
            assert sorted(p[2] for p in parts) == list(range(m[1], m[1] + m[2]))
            seen += [p[2] for p in parts]
    assert sorted(seen) == list(range(nslots))
    if len(items):
        assert np.array_equal(items, _xcd_reference_order(items, seq_of_row))


def test_bench_refuses_more_than_one_gpu():
    """bench.py --gpus N with N > 1 exits with status 2 and a JSON message,
    before it touches a GPU."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=root,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["n_gpus"] == 2 and "one GPU" in d["error"]
