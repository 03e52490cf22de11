"""Seeded synthetic workloads for absorbed-path MLA decode.

Shared by the tests and the benchmark, on both sides of the parity check.
This module holds no arithmetic of the method: it only draws N(0, 1) values
with a seeded CPU generator, rounds them to bf16, and builds the CSR row
pointers. Quantisation, attention and everything else lives either in the
oracle or in the HIP library.

Shapes follow the benchmark shapes of the kernelindex.com "amd-mixed-mla"
pages: 16 query heads of 576 dims, qseqlen 1, one shared 576-d latent KV
head, page size 1, kv_indptr = arange(bs+1) * kv_len
[submission 663509, `ALL_CONFIGS` and `_precompute_metadata`].
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

HEADS = 16
DQK = 576
DV = 512
SM_SCALE = 1.0 / 24.0  # 1/sqrt(576), exact


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    kv_len: int
    kv_format: str          # "fp8" or "mxfp4"
    q_scale_mode: str       # "absmax" or "static"
    seed_q: int
    seed_kv: int


# The five benchmark workloads. Seeds are (100 + i, 200 + i).
WORKLOADS = [
    Workload("bs4_kv1024_fp8", 4, 1024, "fp8", "absmax", 100, 200),
    Workload("bs32_kv1024_fp8", 32, 1024, "fp8", "absmax", 101, 201),
    Workload("bs64_kv8192_fp8", 64, 8192, "fp8", "absmax", 102, 202),
    Workload("bs256_kv8192_fp8", 256, 8192, "fp8", "absmax", 103, 203),
    Workload("bs256_kv1024_mxfp4", 256, 1024, "mxfp4", "absmax", 104, 204),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def indptrs(kv_lens, q_lens=None) -> tuple[np.ndarray, np.ndarray]:
    """qo_indptr and kv_indptr for per-sequence KV lengths and query-row
    counts (qseqlen 1 for every sequence when q_lens is None)."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    if q_lens is None:
        qo = np.arange(kv_lens.size + 1, dtype=np.int32)
    else:
        q_lens = np.asarray(q_lens, dtype=np.int64)
        assert q_lens.size == kv_lens.size
        qo = np.zeros(kv_lens.size + 1, dtype=np.int32)
        qo[1:] = np.cumsum(q_lens)
    kv = np.zeros(kv_lens.size + 1, dtype=np.int64)
    kv[1:] = np.cumsum(kv_lens)
    assert kv[-1] < 2**31
    return qo, kv.astype(np.int32)


def randn_bf16(shape, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def make_q(rows: int, seed: int) -> torch.Tensor:
    """q: (rows, 16, 576) bf16 ~ N(0, 1), one row per query row (= per
    sequence at qseqlen 1)."""
    return randn_bf16((rows, HEADS, DQK), seed)


def make_kv(kv_lens, seed: int) -> torch.Tensor:
    """Latent cache: (sum kv_lens, 576) bf16 ~ N(0, 1), drawn one sequence at a
    time in order so that large caches never need an fp32 copy of the whole."""
    kv_lens = [int(n) for n in kv_lens]
    total = sum(kv_lens)
    out = torch.empty((total, DQK), dtype=torch.bfloat16)
    g = torch.Generator(device="cpu").manual_seed(seed)
    pos = 0
    for n in kv_lens:
        if n:
            out[pos:pos + n] = torch.randn((n, DQK), generator=g,
                                           dtype=torch.float32).to(torch.bfloat16)
        pos += n
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw bf16 payload as a uint16 numpy array (no conversion)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def make_page_table(kv_lens, page_size: int, seed: int, spare_pages: int = 3):
    """A paged layout for sequences of kv_lens rows: every sequence gets
    ceil(len / page_size) pages drawn without replacement from a pool with
    `spare_pages` unused pages, in a seeded random order.
    Returns (page_indptr int32 (b+1), page_ids int32, last_page_len int32 (b),
    num_pages, row_of_token int64 (sum kv_lens): the pool row holding each
    token of the concatenated sequences)."""
    kv_lens = [int(n) for n in kv_lens]
    npages = [(n + page_size - 1) // page_size for n in kv_lens]
    total = sum(npages)
    num_pages = total + spare_pages
    rng = np.random.default_rng(seed)
    ids = rng.permutation(num_pages)[:total].astype(np.int32)
    indptr = np.zeros(len(kv_lens) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(npages)
    last = np.array([n - (p - 1) * page_size if p else 0 for n, p in zip(kv_lens, npages)],
                    dtype=np.int32)
    rows = []
    for b, n in enumerate(kv_lens):
        t = np.arange(n, dtype=np.int64)
        rows.append(ids[indptr[b] + t // page_size].astype(np.int64) * page_size + t % page_size)
    row_of_token = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return indptr, ids, last, num_pages, row_of_token
