"""A decode step driven by a C++ program through the C ABI alone
(tests/host/abi_decode.cpp, built by __graft_entry__.build()): no Python
between the caller and libmla_decode.so. Its outputs are checked against the
oracle, and bit for bit against the same step through the Python binding."""
import os
import struct
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import workloads
from gpu_cases import DEV, GpuCache, GpuDecode, OracleSide, announce, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host", "abi_decode")


def _bits(t: torch.Tensor) -> bytes:
    return t.contiguous().view(torch.int16).numpy().tobytes()


@pytest.mark.parametrize("fmt,q_mode,kv_lens", [
    ("fp8", "absmax", [300, 1, 77, 0, 1025]),
    ("fp8", "static", [4096, 33]),
    ("mxfp4", "absmax", [513, 64, 2, 1000]),
    ("mxfp4", "static", [0, 2048]),
])
def test_c_abi_driver_matches_oracle_and_binding(fmt, q_mode, kv_lens):
    assert os.path.exists(DRIVER), f"{DRIVER} is missing: run __graft_entry__.build()"
    announce(f"C ABI driver {fmt} {q_mode} {kv_lens}")
    batch = len(kv_lens)
    q = workloads.make_q(batch, 40 + batch)
    kv = workloads.make_kv(kv_lens, 41 + batch)
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fin, "wb") as f:
            f.write(struct.pack("<iiif", batch, 0 if fmt == "fp8" else 1,
                                0 if q_mode == "static" else 1, workloads.SM_SCALE))
            f.write(np.asarray(kv_lens, dtype="<i4").tobytes())
            f.write(_bits(q))
            f.write(_bits(kv))
        r = subprocess.run([DRIVER, fin, fout], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, f"driver failed: {r.stdout}\n{r.stderr}"
        raw = open(fout, "rb").read()
    n_out, n_lse, n_q8 = batch * 16 * 512, batch * 16, batch * 16 * 576
    off = 0
    out_bits = np.frombuffer(raw, dtype="<u2", count=n_out, offset=off)
    off += 2 * n_out
    lse = np.frombuffer(raw, dtype="<f4", count=n_lse, offset=off).reshape(batch, 16)
    off += 4 * n_lse
    q8 = np.frombuffer(raw, dtype=np.uint8, count=n_q8, offset=off).reshape(batch, 16, 576)
    off += n_q8
    q_scale = np.frombuffer(raw, dtype="<f4", count=1, offset=off)[0]
    assert off + 4 == len(raw)
    out = (out_bits.astype(np.uint32) << 16).view(np.float32).reshape(batch, 16, 512)

    # the oracle
    qo, kvp = workloads.indptrs(kv_lens)
    orc = OracleSide(q, kv, fmt, q_mode)
    assert q_scale == orc.q_scale
    assert np.array_equal(q8, orc.q8)
    ref, ref_lse = orc.decode(qo, kvp)
    assert_close(out, ref, f"C ABI driver {fmt}")
    assert_lse_close(lse, ref_lse, f"C ABI driver {fmt}")

    # the same step through the Python binding
    cache = GpuCache(kv, fmt)
    dec = GpuDecode(qo, kvp, fmt)
    got = dec.run_fused(q.to(DEV), cache, q_mode, orc.q_scale, init=True)
    assert np.array_equal(got[0].view(np.uint32), out.view(np.uint32))
    assert np.array_equal(got[1].view(np.uint32), lse.view(np.uint32))
    assert np.array_equal(got[2], q8)
    assert np.float32(got[3]) == q_scale
