"""The measurement probe library (libmla_hbm_probe.so) on the GPU: every
streaming read returns 0 on a valid buffer, including a size whose last
1 MiB chunk is partial, and rejects invalid arguments without launching."""
import ctypes
import os

import pytest
import torch

from gpu_cases import DEV, announce

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import mla_latent_kv_bf16_amd  # noqa: F401  (torch's HIP runtime first, as for the decode)
    L = ctypes.CDLL(os.path.join(ROOT, "mla_latent_kv_bf16_amd", "libmla_hbm_probe.so"))
    for fn in (L.mla_hbm_read_probe, L.mla_hbm_read_probe_nt):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                       ctypes.c_void_p]
        fn.restype = ctypes.c_int
    L.mla_hbm_read_probe_lds_nt.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                            ctypes.c_void_p]
    L.mla_hbm_read_probe_lds_nt.restype = ctypes.c_int
    return L


def test_read_probes_run_and_check_arguments():
    announce("hbm read probes")
    L = _lib()
    nbytes = 3 * (1 << 20) + 48          # three whole chunks and a partial one
    buf = torch.ones(nbytes, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    for grid in (1, 3, 256):
        assert L.mla_hbm_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), grid, s) == 0
        assert L.mla_hbm_read_probe_nt(buf.data_ptr(), nbytes, sink.data_ptr(), grid, s) == 0
        assert L.mla_hbm_read_probe_lds_nt(buf.data_ptr(), nbytes, grid, s) == 0
    torch.cuda.synchronize()
    # invalid: empty, unaligned size or address, no buffer, grid out of range
    assert L.mla_hbm_read_probe_lds_nt(buf.data_ptr(), 0, 8, s) == 1
    assert L.mla_hbm_read_probe_lds_nt(buf.data_ptr(), 40, 8, s) == 1
    assert L.mla_hbm_read_probe_lds_nt(buf.data_ptr() + 8, 64, 8, s) == 1
    assert L.mla_hbm_read_probe_lds_nt(None, 64, 8, s) == 1
    assert L.mla_hbm_read_probe_lds_nt(buf.data_ptr(), 64, 0, s) == 1
    assert L.mla_hbm_read_probe_nt(buf.data_ptr(), 64, None, 8, s) == 1
    torch.cuda.synchronize()
    assert torch.all(buf == 1)           # the probes only read
