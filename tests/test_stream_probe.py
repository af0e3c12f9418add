"""The streaming copy kernel the benchmark measures its bandwidth ceiling with
(include/stream_probe.h, libstreamprobe.so)."""

import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "row_wise_normalization_fp32_amd", "libstreamprobe.so")


def _lib():
    lib = ctypes.CDLL(PROBE)
    lib.rn_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.rn_probe_copy.restype = ctypes.c_int
    return lib


def test_probe_library_exports_only_the_declared_entry_point():
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE], capture_output=True, text=True, check=True).stdout
    text = [l.split()[-1] for l in out.splitlines() if " T " in l]
    assert text == ["rn_probe_copy"]


def test_probe_rejects_bad_arguments_before_any_launch():
    lib = _lib()
    a, b = 1 << 20, 1 << 24  # host-side checks only: nothing is dereferenced or launched
    assert lib.rn_probe_copy(None, b, 16, 4, 256, 0, 1, None) == 1
    assert lib.rn_probe_copy(a, b, 17, 4, 256, 0, 1, None) == 2
    assert lib.rn_probe_copy(a + 8, b, 16, 4, 256, 0, 1, None) == 2
    assert lib.rn_probe_copy(a, b, 16, 3, 256, 0, 1, None) == 3
    assert lib.rn_probe_copy(a, b, 16, 4, 128, 0, 1, None) == 3
    assert lib.rn_probe_copy(a, a + 16, 64, 4, 256, 0, 1, None) == 4
    assert lib.rn_probe_copy(a, b, 0, 4, 256, 0, 1, None) == 0


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 77, 16 << 20])
@pytest.mark.parametrize("geom", [(1, 256, 0, 0), (4, 256, 0, 1), (2, 512, 8, 1), (8, 1024, 2, 1)])
def test_probe_copies_exactly(nbytes, geom):
    import torch

    v, b, per_cu, nt = geom
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.randint(-(1 << 15), 1 << 15, (nbytes // 2,), dtype=torch.int16, device="cuda:0")
    buf = torch.full((nbytes // 2 + 4096,), 7, dtype=torch.int16, device="cuda:0")
    dst = buf[2048:2048 + nbytes // 2]  # 4 KiB guard zones on both sides
    st = _lib().rn_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, v, b, cus * per_cu, nt,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(src, dst)
    assert bool((buf[:2048] == 7).all()) and bool((buf[2048 + nbytes // 2:] == 7).all())
