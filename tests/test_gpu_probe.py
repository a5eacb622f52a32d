"""The streaming probes of libgift_probe.so (bench.py --study stream) on
small buffers: read probes leave memory unchanged, write probes zero exactly
the bytes they are given, copy probes copy them; a byte count that is not a
multiple of a launch's width exercises the tails."""

import ctypes
import os

import pytest
import torch

from fac_whitening_gift_amd import build as fb
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _lib():
    if not os.path.exists(fb.PROBE_LIB):
        pytest.fail("libgift_probe.so is not built (python -m fac_whitening_gift_amd.build)")
    lib = ctypes.CDLL(fb.PROBE_LIB)
    vp, sz, i64, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int
    for name, types in (("gift_probe_read", [vp, sz, i, vp]),
                        ("gift_probe_write", [vp, sz, i, vp]),
                        ("gift_probe_copy", [vp, vp, sz, i, vp]),
                        ("gift_probe_tile_read", [vp, i64, i64, vp]),
                        ("gift_probe_tile_write", [vp, i64, i64, i, vp]),
                        ("gift_probe_slab_read", [vp, i64, i64, vp])):
        getattr(lib, name).argtypes = types
        getattr(lib, name).restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("nt", [0, 1])
def test_flat_probes(nt):
    say("stream probes flat nt=%d" % nt)
    lib = _lib()
    st = torch.cuda.current_stream().cuda_stream
    n = 4 * 123457  # floats: 123457 float4, not a multiple of a step
    a = torch.randn(n + 64, device=DEV)
    b = torch.randn(n + 64, device=DEV)
    a0, b0 = a.clone(), b.clone()
    assert lib.gift_probe_read(a.data_ptr(), 4 * n, nt, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(a, a0)
    assert lib.gift_probe_copy(a.data_ptr(), b.data_ptr(), 4 * n, nt, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(b[:n], a0[:n]) and torch.equal(b[n:], b0[n:])
    assert lib.gift_probe_write(b.data_ptr(), 4 * n, nt, st) == 0
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(b[:n])) == 0 and torch.equal(b[n:], b0[n:])


@pytest.mark.parametrize("nt", [0, 1])
def test_tile_and_slab_probes(nt):
    say("stream probes tile/slab nt=%d" % nt)
    lib = _lib()
    st = torch.cuda.current_stream().cuda_stream
    rows, cols = 192, 768
    a = torch.randn(rows * cols + 64, device=DEV)
    a0 = a.clone()
    assert lib.gift_probe_tile_read(a.data_ptr(), rows, cols, st) == 0
    assert lib.gift_probe_slab_read(a.data_ptr(), rows, cols, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(a, a0)
    assert lib.gift_probe_tile_write(a.data_ptr(), rows, cols, nt, st) == 0
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(a[:rows * cols])) == 0
    assert torch.equal(a[rows * cols:], a0[rows * cols:])
