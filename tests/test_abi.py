"""CPU checks of the C ABI: the library loads, exports every function that
include/gift.h declares, and rejects bad arguments synchronously (these
calls return before any HIP call, so they need no GPU)."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

import fac_whitening_gift_amd as fg
from fac_whitening_gift_amd import _lib


def _declared():
    src = open(os.path.join(ROOT, "include", "gift.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gift_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = fg.load()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(fg.EXPORTS)
    assert lib.gift_abi_version() == 4


def test_status_strings():
    for s, name in enumerate(["GIFT_OK", "GIFT_ERR_INVALID_ARG", "GIFT_ERR_UNSUPPORTED_SHAPE",
                              "GIFT_ERR_WORKSPACE_TOO_SMALL", "GIFT_ERR_HIP"]):
        assert fg.status_name(s) == name


def _layer(d_out=64, d_in=128, factor=None, ptr=0x10000):
    L = _lib._Layer()
    L.d_out, L.d_in = d_out, d_in
    L.G = L.q = L.inv_scale = L.G_hat = ptr
    L.W_out = None
    L.factor = factor if factor is not None else ctypes.POINTER(_lib._Factor)()
    return L


def _call_whiten(layers, scaling=fg.SCALE_TENSOR, ws=0x100000, ws_bytes=1 << 30):
    lib = fg.load()
    arr = (_lib._Layer * len(layers))(*layers)
    return lib.gift_whiten_quantize(arr, len(layers), scaling, None, ws, ws_bytes, None)


@pytest.mark.parametrize("case,status", [
    (dict(d_in=130), 2),
    (dict(d_out=0), 2),
    (dict(d_in=1 << 25), 2),
    (dict(ptr=0x10004), 1),
    (dict(ptr=None), 1),
])
def test_layer_validation(case, status):
    assert _call_whiten([_layer(**case)]) == status
    assert fg.load().gift_last_error()


def test_block_scaling_needs_multiple_of_128():
    assert _call_whiten([_layer(d_in=192)], scaling=fg.SCALE_BLOCK128) == 2
    assert _call_whiten([_layer(d_in=48)], scaling=fg.SCALE_MXFP4) == 2
    assert _call_whiten([_layer(d_in=192)], scaling=7) == 1


def test_factor_validation():
    f = _lib._Factor(128, 32, 0x20000, 0x30000, 0x40000, None)
    assert _call_whiten([_layer(d_in=256, factor=ctypes.pointer(f))]) == 1   # d_in mismatch
    for bad in (0, 65, -1):   # the effective rank is 1..64
        f_bad_rank = _lib._Factor(128, bad, 0x20000, 0x30000, 0x40000, None)
        assert _call_whiten([_layer(d_in=128, factor=ctypes.pointer(f_bad_rank))]) == 2
    f_small = _lib._Factor(32, 32, 0x20000, 0x30000, 0x40000, None)
    assert _call_whiten([_layer(d_in=32, factor=ctypes.pointer(f_small))]) == 2
    f_odd = _lib._Factor(80, 32, 0x20000, 0x30000, 0x40000, None)   # d_in % 32 != 0
    assert _call_whiten([_layer(d_in=80, factor=ctypes.pointer(f_odd))]) == 2
    f_packs = _lib._Factor(128, 32, 0x20000, 0x30000, 0x40000, 0x50008)   # misaligned packs
    assert _call_whiten([_layer(d_in=128, factor=ctypes.pointer(f_packs))]) == 1
    assert _call_whiten([_layer(d_in=32, factor=ctypes.pointer(f_small))]) == 2


def test_workspace_validation():
    f = _lib._Factor(128, 32, 0x20000, 0x30000, 0x40000, None)
    layers = [_layer(d_in=128, factor=ctypes.pointer(f))]
    need = fg.load().gift_group_workspace_bytes(
        _lib.OP_WHITEN_QUANTIZE, (_lib._Layer * 1)(*layers), 1, fg.SCALE_TENSOR)
    assert need > 0
    assert _call_whiten(layers, ws_bytes=need - 1) == 3
    assert _call_whiten(layers, ws=0x100010) == 1     # not 256-byte aligned
    assert _call_whiten(layers, ws=None) == 1


def test_error_and_dequant_validation():
    lib = fg.load()
    arr = (_lib._Layer * 1)(_layer())
    assert lib.gift_roundtrip_error(arr, 1, None, 0x100000, 1 << 30, None) == 1
    arr[0].G_hat = None
    assert lib.gift_dequant_unwhiten(arr, 1, 0, 0x100000, 1 << 30, None) == 1
    assert lib.gift_euclid_fp8_roundtrip(arr, -1, 0, None, 0x100000, 1 << 30, None) == 1


def test_refresh_validation():
    lib = fg.load()
    f = _lib._Factor(128, 32, 0x20000, 0x30000, 0x40000, None)
    r = (_lib._RefreshInput * 1)()
    r[0].X, r[0].x_dtype, r[0].n_tokens = 0x60000, fg.DTYPE_BF16, 1024
    r[0].factor = ctypes.pointer(f)
    ok = dict(damp=1e-3, mode=fg.DAMP_FLOOR_PLUS_TAIL, w=64, steps=4)

    def call(n=1, damp=1e-3, mode=fg.DAMP_FLOOR_PLUS_TAIL, w=64, steps=4, ws=0x100000,
             nbytes=1 << 40, flags=None):
        return lib.gift_refresh_factors(r, n, damp, mode, w, steps, flags, ws, nbytes, None)

    assert call(n=0) == 0                      # empty group: nothing to do
    assert call(mode=7) == 1
    assert call(damp=float("nan")) == 1
    assert call(w=40) == 2
    assert call(steps=-1) == 1
    assert call(nbytes=16) == 3
    assert call(ws=0x100010) == 1
    assert call(flags=0x70002) == 1            # dev_flags not 4-byte aligned
    r[0].x_dtype = 9
    assert call() == 1
    r[0].x_dtype = fg.DTYPE_BF16
    r[0].n_tokens = 0
    assert call() == 2
    r[0].n_tokens = 1024
    f.d_in = 100
    assert call() == 2
    f.d_in, f.rank = 128, 65   # the effective rank is 1..64
    assert call() == 2
    f.rank = 48                # and at most the sketch width
    assert call(w=32) == 2
    assert call(w=112) == 2    # widths up to 96
    f.rank = 0
    assert call() == 2
    assert lib.gift_refresh_group_workspace_bytes(r, 1, 64) == 0 or True
    assert lib.gift_factor_pack_bytes(1024) == 1024 * 384
    assert lib.gift_factor_pack_bytes_rank(1024, 32) == 1024 * 384
    assert lib.gift_factor_pack_bytes_rank(1024, 33) == 2 * 1024 * 384
    assert lib.gift_factor_pack_bytes_rank(1024, 64) == 2 * 1024 * 384
    assert lib.gift_factor_pack_bytes_rank(1024, 65) == 0
    assert lib.gift_prepare_factor(None, None) == 1
    assert lib.gift_draw_sketch(None, 10, 64, 0, None) == 1


def test_refresh_workspace_holds_chain_descriptors():
    """A call of more than 16 inputs needs, on top of its inputs' own
    workspaces (the covariance groups of 16 in call order), room for the
    per-input descriptors of its chain: 256-byte aligned, 176 bytes each."""
    lib = fg.load()
    facs = [_lib._Factor(d, 32, 0x20000, 0x30000, 0x40000, None) for d in (128, 256, 384)]
    r = (_lib._RefreshInput * 17)()
    for k in range(17):
        r[k].X, r[k].x_dtype, r[k].n_tokens = 0x60000, fg.DTYPE_BF16, 1000 + 37 * k
        r[k].factor = ctypes.pointer(facs[k % 3])
    need16 = lib.gift_refresh_group_workspace_bytes(r, 16, 64)
    need17 = lib.gift_refresh_group_workspace_bytes(r, 17, 64)
    alone = lib.gift_refresh_workspace_bytes(facs[16 % 3].d_in, r[16].n_tokens, fg.DTYPE_BF16, 64)
    assert need16 > 0 and alone > 0
    assert need17 == need16 + alone + (17 * 176 + 255) // 256 * 256


def test_block_factor_validation():
    """block-A factors: sizes of the packs, and the argument errors that come
    back before any launch."""
    lib = _lib.load()
    assert lib.gift_block_factor_pack_bytes(1024, 32) == 1024 * 384
    assert lib.gift_block_factor_pack_bytes(1024, 64) == 1024 * 768
    assert lib.gift_block_factor_pack_bytes(100, 32) == 0
    assert lib.gift_block_factor_pack_bytes(1024, 48) == 0
    ok = dict(U=0x20000, theta=0x30000, coef=0x40000, packs=0x50000)

    def fac(d_in, block, packs=0x50000):
        f = _lib._Factor(d_in, 0, ok["U"], ok["theta"], ok["coef"], packs, block)
        return ctypes.pointer(f)
    assert _call_whiten([_layer(d_in=128, factor=fac(128, 48))]) == 2          # block size
    assert _call_whiten([_layer(d_in=96, factor=fac(96, 64))]) == 2            # d_in % block
    assert _call_whiten([_layer(d_in=128, factor=fac(128, 32, None))]) == 1    # packs required
    assert _call_whiten([_layer(d_in=128, factor=fac(128, 32))], scaling=2) == 2   # no MXFP4
    assert _call_whiten([_layer(d_in=256, factor=fac(128, 32))]) == 1          # d_in mismatch


def test_refresh_workspace_has_no_partials_for_single_range_bf16():
    """Sixteen bf16 inputs of width 4096 and 16384 tokens form a covariance
    group of 8448 tiles, so every tile takes all tokens in one range and the
    covariance kernel writes A itself: the workspace of each input is A and
    the subspace-iteration buffers only.  The same inputs in fp32 reserve one
    partial tile per (tile, range) on top."""
    lib = fg.load()
    d, n, w = 4096, 16384, 64
    f = _lib._Factor(d, 32, 0x20000, 0x30000, 0x40000, None)
    r = (_lib._RefreshInput * 16)()
    for k in range(16):
        r[k].X, r[k].x_dtype, r[k].n_tokens = 0x60000, fg.DTYPE_BF16, n
        r[k].factor = ctypes.pointer(f)

    def al(x):
        return (x + 255) // 256 * 256
    wmax = 96   # the operand packs of Q, the Gram partials and the triangle are laid out
    # for the largest width, so one layout serves every width
    per = (al(d * d * 4) + 4 * al(d * w * 4) + al(4 * d * w * 4) + al(d // 32 * wmax // 16 * 3 * 64 * 16)
           + al(16 * wmax * wmax * 8) + al(wmax * wmax * 8) + al(64))
    bf16 = lib.gift_refresh_group_workspace_bytes(r, 16, w)
    assert bf16 == 16 * per
    for k in range(16):
        r[k].x_dtype = fg.DTYPE_F32
    npairs = (d // 128) * (d // 128 + 1) // 2
    f32 = lib.gift_refresh_group_workspace_bytes(r, 16, w)
    assert f32 - bf16 >= 16 * npairs * 128 * 128 * 4
    # one such input alone splits its tokens over two ranges: partials needed
    alone = lib.gift_refresh_workspace_bytes(d, n, fg.DTYPE_BF16, w)
    assert alone > per


def test_static_scratch_entry_rejects_groups_beyond_its_array():
    """gift_whiten_quantize_static serves groups whose whiten workspace fits
    its 16 MiB static array; a larger group is refused before anything is
    enqueued (no GPU needed), with the sizes in the message."""
    lib = fg.load()
    assert lib.gift_static_scratch_bytes() == 16 << 20
    f = _lib._Factor(4096, 32, 0x20000, 0x30000, 0x40000, 0x50000)
    layers = [_layer(d_out=11008, d_in=4096, factor=ctypes.pointer(f))]
    arr = (_lib._Layer * 1)(*layers)
    need = lib.gift_group_workspace_bytes(_lib.OP_WHITEN_QUANTIZE, arr, 1, fg.SCALE_TENSOR)
    assert need > 16 << 20
    assert lib.gift_whiten_quantize_static(arr, 1, fg.SCALE_TENSOR, None, None) == 3
    assert b"16777216" in lib.gift_last_error()
    assert lib.gift_whiten_quantize_static(arr, 1, 9, None, None) == 1


def test_probe_library_exports_every_declared_function():
    """libgift_probe.so (the streaming probes of bench.py --study stream)
    exports what include/gift_probe.h declares and rejects bad arguments
    before any launch."""
    from fac_whitening_gift_amd import build as fb
    if not os.path.exists(fb.PROBE_LIB):
        pytest.skip("libgift_probe.so not built")
    src = open(os.path.join(ROOT, "include", "gift_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(gift_probe_\w+)\s*\(", src)))
    assert len(names) == 6
    lib = ctypes.CDLL(fb.PROBE_LIB)
    for n in names:
        assert hasattr(lib, n), n
    vp, sz, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
    lib.gift_probe_read.argtypes = [vp, sz, ctypes.c_int, vp]
    lib.gift_probe_tile_read.argtypes = [vp, i64, i64, vp]
    assert lib.gift_probe_read(None, 1024, 0, None) == 1
    assert lib.gift_probe_read(0x10008, 1024, 0, None) == 1
    assert lib.gift_probe_read(0x10000, 1000, 0, None) == 1
    assert lib.gift_probe_tile_read(0x10000, 100, 4096, None) == 1
    assert lib.gift_probe_tile_read(0x10000, 128, 300, None) == 1
