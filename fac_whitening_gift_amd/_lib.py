"""ctypes binding of libgift.so (include/gift.h): argument marshalling only.

Every computation happens in the HIP kernels behind the C ABI.  This module
turns torch device tensors into the ABI's descriptors and pointers, passes
torch's current HIP stream, and raises on a non-OK status.  If the library
is not built it raises instead of falling back to anything else.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgift.so")

RANK = 32
MAX_RANK = 64
MAX_SKETCH = 96
SKETCH_WIDTH = 64      # the refresh's subspace width for rank <= 32 (rank + 32)


def sketch_width_for(rank):
    """Subspace width of the refresh for a factor of this rank: rank + 32
    oversampling rounded to the 32-column storage, i.e. 64 up to rank 32 and
    96 above."""
    return SKETCH_WIDTH if rank <= RANK else MAX_SKETCH
BLOCK = 128

GIFT_OK = 0
DTYPE_F32, DTYPE_BF16 = 0, 1
DAMP_FLOOR, DAMP_FLOOR_PLUS_TAIL = 0, 1
SCALE_TENSOR, SCALE_BLOCK128, SCALE_MXFP4 = 0, 1, 2
MX_BLOCK = 32
FLAG_NONFINITE, FLAG_ZERO_AMAX = 1, 2
OP_WHITEN_QUANTIZE, OP_DEQUANT_UNWHITEN, OP_EUCLID_ROUNDTRIP, OP_ROUNDTRIP_ERROR = 0, 1, 2, 3
OP_UNWHITEN_F32 = 4

COEF_ALPHA, COEF_BETA, COEF_LAMBDA_ISO, COEF_LAMBDA_FLOOR, COEF_TRACE, COEF_SIGMA2_TAIL = range(6)
COEF_DW = 8
COEF_DU = 8 + RANK
COEF_COUNT = 8 + 2 * RANK


def factor_cols(rank):
    """Storage columns of a rank-r factor: 32 up to rank 32, else 64."""
    return RANK if rank <= RANK else 2 * RANK

EXPORTS = (
    "gift_refresh_factor", "gift_refresh_workspace_bytes", "gift_whiten_quantize",
    "gift_dequant_unwhiten", "gift_euclid_fp8_roundtrip", "gift_roundtrip_error",
    "gift_group_workspace_bytes", "gift_status_string", "gift_last_error",
    "gift_abi_version", "gift_draw_sketch", "gift_factor_pack_bytes", "gift_prepare_factor",
    "gift_refresh_factors", "gift_refresh_group_workspace_bytes", "gift_build_hash",
    "gift_dequant_accumulate", "gift_unwhiten_f32", "gift_block_factor_pack_bytes",
    "gift_whiten_quantize_static", "gift_static_scratch_bytes", "gift_factor_pack_bytes_rank",
)


class GiftError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__("%s: %s" % (status_name(status), detail))
        self.status = status


class _Factor(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("U", ctypes.c_void_p), ("theta", ctypes.c_void_p), ("coef", ctypes.c_void_p),
                ("packs", ctypes.c_void_p), ("block", ctypes.c_int32)]


class _RefreshInput(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("x_dtype", ctypes.c_int32), ("n_tokens", ctypes.c_int64),
                ("factor", ctypes.POINTER(_Factor)), ("sketch", ctypes.c_void_p),
                ("A_out", ctypes.c_void_p), ("seed", ctypes.c_uint64)]


class _Layer(ctypes.Structure):
    _fields_ = [("d_out", ctypes.c_int64), ("d_in", ctypes.c_int64),
                ("G", ctypes.c_void_p), ("q", ctypes.c_void_p), ("inv_scale", ctypes.c_void_p),
                ("G_hat", ctypes.c_void_p), ("factor", ctypes.POINTER(_Factor)),
                ("W_out", ctypes.c_void_p)]


_lib = None


def load():
    """Load libgift.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libgift.so is not built: run python -m fac_whitening_gift_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ, U64, F = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                             ctypes.c_uint64, ctypes.c_float)
    LP = ctypes.POINTER(_Layer)
    sig = {
        "gift_refresh_factor": (I, [P, I, I64, ctypes.POINTER(_Factor), F, I, I, I, U64, P, P, P,
                                    P, SZ, P]),
        "gift_refresh_workspace_bytes": (SZ, [I64, I64, I, I]),
        "gift_whiten_quantize": (I, [LP, I, I, P, P, SZ, P]),
        "gift_whiten_quantize_static": (I, [LP, I, I, P, P]),
        "gift_static_scratch_bytes": (SZ, []),
        "gift_dequant_unwhiten": (I, [LP, I, I, P, SZ, P]),
        "gift_euclid_fp8_roundtrip": (I, [LP, I, I, P, P, SZ, P]),
        "gift_roundtrip_error": (I, [LP, I, P, P, SZ, P]),
        "gift_group_workspace_bytes": (SZ, [I, LP, I, I]),
        "gift_status_string": (ctypes.c_char_p, [I]),
        "gift_last_error": (ctypes.c_char_p, []),
        "gift_abi_version": (I, []),
        "gift_build_hash": (ctypes.c_char_p, []),
        "gift_dequant_accumulate": (I, [LP, I, I, I, P]),
        "gift_unwhiten_f32": (I, [LP, I, P, SZ, P]),
        "gift_draw_sketch": (I, [P, I64, I, U64, P]),
        "gift_factor_pack_bytes": (SZ, [I64]),
        "gift_factor_pack_bytes_rank": (SZ, [I64, I]),
        "gift_block_factor_pack_bytes": (SZ, [I64, I]),
        "gift_prepare_factor": (I, [ctypes.POINTER(_Factor), P]),
        "gift_refresh_factors": (I, [ctypes.POINTER(_RefreshInput), I, F, I, I, I, P, P, SZ, P]),
        "gift_refresh_group_workspace_bytes": (SZ, [ctypes.POINTER(_RefreshInput), I, I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def build_hash():
    """Hash of the sources the loaded libgift.so was built from."""
    return load().gift_build_hash().decode()


def status_name(s):
    return load().gift_status_string(int(s)).decode()


def _check(status):
    if status != GIFT_OK:
        raise GiftError(status, load().gift_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, shape, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


# --------------------------------------------------------------------------
# Python-side holders of device tensors (the ABI structs point into them)
# --------------------------------------------------------------------------

class Factor:
    """Device buffers of one factor: U (d_in x C), theta (C), coef (8 + 2 C),
    and (by default, when d_in % 32 == 0) the operand packs of U.  rank
    (1..64) is the effective rank the refresh keeps; the storage is C = 32
    columns up to rank 32 and C = 64 above, zero from rank on.  block=32 or
    64 makes a block-diagonal factor (block-A-b): U is d_in x 2*block
    ([S_i | S_i^-1] per block row), theta d_in floats, packs always present.

    A factor built from given U / coef values has stale packs until
    gift_prepare_factor(factor) runs; gift_refresh_factor(s) rewrite them.
    packs=False leaves the pointer NULL (every grouped call re-packs U).
    """

    def __init__(self, d_in, device="cuda", U=None, theta=None, coef=None, packs=True,
                 rank=RANK, block=0):
        self.d_in = int(d_in)
        self.block = int(block)
        self.rank = 0 if self.block else int(rank)
        self.cols = 0 if self.block else factor_cols(self.rank)
        ucols = 2 * self.block if self.block else self.cols
        nth = self.d_in if self.block else self.cols
        ncoef = COEF_COUNT if self.block else 8 + 2 * self.cols
        device = U.device if U is not None else device
        self.U = U if U is not None else torch.zeros(d_in, ucols, device=device)
        self.theta = theta if theta is not None else torch.zeros(nth, device=device)
        self.coef = coef if coef is not None else torch.zeros(ncoef, device=device)
        _dev(self.U, torch.float32, (d_in, ucols), "U")
        _dev(self.theta, torch.float32, (nth,), "theta")
        _dev(self.coef, torch.float32, (ncoef,), "coef")
        self.packs = None
        if self.block:
            nb = int(load().gift_block_factor_pack_bytes(self.d_in, self.block))
            if nb == 0:
                raise ValueError("block factor needs block 32 or 64 dividing d_in")
            self.packs = torch.empty(nb, dtype=torch.uint8, device=self.U.device)
        elif packs and self.d_in % 32 == 0:
            nb = int(load().gift_factor_pack_bytes_rank(self.d_in, self.rank))
            self.packs = torch.empty(nb, dtype=torch.uint8, device=self.U.device)
        self._struct = _Factor(self.d_in, self.rank, self.U.data_ptr(), self.theta.data_ptr(),
                               self.coef.data_ptr(),
                               self.packs.data_ptr() if self.packs is not None else None,
                               self.block)

    @property
    def S(self):
        """Block factor: the stacked S_i (d_in x block)."""
        return self.U[:, :self.block]

    @property
    def S_inv(self):
        """Block factor: the stacked S_i^-1 (d_in x block)."""
        return self.U[:, self.block:]

    @property
    def alpha(self):
        return self.coef[COEF_ALPHA]

    @property
    def d_w(self):
        return self.coef[COEF_DW:COEF_DW + self.cols]

    @property
    def d_u(self):
        return self.coef[COEF_DW + self.cols:COEF_DW + 2 * self.cols]


class Layer:
    """One layer of a grouped call: G (d_out x d_in fp32) and its outputs.

    q, inv_scale and G_hat are allocated on G's device when not given:
    E4M3 codes d_out x d_in with inv_scale of 1 float (per tensor) or
    d_out x d_in/128 floats (block128=True); with mxfp4=True, MXFP4 codes
    d_out x d_in/2 bytes and d_out x d_in/32 E8M0 scale bytes.
    """

    def __init__(self, G, factor=None, q=None, inv_scale=None, G_hat=None, W_out=None,
                 block128=False, d_out=None, d_in=None, allocate=True, mxfp4=False):
        if G is not None:
            d_out, d_in = G.shape
            dev = G.device
        else:
            dev = (q if q is not None else G_hat).device
        self.d_out, self.d_in = int(d_out), int(d_in)
        self.G = G
        self.factor = factor
        self.mxfp4 = bool(mxfp4)
        qshape = (self.d_out, self.d_in // 2) if mxfp4 else (self.d_out, self.d_in)
        if allocate:
            if q is None:
                q = torch.empty(qshape, dtype=torch.uint8, device=dev)
            if inv_scale is None:
                if mxfp4:
                    inv_scale = torch.empty(self.d_out, self.d_in // MX_BLOCK, dtype=torch.uint8,
                                            device=dev)
                else:
                    shape = (self.d_out, self.d_in // BLOCK) if block128 else (1,)
                    inv_scale = torch.empty(shape, dtype=torch.float32, device=dev)
            if G_hat is None:
                G_hat = torch.empty(self.d_out, self.d_in, dtype=torch.float32, device=dev)
        self.q, self.inv_scale, self.G_hat, self.W_out = q, inv_scale, G_hat, W_out
        shape = (self.d_out, self.d_in)
        _dev(G, torch.float32, shape, "G")
        _dev(q, torch.uint8, qshape, "q")
        _dev(G_hat, torch.float32, shape, "G_hat")
        _dev(W_out, torch.float32, shape, "W_out")
        _dev(inv_scale, torch.uint8 if mxfp4 else torch.float32, None, "inv_scale")
        if factor is not None and factor.d_in != self.d_in:
            raise ValueError("factor d_in %d != layer d_in %d" % (factor.d_in, self.d_in))


def _layers_array(layers):
    arr = (_Layer * max(1, len(layers)))()
    for i, L in enumerate(layers):
        arr[i].d_out = L.d_out
        arr[i].d_in = L.d_in
        arr[i].G = _ptr(L.G)
        arr[i].q = _ptr(L.q)
        arr[i].inv_scale = _ptr(L.inv_scale)
        arr[i].G_hat = _ptr(L.G_hat)
        arr[i].factor = (ctypes.pointer(L.factor._struct) if L.factor is not None
                         else ctypes.POINTER(_Factor)())
        arr[i].W_out = _ptr(L.W_out)
    return arr


def _workspace(nbytes, device, ws):
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small: %d < %d bytes" %
                             (ws.numel() * ws.element_size(), nbytes))
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _device_of(layers):
    for L in layers:
        for t in (L.G, L.q, L.G_hat):
            if t is not None:
                return t.device
    return torch.device("cuda")


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)
# --------------------------------------------------------------------------

def gift_group_workspace_bytes(op, layers, scaling=SCALE_TENSOR):
    arr = _layers_array(layers)
    return int(load().gift_group_workspace_bytes(op, arr, len(layers), scaling))


def gift_refresh_workspace_bytes(d_in, n_tokens, x_dtype=DTYPE_BF16, sketch_width=SKETCH_WIDTH):
    return int(load().gift_refresh_workspace_bytes(d_in, n_tokens, x_dtype, sketch_width))


def gift_whiten_quantize(layers, scaling=SCALE_TENSOR, flags=None, ws=None, stream=None):
    lib = load()
    arr = _layers_array(layers)
    need = lib.gift_group_workspace_bytes(OP_WHITEN_QUANTIZE, arr, len(layers), scaling)
    ws = _workspace(need, _device_of(layers), ws)
    _check(lib.gift_whiten_quantize(arr, len(layers), scaling, _ptr(flags), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))


def gift_whiten_quantize_static(layers, scaling=SCALE_TENSOR, flags=None, stream=None):
    """gift_whiten_quantize with the library's static device scratch (no
    workspace, nothing allocated); calls on one GPU must not overlap."""
    arr = _layers_array(layers)
    _check(load().gift_whiten_quantize_static(arr, len(layers), scaling, _ptr(flags),
                                              _stream(stream)))


def gift_static_scratch_bytes():
    return int(load().gift_static_scratch_bytes())


def gift_dequant_unwhiten(layers, scaling=SCALE_TENSOR, ws=None, stream=None):
    lib = load()
    arr = _layers_array(layers)
    need = lib.gift_group_workspace_bytes(OP_DEQUANT_UNWHITEN, arr, len(layers), scaling)
    ws = _workspace(need, _device_of(layers), ws)
    _check(lib.gift_dequant_unwhiten(arr, len(layers), scaling, _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def gift_euclid_fp8_roundtrip(layers, scaling=SCALE_TENSOR, flags=None, ws=None, stream=None):
    lib = load()
    arr = _layers_array(layers)
    need = lib.gift_group_workspace_bytes(OP_EUCLID_ROUNDTRIP, arr, len(layers), scaling)
    ws = _workspace(need, _device_of(layers), ws)
    _check(lib.gift_euclid_fp8_roundtrip(arr, len(layers), scaling, _ptr(flags), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)))


def gift_roundtrip_error(layers, out=None, ws=None, stream=None):
    """-> device fp64 tensor (n_layers, 2): sum (G^-G)^2, sum G^2."""
    lib = load()
    arr = _layers_array(layers)
    dev = _device_of(layers)
    if out is None:
        out = torch.empty(len(layers), 2, dtype=torch.float64, device=dev)
    _dev(out, torch.float64, (len(layers), 2), "out")
    need = lib.gift_group_workspace_bytes(OP_ROUNDTRIP_ERROR, arr, len(layers), SCALE_TENSOR)
    ws = _workspace(need, dev, ws)
    _check(lib.gift_roundtrip_error(arr, len(layers), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))
    return out


class GroupCall:
    """One grouped round-trip call prepared once: the layer descriptor array,
    the workspace and the argument list are built here, so calling it only
    enqueues the kernels on the current (or given) stream.  Meant for loops
    and for HIP-graph capture; the layers' tensors must stay where they are.

    op: OP_WHITEN_QUANTIZE, OP_DEQUANT_UNWHITEN, OP_EUCLID_ROUNDTRIP or
    OP_ROUNDTRIP_ERROR (then out is the (n, 2) fp64 result, allocated when
    not given).
    """

    def __init__(self, op, layers, scaling=SCALE_TENSOR, flags=None, ws=None, out=None):
        lib = load()
        self.layers = list(layers)
        self.op = op
        self._arr = _layers_array(self.layers)
        n = len(self.layers)
        dev = _device_of(self.layers)
        sc = SCALE_TENSOR if op == OP_ROUNDTRIP_ERROR else scaling
        need = lib.gift_group_workspace_bytes(op, self._arr, n, sc)
        self.ws = _workspace(need, dev, ws)
        self.flags = flags
        wsp, wsb = _ptr(self.ws), self.ws.numel() * self.ws.element_size()
        if op == OP_WHITEN_QUANTIZE:
            self._fn = lib.gift_whiten_quantize
            self._args = (self._arr, n, scaling, _ptr(flags), wsp, wsb)
        elif op == OP_DEQUANT_UNWHITEN:
            self._fn = lib.gift_dequant_unwhiten
            self._args = (self._arr, n, scaling, wsp, wsb)
        elif op == OP_EUCLID_ROUNDTRIP:
            self._fn = lib.gift_euclid_fp8_roundtrip
            self._args = (self._arr, n, scaling, _ptr(flags), wsp, wsb)
        elif op == OP_ROUNDTRIP_ERROR:
            if out is None:
                out = torch.empty(n, 2, dtype=torch.float64, device=dev)
            _dev(out, torch.float64, (n, 2), "out")
            self.out = out
            self._fn = lib.gift_roundtrip_error
            self._args = (self._arr, n, _ptr(out), wsp, wsb)
        else:
            raise ValueError("unknown op %r" % (op,))

    def __call__(self, stream=None):
        _check(self._fn(*self._args, _stream(stream)))


def gift_dequant_accumulate(layers, scaling=SCALE_TENSOR, first=False, stream=None):
    """G_hat = decode(q) * inv (first) or G_hat + decode(q) * inv, per layer."""
    arr = _layers_array(layers)
    _check(load().gift_dequant_accumulate(arr, len(layers), scaling, 1 if first else 0,
                                          _stream(stream)))


def gift_unwhiten_f32(layers, ws=None, stream=None):
    """G_hat = G_hat A_r^1/2 in place for the whitened layers."""
    lib = load()
    arr = _layers_array(layers)
    need = lib.gift_group_workspace_bytes(OP_UNWHITEN_F32, arr, len(layers), SCALE_TENSOR)
    ws = _workspace(need, _device_of(layers), ws)
    _check(lib.gift_unwhiten_f32(arr, len(layers), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)))


def gift_factor_pack_bytes(d_in):
    return int(load().gift_factor_pack_bytes(d_in))


def gift_block_factor_pack_bytes(d_in, block):
    return int(load().gift_block_factor_pack_bytes(d_in, block))


def gift_prepare_factor(factor, stream=None):
    """Rewrite factor.packs from factor.U."""
    _check(load().gift_prepare_factor(ctypes.byref(factor._struct), _stream(stream)))


def _refresh_array(items):
    arr = (_RefreshInput * max(1, len(items)))()
    for i, it in enumerate(items):
        X, factor = it["X"], it["factor"]
        if X.dtype == torch.bfloat16:
            xdt = DTYPE_BF16
        elif X.dtype == torch.float32:
            xdt = DTYPE_F32
        else:
            raise ValueError("X must be bf16 or fp32")
        if X.dim() != 2 or X.shape[1] != factor.d_in:
            raise ValueError("X must be n_tokens x %d" % factor.d_in)
        _dev(X, X.dtype, None, "X")
        sk, A = it.get("sketch"), it.get("A_out")
        arr[i].X = X.data_ptr()
        arr[i].x_dtype = xdt
        arr[i].n_tokens = X.shape[0]
        arr[i].factor = ctypes.pointer(factor._struct)
        arr[i].sketch = sk.data_ptr() if sk is not None else None
        arr[i].A_out = A.data_ptr() if A is not None else None
        arr[i].seed = int(it.get("seed", 0)) & 0xFFFFFFFFFFFFFFFF
    return arr


def _width(items, sketch_width):
    if sketch_width is not None:
        return sketch_width
    return sketch_width_for(max(it["factor"].rank for it in items))


def gift_refresh_group_workspace_bytes(items, sketch_width=None):
    sketch_width = _width(items, sketch_width)
    arr = _refresh_array(items)
    return int(load().gift_refresh_group_workspace_bytes(arr, len(items), sketch_width))


def gift_refresh_factors(items, damp_eps=1e-3, damping_mode=DAMP_FLOOR_PLUS_TAIL,
                         sketch_width=None, power_steps=4, flags=None, ws=None,
                         stream=None):
    """items: list of dicts {X, factor, [sketch], [A_out], [seed]}; flags: optional
    device int32 word that collects GIFT_FLAG_NONFINITE; sketch_width None:
    sketch_width_for the largest rank of the call."""
    lib = load()
    sketch_width = _width(items, sketch_width)
    for it in items:
        _dev(it.get("sketch"), torch.float32, (it["factor"].d_in, sketch_width), "sketch")
        _dev(it.get("A_out"), torch.float32, (it["factor"].d_in, it["factor"].d_in), "A_out")
    arr = _refresh_array(items)
    need = lib.gift_refresh_group_workspace_bytes(arr, len(items), sketch_width)
    ws = _workspace(need, items[0]["X"].device, ws)
    _check(lib.gift_refresh_factors(arr, len(items), float(damp_eps), damping_mode, sketch_width,
                                    power_steps, _ptr(flags), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))


def gift_refresh_factor(X, factor, damp_eps=1e-3, damping_mode=DAMP_FLOOR_PLUS_TAIL,
                        sketch_width=None, power_steps=4, seed=0, sketch=None,
                        A_out=None, flags=None, ws=None, stream=None):
    lib = load()
    if X.dtype == torch.bfloat16:
        xdt = DTYPE_BF16
    elif X.dtype == torch.float32:
        xdt = DTYPE_F32
    else:
        raise ValueError("X must be bf16 or fp32")
    n_tokens, d_in = X.shape
    if sketch_width is None:
        sketch_width = sketch_width_for(factor.rank) if not factor.block else SKETCH_WIDTH
    if d_in != factor.d_in:
        raise ValueError("X width %d != factor d_in %d" % (d_in, factor.d_in))
    _dev(X, X.dtype, None, "X")
    _dev(sketch, torch.float32, (d_in, sketch_width), "sketch")
    _dev(A_out, torch.float32, (d_in, d_in), "A_out")
    need = lib.gift_refresh_workspace_bytes(d_in, n_tokens, xdt, sketch_width)
    ws = _workspace(need, X.device, ws)
    _check(lib.gift_refresh_factor(_ptr(X), xdt, n_tokens, ctypes.byref(factor._struct),
                                   float(damp_eps), damping_mode, sketch_width, power_steps,
                                   ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), _ptr(sketch),
                                   _ptr(A_out), _ptr(flags), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)))


def gift_draw_sketch(d_in, width=SKETCH_WIDTH, seed=0, out=None, device="cuda", stream=None):
    """-> device fp32 (d_in, width) Gaussian sketch (Philox4x32-10 + Box-Muller)."""
    if out is None:
        out = torch.empty(d_in, width, dtype=torch.float32, device=device)
    _dev(out, torch.float32, (d_in, width), "out")
    _check(load().gift_draw_sketch(_ptr(out), d_in, width,
                                   ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), _stream(stream)))
    return out
