"""Python binding of libepilora.so, the multi-tenant LoRA low-precision
linear layer for MI355X (gfx950).

Argument marshalling only: every function below takes torch tensors that
already live on the GPU, passes their device pointers, sizes and the current
HIP stream to the C entry point of the same name (include/epilora.h), and
raises EpiloraError on a nonzero status.  No computation happens here, and
there is no fallback: if the library is missing, importing the binding's
functions raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libepilora.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
DEV_BAD_INDEX, DEV_WAIT_TIMEOUT, DEV_INTERNAL = 1, 2, 4
W_FP8, W_FP4 = 0, 1
A_BF16, A_FP8 = 0, 1
ACT_FP8, ACT_BF16 = 0, 1
OP_SHRINK, OP_GEMM, OP_EXPAND, OP_DECODE, OP_QUANT_W4 = 1, 2, 3, 4, 5
DECODE_MAX_M = 64
MAX_RANK = 128


class EpiloraError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class LayerArgs(ctypes.Structure):
    """Mirror of epilora_layer_args."""
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64),
        ("xq", ctypes.c_void_p), ("sx", ctypes.c_void_p), ("ldq", ctypes.c_int64),
        ("wfmt", ctypes.c_int32),
        ("w", ctypes.c_void_p), ("sw", ctypes.c_void_p), ("bs", ctypes.c_void_p), ("gs", ctypes.c_void_p),
        ("L", ctypes.c_int32), ("r", ctypes.c_int32),
        ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("ranks", ctypes.c_void_p),
        ("idx", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("z", ctypes.c_void_p),
        ("scale", ctypes.c_float),
        ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64),
        ("xq_out", ctypes.c_void_p), ("sx_out", ctypes.c_void_p), ("ldq_out", ctypes.c_int64),
        ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
        ("nslices", ctypes.c_int32), ("slice_n", ctypes.c_int64 * 4),
        ("afmt", ctypes.c_int32), ("sa", ctypes.c_void_p), ("sb", ctypes.c_void_p),
        ("amode", ctypes.c_int32),
    ]


_lib = None

# (name, restype, argtypes) of every exported symbol.
_I64, _I32, _P, _SZ, _F = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "epilora_version": (ctypes.c_int, []),
    "epilora_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "epilora_workspace_bytes": (_SZ, [_I32, _I64, _I64, _I64, _I32]),
    "epilora_workspace_init": (ctypes.c_int, [_P, _SZ, _P]),
    "epilora_workspace_force_timeout": (ctypes.c_int, [_P, _SZ, _I32, _P]),
    "epilora_device_error": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_I32), _P]),
    "epilora_quant_act": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P, _P]),
    "epilora_quant_weight_fp8": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "epilora_quant_weight_fp4": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "epilora_lora_shrink": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "epilora_rmsnorm_quant_shrink": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _F, _P, _I64, _P, _I64, _P, _P, _I32,
                                                    _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "epilora_lora_shrink_ex": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I32, _P, _I32, _I32, _I32, _P, _P, _P, _P,
                                              _P, _SZ, _P]),
    "epilora_lora_expand_add_ex": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _P, _I32, _I32, _I32, _P, _P, _P, _P,
                                                  _F, _P, _I64, _P, _SZ, _P]),
    "epilora_gemm_lora": (ctypes.c_int, [ctypes.POINTER(LayerArgs), _P]),
    "epilora_lora_expand_add": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _I32, _P, _P, _P, _F, _P, _I64, _P, _SZ, _P]),
    "epilora_decode_lora": (ctypes.c_int, [ctypes.POINTER(LayerArgs), _P]),
    "epilora_decode_lora_noalloc": (ctypes.c_int, [ctypes.POINTER(LayerArgs), _P]),
}


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp4_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn, status):
    if status != OK:
        raise EpiloraError(fn, status, lib().epilora_strerror(status).decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, dtype, name):
    if t is None:
        return
    if t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name}: expected a {dtype} GPU tensor, got {t.dtype} on {t.device}")


def _ld(t):
    return t.stride(0) if t.dim() == 2 else t.shape[-1]


# --- workspace -------------------------------------------------------------------

def epilora_workspace_bytes(op, M, N, K, r):
    return lib().epilora_workspace_bytes(op, M, N, K, r)


def epilora_workspace_init(ws, stream=None):
    _need(ws, torch.uint8, "ws")
    _check("epilora_workspace_init", lib().epilora_workspace_init(_ptr(ws), ws.numel(), _stream(stream)))


def new_workspace(op, M, N, K, r, device="cuda"):
    """Allocate (with torch) and initialise a workspace for `op`."""
    ws = torch.empty(max(epilora_workspace_bytes(op, M, N, K, r), 256), dtype=torch.uint8, device=device)
    epilora_workspace_init(ws)
    return ws


def epilora_workspace_force_timeout(ws, on, stream=None):
    _need(ws, torch.uint8, "ws")
    _check("epilora_workspace_force_timeout",
           lib().epilora_workspace_force_timeout(_ptr(ws), ws.numel(), int(bool(on)), _stream(stream)))


def epilora_device_error(ws, clear=True, stream=None):
    out = ctypes.c_int32(0)
    _check("epilora_device_error", lib().epilora_device_error(_ptr(ws), int(clear), ctypes.byref(out),
                                                              _stream(stream)))
    return out.value


# --- quantization ------------------------------------------------------------------

def epilora_quant_act(x, xq, sx, stream=None):
    """x: bf16 [M][K] -> xq: uint8 [M][K], sx: fp32 [M]."""
    _need(x, torch.bfloat16, "x"); _need(xq, torch.uint8, "xq"); _need(sx, torch.float32, "sx")
    M, K = x.shape
    _check("epilora_quant_act", lib().epilora_quant_act(_ptr(x), M, K, _ld(x), _ptr(xq), _ld(xq), _ptr(sx),
                                                        _stream(stream)))


def epilora_quant_weight_fp8(w, wq, sw, stream=None):
    _need(w, torch.bfloat16, "w"); _need(wq, torch.uint8, "wq"); _need(sw, torch.float32, "sw")
    N, K = w.shape
    _check("epilora_quant_weight_fp8", lib().epilora_quant_weight_fp8(_ptr(w), N, K, _ptr(wq), _ptr(sw),
                                                                      _stream(stream)))


def epilora_quant_weight_fp4(w, wc, bs, gs, ws, stream=None):
    _need(w, torch.bfloat16, "w"); _need(wc, torch.uint8, "wc"); _need(bs, torch.uint8, "bs")
    _need(gs, torch.float32, "gs"); _need(ws, torch.uint8, "ws")
    N, K = w.shape
    _check("epilora_quant_weight_fp4", lib().epilora_quant_weight_fp4(
        _ptr(w), N, K, _ptr(wc), _ptr(bs), _ptr(gs), _ptr(ws), ws.numel(), _stream(stream)))


# --- adapters ------------------------------------------------------------------------

def epilora_lora_shrink(x, A, idx, z, ws, ranks=None, mask=None, sa=None, stream=None):
    """x: bf16 [M][K]; A: bf16 [L][r][K], or [L][S][r][K] for per-slice
    adapters (then z is [M][S r]); uint8 E4M3 codes with row scales sa
    ([L][r] or [L][S][r]) for FP8-stored adapters; idx: int32 [M]; z: fp32."""
    _need(x, torch.bfloat16, "x"); _need(idx, torch.int32, "idx")
    _need(z, torch.float32, "z"); _need(ranks, torch.int32, "ranks"); _need(mask, torch.uint8, "mask")
    _need(A, torch.uint8 if sa is not None else torch.bfloat16, "A"); _need(sa, torch.float32, "sa")
    M, K = x.shape
    if A.dim() == 4 or sa is not None:
        L, S, r = (A.shape[0], A.shape[1], A.shape[2]) if A.dim() == 4 else (A.shape[0], 1, A.shape[1])
        _check("epilora_lora_shrink_ex", lib().epilora_lora_shrink_ex(
            _ptr(x), M, K, _ld(x), _ptr(A), A_FP8 if sa is not None else A_BF16, _ptr(sa), L, S, r, _ptr(ranks),
            _ptr(idx), _ptr(mask), _ptr(z), _ptr(ws), ws.numel(), _stream(stream)))
        return
    L, r, _ = A.shape
    _check("epilora_lora_shrink", lib().epilora_lora_shrink(
        _ptr(x), M, K, _ld(x), _ptr(A), L, r, _ptr(ranks), _ptr(idx), _ptr(mask), _ptr(z),
        _ptr(ws), ws.numel(), _stream(stream)))


def epilora_rmsnorm_quant_shrink(x, gamma, eps, xq, sx, *, xn=None, A=None, idx=None, z=None, ws=None,
                                 ranks=None, mask=None, sa=None, stream=None):
    """RMS normalization of x (bf16 [M][K]) with gamma (bf16 [K]), the
    per-token FP8 quantizer of the result into xq / sx, the normalized rows
    into xn (optional), and with A the shrink of the normalized rows into z
    (A as for epilora_lora_shrink)."""
    _need(x, torch.bfloat16, "x"); _need(gamma, torch.bfloat16, "gamma"); _need(xn, torch.bfloat16, "xn")
    _need(xq, torch.uint8, "xq"); _need(sx, torch.float32, "sx"); _need(z, torch.float32, "z")
    _need(idx, torch.int32, "idx"); _need(ranks, torch.int32, "ranks"); _need(mask, torch.uint8, "mask")
    _need(A, torch.uint8 if sa is not None else torch.bfloat16, "A"); _need(sa, torch.float32, "sa")
    M, K = x.shape
    L = S = r = 0
    if A is not None:
        L, S, r = (A.shape[0], A.shape[1], A.shape[2]) if A.dim() == 4 else (A.shape[0], 1, A.shape[1])
    _check("epilora_rmsnorm_quant_shrink", lib().epilora_rmsnorm_quant_shrink(
        _ptr(x), M, K, _ld(x), _ptr(gamma), float(eps), _ptr(xn), 0 if xn is None else _ld(xn), _ptr(xq),
        0 if xq is None else _ld(xq),
        _ptr(sx), _ptr(A), A_FP8 if sa is not None else A_BF16, _ptr(sa), L, S, r, _ptr(ranks), _ptr(idx),
        _ptr(mask), _ptr(z), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def _slice_array(slices):
    arr = (ctypes.c_int64 * 4)()
    for i, n in enumerate(slices or ()):
        arr[i] = int(n)
    return arr


def epilora_lora_expand_add(z, B, idx, scale, y, ws, ranks=None, mask=None, slices=None, sb=None, stream=None):
    """y[t] += s * B[idx[t]] z[t] (bf16, in place) for active tokens;
    `slices`: output slice widths of a projection with per-slice adapters;
    sb: row scales of an FP8-stored B (uint8 codes)."""
    _need(z, torch.float32, "z"); _need(idx, torch.int32, "idx"); _need(y, torch.bfloat16, "y")
    _need(B, torch.uint8 if sb is not None else torch.bfloat16, "B"); _need(sb, torch.float32, "sb")
    M, N = y.shape
    L, _, r = B.shape
    if slices or sb is not None:
        _check("epilora_lora_expand_add_ex", lib().epilora_lora_expand_add_ex(
            _ptr(z), M, N, _ptr(B), A_FP8 if sb is not None else A_BF16, _ptr(sb), L, r,
            len(slices) if slices else 1, _slice_array(slices) if slices else None, _ptr(ranks), _ptr(idx),
            _ptr(mask), float(scale), _ptr(y), _ld(y), _ptr(ws), ws.numel(), _stream(stream)))
        return
    _check("epilora_lora_expand_add", lib().epilora_lora_expand_add(
        _ptr(z), M, N, _ptr(B), L, r, _ptr(ranks), _ptr(idx), _ptr(mask), float(scale), _ptr(y), _ld(y),
        _ptr(ws), ws.numel(), _stream(stream)))


def _weights(a, w, sw=None, bs=None, gs=None):
    _need(w, torch.uint8, "w")
    if bs is None:
        _need(sw, torch.float32, "sw")
        a.wfmt, a.w, a.sw = W_FP8, _ptr(w), _ptr(sw)
    else:
        _need(bs, torch.uint8, "bs"); _need(gs, torch.float32, "gs")
        a.wfmt, a.w, a.bs, a.gs = W_FP4, _ptr(w), _ptr(bs), _ptr(gs)


def _adapters(a, A, B, idx, ranks, mask, scale, slices=None, sa=None, sb=None):
    fp8 = sa is not None or sb is not None
    ad_t = torch.uint8 if fp8 else torch.bfloat16
    _need(A, ad_t, "A"); _need(B, ad_t, "B"); _need(idx, torch.int32, "idx")
    _need(ranks, torch.int32, "ranks"); _need(mask, torch.uint8, "mask")
    _need(sa, torch.float32, "sa"); _need(sb, torch.float32, "sb")
    if fp8:
        a.afmt, a.sa, a.sb = A_FP8, _ptr(sa), _ptr(sb)
    if B is not None:
        a.L, a.r = B.shape[0], B.shape[2]
    elif A is not None:
        a.L, a.r = A.shape[0], A.shape[-2]
    a.A, a.B, a.idx, a.ranks, a.mask = _ptr(A), _ptr(B), _ptr(idx), _ptr(ranks), _ptr(mask)
    a.scale = float(scale)
    if slices:
        a.nslices = len(slices)
        a.slice_n = _slice_array(slices)


def epilora_gemm_lora(xq, sx, w, y, *, sw=None, bs=None, gs=None, z=None, B=None, idx=None, ranks=None,
                      mask=None, scale=1.0, ws=None, slices=None, sb=None, x16=None, stream=None):
    """y = bf16(dequant(w . xq) [+ s B[idx] z on active rows]); z=None: base
    only; `slices`: output slice widths (per-slice adapters, z [M][S r]);
    x16 (bf16 [M][K], with xq = sx = None): the matched W8A16 GEMM."""
    _need(xq, torch.uint8, "xq"); _need(sx, torch.float32, "sx"); _need(y, torch.bfloat16, "y")
    _need(z, torch.float32, "z"); _need(x16, torch.bfloat16, "x16")
    a = LayerArgs()
    a.M, a.K = (x16 if x16 is not None else xq).shape
    a.N = y.shape[1]
    if x16 is not None:
        a.amode, a.x, a.ldx = ACT_BF16, _ptr(x16), _ld(x16)
    else:
        a.xq, a.sx, a.ldq = _ptr(xq), _ptr(sx), _ld(xq)
    _weights(a, w, sw, bs, gs)
    _adapters(a, None, B, idx, ranks, mask, scale, slices, None, sb)
    a.z = _ptr(z)
    a.y, a.ldy = _ptr(y), _ld(y)
    if ws is not None:
        a.ws, a.ws_bytes = _ptr(ws), ws.numel()
    _check("epilora_gemm_lora", lib().epilora_gemm_lora(ctypes.byref(a), _stream(stream)))


def epilora_decode_lora_noalloc(x, w, y, *, sw=None, bs=None, gs=None, A=None, B=None, idx=None, ranks=None,
                                mask=None, scale=1.0, xq_out=None, sx_out=None, slices=None, sa=None, sb=None,
                                stream=None):
    """The fused decode path on the library's fixed per-GPU scratch (no
    workspace argument; see the header)."""
    a = _decode_args(x, w, y, sw, bs, gs, A, B, idx, ranks, mask, scale, None, xq_out, sx_out, slices, sa, sb)
    _check("epilora_decode_lora_noalloc", lib().epilora_decode_lora_noalloc(ctypes.byref(a), _stream(stream)))


def epilora_decode_lora(x, w, y, *, sw=None, bs=None, gs=None, A=None, B=None, idx=None, ranks=None, mask=None,
                        scale=1.0, ws=None, xq_out=None, sx_out=None, slices=None, sa=None, sb=None, a16=False,
                        stream=None):
    """The fused decode path: quantization, shrink and GEMM in one launch;
    `slices`: output slice widths (per-slice adapters, A [L][S][r][K]);
    sa, sb: row scales of FP8-stored adapters (A, B uint8 codes); a16: the
    matched W8A16 GEMM on the bf16 x (no quantization)."""
    a = _decode_args(x, w, y, sw, bs, gs, A, B, idx, ranks, mask, scale, ws, xq_out, sx_out, slices, sa, sb)
    a.amode = ACT_BF16 if a16 else ACT_FP8
    _check("epilora_decode_lora", lib().epilora_decode_lora(ctypes.byref(a), _stream(stream)))


def _decode_args(x, w, y, sw, bs, gs, A, B, idx, ranks, mask, scale, ws, xq_out, sx_out, slices=None, sa=None,
                 sb=None):
    _need(x, torch.bfloat16, "x"); _need(y, torch.bfloat16, "y")
    _need(xq_out, torch.uint8, "xq_out"); _need(sx_out, torch.float32, "sx_out")
    a = LayerArgs()
    a.M, a.K = x.shape
    a.N = y.shape[1]
    a.x, a.ldx = _ptr(x), _ld(x)
    _weights(a, w, sw, bs, gs)
    _adapters(a, A, B, idx, ranks, mask, scale, slices, sa, sb)
    a.y, a.ldy = _ptr(y), _ld(y)
    a.xq_out, a.sx_out = _ptr(xq_out), _ptr(sx_out)
    a.ldq_out = 0 if xq_out is None else _ld(xq_out)
    if ws is not None:
        a.ws, a.ws_bytes = _ptr(ws), ws.numel()
    return a
