"""The C ABI on the host, without a GPU: the library loads, exports every
function include/epilora.h declares, and rejects bad arguments with the
documented status codes before any HIP call."""

import ctypes
import os
import re

import pytest

import fp4_gemm_amd as ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "epilora.h")

# fake, 256-byte-aligned "device" addresses: validation must reject the call
# before anything dereferences them
P = 0x10000
P2 = 0x20000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(epilora_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return ep.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) == 17
    for n in names:
        assert hasattr(L, n), n
        assert n in ep.SIGNATURES, n
    assert set(ep.SIGNATURES) == set(names)


def test_version_and_strerror(L):
    assert L.epilora_version() == 10000
    for code in range(5):
        assert L.epilora_strerror(code)
    assert L.epilora_strerror(99) == b"unknown status"


def test_layer_args_layout_matches_header():
    # 3 sizes, x+ldx, xq+sx+ldq, wfmt(+pad), 4 weight ptrs, L+r, 6 ptrs, scale(+pad),
    # y+ldy, xq_out+sx_out+ldq_out, ws+ws_bytes
    assert ctypes.sizeof(ep.LayerArgs) == 8 * 3 + 16 + 24 + 8 + 32 + 8 + 48 + 8 + 16 + 24 + 16 + 8 + 32 + 24 + 8
    assert ep.LayerArgs.slice_n.offset == 8 * 3 + 16 + 24 + 8 + 32 + 8 + 48 + 8 + 16 + 24 + 16 + 8
    assert ep.LayerArgs.scale.offset == 8 * 3 + 16 + 24 + 8 + 32 + 8 + 48


def test_workspace_bytes(L):
    assert L.epilora_workspace_bytes(ep.OP_GEMM, 64, 4096, 4096, 64) == 256
    assert L.epilora_workspace_bytes(ep.OP_EXPAND, 64, 4096, 4096, 64) == 256
    assert L.epilora_workspace_bytes(ep.OP_QUANT_W4, 1, 1, 32, 16) == 256
    s1 = L.epilora_workspace_bytes(ep.OP_SHRINK, 1, 0, 4096, 64)
    s2 = L.epilora_workspace_bytes(ep.OP_SHRINK, 2048, 0, 14336, 128)
    assert 256 < s1 < s2 and s1 % 256 == 0 and s2 % 256 == 0
    d = L.epilora_workspace_bytes(ep.OP_DECODE, 32, 4096, 14336, 64)
    assert d >= 32 * 14336 + 32 * 64 * 4
    assert L.epilora_workspace_bytes(99, 1, 1, 1, 1) == 0
    assert L.epilora_workspace_bytes(ep.OP_SHRINK, -1, 0, 4096, 64) == 0


def test_quant_act_validation(L):
    q = L.epilora_quant_act
    assert q(P, 0, 4096, 4096, P2, 4096, P, None) == ep.OK            # M = 0 is a no-op
    assert q(P, -1, 4096, 4096, P2, 4096, P, None) == ep.ERR_INVALID_ARG
    assert q(None, 2, 4096, 4096, P2, 4096, P, None) == ep.ERR_INVALID_ARG
    assert q(P, 2, 4096, 4000, P2, 4096, P, None) == ep.ERR_INVALID_ARG   # ldx < K
    assert q(P, 2, 4104, 4104, P2, 4104, P, None) == ep.ERR_UNSUPPORTED   # K % 16
    assert q(P + 8, 2, 4096, 4096, P2, 4096, P, None) == ep.ERR_UNSUPPORTED  # alignment


def test_weight_quant_validation(L):
    assert L.epilora_quant_weight_fp8(P, 4, 40, P2, P, None) == ep.ERR_UNSUPPORTED
    assert L.epilora_quant_weight_fp8(None, 4, 64, P2, P, None) == ep.ERR_INVALID_ARG
    f4 = L.epilora_quant_weight_fp4
    assert f4(P, 4, 48, P2, P, P, P, 256, None) == ep.ERR_UNSUPPORTED        # K % 32
    assert f4(P, 4, 64, P2, P, P, None, 0, None) == ep.ERR_WORKSPACE
    assert f4(P, 4, 64, P2, P, P, P, 255, None) == ep.ERR_WORKSPACE


def test_shrink_validation(L):
    s = L.epilora_lora_shrink
    ws_need = L.epilora_workspace_bytes(ep.OP_SHRINK, 4, 0, 256, 16)
    args = dict(x=P, M=4, K=256, ldx=256, A=P, Lslots=4, r=16, ranks=None, idx=P, mask=None, z=P2)

    def call(ws=P, ws_bytes=ws_need, **kw):
        a = dict(args, **kw)
        return s(a["x"], a["M"], a["K"], a["ldx"], a["A"], a["Lslots"], a["r"], a["ranks"], a["idx"],
                 a["mask"], a["z"], ws, ws_bytes, None)

    assert call(r=20) == ep.ERR_UNSUPPORTED
    assert call(r=144) == ep.ERR_UNSUPPORTED
    assert call(r=0) == ep.ERR_INVALID_ARG
    assert call(idx=None) == ep.ERR_INVALID_ARG
    assert call(A=None) == ep.ERR_INVALID_ARG
    assert call(Lslots=-1) == ep.ERR_INVALID_ARG
    assert call(ws=None) == ep.ERR_WORKSPACE
    assert call(ws_bytes=ws_need - 1) == ep.ERR_WORKSPACE
    assert call(ws=P + 16) == ep.ERR_UNSUPPORTED
    assert call(M=0) == ep.OK


def _layer(**kw):
    a = ep.LayerArgs()
    a.M, a.N, a.K = 4, 512, 256
    a.x, a.ldx = P, 256
    a.xq, a.sx, a.ldq = P, P, 256
    a.wfmt, a.w, a.sw = ep.W_FP8, P, P
    a.L, a.r, a.B, a.A, a.idx = 4, 16, P, P, P
    a.y, a.ldy = P2, 512
    a.ws, a.ws_bytes = P, 1 << 20
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_gemm_lora_validation(L):
    g = lambda **kw: L.epilora_gemm_lora(ctypes.byref(_layer(**kw)), None)
    assert L.epilora_gemm_lora(None, None) == ep.ERR_INVALID_ARG
    assert g(wfmt=7) == ep.ERR_INVALID_ARG
    assert g(K=48, ldq=48) == ep.ERR_UNSUPPORTED
    assert g(sw=None) == ep.ERR_INVALID_ARG
    assert g(wfmt=ep.W_FP4) == ep.ERR_INVALID_ARG       # no block scales
    assert g(ldy=100) == ep.ERR_INVALID_ARG
    assert g(z=P, B=None) == ep.ERR_INVALID_ARG
    assert g(z=P, ws=None) == ep.ERR_WORKSPACE
    assert g(z=P, r=24) == ep.ERR_UNSUPPORTED
    assert g(M=0) == ep.OK and g(N=0) == ep.OK


def _sl(*w):
    arr = (ctypes.c_int64 * 4)()
    for i, v in enumerate(w):
        arr[i] = v
    return arr


def test_slice_validation(L):
    g = lambda **kw: L.epilora_gemm_lora(ctypes.byref(_layer(z=P, **kw)), None)
    assert g(nslices=5, slice_n=_sl(128, 128, 128, 128)) == ep.ERR_INVALID_ARG      # at most 4 slices
    assert g(nslices=2, slice_n=_sl(256, 128)) == ep.ERR_INVALID_ARG                # widths do not sum to N
    assert g(nslices=2, slice_n=_sl(512, 0)) == ep.ERR_INVALID_ARG                  # empty slice
    assert g(nslices=2, slice_n=_sl(248, 264)) == ep.ERR_UNSUPPORTED                # not whole 16-row tiles
    assert g(M=100, nslices=2, slice_n=_sl(256 + 64, 192)) == ep.ERR_UNSUPPORTED    # prefill: 128-wide tiles
    d = lambda **kw: L.epilora_decode_lora(ctypes.byref(_layer(**kw)), None)
    assert d(nslices=3, slice_n=_sl(256, 128, 112)) == ep.ERR_INVALID_ARG
    assert d(nslices=3, slice_n=_sl(256, 136, 120)) == ep.ERR_UNSUPPORTED
    sh = L.epilora_lora_shrink_ex
    assert sh(P, 4, 256, 256, P, 0, None, 4, 0, 16, None, P, None, P, P, 1 << 20, None) == ep.ERR_INVALID_ARG
    assert sh(P, 4, 256, 256, P, 0, None, 4, 5, 16, None, P, None, P, P, 1 << 20, None) == ep.ERR_INVALID_ARG
    assert sh(P, 65536, 256, 256, P, 0, None, 4, 3, 16, None, P, None, P, P, 1 << 40, None) == ep.ERR_UNSUPPORTED
    e = L.epilora_lora_expand_add_ex
    assert e(P, 4, 512, P, 0, None, 4, 16, 2, _sl(500, 10), None, P, None, 2.0, P2, 512, P, 256,
             None) == ep.ERR_INVALID_ARG


def test_fp8_adapter_validation(L):
    g = lambda **kw: L.epilora_gemm_lora(ctypes.byref(_layer(z=P, **kw)), None)
    assert g(afmt=2) == ep.ERR_INVALID_ARG
    assert g(afmt=ep.A_FP8) == ep.ERR_INVALID_ARG                  # no B row scales
    assert g(afmt=ep.A_FP8, sb=P + 4) == ep.ERR_UNSUPPORTED        # scales not 16-byte aligned
    d = lambda **kw: L.epilora_decode_lora(ctypes.byref(_layer(**kw)), None)
    assert d(afmt=ep.A_FP8, sb=P) == ep.ERR_INVALID_ARG            # no A row scales
    sh = L.epilora_lora_shrink_ex
    assert sh(P, 4, 256, 256, P, ep.A_FP8, None, 4, 1, 16, None, P, None, P, P, 1 << 20, None) == ep.ERR_INVALID_ARG
    e = L.epilora_lora_expand_add_ex
    assert e(P, 4, 512, P, ep.A_FP8, None, 4, 16, 1, None, None, P, None, 2.0, P2, 512, P, 256,
             None) == ep.ERR_INVALID_ARG
    # the workspace need grows with the slices
    w1 = L.epilora_workspace_bytes(ep.OP_DECODE, 8, 6144, 4096, 64)
    w3 = L.epilora_workspace_bytes(ep.OP_DECODE, 8, 6144, 4096, 3 * 64)
    assert w3 > w1


def test_decode_validation(L):
    d = lambda **kw: L.epilora_decode_lora(ctypes.byref(_layer(**kw)), None)
    assert d(M=65) == ep.ERR_UNSUPPORTED
    assert d(x=None) == ep.ERR_INVALID_ARG
    assert d(A=None) == ep.ERR_INVALID_ARG
    assert d(ws_bytes=100) == ep.ERR_WORKSPACE
    assert d(xq_out=P, ldq_out=100) == ep.ERR_INVALID_ARG
    assert d(M=0) == ep.OK


def test_expand_validation(L):
    e = L.epilora_lora_expand_add
    assert e(P, 4, 512, P, 4, 16, None, None, None, 2.0, P2, 100, P, 256, None) == ep.ERR_INVALID_ARG
    assert e(P, 4, 512, None, 4, 16, None, P, None, 2.0, P2, 512, P, 256, None) == ep.ERR_INVALID_ARG
    assert e(P, 4, 512, P, 4, 16, None, P, None, 2.0, P2, 512, None, 0, None) == ep.ERR_WORKSPACE


def test_workspace_and_error_validation(L):
    assert L.epilora_workspace_init(None, 256, None) == ep.ERR_WORKSPACE
    assert L.epilora_workspace_init(P, 100, None) == ep.ERR_WORKSPACE
    assert L.epilora_device_error(None, 0, None, None) == ep.ERR_INVALID_ARG


def test_binding_without_gpu_refuses_cpu_tensors():
    import torch
    x = torch.zeros(2, 32, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        ep.epilora_quant_act(x, torch.zeros(2, 32, dtype=torch.uint8), torch.zeros(2))


def test_norm_validation(L):
    n = L.epilora_rmsnorm_quant_shrink
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("x", P), ("M", 4), ("K", 256), ("ldx", 256), ("gamma", P), ("eps", 1e-5), ("xn", None), ("ldn", 0),
        ("xq", P2), ("ldq", 256), ("sx", P), ("A", None), ("afmt", 0), ("sa", None), ("L", 0), ("S", 1),
        ("r", 16), ("ranks", None), ("idx", None), ("mask", None), ("z", None), ("ws", None), ("wsb", 0),
        ("stream", None))]
    assert n(*args(M=0)) == ep.OK
    assert n(*args(gamma=None)) == ep.ERR_INVALID_ARG
    assert n(*args(eps=-1.0)) == ep.ERR_INVALID_ARG
    assert n(*args(K=264, ldx=272, ldq=272)) == ep.ERR_UNSUPPORTED
    assert n(*args(xn=P, ldn=100)) == ep.ERR_INVALID_ARG
    assert n(*args(A=P, L=4, idx=P, z=P)) == ep.ERR_WORKSPACE          # the shrink needs a workspace
    assert n(*args(A=P, L=4, idx=P, z=None, ws=P, wsb=1 << 20)) == ep.ERR_INVALID_ARG


def test_w8a16_validation(L):
    g = lambda **kw: L.epilora_gemm_lora(ctypes.byref(_layer(**kw)), None)
    assert g(amode=2) == ep.ERR_INVALID_ARG
    assert g(amode=ep.ACT_BF16, x=None) == ep.ERR_INVALID_ARG
    assert g(amode=ep.ACT_BF16, wfmt=ep.W_FP4, bs=P, gs=P) == ep.ERR_UNSUPPORTED   # FP8 weights only
    assert g(amode=ep.ACT_BF16, xq=None, sx=None, M=0) == ep.OK
    d = lambda **kw: L.epilora_decode_lora(ctypes.byref(_layer(**kw)), None)
    assert d(amode=ep.ACT_BF16, xq_out=P, ldq_out=256) == ep.ERR_INVALID_ARG     # nothing is quantized
    assert d(amode=ep.ACT_BF16, wfmt=ep.W_FP4, bs=P, gs=P) == ep.ERR_UNSUPPORTED
