"""Helpers for the GPU parity tests: move the seeded inputs to the device, run
the library's paths through the C ABI, and compare with the CPU oracle.

Tolerance on the bf16 outputs against the oracle's fp64 result y_ref:
max |dY| <= 2e-2 * rms(y_ref) and sum |dY| / sum |y_ref| <= 5e-3 over one
GEMM call's outputs.  Quantized activations, scales and weight codes must be
bit-exact."""

import numpy as np
import torch

import fp4_gemm_amd as ep
import oracle

DEV = "cuda"
MAX_REL_RMS = 2e-2
MEAN_REL = 5e-3


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_np(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_np_to_f64(u):
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def compare(y_bits, y_ref, what=""):
    """Check bf16 GPU output bits against the oracle's fp64 y; returns the
    two error measures."""
    y = bf16_np_to_f64(y_bits)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    d = np.abs(y - y_ref)
    rms = np.sqrt(np.mean(y_ref ** 2))
    max_rel = d.max() / rms if rms > 0 else d.max()
    mean_rel = d.sum() / np.abs(y_ref).sum() if np.abs(y_ref).sum() > 0 else d.sum()
    assert max_rel <= MAX_REL_RMS, f"{what}: max|dY| = {max_rel:.3e} rms"
    assert mean_rel <= MEAN_REL, f"{what}: mean rel = {mean_rel:.3e}"
    return max_rel, mean_rel


class DeviceGemm:
    """One projection's inputs on the device, weights quantized by the
    library's own load-time quantizer."""

    def __init__(self, g, wfmt="fp8", x=None, afmt="bf16", a16=False):
        lay = g.layer
        self.g, self.wfmt, self.afmt, self.a16 = g, wfmt, afmt, a16
        self.M, self.K, self.N = g.M, g.K, g.N
        self.x_np = g.x() if x is None else x
        self.w_np = g.w()
        self.x = to_dev(self.x_np)
        w = to_dev(self.w_np)
        if wfmt == "fp8":
            self.wq = torch.empty(self.N, self.K, dtype=torch.uint8, device=DEV)
            self.sw = torch.empty(self.N, dtype=torch.float32, device=DEV)
            ep.epilora_quant_weight_fp8(w, self.wq, self.sw)
            self.wkw = dict(sw=self.sw)
        else:
            self.wq = torch.empty(self.N, self.K // 2, dtype=torch.uint8, device=DEV)
            self.bs = torch.empty(self.N, self.K // 16, dtype=torch.uint8, device=DEV)
            self.gs = torch.empty(1, dtype=torch.float32, device=DEV)
            ws = ep.new_workspace(ep.OP_QUANT_W4, 1, self.N, self.K, 16)
            ep.epilora_quant_weight_fp4(w, self.wq, self.bs, self.gs, ws)
            self.wkw = dict(bs=self.bs, gs=self.gs)
        del w
        self.slices = g.slices
        self.S = len(g.slices) if g.slices else 1
        self.A_np = g.A_sliced() if g.slices else g.A()
        self.B_np = g.B()
        self.A = to_dev(self.A_np)
        self.B = to_dev(self.B_np)
        self.akw, self.bkw, self.adkw = {}, {}, {}
        if afmt == "fp8":
            # adapters stored in FP8: the library's per-row quantizer on the
            # rows of A (length K) and of B (length r)
            A8 = torch.empty(self.A.shape, dtype=torch.uint8, device=DEV)
            B8 = torch.empty(self.B.shape, dtype=torch.uint8, device=DEV)
            self.sa = torch.empty(self.A.shape[:-1], dtype=torch.float32, device=DEV)
            self.sb = torch.empty(self.B.shape[:-1], dtype=torch.float32, device=DEV)
            ep.epilora_quant_weight_fp8(self.A.reshape(-1, self.K), A8.view(-1, self.K), self.sa.view(-1))
            ep.epilora_quant_weight_fp8(self.B.reshape(-1, self.B.shape[-1]), B8.view(-1, self.B.shape[-1]),
                                        self.sb.view(-1))
            self.A, self.B = A8, B8
            self.akw, self.bkw = dict(sa=self.sa), dict(sb=self.sb)
            self.adkw = dict(sa=self.sa, sb=self.sb)
        self.idx = to_dev(lay.idx.astype(np.int32))
        self.mask = None if lay.mask is None else to_dev(lay.mask.astype(np.uint8))
        self.ranks = None if lay.ranks is None else to_dev(lay.ranks.astype(np.int32))
        self.scale = lay.scale
        self.r = lay.r

    # -- the separate kernels: quant, shrink, GEMM with the epilogue --------
    def quant(self):
        xq = torch.empty(self.M, self.K, dtype=torch.uint8, device=DEV)
        sx = torch.empty(self.M, dtype=torch.float32, device=DEV)
        ep.epilora_quant_act(self.x, xq, sx)
        return xq, sx

    def shrink(self, ws=None):
        ws = ws if ws is not None else ep.new_workspace(ep.OP_SHRINK, self.M, self.N, self.K, self.r * self.S)
        # NaN-filled: every word, inactive rows included, must be written
        z = torch.full((self.M, self.r * self.S), float("nan"), dtype=torch.float32, device=DEV)
        ep.epilora_lora_shrink(self.x, self.A, self.idx, z, ws, ranks=self.ranks, mask=self.mask, **self.akw)
        return z, ws

    def gemm(self, xq, sx, z=None, ws=None):
        """The GEMM; xq = sx = None with a16: the W8A16 GEMM on x."""
        y = torch.empty(self.M, self.N, dtype=torch.bfloat16, device=DEV)
        x16 = self.x if self.a16 else None
        if z is None:
            ep.epilora_gemm_lora(xq, sx, self.wq, y, x16=x16, **self.wkw)
        else:
            ws = ws if ws is not None else ep.new_workspace(ep.OP_GEMM, self.M, self.N, self.K, self.r)
            ep.epilora_gemm_lora(xq, sx, self.wq, y, z=z, B=self.B, idx=self.idx, ranks=self.ranks,
                                 mask=self.mask, scale=self.scale, ws=ws, slices=self.slices, x16=x16,
                                 **self.bkw, **self.wkw)
        return y

    def separate(self):
        xq, sx = (None, None) if self.a16 else self.quant()
        z, ws = self.shrink()
        y = self.gemm(xq, sx, z, ws)
        return dict(xq=xq, sx=sx, z=z, y=y, ws=ws)

    def decode(self, ws=None, keep_xq=True):
        ws = ws if ws is not None else ep.new_workspace(ep.OP_DECODE, self.M, self.N, self.K, self.r * self.S)
        y = torch.empty(self.M, self.N, dtype=torch.bfloat16, device=DEV)
        keep_xq = keep_xq and not self.a16
        xq = torch.empty(self.M, self.K, dtype=torch.uint8, device=DEV) if keep_xq else None
        sx = torch.empty(self.M, dtype=torch.float32, device=DEV) if keep_xq else None
        ep.epilora_decode_lora(self.x, self.wq, y, A=self.A, B=self.B, idx=self.idx, ranks=self.ranks,
                               mask=self.mask, scale=self.scale, ws=ws, xq_out=xq, sx_out=sx,
                               slices=self.slices, a16=self.a16, **self.adkw, **self.wkw)
        return dict(xq=xq, sx=sx, y=y, ws=ws)

    # -- the oracle on the same inputs ----------------------------------------
    def oracle(self, rows=None, cols=None):
        """The oracle's result; with cols, only those output channels (the
        oracle then quantizes only those weight rows)."""
        lay = self.g.layer
        w = self.w_np if cols is None else self.w_np[np.asarray(cols)]
        B = self.B_np if cols is None else self.B_np[:, np.asarray(cols)]
        if self.wfmt == "fp8":
            wq, sw = oracle.quant_weight_fp8(w)
            wkw = dict(wq=wq, sw=sw)
        else:
            wc, bs, gs = oracle.quant_weight_fp4(self.w_np, rows=cols)
            wkw = dict(wc=wc, bs=bs, gs=gs)
        A_or, B_full, akw = self.A_np, self.B_np, {}
        if self.afmt == "fp8":
            A_or, sa = oracle.quant_adapter_fp8(self.A_np)
            B_full, sb = oracle.quant_adapter_fp8(self.B_np)
            assert np.array_equal(to_np(self.A), A_or) and np.array_equal(to_np(self.sa), sa), "adapter codes"
            assert np.array_equal(to_np(self.B), B_full) and np.array_equal(to_np(self.sb), sb), "adapter codes"
            akw = dict(sa=sa, sb=sb)
        if self.a16:
            akw["a16"] = True
        if self.slices:
            out = oracle.linear_lora_sliced(self.x_np, A_or, B_full, lay.idx, lay.scale, self.slices,
                                            ranks=lay.ranks, mask=lay.mask, rows=rows, cols=cols,
                                            weights_of_cols=cols is not None, **akw, **wkw)
        else:
            Bsel = B_full if cols is None else B_full[:, np.asarray(cols)]
            if "sb" in akw and cols is not None:
                akw["sb"] = akw["sb"][:, np.asarray(cols)]
            out = oracle.linear_lora(self.x_np, A_or, Bsel, lay.idx, lay.scale, ranks=lay.ranks,
                                     mask=lay.mask, rows=rows, **akw, **wkw)
        out["w"] = wkw
        return out
