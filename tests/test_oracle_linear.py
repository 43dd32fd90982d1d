"""Pins of the oracle's layer arithmetic against things other than itself:
closed forms (the merged update x (BA)^T), torch's independent FP8 decode
and fp64 matmul, linearity, the inactive-row invariant, quantisation error
bounds, and a brute-force 2 x 4 x 8 evaluation written from the
definitions with Python loops."""

import itertools

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits, custom_layer


def t_e4m3(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64)


def t_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64)


def rand_bf16(rng, shape, std):
    return bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


def make(rng, M=6, K=64, N=40, L=3, r=8):
    x = rand_bf16(rng, (M, K), 1.0)
    w = rand_bf16(rng, (N, K), 0.02)
    A = rand_bf16(rng, (L, r, K), 1.0 / np.sqrt(K))
    B = rand_bf16(rng, (L, N, r), 0.01)
    return x, w, A, B


# --- activation quantisation --------------------------------------------------

def test_quant_roundtrip_on_representable_rows():
    """Rows of e4m3 values times 2**k with one element at +-448 * 2**k give
    sx = 2**k exactly and the codes back exactly."""
    rng = np.random.default_rng(10)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    for k in (-12, -5, 0, 3, 7):
        codes = rng.choice(finite, size=(5, 97))
        codes[:, 13] = rng.choice([0x7E, 0xFE], size=5)
        vals = t_e4m3(codes).numpy() * 2.0 ** k
        x = bf16_bits(vals.astype(np.float32))
        assert np.array_equal(t_bf16(x).numpy(), vals)  # exact in bf16
        xq, sx = oracle.quant_act(x)
        assert np.all(sx == np.float32(2.0 ** k))
        assert np.array_equal(xq, codes)


def test_quant_error_bound_and_scale():
    rng = np.random.default_rng(11)
    x = rand_bf16(rng, (64, 1000), 1.0)
    x[3] = 0  # all-zero row
    x[5] = bf16_bits(rng.standard_normal(1000).astype(np.float32) * np.float32(1e-20))
    xq, sx = oracle.quant_act(x)
    xf = t_bf16(x).numpy()
    amax = np.abs(xf).max(axis=1)
    assert sx[3] == 1.0 and np.all(xq[3] == 0)
    nz = amax > 0
    # sx is amax/448 correctly rounded to fp32
    rel = np.abs(sx[nz].astype(np.float64) * 448.0 - amax[nz]) / amax[nz]
    assert rel.max() <= 2.0 ** -24
    # every code is within half an e4m3 step of x/sx (+ the fp32 rounding)
    q = xf / sx[:, None].astype(np.float64)
    dq = t_e4m3(xq).numpy()
    a = np.abs(q)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -9)))
    step = np.where(a >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)
    err = np.abs(dq - q)
    sat = a > 448.0
    assert np.all(err[~sat] <= 0.5 * step[~sat] + a[~sat] * 2.0 ** -23)
    assert np.all(np.abs(dq[sat]) == 448.0) and np.all(a[sat] <= 448.0 * (1 + 2.0 ** -22))
    # the row maximum always lands on +-448
    amax_pos = np.argmax(np.abs(xf), axis=1)
    assert np.all(np.abs(dq[np.arange(64)[nz], amax_pos[nz]]) == 448.0)


# --- base GEMM ------------------------------------------------------------------

def test_base_matches_independent_dequant_matmul():
    """With every index -1 the layer is the base GEMM: torch's own FP8
    decode of both operands, an fp64 matmul, then the two scales."""
    rng = np.random.default_rng(12)
    x, w, A, B = make(rng, M=7, K=96, N=33)
    wq, sw = oracle.quant_weight_fp8(w)
    out = oracle.linear_lora(x, A, B, np.full(7, -1), 2.0, wq=wq, sw=sw)
    Xd = t_e4m3(out["xq"]) * torch.from_numpy(out["sx"].astype(np.float64))[:, None]
    Wd = t_e4m3(wq) * torch.from_numpy(sw.astype(np.float64))[:, None]
    ref = (Xd @ Wd.T).numpy()
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert np.array_equal(out["y"], out["base"])
    # and it approximates the unquantised bf16 product (FP8 error only)
    exact = (t_bf16(x) @ t_bf16(w).T).numpy()
    rms = np.sqrt(np.mean(exact ** 2))
    assert np.sqrt(np.mean((out["y"] - exact) ** 2)) < 0.08 * rms


def test_weight_quant_is_per_output_channel():
    rng = np.random.default_rng(13)
    w = rand_bf16(rng, (9, 50), 0.02)
    w[4] = bf16_bits(t_bf16(w[4]).numpy().astype(np.float32) * np.float32(64.0))
    wq, sw = oracle.quant_weight_fp8(w)
    amax = np.abs(t_bf16(w).numpy()).max(axis=1)
    assert np.allclose(sw * 448.0, amax, rtol=2.0 ** -23)
    assert np.all(np.abs(t_e4m3(wq).numpy()).max(axis=1) == 448.0)


# --- the adapter term -------------------------------------------------------------

def test_lora_term_equals_merged_update():
    """Active rows: y - base = s * x (B A)^T through a dense Delta W = B A
    (the merge the method avoids, as a closed form)."""
    rng = np.random.default_rng(14)
    x, w, A, B = make(rng, M=8, K=80, N=48, L=3, r=8)
    wq, sw = oracle.quant_weight_fp8(w)
    idx = np.array([0, 2, 1, -1, 2, 0, 1, 1])
    s = 2.0
    out = oracle.linear_lora(x, A, B, idx, s, wq=wq, sw=sw)
    xf = t_bf16(x)
    for t in range(8):
        a = idx[t]
        if a < 0:
            assert np.array_equal(out["y"][t], out["base"][t])
            continue
        dW = t_bf16(B[a]) @ t_bf16(A[a])          # [N][K]
        ref = s * (dW @ xf[t]).numpy()
        got = out["y"][t] - out["base"][t]
        assert np.allclose(got, ref, rtol=1e-9, atol=1e-12)
        # z is the down-projection of the bf16 activations
        assert np.allclose(out["z"][t], (t_bf16(A[a]) @ xf[t]).numpy(), rtol=1e-12, atol=1e-14)


def test_lora_linear_in_B():
    rng = np.random.default_rng(15)
    x, w, A, B = make(rng, M=5, K=64, N=24, L=2, r=6)
    wq, sw = oracle.quant_weight_fp8(w)
    idx = np.array([0, 1, 1, 0, -1])
    f = lambda BB: oracle.linear_lora(x, A, BB, idx, 2.0, wq=wq, sw=sw)
    y1 = f(B)
    lora1 = y1["y"] - y1["base"]
    z = oracle.shrink(x, A, idx)
    term = lambda BB: oracle.expand(z, BB, idx, 2.0)[0]
    # doubling B (exact in bf16) doubles the term exactly
    B2 = bf16_bits(t_bf16(B).numpy().astype(np.float32) * np.float32(2.0))
    assert np.array_equal(term(B2), 2.0 * term(B))
    y2 = f(B2)
    assert np.allclose(y2["y"] - y2["base"], 2.0 * lora1, rtol=1e-12, atol=1e-15)
    # B split into two parts with disjoint support: the terms add
    Ba = B.copy(); Ba[:, :, 1::2] = 0
    Bb = B.copy(); Bb[:, :, 0::2] = 0
    la = f(Ba); lb = f(Bb)
    s = (la["y"] - la["base"]) + (lb["y"] - lb["base"])
    assert np.allclose(s, lora1, rtol=1e-12, atol=1e-15)
    assert np.abs(lora1).max() > 0


def test_inactive_rows_equal_base_bitwise():
    rng = np.random.default_rng(16)
    x, w, A, B = make(rng, M=8, K=32, N=16, L=3, r=4)
    wq, sw = oracle.quant_weight_fp8(w)
    idx = np.array([-1, 0, 1, 2, 2, 7, -5, 1])   # 7 and -5 are out of range
    mask = np.array([1, 1, 0, 1, 1, 1, 1, 1], np.uint8)
    ranks = np.array([4, 4, 0])                   # adapter 2 has rank 0
    out = oracle.linear_lora(x, A, B, idx, 2.0, wq=wq, sw=sw, mask=mask, ranks=ranks)
    inactive = [0, 2, 3, 4, 5, 6]
    assert list(np.nonzero(~out["active"])[0]) == inactive
    for t in inactive:
        assert np.array_equal(out["y"][t], out["base"][t])
        assert not out["z"][t].any()
    for t in (1, 7):
        assert np.abs(out["y"][t] - out["base"][t]).max() > 0


def test_ranks_ignore_padding():
    rng = np.random.default_rng(17)
    x, w, A, B = make(rng, M=6, K=48, N=20, L=3, r=8)
    wq, sw = oracle.quant_weight_fp8(w)
    ranks = np.array([8, 3, 5])
    idx = np.array([0, 1, 2, 1, 2, 0])
    Az, Bz = A.copy(), B.copy()
    for a, rk in enumerate(ranks):
        Az[a, rk:] = 0
        Bz[a, :, rk:] = 0
    y_r = oracle.linear_lora(x, A, B, idx, 2.0, wq=wq, sw=sw, ranks=ranks)["y"]
    y_z = oracle.linear_lora(x, Az, Bz, idx, 2.0, wq=wq, sw=sw)["y"]
    assert np.allclose(y_r, y_z, rtol=1e-13, atol=1e-15)
    y_bad = oracle.linear_lora(x, A, B, idx, 2.0, wq=wq, sw=sw)["y"]
    assert np.abs(y_bad - y_z).max() > 1e-4  # the padding would have mattered


def test_token_permutation():
    rng = np.random.default_rng(18)
    x, w, A, B = make(rng, M=9, K=40, N=30, L=3, r=5)
    wq, sw = oracle.quant_weight_fp8(w)
    idx = np.array([0, 1, 2, -1, 0, 1, 2, 2, 0])
    mask = np.array([1, 0, 1, 1, 1, 1, 0, 1, 1], np.uint8)
    perm = rng.permutation(9)
    y = oracle.linear_lora(x, A, B, idx, 2.0, wq=wq, sw=sw, mask=mask)["y"]
    yp = oracle.linear_lora(x[perm], A, B, idx[perm], 2.0, wq=wq, sw=sw, mask=mask[perm])["y"]
    assert np.allclose(yp, y[perm], rtol=1e-13, atol=1e-15)


def test_sampled_rows_and_cols_match_full():
    rng = np.random.default_rng(19)
    x, w, A, B = make(rng, M=10, K=64, N=50, L=3, r=4)
    wq, sw = oracle.quant_weight_fp8(w)
    idx = np.array([0, 1, 2, -1, 0, 1, 2, 2, 0, 1])
    full = oracle.linear_lora(x, A, B, idx, 2.0, wq=wq, sw=sw)["y"]
    rows, cols = np.array([7, 2, 9]), np.array([49, 0, 13, 14])
    part = oracle.linear_lora(x, A, B, idx, 2.0, wq=wq, sw=sw, rows=rows, cols=cols)["y"]
    assert np.allclose(part, full[np.ix_(rows, cols)], rtol=1e-13, atol=1e-15)


# --- brute force on 2 x 4 x 8 -------------------------------------------------------

def _brute(x, w, A, B, idx, mask, ranks, s):
    """The layer from its definition, element by element, in Python floats
    (fp64), with torch's FP8 conversion for the codes."""
    M, K = x.shape
    N = w.shape[0]
    L, r, _ = A.shape
    xf = t_bf16(x).numpy()
    wf = t_bf16(w).numpy()

    def q_rows(v):
        codes = np.zeros(v.shape, np.uint8)
        scales = np.zeros(v.shape[0], np.float32)
        for i in range(v.shape[0]):
            amax = np.float32(max(abs(float(e)) for e in v[i]))
            sc = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
            scales[i] = sc
            for k in range(v.shape[1]):
                qv = np.float32(np.float32(v[i, k]) / sc)
                codes[i, k] = torch.tensor([float(qv)], dtype=torch.float32).to(
                    torch.float8_e4m3fn).view(torch.uint8).item()
        return codes, scales

    xq, sx = q_rows(xf.astype(np.float32))
    wq, sw = q_rows(wf.astype(np.float32))
    dx = t_e4m3(xq).numpy()
    dw = t_e4m3(wq).numpy()
    y = np.zeros((M, N))
    for t in range(M):
        a = int(idx[t])
        rk = r if ranks is None else int(ranks[a]) if 0 <= a < L else 0
        on = 0 <= a < L and (mask is None or mask[t] != 0) and rk > 0
        z = [sum(float(t_bf16(A[a, j, k])) * xf[t, k] for k in range(K)) for j in range(rk)] if on else []
        for n in range(N):
            acc = sum(dx[t, k] * dw[n, k] for k in range(K))
            base = acc * float(sx[t]) * float(sw[n])
            if on:
                base = base + s * sum(float(t_bf16(B[a, n, j])) * z[j] for j in range(rk))
            y[t, n] = base
    return xq, sx, wq, sw, y


def test_brute_force_2x4x8():
    rng = np.random.default_rng(20)
    M, K, N, L, r = 2, 4, 8, 2, 2
    x = rand_bf16(rng, (M, K), 1.0)
    w = rand_bf16(rng, (N, K), 0.02)
    A = rand_bf16(rng, (L, r, K), 0.5)
    B = rand_bf16(rng, (L, N, r), 0.01)
    wq, sw = oracle.quant_weight_fp8(w)
    n_cases = 0
    for i0, i1, m0, m1 in itertools.product((-1, 0, 1), (-1, 0, 1), (0, 1), (0, 1)):
        for ranks in (None, np.array([2, 1]), np.array([0, 2])):
            idx = np.array([i0, i1])
            mask = np.array([m0, m1], np.uint8)
            out = oracle.linear_lora(x, A, B, idx, 2.0, wq=wq, sw=sw, mask=mask, ranks=ranks)
            bxq, bsx, bwq, bsw, by = _brute(x, w, A, B, idx, mask, ranks, 2.0)
            assert np.array_equal(out["xq"], bxq) and np.array_equal(out["sx"], bsx)
            assert np.array_equal(wq, bwq) and np.array_equal(sw, bsw)
            assert np.allclose(out["y"], by, rtol=1e-12, atol=1e-14), (idx, mask, ranks)
            n_cases += 1
    assert n_cases == 108


# --- 4-bit weights -----------------------------------------------------------------

def test_fp4_encoder_error_bound_and_layout():
    rng = np.random.default_rng(21)
    w = rand_bf16(rng, (12, 128), 0.02)
    w[2, 16:32] = 0  # an all-zero block
    wc, bs, gs = oracle.quant_weight_fp4(w)
    assert wc.shape == (12, 64) and bs.shape == (12, 8)
    wf = t_bf16(w).numpy()
    assert gs == np.float32(np.abs(wf).max() / np.float32(2688.0))
    assert bs[2, 1] == 0 and np.all(wc[2, 8:16] == 0)
    # the block holding the global maximum gets the largest scale, 448
    dbs = t_e4m3(bs).numpy()
    assert dbs.max() == 448.0
    ex = oracle.exact_decode_fp4(wc, bs, gs)
    step_scale = np.repeat(dbs, 16, axis=1) * float(gs)
    v = np.where(step_scale > 0, wf / np.where(step_scale > 0, step_scale, 1), 0)
    a = np.abs(v)
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    bound = np.maximum(half, a - 6.0) * step_scale * (1 + 1e-6) + 1e-30
    assert np.all(np.abs(ex - wf) <= bound)
    # swapping the nibble order breaks the bound (the layout is pinned)
    swapped = ((wc >> 4) | (wc << 4)).astype(np.uint8)
    assert np.any(np.abs(oracle.exact_decode_fp4(swapped, bs, gs) - wf) > bound)


def test_fp4_fold_base_exact_when_products_are_short():
    """Codes of one significant bit times normal block scales: the fold is
    exact, so the 4-bit base equals the exact NVFP4 product (dense fp64)."""
    rng = np.random.default_rng(22)
    N, K = 16, 64
    codes = rng.choice([0, 2, 4, 6, 8, 10, 12, 14], size=(N, K)).astype(np.uint8)
    wc = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    bs = rng.integers(0x20, 0x7E, size=(N, K // 16)).astype(np.uint8)  # >= 2**-3
    gs = np.float32(0.001)
    x = rand_bf16(rng, (5, K), 1.0)
    xq, sx = oracle.quant_act(x)
    got = oracle.base_fp4(xq, sx, wc, bs, gs)
    Wex = oracle.exact_decode_fp4(wc, bs, gs)
    ref = (t_e4m3(xq).numpy() * sx[:, None].astype(np.float64)) @ Wex.T
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_fp4_fold_close_to_exact_nvfp4():
    rng = np.random.default_rng(23)
    w = rand_bf16(rng, (64, 256), 0.02)
    x = rand_bf16(rng, (8, 256), 1.0)
    wc, bs, gs = oracle.quant_weight_fp4(w)
    xq, sx = oracle.quant_act(x)
    got = oracle.base_fp4(xq, sx, wc, bs, gs)
    ref = (t_e4m3(xq).numpy() * sx[:, None].astype(np.float64)) @ oracle.exact_decode_fp4(wc, bs, gs).T
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.sqrt(np.mean((got - ref) ** 2)) < 0.05 * rms


def test_workload_layer_through_oracle():
    lay = custom_layer("t", 101, 3, 64, 32, 2, 4, [1, -1, 0])
    g = lay.gemms[0]
    wq, sw = oracle.quant_weight_fp8(g.w())
    out = oracle.linear_lora(g.x(), g.A(), g.B(), lay.idx, lay.scale, wq=wq, sw=sw)
    assert out["y"].shape == (3, 32) and out["active"].tolist() == [True, False, True]


# --- multi-slice projections ----------------------------------------------------------

def _sliced_inputs(rng, M=7, K=48, slice_n=(24, 8, 8), L=3, r=6):
    N = sum(slice_n)
    S = len(slice_n)
    x = rand_bf16(rng, (M, K), 1.0)
    w = rand_bf16(rng, (N, K), 0.02)
    A = rand_bf16(rng, (L, S, r, K), 1.0 / np.sqrt(K))
    B = rand_bf16(rng, (L, N, r), 0.01)
    return x, w, A, B


def test_sliced_equals_block_diagonal_adapter():
    """A multi-slice projection is one adapter of rank S*r whose A stacks the
    slices' A and whose B is block diagonal (slice s's rows use only columns
    s*r .. s*r+r): the unsliced layer on that merged adapter, computed
    through a dense merged update, gives the same outputs."""
    rng = np.random.default_rng(40)
    slice_n = (24, 8, 8)
    x, w, A, B = _sliced_inputs(rng, slice_n=slice_n)
    L, S, r, K = A.shape
    wq, sw = oracle.quant_weight_fp8(w)
    idx = np.array([0, 2, -1, 1, 2, 0, 1])
    ranks = np.array([6, 4, 0])
    mask = np.array([1, 1, 1, 1, 0, 1, 1], np.uint8)
    for a, rk in enumerate(ranks):   # padding past each rank is zero in the data
        A[a, :, rk:] = 0
        B[a, :, rk:] = 0
    out = oracle.linear_lora_sliced(x, A, B, idx, 2.0, slice_n, wq=wq, sw=sw, ranks=ranks, mask=mask)
    Abig = A.reshape(L, S * r, K)
    Bbig = np.zeros((L, B.shape[1], S * r), np.uint16)
    for s, (n0, n1) in enumerate(oracle.slice_bounds(slice_n)):
        Bbig[:, n0:n1, s * r:(s + 1) * r] = B[:, n0:n1]
    ranks_big = np.where(ranks > 0, S * r, 0)
    ref = oracle.linear_lora(x, Abig, Bbig, idx, 2.0, wq=wq, sw=sw, ranks=ranks_big, mask=mask)
    assert np.array_equal(out["active"], ref["active"])
    assert np.allclose(out["y"], ref["y"], rtol=1e-12, atol=1e-15)
    assert np.allclose(out["z"], ref["z"], rtol=1e-12, atol=1e-15)
    # and through the dense merged update B_big A_big of each active token
    xf = t_bf16(x)
    for t in np.nonzero(out["active"])[0]:
        dW = t_bf16(Bbig[idx[t]]) @ t_bf16(Abig[idx[t]])
        assert np.allclose(out["y"][t] - out["base"][t], 2.0 * (dW @ xf[t]).numpy(), rtol=1e-9, atol=1e-12)
    for t in np.nonzero(~out["active"])[0]:
        assert np.array_equal(out["y"][t], out["base"][t])


def test_one_slice_is_the_plain_layer():
    rng = np.random.default_rng(41)
    x, w, A, B = _sliced_inputs(rng, slice_n=(40,))
    wq, sw = oracle.quant_weight_fp8(w)
    idx = np.array([0, 1, 2, -1, 2, 1, 0])
    a = oracle.linear_lora_sliced(x, A, B, idx, 2.0, (40,), wq=wq, sw=sw)
    b = oracle.linear_lora(x, A[:, 0], B, idx, 2.0, wq=wq, sw=sw)
    for k in ("y", "z", "base", "xq", "sx", "active"):
        assert np.array_equal(a[k], b[k]), k


def test_slices_are_independent():
    """Zeroing slice s's down-projection leaves exactly that slice's outputs
    at the base value and changes no other slice's outputs."""
    rng = np.random.default_rng(42)
    slice_n = (16, 8, 16)
    x, w, A, B = _sliced_inputs(rng, slice_n=slice_n)
    wq, sw = oracle.quant_weight_fp8(w)
    idx = np.array([0, 1, 2, 0, 1, 2, 0])
    full = oracle.linear_lora_sliced(x, A, B, idx, 2.0, slice_n, wq=wq, sw=sw)
    bounds = oracle.slice_bounds(slice_n)
    for s, (n0, n1) in enumerate(bounds):
        A0 = A.copy()
        A0[:, s] = 0
        out = oracle.linear_lora_sliced(x, A0, B, idx, 2.0, slice_n, wq=wq, sw=sw)
        assert np.array_equal(out["y"][:, n0:n1], full["base"][:, n0:n1])
        other = np.r_[0:n0, n1:sum(slice_n)]
        assert np.array_equal(out["y"][:, other], full["y"][:, other])
        assert np.abs(full["y"][:, n0:n1] - full["base"][:, n0:n1]).max() > 0


def test_sliced_sampled_columns():
    rng = np.random.default_rng(43)
    slice_n = (24, 8, 8)
    x, w, A, B = _sliced_inputs(rng, slice_n=slice_n)
    wq, sw = oracle.quant_weight_fp8(w)
    idx = np.array([0, 2, -1, 1, 2, 0, 1])
    full = oracle.linear_lora_sliced(x, A, B, idx, 2.0, slice_n, wq=wq, sw=sw)
    cols = np.array([1, 23, 24, 31, 32, 39])
    rows = np.array([0, 3, 6])
    part = oracle.linear_lora_sliced(x, A, B, idx, 2.0, slice_n, wq=wq[cols], sw=sw[cols], rows=rows, cols=cols,
                                     weights_of_cols=True)
    assert np.array_equal(part["y"], full["y"][np.ix_(rows, cols)])


def test_sliced_brute_force():
    """M=2, K=4, N=8 in slices (4, 2, 2), r=2: Python loops straight from the
    definition (fp64), every index and mask combination."""
    rng = np.random.default_rng(44)
    slice_n = (4, 2, 2)
    x, w, A, B = _sliced_inputs(rng, M=2, K=4, slice_n=slice_n, L=2, r=2)
    wq, sw = oracle.quant_weight_fp8(w)
    xf = t_bf16(x).numpy()
    Af, Bf = t_bf16(A).numpy(), t_bf16(B).numpy()
    for i0, i1, m0, m1 in itertools.product([-1, 0, 1], [-1, 0, 1], [0, 1], [0, 1]):
        idx = np.array([i0, i1])
        mask = np.array([m0, m1], np.uint8)
        out = oracle.linear_lora_sliced(x, A, B, idx, 2.0, slice_n, wq=wq, sw=sw, mask=mask)
        for t in range(2):
            for n in range(8):
                s = 0 if n < 4 else (1 if n < 6 else 2)
                want = out["base"][t][n]
                if idx[t] >= 0 and mask[t]:
                    add = 0.0
                    for j in range(2):
                        zt = 0.0
                        for k in range(4):
                            zt += Af[idx[t], s, j, k] * xf[t, k]
                        add += Bf[idx[t], n, j] * zt
                    want = want + 2.0 * add
                assert abs(out["y"][t][n] - want) <= 1e-12 * max(1.0, abs(want))


# --- adapters stored in FP8 -------------------------------------------------------------

def test_fp8_adapters_equal_bf16_layer_on_exact_values():
    """Adapters whose FP8 codes times a power-of-two row scale are exact in
    bf16: the FP8-adapter layer equals the bf16-adapter layer on those
    values (an independently pinned path), for plain and sliced
    projections."""
    rng = np.random.default_rng(50)
    M, K, N, L, r = 6, 64, 40, 3, 8
    x, w, _, _ = make(rng, M=M, K=K, N=N, L=L, r=r)
    wq, sw = oracle.quant_weight_fp8(w)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    A8 = rng.choice(finite, size=(L, r, K)).astype(np.uint8)
    B8 = rng.choice(finite, size=(L, N, r)).astype(np.uint8)
    sa = (2.0 ** rng.integers(-12, -6, size=(L, r))).astype(np.float32)
    sb = (2.0 ** rng.integers(-14, -8, size=(L, N))).astype(np.float32)
    A16 = bf16_bits((t_e4m3(A8).numpy() * sa[..., None]).astype(np.float32))
    B16 = bf16_bits((t_e4m3(B8).numpy() * sb[..., None]).astype(np.float32))
    assert np.array_equal(t_bf16(A16).numpy(), t_e4m3(A8).numpy() * sa[..., None])  # exact
    idx = np.array([0, 2, -1, 1, 2, 0])
    ranks = np.array([8, 5, 3])
    got = oracle.linear_lora(x, A8, B8, idx, 2.0, wq=wq, sw=sw, ranks=ranks, sa=sa, sb=sb)
    ref = oracle.linear_lora(x, A16, B16, idx, 2.0, wq=wq, sw=sw, ranks=ranks)
    assert np.allclose(got["y"], ref["y"], rtol=1e-13, atol=1e-16)
    assert np.allclose(got["z"], ref["z"], rtol=1e-13, atol=1e-16)
    assert np.array_equal(got["y"][2], got["base"][2])
    # sliced: slice s of A8 with its own scales
    A8s = rng.choice(finite, size=(L, 2, r, K)).astype(np.uint8)
    sas = (2.0 ** rng.integers(-12, -6, size=(L, 2, r))).astype(np.float32)
    A16s = bf16_bits((t_e4m3(A8s).numpy() * sas[..., None]).astype(np.float32))
    got = oracle.linear_lora_sliced(x, A8s, B8, idx, 2.0, (24, 16), wq=wq, sw=sw, ranks=ranks, sa=sas, sb=sb)
    ref = oracle.linear_lora_sliced(x, A16s, B16, idx, 2.0, (24, 16), wq=wq, sw=sw, ranks=ranks)
    assert np.allclose(got["y"], ref["y"], rtol=1e-13, atol=1e-16)


def test_fp8_adapter_quantizer_and_error():
    """The stored codes are the per-row rule (each row's largest magnitude
    lands on 448), and the FP8 adapters' term is within the E4M3 rounding of
    the bf16 adapters' term."""
    rng = np.random.default_rng(51)
    x, w, A, B = make(rng, M=8, K=128, N=48, L=3, r=16)
    wq, sw = oracle.quant_weight_fp8(w)
    A8, sa = oracle.quant_adapter_fp8(A)
    B8, sb = oracle.quant_adapter_fp8(B)
    assert A8.shape == A.shape and sa.shape == A.shape[:2] and sb.shape == B.shape[:2]
    assert np.all(np.abs(t_e4m3(A8).numpy()).max(axis=2) == 448.0)
    assert np.allclose(sa * 448.0, np.abs(t_bf16(A).numpy()).max(axis=2), rtol=2.0 ** -23)
    idx = np.array([0, 1, 2, 0, 1, 2, -1, 0])
    q = oracle.linear_lora(x, A8, B8, idx, 2.0, wq=wq, sw=sw, sa=sa, sb=sb)
    b = oracle.linear_lora(x, A, B, idx, 2.0, wq=wq, sw=sw)
    lq, lb = q["y"] - q["base"], b["y"] - b["base"]
    rel = np.sqrt(np.mean((lq - lb) ** 2)) / np.sqrt(np.mean(lb ** 2))
    assert 0 < rel < 0.1          # E4M3 keeps 3 mantissa bits: a few percent
    # doubling every B row scale doubles the term exactly
    z = oracle.shrink(x, A8, idx, a_scale=sa)
    t1 = oracle.expand(z, B8, idx, 2.0, b_scale=sb)[0]
    t2 = oracle.expand(z, B8, idx, 2.0, b_scale=(sb * np.float32(2.0)).astype(np.float32))[0]
    assert np.array_equal(t2, 2.0 * t1) and np.abs(t1).max() > 0
    assert np.allclose(t1, lq, rtol=1e-12, atol=1e-15)


def test_fp8_adapters_brute_force():
    """M=2, K=4, N=8, r=2: Python loops from the definition over the FP8
    decode of each code (torch's float8_e4m3fn) times the row scales."""
    rng = np.random.default_rng(52)
    x, w, A, B = make(rng, M=2, K=4, N=8, L=2, r=2)
    wq, sw = oracle.quant_weight_fp8(w)
    A8, sa = oracle.quant_adapter_fp8(A)
    B8, sb = oracle.quant_adapter_fp8(B)
    Ad, Bd = t_e4m3(A8).numpy(), t_e4m3(B8).numpy()
    xf = t_bf16(x).numpy()
    for i0, i1 in itertools.product([-1, 0, 1], repeat=2):
        idx = np.array([i0, i1])
        out = oracle.linear_lora(x, A8, B8, idx, 2.0, wq=wq, sw=sw, sa=sa, sb=sb)
        for t in range(2):
            for n in range(8):
                want = out["base"][t][n]
                a = idx[t]
                if a >= 0:
                    acc = 0.0
                    for j in range(2):
                        zt = 0.0
                        for k in range(4):
                            zt += Ad[a, j, k] * float(sa[a, j]) * xf[t, k]
                        acc += Bd[a, n, j] * float(sb[a, n]) * zt
                    want = want + 2.0 * acc
                assert abs(out["y"][t][n] - want) <= 1e-12 * max(1.0, abs(want))


# --- the normalization with the quantizer and shrink fused in ------------------------------

def test_rmsnorm_exact_cases():
    """A constant row c = +-2^k with eps = 0 normalizes to +-1 exactly, so
    xn = +-gamma bit for bit; scaling a row by a power of two (eps = 0)
    leaves xn unchanged bit for bit."""
    rng = np.random.default_rng(60)
    K = 96
    gamma = rand_bf16(rng, (K,), 1.0)
    rows = np.array([[2.0 ** k * sgn] * K for k, sgn in ((-3, 1.0), (0, -1.0), (5, 1.0))], np.float32)
    xn = oracle.rmsnorm(bf16_bits(rows), gamma, 0.0)
    for i, sgn in enumerate((1.0, -1.0, 1.0)):
        want = bf16_bits((t_bf16(gamma).numpy() * sgn).astype(np.float32))
        assert np.array_equal(xn[i], want)
    x = rand_bf16(rng, (5, K), 1.0)
    x4 = bf16_bits((t_bf16(x).numpy() * 4.0).astype(np.float32))
    assert np.array_equal(oracle.rmsnorm(x, gamma, 0.0), oracle.rmsnorm(x4, gamma, 0.0))


def test_rmsnorm_matches_torch():
    """Against torch's own RMS normalization of the same bf16 values: the
    two bf16 roundings (of x * inv, then of the product with gamma) leave
    every element within 2^-7 (two half-ulps of bf16 at the bottom of a
    binade) of it, relatively, and the mean error well below that."""
    rng = np.random.default_rng(61)
    M, K, eps = 9, 512, 1e-5
    x = rand_bf16(rng, (M, K), 1.0)
    x[2] = bf16_bits((t_bf16(x[2]).numpy() * 1e-3).astype(np.float32))
    gamma = rand_bf16(rng, (K,), 0.5)
    xn = t_bf16(oracle.rmsnorm(x, gamma, eps)).numpy()
    ref = torch.nn.functional.rms_norm(t_bf16(x), (K,), t_bf16(gamma), eps).numpy()
    assert np.all(np.abs(xn - ref) <= 2.0 ** -7 * (1 + 2.0 ** -6) * np.abs(ref) + 1e-30)
    assert np.abs(xn - ref).sum() <= 2.0 ** -8 * np.abs(ref).sum()


def test_norm_quant_shrink_brute_force():
    """M=2, K=8, r=2: Python loops from the definition (math.fsum for the
    squares, numpy float32 scalars for the fp32 steps)."""
    import math
    rng = np.random.default_rng(62)
    M, K, L, r = 2, 8, 2, 2
    x = rand_bf16(rng, (M, K), 1.0)
    gamma = rand_bf16(rng, (K,), 1.0)
    A = rand_bf16(rng, (L, r, K), 0.3)
    idx = np.array([1, 0])
    out = oracle.norm_quant_shrink(x, gamma, 1e-6, A, idx)
    xf, gf, Af = t_bf16(x).numpy(), t_bf16(gamma).numpy(), t_bf16(A).numpy()
    for t in range(M):
        ms = np.float32(math.fsum(float(v) ** 2 for v in xf[t]) / K)
        inv = np.float32(np.float32(1.0) / np.float32(np.sqrt(np.float32(ms + np.float32(1e-6)))))
        row = []
        for k in range(K):
            h = t_bf16(bf16_bits(np.array([np.float32(xf[t, k]) * inv], np.float32))).numpy()[0]
            v = t_bf16(bf16_bits(np.array([np.float32(h) * np.float32(gf[k])], np.float32))).numpy()[0]
            row.append(v)
        row = np.array(row)
        assert np.array_equal(t_bf16(out["xn"][t]).numpy(), row)
        for j in range(r):
            zt = math.fsum(Af[idx[t], j, k] * row[k] for k in range(K))
            assert abs(out["z"][t, j] - zt) <= 1e-12 * max(1.0, abs(zt))
    xq, sx = oracle.quant_act(out["xn"])
    assert np.array_equal(xq, out["xq"]) and np.array_equal(sx, out["sx"])


# --- the matched W8A16 GEMM -------------------------------------------------------------

def test_w8a16_equals_w8a8_on_representable_rows():
    """Rows built as e4m3 codes times 2^k (exact in bf16, one element at
    +-448 2^k) quantize to themselves, so the W8A8 layer (independently
    pinned) and the W8A16 layer must agree on them."""
    rng = np.random.default_rng(70)
    M, K, N = 5, 96, 40
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = rng.choice(finite, size=(M, K))
    codes[:, 7] = 0x7E
    x = bf16_bits((t_e4m3(codes).numpy() * 2.0 ** rng.integers(-6, 4, size=(M, 1))).astype(np.float32))
    w = rand_bf16(rng, (N, K), 0.02)
    wq, sw = oracle.quant_weight_fp8(w)
    _, _, A, B = make(rng, M=M, K=K, N=N, L=2, r=4)
    idx = np.array([0, 1, -1, 1, 0])
    a = oracle.linear_lora(x, A, B, idx, 2.0, wq=wq, sw=sw, a16=True)
    b = oracle.linear_lora(x, A, B, idx, 2.0, wq=wq, sw=sw)
    assert np.allclose(a["base"], b["base"], rtol=1e-13, atol=1e-16)
    assert np.allclose(a["y"], b["y"], rtol=1e-13, atol=1e-16)
    assert a["xq"] is None and np.array_equal(b["xq"], codes)


def test_w8a16_matches_torch_matmul():
    """Against torch: its own float8_e4m3fn decode of the weights times the
    per-channel scale, the bf16 activations, an fp64 matmul."""
    rng = np.random.default_rng(71)
    x, w, A, B = make(rng, M=9, K=128, N=36)
    wq, sw = oracle.quant_weight_fp8(w)
    out = oracle.linear_lora(x, A, B, np.full(9, -1), 2.0, wq=wq, sw=sw, a16=True)
    ref = (t_bf16(x) @ (t_e4m3(wq) * torch.from_numpy(sw.astype(np.float64))[:, None]).T).numpy()
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # closer to the unquantized product than the W8A8 layer (no activation rounding)
    exact = (t_bf16(x) @ t_bf16(w).T).numpy()
    w8a8 = oracle.linear_lora(x, A, B, np.full(9, -1), 2.0, wq=wq, sw=sw)["y"]
    assert np.abs(out["y"] - exact).mean() < np.abs(w8a8 - exact).mean()
