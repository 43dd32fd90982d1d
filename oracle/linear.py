"""The multi-tenant LoRA linear layer on an FP8 or 4-bit base, step by step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

For each token t with tenant index a_t the layer computes

    y_t = dequant(W_q . quant(x_t)) + s * B[a_t] (A[a_t] x_t)

("EpiLoRA: Fusing Many LoRA Adapters into Low-Precision GEMMs for Serving
and RL", Background: an adapter adds the low-rank update BA to the frozen
weight, A projecting the input down to rank r and B back up; Design,
"Multi-adapter kernels": the activations are quantized per token, the
down-projection h = x A^T is taken from the bf16 activations, and the GEMM's
epilogue applies the scales and adds h B^T for each adapter group).  a_t = -1
means no adapter.  With a prefill mask the adapter applies only to flagged
tokens ("PreFT: Prefill-only finetuning for efficient inference", abstract:
the adapter is applied to prefill tokens only).

Array conventions (all numpy):
  x        uint16 [M][K]      bf16 bit patterns of the activations
  xq, sx   uint8 [M][K], float32 [M]
  w        uint16 [N][K]      bf16 weights before quantisation
  wq, sw   uint8 [N][K], float32 [N]                    (FP8 base)
  wc, bs, gs  uint8 [N][K/2], uint8 [N][K/16], float32  (4-bit base)
  A        uint16 [L][r][K]   bf16
  B        uint16 [L][N][r]   bf16
  ranks    int32 [L] or None
  idx      int32 [M]          tenant per token, -1 = none
  mask     uint8 [M] or None  nonzero = the adapter applies
Results are float64 unless stated.
"""

import numpy as np

from .formats import (
    FOLD_SHIFT,
    bf16_to_f32,
    f32_to_bf16,
    e2m1_decode_table,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    fold_table,
)

E4M3_MAX = np.float32(448.0)

# ---------------------------------------------------------------------------
# Quantisation (integer results decided in fp32)
# ---------------------------------------------------------------------------


def quant_rows_e4m3(v):
    """Per-row dynamic E4M3 quantisation of a float32 matrix.

    amax = max |v| over the row; scale = fp32(amax / 448) (an IEEE, correctly
    rounded division), 1.0 for an all-zero row; code = E4M3(fp32(v / scale)),
    one correctly rounded division per element, the result rounded to
    nearest-even and saturated at 448 (v / scale may exceed 448 by an ulp
    when the scale was rounded down)."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v), axis=1).astype(np.float32)
    scale = (amax / E4M3_MAX).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    q = (v / scale[:, None]).astype(np.float32)
    return e4m3_encode(q), scale


def quant_act(x):
    """Per-token dynamic FP8 quantisation of the activations (Design,
    "Multi-adapter kernels": K1 quantizes the layer's activations once, with
    a per-token scale).  x: uint16 [M][K] bf16 -> (xq uint8 [M][K],
    sx float32 [M])."""
    return quant_rows_e4m3(bf16_to_f32(x))


def quant_weight_fp8(w):
    """Per-output-channel FP8 weight quantisation done when the model loads
    (Evaluation, Setup: FP8 bases quantized at load).  Same rule as the
    activations, one scale per row n of W[N][K]."""
    return quant_rows_e4m3(bf16_to_f32(w))


def quant_weight_fp4(w, rows=None):
    """4-bit weight encoder in the NVFP4 layout: E2M1 codes, one E4M3 scale
    per 16 consecutive elements along K, one fp32 global scale.

    gs = fp32(amax(W) / 2688) (1.0 if W is all zero);
    bs = E4M3(fp32(amax_block / fp32(6 * gs)));
    codes = E2M1(fp32(w / fp32(e4m3(bs) * gs))), or code 0 where that block
    scale is zero.  Element 2i goes in the low nibble of byte i.
    Returns (wc uint8 [N][K/2], bs uint8 [N][K/16], gs float32).  With
    `rows`, gs still comes from the whole matrix but only those rows are
    encoded (each row's codes depend on its own values and gs only)."""
    wf = bf16_to_f32(w)
    if wf.shape[1] % 16:
        raise ValueError("K must be a multiple of 16")
    amax = np.float32(np.max(np.abs(wf)))
    if rows is not None:
        wf = wf[np.asarray(rows)]
    n, k = wf.shape
    gs = np.float32(amax / np.float32(6.0 * 448.0)) if amax > 0 else np.float32(1.0)
    blocks = wf.reshape(n, k // 16, 16)
    amax_b = np.max(np.abs(blocks), axis=2).astype(np.float32)
    denom = np.float32(np.float32(6.0) * gs)
    bs = e4m3_encode((amax_b / denom).astype(np.float32))
    step = (e4m3_decode(bs).astype(np.float32) * gs).astype(np.float32)
    safe = np.where(step == 0, np.float32(1.0), step).astype(np.float32)
    codes = e2m1_encode((blocks / safe[:, :, None]).astype(np.float32))
    codes = np.where((step == 0)[:, :, None], np.uint8(0), codes).astype(np.uint8)
    codes = codes.reshape(n, k)
    wc = (codes[:, 0::2] | (codes[:, 1::2] << np.uint8(4))).astype(np.uint8)
    return wc, bs, gs


def unpack_fp4(wc):
    """uint8 [N][K/2] -> uint8 [N][K] E2M1 codes (low nibble first)."""
    wc = np.asarray(wc, dtype=np.uint8)
    n, kh = wc.shape
    out = np.empty((n, 2 * kh), dtype=np.uint8)
    out[:, 0::2] = wc & 0xF
    out[:, 1::2] = wc >> 4
    return out


def fold_decode_fp4(wc, bs):
    """The FP8 byte each 4-bit weight becomes inside the GEMM:
    T[code][block scale] (the fold table).  uint8 [N][K]."""
    codes = unpack_fp4(wc)
    n, k = codes.shape
    b = np.repeat(np.asarray(bs, dtype=np.uint8), 16, axis=1)
    return fold_table()[codes, b]


def exact_decode_fp4(wc, bs, gs):
    """The NVFP4 value e2m1(code) * e4m3(bs) * gs, float64 [N][K]
    (a diagnostic; the GEMM uses the fold)."""
    codes = unpack_fp4(wc)
    b = np.repeat(np.asarray(bs, dtype=np.uint8), 16, axis=1)
    return e2m1_decode_table()[codes] * e4m3_decode(b) * float(gs)


# ---------------------------------------------------------------------------
# Base GEMM (sums in fp64)
# ---------------------------------------------------------------------------


def _pick(a, sel):
    return a if sel is None else a[np.asarray(sel)]


def base_fp8(xq, sx, wq, sw, rows=None, cols=None):
    """acc[t][n] = sum_k e4m3(xq[t][k]) * e4m3(wq[n][k]);
    base = (acc * sx[t]) * sw[n].  rows/cols select a subset of tokens and
    output channels (sampled checks at full size)."""
    X = e4m3_decode(_pick(xq, rows))
    W = e4m3_decode(_pick(wq, cols))
    acc = X @ W.T
    s_t = _pick(np.asarray(sx, np.float32), rows).astype(np.float64)
    s_n = _pick(np.asarray(sw, np.float32), cols).astype(np.float64)
    return (acc * s_t[:, None]) * s_n[None, :]


def base_w8a16(x, wq, sw, rows=None, cols=None):
    """The matched engine's GEMM ("EpiLoRA ...", Design, "LoRA RL on the same
    base": a W8A16 GEMM on the FP8 weights whose activations stay in bf16,
    so the engine rounds nothing the trainer does not): each FP8 weight is
    widened exactly, acc[t][n] = sum_k bf16(x[t][k]) * e4m3(wq[n][k]), and
    base = acc * sw[n]; no activation quantization, no activation scale."""
    X = bf16_to_f32(_pick(x, rows)).astype(np.float64)
    W = e4m3_decode(_pick(wq, cols))
    acc = X @ W.T
    s_n = _pick(np.asarray(sw, np.float32), cols).astype(np.float64)
    return acc * s_n[None, :]


def base_fp4(xq, sx, wc, bs, gs, rows=None, cols=None):
    """4-bit base through the fold: each weight is the FP8 byte
    T[code][block scale]; base = (acc * sx[t]) * (gs * 2**3)."""
    X = e4m3_decode(_pick(xq, rows))
    W8 = e4m3_decode(fold_decode_fp4(_pick(wc, cols), _pick(bs, cols)))
    acc = X @ W8.T
    s_t = _pick(np.asarray(sx, np.float32), rows).astype(np.float64)
    return (acc * s_t[:, None]) * (float(np.float32(gs)) * 2.0 ** FOLD_SHIFT)


# ---------------------------------------------------------------------------
# Adapters
# ---------------------------------------------------------------------------


def active_rows(idx, L, r, ranks=None, mask=None):
    """(active bool [M], adapter int [M], rank int [M]).

    A token is adapted when its index lies in [0, L), its mask byte (if a
    mask is given) is nonzero, and its adapter's rank (ranks[a], or r when
    no ranks are given) is positive.  An index outside [-1, L) counts as -1."""
    idx = np.asarray(idx, dtype=np.int64)
    valid = (idx >= 0) & (idx < L)
    a = np.where(valid, idx, 0)
    if ranks is None:
        rk = np.full(idx.shape, r, dtype=np.int64)
    else:
        rk = np.minimum(np.asarray(ranks, dtype=np.int64)[a], r)
    act = valid & (rk > 0)
    if mask is not None:
        act &= np.asarray(mask, dtype=np.uint8) != 0
    return act, a, np.where(act, rk, 0)


def quant_adapter_fp8(m):
    """Adapters stored in FP8 ("EpiLoRA ...", Design, "Multi-adapter
    kernels": adapters may be stored in FP8 and dequantized in registers,
    halving the adapter bytes): E4M3 codes with one fp32 scale per row of
    the matrix's last axis, by the same per-row rule as the weights
    (scale = amax / 448, code = E4M3(v / scale)).  A [L][(S)][r][K] gets one
    scale per rank row, B [L][N][r] one per output row.  m: bf16 bits ->
    (codes uint8 of m's shape, scales float32 of m's shape minus the last
    axis)."""
    m = np.asarray(m)
    codes, sc = quant_rows_e4m3(bf16_to_f32(m.reshape(-1, m.shape[-1])))
    return codes.reshape(m.shape), sc.reshape(m.shape[:-1])


def adapter_values(codes, row_scale=None):
    """An adapter matrix's values in fp64: bf16 bit patterns (row_scale
    None), or FP8 E4M3 codes times their row's fp32 scale (the last axis is
    the row)."""
    if row_scale is None:
        return bf16_to_f32(codes).astype(np.float64)
    return e4m3_decode(codes) * np.asarray(row_scale, np.float32).astype(np.float64)[..., None]


def shrink(x, A, idx, ranks=None, mask=None, a_scale=None):
    """z[t][j] = sum_k A[a_t][j][k] * x[t][k] over the bf16 values, for
    active tokens and j < rank(a_t); zero elsewhere.  float64 [M][r].
    With a_scale ([L][r]), A holds FP8 codes and row j of adapter a is
    e4m3(A[a][j]) * a_scale[a][j]."""
    L, r, _ = A.shape
    act, a, rk = active_rows(idx, L, r, ranks, mask)
    xf = bf16_to_f32(x).astype(np.float64)
    z = np.zeros((xf.shape[0], r), dtype=np.float64)
    for t in np.nonzero(act)[0]:
        sc = None if a_scale is None else a_scale[a[t], : rk[t]]
        Af = adapter_values(A[a[t], : rk[t]], sc)
        z[t, : rk[t]] = Af @ xf[t]
    return z


def expand(z, B, idx, scale, ranks=None, mask=None, cols=None, b_scale=None):
    """lora[t][n] = s * sum_j B[a_t][n][j] * z[t][j] for active tokens,
    zero for the others (which receive no add at all).  float64 [M][N].
    With b_scale ([L][N]), B holds FP8 codes and row n of adapter a is
    e4m3(B[a][n]) * b_scale[a][n]."""
    L, _, r = B.shape
    act, a, rk = active_rows(idx, L, r, ranks, mask)
    Bsel = B if cols is None else B[:, np.asarray(cols)]
    bsel = None if b_scale is None else (b_scale if cols is None else b_scale[:, np.asarray(cols)])
    out = np.zeros((z.shape[0], Bsel.shape[1]), dtype=np.float64)
    for t in np.nonzero(act)[0]:
        Bf = adapter_values(Bsel[a[t], :, : rk[t]], None if bsel is None else bsel[a[t]])
        out[t] = float(np.float32(scale)) * (Bf @ z[t, : rk[t]])
    return out, act


def linear_lora(x, A, B, idx, scale, *, wq=None, sw=None, wc=None, bs=None,
                gs=None, ranks=None, mask=None, rows=None, cols=None, sa=None, sb=None, a16=False):
    """The whole layer: per-token quantisation, base GEMM, shrink and the
    epilogue.  Exactly one weight format is given (wq+sw, or wc+bs+gs).

    Returns a dict with xq, sx (bit-exact targets), z (float64), base,
    y (float64: base plus the adapter term on active rows, base alone on
    the others) and the active-row flags.  `rows` restricts every result
    to a sample of tokens; to sample output channels either pass `cols`, or
    pass the weights and B of the sampled channels only.  With sa and sb
    the adapters are stored in FP8: A and B hold E4M3 codes, sa [L][r] and
    sb [L][N] their row scales (quant_adapter_fp8).  With a16 the base is
    the W8A16 GEMM on the bf16 activations (base_w8a16; FP8 weights only)
    and xq, sx are None."""
    xs = _pick(x, rows)
    if a16:
        xq = sx = None
        base = base_w8a16(xs, wq, sw, cols=cols)
    else:
        xq, sx = quant_act(xs)  # per-token quantisation is row-local
        if wq is not None:
            base = base_fp8(xq, sx, wq, sw, cols=cols)
        else:
            base = base_fp4(xq, sx, wc, bs, gs, cols=cols)
    idx_s = _pick(np.asarray(idx), rows)
    mask_s = None if mask is None else _pick(np.asarray(mask), rows)
    z = shrink(xs, A, idx_s, ranks, mask_s, a_scale=sa)
    lora, act = expand(z, B, idx_s, scale, ranks, mask_s, cols=cols, b_scale=sb)
    y = base.copy()
    y[act] = base[act] + lora[act]
    return dict(xq=xq, sx=sx, z=z, base=base, y=y, active=act)


# ---------------------------------------------------------------------------
# Multi-slice projections
# ---------------------------------------------------------------------------


def slice_bounds(slice_n):
    """[(start, stop)] of consecutive output slices of widths slice_n."""
    ends = np.cumsum(np.asarray(slice_n, dtype=np.int64))
    starts = np.concatenate([[0], ends[:-1]])
    return list(zip(starts.tolist(), ends.tolist()))


def linear_lora_sliced(x, A, B, idx, scale, slice_n, *, wq=None, sw=None, wc=None, bs=None, gs=None,
                       ranks=None, mask=None, rows=None, cols=None, weights_of_cols=False, sa=None, sb=None,
                       a16=False):
    """A projection whose outputs are several consecutive slices, each with
    its own adapter pair: attention's query / key / value (three slices of
    unequal widths) or the MLP's gate / up (two), as in "EpiLoRA ...",
    Evaluation, "Many tenants" and the appendix's account of the expand
    costs (Table 15): the up-projection of slice s adds into the slice's
    output columns only, and its down-projection is the slice's own.

    A: uint16 [L][S][r][K] (slice s of adapter a: A[a][s]);
    B: uint16 [L][N][r] (rows of slice s hold that slice's up-projection);
    slice_n: the S slice widths (sum N).  For output column n in slice s and
    an active token t: y[t][n] = base[t][n] + scale * sum_j
    B[a_t][n][j] * z_s[t][j], with z_s = shrink(x, A[:, s]).  Other rows get
    no add.  The result's z is [M][S * r], slice s in columns s*r .. s*r+r.
    `cols` samples output columns (indices into N); with weights_of_cols the
    weights passed are already those columns' rows, in that order.  With sa
    ([L][S][r]) and sb ([L][N]) the adapters are stored in FP8, and with a16
    the base is the W8A16 GEMM, as in linear_lora."""
    L, S, r, K = A.shape
    bounds = slice_bounds(slice_n)
    if len(bounds) != S or bounds[-1][1] != B.shape[1]:
        raise ValueError("slice widths must match A's slices and B's rows")
    xs = _pick(x, rows)
    wcols = None if weights_of_cols else cols
    if a16:
        xq = sx = None
        base = base_w8a16(xs, wq, sw, cols=wcols)
    else:
        xq, sx = quant_act(xs)
        if wq is not None:
            base = base_fp8(xq, sx, wq, sw, cols=wcols)
        else:
            base = base_fp4(xq, sx, wc, bs, gs, cols=wcols)
    idx_s = _pick(np.asarray(idx), rows)
    mask_s = None if mask is None else _pick(np.asarray(mask), rows)
    colset = np.arange(B.shape[1]) if cols is None else np.asarray(cols)
    y = base.copy()
    z_all = np.zeros((xs.shape[0], S * r), dtype=np.float64)
    act = None
    for s, (n0, n1) in enumerate(bounds):
        z = shrink(xs, A[:, s], idx_s, ranks, mask_s, a_scale=None if sa is None else sa[:, s])
        z_all[:, s * r:(s + 1) * r] = z
        pos = np.nonzero((colset >= n0) & (colset < n1))[0]   # positions in the output
        if pos.size == 0:
            continue
        lora, act = expand(z, B, idx_s, scale, ranks, mask_s, cols=colset[pos], b_scale=sb)
        y[np.ix_(act, pos)] = base[np.ix_(act, pos)] + lora[act]
    if act is None:
        act = active_rows(idx_s, L, r, ranks, mask_s)[0]
    return dict(xq=xq, sx=sx, z=z_all, base=base, y=y, active=act)


# ---------------------------------------------------------------------------
# The normalization in front of qkv and gate_up, with the quantizer and the
# shrink fused into it
# ---------------------------------------------------------------------------


def rmsnorm(x, gamma, eps):
    """RMS normalization of each token row, as the normalization kernel in
    front of the query / key / value and gate / up projections computes it
    ("EpiLoRA ...", appendix "Discussion and Limitations": the down-projection
    can be computed inside the normalization kernel that already reads the
    input).  The pages do not spell the normalization out; this is the
    common decoder form: ms = mean_k x_k^2 (the sum of the exact squares in
    fp64, the mean rounded to fp32), inv = fp32(1 / fp32(sqrt(fp32(ms + eps))))
    with correctly rounded fp32 operations, then h_k = bf16(fp32(x_k * inv))
    and xn_k = bf16(fp32(h_k * gamma_k)).  x, gamma: bf16 bits ([M][K],
    [K]) -> xn bf16 bits [M][K]."""
    xf = bf16_to_f32(x)
    ss = np.sum(xf.astype(np.float64) ** 2, axis=1)
    ms = (ss / xf.shape[1]).astype(np.float32)
    v = (ms + np.float32(eps)).astype(np.float32)
    inv = (np.float32(1.0) / np.sqrt(v).astype(np.float32)).astype(np.float32)
    h = f32_to_bf16((xf * inv[:, None]).astype(np.float32))
    return f32_to_bf16((bf16_to_f32(h) * bf16_to_f32(gamma)[None, :]).astype(np.float32))


def norm_quant_shrink(x, gamma, eps, A=None, idx=None, *, ranks=None, mask=None, sa=None):
    """The normalization with the per-token FP8 quantizer and the shrink
    taken from its output: xn = rmsnorm(x); (xq, sx) = quant_act(xn);
    z = shrink(xn, A) (A [L][r][K], or [L][S][r][K] per slice, giving z
    [M][S r]; FP8-stored when sa is given).  Returns dict(xn, xq, sx, z)."""
    xn = rmsnorm(x, gamma, eps)
    xq, sx = quant_act(xn)
    out = dict(xn=xn, xq=xq, sx=sx, z=None)
    if A is not None:
        if A.ndim == 3:
            out["z"] = shrink(xn, A, idx, ranks, mask, a_scale=sa)
        else:
            out["z"] = np.concatenate([shrink(xn, A[:, s], idx, ranks, mask,
                                              a_scale=None if sa is None else sa[:, s])
                                       for s in range(A.shape[1])], axis=1)
    return out
