"""GPU parity of every entry point against the CPU oracle at small sizes that
still span several tiles, ragged M / N / K tails and the degenerate cases
(no adapter, rank 0, masked tokens, out-of-range indices, all-zero rows)."""

import numpy as np
import pytest
import torch

import fp4_gemm_amd as ep
import oracle
from workloads import bf16_bits, custom_layer

from gpu_harness import DEV, DeviceGemm, bf16_np_to_f64, compare, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


def say(*a):
    print(*a, flush=True)


# --- quantization -------------------------------------------------------------------

def _special_rows(K, rng):
    rows = []
    rows.append(np.zeros(K, np.float32))                                  # all zero -> sx = 1
    mids = (oracle.e4m3_decode(np.arange(0x7E)) + oracle.e4m3_decode(np.arange(1, 0x7F))) / 2
    up = bf16_bits(mids.astype(np.float32))
    near = np.concatenate([mids, (up.astype(np.uint32) << 16).view(np.float32),
                           ((up + 1).astype(np.uint32) << 16).view(np.float32),
                           ((up - 1).astype(np.uint32) << 16).view(np.float32)]).astype(np.float32)
    r = np.resize(near * rng.choice([-1.0, 1.0], size=near.size), K).astype(np.float32)
    r[0] = 448.0                                                           # sx = 1 exactly: ties land on midpoints
    rows.append(r)
    rows.append((rng.standard_normal(K) * 1e-36).astype(np.float32))     # tiny values
    rows.append((rng.standard_normal(K) * 3e37).astype(np.float32))      # huge values
    rows.append(np.resize(np.array([1.0, -0.0, 0.0, 2.0 ** -20], np.float32), K))
    # every bf16 value in [-448, 448] (as many as fit), at sx = 1: each one
    # goes through the E4M3 conversion unchanged
    allb = np.arange(0x10000, dtype=np.uint32)
    vals = (allb << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448)]
    r = np.resize(rng.permutation(vals), K).astype(np.float32)
    r[0] = 448.0
    rows.append(r)
    # scales either side of 2^-64 (the reciprocal-quotient threshold), and a
    # scale that is no power of two with values spread over many binades
    for amax in (448.0 * 2.0 ** -64 * 1.0078125, 448.0 * 2.0 ** -64 * 0.9921875):
        r = (rng.standard_normal(K) * amax / 4).astype(np.float32)
        r[0] = amax
        rows.append(r)
    r = (rng.choice([-1.0, 1.0], K) * 2.0 ** rng.uniform(-40, 6.8, K)).astype(np.float32)
    r[0] = 113.37
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("M,K", [(1, 16), (5, 256), (37, 4096), (3, 14336), (2, 40960)])
def test_quant_act_bit_exact(M, K):
    say(f"quant_act M={M} K={K}")
    rng = np.random.default_rng(1000 + K)
    x = bf16_bits(rng.standard_normal((M, K)).astype(np.float32) * np.float32(rng.uniform(0.01, 100)))
    x = np.concatenate([x, bf16_bits(_special_rows(K, rng))])
    xq_ref, sx_ref = oracle.quant_act(x)
    xd = to_dev(x)
    xq = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    sx = torch.empty(x.shape[0], dtype=torch.float32, device=DEV)
    ep.epilora_quant_act(xd, xq, sx)
    assert np.array_equal(to_np(sx).view(np.uint32), sx_ref.view(np.uint32))
    got = to_np(xq)
    bad = np.argwhere(got != xq_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"


def test_quant_act_strided_rows():
    rng = np.random.default_rng(5)
    x = bf16_bits(rng.standard_normal((6, 512)).astype(np.float32))
    xq_ref, sx_ref = oracle.quant_act(x[:, :256])
    xd = to_dev(x)[:, :256]
    out = torch.full((6, 384), 0xAB, dtype=torch.uint8, device=DEV)
    sx = torch.empty(6, dtype=torch.float32, device=DEV)
    ep.epilora_quant_act(xd, out[:, :256], sx)
    got = to_np(out)
    assert np.array_equal(got[:, :256], xq_ref) and np.all(got[:, 256:] == 0xAB)
    assert np.array_equal(to_np(sx), sx_ref)


@pytest.mark.parametrize("N,K", [(3, 32), (300, 512), (64, 4096)])
def test_weight_quantizers_bit_exact(N, K):
    say(f"weight quant N={N} K={K}")
    rng = np.random.default_rng(2000 + N)
    w = bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    w[0, :16] = 0                     # a zero block
    w[-1] = 0                         # a zero row
    wd = to_dev(w)
    wq = torch.empty(N, K, dtype=torch.uint8, device=DEV)
    sw = torch.empty(N, dtype=torch.float32, device=DEV)
    ep.epilora_quant_weight_fp8(wd, wq, sw)
    wq_ref, sw_ref = oracle.quant_weight_fp8(w)
    assert np.array_equal(to_np(wq), wq_ref) and np.array_equal(to_np(sw), sw_ref)
    wc = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    bs = torch.empty(N, K // 16, dtype=torch.uint8, device=DEV)
    gs = torch.empty(1, dtype=torch.float32, device=DEV)
    ws = ep.new_workspace(ep.OP_QUANT_W4, 1, N, K, 16)
    ep.epilora_quant_weight_fp4(wd, wc, bs, gs, ws)
    wc_ref, bs_ref, gs_ref = oracle.quant_weight_fp4(w)
    assert to_np(gs)[0] == gs_ref
    assert np.array_equal(to_np(bs), bs_ref)
    assert np.array_equal(to_np(wc), wc_ref)


# --- shrink -----------------------------------------------------------------------------

SHRINK_CASES = [
    # M, K, L, r, idx kind, mask, ranks
    (1, 4096, 1, 64, "zero", False, False),
    (7, 256, 4, 16, "mixed", True, False),
    (33, 4224, 6, 32, "mixed", False, True),
    (100, 512, 3, 128, "sorted", True, True),
    (16, 14336, 64, 64, "distinct", False, False),
    (9, 8192, 12, 128, "distinct", False, True),  # two rank rows per unit
    (3, 29568, 5, 32, "mixed", True, True),       # one row per unit, two rounds of loads
    # prefill batches: 64-token tiles, ragged token and K tails, many splits
    (65, 256, 2, 16, "mixed", False, False),
    (300, 4112, 8, 128, "mixed", True, True),
    (517, 14336, 16, 16, "mixed", True, False),
    (2048, 4096, 32, 64, "sorted", False, True),
]


def _idx(kind, M, L, rng):
    if kind == "zero":
        return np.zeros(M, np.int32)
    if kind == "sorted":
        return np.sort(rng.integers(-1, L, M)).astype(np.int32)
    if kind == "distinct":
        return rng.permutation(L)[:M].astype(np.int32)
    return rng.integers(-1, L, M).astype(np.int32)


@pytest.mark.parametrize("M,K,L,r,kind,use_mask,use_ranks", SHRINK_CASES)
def test_shrink_vs_oracle(M, K, L, r, kind, use_mask, use_ranks):
    say(f"shrink M={M} K={K} L={L} r={r} {kind}")
    rng = np.random.default_rng(3000 + M + K)
    idx = _idx(kind, M, L, rng)
    mask = rng.integers(0, 2, M).astype(np.uint8) if use_mask else None
    ranks = rng.choice([0, 8, r // 2, r, 21 if r > 21 else r], size=L).astype(np.int32) if use_ranks else None
    lay = custom_layer("s", 300 + M, M, K, 64, L, r, idx, mask=mask, ranks=ranks)
    d = DeviceGemm(lay.gemms[0])
    z, ws = d.shrink()
    z_ref = oracle.shrink(d.x_np, d.A_np, idx, ranks, mask)
    zg = to_np(z).astype(np.float64)
    scale = max(np.sqrt(np.mean(z_ref ** 2)), 1e-30)
    assert np.abs(zg - z_ref).max() <= 1e-4 * scale
    act, _, _ = oracle.active_rows(idx, L, r, ranks, mask)
    assert not zg[~act].any()
    # deterministic: the same call again gives the same bits
    z2, _ = d.shrink(ws)
    assert torch.equal(z, z2)


# --- the GEMM with its epilogue -----------------------------------------------------------

GEMM_CASES = [
    # M, K, N, L, r, kind, mask, ranks, wfmt
    (1, 256, 512, 1, 16, "zero", False, False, "fp8"),
    (5, 160, 200, 4, 16, "mixed", True, False, "fp8"),
    (16, 4096, 1024, 8, 64, "mixed", False, False, "fp8"),
    (17, 512, 300, 4, 32, "mixed", True, True, "fp8"),
    (33, 384, 128, 40, 64, "distinct", False, False, "fp8"),
    (64, 1024, 272, 5, 128, "mixed", True, True, "fp8"),
    (65, 256, 512, 4, 16, "sorted", False, False, "fp8"),
    (130, 4096, 384, 6, 64, "sorted", True, True, "fp8"),
    (257, 288, 200, 9, 32, "mixed", False, False, "fp8"),
    (1, 256, 512, 1, 16, "zero", False, False, "fp4"),
    (20, 4096, 512, 4, 64, "mixed", True, False, "fp4"),
    (150, 1024, 300, 6, 32, "sorted", False, True, "fp4"),
    # enough tiles for the 256 x 128 prefill tiles, ragged edges
    (1100, 256, 13100, 6, 64, "sorted", True, True, "fp8"),
    (700, 384, 12000, 5, 32, "mixed", False, False, "fp4"),
    (1030, 160, 13100, 4, 16, "mixed", True, False, "fp4"),
    # enough 256 x 256 tiles for that kernel, base-only and with its adapter
    # epilogue (bf16 adapters, one slice): ragged edges, masks, own ranks
    (2048, 256, 16384, 8, 64, "sorted", False, False, "fp8"),
    (2100, 160, 16000, 4, 32, "mixed", True, False, "fp4"),
    (2050, 192, 16400, 7, 128, "mixed", True, True, "fp8"),
]


@pytest.mark.parametrize("M,K,N,L,r,kind,use_mask,use_ranks,wfmt", GEMM_CASES)
def test_gemm_lora_vs_oracle(M, K, N, L, r, kind, use_mask, use_ranks, wfmt):
    say(f"gemm_lora M={M} K={K} N={N} L={L} r={r} {kind} {wfmt}")
    rng = np.random.default_rng(4000 + M + K + N)
    idx = _idx(kind, M, L, rng)
    mask = rng.integers(0, 2, M).astype(np.uint8) if use_mask else None
    ranks = rng.choice([0, 16, r // 2, r], size=L).astype(np.int32) if use_ranks else None
    lay = custom_layer("g", 500 + M + N, M, K, N, L, r, idx, mask=mask, ranks=ranks, wfmt=wfmt)
    d = DeviceGemm(lay.gemms[0], wfmt)
    out = d.separate()
    ref = d.oracle()
    assert np.array_equal(to_np(out["xq"]), ref["xq"])
    assert np.array_equal(to_np(out["sx"]), ref["sx"])
    if wfmt == "fp8":
        assert np.array_equal(to_np(d.wq), ref["w"]["wq"])
    else:
        assert np.array_equal(to_np(d.wq), ref["w"]["wc"]) and np.array_equal(to_np(d.bs), ref["w"]["bs"])
    compare(to_np(out["y"]), ref["y"], f"M={M} N={N} {wfmt}")
    # rows without an adapter equal the base-only GEMM bit for bit
    base = d.gemm(out["xq"], out["sx"])
    inactive = ~ref["active"]
    yb, yl = to_np(base), to_np(out["y"])
    assert np.array_equal(yl[inactive], yb[inactive])
    compare(yb, ref["base"], "base only")
    # and the call is deterministic
    again = d.gemm(out["xq"], out["sx"], out["z"], out["ws"])
    assert torch.equal(again, out["y"])
    assert ep.epilora_device_error(out["ws"]) == 0


def test_bad_index_sets_device_error():
    lay = custom_layer("bad", 900, 6, 256, 256, 4, 16, [0, 7, -1, -3, 3, 1])
    d = DeviceGemm(lay.gemms[0])
    out = d.separate()
    assert ep.epilora_device_error(out["ws"]) & ep.DEV_BAD_INDEX
    ref = d.oracle()
    compare(to_np(out["y"]), ref["y"], "bad index")
    base = to_np(d.gemm(out["xq"], out["sx"]))
    assert np.array_equal(to_np(out["y"])[[1, 2, 3]], base[[1, 2, 3]])
    assert ep.epilora_device_error(out["ws"]) == 0  # cleared by the previous read


def test_expand_add_baseline():
    """The unfused baseline: base GEMM, then the separate expand-add."""
    rng = np.random.default_rng(7)
    idx = rng.integers(-1, 5, 40).astype(np.int32)
    lay = custom_layer("e", 901, 40, 512, 384, 5, 32, idx)
    d = DeviceGemm(lay.gemms[0])
    xq, sx = d.quant()
    z, ws = d.shrink()
    y = d.gemm(xq, sx)
    ep.epilora_lora_expand_add(z, d.B, d.idx, d.scale, y, ws)
    ref = d.oracle()
    # This path rounds to bf16 twice: the base GEMM's output, then the sum.
    # Half a bf16 ulp is at most 2^-8 of the value, so
    # |dY| <= 2^-8 (|base| + |y|) plus the fp32 arithmetic.  Rows without an
    # adapter are rounded once.
    yg = bf16_np_to_f64(to_np(y))
    rms = np.sqrt(np.mean(ref["y"] ** 2))
    bound = 2.0 ** -8 * (np.abs(ref["base"]) + np.abs(ref["y"])) * 1.001 + 1e-4 * rms
    assert np.all(np.abs(yg - ref["y"]) <= bound)
    assert np.abs(yg - ref["y"]).sum() <= 5e-3 * np.abs(ref["y"]).sum()
    compare(to_np(y)[~ref["active"]], ref["y"][~ref["active"]], "expand baseline, inactive rows")


# --- the fused decode path ------------------------------------------------------------------

DECODE_CASES = [
    (1, 4096, 1024, 1, 64, "zero", False, False, "fp8"),
    (4, 256, 512, 4, 16, "mixed", True, True, "fp8"),
    (16, 512, 200, 8, 32, "mixed", False, False, "fp8"),
    (32, 4096, 512, 64, 64, "distinct", False, False, "fp8"),
    (64, 1024, 256, 9, 16, "mixed", True, False, "fp8"),
    (1, 4096, 512, 1, 64, "zero", False, False, "fp4"),
    (24, 512, 300, 6, 32, "mixed", True, True, "fp4"),
]


@pytest.mark.parametrize("M,K,N,L,r,kind,use_mask,use_ranks,wfmt", DECODE_CASES)
def test_decode_matches_separate_and_oracle(M, K, N, L, r, kind, use_mask, use_ranks, wfmt):
    say(f"decode M={M} K={K} N={N} L={L} r={r} {kind} {wfmt}")
    rng = np.random.default_rng(6000 + M + K + N)
    idx = _idx(kind, M, L, rng)
    mask = rng.integers(0, 2, M).astype(np.uint8) if use_mask else None
    ranks = rng.choice([0, 16, r], size=L).astype(np.int32) if use_ranks else None
    lay = custom_layer("d", 700 + M + N, M, K, N, L, r, idx, mask=mask, ranks=ranks, wfmt=wfmt)
    d = DeviceGemm(lay.gemms[0], wfmt)
    fused = d.decode()
    sep = d.separate()
    # the same kernels in one launch: bit-identical to the separate calls
    assert torch.equal(fused["xq"], sep["xq"]) and torch.equal(fused["sx"], sep["sx"])
    assert torch.equal(fused["y"], sep["y"])
    ref = d.oracle()
    compare(to_np(fused["y"]), ref["y"], "decode")
    assert ep.epilora_device_error(fused["ws"]) == 0
    # the workspace is clean again: a second call on it gives the same bits
    again = d.decode(ws=fused["ws"], keep_xq=False)
    assert torch.equal(again["y"], fused["y"])
    assert ep.epilora_device_error(fused["ws"]) == 0


def test_decode_workspace_shared_by_different_calls():
    # The fused path hands z over in the workspace: every call must see only
    # its own z.  Two layers of one shape and one of another share a
    # workspace; each call equals its own separate calls bit for bit (a z
    # left over from the previous call would change y).
    say("decode: one workspace, different inputs and shapes in turn")
    d1 = DeviceGemm(custom_layer("w1", 1201, 16, 2048, 512, 4, 64, [0, 1, 2, 3] * 4).gemms[0])
    d2 = DeviceGemm(custom_layer("w2", 1202, 16, 2048, 512, 4, 64, [3, 2, -1, 0] * 4).gemms[0])
    d3 = DeviceGemm(custom_layer("w3", 1203, 3, 256, 384, 2, 16, [1, 0, 1]).gemms[0])
    ws = ep.new_workspace(ep.OP_DECODE, 16, 512, 2048, 64)
    for d in (d1, d2, d3, d1, d2):
        fused = d.decode(ws=ws)
        sep = d.separate()
        assert torch.equal(fused["y"], sep["y"])
        assert ep.epilora_device_error(ws) == 0


def test_decode_fresh_rows_each_call():
    # More than 4 tokens: the quantized rows reach the GEMM workgroups through
    # the workspace (the same addresses every call), written by quantizing
    # workgroups of the same grid behind a flag (8, 24 tokens) or by the
    # quantizer launched just before (48, 64), and read through the caches.
    # Different activations in turn on one workspace: every call must read
    # its own rows.
    for M in (8, 24, 48, 64):
        say(f"decode M={M}: one workspace, different activations in turn")
        ds = [DeviceGemm(custom_layer(f"f{i}", 1300 + 7 * i + M, M, 4096, 1024, 8, 32,
                                      list(range(-1, 7)) * (M // 8)).gemms[0]) for i in range(2)]
        ws = ep.new_workspace(ep.OP_DECODE, M, 1024, 4096, 32)
        for d in (ds[0], ds[1], ds[0], ds[1]):
            fused = d.decode(ws=ws, keep_xq=False)
            sep = d.separate()
            assert torch.equal(fused["y"], sep["y"])
            assert ep.epilora_device_error(ws) == 0


def test_decode_base_only():
    lay = custom_layer("db", 950, 3, 512, 256, 1, 16, [-1, -1, -1])
    d = DeviceGemm(lay.gemms[0])
    y = torch.empty(3, 256, dtype=torch.bfloat16, device=DEV)
    ws = ep.new_workspace(ep.OP_DECODE, 3, 256, 512, 16)
    ep.epilora_decode_lora(d.x, d.wq, y, sw=d.sw, ws=ws)
    xq, sx = d.quant()
    assert torch.equal(y, d.gemm(xq, sx))


def test_decode_inactive_tiles_leave_no_stale_z():
    # A fused call whose batch has one whole 16-token shrink tile without an
    # active token (tokens 16-31) and one partly inactive tile (tokens 0-15),
    # then calls on the same workspace in which those tokens are active: a z
    # word left behind by the first call would be taken as the second call's
    # published z.  Each call must equal its separate calls bit for bit.
    say("decode: inactive shrink tiles, then the same tokens active")
    M, K, N, L, r = 40, 1024, 256, 5, 32
    idx_a = np.array([0, -1, 1, -1, 2, -1, 3, -1] * 2 + [-1] * 16 + [4, 0, 1, 2, 3, 4, 0, 1], np.int32)
    mask_a = np.ones(M, np.uint8)
    mask_a[8:16] = 0
    idx_b = np.array([(t % L) for t in range(M)], np.int32)
    ws = ep.new_workspace(ep.OP_DECODE, M, N, K, r)
    da = DeviceGemm(custom_layer("stale_a", 1301, M, K, N, L, r, idx_a, mask=mask_a).gemms[0])
    db = DeviceGemm(custom_layer("stale_b", 1302, M, K, N, L, r, idx_b).gemms[0])
    for d in (da, db, da, db, db):
        fused = d.decode(ws=ws)
        sep = d.separate()
        assert torch.equal(fused["y"], sep["y"])
        assert ep.epilora_device_error(ws) == 0


@pytest.mark.parametrize("M", [1, 24])
def test_decode_forced_timeout_then_recovers(M):
    # The failure path of the bounded waits, forced from the host: every wait
    # for z gives up at once (M = 1: the rows in LDS; M = 24: the rows
    # quantized by a launch of their own), every kernel still runs to its end, the call raises
    # EPILORA_DEV_WAIT_TIMEOUT, and after epilora_workspace_init the next call
    # on the workspace is bitwise correct again.
    say(f"decode: forced timeout M={M}")
    L, r = 3, 16
    idx = np.arange(M, dtype=np.int32) % L
    d = DeviceGemm(custom_layer("timeout", 1400 + M, M, 512, 384, L, r, idx).gemms[0])
    ws = ep.new_workspace(ep.OP_DECODE, M, 384, 512, r)
    ep.epilora_workspace_force_timeout(ws, True)
    d.decode(ws=ws)
    torch.cuda.synchronize()
    assert ep.epilora_device_error(ws) & ep.DEV_WAIT_TIMEOUT
    ep.epilora_workspace_init(ws)
    fused = d.decode(ws=ws)
    sep = d.separate()
    assert torch.equal(fused["y"], sep["y"])
    assert ep.epilora_device_error(ws) == 0


def test_decode_graph_replays_are_deterministic():
    # Bitwise reproducibility of the fused path over many replays of one
    # captured graph (a layer's four projections on one shared workspace),
    # with eager work and synchronizations between replays; stops at the
    # first replay that differs.
    say("decode: 200 graph replays, bitwise equal")
    from workloads import config
    lay = config(3)
    ds = [DeviceGemm(g) for g in lay.gemms]
    ws = ep.new_workspace(ep.OP_DECODE, lay.M, max(d.N for d in ds), max(d.K for d in ds), lay.r)
    ys = [torch.empty(d.M, d.N, dtype=torch.bfloat16, device=DEV) for d in ds]

    def step():
        for d, y in zip(ds, ys):
            ep.epilora_decode_lora(d.x, d.wq, y, A=d.A, B=d.B, idx=d.idx, ranks=d.ranks, mask=d.mask,
                                   scale=d.scale, ws=ws, **d.wkw)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    for d, y in zip(ds, ref):
        assert torch.equal(y, d.separate()["y"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(200):
        for y in ys:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for j, (y, y0) in enumerate(zip(ys, ref)):
            assert torch.equal(y, y0), f"replay {i}, projection {j}"
    assert ep.epilora_device_error(ws) == 0


# --- projections with per-slice adapters (qkv: 3 slices, gate_up: 2) ---------------------

SLICE_CASES = [
    # M, K, slice widths, L, r, idx kind, mask, ranks, wfmt
    (1, 4096, (4096, 1024, 1024), 1, 64, "zero", False, False, "fp8"),
    (5, 512, (256, 64, 64), 4, 16, "mixed", True, True, "fp8"),
    (24, 1024, (512, 512), 6, 32, "mixed", False, True, "fp4"),
    (64, 512, (160, 48, 48, 80), 9, 16, "mixed", True, False, "fp8"),
    (300, 512, (512, 128, 128), 6, 64, "sorted", True, True, "fp8"),
    (1100, 256, (6144, 6144), 4, 128, "sorted", False, False, "fp8"),
    (200, 1024, (384, 128, 256), 5, 32, "mixed", False, True, "fp4"),
]


@pytest.mark.parametrize("M,K,slices,L,r,kind,use_mask,use_ranks,wfmt", SLICE_CASES)
def test_sliced_vs_oracle(M, K, slices, L, r, kind, use_mask, use_ranks, wfmt):
    N = sum(slices)
    say(f"sliced M={M} K={K} slices={slices} L={L} r={r} {kind} {wfmt}")
    rng = np.random.default_rng(8000 + M + K + N)
    idx = _idx(kind, M, L, rng)
    mask = rng.integers(0, 2, M).astype(np.uint8) if use_mask else None
    ranks = rng.choice([0, 16, r // 2, r], size=L).astype(np.int32) if use_ranks else None
    lay = custom_layer("sl", 800 + M + N, M, K, N, L, r, idx, mask=mask, ranks=ranks, wfmt=wfmt, slices=slices)
    d = DeviceGemm(lay.gemms[0], wfmt)
    sep = d.separate()
    ref = d.oracle()
    assert np.array_equal(to_np(sep["xq"]), ref["xq"])
    # the shrink: every slice's z against the oracle's, zero rows elsewhere
    zg = to_np(sep["z"]).astype(np.float64)
    scale = max(np.sqrt(np.mean(ref["z"] ** 2)), 1e-30)
    assert np.abs(zg - ref["z"]).max() <= 1e-4 * scale
    assert not zg[~ref["active"]].any()
    compare(to_np(sep["y"]), ref["y"], f"sliced gemm M={M}")
    base = to_np(d.gemm(sep["xq"], sep["sx"]))
    assert np.array_equal(to_np(sep["y"])[~ref["active"]], base[~ref["active"]])
    if M <= ep.DECODE_MAX_M:
        fused = d.decode()
        assert torch.equal(fused["y"], sep["y"])
        assert ep.epilora_device_error(fused["ws"]) == 0
    # the separate up-projection: base GEMM, then the sliced expand-add
    y = d.gemm(sep["xq"], sep["sx"])
    ep.epilora_lora_expand_add(sep["z"], d.B, d.idx, d.scale, y, sep["ws"], ranks=d.ranks, mask=d.mask,
                               slices=slices)
    yg = bf16_np_to_f64(to_np(y))
    rms = np.sqrt(np.mean(ref["y"] ** 2))
    bound = 2.0 ** -8 * (np.abs(ref["base"]) + np.abs(ref["y"])) * 1.001 + 1e-4 * rms
    assert np.all(np.abs(yg - ref["y"]) <= bound)
    assert ep.epilora_device_error(sep["ws"]) == 0


# --- adapters stored in FP8 (E4M3 codes, one fp32 scale per row) --------------------------

FP8_ADAPTER_CASES = [
    # M, K, N, slices, L, r, idx kind, mask, ranks, wfmt
    (1, 4096, 2048, None, 1, 64, "zero", False, False, "fp8"),
    (7, 512, 384, None, 4, 16, "mixed", True, True, "fp8"),
    (32, 1024, 512, (256, 128, 128), 40, 32, "distinct", False, True, "fp8"),
    (64, 512, 256, None, 9, 128, "mixed", True, False, "fp4"),
    (300, 512, 640, (384, 256), 6, 64, "sorted", True, True, "fp8"),
    (1100, 256, 6144, None, 4, 128, "sorted", False, True, "fp8"),
    (150, 1024, 300, None, 5, 48, "mixed", False, True, "fp4"),
]


@pytest.mark.parametrize("M,K,N,slices,L,r,kind,use_mask,use_ranks,wfmt", FP8_ADAPTER_CASES)
def test_fp8_adapters_vs_oracle(M, K, N, slices, L, r, kind, use_mask, use_ranks, wfmt):
    say(f"fp8 adapters M={M} K={K} N={N} slices={slices} L={L} r={r} {kind} {wfmt}")
    rng = np.random.default_rng(9000 + M + K + N)
    idx = _idx(kind, M, L, rng)
    mask = rng.integers(0, 2, M).astype(np.uint8) if use_mask else None
    ranks = rng.choice([0, 16, r // 2, r, 13], size=L).astype(np.int32) if use_ranks else None
    lay = custom_layer("a8", 900 + M + N, M, K, N, L, r, idx, mask=mask, ranks=ranks, wfmt=wfmt, slices=slices)
    d = DeviceGemm(lay.gemms[0], wfmt, afmt="fp8")
    sep = d.separate()
    ref = d.oracle()   # also checks the library's adapter codes and scales bit for bit
    zg = to_np(sep["z"]).astype(np.float64)
    scale = max(np.sqrt(np.mean(ref["z"] ** 2)), 1e-30)
    assert np.abs(zg - ref["z"]).max() <= 1e-4 * scale
    compare(to_np(sep["y"]), ref["y"], f"fp8 adapters M={M}")
    base = to_np(d.gemm(sep["xq"], sep["sx"]))
    assert np.array_equal(to_np(sep["y"])[~ref["active"]], base[~ref["active"]])
    if M <= ep.DECODE_MAX_M:
        fused = d.decode()
        assert torch.equal(fused["y"], sep["y"])
        assert ep.epilora_device_error(fused["ws"]) == 0
    y = d.gemm(sep["xq"], sep["sx"])
    ep.epilora_lora_expand_add(sep["z"], d.B, d.idx, d.scale, y, sep["ws"], ranks=d.ranks, mask=d.mask,
                               slices=slices, sb=d.sb)
    yg = bf16_np_to_f64(to_np(y))
    rms = np.sqrt(np.mean(ref["y"] ** 2))
    bound = 2.0 ** -8 * (np.abs(ref["base"]) + np.abs(ref["y"])) * 1.001 + 1e-4 * rms
    assert np.all(np.abs(yg - ref["y"]) <= bound)
    assert ep.epilora_device_error(sep["ws"]) == 0


# --- the normalization with the quantizer and shrink fused in -----------------------------

NORM_CASES = [
    # M, K, L, r, slices, adapter format, with adapters
    (1, 4096, 1, 64, 1, "bf16", True),
    (7, 512, 4, 16, 1, "bf16", True),
    (33, 4096, 6, 32, 3, "bf16", True),
    (64, 8192, 9, 16, 1, "fp8", True),
    (300, 1024, 6, 64, 2, "bf16", True),
    (2048, 4096, 16, 128, 1, "bf16", True),
    (5, 256, 1, 16, 1, "bf16", False),
]


@pytest.mark.parametrize("M,K,L,r,S,afmt,with_a", NORM_CASES)
def test_norm_quant_shrink_vs_oracle(M, K, L, r, S, afmt, with_a):
    say(f"norm+quant+shrink M={M} K={K} L={L} r={r} S={S} {afmt} adapters={with_a}")
    rng = np.random.default_rng(9500 + M + K)
    x = bf16_bits((rng.standard_normal((M, K)) * rng.uniform(0.1, 10.0, (M, 1))).astype(np.float32))
    x[0, : K // 2] = 0                                   # a half-zero row
    gamma = bf16_bits((1.0 + 0.2 * rng.standard_normal(K)).astype(np.float32))
    idx = rng.integers(-1, L, M).astype(np.int32)
    ranks = rng.choice([0, 16, r], size=L).astype(np.int32) if M > 40 else None
    eps = 1e-5
    A_np = bf16_bits((rng.standard_normal((L, S, r, K)) / np.sqrt(K)).astype(np.float32))
    sa_np = None
    xd, gd = to_dev(x), to_dev(gamma)
    xn = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    xq = torch.empty(M, K, dtype=torch.uint8, device=DEV)
    sx = torch.empty(M, dtype=torch.float32, device=DEV)
    z = torch.empty(M, S * r, dtype=torch.float32, device=DEV)
    kw = {}
    if with_a:
        A_dev = to_dev(A_np if S > 1 else A_np[:, 0])
        if afmt == "fp8":
            A8 = torch.empty(A_dev.shape, dtype=torch.uint8, device=DEV)
            sa = torch.empty(A_dev.shape[:-1], dtype=torch.float32, device=DEV)
            ep.epilora_quant_weight_fp8(A_dev.reshape(-1, K), A8.view(-1, K), sa.view(-1))
            A_dev, kw["sa"] = A8, sa
            sa_np = to_np(sa).reshape(L, S, r) if S > 1 else to_np(sa)
        ws = ep.new_workspace(ep.OP_SHRINK, M, 0, K, S * r)
        kw.update(A=A_dev, idx=to_dev(idx), z=z, ws=ws, ranks=None if ranks is None else to_dev(ranks))
    ep.epilora_rmsnorm_quant_shrink(xd, gd, eps, xq, sx, xn=xn, **kw)
    torch.cuda.synchronize()
    xn_g = to_np(xn)
    ref = oracle.rmsnorm(x, gamma, eps)
    diff = xn_g != ref
    ulp = np.abs(xn_g.astype(np.int64) - ref.astype(np.int64))
    say(f"  xn: {int(diff.sum())} of {diff.size} values differ from the oracle (max {int(ulp.max())} ulp)")
    assert ulp.max() <= 1 and diff.mean() <= 1e-4
    # the codes and scales of the GPU's own normalized rows: bit for bit
    xq_ref, sx_ref = oracle.quant_act(xn_g)
    assert np.array_equal(to_np(sx), sx_ref) and np.array_equal(to_np(xq), xq_ref)
    if not with_a:
        return
    A_or = A_np if S > 1 else A_np[:, 0]
    if afmt == "fp8":
        A_or, sa_or = oracle.quant_adapter_fp8(A_or)
        assert np.array_equal(to_np(kw["A"]), A_or) and np.array_equal(to_np(kw["sa"]), sa_or)
    zs = [oracle.shrink(xn_g, A_or if S == 1 else A_or[:, s], idx, ranks,
                        a_scale=None if sa_np is None else (sa_np if S == 1 else sa_np[:, s])) for s in range(S)]
    z_ref = np.concatenate(zs, axis=1)
    zg = to_np(z).astype(np.float64)
    scale = max(np.sqrt(np.mean(z_ref ** 2)), 1e-30)
    assert np.abs(zg - z_ref).max() <= 1e-4 * scale
    act = oracle.active_rows(idx, L, r, ranks)[0]
    assert not zg[~act].any()
    assert ep.epilora_device_error(kw["ws"]) == 0
    # bitwise the separate shrink on the normalized rows (same summation order)
    z2 = torch.empty_like(z)
    ep.epilora_lora_shrink(xn, kw["A"], kw["idx"], z2, kw["ws"], ranks=kw["ranks"], sa=kw.get("sa"))
    assert torch.equal(z, z2)


def test_norm_path_equals_fused_decode():
    # qkv-shaped projection with per-slice adapters: normalization kernel
    # (quantizer and shrink inside), then the GEMM with z given, against the
    # fused decode path on the normalized rows: bit for bit.
    say("norm path vs fused decode, qkv shape")
    from workloads import config
    g = config(2, sliced=True).gemm("qkv")
    rng = np.random.default_rng(77)
    gamma = bf16_bits((1.0 + 0.1 * rng.standard_normal(g.K)).astype(np.float32))
    d = DeviceGemm(g)
    xn = torch.empty(d.M, d.K, dtype=torch.bfloat16, device=DEV)
    xq = torch.empty(d.M, d.K, dtype=torch.uint8, device=DEV)
    sx = torch.empty(d.M, dtype=torch.float32, device=DEV)
    z = torch.empty(d.M, d.S * d.r, dtype=torch.float32, device=DEV)
    ws = ep.new_workspace(ep.OP_SHRINK, d.M, d.N, d.K, d.S * d.r)
    ep.epilora_rmsnorm_quant_shrink(d.x, to_dev(gamma), 1e-5, xq, sx, xn=xn, A=d.A, idx=d.idx, z=z, ws=ws)
    y = d.gemm(xq, sx, z, ws)
    d2 = DeviceGemm(g, x=to_np(xn))
    fused = d2.decode()
    assert torch.equal(fused["xq"], xq) and torch.equal(fused["sx"], sx)
    assert torch.equal(fused["y"], y)
    ref = d2.oracle(cols=np.arange(0, d.N, 7))
    from gpu_harness import compare
    compare(to_np(y)[:, np.arange(0, d.N, 7)], ref["y"], "norm path")


# --- the matched W8A16 GEMM ----------------------------------------------------------------

A16_CASES = [
    # M, K, N, slices, L, r, idx kind, mask, ranks, adapter format
    (1, 4096, 1024, None, 1, 64, "zero", False, False, "bf16"),
    (4, 1024, 512, None, 4, 16, "mixed", True, True, "bf16"),
    (24, 4096, 512, None, 6, 32, "mixed", False, False, "bf16"),
    (64, 512, 256, (128, 128), 9, 16, "mixed", True, False, "fp8"),
    (200, 1024, 384, None, 6, 64, "sorted", True, True, "bf16"),
    (1100, 512, 2048, (1024, 1024), 4, 128, "sorted", False, True, "bf16"),
    (130, 4096, 300, None, 5, 32, "mixed", False, False, "fp8"),
]


@pytest.mark.parametrize("M,K,N,slices,L,r,kind,use_mask,use_ranks,afmt", A16_CASES)
def test_w8a16_vs_oracle(M, K, N, slices, L, r, kind, use_mask, use_ranks, afmt):
    say(f"W8A16 M={M} K={K} N={N} slices={slices} L={L} r={r} {kind} adapters {afmt}")
    rng = np.random.default_rng(9700 + M + K + N)
    idx = _idx(kind, M, L, rng)
    mask = rng.integers(0, 2, M).astype(np.uint8) if use_mask else None
    ranks = rng.choice([0, 16, r // 2, r], size=L).astype(np.int32) if use_ranks else None
    lay = custom_layer("a16", 970 + M + N, M, K, N, L, r, idx, mask=mask, ranks=ranks, slices=slices)
    d = DeviceGemm(lay.gemms[0], afmt=afmt, a16=True)
    sep = d.separate()
    ref = d.oracle()
    compare(to_np(sep["y"]), ref["y"], f"W8A16 M={M}")
    base = to_np(d.gemm(None, None))
    compare(base, ref["base"], "W8A16 base")
    assert np.array_equal(to_np(sep["y"])[~ref["active"]], base[~ref["active"]])
    if M <= ep.DECODE_MAX_M:
        fused = d.decode()
        assert torch.equal(fused["y"], sep["y"])
        assert ep.epilora_device_error(fused["ws"]) == 0
    again = d.gemm(None, None, sep["z"], sep["ws"])
    assert torch.equal(again, sep["y"])
