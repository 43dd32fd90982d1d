"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times: the fused decode path for the decode batches (M <= 64)
and quant + shrink + tiled GEMM for the 2048-token prefill GEMMs.  The oracle
computes a seeded sample of tokens and output channels; quantized
activations and weight codes of the sample are bit-exact."""

import numpy as np
import pytest
import torch

import fp4_gemm_amd as ep
from workloads import config

from gpu_harness import DeviceGemm, compare, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


def say(*a):
    print(*a, flush=True)


def sample(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=min(n, k), replace=False))


def check(d, out, rows=None, ncols=256, seed=0, what=""):
    cols = sample(d.N, ncols, seed)
    ref = d.oracle(rows=rows, cols=cols)
    xq = to_np(out["xq"]) if rows is None else to_np(out["xq"])[rows]
    sx = to_np(out["sx"]) if rows is None else to_np(out["sx"])[rows]
    assert np.array_equal(xq, ref["xq"]), f"{what}: activation codes"
    assert np.array_equal(sx, ref["sx"]), f"{what}: activation scales"
    if d.wfmt == "fp8":
        assert np.array_equal(to_np(d.wq)[cols], ref["w"]["wq"]), f"{what}: weight codes"
    else:
        assert np.array_equal(to_np(d.wq)[cols], ref["w"]["wc"]), f"{what}: 4-bit codes"
        assert np.array_equal(to_np(d.bs)[cols], ref["w"]["bs"]), f"{what}: block scales"
    y = to_np(out["y"])
    y = y[:, cols] if rows is None else y[np.ix_(rows, cols)]
    mx, mean = compare(y, ref["y"], what)
    say(f"  {what}: max|dY|/rms {mx:.2e}  mean rel {mean:.2e}")
    return ref


def test_config1_toy():
    lay = config(1)
    d = DeviceGemm(lay.gemms[0])
    ref = d.oracle()
    for out in (d.decode(), d.separate()):
        compare(to_np(out["y"]), ref["y"], "toy")
        assert np.array_equal(to_np(out["xq"]), ref["xq"])


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down"])
def test_config2_llama8b_decode(name):
    say(f"config 2 {name}")
    d = DeviceGemm(config(2).gemm(name))
    fused = d.decode()
    check(d, fused, seed=21, what=f"cfg2 {name} fused")
    sep = d.separate()
    assert torch.equal(sep["y"], fused["y"])
    assert ep.epilora_device_error(fused["ws"]) == 0


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down"])
def test_config3_multitenant_decode(name):
    say(f"config 3 {name}")
    lay = config(3)
    d = DeviceGemm(lay.gemm(name))
    fused = d.decode()
    ref = check(d, fused, seed=31, what=f"cfg3 {name} fused")
    assert ref["active"].sum() == 28
    # rows without an adapter equal the base GEMM bit for bit
    xq, sx = d.quant()
    base = to_np(d.gemm(xq, sx))
    y = to_np(fused["y"])
    assert np.array_equal(y[lay.idx < 0], base[lay.idx < 0])


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down"])
def test_config4_72b_preft(name):
    for M in (64, 8, 1):
        say(f"config 4 {name} M={M}")
        lay = config(4, M=M)
        d = DeviceGemm(lay.gemm(name))
        fused = d.decode()
        ref = check(d, fused, seed=40 + M, what=f"cfg4 {name} M={M}")
        # PreFT: masked-off rows equal the base GEMM exactly
        y = torch.empty_like(fused["y"])
        ws = ep.new_workspace(ep.OP_DECODE, d.M, d.N, d.K, 16)
        ep.epilora_decode_lora(d.x, d.wq, y, ws=ws, **d.wkw)
        off = lay.mask == 0
        assert np.array_equal(to_np(fused["y"])[off], to_np(y)[off])
        assert ref["active"].sum() == int(np.ceil(0.75 * M))
        del d


@pytest.mark.parametrize("wfmt,segments,name", [
    ("fp8", 16, "gate_up"), ("fp8", 16, "down"), ("fp4", 16, "gate_up"), ("fp4", 16, "down"),
    ("fp8", 32, "gate_up"), ("fp8", 32, "down"), ("fp4", 32, "gate_up"), ("fp4", 32, "down"),
])
def test_config5_prefill(wfmt, segments, name):
    say(f"config 5 {wfmt} {segments} segments {name}")
    lay = config(5, segments=segments, wfmt=wfmt)
    d = DeviceGemm(lay.gemm(name), wfmt)
    out = d.separate()
    # a seeded sample plus the first and last token of every segment
    starts = np.flatnonzero(np.r_[True, lay.idx[1:] != lay.idx[:-1]])
    ends = np.r_[starts[1:] - 1, d.M - 1]
    rows = np.unique(np.concatenate([sample(d.M, 96, 50 + segments), starts, ends]))
    ref = check(d, out, rows=rows, seed=51, what=f"cfg5 {wfmt} {name}")
    assert ep.epilora_device_error(out["ws"]) == 0
    if wfmt == "fp4":
        # Diagnostic: how far the GPU's 4-bit path (weights folded to FP8
        # bytes) lies from exact NVFP4 arithmetic on the same codes.
        import oracle
        wc, bs, gs = ref["w"]["wc"], ref["w"]["bs"], ref["w"]["gs"]
        wx = oracle.exact_decode_fp4(wc, bs, gs)
        xq = to_np(out["xq"])[rows]
        sx = to_np(out["sx"])[rows].astype(np.float64)
        exact = (oracle.e4m3_decode(xq) @ wx.T) * sx[:, None]
        base = ref["base"]
        dev = np.abs(base - exact)
        rms = np.sqrt(np.mean(exact ** 2))
        say(f"  4-bit fold vs exact NVFP4 (base term): max|d|/rms {dev.max() / rms:.3e}  "
            f"mean rel {dev.sum() / np.abs(exact).sum():.3e}")


@pytest.mark.parametrize("name", ["qkv", "gate_up"])
def test_config2_sliced_adapters(name):
    # the Llama-8B decode projections with one adapter pair per output slice
    say(f"config 2 sliced {name}")
    d = DeviceGemm(config(2, sliced=True).gemm(name))
    fused = d.decode()
    check(d, fused, seed=23, what=f"cfg2 sliced {name} fused")
    sep = d.separate()
    assert torch.equal(sep["y"], fused["y"])


def test_config3_sliced_qkv():
    say("config 3 sliced qkv")
    d = DeviceGemm(config(3, sliced=True).gemm("qkv"))
    fused = d.decode()
    check(d, fused, seed=33, what="cfg3 sliced qkv fused")


@pytest.mark.parametrize("wfmt", ["fp8", "fp4"])
def test_config5_sliced_gate_up(wfmt):
    say(f"config 5 sliced gate_up {wfmt}")
    lay = config(5, segments=32, wfmt=wfmt, sliced=True)
    d = DeviceGemm(lay.gemm("gate_up"), wfmt)
    out = d.separate()
    starts = np.flatnonzero(np.r_[True, lay.idx[1:] != lay.idx[:-1]])
    rows = np.unique(np.concatenate([sample(d.M, 64, 55), starts]))
    check(d, out, rows=rows, seed=56, what=f"cfg5 sliced gate_up {wfmt}")


@pytest.mark.parametrize("name", ["qkv", "gate_up", "down"])
def test_config3_fp8_adapters(name):
    # the many-distinct-adapters decode batch with adapters stored in FP8
    say(f"config 3 FP8 adapters {name}")
    d = DeviceGemm(config(3).gemm(name), afmt="fp8")
    fused = d.decode()
    check(d, fused, seed=34, what=f"cfg3 fp8 adapters {name}")


def test_config5_fp8_adapters():
    say("config 5 FP8 adapters gate_up 32 segments")
    lay = config(5, segments=32)
    d = DeviceGemm(lay.gemm("gate_up"), afmt="fp8")
    out = d.separate()
    starts = np.flatnonzero(np.r_[True, lay.idx[1:] != lay.idx[:-1]])
    rows = np.unique(np.concatenate([sample(d.M, 64, 57), starts]))
    check(d, out, rows=rows, seed=58, what="cfg5 fp8 adapters gate_up")


@pytest.mark.parametrize("name", ["qkv", "down"])
def test_config2_w8a16(name):
    # the matched engine's GEMM on the Llama-8B decode projections
    say(f"config 2 W8A16 {name}")
    d = DeviceGemm(config(2).gemm(name), a16=True)
    fused = d.decode()
    cols = sample(d.N, 256, 24)
    ref = d.oracle(cols=cols)
    mx, mean = compare(to_np(fused["y"])[:, cols], ref["y"], f"cfg2 W8A16 {name}")
    say(f"  cfg2 W8A16 {name}: max|dY|/rms {mx:.2e}  mean rel {mean:.2e}")


def test_config5_w8a16_gate_up():
    say("config 5 W8A16 gate_up 16 segments")
    lay = config(5, segments=16)
    d = DeviceGemm(lay.gemm("gate_up"), a16=True)
    out = d.separate()
    rows = sample(d.M, 64, 59)
    cols = sample(d.N, 256, 60)
    ref = d.oracle(rows=rows, cols=cols)
    compare(to_np(out["y"])[np.ix_(rows, cols)], ref["y"], "cfg5 W8A16 gate_up")
