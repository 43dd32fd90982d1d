"""The fused decode path on the library's fixed scratch
(epilora_decode_lora_noalloc), through the C ABI, against the same path on a
caller-owned workspace (epilora_decode_lora): two calls in a row, the second
with a smaller batch and a smaller layer, each bitwise equal to the
workspace path and within tolerance of the oracle."""

import numpy as np
import pytest
import torch

import fp4_gemm_amd as ep
from workloads import custom_layer

from gpu_harness import DEV, DeviceGemm, compare, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


def _noalloc(d):
    y = torch.empty(d.M, d.N, dtype=torch.bfloat16, device=DEV)
    xq = torch.empty(d.M, d.K, dtype=torch.uint8, device=DEV)
    sx = torch.empty(d.M, dtype=torch.float32, device=DEV)
    ep.epilora_decode_lora_noalloc(d.x, d.wq, y, A=d.A, B=d.B, idx=d.idx, ranks=d.ranks, mask=d.mask,
                                   scale=d.scale, xq_out=xq, sx_out=sx, **d.wkw)
    return dict(y=y, xq=xq, sx=sx)


def test_noalloc_matches_workspace_path_twice():
    rng = np.random.default_rng(77)
    big = custom_layer("na1", 1501, 24, 4096, 1024, 6, 64, rng.integers(-1, 6, 24), wfmt="fp8")
    small = custom_layer("na2", 1502, 3, 512, 384, 2, 16, [1, -1, 0], wfmt="fp4")
    for lay, wfmt in ((big, "fp8"), (small, "fp4")):
        d = DeviceGemm(lay.gemms[0], wfmt)
        print(f"noalloc M={d.M} K={d.K} N={d.N} {wfmt}", flush=True)
        got = _noalloc(d)
        want = d.decode()
        assert torch.equal(got["y"], want["y"])
        assert torch.equal(got["xq"], want["xq"]) and torch.equal(got["sx"], want["sx"])
        ref = d.oracle()
        compare(to_np(got["y"]), ref["y"], f"noalloc M={d.M}")
        assert np.array_equal(to_np(got["xq"]), ref["xq"])


def test_noalloc_rejects_oversized_call():
    d = DeviceGemm(custom_layer("na3", 1503, 64, 262144, 16, 1, 16, np.zeros(64, np.int32)).gemms[0])
    y = torch.empty(d.M, d.N, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ep.EpiloraError) as e:
        ep.epilora_decode_lora_noalloc(d.x, d.wq, y, A=d.A, B=d.B, idx=d.idx, scale=d.scale, **d.wkw)
    assert e.value.status == ep.ERR_WORKSPACE
