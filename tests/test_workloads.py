"""The seeded input recipe: determinism and the structure each workload
promises (shapes, tenant draws, masks, segments, ranks)."""

import numpy as np

from workloads import GEMMS_8B, GEMMS_72B, config


def test_config1_toy():
    lay = config(1)
    g = lay.gemms[0]
    assert (lay.M, g.K, g.N, lay.L, lay.r) == (4, 256, 512, 4, 16)
    assert lay.idx.tolist() == [0, 1, -1, 3] and lay.scale == 2.0
    x1, x2 = g.x(), g.x()
    assert x1.dtype == np.uint16 and np.array_equal(x1, x2)
    A = g.A()
    assert A.shape == (4, 16, 256) and not A[2].any() and A[3].any()


def test_config2_and_3_shapes_and_tenants():
    l2 = config(2)
    assert [(g.name, g.K, g.N) for g in l2.gemms] == list(GEMMS_8B)
    assert l2.M == 1 and l2.r == 64 and l2.idx.tolist() == [0]
    l3 = config(3)
    assert l3.M == 32 and l3.L == 64
    act = l3.idx[l3.idx >= 0]
    assert (l3.idx == -1).sum() == 4 and len(set(act.tolist())) == 28
    assert act.min() >= 0 and act.max() < 64


def test_config4_preft_mask_and_zipf():
    for M, n_on in ((1, 1), (8, 6), (64, 48)):
        lay = config(4, M=M)
        assert [(g.K, g.N) for g in lay.gemms] == [(k, n) for _, k, n in GEMMS_72B]
        assert lay.mask.tolist() == [1] * n_on + [0] * (M - n_on)
        assert lay.L == 512 and lay.r == 16
        assert lay.idx.min() >= 0 and lay.idx.max() < 512
    # Zipf(1.1): small indices dominate
    big = config(4, M=64).idx
    assert np.median(big) < 64


def test_config5_segments():
    for S in (16, 32):
        lay = config(5, segments=S)
        assert lay.M == 2048 and lay.L == S and lay.r == 128
        lens = np.bincount(lay.idx, minlength=S)
        assert lens.sum() == 2048 and lens.min() >= 1
        assert np.all(np.diff(lay.idx) >= 0)  # contiguous, sorted segments
        assert sorted(set(lay.ranks.tolist())) == [16, 32, 64, 128]
        assert np.bincount(lay.ranks)[[16, 32, 64, 128]].tolist() == [S // 4] * 4
    g = config(5, M=64).gemm("down")
    B = g.B()
    for a in range(g.layer.L):
        rk = g.layer.ranks[a]
        assert not B[a, :, rk:].any()
        if a in g.layer.referenced_adapters():
            assert B[a, :, :rk].any()


def test_distributions():
    g = config(1).gemms[0]
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    assert abs(f(g.x()).std() - 1.0) < 0.1
    assert abs(f(g.w()).std() - 0.02) < 0.002
    A = f(g.A([0]))[0]
    assert abs(A.std() - 1 / 16) < 0.006
