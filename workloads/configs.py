"""The five synthetic workloads and their seeded generators (no layer
arithmetic here; see the package docstring)."""

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

# (name, K in, N out) per projection of one decoder layer.
GEMMS_8B = (("qkv", 4096, 6144), ("o", 4096, 4096),
            ("gate_up", 4096, 28672), ("down", 14336, 4096))
GEMMS_72B = (("qkv", 8192, 10240), ("o", 8192, 8192),
             ("gate_up", 8192, 59136), ("down", 29568, 8192))
# Output slices of the projections that concatenate several outputs, each
# with its own adapter pair when the adapters are per slice: query / key /
# value under grouped-query attention (8 key-value heads of 128) and the
# MLP's gate / up.
SLICES_8B = {"qkv": (4096, 1024, 1024), "gate_up": (14336, 14336)}
SLICES_72B = {"qkv": (8192, 1024, 1024), "gate_up": (29568, 29568)}

# Tensor tags inside a seed key.
_X, _W, _A, _B, _IDX, _MASK, _SEG = range(7)

X_STD, W_STD, B_STD = 1.0, 0.02, 0.01
LORA_SCALE = 2.0


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def bf16_bits(v):
    """float32 array -> bf16 bit patterns (uint16), by torch's conversion
    (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal_bf16(rng, shape, std):
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return bf16_bits(v)


@dataclass
class GemmCase:
    """One projection's inputs.  x, w, A and B are drawn on demand."""
    name: str
    M: int
    K: int
    N: int
    layer: "Layer"
    gemm_id: int
    slices: Optional[tuple] = None   # output slice widths (per-slice adapters)

    def key(self, tag, *rest):
        return (self.layer.seed, self.gemm_id, tag) + tuple(rest)

    def x(self):
        """uint16 [M][K] bf16 activations."""
        return _normal_bf16(_rng(*self.key(_X, self.layer.x_variant)),
                            (self.M, self.K), X_STD)

    def w(self):
        """uint16 [N][K] bf16 weights (quantised by the caller)."""
        return _normal_bf16(_rng(*self.key(_W)), (self.N, self.K), W_STD)

    def _adapters(self, which):
        if which is None:
            which = self.layer.referenced_adapters()
        return sorted(set(int(a) for a in which))

    def A(self, which=None):
        """uint16 [L][r][K]: rows j >= rank of each adapter are zero; slots
        not in `which` (default: the adapters some token references) are
        zero too, since no output can depend on them."""
        lay = self.layer
        out = np.zeros((lay.L, lay.r, self.K), dtype=np.uint16)
        std = 1.0 / np.sqrt(self.K)
        for a in self._adapters(which):
            rk = lay.rank_of(a)
            out[a, :rk] = _normal_bf16(_rng(*self.key(_A, a)), (rk, self.K), std)
        return out

    def A_sliced(self, which=None):
        """uint16 [L][S][r][K]: the per-slice down-projections of a
        projection with output slices (S = 1 without slices), drawn per
        (adapter, slice); zero past each adapter's rank and for slots no
        token references."""
        lay = self.layer
        S = len(self.slices) if self.slices else 1
        out = np.zeros((lay.L, S, lay.r, self.K), dtype=np.uint16)
        std = 1.0 / np.sqrt(self.K)
        for a in self._adapters(which):
            rk = lay.rank_of(a)
            for sl in range(S):
                out[a, sl, :rk] = _normal_bf16(_rng(*self.key(_A, a, 1000 + sl)), (rk, self.K), std)
        return out

    def B(self, which=None):
        """uint16 [L][N][r]: columns j >= rank of each adapter are zero."""
        lay = self.layer
        out = np.zeros((lay.L, self.N, lay.r), dtype=np.uint16)
        for a in self._adapters(which):
            rk = lay.rank_of(a)
            out[a, :, :rk] = _normal_bf16(_rng(*self.key(_B, a)), (self.N, rk), B_STD)
        return out


@dataclass
class Layer:
    """A set of projections that share one batch's tenant metadata."""
    name: str
    seed: int
    M: int
    L: int
    r: int
    idx: np.ndarray                      # int32 [M], -1 = no adapter
    mask: Optional[np.ndarray] = None    # uint8 [M] or None
    ranks: Optional[np.ndarray] = None   # int32 [L] or None (all rank r)
    scale: float = LORA_SCALE
    wfmt: str = "fp8"
    x_variant: int = 0
    shapes: Sequence = ()
    slices: Optional[dict] = None        # projection name -> slice widths
    gemms: List[GemmCase] = field(default_factory=list)

    def __post_init__(self):
        sl = self.slices or {}
        self.gemms = [GemmCase(n, self.M, k, nn, self, i, sl.get(n))
                      for i, (n, k, nn) in enumerate(self.shapes)]

    def rank_of(self, a):
        return self.r if self.ranks is None else int(self.ranks[a])

    def referenced_adapters(self):
        return sorted(set(int(a) for a in self.idx if 0 <= a < self.L))

    def gemm(self, name):
        for g in self.gemms:
            if g.name == name:
                return g
        raise KeyError(name)


def _segments(rng, M, S):
    """Segment lengths from a flat Dirichlet: floor(p*M), the remainder
    handed out by largest fractional part, every segment at least 1."""
    p = rng.dirichlet(np.ones(S))
    raw = p * M
    lens = np.floor(raw).astype(np.int64)
    order = np.argsort(-(raw - lens), kind="stable")
    for i in order[: M - int(lens.sum())]:
        lens[i] += 1
    while (lens == 0).any():
        lens[int(np.argmax(lens))] -= 1
        lens[int(np.argmin(lens))] += 1
    return lens


def config(n, *, M=None, segments=16, wfmt="fp8", sliced=False):
    """The five workloads.

    1  toy: M=4, K=256 -> N=512, 4 tenants of rank 16, idx [0, 1, -1, 3].
    2  Llama-8B-shaped decode layer: M=1, one rank-64 tenant.
    3  Llama-8B-shaped multi-tenant decode: M=32, 64 resident rank-64
       adapters; 32 distinct tenants drawn from 0..63, then 4 tokens set
       to -1.
    4  72B-shaped prefill-only (PreFT) layer: M in {1, 8, 64}, 512 rank-16
       adapters, Zipf(1.1) tenants, mask = the first ceil(0.75 M) tokens.
    5  prefill GEMMs (gate_up, down) at M=2048 in `segments` contiguous
       tenant segments (flat Dirichlet lengths), ranks cycling through
       16/32/64/128 over a seeded shuffle of the segments, padded to 128;
       wfmt "fp8" or "fp4".
    With sliced=True the projections that concatenate several outputs (qkv:
    3 slices, gate_up: 2) carry one adapter pair per slice (A_sliced()).
    """
    if n == 1:
        idx = np.array([0, 1, -1, 3], dtype=np.int32)
        return Layer("toy", 1, 4, 4, 16, idx, shapes=(("toy", 256, 512),))
    if n == 2:
        return Layer("llama8b_decode_m1" + ("_sliced" if sliced else ""), 2, 1, 1, 64, np.zeros(1, np.int32),
                     shapes=GEMMS_8B, slices=SLICES_8B if sliced else None)
    if n == 3:
        rng = _rng(3, 0, _IDX)
        idx = rng.choice(64, size=32, replace=False).astype(np.int32)
        off = rng.choice(32, size=4, replace=False)
        idx[off] = -1
        return Layer("llama8b_decode_m32_tenants" + ("_sliced" if sliced else ""), 3, 32, 64, 64, idx,
                     shapes=GEMMS_8B, slices=SLICES_8B if sliced else None)
    if n == 4:
        M = 1 if M is None else int(M)
        rng = _rng(4, M, _IDX)
        p = np.arange(1, 513, dtype=np.float64) ** -1.1
        idx = rng.choice(512, size=M, p=p / p.sum()).astype(np.int32)
        mask = np.zeros(M, dtype=np.uint8)
        mask[: -(-3 * M // 4)] = 1  # ceil(0.75 M)
        return Layer(f"qwen72b_preft_m{M}" + ("_sliced" if sliced else ""), 4, M, 512, 16, idx, mask=mask,
                     shapes=GEMMS_72B, x_variant=M, slices=SLICES_72B if sliced else None)
    if n == 5:
        M = 2048 if M is None else int(M)
        S = int(segments)
        rng = _rng(5, S, _SEG)
        lens = _segments(rng, M, S)
        perm = rng.permutation(S)
        ranks = np.zeros(S, dtype=np.int32)
        for i, s in enumerate(perm):
            ranks[s] = (16, 32, 64, 128)[i % 4]
        idx = np.repeat(np.arange(S, dtype=np.int32), lens)
        return Layer(f"llama8b_prefill_m{M}_s{S}_{wfmt}" + ("_sliced" if sliced else ""), 5, M, S, 128, idx,
                     ranks=ranks, wfmt=wfmt, x_variant=S,
                     shapes=(GEMMS_8B[2], GEMMS_8B[3]), slices=SLICES_8B if sliced else None)
    raise ValueError(f"no config {n}")


def custom_layer(name, seed, M, K, N, L, r, idx, *, mask=None, ranks=None,
                 scale=LORA_SCALE, wfmt="fp8", slices=None):
    """A one-projection layer of any shape (parity sweeps, edge cases);
    `slices`: output slice widths for per-slice adapters."""
    return Layer(name, seed, M, L, r, np.asarray(idx, dtype=np.int32),
                 mask=None if mask is None else np.asarray(mask, np.uint8),
                 ranks=None if ranks is None else np.asarray(ranks, np.int32),
                 scale=scale, wfmt=wfmt, shapes=((name, K, N),),
                 slices=None if slices is None else {name: tuple(slices)})
