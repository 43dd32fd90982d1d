// The shrink's workgroup-level pieces, shared by the shrink kernel and the
// fused decode path.
#pragma once

#include "adapters.h"
#include "layout.h"

namespace epilora {

constexpr int kShrinkThreads = 256;
constexpr int kMaxJB = 8;  // r <= 128 -> at most 8 blocks of 16 rank rows

// ---------------------------------------------------------------------------
// Shrink.  Workgroup (tile, split): 16 consecutive tokens and a range of
// 128-wide K steps; its 4 waves take every 4th step.  For each adapter that
// some token of the tile uses, a wave multiplies that adapter's A rows (16 at
// a time, the matrix-core rows) by the bf16 activations of the tokens using
// it (the other token columns are zero), on bf16 MFMA with fp32
// accumulation.  Columns of different adapters are disjoint, so one set of
// accumulators serves every adapter.  Lane l holds rank row (l % 16) of A and
// token column (l % 16) of x, and elements [32 (l / 16), +32) of each
// 128-wide step, 8 per MFMA: A and x use the same K positions, so each MFMA
// pairs matching elements.
// The 4 waves are summed in LDS in wave order; splits write fp32 partials
// and the last workgroup of a tile (an agent-scope counter) adds them in
// split order, so the result does not depend on timing.
// ---------------------------------------------------------------------------
struct ShrinkParams {
  const uint16_t* x;
  int64_t M, K, ldx;
  AdapterArgs ad;
  float* z;
  int* ctrl;
  int* counters;
  float* partials;
  int splits;
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// One workgroup's contribution to z for 16 tokens; sums the waves and
// leaves the [16][r] result in `out` (LDS).
__device__ __forceinline__ void shrink_tile(const ShrinkParams& p, int64_t t0, int s_begin, int s_end,
                                            float* red, bool report) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int r = p.ad.r;
  const int64_t K = p.K;
  int rank_c;
  const int a_c = resolve_token(t0 + col, p.M, p.ad, p.ctrl + kCtrlError, report && lane < 16 && wave == 0, rank_c);

  f32x4 acc[kMaxJB];
#pragma unroll
  for (int j = 0; j < kMaxJB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint64_t pending = __ballot(lane < 16 && a_c >= 0);
  while (pending) {
    const int leader = __ffsll((unsigned long long)pending) - 1;
    const int a = __shfl(a_c, leader);
    const int rank = __shfl(rank_c, leader);
    const uint64_t members = __ballot(lane < 16 && a_c == a);
    pending &= ~members;
    const bool member = (members >> col) & 1;
    const int jbn = (rank + 15) >> 4;
    const uint16_t* Aa = p.ad.A + (int64_t)a * r * K;
    const uint16_t* xr = p.x + (t0 + col) * p.ldx;
    for (int s = s_begin + wave; s < s_end; s += 4) {
      const int64_t k = (int64_t)s * kShrinkStep + grp * 32;
      uint4 xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[i] = (member && k + i * 8 < K) ? ld16(xr + k + i * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int jb = 0; jb < kMaxJB; ++jb) {
        if (jb < jbn) {
          const int j = jb * 16 + col;
          const bool rowok = j < rank;
          const uint16_t* ar = Aa + (int64_t)j * K + k;
          uint4 av[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            av[i] = (rowok && k + i * 8 < K) ? ld16(ar + i * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[jb] = mfma_bf16_16x16x32(as_bf16x8(av[i]), as_bf16x8(xv[i]), acc[jb]);
        }
      }
    }
  }

  // acc[jb][v] = z[token col][jb*16 + 4*grp + v]; sum the 4 waves in order.
  const int jbr = r >> 4;
#pragma unroll
  for (int jb = 0; jb < kMaxJB; ++jb)
    if (jb < jbr)
      *reinterpret_cast<float4*>(&red[(wave * 16 + col) * r + jb * 16 + 4 * grp]) =
          make_float4(acc[jb][0], acc[jb][1], acc[jb][2], acc[jb][3]);
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * r; e += kShrinkThreads) {
    float v = red[e];
    v += red[16 * r + e];
    v += red[32 * r + e];
    v += red[48 * r + e];
    red[e] = v;
  }
  __syncthreads();
}

// Write this workgroup's [16][r] sums (in LDS `red`) to z, or to its split's
// partial; the last split of a tile adds the partials in split order.
// Returns true in the workgroup that wrote the tile's final z.
__device__ __forceinline__ bool shrink_finish(const ShrinkParams& p, int tile, int split, const float* red) {
  __shared__ int last;
  const int64_t t0 = (int64_t)tile * kShrinkTokens;
  const int r = p.ad.r;
  if (p.splits == 1) {
    for (int e = threadIdx.x; e < 16 * r; e += kShrinkThreads) {
      const int64_t t = t0 + e / r;
      if (t < p.M) p.z[t * r + e % r] = red[e];
    }
    return true;
  }
  for (int e = threadIdx.x; e < 16 * r; e += kShrinkThreads) {
    const int64_t t = t0 + e / r;
    if (t < p.M) p.partials[((int64_t)split * p.M + t) * r + e % r] = red[e];
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last = atomic_add_acq_rel(&p.counters[tile], 1) == p.splits - 1;
  __syncthreads();
  if (!last) return false;
  __threadfence();
  for (int e = threadIdx.x; e < 16 * r; e += kShrinkThreads) {
    const int64_t t = t0 + e / r;
    if (t >= p.M) continue;
    float v = 0.f;
    for (int s = 0; s < p.splits; ++s) v += p.partials[((int64_t)s * p.M + t) * r + e % r];
    p.z[t * r + e % r] = v;
  }
  if (threadIdx.x == 0) store_relaxed(&p.counters[tile], 0);
  return true;
}

// K-step range of split `split`.
__device__ __forceinline__ void shrink_range(const ShrinkParams& p, int split, int& s_begin, int& s_end) {
  const int steps = (int)cdiv(p.K, kShrinkStep);
  const int spw = (int)cdiv(steps, p.splits);
  s_begin = split * spw;
  s_end = min(steps, s_begin + spw);
}

}  // namespace epilora
