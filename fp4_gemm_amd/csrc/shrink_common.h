// The shrink's workgroup-level pieces: the 16-token tile with split-K
// partials and their fixed-order combine (the normalization kernel's shrink
// over more than 64 tokens; the combine also serves the prefill shrink), and
// the unit shrink of decode batches, shared by the shrink kernel and the
// fused decode path.
#pragma once

#include "adapters.h"
#include "layout.h"

namespace epilora {

constexpr int kMaxJB = 8;  // r <= 128 -> at most 8 blocks of 16 rank rows
// The shrink's work is laid out over this many waves whatever the block size
// (further waves of a larger block idle), so its sums round the same way in
// every kernel that carries it.
constexpr int kShrinkWaves = 4;

// ---------------------------------------------------------------------------
// Shrink tile.  A workgroup owns 16 consecutive tokens and a range of
// 128-wide K steps.  For each adapter that some token of the tile uses, the
// adapter's A rows (16 at a time, the matrix-core rows) multiply the bf16
// activations of the tokens using it (the other token columns are zero), on
// bf16 MFMA with fp32 accumulation; columns of different adapters are
// disjoint, so one set of accumulators serves every adapter.  Lane l holds
// rank row (l % 16) of A and token column (l % 16) of x, elements
// [32 (l / 16), +32) of each step, 8 per MFMA: both operands see the same K
// positions, so each MFMA pairs matching elements.
// The waves form a WJ x WS grid: wave w takes the rank blocks jb with
// jb % WJ == w % WJ and every WS-th step from w / WJ, so a small rank still
// keeps every wave busy.  The waves are summed in LDS in wave order; split
// workgroups publish fp32 partials with device-coherent stores, and the
// last one of a tile (an agent-scope counter) adds them in a fixed order
// (consecutive splits in chunks, then the chunks), so the result does not
// depend on timing.
// ---------------------------------------------------------------------------
struct ShrinkParams {
  const uint16_t* x;
  int64_t M, K, ldx;
  AdapterArgs ad;
  float* z;  // [M][ad.zld]
  int* ctrl;
  int* counters;
  float* partials;
  int splits;
  uint32_t zflip;  // z words are stored XOR this (the fused path stores complements)
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// One workgroup's sums for 16 tokens over its K steps; leaves the [16][r]
// result in `red` (LDS of kShrinkWaves * 16 * r floats) and returns the
// tile's active tokens as a bit mask (bit i: token t0 + i).  Every thread of
// the block must call it.
// The activations the shrink multiplies, as loaded: 8 bf16 of token column
// `col` at K offset k.  The shrink taken inside the normalization kernel
// passes a transform that normalizes them on the fly.
struct XIdentity {
  __device__ __forceinline__ uint4 operator()(const uint4& v, int64_t, int) const { return v; }
};

// `slice`: which of the projection's output slices (its own A) this is.
// `xt` maps the loaded activations to the values the shrink multiplies.
// GEN: the general adapters (several output slices, FP8 storage) may occur;
// without it the code assumes one slice of bf16 adapters (fewer registers in
// the kernels that carry this code beside a weight stream).
template <int NW, bool GEN = true, typename XT = XIdentity>
__device__ __forceinline__ uint64_t shrink_tile(const ShrinkParams& p, int64_t t0, int slice, int s_begin, int s_end,
                                                float* red, bool report, const XT& xt = XT()) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int r = p.ad.r;
  const int64_t K = p.K;
  const int JB = r >> 4;
  const int WJ = JB < kShrinkWaves ? JB : kShrinkWaves;
  const int WS = kShrinkWaves / WJ;
  const int wj = wave % WJ, ws = wave / WJ;
  const bool working = wave < kShrinkWaves;
  int rank_c;
  const int a_c = resolve_token(t0 + col, p.M, p.ad, p.ctrl + kCtrlError, report && lane < 16 && wave == 0, rank_c);

  f32x4 acc[kMaxJB];
#pragma unroll
  for (int j = 0; j < kMaxJB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint64_t active = __ballot(lane < 16 && a_c >= 0);
  uint64_t pending = working ? active : 0;
  while (pending) {
    const int leader = __ffsll((unsigned long long)pending) - 1;
    const int a = __shfl(a_c, leader);
    const int rank = __shfl(rank_c, leader);
    const uint64_t members = __ballot(lane < 16 && a_c == a);
    pending &= ~members;
    const bool member = (members >> col) & 1;
    const int jbn = (rank + 15) >> 4;
    const int64_t aoff = ((int64_t)a * (GEN ? p.ad.S : 1) + slice) * r * K;  // elements
    const uint16_t* Aa = p.ad.A + aoff;
    const uint8_t* Aa8 = p.ad.A8() + aoff;
    const uint16_t* xr = p.x + (t0 + col) * p.ldx;
    for (int s = s_begin + ws; s < s_end; s += WS) {
      const int64_t k = (int64_t)s * kShrinkStep + grp * 32;
      uint4 xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[i] = (member && k + i * 8 < K) ? xt(ld16(xr + k + i * 8), k + i * 8, col) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int jb = 0; jb < kMaxJB; ++jb) {
        if (jb < jbn && jb % WJ == wj) {
          const int j = jb * 16 + col;
          const bool rowok = j < rank;
          uint4 av[4];
          if (GEN && p.ad.afmt != 0) {  // FP8 codes: 32 bytes, widened to bf16 exactly
            const uint8_t* ar8 = Aa8 + (int64_t)j * K + k;
            const uint4 q0 = (rowok && k < K) ? ld16(ar8) : make_uint4(0, 0, 0, 0);
            const uint4 q1 = (rowok && k + 16 < K) ? ld16(ar8 + 16) : make_uint4(0, 0, 0, 0);
            av[0] = fp8x8_to_bf16x8(q0.x, q0.y);
            av[1] = fp8x8_to_bf16x8(q0.z, q0.w);
            av[2] = fp8x8_to_bf16x8(q1.x, q1.y);
            av[3] = fp8x8_to_bf16x8(q1.z, q1.w);
          } else {
            const uint16_t* ar = Aa + (int64_t)j * K + k;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              av[i] = (rowok && k + i * 8 < K) ? ld16(ar + i * 8) : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[jb] = mfma_bf16_16x16x32(as_bf16x8(av[i]), as_bf16x8(xv[i]), acc[jb]);
        }
      }
    }
  }

  // acc[jb][v] = z[token col][jb*16 + 4*grp + v]; sum the waves in order.
  if (working) {
#pragma unroll
    for (int jb = 0; jb < kMaxJB; ++jb)
      if (jb < JB)
        *reinterpret_cast<float4*>(&red[(wave * 16 + col) * r + jb * 16 + 4 * grp]) =
            make_float4(acc[jb][0], acc[jb][1], acc[jb][2], acc[jb][3]);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * r; e += NW * kWave) {
    float v = red[e];
#pragma unroll
    for (int w = 1; w < kShrinkWaves; ++w) v += red[w * 16 * r + e];
    red[e] = v;
  }
  __syncthreads();
  return active;
}

// The fixed-order sum of the split partials ([splits][M][r] fp32) of the
// tile of `rows` tokens at t0, taken by the tile's last split.  The
// quads (4 floats) of the tile times chunks of consecutive splits are spread
// over the threads; each chunk is summed in split order, then the chunk sums
// in chunk order (the chunking depends on the tile shape only, not on the
// block size).  With one split the partial passes through unchanged.
// `sums`: LDS of max(kShrinkWaves * kWave, rows * r / 4) float4s.
// sink(q, v) receives quad q of the tile.  Every thread of the block calls
// it; it ends with a barrier.
template <int NTHREADS, typename Sink>
__device__ __forceinline__ void combine_partials(const float* partials, int splits, int64_t M, int64_t t0,
                                                 int64_t rows, int r, float* sums, Sink sink) {
  const uint32_t tile_bytes = (uint32_t)(rows * r * 4);
  const int quads = (int)(rows * r / 4);
  auto part = [&](int s) { return make_rsrc(partials + ((int64_t)s * M + t0) * r, tile_bytes); };
  if (splits == 1) {
    for (int q = threadIdx.x; q < quads; q += NTHREADS) {
      const uint4 u = buf_load16<kCoherent>(part(0), 16u * q);
      sink(q, make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)));
    }
    __syncthreads();
    return;
  }
  const int threads = kShrinkWaves * kWave;  // the chunking, not the block size
  int chunks = threads / quads;
  if (chunks < 1) chunks = 1;
  if (chunks > splits) chunks = splits;
  const int per = (splits + chunks - 1) / chunks;
  for (int item = threadIdx.x; item < quads * chunks; item += NTHREADS) {
    const int q = item % quads, c = item / quads;
    const int s0 = c * per, s1 = min(splits, s0 + per);
    // Loads of up to 8 splits are in flight together; they are added in
    // split order all the same.
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    auto add = [&](uint4 u) {
      v.x += __uint_as_float(u.x);
      v.y += __uint_as_float(u.y);
      v.z += __uint_as_float(u.z);
      v.w += __uint_as_float(u.w);
    };
    int s = s0;
    for (; s + 8 <= s1; s += 8) {
      uint4 u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = buf_load16<kCoherent>(part(s + j), 16u * q);
#pragma unroll
      for (int j = 0; j < 8; ++j) add(u[j]);
    }
    for (; s < s1; ++s) add(buf_load16<kCoherent>(part(s), 16u * q));
    *reinterpret_cast<float4*>(&sums[4 * item]) = v;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < quads; q += NTHREADS) {
    float4 v = *reinterpret_cast<const float4*>(&sums[4 * q]);
    for (int c = 1; c < chunks; ++c) {
      const float4 w = *reinterpret_cast<const float4*>(&sums[4 * (c * quads + q)]);
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    sink(q, v);
  }
  __syncthreads();
}

// The split partials of one slice: [splits][M][r] fp32, one such block per
// slice.
__device__ __forceinline__ float* slice_partials(const ShrinkParams& p, int slice) {
  return p.partials + (int64_t)slice * p.splits * p.M * p.ad.r;
}

// Store this workgroup's [rows][r] sums (in LDS `red`) as its split's
// partial with device-coherent stores; returns once they have completed.
template <int NW, int TT = kShrinkTokens>
__device__ __forceinline__ void shrink_store_partial(const ShrinkParams& p, int tile, int slice, int split,
                                                     const float* red) {
  const int64_t t0 = (int64_t)tile * TT;
  const int r = p.ad.r;
  const int64_t rows = p.M - t0 < TT ? p.M - t0 : TT;
  const auto pr = make_rsrc(slice_partials(p, slice) + ((int64_t)split * p.M + t0) * r, (uint32_t)(rows * r * 4));
  for (int e = 4 * threadIdx.x; e < rows * r; e += 4 * NW * kWave)
    buf_store16<kCoherent>(pr, 4 * e, *reinterpret_cast<const uint4*>(&red[e]));
  wait_all_memory();
  __syncthreads();
}

// Write this workgroup's [TT][r] sums (in LDS `red`) to z, or to its split's
// partial; the last split of a tile adds the partials (combine_partials).  z
// and the partials are written and read device-coherently.  Returns true in
// the workgroup that wrote the tile's final z, after every one of its z
// stores has completed.
// `active`: the tile's active tokens (bit i: token t0 + i).  The separate
// shrink writes every row (zeros for inactive tokens).  The fused path
// (zflip != 0) stores only the rows of active tokens: those are exactly the
// words every consumer polls, so each z store of a call has been seen by
// every consumer before any of them counts itself done, and the clear of the
// region by the last one is ordered after all of them.  A store to a row no
// consumer polls could otherwise land after that clear and survive, as a
// stale nonzero word, into the next call on the same workspace.
// `slice`: the tile's z goes to columns slice * r .. + r of the [M][S r] z.
template <int NW, int TT = kShrinkTokens, bool GEN = true>
__device__ __forceinline__ bool shrink_finish(const ShrinkParams& p, int tile, int slice, int split, float* red,
                                              uint64_t active) {
  __shared__ int last;
  const int64_t t0 = (int64_t)tile * TT;
  const int r = p.ad.r, zld = GEN ? p.ad.zld : p.ad.r;
  const int64_t rows = p.M - t0 < TT ? p.M - t0 : TT;
  const auto zr = make_rsrc(p.z + t0 * zld + slice * r, (uint32_t)(((rows - 1) * zld + r) * 4));
  auto zoff = [&](int e) { return (uint32_t)(((e / r) * zld + e % r) * 4); };  // e: a word of the tile, row-major
  const uint32_t f = p.zflip;
  auto keep = [&](int e) { return f == 0u || ((active >> (e / r)) & 1ull) != 0; };
  // FP8 adapters: the sums are of the codes, z_j = sa[a][slice][j] * sum
  // (the row scale applied once, to the finished sum).
  auto scaled = [&](int e, float4 v) {
    if (!GEN || p.ad.afmt == 0) return v;
    int rk;
    const int a = resolve_token(t0 + e / r, p.M, p.ad, nullptr, false, rk);
    if (a < 0) return v;
    const float4 sc = *reinterpret_cast<const float4*>(p.ad.sa + ((int64_t)a * p.ad.S + slice) * r + e % r);
    return make_float4(v.x * sc.x, v.y * sc.y, v.z * sc.z, v.w * sc.w);
  };
  auto word = [&](const float4& v) {
    return make_uint4(__float_as_uint(v.x) ^ f, __float_as_uint(v.y) ^ f, __float_as_uint(v.z) ^ f,
                      __float_as_uint(v.w) ^ f);
  };
  if (p.splits == 1) {
    for (int e = 4 * threadIdx.x; e < rows * r; e += 4 * NW * kWave) {
      const float4 v = *reinterpret_cast<const float4*>(&red[e]);
      if (keep(e)) buf_store16<kCoherent>(zr, zoff(e), word(scaled(e, v)));
    }
    wait_all_memory();
    __syncthreads();
    return true;
  }
  shrink_store_partial<NW, TT>(p, tile, slice, split, red);
  int* counter = &p.counters[GEN ? tile * p.ad.S + slice : tile];
  if (threadIdx.x == 0) last = atomic_add_relaxed(counter, 1) == p.splits - 1;
  __syncthreads();
  if (!last) return false;
  // `red` is free again and holds the chunk sums.
  combine_partials<NW * kWave>(slice_partials(p, slice), p.splits, p.M, t0, rows, r, red, [&](int q, const float4& v) {
    if (keep(4 * q)) buf_store16<kCoherent>(zr, zoff(4 * q), word(scaled(4 * q, v)));
  });
  if (threadIdx.x == 0) store_relaxed(counter, 0);
  wait_all_memory();
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------------------
// Decode batches (M <= kShrinkWideM): one workgroup per unit (token t, output
// slice, block of RW consecutive rank rows) over the whole of K, so no sum
// crosses workgroups and z is stored as soon as the unit's loads are in.
// With few tokens, tiles of 16 tokens leave the matrix cores' columns mostly
// empty anyway (and a tile of distinct tenants would take its adapters one
// after another); a unit is a matrix-vector product on the vector ALUs.
// The first kShrinkWaves waves take the 8-element chunks tid, tid + 256, ...
// of K (further waves of a larger block idle, so the sums round the same way
// in every kernel that carries this code); each thread requests its chunks
// of x and of the RW rows of A at once, 8 / RW chunks of each per round
// (one round when RW * K <= 16384), and sums its chunks in K order, one fp32 FMA
// per element (bf16 products are exact in fp32); the 64 lanes of a wave
// meet in a fixed tree (DPP moves, then two swaps across rows) and the
// waves in wave order.  FP8 adapters: the codes are widened exactly and the
// row scale sa multiplies the finished sum.  z rows of inactive tokens are
// written as zeros by the separate shrink and not at all by the fused path
// (zflip != 0), which stores exactly the words its consumers poll.
// ---------------------------------------------------------------------------
// Rows per unit: as many as one round of loads covers (RW * K <= 16384),
// more when that would make over 256 units (each unit reads its token's
// activations again; with one row per unit that doubles the shrink's reads).
__host__ __device__ inline int shrink_unit_rows(int64_t M, int S, int r, int64_t K) {
  int rw = K <= 4096 ? 4 : (K <= 8192 ? 2 : 1);
  while (rw < 4 && M * S * (r / rw) > 256) rw *= 2;
  return rw;
}
__host__ __device__ inline int64_t shrink_units(int64_t M, int S, int r, int64_t K) {
  return M * S * (r / shrink_unit_rows(M, S, r, K));
}

// Sum over the 64 lanes of a wave, the same bits in every lane.
__device__ __forceinline__ float wave_tree_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // lane ^ 2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // half-row mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}

template <int RW, bool GEN, typename XT>
__device__ __forceinline__ void shrink_unit_rows_of(const ShrinkParams& p, int64_t t, int slice, int j0, float* red,
                                                    bool report, const XT& xt) {
  constexpr int CG = 8 / RW;                   // chunks of K per thread and round
  constexpr int NTS = kShrinkWaves * kWave;    // the threads that take chunks
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool working = tid < NTS;
  const int64_t K = p.K;
  const int nck = (int)(K >> 3);
  const int r = p.ad.r, S = GEN ? p.ad.S : 1, zld = GEN ? p.ad.zld : r;
  const bool a8 = GEN && p.ad.afmt != 0;
  const uint16_t* xr = p.x + t * p.ldx;
  // The token's slot and mask byte and the first round of activations are
  // requested together (none depends on another); the adapter's rows and
  // its rank then go out together too.  Rows past the rank are read (they
  // lie inside the slot) and dropped at the end, so no load waits for the
  // rank: two round trips to memory before the sums instead of four.
  const int a_raw = p.ad.idx[t];
  const int mk = p.ad.mask != nullptr ? (int)p.ad.mask[t] : 1;
  uint4 xv[CG];
#pragma unroll
  for (int i = 0; i < CG; ++i) {
    const int kc = tid + i * NTS;
    xv[i] = (working && kc < nck) ? ld16(xr + 8 * (int64_t)kc) : make_uint4(0, 0, 0, 0);
  }
  if (a_raw < -1 || a_raw >= p.ad.L) {
    if (report && p.ctrl != nullptr) atomic_or_relaxed(p.ctrl + kCtrlError, EPILORA_DEV_BAD_INDEX);
  }
  const int a = (a_raw >= 0 && a_raw < p.ad.L && mk != 0) ? a_raw : -1;  // uniform over the block
  int rank = 0;
  if (a >= 0) {
    rank = p.ad.ranks != nullptr ? p.ad.ranks[a] : r;
    rank = rank < r ? rank : r;
  }
  float acc[RW];
#pragma unroll
  for (int q = 0; q < RW; ++q) acc[q] = 0.f;
  if (a >= 0) {
    const int64_t arow = (((int64_t)a * S + slice) * r + j0) * K;  // elements
    for (int c0 = tid; c0 < nck; c0 += NTS * CG) {
      if (c0 != tid) {
#pragma unroll
        for (int i = 0; i < CG; ++i) {
          const int kc = c0 + i * NTS;
          xv[i] = (working && kc < nck) ? ld16(xr + 8 * (int64_t)kc) : make_uint4(0, 0, 0, 0);
        }
      }
      uint4 av[RW][CG];
#pragma unroll
      for (int q = 0; q < RW; ++q)
#pragma unroll
        for (int i = 0; i < CG; ++i) {
          const int kc = c0 + i * NTS;
          const bool ok = working && kc < nck;
          if (a8) {
            const uint2 w = ok ? *reinterpret_cast<const uint2*>(p.ad.A8() + arow + q * K + 8 * (int64_t)kc)
                               : make_uint2(0, 0);
            av[q][i] = make_uint4(w.x, w.y, 0, 0);
          } else {
            av[q][i] = ok ? ld16(p.ad.A + arow + q * K + 8 * (int64_t)kc) : make_uint4(0, 0, 0, 0);
          }
        }
#pragma unroll
      for (int i = 0; i < CG; ++i) {
        const int kc = c0 + i * NTS;
        const uint4 x8 = (working && kc < nck) ? xt(xv[i], 8 * (int64_t)kc, 0) : xv[i];
        const uint32_t xw[4] = {x8.x, x8.y, x8.z, x8.w};
#pragma unroll
        for (int q = 0; q < RW; ++q) {
          const uint4 v = a8 ? fp8x8_to_bf16x8(av[q][i].x, av[q][i].y) : av[q][i];
          const uint32_t aw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float xe = (e & 1) ? bf16_hi(xw[e >> 1]) : bf16_lo(xw[e >> 1]);
            const float ae = (e & 1) ? bf16_hi(aw[e >> 1]) : bf16_lo(aw[e >> 1]);
            acc[q] = fmaf(ae, xe, acc[q]);
          }
        }
      }
    }
  }
  const bool active = a >= 0 && rank > 0;
#pragma unroll
  for (int q = 0; q < RW; ++q) {
    const float v = wave_tree_sum(acc[q]);
    if (lane == 0 && wave < kShrinkWaves) red[wave * RW + q] = v;
  }
  __syncthreads();
  if (tid == 0 && (active || p.zflip == 0u)) {
    float zv[RW];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
      float v = red[q];
#pragma unroll
      for (int w = 1; w < kShrinkWaves; ++w) v += red[w * RW + q];
      if (!active || j0 + q >= rank) v = 0.f;
      else if (a8) v *= p.ad.sa[((int64_t)a * S + slice) * r + j0 + q];
      zv[q] = v;
    }
    const uint32_t f = p.zflip;
    const auto zr = make_rsrc(p.z + t * zld + slice * r + j0, (uint32_t)(RW * 4));
    if constexpr (RW == 4)
      buf_store16<kCoherent>(zr, 0u, make_uint4(__float_as_uint(zv[0]) ^ f, __float_as_uint(zv[1]) ^ f,
                                                __float_as_uint(zv[2]) ^ f, __float_as_uint(zv[3]) ^ f));
    else if constexpr (RW == 2)
      buf_store8<kCoherent>(zr, 0u, make_uint2(__float_as_uint(zv[0]) ^ f, __float_as_uint(zv[1]) ^ f));
    else
      buf_store4<kCoherent>(zr, 0u, __float_as_uint(zv[0]) ^ f);
  }
}

// Unit `unit` of a decode batch's shrink (units in token, slice, row-block
// order).  `red`: LDS of kShrinkWaves * 4 floats.  Every thread of the block
// calls it; it ends with no pending barrier.  A token is active as in
// resolve_token (slot in [0, L), mask byte nonzero, rank > 0); an index
// outside [-1, L) is reported once per token.
template <bool GEN, typename XT = XIdentity>
__device__ __forceinline__ void shrink_unit(const ShrinkParams& p, int unit, float* red, const XT& xt = XT()) {
  const int r = p.ad.r, S = GEN ? p.ad.S : 1;
  const int RW = shrink_unit_rows(p.M, S, r, p.K), nrb = r / RW;
  const int rb = unit % nrb, rest = unit / nrb;
  const int slice = rest % S;
  const int64_t t = rest / S;
  const bool report = threadIdx.x == 0 && slice == 0 && rb == 0;
  if (RW == 4) shrink_unit_rows_of<4, GEN>(p, t, slice, rb * 4, red, report, xt);
  else if (RW == 2) shrink_unit_rows_of<2, GEN>(p, t, slice, rb * 2, red, report, xt);
  else shrink_unit_rows_of<1, GEN>(p, t, slice, rb, red, report, xt);
}

// K-step range of split `split`.
__device__ __forceinline__ void shrink_range(const ShrinkParams& p, int split, int& s_begin, int& s_end) {
  const int steps = (int)cdiv(p.K, kShrinkStep);
  const int spw = (int)cdiv(steps, p.splits);
  s_begin = min(steps, split * spw);
  s_end = min(steps, s_begin + spw);
}

}  // namespace epilora
