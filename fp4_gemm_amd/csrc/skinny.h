// The weight-streaming GEMM for small batches (M <= 64 tokens), shared by
// the skinny GEMM kernel and the fused decode kernel.
//
// Persistent workgroups: workgroup g of G owns the 16-row tiles g, g + G,
// g + 2G, ... of the output and streams them back to back.  Its NW waves
// split the 128-wide K steps of every tile into NW contiguous ranges.  The
// product is taken swap-AB: the weight rows are the 16-row operand of
// v_mfma_f32_16x16x128_f8f6f4 and the tokens (up to MB blocks of 16) its
// 16-column operand, so C[n][t] sits in lane (t % 16) + 16 * ((n % 16) / 4),
// register n % 4.  Lane l takes 32 consecutive bytes of weight row l % 16 and
// of token row l % 16 at the same K offset 32 * (l / 16): both operands see
// the same K positions, so each MFMA pairs matching elements.
//
// Weights stream in batches of U steps through buffer resources
// (out-of-range offsets read as zero) with two batches in flight, across tile
// boundaries: the next tile's first batch is on its way while the current
// tile's epilogue runs.  FP8 weights are requested in whole 128-byte lines:
// for each 128-byte K step, lane l loads 16 bytes of rows l / 8 and
// 8 + l / 8 at chunk l % 8, so one load instruction covers eight full lines
// (a wave spreading an instruction over sixteen half lines streams about a
// quarter slower).  The wave then puts the step through its own 2 KB of LDS
// (chunk c of row n at position c ^ (n % 8), no bank conflicts on either
// side) and reads it back in the matrix-core layout above.  Small quantized activations (M * K <= 32 KB) sit in
// LDS for the whole kernel; larger ones are loaded with the weights.
//
// A tile's epilogue sums the NW partial accumulators in wave order through
// LDS, applies the scales, and adds the adapter term of each active token:
// an fp32 dot over the rank, each output taken by 2^sh lanes that hold CPL
// 8-rank chunks each, summed over the chunks in one fixed tree (by chunk
// index: DPP moves across the lanes' bits first, then the lane's own chunks),
// so that every layout of lanes rounds the same way.  With two or more token
// blocks and the activations not in LDS the loop runs batch-major instead
// (run_batches): each wave loads its activations of a K batch once and runs
// them against every tile of the workgroup.  In the fused decode kernel z is
// produced by other workgroups of the same grid, so the streaming loop only
// reduces each finished tile into an LDS stash (StashCfg<MB>::n tiles; the
// host never gives a workgroup more); once the last tile is in, the
// workgroup polls z into LDS, counts itself done and runs the epilogues of
// all its tiles as one list (their first B chunks requested before the
// stream at one token block).  Keeping the wait, the hand-off and the
// epilogues out of the loop keeps the loop's code small: a loop that also
// carried them streamed measurably slower even when they never ran.
#pragma once

#include "gemm_common.h"
#include "occupancy.h"
#include "quant_row.h"

namespace epilora {

constexpr int kXInLdsMax = 32768;  // bytes of quantized activations kept in LDS
constexpr int kSelfQuantMaxM = 4;  // the fused kernel quantizes up to this many rows itself
constexpr uint32_t kLdsBudget = 65536;
// The fused kernel takes quantized rows that are not kept in LDS from
// quantizing workgroups of its own grid for up to 32 tokens, and from a
// quantizer launch just before it for more: with 64 quantizing workgroups
// ahead of the GEMM and every GEMM workgroup waiting for all of them, the
// 72B-shaped layer at 64 tokens took 387 us against 380 with the launch.
constexpr int kQuantBeforeMB = 3;

// Tiles of one fused workgroup, held in LDS until z is published.
template <int MB>
struct StashCfg {
  static constexpr int n = MB == 1 ? 8 : 4;
};
inline int stash_tiles(int MB) { return MB == 1 ? 8 : 4; }

template <int MB>
struct SkinnyCfg {
  static constexpr int U = MB == 1 ? 4 : (MB == 2 ? 2 : 1);  // steps per load batch
  static constexpr int T = MB * 16;                            // token slots
};

__host__ __device__ inline uint32_t align16(uint32_t v) { return (v + 15u) & ~15u; }

// LDS layout of a skinny workgroup (byte offsets); host and device agree.
struct SkLayout {
  uint32_t part, red, tbl, tok, sx, zs, xs, stash, wst, total;
};

constexpr uint32_t kWaveStage = 2048;  // LDS per wave for one FP8 weight step (16 rows x 128 bytes)

// zplanes: z of that many output slices side by side ([zplanes][T][r]).
__host__ __device__ inline SkLayout sk_layout(int MB, int NW, int r, uint32_t xbytes, int nstash, int fmt,
                                              int zplanes = 1) {
  const uint32_t T = MB * 16;
  SkLayout L;
  L.part = 0;                                            // float [NW][T][16]
  L.red = align16(L.part + NW * T * 16 * 4);             // float [T][16]
  L.tbl = align16(L.red + T * 16 * 4);                   // uint2 [256]
  L.tok = align16(L.tbl + 256 * 8);                      // TokenSlot [T]
  L.sx = align16(L.tok + T * 8);                         // float [T]
  L.zs = align16(L.sx + T * 4);                          // float [T][r]
  L.xs = align16(L.zs + T * r * 4 * (zplanes > 1 ? zplanes : 1));  // uint8 [M][K]
  L.stash = align16(L.xs + xbytes);                      // float [nstash][T][16]
  L.wst = align16(L.stash + nstash * T * 16 * 4);        // uint8 [NW][kWaveStage] (FP8 weights)
  L.total = align16(L.wst + (fmt == EPILORA_W_FP8 ? NW * kWaveStage : 0u) + 16);  // + one flag word
  return L;
}

// What a persistent skinny grid does.
struct SkinnyJob {
  GemmParams g;
  int tiles;            // cdiv(N, 16)
  int gwgs;             // persistent workgroups G (<= tiles)
  const uint16_t* x;    // fused: the bf16 activations (self-quantized when kept in LDS)
  int64_t ldx;
  int* qflag;           // fused, activations not in LDS: rows quantized
  int qtarget;
  int64_t wait_ticks;
  int zplanes;          // fused: output slices whose z fit in LDS at once (sk_layout)
  int* done;            // fused with flags: the done sub-counters (kDoneGroups, kDoneStride words apart)
  int flags;            // fused: a flag is counted or z handed over (the workgroups count themselves done)
};

// XV 16-byte vectors of activations per lane and step: 2 (32 FP8 codes) or
// 4 (32 bf16 values, the W8A16 GEMM).
template <int MB, int U, int XV>
struct SkinnyBatch {
  u32x4 wa[U], wb[U];        // FP8: 32 bytes; 4-bit: wa = 32 codes, wb.x = two block scales
  u32x4 xv[U][MB][XV];
};

// Thread 0 polls *flag (device-coherent loads, s_sleep between them) until it
// reaches target, the wall-clock limit passes, or another workgroup has
// already timed out; the verdict is broadcast through LDS.  A nonzero
// `force` word (set from the host to test the timeout path) ends the wait at
// once as expired.
__device__ __forceinline__ bool wait_flag(int* flag, int target, int64_t ticks, int* err, int* force, int* verdict) {
  if (threadIdx.x == 0) {
    int ok = 1;
    const int forced = load_relaxed(force);
    if (forced != 0) {
      ok = 0;
    } else if (load_relaxed(flag) < target) {
      const int64_t start = wall_clock64();
      while (load_relaxed(flag) < target) {
        if (wall_clock64() - start > ticks || (load_relaxed(err) & EPILORA_DEV_WAIT_TIMEOUT)) {
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
    }
    *verdict = ok;
  }
  __syncthreads();
  return *verdict != 0;
}

// The fused kernel quantizes the M <= kSelfQuantMaxM bf16 rows of x into
// LDS (codes [M][K], scales [M]) with quant_row's arithmetic, so the same
// bits, in two phases: the loads are requested before the first weight
// batches (vector loads return in order, so a load issued after the weights
// would wait for them) and the rest runs once they are in.  The M rows are
// one run of 16-byte vectors; each thread keeps up to RV of its vectors in
// registers between the phases (a longer run is read again in the second
// phase).  The row maxima meet in one LDS round; `red` is
// kSelfQuantMaxM * NT / 64 words of LDS.
template <int NT, int RV>
struct SelfQuant {
  uint4 v[RV];

  __device__ __forceinline__ void issue(const uint16_t* __restrict__ x, int64_t ldx, int M, int64_t K) {
    const int nv = (int)(K / 8);
#pragma unroll
    for (int i = 0; i < RV; ++i) {
      const int j = threadIdx.x + i * NT;
      if (j < M * nv) {
        const int t = j / nv;
        v[i] = *reinterpret_cast<const uint4*>(x + t * ldx + 8 * (j - t * nv));
      }
    }
  }

  // Ends with a barrier.
  __device__ __forceinline__ void finish(const uint16_t* __restrict__ x, int64_t ldx, int M, int64_t K, uint8_t* qs,
                                         float* sxs, uint32_t* red) const {
    constexpr int W = NT / kWave;
    const int nv = (int)(K / 8);
    const int total = M * nv;
    const int tid = threadIdx.x;
    uint32_t m[kSelfQuantMaxM];
#pragma unroll
    for (int u = 0; u < kSelfQuantMaxM; ++u) m[u] = 0;
#pragma unroll
    for (int i = 0; i < RV; ++i) {
      const int j = tid + i * NT;
      if (j < total) {
        const int t = j / nv;
        const uint32_t a = absmax8(v[i]);
#pragma unroll
        for (int u = 0; u < kSelfQuantMaxM; ++u)
          if (u == t) m[u] = max(m[u], a);
      }
    }
    for (int j = tid + RV * NT; j < total; j += NT) {
      const int t = j / nv;
      const uint32_t a = absmax8(*reinterpret_cast<const uint4*>(x + t * ldx + 8 * (j - t * nv)));
#pragma unroll
      for (int u = 0; u < kSelfQuantMaxM; ++u)
        if (u == t) m[u] = max(m[u], a);
    }
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int u = 0; u < kSelfQuantMaxM; ++u) {
      if (u < M) {
        const uint32_t w = wave_max_u32(m[u]);
        if (lane == 0) red[u * W + wave] = w;
      }
    }
    __syncthreads();
    float sc[kSelfQuantMaxM];
    QuotRow qc[kSelfQuantMaxM];
#pragma unroll
    for (int u = 0; u < kSelfQuantMaxM; ++u) {
      uint32_t a = 0;
      if (u < M) {
#pragma unroll
        for (int w = 0; w < W; ++w) a = max(a, red[u * W + w]);
      }
      sc[u] = row_scale(a);
      qc[u] = quot_consts(sc[u]);
      if (tid == 0 && u < M) sxs[u] = sc[u];
    }
#pragma unroll
    for (int i = 0; i < RV; ++i) {
      const int j = tid + i * NT;
      if (j < total) {
        const int t = j / nv;
        QuotRow q = qc[0];
#pragma unroll
        for (int u = 1; u < kSelfQuantMaxM; ++u)
          if (u == t) q = qc[u];
        *reinterpret_cast<uint2*>(qs + 8 * j) = encode8(v[i], q);
      }
    }
    for (int j = tid + RV * NT; j < total; j += NT) {
      const int t = j / nv;
      QuotRow q = qc[0];
#pragma unroll
      for (int u = 1; u < kSelfQuantMaxM; ++u)
        if (u == t) q = qc[u];
      *reinterpret_cast<uint2*>(qs + 8 * j) = encode8(*reinterpret_cast<const uint4*>(x + t * ldx + 8 * (j - t * nv)), q);
    }
    __syncthreads();
  }
};

// The W8A16 GEMM's fused kernel keeps the few bf16 rows of x in LDS as they
// are (no quantization): the loads are requested before the weights, as in
// SelfQuant, and stored once they are in.  Row scales read 1.
template <int NT, int RV>
struct SelfCopy {
  uint4 v[RV];

  __device__ __forceinline__ void issue(const uint16_t* __restrict__ x, int64_t ldx, int M, int64_t K) {
    const int nv = (int)(K / 8);
#pragma unroll
    for (int i = 0; i < RV; ++i) {
      const int j = threadIdx.x + i * NT;
      if (j < M * nv) {
        const int t = j / nv;
        v[i] = *reinterpret_cast<const uint4*>(x + t * ldx + 8 * (j - t * nv));
      }
    }
  }

  // Ends with a barrier.
  __device__ __forceinline__ void finish(const uint16_t* __restrict__ x, int64_t ldx, int M, int64_t K, uint8_t* xs,
                                         float* sxs) const {
    const int nv = (int)(K / 8);
    const int total = M * nv;
#pragma unroll
    for (int i = 0; i < RV; ++i) {
      const int j = threadIdx.x + i * NT;
      if (j < total) *reinterpret_cast<uint4*>(xs + 16 * j) = v[i];
    }
    for (int j = threadIdx.x + RV * NT; j < total; j += NT) {
      const int t = j / nv;
      *reinterpret_cast<uint4*>(xs + 16 * j) = *reinterpret_cast<const uint4*>(x + t * ldx + 8 * (j - t * nv));
    }
    for (int t = threadIdx.x; t < M; t += NT) sxs[t] = 1.0f;
    __syncthreads();
  }
};

// UB (> 0) overrides the steps per load batch.  GEN: the general adapters
// (several output slices, FP8 storage) may occur; without it the epilogue
// assumes one slice of bf16 adapters and carries none of that code, which
// keeps the registers of the weight stream free.  A16: the matched W8A16
// GEMM ("EpiLoRA ...", Design, "LoRA RL on the same base"): the activations
// stay bf16 (p.x16), each FP8 weight is widened to bf16 exactly in
// registers, the products run on bf16 matrix cores (four 16x16x32 steps per
// 128-wide K step, lane l taking the same 8 K positions of its 32 in both
// operands) and the accumulators take no activation scale (it reads 1).
template <int MB, int FMT, int NW, bool XLDS, bool FUSED, int UB = 0, bool GEN = true, bool A16 = false>
struct Skinny {
  // The fused kernel's 8-wave workgroups take half batches so that two fit
  // on a compute unit (four waves per SIMD), beside a producer workgroup.
  // (The W8A16 GEMM's activations take twice the registers: half batches.)
  static constexpr int U0 = UB > 0 ? UB : ((FUSED && NW == 8 && MB == 1) ? 2 : SkinnyCfg<MB>::U);
  static constexpr int U = (A16 && U0 > 1) ? U0 / 2 : U0;
  static constexpr int T = MB * 16;
  // Rows quantized inside this grid, announced by the quantized-rows flag.
  // They are read through the caches all the same: a launch starts with no
  // stale L2 lines for memory written before it, no workgroup touches the
  // rows before the flag, and their producers write them through to the
  // point of coherence before they count the flag up, so a workgroup's first
  // read of a line misses to the rows of this call, and every later read of
  // it on that XCD hits.  (Reading them device-coherently sent every weight
  // batch's activations past the L2: the 72B-shaped layer at 8 tokens took
  // 229 us instead of 214.)  Only the tiny scale vector is read coherently.
  static constexpr bool kRowsInGrid = FUSED && !XLDS && !A16 && MB < kQuantBeforeMB;
  static constexpr int XPOL = kCached;
  static constexpr int XB = A16 ? 2 : 1;   // bytes per activation element
  static constexpr int XV = A16 ? 4 : 2;   // 16-byte activation vectors per lane and step
  static_assert(!A16 || FMT == EPILORA_W_FP8, "W8A16 takes FP8 weights");

  const SkinnyJob& J;
  const GemmParams& p;
  SkLayout L;
  float *part, *red, *sxs, *zs, *stash;
  uint2* tbl;
  TokenSlot* tok;
  uint8_t* xs;
  uint8_t* wst;  // this wave's FP8 weight step
  int* verdict;
  int g, lane, wave, row;
  int sb, se, nb, total;
  uint32_t kofs, xbase[MB];
  __amdgpu_buffer_rsrc_t xr;
  bool adapters;
  int zslice;    // unfused: the slice whose z is staged in LDS
  float gscale;  // 4-bit weights: gs * 8
  int done_old;  // fused, thread 0: what the done sub-counter returned (-1: not counted yet)
  // Fused one-block grids with one adapter slice: the outputs of all the
  // workgroup's tiles form one list (outputs_flat); the B chunks and weight
  // scales of this thread's first kFlatPre outputs are requested before the
  // stream and held through it.  With several output slices the z of every
  // slice the tiles span sits in LDS at once (J.zplanes planes), when it fits.
  static constexpr bool kFlat = FUSED && MB == 1;  // (with the general adapters: one slice only)
  __device__ __forceinline__ bool flat() const { return kFlat && (!GEN || p.ad.S <= 1 || J.zplanes >= p.ad.S); }
  static constexpr int kFlatPre = 2;
  uint4 fpre_b[kFlatPre];
  float fpre_ws[kFlatPre];

  __device__ __forceinline__ Skinny(const SkinnyJob& j, char* lds, int gidx) : J(j), p(j.g), g(gidx) {
    const int64_t M = p.M, K = p.K;
    L = sk_layout(MB, NW, p.ad.r, XLDS ? (uint32_t)(M * K * XB) : 0u,
                  (FUSED || (MB >= 2 && !XLDS && !A16)) ? StashCfg<MB>::n : 0, FMT, FUSED ? J.zplanes : 1);
    part = reinterpret_cast<float*>(lds + L.part);
    red = reinterpret_cast<float*>(lds + L.red);
    tbl = reinterpret_cast<uint2*>(lds + L.tbl);
    tok = reinterpret_cast<TokenSlot*>(lds + L.tok);
    sxs = reinterpret_cast<float*>(lds + L.sx);
    zs = reinterpret_cast<float*>(lds + L.zs);
    xs = reinterpret_cast<uint8_t*>(lds + L.xs);
    wst = reinterpret_cast<uint8_t*>(lds + L.wst) + (threadIdx.x >> 6) * kWaveStage;
    stash = reinterpret_cast<float*>(lds + L.stash);
    verdict = reinterpret_cast<int*>(lds + L.total - 16);
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    row = lane & 15;
    kofs = (uint32_t)(lane >> 4) * 32;
    const int steps = (int)cdiv(K, 128);
    const int spw = (int)cdiv(steps, NW);
    sb = min(steps, wave * spw);
    se = min(steps, sb + spw);
    nb = (int)cdiv(spw, U);
    int mine = (int)cdiv(J.tiles - g, J.gwgs);
    if (FUSED && mine > StashCfg<MB>::n) {  // the host never launches so (the stash holds n tiles)
      mine = 0;
      if (threadIdx.x == 0 && p.ctrl != nullptr) atomic_or_relaxed(p.ctrl + kCtrlError, EPILORA_DEV_INTERNAL);
    }
    total = mine * nb;
    done_old = -1;
    adapters = p.z != nullptr;
    gscale = FMT == EPILORA_W_FP4 ? weight_scale<FMT>(p.wt, 0) : 0.f;
    xr = A16 ? make_rsrc(p.x16, (uint32_t)(((M - 1) * p.ldx16 + K) * 2)) : make_rsrc(p.xq, (uint32_t)((M - 1) * p.ldq + K));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {  // byte offsets of the token rows (in LDS or in memory)
      const int64_t t = mb * 16 + row;
      xbase[mb] = t < M ? (uint32_t)(t * (XLDS ? K : (A16 ? p.ldx16 : p.ldq)) * XB) : kOutOfRange;
    }
  }

  __device__ __forceinline__ int64_t n0_of(int j) const { return (int64_t)(g + (j / nb) * J.gwgs) * 16; }
  __device__ __forceinline__ bool af8() const { return GEN && p.ad.afmt != 0; }
  __device__ __forceinline__ int zld() const { return GEN ? p.ad.zld : p.ad.r; }
  __device__ __forceinline__ int slice(int64_t n) const { return GEN ? slice_of(p.ad, n) : 0; }

  // ---- loads ----------------------------------------------------------------
  // Weights of step batch `batch` (U steps) of tile `tile` (the workgroup's
  // tile index: rows (g + tile * G) * 16 ...) into wa / wb.
  __device__ __forceinline__ void load_w_at(u32x4 (&wa)[U], u32x4 (&wb)[U], int tile, int batch, bool live) const {
    const int64_t K = p.K;
    const int64_t n0 = live ? (int64_t)(g + tile * J.gwgs) * 16 : 0;
    const int64_t rows = live ? (p.N - n0 < 16 ? p.N - n0 : 16) : 0;
    const int64_t wrow = FMT == EPILORA_W_FP8 ? K : K / 2;
    const auto wr = make_rsrc(p.wt.w + n0 * wrow, (uint32_t)(rows * wrow));
    const auto sr = make_rsrc(FMT == EPILORA_W_FP4 ? p.wt.bs + n0 * (K / 16) : p.wt.w,
                              FMT == EPILORA_W_FP4 ? (uint32_t)(rows * (K / 16)) : 0u);
    const uint32_t wbase = row < rows ? (uint32_t)(row * wrow) : kOutOfRange;
    const uint32_t sbase = row < rows ? (uint32_t)(row * (K / 16)) : kOutOfRange;
    // FP8: rows l / 8 and 8 + l / 8, chunk l % 8 of each step
    const int r0 = lane >> 3;
    const uint32_t c16 = (uint32_t)(lane & 7) * 16u;
    const uint32_t wbase0 = r0 < rows ? (uint32_t)(r0 * wrow) + c16 : kOutOfRange;
    const uint32_t wbase1 = r0 + 8 < rows ? (uint32_t)((r0 + 8) * wrow) + c16 : kOutOfRange;
    const int s0 = sb + (live ? batch : 0) * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (FMT == EPILORA_W_FP8) {
        const uint32_t k = (uint32_t)(s0 + u) * 128u;
        const bool ok = s0 + u < se && (int64_t)(k + c16) < K;
        wa[u] = bufv_load16<kCached>(wr, ok ? wbase0 + k : kOutOfRange);
        wb[u] = bufv_load16<kCached>(wr, ok ? wbase1 + k : kOutOfRange);
      } else {
        const uint32_t k = (uint32_t)(s0 + u) * 128u + kofs;
        const bool ok = s0 + u < se && (int64_t)k < K;
        wa[u] = bufv_load16<kCached>(wr, ok ? wbase + k / 2 : kOutOfRange);
        wb[u] = u32x4{buf_load2<kCached>(sr, ok ? sbase + k / 16 : kOutOfRange), 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void load_w(SkinnyBatch<MB, U, XV>& b, int j) const {
    load_w_at(b.wa, b.wb, j < total ? j / nb : 0, j < total ? j % nb : 0, j < total);
  }

  // Activations of step batch `batch` into xv (unless they sit in LDS).
  __device__ __forceinline__ void load_x_at(u32x4 (&xv)[U][MB][XV], int batch, bool live) const {
    if (XLDS) return;
    const int s0 = sb + (live ? batch : 0) * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t k = (uint32_t)(s0 + u) * 128u + kofs;
      const bool ok = live && s0 + u < se && (int64_t)k < p.K;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint32_t off = ok ? xbase[mb] + k * XB : kOutOfRange;
#pragma unroll
        for (int v = 0; v < XV; ++v) xv[u][mb][v] = bufv_load16<XPOL>(xr, off + 16 * v);
      }
    }
  }
  __device__ __forceinline__ void load_x(SkinnyBatch<MB, U, XV>& b, int j) const {
    load_x_at(b.xv, j < total ? j % nb : 0, j < total);
  }

  // ---- multiply a batch (steps past the range were loaded as zeros) ---------
  __device__ __forceinline__ void compute_at(const u32x4 (&wa)[U], const u32x4 (&wb)[U],
                                             const u32x4 (&xv)[U][MB][XV], int batch, bool live,
                                             f32x4 (&acc)[MB]) const {
    const int s0 = sb + (live ? batch : 0) * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      i32x8 wf;
      if (FMT == EPILORA_W_FP8) {
        const int r0 = lane >> 3;
        const uint32_t pw = (uint32_t)((lane & 7) ^ (r0 & 7)) * 16u;
        *reinterpret_cast<u32x4*>(wst + r0 * 128 + pw) = wa[u];
        *reinterpret_cast<u32x4*>(wst + (r0 + 8) * 128 + pw) = wb[u];
        const uint32_t p0 = (uint32_t)((2 * (lane >> 4)) ^ (row & 7)) * 16u;
        const u32x4 q0 = *reinterpret_cast<const u32x4*>(wst + row * 128 + p0);
        const u32x4 q1 = *reinterpret_cast<const u32x4*>(wst + row * 128 + (p0 ^ 16u));
        wf = cat8(q0, q1);
      } else {
        const uint32_t sc = wb[u].x;
        const uint2 t0 = tbl[sc & 0xFFu], t1 = tbl[(sc >> 8) & 0xFFu];
        uint32_t o[8];
        fold8(wa[u].x, t0.x, t0.y, o[0], o[1]);
        fold8(wa[u].y, t0.x, t0.y, o[2], o[3]);
        fold8(wa[u].z, t1.x, t1.y, o[4], o[5]);
        fold8(wa[u].w, t1.x, t1.y, o[6], o[7]);
        wf = i32x8{(int)o[0], (int)o[1], (int)o[2], (int)o[3], (int)o[4], (int)o[5], (int)o[6], (int)o[7]};
      }
      const uint32_t k = (uint32_t)(s0 + u) * 128u + kofs;
      const bool kin = s0 + u < se && (int64_t)k < p.K;
      // W8A16: the lane's 32 FP8 weights as four groups of 8 bf16; group q
      // meets the lane's activations at the same 8 K positions.
      uint4 w16[4];
      if (A16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) w16[q] = fp8x8_to_bf16x8((uint32_t)wf[2 * q], (uint32_t)wf[2 * q + 1]);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        u32x4 xq4[XV];
        if (XLDS) {
          const bool ok = kin && xbase[mb] != kOutOfRange;
          const u32x4* q = reinterpret_cast<const u32x4*>(xs + (ok ? xbase[mb] + k * XB : 0u));
          const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int v = 0; v < XV; ++v) {
            const u32x4 qv = q[v];
            xq4[v] = ok ? qv : zero;
          }
        } else {
#pragma unroll
          for (int v = 0; v < XV; ++v) xq4[v] = xv[u][mb][v];
        }
        if (A16) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[mb] = mfma_bf16_16x16x32(as_bf16x8(w16[q]), __builtin_bit_cast(bf16x8, xq4[q]), acc[mb]);
        } else {
          acc[mb] = mfma_fp8_16x16x128(wf, cat8(xq4[0], xq4[1]), acc[mb]);
        }
      }
    }
  }
  __device__ __forceinline__ void compute(const SkinnyBatch<MB, U, XV>& b, int j, f32x4 (&acc)[MB]) const {
    compute_at(b.wa, b.wb, b.xv, j < total ? j % nb : 0, j < total, acc);
  }

  // ---- epilogue pieces --------------------------------------------------------
  // Token t's index and mask byte, loaded by thread t before the weights are
  // requested (a later load would return only after them), and resolved into
  // tok[] afterwards, as resolve_token does it.
  // The loads are unconditional and bounds-checked (past M, without adapters
  // or without a mask they read zero) and nothing tests their values before
  // resolve_tokens: a load under a branch let the compiler test the mask byte
  // at once, which held the weight requests behind it.
  struct TokenLoad {
    int a, m;
  };
  __device__ __forceinline__ TokenLoad load_token() const {
    TokenLoad tl;
    const uint32_t t = threadIdx.x < T ? threadIdx.x : 0u;
    const auto ir = make_rsrc(p.ad.idx, adapters ? (uint32_t)(p.M * 4) : 0u);
    const auto mr = make_rsrc(p.ad.mask, (adapters && p.ad.mask != nullptr) ? (uint32_t)p.M : 0u);
    tl.a = (int)buf_load4<kCached>(ir, 4u * t);
    tl.m = (int)__builtin_amdgcn_raw_buffer_load_b8(mr, t, 0, 0);
    return tl;
  }
  __device__ __forceinline__ void resolve_tokens(const TokenLoad& tl, bool report) const {
    const int t = threadIdx.x;
    if (t >= T) return;
    int a = -1, rk = 0;
    if (adapters && t < p.M) {
      a = tl.a;
      if (a < -1 || a >= p.ad.L) {
        if (report) atomic_or_relaxed(p.ctrl + kCtrlError, EPILORA_DEV_BAD_INDEX);
        a = -1;
      }
      if (a >= 0 && p.ad.mask != nullptr && tl.m == 0) a = -1;
      if (a >= 0) {
        rk = p.ad.ranks != nullptr ? p.ad.ranks[a] : p.ad.r;
        rk = rk < p.ad.r ? rk : p.ad.r;
        if (rk <= 0) a = -1, rk = 0;
      }
    }
    tok[t] = TokenSlot{a, rk};
  }

  // ---- the adapter epilogue ---------------------------------------------------
  // Each output (t, n) of a tile is a dot of B[a_t][n][0 .. rank) with z[t]
  // taken by a group of 2^sh lanes: lane jl of the group takes the 8-element
  // chunks jl, jl + 2^sh, ... of the row, at most CPL of them, and the
  // partial dots meet through DPP moves.  A few lanes per output keep the
  // arithmetic per output small at low rank (rank 16: one lane, two chunks);
  // CPL = 1 spreads a row over up to 16 lanes, for the tile-major loop, where
  // the weight registers are live and a tile has at most 256 outputs.
  // Without adapters a thread writes whole outputs (sh = 0).  Output o of
  // the tile is taken by lanes o * 2^sh ... modulo the block size, whose
  // quotient is a multiple of 16, so a thread meets a single row
  // n0 + (tid >> sh) % 16.
  template <int CPL>
  __device__ __forceinline__ int lane_shift() const {
    if (!adapters) return 0;
    const int need = ((p.ad.r >> 3) + CPL - 1) / CPL;
    return need <= 1 ? 0 : need <= 2 ? 1 : need <= 4 ? 2 : need <= 8 ? 3 : 4;
  }

  // What the epilogue of a tile requests while the tile streams: the weight
  // scale of the thread's row (row_ws, any time) and the first B chunk of
  // its first output (pre_b, once tok[] is resolved; as stored: FP8 codes are
  // widened when used).
  struct EpiPre {
    uint4 b;
    float ws;
  };
  // CPL and group depth inside the tile-major streaming loop and after the
  // stream (the batch-major loop and the fused stash).
  static constexpr int kCplLoop = 1, kGLoop = 1;
  static constexpr int kCplEnd = MB == 1 ? 1 : 4;
  static constexpr int kGEnd = MB == 1 ? 2 : (GEN ? 2 : 4);

  // The raw 16 bytes (bf16) or 8 bytes (FP8, in .x/.y) of chunk c of
  // B[ts.a][n], or zeros when the chunk lies past the rank, the row past N or
  // the token has no adapter.
  __device__ __forceinline__ uint4 b_raw(const TokenSlot& ts, int64_t n, int c) const {
    uint4 v = zero4();
    if (ts.a < 0 || n >= p.N || c * 8 >= ts.rank) return v;
    const int64_t off = ((int64_t)ts.a * p.N + n) * p.ad.r + c * 8;  // elements
    if (af8()) {
      const uint2 w = *reinterpret_cast<const uint2*>(p.ad.B8() + off);
      v.x = w.x;
      v.y = w.y;
    } else {
      v = *reinterpret_cast<const uint4*>(p.ad.B + off);
    }
    return v;
  }

  template <int CPL>
  __device__ __forceinline__ float row_ws(int64_t n0) const {
    if (FMT == EPILORA_W_FP4) return gscale;
    const int64_t n = n0 + ((threadIdx.x >> lane_shift<CPL>()) & 15);
    return n < p.N ? p.wt.sw[n] : 0.f;
  }
  template <int CPL>
  __device__ __forceinline__ uint4 pre_b(int64_t n0) const {
    if (!adapters) return zero4();
    const int sh = lane_shift<CPL>();
    const int o = (int)(threadIdx.x >> sh);
    if (o >= p.M * 16) return zero4();
    return b_raw(tok[o >> 4], n0 + (o & 15), threadIdx.x & ((1 << sh) - 1));
  }

  // Outputs of the tile at n0 from its reduced accumulators `base` ([T][16]).
  // G groups of outputs per lane have their B chunks requested before any
  // is used, so their latencies overlap.
  template <int G, int CPL>
  __device__ __forceinline__ void outputs(int64_t n0, const float* base, const EpiPre& pre) const {
    static_assert(CPL == 1 || CPL == 2 || CPL == 4, "chunks per lane");
    constexpr int NT = NW * kWave;
    const int total_o = (int)p.M * 16;
    if (!adapters) {
      const int64_t n = n0 + (threadIdx.x & 15);
      if (n >= p.N) return;
      for (int o = threadIdx.x; o < total_o; o += NT) {
        const int t = o >> 4;
        p.y[(int64_t)t * p.ldy + n] = (uint16_t)f32_to_bf16((base[o] * sxs[t]) * pre.ws);
      }
      return;
    }
    const int sh = lane_shift<CPL>();
    const int jl = threadIdx.x & ((1 << sh) - 1);
    const int per = NT >> sh;
    const int first = (int)(threadIdx.x >> sh);
    const int64_t n = n0 + (first & 15);
    const int r = p.ad.r;
    const int nch = r >> 3;
    for (int o0 = first; o0 < total_o; o0 += per * G) {
      uint4 raw[G][CPL];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const int o = o0 + gi * per;
        const TokenSlot ts = o < total_o ? tok[o >> 4] : TokenSlot{-1, 0};
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const int c = jl + (q << sh);
          raw[gi][q] = (o == first && q == 0) ? pre.b : (c < nch ? b_raw(ts, n, c) : zero4());
        }
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const int o = o0 + gi * per;
        if (o >= total_o) break;
        const int t = o >> 4;
        const TokenSlot ts = tok[t];
        // One partial dot per chunk (its elements in order), then a fixed
        // tree over the chunk index, lowest bit first: the lane bits through
        // DPP moves, the rest within the lane.  The tree is the same for any
        // lanes-per-output, so every path that writes these outputs (tile- or
        // batch-major, fused or not) gets the same bits.
        float part[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const int c = jl + (q << sh);
          float d = 0.f;
          if (ts.a >= 0 && c < nch && c * 8 < ts.rank) {
            const uint4 v = af8() ? fp8x8_to_bf16x8(raw[gi][q].x, raw[gi][q].y) : raw[gi][q];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            const float4 z0 = *reinterpret_cast<const float4*>(zs + t * r + c * 8);
            const float4 z1 = *reinterpret_cast<const float4*>(zs + t * r + c * 8 + 4);
            const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
            const int lim = ts.rank - c * 8;  // elements of the chunk inside the rank
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float b = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
              if (e < lim) d = fmaf(b, zv[e], d);
            }
          }
          if (sh >= 1) d += dpp_mov<0xB1>(d);   // quad_perm [1, 0, 3, 2]: chunk bit 0
          if (sh >= 2) d += dpp_mov<0x4E>(d);   // quad_perm [2, 3, 0, 1]: bit 1
          if (sh >= 3) d += dpp_mov<0x141>(d);  // row_half_mirror: bit 2 (quads already uniform)
          if (sh >= 4) d += dpp_mov<0x140>(d);  // row_mirror: bit 3 (half rows already uniform)
          part[q] = d;
        }
        float l;
        if constexpr (CPL == 1) l = part[0];
        else if constexpr (CPL == 2) l = part[0] + part[1];
        else l = (part[0] + part[1]) + (part[2] + part[3]);
        if (jl == 0 && n < p.N) {
          float y = (base[o] * sxs[t]) * pre.ws;
          if (ts.a >= 0 && af8()) l *= p.ad.sb[(int64_t)ts.a * p.N + n];  // FP8 adapters: the row scale
          if (ts.a >= 0) y = y + p.ad.scale * l;
          p.y[(int64_t)t * p.ldy + n] = (uint16_t)f32_to_bf16(y);
        }
      }
    }
  }

  // Outputs of all `mine` tiles of a batch-major workgroup (sums in the
  // stash, [S][T][16]; pw[s]: this thread's row weight scale of tile s, as
  // row_ws<CPL>), z of one slice in LDS.  The same arithmetic as outputs(),
  // with the outputs of all the tiles in one list, so that G outputs per lane
  // have their B chunks in flight together whichever tile they belong to.
  template <int G, int CPL>
  __device__ __forceinline__ void outputs_all(int mine, const float (&pw)[StashCfg<MB>::n]) const {
    constexpr int S = StashCfg<MB>::n;
    constexpr int NT = NW * kWave;
    const int total_o = (int)p.M * 16;
    if (!adapters) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int64_t n = n0_of(s * nb) + (threadIdx.x & 15);
        if (s >= mine || n >= p.N) continue;
        const float* base = stash + s * T * 16;
        for (int o = threadIdx.x; o < total_o; o += NT) {
          const int t = o >> 4;
          p.y[(int64_t)t * p.ldy + n] = (uint16_t)f32_to_bf16((base[o] * sxs[t]) * pw[s]);
        }
      }
      return;
    }
    const int sh = lane_shift<CPL>();
    const int jl = threadIdx.x & ((1 << sh) - 1);
    const int per = NT >> sh;
    const int first = (int)(threadIdx.x >> sh);
    const int r = p.ad.r;
    const int nch = r >> 3;
    const int ipt = first < total_o ? (total_o - 1 - first) / per + 1 : 0;  // outputs per tile
    const int items = mine * ipt;
    for (int f0 = 0; f0 < items; f0 += G) {
      uint4 raw[G][CPL];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const int f = f0 + gi;
        const int s = f < items ? f / ipt : 0;
        const int o = first + (f - s * ipt) * per;
        const int64_t n = n0_of(s * nb) + (first & 15);
        const TokenSlot ts = f < items ? tok[o >> 4] : TokenSlot{-1, 0};
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const int c = jl + (q << sh);
          raw[gi][q] = c < nch ? b_raw(ts, n, c) : zero4();
        }
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const int f = f0 + gi;
        if (f >= items) break;
        const int s = f / ipt;
        const int o = first + (f - s * ipt) * per;
        const int t = o >> 4;
        const int64_t n = n0_of(s * nb) + (first & 15);
        float ws = pw[0];
#pragma unroll
        for (int s2 = 1; s2 < S; ++s2)
          if (s == s2) ws = pw[s2];
        const TokenSlot ts = tok[t];
        float part[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const int c = jl + (q << sh);
          float d = 0.f;
          if (ts.a >= 0 && c < nch && c * 8 < ts.rank) {
            const uint4 v = af8() ? fp8x8_to_bf16x8(raw[gi][q].x, raw[gi][q].y) : raw[gi][q];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            const float4 z0 = *reinterpret_cast<const float4*>(zs + t * r + c * 8);
            const float4 z1 = *reinterpret_cast<const float4*>(zs + t * r + c * 8 + 4);
            const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
            const int lim = ts.rank - c * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float b = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
              if (e < lim) d = fmaf(b, zv[e], d);
            }
          }
          if (sh >= 1) d += dpp_mov<0xB1>(d);
          if (sh >= 2) d += dpp_mov<0x4E>(d);
          if (sh >= 3) d += dpp_mov<0x141>(d);
          if (sh >= 4) d += dpp_mov<0x140>(d);
          part[q] = d;
        }
        float l;
        if constexpr (CPL == 1) l = part[0];
        else if constexpr (CPL == 2) l = part[0] + part[1];
        else l = (part[0] + part[1]) + (part[2] + part[3]);
        if (jl == 0 && n < p.N) {
          float y = (stash[s * T * 16 + o] * sxs[t]) * ws;
          if (ts.a >= 0 && af8()) l *= p.ad.sb[(int64_t)ts.a * p.N + n];
          if (ts.a >= 0) y = y + p.ad.scale * l;
          p.y[(int64_t)t * p.ldy + n] = (uint16_t)f32_to_bf16(y);
        }
      }
    }
  }
  // The list above with its depth by rank: up to rank 16 two chunks per
  // output (one lane each) and eight outputs per lane, else four and four.
  __device__ __forceinline__ void outputs_batch(int mine, const float (&pw)[StashCfg<MB>::n]) const {
    if (adapters && p.ad.r <= 16) outputs_all<8, 2>(mine, pw);
    else outputs_all<4, 4>(mine, pw);
  }

  // ---- fused one-block grids: the outputs of all tiles in one list -----------
  // Item g of the list (g < mine * M * 16) is output o = g % (M * 16) of the
  // workgroup's tile s = g / (M * 16); each takes 2^sh lanes as in outputs()
  // (CPL = 1), and lane group `first` takes items first, first + per, ...
  // The tiles' outputs then run side by side instead of one tile after
  // another, and a thread's first items need nothing but the prefetch.
  __device__ __forceinline__ float wscale_at(int64_t n) const {
    if (FMT == EPILORA_W_FP4) return gscale;
    return n < p.N ? p.wt.sw[n] : 0.f;
  }
  // The requests for items first + k * per, k < P, into b / ws.
  template <int P>
  __device__ __forceinline__ void flat_request(int k0, int mine, uint4 (&b)[P], float (&ws)[P]) const {
    const int sh = lane_shift<1>();
    const int jl = threadIdx.x & ((1 << sh) - 1);
    const int per = (NW * kWave) >> sh, first = (int)(threadIdx.x >> sh);
    const int total_o = (int)p.M * 16, items = mine * total_o;
    const int nch = p.ad.r >> 3;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const int g = first + (k0 + k) * per;
      int s = 0, o = 0;
      if (g < items) {
        s = g / total_o;
        o = g - s * total_o;
      }
      const int64_t n = n0_of(s * nb) + (o & 15);
      const TokenSlot ts = (adapters && g < items) ? tok[o >> 4] : TokenSlot{-1, 0};
      b[k] = jl < nch ? b_raw(ts, n, jl) : zero4();
      ws[k] = g < items ? wscale_at(n) : 0.f;
    }
  }
  __device__ __forceinline__ void flat_prefetch() {
    flat_request<kFlatPre>(0, total / nb, fpre_b, fpre_ws);
  }
  template <int P>
  __device__ __forceinline__ void flat_group(int k0, int mine, int sl0, const uint4 (&b)[P],
                                             const float (&ws)[P]) const {
    const int sh = lane_shift<1>();
    const int jl = threadIdx.x & ((1 << sh) - 1);
    const int per = (NW * kWave) >> sh, first = (int)(threadIdx.x >> sh);
    const int total_o = (int)p.M * 16, items = mine * total_o;
    const int r = p.ad.r, nch = r >> 3;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const int g = first + (k0 + k) * per;
      if (g >= items) break;
      const int s = g / total_o, o = g - s * total_o, t = o >> 4;
      const int64_t n = n0_of(s * nb) + (o & 15);
      const TokenSlot ts = tok[t];
      float d = 0.f;
      if (ts.a >= 0 && jl < nch && jl * 8 < ts.rank) {
        const uint4 v = af8() ? fp8x8_to_bf16x8(b[k].x, b[k].y) : b[k];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        const float* zt = zs + (slice(n) - sl0) * (int)p.M * r + t * r + jl * 8;  // z of the tile's slice
        const float4 z0 = *reinterpret_cast<const float4*>(zt);
        const float4 z1 = *reinterpret_cast<const float4*>(zt + 4);
        const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
        const int lim = ts.rank - jl * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float bb = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
          if (e < lim) d = fmaf(bb, zv[e], d);
        }
      }
      if (sh >= 1) d += dpp_mov<0xB1>(d);
      if (sh >= 2) d += dpp_mov<0x4E>(d);
      if (sh >= 3) d += dpp_mov<0x141>(d);
      if (sh >= 4) d += dpp_mov<0x140>(d);
      if (jl == 0 && n < p.N) {
        float y = (stash[s * T * 16 + o] * sxs[t]) * ws[k];
        if (ts.a >= 0 && af8()) d *= p.ad.sb[(int64_t)ts.a * p.N + n];
        if (ts.a >= 0) y = y + p.ad.scale * d;
        p.y[(int64_t)t * p.ldy + n] = (uint16_t)f32_to_bf16(y);
      }
    }
  }
  // Every output of the workgroup's `mine` tiles (sums in the stash, z of
  // the one slice in LDS).  The same arithmetic as outputs<G, 1>.
  __device__ __forceinline__ void outputs_flat(int mine, int sl0) const {
    const int sh = lane_shift<1>();
    const int per = (NW * kWave) >> sh, first = (int)(threadIdx.x >> sh);
    const int items = mine * (int)p.M * 16;
    flat_group<kFlatPre>(0, mine, sl0, fpre_b, fpre_ws);
    for (int k0 = kFlatPre; first + k0 * per < items; k0 += kFlatPre) {
      uint4 b[kFlatPre];
      float ws[kFlatPre];
      flat_request<kFlatPre>(k0, mine, b, ws);
      flat_group<kFlatPre>(k0, mine, sl0, b, ws);
    }
  }

  // Fused: z is published in place.  Every word of the z region reads zero
  // until its producer stores it (as its bitwise complement), so the
  // workgroup polls the words of its active tokens until none is missing,
  // staging them into LDS (rows of inactive tokens as zero), under the
  // wall-clock limit.  Returns false on a timeout (or when the host has set
  // the workspace's force-timeout word, read with the first poll).  Ends with
  // a barrier.
  __device__ __forceinline__ bool poll_z(int slice, float* dst = nullptr) const {
    float* zd = dst != nullptr ? dst : zs;
    const int r = p.ad.r;
    const int n = (int)p.M * r;
    const auto zr = make_rsrc(p.z + slice * r, (uint32_t)(((p.M - 1) * zld() + r) * 4));
    int* err = p.ctrl + kCtrlError;
    const int64_t start = wall_clock64();
    for (;;) {
      const int forced = threadIdx.x == 0 ? load_relaxed(p.ctrl + kCtrlForceTimeout) : 0;
      int missing = 0;
      for (int e = threadIdx.x; e < n; e += NW * kWave) {
        if (tok[e / r].a < 0) {
          zd[e] = 0.f;
        } else {
          const uint32_t w = buf_load4<kCoherent>(zr, 4u * ((e / r) * zld() + e % r));
          if (w == 0u) missing = 1;
          else zd[e] = __uint_as_float(~w);
        }
      }
      if (threadIdx.x == 0) *verdict = 0;
      __syncthreads();
      if (missing) *verdict = 1;
      __syncthreads();
      if (threadIdx.x == 0) {
        int state = *verdict;  // 0: complete, 1: poll again, 2: give up
        if (forced != 0 ||
            (state != 0 && (wall_clock64() - start > J.wait_ticks || (load_relaxed(err) & EPILORA_DEV_WAIT_TIMEOUT))))
          state = 2;
        *verdict = state;
      }
      __syncthreads();
      const int state = *verdict;
      __syncthreads();
      if (state == 0) return true;
      if (state == 2) return false;
      __builtin_amdgcn_s_sleep(2);
    }
  }

  // One slice's z (M x r fp32, columns slice * r .. + r of the [M][S r] z)
  // into LDS, rows of inactive tokens as zero.  Starts and ends with a
  // barrier (the previous slice's values may still be read).
  __device__ __forceinline__ void stage_z(int slice) const {
    const int r = p.ad.r;
    const auto zr = make_rsrc(p.z + slice * r, (uint32_t)(((p.M - 1) * zld() + r) * 4));
    __syncthreads();
    for (int e = threadIdx.x; e < p.M * r; e += NW * kWave)
      zs[e] = tok[e / r].a >= 0 ? __uint_as_float(buf_load4<XPOL>(zr, 4u * ((e / r) * zld() + e % r))) : 0.f;
    __syncthreads();
  }

  // Sums the NW waves' partial accumulators of the finished tile into `dst`
  // ([T][16], wave order) and clears the accumulators.  Ends with a barrier.
  __device__ __forceinline__ void reduce_tile(f32x4 (&acc)[MB], float* dst) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int t = mb * 16 + row;
      *reinterpret_cast<float4*>(&part[(wave * T + t) * 16 + 4 * (lane >> 4)]) =
          make_float4(acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]);
      acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    const int outs = (int)p.M * 16;
    for (int e = threadIdx.x; e < outs; e += NW * kWave) {
      float v = part[e];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += part[w * T * 16 + e];
      dst[e] = v;
    }
    __syncthreads();
  }

  // Tile j / nb is complete in `acc`.  Fused: reduce it into its stash slot.
  // Otherwise z is ready: write its outputs, then request the next tile's
  // first B slice and weight scale.
  __device__ __forceinline__ void tile_done(int j, f32x4 (&acc)[MB], EpiPre& pre) {
    if (FUSED) {
      reduce_tile(acc, stash + (j / nb) * T * 16);
      return;
    }
    reduce_tile(acc, red);
    if (GEN && adapters && p.ad.S > 1) {  // a tile lies inside one slice; the slices come in order
      const int sl = slice(n0_of(j));
      if (sl != zslice) {
        stage_z(sl);
        zslice = sl;
      }
    }
    outputs<kGLoop, kCplLoop>(n0_of(j), red, pre);
    if (j + 1 < total) {
      pre.b = pre_b<kCplLoop>(n0_of(j + 1));
      pre.ws = row_ws<kCplLoop>(n0_of(j + 1));
    }
  }

  // ---- fused: counting the workgroups done ----------------------------------
  // Once a workgroup has every z word it needs in LDS (and long after it
  // passed the quantized-rows flag) it reads neither again, so it counts
  // itself done right then: the returning atomic is in flight while the
  // epilogues run and is waited for only in done_finish.  The last of each
  // of kDoneGroups groups counts the group; the last group puts the flag back
  // to zero and tells its workgroup to clear z; each counter is reset by the
  // one that completed it.
  __device__ __forceinline__ void done_issue() {
    if (!FUSED || !J.flags || threadIdx.x != 0 || done_old >= 0) return;
    const int groups = J.gwgs < kDoneGroups ? J.gwgs : kDoneGroups;
    done_old = atomic_add_relaxed(J.done + (g % groups) * kDoneStride, 1);
  }
  // Every thread calls it (with flags); true in the one workgroup that is
  // to clear z.  Ends with a barrier.
  __device__ __forceinline__ bool done_finish() {
    done_issue();
    if (threadIdx.x == 0) {
      const int groups = J.gwgs < kDoneGroups ? J.gwgs : kDoneGroups;
      const int grp = g % groups;
      const int members = J.gwgs / groups + (grp < J.gwgs % groups ? 1 : 0);
      int last = 0;
      if (done_old == members - 1) {
        store_relaxed(J.done + grp * kDoneStride, 0);
        if (atomic_add_relaxed(p.ctrl + kCtrlGemmDone, 1) == groups - 1) {
          store_relaxed(p.ctrl + kCtrlQuantDone, 0);
          store_relaxed(p.ctrl + kCtrlGemmDone, 0);
          last = 1;
        }
      }
      *verdict = last;
    }
    __syncthreads();
    return *verdict != 0;
  }

  // Fused: every tile of the workgroup is in the stash.  Request the first B
  // slice of each, poll z into LDS, write the outputs (pw: each tile's weight
  // scale, requested at the start).
  __device__ __forceinline__ void finish_stash(bool& ok, const float (&pw)[StashCfg<MB>::n]) {
    constexpr int S = StashCfg<MB>::n;
    const int mine = total / nb;
    if (flat()) {
      // the tiles come in output order: the slices they span, sl0 .. sl1,
      // each polled into its own plane
      const int sl0 = mine > 0 ? slice(n0_of(0)) : 0;
      const int sl1 = mine > 0 ? slice(n0_of((mine - 1) * nb)) : 0;
      if (adapters) {
        for (int sl = sl0; sl <= sl1; ++sl) {
          ok = poll_z(sl, zs + (sl - sl0) * (int)p.M * p.ad.r);
          if (!ok) return;
        }
        done_issue();  // every z word this workgroup needs is in LDS
      }
      outputs_flat(mine, sl0);
      return;
    }
    if constexpr (MB >= 2) {  // batch-major: all tiles in one list when they share a slice
      if (mine == 0 || slice(n0_of(0)) == slice(n0_of((mine - 1) * nb))) {
        if (adapters) {
          ok = poll_z(mine > 0 ? slice(n0_of(0)) : 0);
          if (!ok) return;
          done_issue();  // every z word this workgroup needs is in LDS
        }
        outputs_batch(mine, pw);
        return;
      }
    }
    uint4 pb[S];
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (s < mine) pb[s] = pre_b<kCplEnd>(n0_of(s * nb));
    // The tiles come in output order: for each slice they span (one unless
    // the projection has several), poll that slice's z into LDS, then write
    // the outputs of the tiles inside it.
    const int sl0 = mine > 0 ? slice(n0_of(0)) : 0;
    const int sl1 = mine > 0 ? slice(n0_of((mine - 1) * nb)) : 0;
    for (int sl = sl0; sl <= sl1; ++sl) {
      if (adapters) {
        if (sl > sl0) __syncthreads();  // the previous slice's z is no longer read
        ok = poll_z(sl);
        if (!ok) return;
        if (sl == sl1) done_issue();  // every z word this workgroup needs is in LDS
      }
#pragma unroll
      for (int s = 0; s < S; ++s)
        if (s < mine && (sl0 == sl1 || slice(n0_of(s * nb)) == sl))
          outputs<kGEnd, kCplEnd>(n0_of(s * nb), stash + s * T * 16, EpiPre{pb[s], pw[s]});
    }
  }

  // ---- the whole job, two or more token blocks: batch-major ----------------
  // With 17-64 tokens the activations of a step (up to 8 KB per wave) outweigh
  // its 2 KB of weights, so reading them again for every 16-row tile made the
  // caches, not HBM, the limit.  Here each wave takes its K batches in turn
  // and, for each, loads its activations once into registers (double
  // buffered across batches) and runs them against every tile of the
  // workgroup (at most S, which the host guarantees), each tile with its own
  // accumulators and its own weight registers: the load of a tile's next
  // batch is issued right after its current batch is multiplied, so the
  // weights of the other tiles stay in flight meanwhile.  Each wave still
  // sums its own K range of a tile in step order, so the results are bitwise
  // those of the tile-major loop; the tiles are reduced across the waves
  // after the last batch (into the stash when fused, else straight to the
  // outputs).
  __device__ __forceinline__ void run_batches() {
    constexpr int S = StashCfg<MB>::n;
    constexpr int NT = NW * kWave;
    const int64_t M = p.M;
    int* err = p.ctrl != nullptr ? p.ctrl + kCtrlError : nullptr;
    const int mine = total / nb;
    const TokenLoad tl = load_token();
    __builtin_amdgcn_sched_barrier(0);
    // Every load below is issued unconditionally (a dead one gets an
    // out-of-range offset and reads zero without touching memory), so the
    // number of loads in flight at each multiply is known when compiling and
    // each waits only for its own registers.
    u32x4 wa[S][U], wb[S][U];
#pragma unroll
    for (int t = 0; t < S; ++t) load_w_at(wa[t], wb[t], t, 0, t < mine);
    __builtin_amdgcn_sched_barrier(0);
    if (FMT == EPILORA_W_FP4) build_fold_table(tbl);
    resolve_tokens(tl, g == 0);
    float pw[S];  // each tile's weight scale for the epilogue
#pragma unroll
    for (int t = 0; t < S; ++t) pw[t] = t < mine ? row_ws<kCplEnd>(n0_of(t * nb)) : 0.f;
    bool ok = true;
    if (kRowsInGrid) {  // the quantized rows come from other workgroups
      ok = wait_flag(J.qflag, J.qtarget, J.wait_ticks, err, p.ctrl + kCtrlForceTimeout, verdict);
      const auto sr = make_rsrc(p.sx, (uint32_t)(M * 4));
      for (int t = threadIdx.x; t < M; t += NT) sxs[t] = __uint_as_float(buf_load4<kCoherent>(sr, 4u * t));
    } else {
      for (int t = threadIdx.x; t < M; t += NT) sxs[t] = A16 ? 1.0f : p.sx[t];
    }
    __syncthreads();

    f32x4 acc[S][MB];
#pragma unroll
    for (int t = 0; t < S; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[t][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 x0[U][MB][XV], x1[U][MB][XV];
    load_x_at(x0, 0, true);
    for (int b = 0; b < nb; b += 2) {
      load_x_at(x1, b + 1, b + 1 < nb);
#pragma unroll
      for (int t = 0; t < S; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        if (t < mine) compute_at(wa[t], wb[t], x0, b, true, acc[t]);
        __builtin_amdgcn_sched_barrier(0);
        load_w_at(wa[t], wb[t], t, b + 1, t < mine && b + 1 < nb);
      }
      if (b + 1 >= nb) break;
      load_x_at(x0, b + 2, b + 2 < nb);
#pragma unroll
      for (int t = 0; t < S; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        if (t < mine) compute_at(wa[t], wb[t], x1, b + 1, true, acc[t]);
        __builtin_amdgcn_sched_barrier(0);
        load_w_at(wa[t], wb[t], t, b + 2, t < mine && b + 2 < nb);
      }
    }

    if (FUSED) {
#pragma unroll
      for (int t = 0; t < S; ++t)
        if (t < mine) reduce_tile(acc[t], stash + t * T * 16);
      if (ok) finish_stash(ok, pw);
    } else if (mine == 0 || slice(n0_of(0)) == slice(n0_of((mine - 1) * nb))) {
      // all tiles in one slice: reduce them all, then one list of outputs
#pragma unroll
      for (int t = 0; t < S; ++t)
        if (t < mine) reduce_tile(acc[t], stash + t * T * 16);
      if (adapters) stage_z(mine > 0 ? slice(n0_of(0)) : 0);
      outputs_batch(mine, pw);
    } else {
      uint4 pb[S];
#pragma unroll
      for (int t = 0; t < S; ++t)
        if (t < mine) pb[t] = pre_b<kCplEnd>(n0_of(t * nb));
      if (adapters) {
        zslice = mine > 0 ? slice(n0_of(0)) : 0;
        stage_z(zslice);
      }
#pragma unroll
      for (int t = 0; t < S; ++t) {
        if (t < mine) {
          reduce_tile(acc[t], red);
          if (GEN && adapters && p.ad.S > 1) {
            const int sl = slice(n0_of(t * nb));
            if (sl != zslice) {
              stage_z(sl);
              zslice = sl;
            }
          }
          outputs<kGEnd, kCplEnd>(n0_of(t * nb), red, EpiPre{pb[t], pw[t]});
        }
      }
    }
    if (!ok && threadIdx.x == 0 && err != nullptr) atomic_or_relaxed(err, EPILORA_DEV_WAIT_TIMEOUT);
  }

  // ---- the whole job --------------------------------------------------------
  __device__ __forceinline__ void run() {
    if constexpr (MB >= 2 && !XLDS && !A16) {  // (W8A16: too few registers for it)
      run_batches();
      return;
    }
    constexpr int NT = NW * kWave;
    constexpr int RV = NW == 8 ? 4 : 8;
    const int64_t M = p.M, K = p.K;
    int* err = p.ctrl != nullptr ? p.ctrl + kCtrlError : nullptr;
    // Activation loads first, then the first two weight batches; the set-up
    // below overlaps them.
    SelfQuant<NT, RV> sq;
    SelfCopy<NT, RV> sc;
    if (XLDS && FUSED && !A16) sq.issue(J.x, J.ldx, (int)M, K);
    if (XLDS && FUSED && A16) sc.issue(J.x, J.ldx, (int)M, K);
    const TokenLoad tl = load_token();
    __builtin_amdgcn_sched_barrier(0);
    SkinnyBatch<MB, U, XV> A, B;
    load_w(A, 0);
    load_w(B, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (FMT == EPILORA_W_FP4) build_fold_table(tbl);
    resolve_tokens(tl, g == 0);
    __syncthreads();  // tok[] is read below by threads of other waves
    if (XLDS && FUSED && !A16) sq.finish(J.x, J.ldx, (int)M, K, xs, sxs, reinterpret_cast<uint32_t*>(red));
    if (XLDS && FUSED && A16) sc.finish(J.x, J.ldx, (int)M, K, xs, sxs);
    if (XLDS && !FUSED) {  // the skinny GEMM kernel: copy the quantized (or bf16) rows
      const int64_t row_bytes = K * XB;
      const int64_t nv = M * row_bytes / 16;
      const uint8_t* src = A16 ? reinterpret_cast<const uint8_t*>(p.x16) : p.xq;
      const int64_t ld_bytes = A16 ? p.ldx16 * 2 : p.ldq;
      for (int64_t v = threadIdx.x; v < nv; v += NT) {
        const int64_t t = v * 16 / row_bytes, c = v * 16 % row_bytes;
        *reinterpret_cast<uint4*>(xs + 16 * v) = *reinterpret_cast<const uint4*>(src + t * ld_bytes + c);
      }
    }
    if (!FUSED) {
      for (int t = threadIdx.x; t < M; t += NT) sxs[t] = A16 ? 1.0f : p.sx[t];
      if (adapters) {
        zslice = total > 0 ? slice(n0_of(0)) : 0;
        stage_z(zslice);
      }
    }
    __syncthreads();

    bool ok = true;
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    EpiPre pre{zero4(), 0.f};
    if (!FUSED) pre = EpiPre{pre_b<kCplLoop>(n0_of(0)), row_ws<kCplLoop>(n0_of(0))};
    float pw[StashCfg<MB>::n];  // fused: the weight scale of each tile, needed after the stream
#pragma unroll
    for (int s = 0; s < StashCfg<MB>::n; ++s)
      pw[s] = (FUSED && !flat() && s < total / nb) ? row_ws<kCplEnd>(n0_of(s * nb)) : 0.f;
    if (flat()) flat_prefetch();

    if (kRowsInGrid) {  // the quantized rows come from other workgroups
      ok = wait_flag(J.qflag, J.qtarget, J.wait_ticks, err, p.ctrl + kCtrlForceTimeout, verdict);
      const auto sr = make_rsrc(p.sx, (uint32_t)(M * 4));
      for (int t = threadIdx.x; t < M; t += NT) sxs[t] = __uint_as_float(buf_load4<kCoherent>(sr, 4u * t));
      __syncthreads();
    } else if (FUSED && !XLDS) {  // rows quantized by an earlier launch, or the caller's bf16 rows
      for (int t = threadIdx.x; t < M; t += NT) sxs[t] = A16 ? 1.0f : p.sx[t];
      __syncthreads();
    }
    load_x(A, 0);
    load_x(B, 1);

    // Two batches in flight; a tile's reduction (and, unfused, its epilogue)
    // runs before the batch that just finished is refilled.
    for (int j = 0; j < total; j += 2) {
      const bool endA = j % nb == nb - 1;
      const bool endB = j + 1 < total && (j + 1) % nb == nb - 1;
      __builtin_amdgcn_sched_barrier(0);
      compute(A, j, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (endA) tile_done(j, acc, pre);
      __builtin_amdgcn_sched_barrier(0);
      load_w(A, j + 2);
      load_x(A, j + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(B, j + 1, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (endB) tile_done(j + 1, acc, pre);
      __builtin_amdgcn_sched_barrier(0);
      load_w(B, j + 3);
      load_x(B, j + 3);
    }
    if (FUSED && ok) finish_stash(ok, pw);
    if (!ok && threadIdx.x == 0 && err != nullptr) atomic_or_relaxed(err, EPILORA_DEV_WAIT_TIMEOUT);
  }
};

// Host side: the launch shape of a persistent skinny grid.  Eight waves per
// workgroup when there are at most 256 tiles and few tokens, else four.  The
// grid takes as few rounds of tiles as the resident slots (`resident`) allow
// and, for that many rounds, as few workgroups as give every workgroup the
// same number of tiles to within one, so slots stay free for others.
inline int skinny_waves(int64_t N, int MB) { return (cdiv(N, 16) <= 256 && MB <= 2) ? 8 : 4; }
// `max_rounds` (> 0) caps the tiles of one workgroup (the fused kernel's
// stash); the grid may then exceed the resident slots, which is safe because
// a fused workgroup waits only on workgroups dispatched before it.
inline int skinny_groups(int64_t N, int resident, int max_rounds = 0) {
  const int64_t tiles = cdiv(N, 16);
  const int64_t slots = resident > 0 ? resident : 1;
  int64_t rounds = cdiv(tiles, slots);
  if (max_rounds > 0 && rounds > max_rounds) rounds = max_rounds;
  return (int)cdiv(tiles, rounds);
}
// Workgroups of a batch-major grid (at most S = stash_tiles(MB) tiles each).
// Every workgroup reads all M activation rows over the whole of K, so from 33
// tokens on (X bytes per workgroup >= 3/4 of its weight bytes) each takes
// the full S tiles even where that leaves compute units idle: at 64 tokens
// the 72B-shaped qkv, o and down projections (640, 512, 512 tiles) ran
// 30-40% faster on 160 / 128 / 128 workgroups than spread over 320 / 512 /
// 512 with fewer tiles each.  Below that the grid spreads over the resident
// slots as tile-major grids do.
inline int skinny_batch_groups(int64_t N, int MB, int resident) {
  const int S = stash_tiles(MB);
  if (MB >= 3) return (int)cdiv(cdiv(N, 16), S);
  return skinny_groups(N, resident, S);
}
// Whether the quantized activations live in LDS (the fused kernel then
// quantizes them itself), and the LDS bytes of the workgroup.
// xb: bytes per activation element (1 FP8, 2 bf16 for the W8A16 GEMM).
inline bool skinny_x_in_lds(int64_t M, int64_t K, int MB, int NW, int r, bool fused, int fmt, int xb = 1) {
  if (M * K * xb > kXInLdsMax || (fused && M > kSelfQuantMaxM)) return false;
  const int nstash = fused ? stash_tiles(MB) : 0;
  return sk_layout(MB, NW, r, (uint32_t)(M * K * xb), nstash, fmt).total <= kLdsBudget;
}
inline uint32_t skinny_lds(int64_t M, int64_t K, int MB, int NW, int r, bool fused, bool xlds, int fmt, int xb = 1,
                           int zplanes = 1) {
  // fused grids and batch-major ones (several token blocks, FP8 codes read
  // from memory) keep the sums of all their tiles
  const int nstash = (fused || (MB >= 2 && !xlds && xb == 1)) ? stash_tiles(MB) : 0;
  return sk_layout(MB, NW, r, xlds ? (uint32_t)(M * K * xb) : 0u, nstash, fmt, zplanes).total;
}

}  // namespace epilora
