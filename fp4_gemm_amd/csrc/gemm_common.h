// Pieces shared by the GEMM kernels and the fused decode path: parameters,
// weight-fragment loads (FP8, or 4-bit folded to FP8), the skinny main loop
// and its epilogue.
#pragma once

#include "adapters.h"
#include "layout.h"

namespace epilora {

struct GemmParams {
  const uint8_t* xq;
  const float* sx;
  int64_t ldq;
  int64_t M, N, K;
  WeightArgs wt;
  AdapterArgs ad;
  const float* z;  // null: base only
  uint16_t* y;
  int64_t ldy;
  int* ctrl;
};

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// The 8 fold-table magnitudes of every block-scale code, as two dwords per
// code (codes 0..3, codes 4..7), built in LDS by the calling workgroup.
__device__ __forceinline__ void build_fold_table(uint2* tbl) {
  for (int b = threadIdx.x; b < 256; b += blockDim.x) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      lo |= fold_entry(c, b) << (8 * c);
      hi |= fold_entry(c + 4, b) << (8 * c);
    }
    tbl[b] = make_uint2(lo, hi);
  }
}

// Raw bytes of one lane's 32-element slice of a weight row.
struct RawW {
  uint4 a;      // FP8: elements 0..15; 4-bit: 32 packed codes
  uint4 b;      // FP8: elements 16..31
  uint32_t s;   // 4-bit: the two block scales
};

template <int FMT>
__device__ __forceinline__ RawW load_w_raw(const WeightArgs& wt, int64_t n, int64_t K, int64_t k, bool ok) {
  RawW r;
  r.a = zero4();
  r.b = zero4();
  r.s = 0;
  if (!ok) return r;
  if (FMT == EPILORA_W_FP8) {
    const uint4* p = reinterpret_cast<const uint4*>(wt.w + n * K + k);
    r.a = p[0];
    r.b = p[1];
  } else {
    r.a = *reinterpret_cast<const uint4*>(wt.w + n * (K / 2) + k / 2);
    r.s = *reinterpret_cast<const uint16_t*>(wt.bs + n * (K / 16) + k / 16);
  }
  return r;
}

// 32 FP8 bytes in element order (the 4-bit codes go through the fold table).
template <int FMT>
__device__ __forceinline__ i32x8 w_frag(const RawW& r, const uint2* tbl) {
  if (FMT == EPILORA_W_FP8) return as_i32x8(r.a, r.b);
  i32x8 f;
  const uint2 t0 = tbl[r.s & 0xFFu], t1 = tbl[(r.s >> 8) & 0xFFu];
  uint32_t o0, o1;
  fold8(r.a.x, t0.x, t0.y, o0, o1); f[0] = o0; f[1] = o1;
  fold8(r.a.y, t0.x, t0.y, o0, o1); f[2] = o0; f[3] = o1;
  fold8(r.a.z, t1.x, t1.y, o0, o1); f[4] = o0; f[5] = o1;
  fold8(r.a.w, t1.x, t1.y, o0, o1); f[6] = o0; f[7] = o1;
  return f;
}

// The scale a row's accumulator takes after the activation scale:
// sw[n] for FP8 weights, gs * 8 for 4-bit ones (the fold pre-scales by 1/8).
template <int FMT>
__device__ __forceinline__ float weight_scale(const WeightArgs& wt, int64_t n) {
  if (FMT == EPILORA_W_FP8) return wt.sw[n];
  return wt.gs[0] * 8.0f;
}

// ---------------------------------------------------------------------------
// Skinny main loop (M <= 64 tokens).  A workgroup owns 16 weight rows; its 4
// waves split the K steps (128 wide) into 4 contiguous ranges.  Swap-AB: the
// weight rows are the matrix core's 16-row operand and the (up to 4 blocks
// of 16) tokens its 16-column operand, so C[n][t] sits in lane
// (t % 16) + 16 * ((n % 16) / 4), register n % 4.  Lane l loads 32
// consecutive bytes of weight row (l % 16) and of token row (l % 16) at the
// same K offset 32 * (l / 16): both operands see the same K positions.  U
// steps are loaded before any is multiplied, to keep enough bytes in flight.
// ---------------------------------------------------------------------------
template <int MB, int FMT, int U>
__device__ __forceinline__ void skinny_mainloop(const GemmParams& p, int64_t n0, f32x4 (&acc)[MB],
                                                const uint2* tbl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int steps = (int)cdiv(p.K, 128);
  const int spw = (int)cdiv(steps, 4);
  const int sb = wave * spw;
  const int se = min(steps, sb + spw);
  const int64_t n = n0 + (lane & 15);
  const bool nok = n < p.N;
  const int kofs = (lane >> 4) * 32;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = sb; s < se; s += U) {
    RawW w[U];
    uint4 xa[U][MB], xb[U][MB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (int64_t)(s + u) * 128 + kofs;
      const bool ok = (s + u < se) && k < p.K;
      w[u] = load_w_raw<FMT>(p.wt, n, p.K, k, ok && nok);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int64_t t = mb * 16 + (lane & 15);
        if (ok && t < p.M) {
          const uint4* xp = reinterpret_cast<const uint4*>(p.xq + t * p.ldq + k);
          xa[u][mb] = xp[0];
          xb[u][mb] = xp[1];
        } else {
          xa[u][mb] = zero4();
          xb[u][mb] = zero4();
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const i32x8 wf = w_frag<FMT>(w[u], tbl);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_fp8_16x16x128(wf, as_i32x8(xa[u][mb], xb[u][mb]), acc[mb]);
    }
  }
}

// Token metadata the skinny epilogue needs, resolved once per workgroup.
struct TokenSlot {
  int a;
  int rank;
};

// Cross-wave sum (fixed wave order), scales, the adapter term for active
// rows (fp32 dot over the rank), bf16 store.  `part` is LDS of
// [4][MB * 16][16] floats; `tok` holds M entries.
template <int MB, int FMT>
__device__ __forceinline__ void skinny_epilogue(const GemmParams& p, int64_t n0, const f32x4 (&acc)[MB],
                                                float* part, const TokenSlot* tok, const float* z) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int T = MB * 16;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int t = mb * 16 + (lane & 15);
    *reinterpret_cast<float4*>(&part[(wave * T + t) * 16 + 4 * (lane >> 4)]) =
        make_float4(acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]);
  }
  __syncthreads();
  const int r = p.ad.r;
  for (int e = threadIdx.x; e < T * 16; e += blockDim.x) {
    const int t = e >> 4;
    const int64_t n = n0 + (e & 15);
    if (t >= p.M || n >= p.N) continue;
    float v = part[e];
    v += part[T * 16 + e];
    v += part[2 * T * 16 + e];
    v += part[3 * T * 16 + e];
    float y = (v * p.sx[t]) * weight_scale<FMT>(p.wt, n);
    if (z != nullptr && tok[t].a >= 0) {
      const int rank = tok[t].rank;
      const uint16_t* br = p.ad.B + ((int64_t)tok[t].a * p.N + n) * r;
      const float* zr = z + (int64_t)t * r;
      float l = 0.f;
      int j = 0;
      for (; j + 8 <= rank; j += 8) {
        const uint4 b = *reinterpret_cast<const uint4*>(br + j);
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          l = fmaf(bf16_lo(bw[i]), zr[j + 2 * i], l);
          l = fmaf(bf16_hi(bw[i]), zr[j + 2 * i + 1], l);
        }
      }
      for (; j < rank; ++j) l = fmaf(bf16_to_f32(br[j]), zr[j], l);
      y = y + p.ad.scale * l;
    }
    p.y[(int64_t)t * p.ldy + n] = (uint16_t)f32_to_bf16(y);
  }
}

}  // namespace epilora
