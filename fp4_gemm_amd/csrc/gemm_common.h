// Pieces shared by the GEMM kernels and the fused decode path: parameters,
// weight-fragment loads (FP8, or 4-bit folded to FP8) and weight scales.
#pragma once

#include "adapters.h"
#include "layout.h"

namespace epilora {

struct GemmParams {
  const uint8_t* xq;
  const float* sx;
  int64_t ldq;
  const uint16_t* x16;  // the W8A16 GEMM: bf16 activations [M][ldx16] (xq, sx unused)
  int64_t ldx16;
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

// Token metadata an epilogue needs, resolved once per workgroup.
struct TokenSlot {
  int a;
  int rank;
};

// The prefill GEMM (M > 64), gemm_wide.hip.
void launch_gemm_wide(const GemmParams& p, hipStream_t stream);
// The prefill GEMM with 256 x 256 tiles, gemm_big.hip, for shapes that
// gemm_big_fits accepts.
bool gemm_big_fits(const GemmParams& p);
void launch_gemm_big(const GemmParams& p, hipStream_t stream);

}  // namespace epilora
