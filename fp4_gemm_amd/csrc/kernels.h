// Host-side launchers of the gfx950 kernels (internal to the library; the
// public ABI is include/epilora.h).  Every launcher assumes its arguments
// were validated by the API layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace epilora {

constexpr int kMaxSlices = 4;

// Adapter metadata as the kernels see it.  A projection's outputs may be S
// consecutive slices, each with its own adapter pair: A holds the slices'
// down-projections side by side ([L][S][r][K]), B the rows of each slice's
// up-projection in place ([L][N][r]), z the slices' results side by side
// ([M][S r]).  S = 1 is the plain layer.
// Adapters are bf16, or stored in FP8 (afmt 1): then A and B hold E4M3 codes
// (one byte per element, the same shapes) and each row carries one fp32
// scale, sa [L][S][r] for A's rank rows and sb [L][N] for B's output rows.
struct AdapterArgs {
  const uint16_t* A;     // [L][S][r][K] (bf16, or E4M3 bytes when afmt == 1)
  const uint16_t* B;     // [L][N][r]    (bf16, or E4M3 bytes when afmt == 1)
  const int32_t* ranks;  // [L] or null (one rank for every slice of an adapter)
  const int32_t* idx;    // [M] or null (no adapters)
  const uint8_t* mask;   // [M] or null
  int32_t L, r;
  float scale;
  int32_t S;                     // slices, 1..kMaxSlices
  int32_t zld;                   // z row stride: S * r
  int64_t slice_end[kMaxSlices]; // end (exclusive) of each slice's outputs
  int32_t afmt;                  // 0: bf16 adapters; 1: FP8 adapters with row scales
  const float* sa;               // [L][S][r] (afmt 1)
  const float* sb;               // [L][N]    (afmt 1)

  __host__ __device__ const uint8_t* A8() const { return reinterpret_cast<const uint8_t*>(A); }
  __host__ __device__ const uint8_t* B8() const { return reinterpret_cast<const uint8_t*>(B); }
};

// The slice output n falls in.
__host__ __device__ inline int slice_of(const AdapterArgs& ad, int64_t n) {
  int s = 0;
#pragma unroll
  for (int i = 0; i < kMaxSlices - 1; ++i) s += (i < ad.S - 1 && n >= ad.slice_end[i]) ? 1 : 0;
  return s;
}

// Base-weight operand.
struct WeightArgs {
  int32_t fmt;           // 0 = FP8 per channel, 1 = 4-bit (fold to FP8)
  const uint8_t* w;
  const float* sw;
  const uint8_t* bs;
  const float* gs;
};

hipError_t launch_quant_rows(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* xq,
                             int64_t ldq, float* scale, hipStream_t stream);
hipError_t launch_quant_weight_fp4(const uint16_t* w, int64_t N, int64_t K, uint8_t* wc, uint8_t* bs,
                                   float* gs, void* ws, hipStream_t stream);
hipError_t launch_fill_u32(void* p, uint32_t v, int64_t n, hipStream_t stream);

hipError_t launch_shrink(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const AdapterArgs& ad,
                         float* z, void* ws, hipStream_t stream);
hipError_t launch_expand_add(const float* z, int64_t M, int64_t N, const AdapterArgs& ad, uint16_t* y,
                             int64_t ldy, void* ws, hipStream_t stream);

// The GEMM with the multi-adapter epilogue.  z == null: base only.  x16
// non-null: the matched W8A16 GEMM on bf16 activations [M][ldx16] (xq, sx
// unused; FP8 weights).
hipError_t launch_gemm_lora(const uint8_t* xq, const float* sx, int64_t ldq, const uint16_t* x16, int64_t ldx16,
                            int64_t M, int64_t N, int64_t K, const WeightArgs& wt, const AdapterArgs& ad,
                            const float* z, uint16_t* y, int64_t ldy, void* ws, hipStream_t stream);

// The RMS normalization with the quantizer and (when ad.idx is set) the
// shrink from its output.
hipError_t launch_norm_quant_shrink(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                                    float eps, uint16_t* xn, int64_t ldn, uint8_t* xq, int64_t ldq, float* sx,
                                    const AdapterArgs& ad, float* z, void* ws, hipStream_t stream);

// The fused decode path.
// x16: the matched W8A16 GEMM (x stays bf16; xq_out / sx_out unused).
hipError_t launch_decode_lora(const uint16_t* x, int64_t ldx, int64_t M, int64_t N, int64_t K,
                              const WeightArgs& wt, const AdapterArgs& ad, uint16_t* y, int64_t ldy,
                              uint8_t* xq_out, float* sx_out, int64_t ldq_out, void* ws, bool x16,
                              hipStream_t stream);

}  // namespace epilora
