// Quantization kernels: per-row dynamic E4M3 (activations, and FP8 weights at
// load time), the NVFP4-layout 4-bit weight encoder, and the workspace fill.
#include "device.h"
#include "kernels.h"
#include "quant_row.h"
#include "layout.h"

namespace epilora {

constexpr int kQuantThreads = 256;

__global__ __launch_bounds__(kQuantThreads) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, uint8_t* __restrict__ xq,
    int64_t ldq, float* __restrict__ scale_out) {
  __shared__ uint32_t red[kQuantThreads / kWave];
  const int64_t row = blockIdx.x;
  const auto qr = make_rsrc(xq + row * ldq, (uint32_t)K);
  const auto sr = make_rsrc(scale_out + row, 4u);
  quant_row<kQuantThreads, kCached>(x + row * ldx, K, qr, 0u, sr, 0u, red);
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* xq,
                             int64_t ldq, float* scale, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)M), dim3(kQuantThreads), 0, stream, x, M, K, ldx,
                     xq, ldq, scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 4-bit weights (NVFP4 layout).  Three launches: clear the amax word, the
// global amax (an order-independent integer max), then one thread per block
// of 16 elements encodes its scale and codes.
// ---------------------------------------------------------------------------
__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ w, int64_t n_vec,
                                                   uint32_t* amax_out) {
  __shared__ uint32_t red[4];
  uint32_t m = 0;
  const uint4* src = reinterpret_cast<const uint4*>(w);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n_vec; i += (int64_t)gridDim.x * blockDim.x)
    m = max(m, absmax8(src[i]));
  m = block_max_u32<256>(m, red);
  if (threadIdx.x == 0) atomicMax(amax_out, m);
}

__global__ __launch_bounds__(256) void fp4_encode_kernel(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                         const uint32_t* __restrict__ amax_bits,
                                                         uint8_t* __restrict__ wc, uint8_t* __restrict__ bs,
                                                         float* __restrict__ gs_out) {
  const int64_t nb = K / 16;
  const int64_t total = N * nb;
  const float amax = bf16_to_f32((uint16_t)*amax_bits);
  const float gs = amax == 0.0f ? 1.0f : amax / 2688.0f;
  const float denom = 6.0f * gs;
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < total; b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = b / nb, kb = b % nb;
    const uint4* src = reinterpret_cast<const uint4*>(w + n * K + kb * 16);
    const uint4 v0 = src[0], v1 = src[1];
    const uint32_t m = max(absmax8(v0), absmax8(v1));
    const uint32_t scode = e4m3_encode(bf16_to_f32((uint16_t)m) / denom);
    const float step = e4m3_decode(scode) * gs;
    const uint32_t ww[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t packed[2] = {0, 0};
    if (step != 0.0f) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t c0 = e2m1_encode(bf16_lo(ww[i]) / step);
        const uint32_t c1 = e2m1_encode(bf16_hi(ww[i]) / step);
        packed[i >> 2] |= (c0 | (c1 << 4)) << (8 * (i & 3));
      }
    }
    *reinterpret_cast<uint2*>(wc + n * (K / 2) + kb * 8) = make_uint2(packed[0], packed[1]);
    bs[n * nb + kb] = (uint8_t)scode;
    if (b == 0) *gs_out = gs;
  }
}

hipError_t launch_quant_weight_fp4(const uint16_t* w, int64_t N, int64_t K, uint8_t* wc, uint8_t* bs,
                                   float* gs, void* ws, hipStream_t stream) {
  uint32_t* amax = reinterpret_cast<uint32_t*>(ws) + kCtrlAmax;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, stream, amax, 0u, (int64_t)1);
  const int64_t n_vec = N * K / 8;
  const int64_t blocks = n_vec == 0 ? 1 : (cdiv(n_vec, 256) < 2048 ? cdiv(n_vec, 256) : 2048);
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, n_vec, amax);
  const int64_t total = N * (K / 16);
  const int64_t eb = total == 0 ? 1 : (cdiv(total, 256) < 8192 ? cdiv(total, 256) : 8192);
  hipLaunchKernelGGL(fp4_encode_kernel, dim3((unsigned)eb), dim3(256), 0, stream, w, N, K, amax, wc, bs, gs);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* p, uint32_t v, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = cdiv(n, 256) < 1024 ? cdiv(n, 256) : 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint32_t*>(p), v, n);
  return hipGetLastError();
}

}  // namespace epilora
