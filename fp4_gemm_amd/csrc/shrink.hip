// The shrink (down-projection z = A[a_t] x_t from the bf16 activations) and
// the separate expand-add kernel of the unfused baseline path.
#include "shrink_common.h"

namespace epilora {

constexpr int kShrinkThreads = 256;

__global__ __launch_bounds__(kShrinkThreads) void shrink_kernel(ShrinkParams p) {
  extern __shared__ float red[];  // [4 waves][16 tokens][r]
  int s_begin, s_end;
  shrink_range(p, blockIdx.y, s_begin, s_end);
  shrink_tile<4>(p, (int64_t)blockIdx.x * kShrinkTokens, s_begin, s_end, red, blockIdx.y == 0);
  shrink_finish<4>(p, blockIdx.x, blockIdx.y, red);
}

hipError_t launch_shrink(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const AdapterArgs& ad,
                         float* z, void* ws, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const ShrinkWs lay = shrink_ws(kStateBytes, M, K, ad.r);
  ShrinkParams p;
  p.x = x; p.M = M; p.K = K; p.ldx = ldx; p.ad = ad; p.z = z;
  p.ctrl = reinterpret_cast<int*>(ws);
  p.counters = reinterpret_cast<int*>(reinterpret_cast<char*>(ws) + lay.counters);
  p.partials = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + lay.partials);
  p.splits = shrink_splits(M, K, ad.r);
  const dim3 grid((unsigned)cdiv(M, kShrinkTokens), (unsigned)p.splits);
  const size_t lds = (size_t)kShrinkWaves * 16 * ad.r * sizeof(float);
  hipLaunchKernelGGL(shrink_kernel, grid, dim3(kShrinkThreads), lds, stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Expand-add (the unfused baseline's separate up-projection): for an active
// token t and output n, y[t][n] = bf16(y[t][n] + s * sum_j B[a][n][j] z[t][j]).
// One thread per output element, fp32 dot over the rank; inactive rows are
// not touched.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void expand_add_kernel(const float* __restrict__ z, int64_t M, int64_t N,
                                                         AdapterArgs ad, uint16_t* __restrict__ y, int64_t ldy,
                                                         int* ctrl) {
  const int64_t t = blockIdx.y;
  int rank;
  const int a = resolve_token(t, M, ad, ctrl + kCtrlError, blockIdx.x == 0 && threadIdx.x == 0, rank);
  if (a < 0) return;
  const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const int r = ad.r;
  const uint16_t* br = ad.B + ((int64_t)a * N + n) * r;
  const float* zr = z + t * r;
  float acc = 0.f;
  int j = 0;
  for (; j + 8 <= rank; j += 8) {
    const uint4 b = ld16(br + j);
    const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo(w[i]), zr[j + 2 * i], acc);
      acc = fmaf(bf16_hi(w[i]), zr[j + 2 * i + 1], acc);
    }
  }
  for (; j < rank; ++j) acc = fmaf(bf16_to_f32(br[j]), zr[j], acc);
  uint16_t* yp = y + t * ldy + n;
  *yp = (uint16_t)f32_to_bf16(bf16_to_f32(*yp) + ad.scale * acc);
}

hipError_t launch_expand_add(const float* z, int64_t M, int64_t N, const AdapterArgs& ad, uint16_t* y,
                             int64_t ldy, void* ws, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv(N, 256), (unsigned)M);
  hipLaunchKernelGGL(expand_add_kernel, grid, dim3(256), 0, stream, z, M, N, ad, y, ldy,
                     reinterpret_cast<int*>(ws));
  return hipGetLastError();
}

}  // namespace epilora
