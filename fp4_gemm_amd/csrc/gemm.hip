// The low-precision GEMM with the multi-adapter epilogue: a skinny
// weight-streaming kernel for decode batches (M <= 64); larger batches
// (prefill) go to the LDS-tiled matrix-core kernel of gemm_wide.hip.
#include "skinny.h"

namespace epilora {

// ---------------------------------------------------------------------------
// Skinny kernel (M <= 64): persistent workgroups over 16-row tiles; see
// skinny.h.
// ---------------------------------------------------------------------------
template <int MB, int FMT, int NW, bool XLDS, bool GEN, bool A16>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(SkinnyJob J) {
  extern __shared__ __align__(16) char lds[];
  Skinny<MB, FMT, NW, XLDS, false, 0, GEN, A16> s(J, lds, blockIdx.x);
  s.run();
}

// ---------------------------------------------------------------------------

template <int MB, int FMT, int NW, bool XLDS, bool GEN, bool A16>
static void launch_skinny_g(SkinnyJob& J, hipStream_t stream) {
  const GemmParams& p = J.g;
  const size_t lds = skinny_lds(p.M, p.K, MB, NW, p.ad.r, false, XLDS, FMT, A16 ? 2 : 1);
  // two or more token blocks without the activations in LDS run batch-major
  // over at most stash_tiles(MB) tiles per workgroup
  const int resident = resident_groups(gemm_skinny_kernel<MB, FMT, NW, XLDS, GEN, A16>, NW * 64, lds);
  J.gwgs = (MB >= 2 && !XLDS && !A16) ? skinny_batch_groups(p.N, MB, resident) : skinny_groups(p.N, resident);
  hipLaunchKernelGGL((gemm_skinny_kernel<MB, FMT, NW, XLDS, GEN, A16>), dim3(J.gwgs), dim3(NW * 64), lds, stream, J);
}

// The W8A16 GEMM and the general adapters (slices, FP8 storage) run in
// kernels of their own.
template <int MB, int FMT, int NW, bool XLDS, bool A16>
static void launch_skinny_x(SkinnyJob& J, hipStream_t stream) {
  const AdapterArgs& ad = J.g.ad;
  if constexpr (A16) {
    launch_skinny_g<MB, FMT, NW, XLDS, true, true>(J, stream);
  } else {
    if (J.g.z != nullptr && (ad.S > 1 || ad.afmt != 0)) launch_skinny_g<MB, FMT, NW, XLDS, true, false>(J, stream);
    else launch_skinny_g<MB, FMT, NW, XLDS, false, false>(J, stream);
  }
}

template <int MB, int FMT, int NW, bool A16>
static void launch_skinny_nw(const GemmParams& p, hipStream_t stream) {
  SkinnyJob J{};
  J.g = p;
  J.tiles = (int)cdiv(p.N, 16);
  if (skinny_x_in_lds(p.M, p.K, MB, NW, p.ad.r, false, FMT, A16 ? 2 : 1)) launch_skinny_x<MB, FMT, NW, true, A16>(J, stream);
  else launch_skinny_x<MB, FMT, NW, false, A16>(J, stream);
}

template <int MB, int FMT, bool A16>
static void launch_skinny(const GemmParams& p, hipStream_t stream) {
  if (skinny_waves(p.N, MB) == 8) launch_skinny_nw<MB, FMT, 8, A16>(p, stream);
  else launch_skinny_nw<MB, FMT, 4, A16>(p, stream);
}

template <int FMT, bool A16>
static void dispatch_gemm(const GemmParams& p, hipStream_t stream) {
  if (p.M <= 16) launch_skinny<1, FMT, A16>(p, stream);
  else if (p.M <= 32) launch_skinny<2, FMT, A16>(p, stream);
  else if (p.M <= 48) launch_skinny<3, FMT, A16>(p, stream);
  else if (p.M <= 64) launch_skinny<4, FMT, A16>(p, stream);
  else launch_gemm_wide(p, stream);
}

hipError_t launch_gemm_lora(const uint8_t* xq, const float* sx, int64_t ldq, const uint16_t* x16, int64_t ldx16,
                            int64_t M, int64_t N, int64_t K, const WeightArgs& wt, const AdapterArgs& ad,
                            const float* z, uint16_t* y, int64_t ldy, void* ws, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmParams p;
  p.xq = xq; p.sx = sx; p.ldq = ldq; p.x16 = x16; p.ldx16 = ldx16; p.M = M; p.N = N; p.K = K;
  p.wt = wt; p.ad = ad; p.z = z; p.y = y; p.ldy = ldy;
  p.ctrl = reinterpret_cast<int*>(ws);
  if (x16 != nullptr) dispatch_gemm<EPILORA_W_FP8, true>(p, stream);
  else if (wt.fmt == EPILORA_W_FP8) dispatch_gemm<EPILORA_W_FP8, false>(p, stream);
  else dispatch_gemm<EPILORA_W_FP4, false>(p, stream);
  return hipGetLastError();
}

}  // namespace epilora
