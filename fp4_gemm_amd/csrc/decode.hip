// The fused small-batch (decode) path in one persistent launch.
//
// The method launches the down-projection first and the GEMM as its
// programmatic dependent, which waits for the down-projection only before
// its epilogue, so the GEMM's weight streaming overlaps it ("EpiLoRA: Fusing
// Many LoRA Adapters into Low-Precision GEMMs for Serving and RL", Design,
// "Multi-adapter kernels", The decode path; Background, "Programmatic
// dependent launch").  HIP has no programmatic dependent launch, so one grid
// plays both kernels:
//   workgroups [0, M)          quantize one token row each, then count up
//                              the quantized-rows flag (release, agent scope);
//   the next tiles*splits      compute the shrink (bf16 x, fp32 partials,
//                              fixed-order combine) and count up the z flag;
//   the rest                   own 16 weight rows each: wait for the
//                              quantized rows (acquire), stream the weights
//                              through the matrix cores, and wait for z only
//                              before the epilogue.
// Workgroups are dispatched in index order, so the producers are resident
// before any consumer spins; every wait is bounded by a wall-clock limit and
// a timeout raises EPILORA_DEV_WAIT_TIMEOUT instead of hanging.  The last
// GEMM workgroup to finish puts the flags back to zero for the next call.
// The GEMM part runs the same main loop and epilogue code as the skinny GEMM
// kernel, so rows without an adapter are bitwise equal to the base GEMM.
#include "gemm_common.h"
#include "quant_row.h"
#include "shrink_common.h"

namespace epilora {

struct DecodeParams {
  const uint16_t* x;
  int64_t ldx;
  GemmParams g;   // g.xq / g.sx: where the quantized rows go; g.z: ws z
  ShrinkParams s;
  int nq, ns, tiles;
  int64_t wait_ticks;
};

// Thread 0 spins (with s_sleep) until *flag >= target, the limit passes, or
// another workgroup has already timed out (then it gives up at once); the
// verdict is shared through LDS.  Followed by an agent-scope acquire in every
// thread so later loads see the producers' data.
__device__ __forceinline__ bool wait_flag(int* flag, int target, int64_t ticks, int* err, int* verdict) {
  if (threadIdx.x == 0) {
    int ok = 1;
    if (load_acquire(flag) < target) {
      const int64_t start = wall_clock64();
      while (load_acquire(flag) < target) {
        if (wall_clock64() - start > ticks || (load_acquire(err) & EPILORA_DEV_WAIT_TIMEOUT)) {
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    *verdict = ok;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return *verdict != 0;
}

template <int MB, int FMT, int U>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int verdict;
  int* ctrl = p.g.ctrl;
  const int bid = blockIdx.x;

  if (bid < p.nq) {  // ---- quantize one token row
    quant_row(p.x + (int64_t)bid * p.ldx, p.g.K, const_cast<uint8_t*>(p.g.xq) + (int64_t)bid * p.g.ldq,
              const_cast<float*>(p.g.sx) + bid, reinterpret_cast<uint32_t*>(smem));
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) atomic_add_release(ctrl + kCtrlQuantDone, 1);
    return;
  }
  if (bid < p.nq + p.ns) {  // ---- shrink
    const int sb = bid - p.nq;
    const int tile = sb % p.tiles, split = sb / p.tiles;
    int s_begin, s_end;
    shrink_range(p.s, split, s_begin, s_end);
    float* red = reinterpret_cast<float*>(smem);
    shrink_tile(p.s, (int64_t)tile * kShrinkTokens, s_begin, s_end, red, split == 0);
    if (shrink_finish(p.s, tile, split, red)) {
      __threadfence();
      __syncthreads();
      if (threadIdx.x == 0) atomic_add_release(ctrl + kCtrlZDone, 1);
    }
    return;
  }

  // ---- GEMM workgroup
  const int gb = bid - p.nq - p.ns;
  const int64_t n0 = (int64_t)gb * 16;
  float* part = reinterpret_cast<float*>(smem);
  uint2* tbl = reinterpret_cast<uint2*>(smem + 4 * MB * 16 * 16 * sizeof(float));
  TokenSlot* tok = reinterpret_cast<TokenSlot*>(smem + 4 * MB * 16 * 16 * sizeof(float) + 256 * sizeof(uint2));
  if (FMT == EPILORA_W_FP4) build_fold_table(tbl);
  const bool adapters = p.ns > 0;
  for (int t = threadIdx.x; t < MB * 16; t += blockDim.x) {
    int rk = 0;
    const int a = adapters ? resolve_token(t, p.g.M, p.g.ad, ctrl + kCtrlError, gb == 0, rk) : -1;
    tok[t] = TokenSlot{a, rk};
  }
  __syncthreads();

  bool ok = wait_flag(ctrl + kCtrlQuantDone, p.nq, p.wait_ticks, ctrl + kCtrlError, &verdict);
  f32x4 acc[MB];
  if (ok) skinny_mainloop<MB, FMT, U>(p.g, n0, acc, tbl);
  if (ok && adapters) ok = wait_flag(ctrl + kCtrlZDone, p.tiles, p.wait_ticks, ctrl + kCtrlError, &verdict);
  if (ok) {
    skinny_epilogue<MB, FMT>(p.g, n0, acc, part, tok, adapters ? p.g.z : nullptr);
  } else if (threadIdx.x == 0) {
    __hip_atomic_fetch_or(ctrl + kCtrlError, EPILORA_DEV_WAIT_TIMEOUT, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }

  __syncthreads();
  if (threadIdx.x == 0) {
    const int ng = (int)gridDim.x - p.nq - p.ns;
    if (atomic_add_acq_rel(ctrl + kCtrlGemmDone, 1) == ng - 1) {
      store_relaxed(ctrl + kCtrlQuantDone, 0);
      store_relaxed(ctrl + kCtrlZDone, 0);
      store_relaxed(ctrl + kCtrlGemmDone, 0);
    }
  }
}

template <int MB, int FMT, int U>
static void launch_decode(const DecodeParams& p, int ng, hipStream_t stream) {
  const size_t gemm_lds = 4 * MB * 16 * 16 * sizeof(float) + 256 * sizeof(uint2) + MB * 16 * sizeof(TokenSlot);
  const size_t shrink_lds = (size_t)4 * 16 * p.s.ad.r * sizeof(float);
  const size_t lds = gemm_lds > shrink_lds ? gemm_lds : shrink_lds;
  hipLaunchKernelGGL((decode_kernel<MB, FMT, U>), dim3((unsigned)(p.nq + p.ns + ng)), dim3(256), lds, stream, p);
}

template <int FMT>
static void dispatch_decode(const DecodeParams& p, int ng, hipStream_t stream) {
  const int64_t M = p.g.M;
  if (M <= 16) launch_decode<1, FMT, 8>(p, ng, stream);
  else if (M <= 32) launch_decode<2, FMT, 4>(p, ng, stream);
  else if (M <= 48) launch_decode<3, FMT, 2>(p, ng, stream);
  else launch_decode<4, FMT, 2>(p, ng, stream);
}

hipError_t launch_decode_lora(const uint16_t* x, int64_t ldx, int64_t M, int64_t N, int64_t K,
                              const WeightArgs& wt, const AdapterArgs& ad, uint16_t* y, int64_t ldy,
                              uint8_t* xq_out, float* sx_out, int64_t ldq_out, void* ws, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  char* wsb = reinterpret_cast<char*>(ws);
  const DecodeWs lay = decode_ws(M, K, ad.r);
  DecodeParams p;
  p.x = x;
  p.ldx = ldx;
  GemmParams& g = p.g;
  g.xq = xq_out != nullptr ? xq_out : reinterpret_cast<uint8_t*>(wsb + lay.xq);
  g.ldq = xq_out != nullptr ? ldq_out : K;
  g.sx = sx_out != nullptr ? sx_out : reinterpret_cast<float*>(wsb + lay.sx);
  g.M = M; g.N = N; g.K = K;
  g.wt = wt; g.ad = ad;
  g.z = reinterpret_cast<float*>(wsb + lay.z);
  g.y = y; g.ldy = ldy;
  g.ctrl = reinterpret_cast<int*>(ws);
  ShrinkParams& s = p.s;
  s.x = x; s.M = M; s.K = K; s.ldx = ldx; s.ad = ad;
  s.z = reinterpret_cast<float*>(wsb + lay.z);
  s.ctrl = g.ctrl;
  s.counters = reinterpret_cast<int*>(wsb + lay.shrink.counters);
  s.partials = reinterpret_cast<float*>(wsb + lay.shrink.partials);
  s.splits = shrink_splits(M, K);
  p.nq = (int)M;
  p.tiles = (int)cdiv(M, kShrinkTokens);
  p.ns = ad.idx != nullptr ? p.tiles * s.splits : 0;
  p.wait_ticks = 100000000;  // 1 s at the 100 MHz constant wall clock
  const int ng = (int)cdiv(N, 16);
  if (wt.fmt == EPILORA_W_FP8) dispatch_decode<EPILORA_W_FP8>(p, ng, stream);
  else dispatch_decode<EPILORA_W_FP4>(p, ng, stream);
  return hipGetLastError();
}

}  // namespace epilora
