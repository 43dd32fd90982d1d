// The RMS normalization in front of the query / key / value and gate / up
// projections, with the per-token FP8 quantizer and the shrink taken from
// its output in the same kernel ("EpiLoRA: Fusing Many LoRA Adapters into
// Low-Precision GEMMs for Serving and RL", appendix "Discussion and
// Limitations": computing the down-projection inside the normalization kernel
// that already reads the input hides it for these projections).  The GEMM
// that follows then finds z ready and never waits.
//
// For each token row: ms = mean of x^2 (the exact squares summed in fp64,
// the mean rounded to fp32), inv = 1 / sqrt(ms + eps) in correctly rounded
// fp32, xn_k = bf16(bf16(x_k * inv) * gamma_k).  The quantizer and the shrink
// read xn.
//
// The grid follows the shrink's (units of one token for decode batches,
// 16-token tiles and K splits beyond); each workgroup takes inv of its
// tokens over the whole row (rows are read from L2 again by each workgroup;
// at these sizes a few KB), and the shrink reads the activations normalized
// as they are loaded.  One workgroup per token also writes the normalized
// row (if asked), its E4M3 codes and scale: the same arithmetic as the
// separate quantizer on xn, so the same bits.
#include "quant_row.h"
#include "shrink_common.h"

namespace epilora {

namespace {

constexpr int kNormThreads = 256;

struct NormParams {
  ShrinkParams s;        // s.x: the raw activations; s.ad.idx null: no shrink
  const uint16_t* gamma; // [K]
  float eps;
  uint16_t* xn;          // [M][ldn] or null
  int64_t ldn;
  uint8_t* xq;           // [M][ldq]
  int64_t ldq;
  float* sx;             // [M]
};

// bf16(bf16(x * inv) * gamma) for 8 values.
__device__ __forceinline__ uint4 norm8(const uint4& v, const uint4& g, float inv) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {g.x, g.y, g.z, g.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = f32_to_bf16(bf16_to_f32((uint16_t)f32_to_bf16(bf16_lo(w[i]) * inv)) * bf16_lo(gw[i]));
    const uint32_t hi = f32_to_bf16(bf16_to_f32((uint16_t)f32_to_bf16(bf16_hi(w[i]) * inv)) * bf16_hi(gw[i]));
    o[i] = lo | (hi << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

struct XNorm {
  const uint16_t* gamma;
  const float* inv;  // LDS, per token column of the tile
  __device__ __forceinline__ uint4 operator()(const uint4& v, int64_t k, int col) const {
    return norm8(v, *reinterpret_cast<const uint4*>(gamma + k), inv[col]);
  }
};

// inv of token t (0 past M), taken by one wave: the exact squares summed in
// fp64 per lane over the chunks lane, lane + 64, ..., then a fixed tree.
__device__ __forceinline__ float token_inv(const NormParams& p, int64_t t, int lane) {
  const ShrinkParams& s = p.s;
  const int nv = (int)(s.K / 8);
  double ss = 0.0;
  if (t < s.M) {
    const uint4* row = reinterpret_cast<const uint4*>(s.x + t * s.ldx);
    for (int j = lane; j < nv; j += kWave) {
      const uint4 v = row[j];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double a = bf16_lo(w[i]), b = bf16_hi(w[i]);
        ss += a * a + b * b;  // each square is exact in fp64
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
  const float ms = (float)(ss / (double)s.K);
  return t < s.M ? 1.0f / sqrtf(ms + p.eps) : 0.0f;
}

// Token t's normalized row (if asked), E4M3 codes and scale.  Every thread
// of the block calls it.
__device__ __forceinline__ void write_row(const NormParams& p, int64_t t, float inv, uint32_t* mx) {
  const ShrinkParams& s = p.s;
  const int nv = (int)(s.K / 8);
  const uint4* row = reinterpret_cast<const uint4*>(s.x + t * s.ldx);
  const uint4* g = reinterpret_cast<const uint4*>(p.gamma);
  uint32_t amax = 0;
  for (int j = threadIdx.x; j < nv; j += kNormThreads) {
    const uint4 xn8 = norm8(row[j], g[j], inv);
    if (p.xn != nullptr) *reinterpret_cast<uint4*>(p.xn + t * p.ldn + 8 * j) = xn8;
    amax = max(amax, absmax8(xn8));
  }
  if (p.xq == nullptr) return;  // the normalized rows only (a uniform branch)
  amax = block_max_u32<kNormThreads>(amax, mx);
  const float sc = row_scale(amax);
  const QuotRow qc = quot_consts(sc);
  if (threadIdx.x == 0) p.sx[t] = sc;
  for (int j = threadIdx.x; j < nv; j += kNormThreads)
    *reinterpret_cast<uint2*>(p.xq + t * p.ldq + 8 * j) = encode8(norm8(row[j], g[j], inv), qc);
  __syncthreads();  // mx is reused by the next token
}

// Batches of more than 64 tokens: grid (16-token tiles, K splits, output
// slices), as the 16-token shrink.  Every workgroup first takes inv of its
// 16 tokens over the whole row, then runs the shrink over its K range with
// the activations normalized as they are loaded; the (split 0, slice 0)
// workgroup of a tile also writes the tile's rows.
__global__ __launch_bounds__(kNormThreads) void norm_shrink_kernel(NormParams p) {
  extern __shared__ float red[];  // the shrink's [4 waves][16 tokens][r]
  __shared__ float inv_s[kShrinkTokens];
  __shared__ uint32_t mx[kNormThreads / kWave];
  const ShrinkParams& s = p.s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kShrinkTokens;

  // inv of the tile's tokens: wave w takes tokens 4w .. 4w+3
  for (int u = 0; u < kShrinkTokens / 4; ++u) {
    const int c = wave * (kShrinkTokens / 4) + u;
    const float inv = token_inv(p, t0 + c, lane);
    if (lane == 0) inv_s[c] = inv;
  }
  __syncthreads();

  if (blockIdx.y == 0 && blockIdx.z == 0 && (p.xq != nullptr || p.xn != nullptr))  // the tile's rows
    for (int c = 0; c < kShrinkTokens && t0 + c < s.M; ++c) write_row(p, t0 + c, inv_s[c], mx);

  if (s.ad.idx == nullptr) return;
  int s_begin, s_end;
  shrink_range(s, blockIdx.y, s_begin, s_end);
  const XNorm xt{p.gamma, inv_s};
  const int slice = blockIdx.z;
  const uint64_t active = shrink_tile<4>(s, t0, slice, s_begin, s_end, red, blockIdx.y == 0 && slice == 0, xt);
  shrink_finish<4>(s, blockIdx.x, slice, blockIdx.y, red, active);
}

// Decode batches (M <= 64): one workgroup per shrink unit (token, slice,
// block of rank rows), or per token without adapters.  Wave 0 takes inv of
// the unit's token; the unit with the token's first slice and row block
// also writes its rows; then the unit's shrink reads x normalized on the fly.
__global__ __launch_bounds__(kNormThreads) void norm_unit_kernel(NormParams p) {
  __shared__ float inv_s[1];
  __shared__ uint32_t mx[kNormThreads / kWave];
  __shared__ float red[kShrinkWaves * 4];
  const ShrinkParams& s = p.s;
  const bool shrink = s.ad.idx != nullptr;
  const int unit = (int)blockIdx.x;
  int64_t t = unit;
  bool first = true;
  if (shrink) {
    const int S = s.ad.S, nrb = s.ad.r / shrink_unit_rows(s.M, S, s.ad.r, s.K);
    t = unit / nrb / S;
    first = unit % (nrb * S) == 0;
  }
  if (threadIdx.x < kWave) {
    const float inv = token_inv(p, t, threadIdx.x);
    if (threadIdx.x == 0) inv_s[0] = inv;
  }
  __syncthreads();
  if (first && (p.xq != nullptr || p.xn != nullptr)) write_row(p, t, inv_s[0], mx);
  if (shrink) shrink_unit<true>(s, unit, red, XNorm{p.gamma, inv_s});
}

}  // namespace

hipError_t launch_norm_quant_shrink(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                                    float eps, uint16_t* xn, int64_t ldn, uint8_t* xq, int64_t ldq, float* sx,
                                    const AdapterArgs& ad, float* z, void* ws, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  NormParams p{};
  ShrinkParams& s = p.s;
  s.x = x; s.M = M; s.K = K; s.ldx = ldx; s.ad = ad; s.z = z;
  s.zflip = 0u;
  s.ctrl = reinterpret_cast<int*>(ws);
  const bool shrink = ad.idx != nullptr;
  if (shrink) {
    const ShrinkWs lay = shrink_ws(kStateBytes, M, K, ad.r, ad.S);
    s.counters = reinterpret_cast<int*>(reinterpret_cast<char*>(ws) + lay.counters);
    s.partials = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + lay.partials);
    s.splits = shrink_splits(M, K, ad.r);
  } else {
    s.splits = 1;
  }
  p.gamma = gamma; p.eps = eps; p.xn = xn; p.ldn = ldn; p.xq = xq; p.ldq = ldq; p.sx = sx;
  if (M <= kShrinkWideM) {
    const int64_t units = shrink ? shrink_units(M, ad.S, ad.r, K) : M;
    hipLaunchKernelGGL(norm_unit_kernel, dim3((unsigned)units), dim3(kNormThreads), 0, stream, p);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)cdiv(M, kShrinkTokens), shrink ? (unsigned)s.splits : 1u, shrink ? (unsigned)ad.S : 1u);
  const size_t lds = shrink ? (size_t)kShrinkWaves * 16 * ad.r * sizeof(float) : 0;
  hipLaunchKernelGGL(norm_shrink_kernel, grid, dim3(kNormThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace epilora
