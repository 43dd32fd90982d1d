// The shrink (down-projection z = A[a_t] x_t from the bf16 activations) and
// the separate expand-add kernel of the unfused baseline path.
#include "shrink_common.h"

namespace epilora {

constexpr int kShrinkThreads = 256;

// Decode batches (M <= 64): one workgroup per unit (shrink_unit).
__global__ __launch_bounds__(kShrinkThreads) void shrink_unit_kernel(ShrinkParams p) {
  __shared__ float red[kShrinkWaves * 4];
  shrink_unit<true>(p, (int)blockIdx.x, red);
}

// ---------------------------------------------------------------------------
// Prefill batches (M > 64): a workgroup covers 64 tokens, wave w the tokens
// 16w .. 16w+15 against every rank block, over the range of K steps of its
// split.  For each adapter present in the 64 tokens, the adapter's rows of
// the step (r x 128 bf16) are staged in LDS once for all four waves (the
// next step's rows are loaded into registers while the current step is
// multiplied), and each wave with member tokens multiplies them by its
// tokens' x (other tokens zero) on bf16 MFMA.  Each (token, rank) sum is
// owned by one wave, so the partials need no cross-wave reduction; the
// splits are combined by the last one of the tile in a fixed order
// (shrink_finish), as the normalization kernel's 16-token shrink does.
// ---------------------------------------------------------------------------
constexpr int kWideRows = 128;  // rank rows staged (r <= 128)

// A rows in LDS: [128 ranks][128 K] bf16, 256-byte rows whose 16-byte chunks
// are XOR-swizzled by (row % 16).
__device__ __forceinline__ int swz_a(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

__global__ __launch_bounds__(kShrinkThreads) void shrink_wide_kernel(ShrinkParams p) {
  __shared__ __align__(16) uint8_t sa[kWideRows * 256];
  __shared__ __align__(16) float red[kShrinkWideTokens * kWideRows];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int r = p.ad.r;
  const int64_t K = p.K;
  const int tile = blockIdx.x, split = blockIdx.y, slice = blockIdx.z;
  const int64_t t0 = (int64_t)tile * kShrinkWideTokens;
  int s_begin, s_end;
  shrink_range(p, split, s_begin, s_end);
  int rank_l;  // lane l resolves token t0 + l (the same in every wave)
  const int a_l = resolve_token(t0 + lane, p.M, p.ad, p.ctrl + kCtrlError, split == 0 && slice == 0 && wave == 0, rank_l);

  f32x4 acc[kMaxJB];
#pragma unroll
  for (int j = 0; j < kMaxJB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Staging: 128 rows x 16 chunks = 2048 16-byte chunks, 8 per thread.
  uint4 stg[8];
  // FP8 adapters: 8 codes per chunk, widened to bf16 exactly on the way.
  const bool af8 = p.ad.afmt != 0;
  auto a_load = [&](int64_t aoff, int rank, int s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = tid + i * kShrinkThreads;
      const int row = e >> 4, c = e & 15;
      const int64_t k = (int64_t)s * kShrinkStep + 8 * c;
      const bool ok = row < rank && k < K;
      if (af8) {
        const uint2 q = ok ? *reinterpret_cast<const uint2*>(p.ad.A8() + aoff + (int64_t)row * K + k) : make_uint2(0, 0);
        stg[i] = fp8x8_to_bf16x8(q.x, q.y);
      } else {
        stg[i] = ok ? ld16(p.ad.A + aoff + (int64_t)row * K + k) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto a_store = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = tid + i * kShrinkThreads;
      *reinterpret_cast<uint4*>(sa + swz_a(e >> 4, e & 15)) = stg[i];
    }
  };

  uint64_t pending = __ballot(a_l >= 0);
  while (pending) {
    const int leader = __ffsll((unsigned long long)pending) - 1;
    const int a = __shfl(a_l, leader);
    const int rank = __shfl(rank_l, leader);
    const uint64_t members = __ballot(a_l == a);
    pending &= ~members;
    const int jbn = (rank + 15) >> 4;
    const bool mine = ((members >> (16 * wave)) & 0xFFFFull) != 0;
    const bool member = (members >> (16 * wave + col)) & 1;
    const int64_t Aa = ((int64_t)a * p.ad.S + slice) * r * K;  // element offset of the slot
    const uint16_t* xr = p.x + (t0 + 16 * wave + col) * p.ldx;
    if (s_begin < s_end) a_load(Aa, rank, s_begin);
    for (int s = s_begin; s < s_end; ++s) {
      __syncthreads();  // the previous step's rows are no longer read
      a_store();
      __syncthreads();
      if (s + 1 < s_end) a_load(Aa, rank, s + 1);
      if (mine) {
        const int64_t k = (int64_t)s * kShrinkStep + grp * 32;
        uint4 xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[i] = (member && k + i * 8 < K) ? ld16(xr + k + i * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int jb = 0; jb < kMaxJB; ++jb) {
          if (jb < jbn) {
            const int row = jb * 16 + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint4 av = *reinterpret_cast<const uint4*>(sa + swz_a(row, grp * 4 + i));
              acc[jb] = mfma_bf16_16x16x32(as_bf16x8(av), as_bf16x8(xv[i]), acc[jb]);
            }
          }
        }
      }
    }
  }
  // acc[jb][v] = z[token 16*wave + col][jb*16 + 4*grp + v]
#pragma unroll
  for (int jb = 0; jb < kMaxJB; ++jb)
    if (jb < (r >> 4))
      *reinterpret_cast<float4*>(&red[(16 * wave + col) * r + jb * 16 + 4 * grp]) =
          make_float4(acc[jb][0], acc[jb][1], acc[jb][2], acc[jb][3]);
  __syncthreads();
  shrink_finish<4, kShrinkWideTokens>(p, tile, slice, split, red, __ballot(a_l >= 0));
}

hipError_t launch_shrink(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const AdapterArgs& ad,
                         float* z, void* ws, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const ShrinkWs lay = shrink_ws(kStateBytes, M, K, ad.r, ad.S);
  ShrinkParams p;
  p.x = x; p.M = M; p.K = K; p.ldx = ldx; p.ad = ad; p.z = z;
  p.ctrl = reinterpret_cast<int*>(ws);
  p.counters = reinterpret_cast<int*>(reinterpret_cast<char*>(ws) + lay.counters);
  p.partials = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + lay.partials);
  p.splits = shrink_splits(M, K, ad.r);
  p.zflip = 0u;
  if (M > kShrinkWideM) {
    const dim3 grid((unsigned)cdiv(M, kShrinkWideTokens), (unsigned)p.splits, (unsigned)ad.S);
    hipLaunchKernelGGL(shrink_wide_kernel, grid, dim3(kShrinkThreads), 0, stream, p);
    return hipGetLastError();
  }
  const int64_t units = shrink_units(M, ad.S, ad.r, K);
  hipLaunchKernelGGL(shrink_unit_kernel, dim3((unsigned)units), dim3(kShrinkThreads), 0, stream, p);
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
  const int64_t boff = ((int64_t)a * N + n) * r;  // elements
  const uint16_t* br = ad.B + boff;
  const float* zr = z + t * ad.zld + slice_of(ad, n) * r;
  float acc = 0.f;
  int j = 0;
  for (; j + 8 <= rank; j += 8) {
    uint4 b;
    if (ad.afmt != 0) {
      const uint2 q = *reinterpret_cast<const uint2*>(ad.B8() + boff + j);
      b = fp8x8_to_bf16x8(q.x, q.y);
    } else {
      b = ld16(br + j);
    }
    const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo(w[i]), zr[j + 2 * i], acc);
      acc = fmaf(bf16_hi(w[i]), zr[j + 2 * i + 1], acc);
    }
  }
  for (; j < rank; ++j)
    acc = fmaf(ad.afmt != 0 ? e4m3_decode(ad.B8()[boff + j]) : bf16_to_f32(br[j]), zr[j], acc);
  if (ad.afmt != 0) acc *= ad.sb[(int64_t)a * N + n];  // FP8 adapters: the row scale, once
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
