// The low-precision GEMM with the multi-adapter epilogue: a skinny
// weight-streaming kernel for decode batches (M <= 64) and an LDS-tiled
// matrix-core kernel for larger batches (prefill).
#include "skinny.h"

namespace epilora {

// ---------------------------------------------------------------------------
// Skinny kernel (M <= 64): persistent workgroups over 16-row tiles; see
// skinny.h.
// ---------------------------------------------------------------------------
template <int MB, int FMT, int NW, bool XLDS>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(SkinnyJob J) {
  extern __shared__ __align__(16) char lds[];
  Skinny<MB, FMT, NW, XLDS, false> s(J, lds, blockIdx.x);
  s.run();
}

// ---------------------------------------------------------------------------
// Tiled kernel (M > 64).  Workgroup tile 128 tokens x 128 outputs, K steps of
// 128; 4 waves in a 2 x 2 grid, 64 x 64 each (4 x 4 MFMA 16x16x128 blocks).
// Operand tiles are staged in LDS (double buffered, next tile's global loads
// in flight while the current one is multiplied), row-major with 128-byte
// rows whose 16-byte chunks are XOR-swizzled by (row % 8), so that the 8
// rows read by consecutive lanes hit distinct banks.  4-bit weights are
// folded to FP8 when staged, so the inner loop is the same for both formats.
// The epilogue computes the adapter term on bf16 MFMA: z (split into a bf16
// high part and a bf16 remainder) times B[a] for each adapter group present
// in the wave's 64 tokens; tokens outside the group contribute zero columns.
// ---------------------------------------------------------------------------
constexpr int kBM = 128, kBN = 128, kBK = 128;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ uint4 lds16(const uint8_t* base, int off) {
  return *reinterpret_cast<const uint4*>(base + off);
}

// bf16x8 of 8 floats: high parts (upper 16 bits) and rounded remainders.
__device__ __forceinline__ void split_bf16x8(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u0 = __float_as_uint(v[2 * i]) & 0xFFFF0000u;
    const uint32_t u1 = __float_as_uint(v[2 * i + 1]) & 0xFFFF0000u;
    h[i] = (u0 >> 16) | u1;
    l[i] = f32_to_bf16(v[2 * i] - __uint_as_float(u0)) | (f32_to_bf16(v[2 * i + 1] - __uint_as_float(u1)) << 16);
  }
  hi = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
  lo = as_bf16x8(make_uint4(l[0], l[1], l[2], l[3]));
}

template <int FMT>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmParams p) {
  __shared__ __align__(16) uint8_t sA[2][kBM * kBK];
  __shared__ __align__(16) uint8_t sB[2][kBN * kBK];
  __shared__ uint2 tbl[FMT == EPILORA_W_FP4 ? 256 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t tiles_m = cdiv(p.M, kBM);
  const int64_t tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int64_t K = p.K;
  if (FMT == EPILORA_W_FP4) build_fold_table(tbl);

  // Global -> register staging assignment.
  uint4 ra[4];
  RawW rb[FMT == EPILORA_W_FP8 ? 4 : 2];
  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = (tid >> 3) + 32 * q, c = tid & 7;
      const int64_t t = m0 + row, k = k0 + c * 16;
      ra[q] = (t < p.M && k < K) ? *reinterpret_cast<const uint4*>(p.xq + t * p.ldq + k) : zero4();
    }
    if (FMT == EPILORA_W_FP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = (tid >> 3) + 32 * q, c = tid & 7;
        const int64_t n = n0 + row, k = k0 + c * 16;
        rb[q].a = (n < p.N && k < K) ? *reinterpret_cast<const uint4*>(p.wt.w + n * K + k) : zero4();
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = (tid >> 2) + 64 * q, c = tid & 3;
        const int64_t n = n0 + row, k = k0 + c * 32;
        rb[q] = load_w_raw<EPILORA_W_FP4>(p.wt, n, K, k, n < p.N && k < K);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = (tid >> 3) + 32 * q, c = tid & 7;
      *reinterpret_cast<uint4*>(&sA[buf][swz(row, c)]) = ra[q];
    }
    if (FMT == EPILORA_W_FP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = (tid >> 3) + 32 * q, c = tid & 7;
        *reinterpret_cast<uint4*>(&sB[buf][swz(row, c)]) = rb[q].a;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = (tid >> 2) + 64 * q, c = tid & 3;
        const i32x8 f = w_frag<EPILORA_W_FP4>(rb[q], tbl);
        *reinterpret_cast<uint4*>(&sB[buf][swz(row, 2 * c)]) = make_uint4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<uint4*>(&sB[buf][swz(row, 2 * c + 1)]) = make_uint4(f[4], f[5], f[6], f[7]);
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)cdiv(K, kBK);
  if (FMT == EPILORA_W_FP4) __syncthreads();  // fold table ready
  gload(0);
  sstore(0);
  __syncthreads();
  const int c0 = (lane >> 4) * 2;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    i32x8 af[4], bfr[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int row = wm * 64 + tb * 16 + (lane & 15);
      af[tb] = as_i32x8(lds16(sA[cur], swz(row, c0)), lds16(sA[cur], swz(row, c0 + 1)));
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int row = wn * 64 + nb * 16 + (lane & 15);
      bfr[nb] = as_i32x8(lds16(sB[cur], swz(row, c0)), lds16(sB[cur], swz(row, c0 + 1)));
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[tb][nb] = mfma_fp8_16x16x128(af[tb], bfr[nb], acc[tb][nb]);
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue -----------------------------------------------------------
  // acc[tb][nb][v]: token m0 + wm*64 + tb*16 + 4*(lane/16) + v,
  //                 output n0 + wn*64 + nb*16 + lane%16.
  const int64_t tw0 = m0 + wm * 64;
  const int64_t nw0 = n0 + wn * 64;
  float wsc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int64_t n = nw0 + nb * 16 + (lane & 15);
    wsc[nb] = n < p.N ? weight_scale<FMT>(p.wt, n) : 0.f;
  }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t t = tw0 + tb * 16 + 4 * (lane >> 4) + v;
      const float xs = t < p.M ? p.sx[t] : 0.f;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[tb][nb][v] = (acc[tb][nb][v] * xs) * wsc[nb];
    }

  uint64_t active = 0;
  f32x4 lacc[4][4];
  if (p.z != nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) lacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int r = p.ad.r;
    int rank_l;
    const int a_l = resolve_token(tw0 + lane, p.M, p.ad, p.ctrl + kCtrlError, tn == 0 && wn == 0, rank_l);
    active = __ballot(a_l >= 0);
    uint64_t pending = active;
    while (pending) {
      const int leader = __ffsll((unsigned long long)pending) - 1;
      const int a = __shfl(a_l, leader);
      const int rank = __shfl(rank_l, leader);
      const uint64_t members = __ballot(a_l == a);
      pending &= ~members;
      for (int kc = 0; kc * 32 < rank; ++kc) {
        const int j0 = kc * 32 + (lane >> 4) * 8;
        bf16x8 bfrag[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int64_t n = nw0 + nb * 16 + (lane & 15);
          uint4 b = zero4();
          if (n < p.N && j0 < rank) {
            b = *reinterpret_cast<const uint4*>(p.ad.B + ((int64_t)a * p.N + n) * r + j0);
            if (j0 + 8 > rank) {
              uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (j0 + e >= rank) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
              b = make_uint4(w[0], w[1], w[2], w[3]);
            }
          }
          bfrag[nb] = as_bf16x8(b);
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          if (((members >> (tb * 16)) & 0xFFFFull) == 0) continue;
          const int tt = tb * 16 + (lane & 15);
          const bool mem = (members >> tt) & 1;
          float zv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) zv[e] = 0.f;
          if (mem && j0 < rank) {
            const float4* zp = reinterpret_cast<const float4*>(p.z + (tw0 + tt) * r + j0);
            const float4 z0 = zp[0], z1 = zp[1];
            zv[0] = z0.x; zv[1] = z0.y; zv[2] = z0.z; zv[3] = z0.w;
            zv[4] = z1.x; zv[5] = z1.y; zv[6] = z1.z; zv[7] = z1.w;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (j0 + e >= rank) zv[e] = 0.f;
          }
          bf16x8 zh, zl;
          split_bf16x8(zv, zh, zl);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            lacc[tb][nb] = mfma_bf16_16x16x32(zh, bfrag[nb], lacc[tb][nb]);
            lacc[tb][nb] = mfma_bf16_16x16x32(zl, bfrag[nb], lacc[tb][nb]);
          }
        }
      }
    }
  }

#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tt = tb * 16 + 4 * (lane >> 4) + v;
      const int64_t t = tw0 + tt;
      if (t >= p.M) continue;
      const bool act = (active >> tt) & 1;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int64_t n = nw0 + nb * 16 + (lane & 15);
        if (n >= p.N) continue;
        float y = acc[tb][nb][v];
        if (act) y = y + p.ad.scale * lacc[tb][nb][v];
        p.y[t * p.ldy + n] = (uint16_t)f32_to_bf16(y);
      }
    }
}

// ---------------------------------------------------------------------------

template <int MB, int FMT, int NW, bool XLDS>
static void launch_skinny_x(SkinnyJob& J, hipStream_t stream) {
  const GemmParams& p = J.g;
  const size_t lds = skinny_lds(p.M, p.K, MB, NW, p.ad.r, false, XLDS);
  J.gwgs = skinny_groups(p.N, resident_groups(gemm_skinny_kernel<MB, FMT, NW, XLDS>, NW * 64, lds));
  hipLaunchKernelGGL((gemm_skinny_kernel<MB, FMT, NW, XLDS>), dim3(J.gwgs), dim3(NW * 64), lds, stream, J);
}

template <int MB, int FMT, int NW>
static void launch_skinny_nw(const GemmParams& p, hipStream_t stream) {
  SkinnyJob J{};
  J.g = p;
  J.tiles = (int)cdiv(p.N, 16);
  if (skinny_x_in_lds(p.M, p.K, MB, NW, p.ad.r, false)) launch_skinny_x<MB, FMT, NW, true>(J, stream);
  else launch_skinny_x<MB, FMT, NW, false>(J, stream);
}

template <int MB, int FMT>
static void launch_skinny(const GemmParams& p, hipStream_t stream) {
  if (skinny_waves(p.N, MB) == 8) launch_skinny_nw<MB, FMT, 8>(p, stream);
  else launch_skinny_nw<MB, FMT, 4>(p, stream);
}

template <int FMT>
static void dispatch_gemm(const GemmParams& p, hipStream_t stream) {
  if (p.M <= 16) launch_skinny<1, FMT>(p, stream);
  else if (p.M <= 32) launch_skinny<2, FMT>(p, stream);
  else if (p.M <= 48) launch_skinny<3, FMT>(p, stream);
  else if (p.M <= 64) launch_skinny<4, FMT>(p, stream);
  else {
    const unsigned grid = (unsigned)(cdiv(p.M, kBM) * cdiv(p.N, kBN));
    hipLaunchKernelGGL(gemm_tiled_kernel<FMT>, dim3(grid), dim3(256), 0, stream, p);
  }
}

hipError_t launch_gemm_lora(const uint8_t* xq, const float* sx, int64_t ldq, int64_t M, int64_t N, int64_t K,
                            const WeightArgs& wt, const AdapterArgs& ad, const float* z, uint16_t* y,
                            int64_t ldy, void* ws, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmParams p;
  p.xq = xq; p.sx = sx; p.ldq = ldq; p.M = M; p.N = N; p.K = K;
  p.wt = wt; p.ad = ad; p.z = z; p.y = y; p.ldy = ldy;
  p.ctrl = reinterpret_cast<int*>(ws);
  if (wt.fmt == EPILORA_W_FP8) dispatch_gemm<EPILORA_W_FP8>(p, stream);
  else dispatch_gemm<EPILORA_W_FP4>(p, stream);
  return hipGetLastError();
}

}  // namespace epilora
