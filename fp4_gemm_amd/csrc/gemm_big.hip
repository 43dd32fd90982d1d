// The prefill GEMM without adapters for problems with many 256 x 256 output
// tiles, on the 32 x 32 FP8 matrix cores of gfx950.
//
// One workgroup of 4 waves computes a 256 x 256 tile of Y (tokens x
// outputs), each wave a 128 x 128 quarter held as 4 x 4 accumulator blocks of
// v_mfma_f32_32x32x64_f8f6f4 (256 accumulator registers per lane, one wave
// per SIMD).  A wave's quarter is large so that each operand byte read from
// LDS feeds many MFMA cycles (a 128-deep K step reads 32 KB of fragments per
// wave for 32 MFMAs of 64 cycles), and the tile so that each byte brought
// into LDS feeds twice the MFMA work of a 256 x 128 tile.
//
// K advances in steps of 128, each taken as two halves of 64 (one MFMA
// depth).  Both operand tiles (256 rows of 128 bytes each) are staged in LDS,
// double buffered, each row's 16-byte chunks XOR-swizzled by (row / 2) % 8
// so that the 16 rows a fragment read touches fall in distinct banks.  FP8
// tiles go from memory straight into LDS (buffer loads with the lds bit); the
// fragments of the next half are read from LDS while the current half is
// multiplied (two register sets).  One barrier per step, between its halves:
// it makes step k+1's operands visible and frees step k's buffer, whose next
// contents (step k+2) are requested right after it.  4-bit weights are loaded
// into registers and folded to FP8 bytes (a per-block 8-entry table) as they
// are written to LDS.
//
// Epilogue: (acc * sx_t) * sw_n (or gs * 8), the tile's scales having been
// put in LDS with the first operands; the bf16 tile goes out through LDS as
// full 16-byte row chunks.  With adapters the 256 x 128 kernel runs instead:
// its epilogue needs registers that these accumulators leave no room for.
#include "gemm_common.h"

namespace epilora {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBM = 256, kBN = 256;  // tile
constexpr int kWM = 128, kWN = 128;  // a wave's quarter
constexpr int kStep = 128;
constexpr int kBuf = (kBM + kBN) * kStep;  // one step's operands, 64 KB

// C[32][32] += A[32][64] * B[64][32], E4M3 operands (32 bytes per lane: row
// or column l % 32, K bytes [32 (l / 32), +32)).  Lane l holds C column
// l % 32, rows 8 (e / 4) + 4 (l / 32) + e % 4 for e = 0..15.
__device__ __forceinline__ f32x16 mfma_fp8_32(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 128-byte operand rows; 16-byte chunk c of row r sits at slot c ^ ((r / 2) % 8).
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

}  // namespace

template <int FMT>
__global__ __launch_bounds__(kThreads) void gemm_big_kernel(GemmParams p, int tiles_m, int tiles_n) {
  // Two operand buffers as distinct objects, so that the compiler sees that
  // the loads filling one never alias the fragment reads of the other.  Each
  // holds A ([256][128]) then B ([256][128]); the output quarters of waves
  // 0, 1 go to buf0 and 2, 3 to buf1 at the end.
  __shared__ __align__(16) uint8_t buf0[kBuf];
  __shared__ __align__(16) uint8_t buf1[kBuf];
  __shared__ uint2 tbl[FMT == EPILORA_W_FP4 ? 256 : 1];
  __shared__ float s_xs[kBM], s_ws[kBN];  // the tile's token and output scales

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int l32 = lane & 31, hl = lane >> 5;

  // ---- tile of this workgroup: a contiguous run of tiles per XCD ----------
  const int nt = tiles_m * tiles_n;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int per = nt >> 3, rem = nt & 7;
  const int tile = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
  const int64_t m0 = (int64_t)(tile % tiles_m) * kBM, n0 = (int64_t)(tile / tiles_m) * kBN;
  const int64_t K = p.K;
  if (FMT == EPILORA_W_FP4) build_fold_table(tbl);

  // ---- staging -------------------------------------------------------------
  // One wave instruction fills 8 rows of 128 bytes, lane i the 16 bytes at
  // slot i % 8 of row i / 8, so lane i fetches the chunk the swizzle puts in
  // that slot.  Rows past M or N fall outside the buffer resource and read as
  // zero; chunks past K get an out-of-range offset.
  const int rows_a = (int)(p.M - m0 < kBM ? p.M - m0 : kBM);
  const int rows_b = (int)(p.N - n0 < kBN ? p.N - n0 : kBN);
  const auto rA = make_rsrc(p.xq + m0 * p.ldq, (uint32_t)((rows_a - 1) * p.ldq + K));
  const auto rB = make_rsrc(p.wt.w + n0 * (FMT == EPILORA_W_FP8 ? K : K / 2),
                            (uint32_t)(rows_b * (FMT == EPILORA_W_FP8 ? K : K / 2)));
  const auto rS = make_rsrc(FMT == EPILORA_W_FP4 ? p.wt.bs + n0 * (K / 16) : p.wt.w,
                            FMT == EPILORA_W_FP4 ? (uint32_t)(rows_b * (K / 16)) : 0u);
  const int dma_row = lane >> 3;
  auto dma = [&](__amdgpu_buffer_rsrc_t rsrc, int64_t ld, uint8_t* dst, int kt) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = wave * 8 + q;
      const int row = 8 * j + dma_row;
      const int chunk = (lane & 7) ^ ((row >> 1) & 7);
      const uint32_t k = (uint32_t)kt * kStep + 16u * chunk;
      const uint32_t off = (int64_t)k < K ? (uint32_t)(row * ld) + k : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(dst + j * 1024), 16,
                                               off, 0, 0, 0);
    }
  };
  constexpr int QB4 = kBN * 4 / kThreads;  // 4-bit: 32-code chunks per thread
  uint4 rb[FMT == EPILORA_W_FP4 ? QB4 : 1];
  uint32_t rs[FMT == EPILORA_W_FP4 ? QB4 : 1];
  auto load_b4 = [&](int kt) {
#pragma unroll
    for (int q = 0; q < QB4; ++q) {
      const int row = (tid >> 2) + (kThreads / 4) * q, c = tid & 3;
      const uint32_t k = (uint32_t)kt * kStep + 32u * c;
      const bool ok = (int64_t)k < K;
      rb[q] = buf_load16<kCached>(rB, ok ? (uint32_t)(row * (K / 2)) + k / 2 : kOutOfRange);
      rs[q] = buf_load2<kCached>(rS, ok ? (uint32_t)(row * (K / 16)) + k / 16 : kOutOfRange);
    }
  };
  auto store_b4 = [&](uint8_t* b) {
#pragma unroll
    for (int q = 0; q < QB4; ++q) {
      const int row = (tid >> 2) + (kThreads / 4) * q, c = tid & 3;
      RawW raw;
      raw.a = rb[q];
      raw.b = zero4();
      raw.s = rs[q];
      const i32x8 f = w_frag<EPILORA_W_FP4>(raw, tbl);
      *reinterpret_cast<uint4*>(b + swz(row, 2 * c)) = make_uint4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<uint4*>(b + swz(row, 2 * c + 1)) = make_uint4(f[4], f[5], f[6], f[7]);
    }
  };
  // Request step kt's operands: A (and FP8 B) into buf, 4-bit B into rb/rs.
  auto stage = [&](int kt, uint8_t* buf) {
    dma(rA, p.ldq, buf, kt);
    if (FMT == EPILORA_W_FP8) dma(rB, K, buf + kBM * kStep, kt);
    else load_b4(kt);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // The tile's scales, requested now and put in LDS with the first operands.
  const float pre_xs = m0 + tid < p.M ? p.sx[m0 + tid] : 0.f;
  const float pre_ws = n0 + tid < p.N ? weight_scale<FMT>(p.wt, n0 + tid) : 0.f;

  // Fragments of one half step: lane l reads 32 bytes (chunks c, c + 1, c =
  // 4 h + 2 (l / 32)) of row l % 32 of each 32-row block, for both operands,
  // so the two see the same K positions.
  struct Frags {
    i32x8 a[4], b[4];
  };
  Frags X, Y;
  auto read_block = [&](const uint8_t* buf, int row, int c) {
    return as_i32x8(lds16(buf + swz(row, c)), lds16(buf + swz(row, c + 1)));
  };
  // Multiply one half step from `use`, reading half h of `src` into `nxt`
  // (block i's fragments once block row i of the MFMAs has been issued).
  auto half = [&](const Frags& use, const uint8_t* src, int h, Frags& nxt) {
    const int c = 4 * h + 2 * hl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_fp8_32(use.a[i], use.b[j], acc[i][j]);
      nxt.a[i] = read_block(src, wm * kWM + 32 * i + l32, c);
      nxt.b[i] = read_block(src + kBM * kStep, wn * kWN + 32 * i + l32, c);
    }
  };
  const int nk = (int)cdiv(K, kStep);
  const int nk2 = nk + (nk & 1);
  // Step k: X holds its first half's fragments (from `self`).
  auto step = [&](int k, uint8_t* self, uint8_t* next) {
    half(X, self, 1, Y);
    // 4-bit B of step k+1 (in registers since step k-1) goes into `next`,
    // which no wave reads until after the barrier.
    if (FMT == EPILORA_W_FP4 && k + 1 < nk2) store_b4(next + kBM * kStep);
    wait_all_memory();  // step k+1's operands have landed; self is read
    __syncthreads();
    if (k + 2 < nk2) stage(k + 2, self);
    half(Y, next, 0, X);  // at the last step these reads are never used
  };

  stage(0, buf0);
  if (FMT == EPILORA_W_FP4) {
    __syncthreads();  // the fold table is built
    store_b4(buf0 + kBM * kStep);
  }
  if (nk2 > 1) stage(1, buf1);
  wait_all_memory();
  s_xs[tid] = pre_xs;
  s_ws[tid] = pre_ws;
  __syncthreads();
  {
    const int c = 2 * hl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      X.a[i] = read_block(buf0, wm * kWM + 32 * i + l32, c);
      X.b[i] = read_block(buf0 + kBM * kStep, wn * kWN + 32 * i + l32, c);
    }
  }
  for (int kt = 0; kt < nk2; kt += 2) {
    step(kt, buf0, buf1);
    step(kt + 1, buf1, buf0);
  }
  wait_all_memory();
  __syncthreads();  // every wave is done with the operand buffers

  // ---- epilogue: scales --------------------------------------------------
  // acc[i][j][e]: token m0 + wm*128 + 32 i + 8 (e / 4) + 4 (l / 32) + e % 4,
  //               output n0 + wn*128 + 32 j + l % 32.
  const int64_t tw0 = m0 + wm * kWM, nw0 = n0 + wn * kWN;
  auto trow = [&](int i, int e) { return 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3); };
  {
    float wsc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wsc[j] = s_ws[wn * kWN + 32 * j + l32];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float xs = s_xs[wm * kWM + trow(i, e)];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j][e] = (acc[i][j][e] * xs) * wsc[j];
      }
  }

  // ---- store: each wave's bf16 quarter through LDS as 16-byte row chunks --
  uint16_t* sy = reinterpret_cast<uint16_t*>(wave < 2 ? buf0 : buf1) + (wave & 1) * (kWM * kWN);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = trow(i, e);
#pragma unroll
      for (int j = 0; j < 4; ++j) sy[row * kWN + 32 * j + l32] = (uint16_t)f32_to_bf16(acc[i][j][e]);
    }
  __syncthreads();
  const bool vec = (((uintptr_t)p.y | (uintptr_t)(p.ldy * 2)) & 15) == 0;
  constexpr int CPR = kWN / 8;  // 16-byte chunks per row of the quarter
  for (int e = lane; e < kWM * CPR; e += 64) {
    const int row = e / CPR, c = e % CPR;
    const int64_t t = tw0 + row, n = nw0 + c * 8;
    if (t >= p.M || n >= p.N) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(sy + row * kWN + c * 8);
    uint16_t* dst = p.y + t * p.ldy + n;
    if (vec && n + 8 <= p.N) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      for (int q = 0; q < 8 && n + q < p.N; ++q) dst[q] = (uint16_t)(w[q >> 1] >> (16 * (q & 1)));
    }
  }
}

template <int FMT>
static void launch_big(const GemmParams& p, hipStream_t stream) {
  const int tm = (int)cdiv(p.M, kBM), tn = (int)cdiv(p.N, kBN);
  hipLaunchKernelGGL((gemm_big_kernel<FMT>), dim3(tm * tn), dim3(kThreads), 0, stream, p, tm, tn);
}

bool gemm_big_fits(const GemmParams& p) {
  // Base only, and at least two full rounds of workgroups over the 256
  // compute units, so that a partial last round costs little.
  return p.z == nullptr && p.x16 == nullptr && cdiv(p.M, kBM) * cdiv(p.N, kBN) >= 512;
}

void launch_gemm_big(const GemmParams& p, hipStream_t stream) {
  if (p.wt.fmt == EPILORA_W_FP8) launch_big<EPILORA_W_FP8>(p, stream);
  else launch_big<EPILORA_W_FP4>(p, stream);
}

}  // namespace epilora
