// The prefill GEMM (M > 64) with the multi-adapter epilogue, on the FP8
// matrix cores of gfx950.
//
// One workgroup of 4 waves computes a BM x BN tile of Y (tokens x outputs),
// each wave a (BM/2) x (BN/2) quarter held as 16 x 16 accumulator blocks of
// v_mfma_f32_16x16x128_f8f6f4 (up to 8 x 8 blocks: 256 accumulator registers
// per lane, one wave per SIMD).  K advances in steps of 128: both operand
// tiles (BM and BN rows of 128 bytes) are staged in LDS, double buffered,
// each 128-byte row's 16-byte chunks XOR-swizzled by (row % 8) so that the 8
// rows consecutive lanes read fall in distinct banks.  The next step's FP8
// tiles go from memory straight into the other buffer (buffer loads with the
// lds bit) while the current step is multiplied; one barrier per step.
// 4-bit weights are loaded into registers and folded to FP8 bytes (a
// per-block 8-entry table, v_perm_b32) as they are written to LDS, so the
// inner loop is the same for both formats.
//
// Tiles are numbered so that each of the 8 XCDs (workgroups are dispatched to
// them in turn) takes a contiguous run, M-tiles fastest: the workgroups one
// XCD runs together share a few weight tiles in that XCD's L2.
//
// Epilogue: the accumulators are scaled in place, (acc * sx_t) * sw_n (or
// gs * 8).  With adapters, z for the tile's tokens (the columns of the output
// slice the tile lies in, for projections with per-slice adapters) is staged
// in LDS as bf16
// and the distinct adapters of the tile's tokens are taken in turn: every
// 16-token block holding one of the adapter's tokens multiplies z (other
// tokens zero) by the adapter's B rows on bf16 MFMA; only the adapter's own
// tokens then add s * (B z), the other rows get no add at all.  The bf16 tile
// goes out through LDS as full 16-byte row chunks.
#include "gemm_common.h"
#include "occupancy.h"

namespace epilora {

namespace {

constexpr int kWideThreads = 256;
constexpr int kStep = 128;

__device__ __forceinline__ int swz8(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

}  // namespace

// A16: the matched W8A16 GEMM ("EpiLoRA ...", Design, "LoRA RL on the same
// base"): the activations stay bf16 (p.x16).  A K step then covers 64
// elements: 128-byte bf16 activation rows and 64-byte FP8 weight rows (the
// first four chunks of the same swizzled 128-byte LDS rows).  Lane l takes
// the 8 activations of chunk 4h + l/16 and the 8 weights at the same K
// positions for the bf16 MFMA of half h, widening the weights to bf16
// exactly; the accumulators take no activation scale.
template <int FMT, int BM, int BN, bool A16 = false>
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(BM == 128 ? 2 : 1))) void gemm_wide_kernel(GemmParams p, int tiles_m, int tiles_n) {
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 16, TN = WN / 16;
  static_assert(!A16 || FMT == EPILORA_W_FP8, "W8A16 takes FP8 weights");
  constexpr int KE = A16 ? 64 : kStep;  // K elements per step
  // Two operand buffers as distinct objects, so that the compiler sees that
  // the loads filling one never alias the reads of the other (and does not
  // wait for them before those reads).  Each holds A ([BM][128]) then B
  // ([BN][128]).
  // The epilogue reuses them: bf16 z rows (256 bytes per token) in buf0 and
  // NSLOT 32 KB slots of B rows in buf1.  128-row tiles take one slot, so the
  // workgroup holds 64 KB of LDS and two run on a compute unit: one's
  // epilogue (a chain of memory round trips) overlaps the other's main loop.
  constexpr int NSLOT = BM == 128 ? 1 : 2;
  constexpr int kOps = (BM + BN) * kStep;
  constexpr int kBuf0 = kOps > BM * 256 ? kOps : BM * 256;
  constexpr int kBuf = kBuf0 > NSLOT * 32768 ? kBuf0 : NSLOT * 32768;
  static_assert(NSLOT * 32768 <= kBuf && BM * 256 <= kBuf, "epilogue LDS regions");
  __shared__ __align__(16) uint8_t buf0[kBuf];
  __shared__ __align__(16) uint8_t buf1[kBuf];
  __shared__ uint2 tbl[FMT == EPILORA_W_FP4 ? 256 : 1];
  __shared__ TokenSlot tok[BM];
  __shared__ int groups[BM];  // the first token of each distinct adapter
  __shared__ int counts[kWideThreads / 64];
  __shared__ float s_xs[BM], s_ws[BN];  // the tile's token and output scales

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // ---- tile of this workgroup: a contiguous run of tiles per XCD ----------
  // The run is taken in groups of kGroupN output columns: inside a group the
  // column index moves fastest, so the tiles an XCD holds at once share both
  // their activation and their weight blocks in its L2.  (Token blocks
  // moving fastest put every activation block of the problem in flight on
  // each XCD at once, more than its L2 holds; the 2048-token gate_up GEMM
  // with adapters ran 7% slower that way.)
  constexpr int kGroupN = 16;
  const int nt = tiles_m * tiles_n;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int per = nt >> 3, rem = nt & 7;
  const int tile = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
  const int grp = tile / (kGroupN * tiles_m), in_grp = tile % (kGroupN * tiles_m);
  const int cols = tiles_n - grp * kGroupN < kGroupN ? tiles_n - grp * kGroupN : kGroupN;  // of this group
  const int64_t m0 = (int64_t)(in_grp / cols) * BM, n0 = (int64_t)(grp * kGroupN + in_grp % cols) * BN;
  const int64_t K = p.K;
  if (FMT == EPILORA_W_FP4) build_fold_table(tbl);

  // ---- staging -------------------------------------------------------------
  // FP8 operands go straight from memory to LDS (buffer loads with the lds
  // bit): one wave instruction fills 8 rows of 128 bytes, lane i the 16 bytes
  // at slot i % 8 of row i / 8, so lane i fetches chunk (i % 8) ^ (i / 8) of
  // that row to realize the swizzle.  Out-of-range rows fall outside the
  // buffer resource and read as zero; chunks past K get an out-of-range
  // offset.  4-bit weights go through registers and the fold.
  const int rows_a = (int)(p.M - m0 < BM ? p.M - m0 : BM);
  const int rows_b = (int)(p.N - n0 < BN ? p.N - n0 : BN);
  const int64_t lda = A16 ? p.ldx16 * 2 : p.ldq;  // bytes
  const auto rA = A16 ? make_rsrc(p.x16 + m0 * p.ldx16, (uint32_t)(((rows_a - 1) * p.ldx16 + K) * 2))
                      : make_rsrc(p.xq + m0 * p.ldq, (uint32_t)((rows_a - 1) * p.ldq + K));
  const auto rB = make_rsrc(p.wt.w + n0 * (FMT == EPILORA_W_FP8 ? K : K / 2),
                            (uint32_t)(rows_b * (FMT == EPILORA_W_FP8 ? K : K / 2)));
  const auto rS = make_rsrc(FMT == EPILORA_W_FP4 ? p.wt.bs + n0 * (K / 16) : p.wt.w,
                            FMT == EPILORA_W_FP4 ? (uint32_t)(rows_b * (K / 16)) : 0u);
  const int dma_row = lane >> 3, dma_chunk = (lane & 7) ^ (lane >> 3);
  // step_bytes: bytes of a row per K step; row_bytes: bytes of a whole row
  // (chunks at or past it read as zero).
  auto dma = [&](__amdgpu_buffer_rsrc_t rsrc, int64_t ld, int per_wave, uint8_t* dst, int kt, uint32_t step_bytes,
                 int64_t row_bytes) {
    const uint32_t k = (uint32_t)kt * step_bytes + 16u * dma_chunk;
    const bool in = 16u * dma_chunk < step_bytes && (int64_t)k < row_bytes;
#pragma unroll
    for (int q = 0; q < per_wave; ++q) {
      const int j = wave * per_wave + q;
      const uint32_t off = in ? (uint32_t)((8 * j + dma_row) * ld) + k : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(dst + j * 1024), 16,
                                               off, 0, 0, 0);
    }
  };
  constexpr int QB4 = BN * 4 / kWideThreads;  // 4-bit: 32-code chunks per thread
  uint4 rb[FMT == EPILORA_W_FP4 ? QB4 : 1];
  uint32_t rs[FMT == EPILORA_W_FP4 ? QB4 : 1];
  auto load_b4 = [&](int kt) {
#pragma unroll
    for (int q = 0; q < QB4; ++q) {
      const int row = (tid >> 2) + (kWideThreads / 4) * q, c = tid & 3;
      const uint32_t k = (uint32_t)kt * kStep + 32u * c;
      const bool ok = (int64_t)k < K;
      rb[q] = buf_load16<kCached>(rB, ok ? (uint32_t)(row * (K / 2)) + k / 2 : kOutOfRange);
      rs[q] = buf_load2<kCached>(rS, ok ? (uint32_t)(row * (K / 16)) + k / 16 : kOutOfRange);
    }
  };
  auto store_b4 = [&](uint8_t* b) {
#pragma unroll
    for (int q = 0; q < QB4; ++q) {
      const int row = (tid >> 2) + (kWideThreads / 4) * q, c = tid & 3;
      RawW raw;
      raw.a = rb[q];
      raw.b = zero4();
      raw.s = rs[q];
      const i32x8 f = w_frag<EPILORA_W_FP4>(raw, tbl);
      *reinterpret_cast<uint4*>(b + swz8(row, 2 * c)) = make_uint4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<uint4*>(b + swz8(row, 2 * c + 1)) = make_uint4(f[4], f[5], f[6], f[7]);
    }
  };
  auto stage = [&](int kt, uint8_t* buf) {  // request step kt's operands into buf
    dma(rA, lda, BM / 32, buf, kt, kStep, A16 ? 2 * K : K);
    if (FMT == EPILORA_W_FP8) dma(rB, K, BN / 32, buf + BM * kStep, kt, KE, K);
    else load_b4(kt);
  };
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline over K steps, two operand buffers: while step k is
  // multiplied from registers, step k+1's fragments are read from the other
  // buffer and step k+2's operands stream into the buffer step k came from.
  // One barrier per step: it makes step k+1's operands visible and frees the
  // buffer of step k (whose fragments every wave has already read).  The loop
  // body is unrolled twice so that each buffer's role is fixed in the code
  // (the compiler then sees that the fragment reads never alias the incoming
  // operands and does not wait for them); an odd step count is padded with
  // a zero step.  Lane l reads 32 bytes of row l % 16 at K offset 32 * (l / 16)
  // of a step (chunks c0, c0 + 1) for both operands: the two see the same K
  // positions.
  const int c0 = (lane >> 4) * 2;
  // The tile's token indices and mask bytes, requested now and used only by
  // the epilogue (thread t holds token m0 + t).  The loads are unconditional
  // and bounds-checked (past M, without adapters or without a mask they read
  // zero) and nothing tests them before the epilogue: a load under a branch
  // let the compiler test the mask byte at once, which held the operand
  // requests behind it.
  const uint32_t tok_rows = p.z != nullptr ? (uint32_t)rows_a : 0u;
  const auto rI = make_rsrc(p.z != nullptr ? p.ad.idx + m0 : nullptr, 4u * tok_rows);
  const auto rM = make_rsrc(p.ad.mask != nullptr ? p.ad.mask + m0 : nullptr, p.ad.mask != nullptr ? tok_rows : 0u);
  const uint32_t tt0 = tid < BM ? (uint32_t)tid : 0u;
  const int pre_a = (int)buf_load4<kCached>(rI, 4u * tt0);
  const int pre_m = (int)__builtin_amdgcn_raw_buffer_load_b8(rM, tt0, 0, 0);
  const int nk = (int)cdiv(K, KE);
  const int nk2 = nk + (nk & 1);
  i32x8 af[TM], bf[TN];
  // A fragment of a row: FP8, 32 codes (chunks c0, c0 + 1); W8A16, the 8
  // bf16 of chunk g = l / 16 (half 0) and of chunk 4 + g (half 1).
  auto frag_a = [&](const uint8_t* a, int row) {
    if (A16)
      return as_i32x8(*reinterpret_cast<const uint4*>(a + swz8(row, lane >> 4)),
                      *reinterpret_cast<const uint4*>(a + swz8(row, 4 + (lane >> 4))));
    return as_i32x8(*reinterpret_cast<const uint4*>(a + swz8(row, c0)),
                    *reinterpret_cast<const uint4*>(a + swz8(row, c0 + 1)));
  };
  // B fragment: FP8, 32 codes; W8A16, the 8 codes at the A fragment's K
  // positions of each half (bytes 32 h + 8 g), raw in dwords 0..3.
  auto frag_b = [&](const uint8_t* b, int row) {
    if (A16) {
      const int g = lane >> 4;
      const uint2 h0 = *reinterpret_cast<const uint2*>(b + swz8(row, g >> 1) + 8 * (g & 1));
      const uint2 h1 = *reinterpret_cast<const uint2*>(b + swz8(row, 2 + (g >> 1)) + 8 * (g & 1));
      i32x8 f;
      f[0] = (int)h0.x; f[1] = (int)h0.y; f[2] = (int)h1.x; f[3] = (int)h1.y;
      f[4] = f[5] = f[6] = f[7] = 0;
      return f;
    }
    return as_i32x8(*reinterpret_cast<const uint4*>(b + swz8(row, c0)),
                    *reinterpret_cast<const uint4*>(b + swz8(row, c0 + 1)));
  };
  auto read_frags = [&](const uint8_t* buf, i32x8 (&fa)[TM], i32x8 (&fb)[TN]) {
    const uint8_t* a = buf;
    const uint8_t* b = buf + BM * kStep;
#pragma unroll
    for (int nb = 0; nb < TN; ++nb) fb[nb] = frag_b(b, wn * WN + nb * 16 + (lane & 15));
#pragma unroll
    for (int tb = 0; tb < TM; ++tb) fa[tb] = frag_a(a, wm * WM + tb * 16 + (lane & 15));
  };
  // Step k from registers, step k+1's fragments from `next` (when there is a
  // step k+1), step k+2's operands into `self` (when there is one).
  auto step = [&](int k, uint8_t* self, const uint8_t* next) {
    wait_all_memory();  // step k+1's operands have landed
    __syncthreads();
    // Step k+2's requests, then the step's MFMAs with step k+1's A fragments
    // read as each block's registers free up and its B fragments at the end.
    // (At the last step the fragment reads fetch whatever the other buffer
    // holds; they are never used.)
    if (k + 2 < nk2) stage(k + 2, self);
    const uint8_t* na = next;
    const uint8_t* nbp = next + BM * kStep;
    // W8A16: the weights of the step widened once, used by every token block
    uint4 bw[A16 ? TN : 1][2];
    if (A16) {
#pragma unroll
      for (int nb = 0; nb < TN; ++nb)
#pragma unroll
        for (int h = 0; h < 2; ++h) bw[nb][h] = fp8x8_to_bf16x8((uint32_t)bf[nb][2 * h], (uint32_t)bf[nb][2 * h + 1]);
    }
#pragma unroll
    for (int tb = 0; tb < TM; ++tb) {
#pragma unroll
      for (int nb = 0; nb < TN; ++nb) {
        if (A16) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            acc[tb][nb] = mfma_bf16_16x16x32(
                __builtin_bit_cast(bf16x8, u32x4{(uint32_t)af[tb][4 * h], (uint32_t)af[tb][4 * h + 1],
                                                 (uint32_t)af[tb][4 * h + 2], (uint32_t)af[tb][4 * h + 3]}),
                as_bf16x8(bw[nb][h]), acc[tb][nb]);
        } else {
          acc[tb][nb] = mfma_fp8_16x16x128(af[tb], bf[nb], acc[tb][nb]);
        }
      }
      af[tb] = frag_a(na, wm * WM + tb * 16 + (lane & 15));
    }
    i32x8 bn[TN];
#pragma unroll
    for (int nb = 0; nb < TN; ++nb) bn[nb] = frag_b(nbp, wn * WN + nb * 16 + (lane & 15));
#pragma unroll
    for (int nb = 0; nb < TN; ++nb) bf[nb] = bn[nb];
    if (FMT == EPILORA_W_FP4 && k + 2 < nk2) store_b4(self + BM * kStep);
  };

  // The tile's scales, requested now and put in LDS with the first operands.
  float pre_xs = 0.f, pre_ws = 0.f;
  if (tid < BM && m0 + tid < p.M) pre_xs = A16 ? 1.0f : p.sx[m0 + tid];
  if (tid < BN && n0 + tid < p.N) pre_ws = weight_scale<FMT>(p.wt, n0 + tid);
  stage(0, buf0);
  if (FMT == EPILORA_W_FP4) {
    __syncthreads();  // the fold table is built
    store_b4(buf0 + BM * kStep);
  }
  if (nk2 > 1) {
    stage(1, buf1);
    if (FMT == EPILORA_W_FP4) store_b4(buf1 + BM * kStep);
  }
  wait_all_memory();
  if (tid < BM) s_xs[tid] = pre_xs;
  if (tid < BN) s_ws[tid] = pre_ws;
  __syncthreads();
  read_frags(buf0, af, bf);
  for (int kt = 0; kt < nk2; kt += 2) {
    step(kt, buf0, buf1);
    step(kt + 1, buf1, buf0);
  }
  wait_all_memory();
  __syncthreads();  // every wave is done with the operand buffers

  // ---- epilogue: scales --------------------------------------------------
  // acc[tb][nb][v]: token m0 + wm*WM + tb*16 + 4*(lane/16) + v,
  //                 output n0 + wn*WN + nb*16 + lane%16.
  const int64_t tw0 = m0 + wm * WM, nw0 = n0 + wn * WN;
  {
    float wsc[TN];
#pragma unroll
    for (int nb = 0; nb < TN; ++nb) wsc[nb] = s_ws[wn * WN + nb * 16 + (lane & 15)];
#pragma unroll
    for (int tb = 0; tb < TM; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float xs = s_xs[wm * WM + tb * 16 + 4 * (lane >> 4) + v];
#pragma unroll
        for (int nb = 0; nb < TN; ++nb) acc[tb][nb][v] = (acc[tb][nb][v] * xs) * wsc[nb];
      }
  }

  // ---- epilogue: adapters ------------------------------------------------
  // z rows of the tile's tokens are requested into registers first (their
  // latency then overlaps the token bookkeeping and the first adapter's B
  // request), then rounded to bf16 (nearest even) into buf0: 256-byte rows
  // (128 ranks), 16-byte chunks swizzled by (token % 16).
  if (p.z != nullptr) {
    const int r = p.ad.r;
    const bool af8 = p.ad.afmt != 0;
    // The tile's outputs lie inside one output slice (the host requires
    // slice widths that are multiples of the tile width): its z columns.
    const int zsl = slice_of(p.ad, n0);
    constexpr int ZIT = BM * 16 / kWideThreads;  // bf16 chunks (8 ranks) per thread
    constexpr int ZB = ZIT;                      // chunks in flight: all
    float4 zf[ZB][2];
    auto z_load = [&](int i0) {
#pragma unroll
      for (int i = 0; i < ZB; ++i) {
        const int e = tid + (i0 + i) * kWideThreads;
        const int t = e >> 4, cb = e & 15;
        const bool ok = m0 + t < p.M && 8 * cb < r;
        const float4* src = reinterpret_cast<const float4*>(p.z + (m0 + t) * p.ad.zld + zsl * r + 8 * cb);
        zf[i][0] = ok ? src[0] : make_float4(0.f, 0.f, 0.f, 0.f);
        zf[i][1] = ok ? src[1] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    auto z_store = [&](int i0) {
#pragma unroll
      for (int i = 0; i < ZB; ++i) {
        const int e = tid + (i0 + i) * kWideThreads;
        const int t = e >> 4, cb = e & 15;
        const float4 f0 = zf[i][0], f1 = zf[i][1];
        *reinterpret_cast<uint4*>(buf0 + t * 256 + ((cb ^ (t & 15)) << 4)) =
            make_uint4(f32_to_bf16(f0.x) | (f32_to_bf16(f0.y) << 16), f32_to_bf16(f0.z) | (f32_to_bf16(f0.w) << 16),
                       f32_to_bf16(f1.x) | (f32_to_bf16(f1.y) << 16), f32_to_bf16(f1.z) | (f32_to_bf16(f1.w) << 16));
      }
    };
    z_load(0);
    // Resolve the tile's tokens (index and mask were loaded before the main
    // loop), then list the distinct adapters in order of first appearance: a
    // token starting a run of equal adapters is listed unless an earlier
    // token has its adapter (checked 64 tokens at a time by the wave), and a
    // wave-level prefix count places it.
    if (tid < BM) {
      int a = -1, rk = 0;
      if (m0 + tid < p.M) {
        a = pre_a;
        if (a < -1 || a >= p.ad.L) {
          if (n0 == 0) atomic_or_relaxed(p.ctrl + kCtrlError, EPILORA_DEV_BAD_INDEX);
          a = -1;
        }
        if (a >= 0 && p.ad.mask != nullptr && pre_m == 0) a = -1;
        if (a >= 0) {
          rk = p.ad.ranks != nullptr ? p.ad.ranks[a] : r;
          rk = rk < r ? rk : r;
          if (rk <= 0) a = -1, rk = 0;
        }
      }
      tok[tid] = TokenSlot{a, rk};
    }
    __syncthreads();
    bool first = false;
    {
      const int my_a = tid < BM ? tok[tid].a : -1;
      const bool start = my_a >= 0 && (tid == 0 || tok[tid - 1].a != my_a);
      uint64_t cand = __ballot(start);
      while (cand) {
        const int l = __ffsll((unsigned long long)cand) - 1;
        cand &= cand - 1;
        const int t = wave * 64 + l;
        const int ac = __shfl(my_a, l);
        bool dup = false;
        for (int u0 = 0; u0 < t && !dup; u0 += 64) {
          const int u = u0 + lane;
          dup = __ballot(u < t && tok[u].a == ac) != 0;
        }
        if (lane == l) first = !dup;
      }
    }
    const uint64_t fb = __ballot(first);
    if (lane == 0) counts[wave] = __popcll(fb);
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += counts[w];
    if (first) groups[base + __popcll(fb & ((1ull << lane) - 1))] = tid;  // the group's first token
    int ngroups = 0;
    for (int w = 0; w < kWideThreads / 64; ++w) ngroups += counts[w];
    wait_vm_keep<63>();  // the group list is written (z may still be loading)
    lds_barrier();
    // The adapters' B rows, PB output blocks of each wave at a time (a
    // "unit": 128 rows of 256 bytes, 64 per half of the tile's outputs), go
    // to one of two 32 KB slots in buf1 straight from memory; the first unit
    // is requested before z is written to LDS, and each next unit once this
    // unit's fragments are in registers, so it lands while this one is
    // multiplied (z comes from buf0, a separate object, so those accesses
    // need not wait for it).
    constexpr int PB = TN < 4 ? TN : 4;
    constexpr int NPASS = TN / PB;
    const int units = ngroups * NPASS;
    auto b_dma = [&](int u, int slot) {
      const TokenSlot lead = tok[groups[u / NPASS]];
      const int pb = (u % NPASS) * PB;
      // bf16 rows: 16-byte chunk c holds ranks 8c .. 8c+7; FP8 rows: chunk c
      // holds ranks 16c .. 16c+15 (only the first r / 16 chunks are used).
      const int esz = af8 ? 1 : 2, per_chunk = 16 / esz;
      const auto rBa = make_rsrc(reinterpret_cast<const uint8_t*>(p.ad.B) + (int64_t)lead.a * p.N * r * esz,
                                 (uint32_t)(p.N * r * esz));
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = wave * 8 + q;  // 4 rows of 256 bytes per wave instruction
        const int R = 4 * j + (lane >> 4), c = (lane & 15) ^ (R & 15);
        const int64_t n = n0 + (R >> 6) * WN + pb * 16 + (R & 63);
        const uint32_t off = per_chunk * c < lead.rank ? (uint32_t)((n * r + per_chunk * c) * esz) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rBa, (__attribute__((address_space(3))) void*)(buf1 + slot * 32768 + j * 1024), 16, off, 0, 0, 0);
      }
    };
    if (units > 0) b_dma(0, 0);
    z_store(0);
#pragma unroll
    for (int i0 = ZB; i0 < ZIT; i0 += ZB) {
      z_load(i0);
      z_store(i0);
    }
    for (int gi = 0; gi < ngroups; ++gi)
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {  // static, so acc is indexed statically
      const int u = gi * NPASS + pass;
      const int pb = pass * PB;
      wait_all_memory();  // unit u has landed
      __syncthreads();    // ... for every wave, and unit u - 1's slot is free
      const TokenSlot lead = tok[groups[gi]];
      const int a = lead.a, rank = lead.rank;
      const int nch = (rank + 31) / 32;  // 32-rank chunks
      uint8_t* slot = buf1 + (NSLOT == 2 ? (u & 1) : 0) * 32768;
      if (!af8 && (rank & 7)) {  // clear the ranks past the adapter's rank in its partial chunk
        const int cp = rank >> 3;
        for (int R = tid; R < 128; R += kWideThreads) {
          uint16_t* q = reinterpret_cast<uint16_t*>(slot + R * 256 + ((cp ^ (R & 15)) << 4));
          for (int e = rank & 7; e < 8; ++e) q[e] = 0;
        }
        __syncthreads();
      }
      if (af8 && (rank & 15)) {
        const int cp = rank >> 4;
        for (int R = tid; R < 128; R += kWideThreads) {
          uint8_t* q = slot + R * 256 + ((cp ^ (R & 15)) << 4);
          for (int e = rank & 15; e < 16; ++e) q[e] = 0;
        }
        __syncthreads();
      }
      uint4 bfr[PB][4];
      float sbv[PB];  // FP8 adapters: the row scale of this lane's output in each block
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        const int R = wn * 64 + i * 16 + (lane & 15);
        const int64_t n = n0 + wn * WN + (pb + i) * 16 + (lane & 15);
        sbv[i] = (af8 && n < p.N) ? p.ad.sb[(int64_t)a * p.N + n] : 1.0f;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          if (kc >= nch) {
            bfr[i][kc] = zero4();
          } else if (af8) {  // ranks 32 kc + 8 (l / 16) .. + 8: half of a 16-byte chunk, widened
            const int g = lane >> 4;
            const uint2 q = *reinterpret_cast<const uint2*>(slot + R * 256 + (((kc * 2 + (g >> 1)) ^ (R & 15)) << 4) +
                                                            8 * (g & 1));
            bfr[i][kc] = fp8x8_to_bf16x8(q.x, q.y);
          } else {
            bfr[i][kc] = *reinterpret_cast<const uint4*>(slot + R * 256 + (((kc * 4 + (lane >> 4)) ^ (R & 15)) << 4));
          }
        }
      }
      if (u + 1 < units) {
        if (NSLOT == 1) __syncthreads();  // every wave has read the slot
        b_dma(u + 1, NSLOT == 2 ? (u + 1) & 1 : 0);
      }
#pragma unroll
      for (int tb = 0; tb < TM; ++tb) {
        const int tt = wm * WM + tb * 16 + (lane & 15);
        const bool mem = tok[tt].a == a;
        if (__ballot(mem) == 0) continue;
        const uint8_t* zrow = buf0 + tt * 256;
        f32x4 lacc[PB];
#pragma unroll
        for (int i = 0; i < PB; ++i) lacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          if (kc >= nch) break;
          const int j0 = kc * 32 + (lane >> 4) * 8;
          uint4 zq = *reinterpret_cast<const uint4*>(zrow + (((kc * 4 + (lane >> 4)) ^ (tt & 15)) << 4));
          if (!mem || j0 >= rank) {
            zq = zero4();
          } else if (j0 + 8 > rank) {
            uint32_t w[4] = {zq.x, zq.y, zq.z, zq.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (j0 + e >= rank) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
            zq = make_uint4(w[0], w[1], w[2], w[3]);
          }
          const bf16x8 zf = as_bf16x8(zq);
#pragma unroll
          for (int i = 0; i < PB; ++i) lacc[i] = mfma_bf16_16x16x32(zf, as_bf16x8(bfr[i][kc]), lacc[i]);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tr = wm * WM + tb * 16 + 4 * (lane >> 4) + v;
          if (tok[tr].a == a) {
#pragma unroll
            for (int i = 0; i < PB; ++i)
              acc[tb][pb + i][v] = acc[tb][pb + i][v] + p.ad.scale * (af8 ? lacc[i][v] * sbv[i] : lacc[i][v]);
          }
        }
      }
    }
    __syncthreads();  // z is read for the last time; the store below reuses the buffers
  }

  // ---- store: each wave's bf16 quarter through LDS as 16-byte row chunks --
  // Rows of the quarter are WN + 8 elements apart: the four rows one store
  // instruction writes then fall on different banks (at WN = 64 elements,
  // 128 bytes, two of them shared every bank).
  constexpr int SW = WN + 8;
  static_assert(2 * WM * SW * 2 <= kBuf, "store staging");
  uint16_t* sy = reinterpret_cast<uint16_t*>(wave < 2 ? buf0 : buf1) + (wave & 1) * (WM * SW);
#pragma unroll
  for (int tb = 0; tb < TM; ++tb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = tb * 16 + 4 * (lane >> 4) + v;
#pragma unroll
      for (int nb = 0; nb < TN; ++nb) sy[row * SW + nb * 16 + (lane & 15)] = (uint16_t)f32_to_bf16(acc[tb][nb][v]);
    }
  __syncthreads();
  const bool vec = (((uintptr_t)p.y | (uintptr_t)(p.ldy * 2)) & 15) == 0;
  constexpr int CPR = WN / 8;  // 16-byte chunks per row of the quarter
  for (int e = lane; e < WM * CPR; e += 64) {
    const int row = e / CPR, c = e % CPR;
    const int64_t t = tw0 + row, n = nw0 + c * 8;
    if (t >= p.M || n >= p.N) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(sy + row * SW + c * 8);
    uint16_t* dst = p.y + t * p.ldy + n;
    if (vec && n + 8 <= p.N) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      for (int q = 0; q < 8 && n + q < p.N; ++q) dst[q] = (uint16_t)(w[q >> 1] >> (16 * (q & 1)));
    }
  }
}

template <int FMT, int BM, int BN, bool A16 = false>
static void launch_wide(const GemmParams& p, hipStream_t stream) {
  const int tm = (int)cdiv(p.M, BM), tn = (int)cdiv(p.N, BN);
  hipLaunchKernelGGL((gemm_wide_kernel<FMT, BM, BN, A16>), dim3(tm * tn), dim3(kWideThreads), 0, stream, p, tm, tn);
}

// Tile shape: the largest tile that still gives every compute unit a tile
// in the first round; but with adapters, where 256 x 128 tiles would take
// several rounds, 128 x 128 (two workgroups per compute unit hide each
// other's epilogue).
template <int FMT>
static void dispatch_wide(const GemmParams& p, hipStream_t stream) {
  const int64_t cus = device_cus();
  const int64_t wide_tiles = cdiv(p.M, 256) * cdiv(p.N, 128);
  if (wide_tiles >= cus && (p.z == nullptr || wide_tiles <= cus)) launch_wide<FMT, 256, 128>(p, stream);
  else launch_wide<FMT, 128, 128>(p, stream);
}

void launch_gemm_wide(const GemmParams& p, hipStream_t stream) {
  if (p.x16 != nullptr) {  // the W8A16 GEMM: 128 x 128 tiles
    launch_wide<EPILORA_W_FP8, 128, 128, true>(p, stream);
    return;
  }
  if (gemm_big_fits(p)) {
    launch_gemm_big(p, stream);
    return;
  }
  if (p.wt.fmt == EPILORA_W_FP8) dispatch_wide<EPILORA_W_FP8>(p, stream);
  else dispatch_wide<EPILORA_W_FP4>(p, stream);
}

}  // namespace epilora
