// Device-side helpers shared by the gfx950 kernels: number formats, wave
// reductions, matrix-core wrappers and agent-scope flags.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace epilora {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// FP8 E4M3FN (OCP): bias 7, 3 mantissa bits, max 448, S.1111.111 = NaN
// ---------------------------------------------------------------------------

// fp32 -> E4M3 code: nearest, ties to even, |q| >= 448 saturates to 448, the
// sign is kept (-0 -> 0x80).  Pure integer/exact arithmetic.
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {          // |q| >= 448 (or NaN): saturate
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {    // |q| < 2^-6: subnormal grid, step 2^-9
    // the scaling by 2^9 is exact; rint rounds to nearest even
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {                         // normal: keep 3 of the 23 mantissa bits
    const uint32_t mant = a & 0x7FFFFFu;
    code = (((a >> 23) - 120u) << 3) | (mant >> 20);
    const uint32_t rem = mant & 0xFFFFFu;
    code += (rem > 0x80000u) || (rem == 0x80000u && (code & 1u));
  }
  return code | sign;
}

// E4M3 code -> fp32 (exact).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 0x7u;
  if (e == 0xFu && m == 0x7u) return __uint_as_float(0x7FC00000u);
  if (e == 0) return __uint_as_float(s | __float_as_uint((float)m * 0.001953125f));
  return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

// Two E4M3 codes (bytes 0, 1 of w, or 2, 3 with HI) -> two bf16 in one dword,
// the lower byte in the low half.  The hardware conversion to fp32 is exact
// and every E4M3 value has at most 4 significant bits, so the upper half of
// each fp32 is the exact bf16.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return (__float_as_uint(f.x) >> 16) | (__float_as_uint(f.y) & 0xFFFF0000u);
}
// Eight E4M3 codes (element order in lo, then hi) -> eight bf16.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return make_uint4(fp8x2_to_bf16x2<false>(lo), fp8x2_to_bf16x2<true>(lo), fp8x2_to_bf16x2<false>(hi),
                    fp8x2_to_bf16x2<true>(hi));
}

// E2M1 magnitude code (0..7) -> fp32.
__device__ __forceinline__ float e2m1_magnitude(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  if (e == 0) return m ? 0.5f : 0.0f;
  return __uint_as_float(((e + 126u) << 23) | (m << 22));
}

// fp32 -> E2M1 code: nearest, ties to the even code, saturated at 6.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const float a = fabsf(v);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return c | ((__float_as_uint(v) >> 28) & 0x8u);
}

// One entry of the fold table: the FP8 byte that a 4-bit magnitude code c
// (0..7) becomes under block scale b: E4M3(e2m1(c) * e4m3(b) / 8).  The
// product is exact in fp32; only the encode rounds.  NaN scales give 0x7F.
__device__ __forceinline__ uint32_t fold_entry(uint32_t c, uint32_t b) {
  if ((b & 0x7Fu) == 0x7Fu) return 0x7Fu;
  return e4m3_encode(e2m1_magnitude(c) * e4m3_decode(b) * 0.125f);
}

// Decode 8 packed E2M1 codes (one dword, element 0 in the low nibble) into 8
// FP8 bytes, in element order, given the 8-entry magnitude table of their
// block (tlo: codes 0..3, thi: codes 4..7).  The sign nibble bit flips the
// sign bit of the looked-up byte.
__device__ __forceinline__ void fold8(uint32_t d, uint32_t tlo, uint32_t thi,
                                      uint32_t& out0, uint32_t& out1) {
  const uint32_t sel_even = d & 0x07070707u;
  const uint32_t sel_odd = (d >> 4) & 0x07070707u;
  const uint32_t even = __builtin_amdgcn_perm(thi, tlo, sel_even) ^ ((d & 0x08080808u) << 4);
  const uint32_t odd = __builtin_amdgcn_perm(thi, tlo, sel_odd) ^ (d & 0x80808080u);
  out0 = __builtin_amdgcn_perm(odd, even, 0x05010400u);  // e0 e1 e2 e3
  out1 = __builtin_amdgcn_perm(odd, even, 0x07030602u);  // e4 e5 e6 e7
}

// ---------------------------------------------------------------------------
// Reductions
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
    v = v > o ? v : o;
  }
  return v;
}

// A lane's value moved by one DPP control (0xB1 swaps neighbours, 0x4E
// swaps pairs, 0x141 mirrors each half row, 0x140 each row of 16 lanes), no
// LDS; the epilogues' fixed reduction trees are built from these.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// ---------------------------------------------------------------------------
// Matrix cores
// ---------------------------------------------------------------------------

// C[16][16] += A[16][128] * B[128][16], both operands E4M3 (32 bytes per
// lane).  Zero scale operands select the unscaled instruction.
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// C[16][16] += A[16][32] * B[32][16], bf16 operands (8 per lane).
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ i32x8 as_i32x8(const uint4& lo, const uint4& hi) {
  i32x8 r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// ---------------------------------------------------------------------------
// Buffer loads and stores.  A raw buffer resource returns 0 for any access
// at or past its byte size, which serves as the bounds check.  Cache policy
// kCoherent (sc1) makes an access device-coherent: a store writes through to
// the point of coherence shared by all XCDs and a load reads from it, so
// data handed between workgroups of one grid needs no L2-wide writeback or
// invalidate.
// ---------------------------------------------------------------------------
constexpr int kCached = 0;
constexpr int kCoherent = 16;
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past any buffer this library builds

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int POLICY>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int POLICY>
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POLICY);
}
template <int POLICY>
__device__ __forceinline__ uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, POLICY);
}
template <int POLICY>
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, off, 0, POLICY);
}
template <int POLICY>
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint2& v) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, off, 0, POLICY);
}
template <int POLICY>
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, POLICY);
}

// Native-vector forms for hot loops (the union-based HIP vector types do not
// always stay in registers).
template <int POLICY>
__device__ __forceinline__ u32x4 bufv_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY);
}
__device__ __forceinline__ i32x8 cat8(const u32x4& lo, const u32x4& hi) {
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Wait until every memory access this wave issued has completed.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N vector-memory operations of this wave are still
// outstanding (they complete in issue order) and every LDS operation has
// completed.  s_waitcnt fields: vmcnt bits [3:0] and [15:14], expcnt [6:4]
// (7: no wait), lgkmcnt [11:8] (0: wait for all).
template <int N>
__device__ __forceinline__ void wait_vm_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without the memory fence of __syncthreads (which waits
// for every outstanding memory operation, loads into LDS included).  LDS
// accesses are ordered by it as long as each wave has waited for its own
// (lgkmcnt, and vmcnt for loads into LDS) before it; the empty asm keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Agent-scope counters and flags (visible across the chip's XCDs)
// ---------------------------------------------------------------------------

__device__ __forceinline__ void store_relaxed(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_or_relaxed(int* p, int v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int atomic_add_relaxed(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A device-coherent read of a flag word, without acquire side effects.
__device__ __forceinline__ int load_relaxed(int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace epilora
