// Per-row dynamic E4M3 quantization as a workgroup-level device function,
// used by the quantization kernel and by the fused decode path.
#pragma once

#include "device.h"

namespace epilora {

// ---------------------------------------------------------------------------
// Per-row dynamic E4M3.  One workgroup of NT threads per row.  Each thread
// holds up to kRegVecs 16-byte vectors (8 bf16 each) of the row in registers,
// so a row of up to 128 * NT elements is read from HBM once; longer rows are
// read a second time for the encode pass.
// amax: the largest |x| is the largest 15-bit bf16 magnitude, an integer max.
// scale: amax / 448, an IEEE division (built with correctly rounded fp32
// division); 1.0 for an all-zero row.  code: E4M3(RN(x / scale)), the
// quotient rounded exactly as IEEE division rounds it (quot below).
// ---------------------------------------------------------------------------
constexpr int kRegVecs = 16;

__device__ __forceinline__ uint32_t absmax8(const uint4& v) {
  uint32_t m = 0;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return m;
}

// The quotient x / s rounded to nearest even, bit for bit what IEEE division
// gives, for a row scale s > 0 and |x| <= 448 s.  With rs = RN(1/s),
// q0 = RN(x rs) is within one ulp of x / s, the residual x - q0 s is exact
// under a fused multiply-add, and one correction q0 + (x - q0 s) rs rounds to
// the correctly rounded quotient (Markstein's theorem on division with a
// correctly rounded reciprocal).  The theorem needs the residual to stay
// normal: s >= 2^-64 keeps it normal for every |x / s| >= 2^-11, and smaller
// quotients (a +-1 ulp error there) all encode to a signed zero anyway.  A
// row with s < 2^-64 has every |x| <= 448 s < 2^-55, so both x and s are
// multiplied by f = 2^127 first: exact (a power of two, no overflow, and
// subnormals only gain precision), the same real quotient, and a divisor of
// at least 2^-15.  One branch-free sequence thus serves every row.  The sign
// of a zero quotient is x's, as IEEE division gives it.
struct QuotRow {
  float f;   // 1, or 2^127 for a row scale below 2^-64
  float s;   // the row scale times f
  float rs;  // RN(1 / s), an IEEE division once per row
};

__device__ __forceinline__ QuotRow quot_consts(float s) {
  QuotRow q;
  q.f = s >= 0x1p-64f ? 1.0f : 0x1p127f;
  q.s = s * q.f;
  q.rs = 1.0f / q.s;
  return q;
}

__device__ __forceinline__ float quot(float x, const QuotRow& q) {
  const float xs = x * q.f;
  const float q0 = xs * q.rs;
  const float r = fmaf(-q0, q.s, xs);
  return copysignf(fmaf(r, q.rs, q0), x);
}

// Eight bf16 values to E4M3 codes: E4M3(RN(x / s)).  |x / s| <= 448 (1 + 2^-23)
// here, so the hardware conversion (round to nearest even, OCP E4M3FN on this
// target, signed zero kept) never meets its overflow range.
__device__ __forceinline__ uint2 encode8(const uint4& v, const QuotRow& q) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(quot(bf16_lo(w[2 * h]), q), quot(bf16_hi(w[2 * h]), q), 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(quot(bf16_lo(w[2 * h + 1]), q), quot(bf16_hi(w[2 * h + 1]), q), c,
                                        true);
    out[h] = (uint32_t)c;
  }
  return make_uint2(out[0], out[1]);
}

// Block-wide max of a uint32 over NT threads (`red`: NT / 64 words of LDS).
template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t m = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) m = m > red[i] ? m : red[i];
  return m;
}

__device__ __forceinline__ float row_scale(uint32_t amax_bits) {
  const float amax = bf16_to_f32((uint16_t)amax_bits);
  return amax == 0.0f ? 1.0f : amax / 448.0f;
}

// Quantize one row of K bf16 values into E4M3 codes (to byte offset `qoff`
// of buffer `qr`) and its scale (to byte offset `soff` of buffer `sr`), with
// the NT threads of the calling workgroup; stores use cache policy POLICY.
// `red` is NT / 64 words of LDS.  Each thread keeps up to kRegVecs 16-byte
// vectors of the row in registers; a longer row is read twice.
template <int NT, int POLICY>
__device__ __forceinline__ void quant_row(const uint16_t* __restrict__ xrow, int64_t K, __amdgpu_buffer_rsrc_t qr,
                                          uint32_t qoff, __amdgpu_buffer_rsrc_t sr, uint32_t soff, uint32_t* red) {
  const uint4* src = reinterpret_cast<const uint4*>(xrow);
  const int nv = (int)(K / 8);
  const int tid = threadIdx.x;

  uint4 v[kRegVecs];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < kRegVecs; ++i) {
    const int j = tid + i * NT;
    if (j < nv) {
      v[i] = src[j];
      amax = max(amax, absmax8(v[i]));
    }
  }
  for (int j = tid + kRegVecs * NT; j < nv; j += NT) amax = max(amax, absmax8(src[j]));
  amax = block_max_u32<NT>(amax, red);
  const float s = row_scale(amax);
  const QuotRow qc = quot_consts(s);
  if (tid == 0) buf_store4<POLICY>(sr, soff, __float_as_uint(s));
#pragma unroll
  for (int i = 0; i < kRegVecs; ++i) {
    const int j = tid + i * NT;
    if (j < nv) buf_store8<POLICY>(qr, qoff + 8 * j, encode8(v[i], qc));
  }
  for (int j = tid + kRegVecs * NT; j < nv; j += NT) buf_store8<POLICY>(qr, qoff + 8 * j, encode8(src[j], qc));
}

}  // namespace epilora
