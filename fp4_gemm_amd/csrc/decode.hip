// The fused small-batch (decode) path: workspace layout and launch
// parameters (the kernel and its launch shapes are in decode.h).
#include "decode.h"

namespace epilora {

// Shrink workgroups of the fused grid at most (each takes units in turn).
// They are dispatched before the GEMM workgroups; a thousand of them (64
// tokens, K = 29568: one rank row per unit) held the GEMM workgroups back by
// 8 us and crowded them onto fewer compute units, while 64 or fewer left the
// 2048 units of the 8B-shaped down projection at 32 tokens too long in turn.
constexpr int kDecodeShrinkWgs = 256;

hipError_t launch_decode_lora(const uint16_t* x, int64_t ldx, int64_t M, int64_t N, int64_t K,
                              const WeightArgs& wt, const AdapterArgs& ad, uint16_t* y, int64_t ldy,
                              uint8_t* xq_out, float* sx_out, int64_t ldq_out, void* ws, bool x16,
                              hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  char* wsb = reinterpret_cast<char*>(ws);
  const DecodeWs lay = decode_ws(M, K, ad.r, ad.S);
  int* ctrl = reinterpret_cast<int*>(ws);
  DecodeParams p{};
  SkinnyJob& J = p.job;
  GemmParams& g = J.g;
  g.xq = xq_out != nullptr ? xq_out : reinterpret_cast<uint8_t*>(wsb + lay.xq);
  g.ldq = xq_out != nullptr ? ldq_out : K;
  g.sx = sx_out != nullptr ? sx_out : reinterpret_cast<float*>(wsb + lay.sx);
  g.M = M; g.N = N; g.K = K;
  g.x16 = x16 ? x : nullptr;
  g.ldx16 = ldx;
  g.wt = wt; g.ad = ad;
  const bool adapters = ad.idx != nullptr;
  g.z = adapters ? reinterpret_cast<float*>(wsb + kZOffset) : nullptr;
  g.y = y; g.ldy = ldy;
  g.ctrl = ctrl;
  J.tiles = (int)cdiv(N, 16);
  J.x = x;
  J.ldx = ldx;
  J.qflag = ctrl + kCtrlQuantDone;
  J.wait_ticks = 100000000;  // 1 s at the 100 MHz constant wall clock
  ShrinkParams& s = p.s;
  s.x = x; s.M = M; s.K = K; s.ldx = ldx; s.ad = ad;
  s.z = reinterpret_cast<float*>(wsb + kZOffset);
  s.zflip = ~0u;
  s.ctrl = ctrl;
  J.done = reinterpret_cast<int*>(wsb + kDoneOffset);
  s.counters = reinterpret_cast<int*>(wsb + lay.shrink.counters);
  s.partials = reinterpret_cast<float*>(wsb + lay.shrink.partials);
  s.splits = 1;
  p.units = adapters ? (int)shrink_units(M, ad.S, ad.r, K) : 0;
  p.ns = p.units < kDecodeShrinkWgs ? p.units : kDecodeShrinkWgs;
  const bool want_xq = xq_out != nullptr || sx_out != nullptr;
  if (x16) decode_dispatch_a16(p, want_xq, stream);
  else if (wt.fmt == EPILORA_W_FP8) decode_dispatch_fp8(p, want_xq, stream);
  else decode_dispatch_fp4(p, want_xq, stream);
  return hipGetLastError();
}

}  // namespace epilora
