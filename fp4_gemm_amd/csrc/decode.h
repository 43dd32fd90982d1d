// The fused small-batch (decode) path in one persistent launch (with more
// than 32 tokens, a quantizer launch before it).
//
// The method launches the down-projection first and the GEMM as its
// programmatic dependent, which waits for the down-projection only before
// its epilogue, so the GEMM's weight streaming overlaps it ("EpiLoRA: Fusing
// Many LoRA Adapters into Low-Precision GEMMs for Serving and RL", Design,
// "Multi-adapter kernels", The decode path; Background, "Programmatic
// dependent launch").  HIP has no programmatic dependent launch, so one grid
// plays both kernels:
//   workgroups [0, nq)         quantize one token row each and count up the
//                              quantized-rows flag (nq = 0 when every GEMM
//                              workgroup quantizes the few rows into its own
//                              LDS and the caller keeps no copy, and with
//                              more than 32 tokens, whose rows a quantizer
//                              launch writes beforehand: every GEMM
//                              workgroup reads all M rows, which then go
//                              through its XCD's L2 instead of past it);
//   the next M*S*(r/RW)        compute the shrink, one unit (token, output
//                              slice with its own adapter pair, RW rank
//                              rows) each over the whole of K, and store z
//                              in place, each word as its bitwise
//                              complement into a region that reads zero
//                              until then;
//   the rest                   own 16-row weight tiles: request their first
//                              weight batch, obtain the quantized rows,
//                              stream the weights through the matrix cores
//                              into an LDS stash, and poll z itself (no flag)
//                              only once all their tiles are in, before the
//                              epilogues.
// Data crosses workgroups only through device-coherent stores and loads
// (sc1): z words in place, the quantized rows behind a flag that their
// producer bumps (a relaxed agent-scope atomic) only after its stores have
// completed, so no workgroup has to write back or invalidate its L2.  Workgroups are dispatched in index order, so the
// producers are resident before any consumer spins; every wait is bounded by
// a wall-clock limit and a timeout raises EPILORA_DEV_WAIT_TIMEOUT instead of
// hanging.  Each GEMM workgroup counts itself done as soon as z is in its
// LDS (the atomic's round trip overlaps its epilogues); the last one puts
// the flags back to zero and clears z for the next call.  The quantizer, shrink and GEMM arithmetic is the same code
// as in the separate kernels, with the same summation orders, so every output
// is bitwise equal to the separate quant + shrink + GEMM calls.
#pragma once

#include "quant_row.h"
#include "shrink_common.h"
#include "skinny.h"

namespace epilora {

struct DecodeParams {
  SkinnyJob job;  // job.g.xq / job.g.sx: where the quantized rows go; job.g.z: ws z
  ShrinkParams s;
  int nq, ns;  // quantizing and shrink workgroups
  int units;   // shrink units (shrink_unit), taken by the ns workgroups in turn
  int count_q;  // the GEMM workgroups wait for the quantized rows
};

// A16: the matched W8A16 GEMM (bf16 activations read as they are, no
// quantizing workgroups, no wait for quantized rows).
template <int MB, int FMT, int NW, bool XLDS, int UB = 0, bool GEN = false, bool A16 = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu((XLDS && NW == 8 && !GEN) ? 4 : 2))) void decode_kernel(DecodeParams p) {
  extern __shared__ __align__(16) char smem[];
  const GemmParams& g = p.job.g;
  int* ctrl = g.ctrl;
  const int bid = blockIdx.x;

  if (bid < p.nq) {  // ---- quantize one token row
    const auto qr = make_rsrc(g.xq + (int64_t)bid * g.ldq, (uint32_t)g.K);
    const auto sr = make_rsrc(g.sx + bid, 4u);
    quant_row<NW * 64, kCoherent>(p.job.x + (int64_t)bid * p.job.ldx, g.K, qr, 0u, sr, 0u,
                                  reinterpret_cast<uint32_t*>(smem));
    if (p.count_q) {
      wait_all_memory();
      __syncthreads();
      if (threadIdx.x == 0) atomic_add_relaxed(ctrl + kCtrlQuantDone, 1);
    }
    return;
  }
  if (bid < p.nq + p.ns) {  // ---- shrink: units bid - nq, + ns, ...
    for (int u = bid - p.nq; u < p.units; u += p.ns) {
      if (u != bid - p.nq) __syncthreads();  // the previous unit's sums are read
      shrink_unit<GEN>(p.s, u, reinterpret_cast<float*>(smem));
    }
    return;
  }

  // ---- GEMM workgroup (persistent over its tiles)
  Skinny<MB, FMT, NW, XLDS, true, UB, GEN, A16> sk(p.job, smem, bid - p.nq - p.ns);
  sk.run();
  if (!p.job.flags) return;
  // Count the workgroup done (if the epilogue has not already) and, in the
  // last one, clear z.
  if (sk.done_finish() && p.ns > 0) {
    const int n = (int)(g.M * p.s.ad.zld);
    const auto zr = make_rsrc(g.z, (uint32_t)(n * 4));
    for (int e = 4 * threadIdx.x; e < n; e += 4 * NW * 64) buf_store16<kCoherent>(zr, 4u * e, make_uint4(0u, 0u, 0u, 0u));
  }
}

template <int MB, int FMT, int NW, bool XLDS, int UB, bool GEN, bool A16>
static void launch_decode_u(DecodeParams& p, bool want_xq, hipStream_t stream) {
  const GemmParams& g = p.job.g;
  const int r = p.s.ad.r;
  // Quantized rows: kept in LDS (each GEMM workgroup quantizes them, and M
  // workgroups also write xq_out when the caller asks for it), produced by M
  // workgroups of this grid behind the quantized-rows flag, or (more than 32
  // tokens) by the quantizer kernel launched just before.
  constexpr bool before = !XLDS && !A16 && MB >= kQuantBeforeMB;
  if (before && launch_quant_rows(p.job.x, g.M, g.K, p.job.ldx, const_cast<uint8_t*>(g.xq), g.ldq,
                                  const_cast<float*>(g.sx), stream) != hipSuccess)
    return;
  p.nq = (A16 || before || (XLDS && !want_xq)) ? 0 : (int)g.M;
  p.job.qtarget = (int)g.M;
  p.count_q = (XLDS || A16 || before) ? 0 : 1;
  p.job.flags = p.count_q || p.ns > 0;
  // One-block grids over several output slices keep the z of every slice in
  // LDS at once (the outputs of all tiles then run as one list) when that
  // fits the budget.  The LDS exceeds the shrink's kShrinkWaves * 4 floats.
  p.job.zplanes = 1;
  size_t lds = skinny_lds(g.M, g.K, MB, NW, r, true, XLDS, FMT, A16 ? 2 : 1);
  if (MB == 1 && GEN && p.s.ad.S > 1) {
    const size_t wide = skinny_lds(g.M, g.K, MB, NW, r, true, XLDS, FMT, A16 ? 2 : 1, p.s.ad.S);
    if (wide <= kLdsBudget) {
      p.job.zplanes = p.s.ad.S;
      lds = wide;
    }
  }
  // The quantizing and shrink workgroups are dispatched first and hold their
  // slots only until they finish.
  const int resident = resident_groups(decode_kernel<MB, FMT, NW, XLDS, UB, GEN, A16>, NW * 64, lds);
  p.job.gwgs = (MB >= 2 && !XLDS && !A16) ? skinny_batch_groups(g.N, MB, resident)
                                          : skinny_groups(g.N, resident, StashCfg<MB>::n);
  const unsigned grid = (unsigned)(p.nq + p.ns + p.job.gwgs);
  hipLaunchKernelGGL((decode_kernel<MB, FMT, NW, XLDS, UB, GEN, A16>), dim3(grid), dim3(NW * 64), lds, stream, p);
}

// Single-token-block eight-wave grids over short K and at most 512 tiles
// (the Llama-8B qkv and o projections) stream faster in single-step batches;
// longer streams (gate_up, down) in two-step batches, as measured.
template <int MB, int FMT, int NW, bool XLDS, bool A16>
static void launch_decode_x(DecodeParams& p, bool want_xq, hipStream_t stream) {
  const GemmParams& g = p.job.g;
  // the W8A16 GEMM and the general adapters (slices, FP8 storage) run in
  // kernels of their own
  if constexpr (A16) {
    launch_decode_u<MB, FMT, NW, XLDS, 0, true, true>(p, want_xq, stream);
  } else {
    if (g.ad.idx != nullptr && (g.ad.S > 1 || g.ad.afmt != 0))
      launch_decode_u<MB, FMT, NW, XLDS, 0, true, false>(p, want_xq, stream);
    else if (MB == 1 && NW == 8 && g.K <= 4096 && cdiv(g.N, 16) <= 512)
      launch_decode_u<MB, FMT, NW, XLDS, 1, false, false>(p, want_xq, stream);
    else
      launch_decode_u<MB, FMT, NW, XLDS, 0, false, false>(p, want_xq, stream);
  }
}

template <int MB, int FMT, bool A16>
static void launch_decode_nw(DecodeParams& p, bool want_xq, hipStream_t stream) {
  const GemmParams& g = p.job.g;
  // Eight-wave workgroups for up to 32 tokens whatever N (each tile's K then
  // splits over eight waves, and a workgroup takes more, shorter tiles): the
  // fused Llama-8B gate_up projection measured 2 us faster per launch than
  // with four-wave workgroups, which the unfused skinny kernel keeps for
  // large N.
  // The activations sit in LDS only for up to kSelfQuantMaxM tokens, so only
  // the one-block variants have that form.
  constexpr int xb = A16 ? 2 : 1;
  constexpr int NW = MB <= 2 ? 8 : 4;
  // Two token blocks over more than four tiles per compute unit: eight-wave
  // workgroups of four tiles (one per compute unit) would take two rounds,
  // four-wave ones (two per compute unit) take one (the 8B-shaped gate_up
  // projection at 32 tokens: 80 -> 73 us).
  if constexpr (MB == 2 && !A16) {
    if (cdiv(g.N, 16) > 4 * device_cus()) {
      launch_decode_x<MB, FMT, 4, false, A16>(p, want_xq, stream);
      return;
    }
  }
  if constexpr (MB == 1) {
    if (skinny_x_in_lds(g.M, g.K, MB, NW, p.s.ad.r, true, FMT, xb)) {
      launch_decode_x<MB, FMT, NW, true, A16>(p, want_xq, stream);
      return;
    }
  }
  launch_decode_x<MB, FMT, NW, false, A16>(p, want_xq, stream);
}

template <int FMT, bool A16>
static void dispatch_decode(DecodeParams& p, bool want_xq, hipStream_t stream) {
  const int64_t M = p.job.g.M;
  if (M <= 16) launch_decode_nw<1, FMT, A16>(p, want_xq, stream);
  else if (M <= 32) launch_decode_nw<2, FMT, A16>(p, want_xq, stream);
  else if (M <= 48) launch_decode_nw<3, FMT, A16>(p, want_xq, stream);
  else launch_decode_nw<4, FMT, A16>(p, want_xq, stream);
}

// One translation unit per weight and activation format (they compile in
// parallel): decode_fp8.hip, decode_fp4.hip, decode_a16.hip.
void decode_dispatch_fp8(DecodeParams& p, bool want_xq, hipStream_t stream);
void decode_dispatch_fp4(DecodeParams& p, bool want_xq, hipStream_t stream);
void decode_dispatch_a16(DecodeParams& p, bool want_xq, hipStream_t stream);

}  // namespace epilora
