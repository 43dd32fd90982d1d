// Workspace layout and launch-shape rules shared by the host API and the
// kernels.  Host and device code both include this file.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace epilora {

// Control block at the start of every workspace (int32 words).
constexpr size_t kCtrlBytes = 256;
constexpr int kCtrlError = 0;      // device error word (sticky bits)
constexpr int kCtrlAmax = 1;       // 4-bit weight quantizer: global amax bits
constexpr int kCtrlForceTimeout = 2;  // nonzero: the fused path's bounded waits give up at once
constexpr int kCtrlQuantDone = 8;  // fused path: rows quantized
constexpr int kCtrlGemmDone = 10;  // fused path: GEMM workgroups finished

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Counters that must read zero at the start of a call sit at fixed offsets
// right after the control block, whatever the call's shape, so that a
// workspace can serve calls of different shapes: every counter is put back
// to zero by the call that used it, and data regions never overlap them.
//   done sub-counters: the fused path's GEMM workgroups count themselves done
//   in kDoneGroups counters 256 bytes apart (one contended word would
//   serialize hundreds of atomics), then the last of each group in the
//   kCtrlGemmDone word;
//   tile counters: the shrink's per-tile split counters;
//   the fused path's z ([M][r] fp32 words, M <= 64, r <= 128): a word reads
//   zero until its producer stores it, as its bitwise complement, so GEMM
//   workgroups poll z itself; the last of them clears it again.
constexpr int kDoneGroups = 16;
constexpr int kDoneStride = 64;  // int32 words
constexpr size_t kDoneOffset = kCtrlBytes;
constexpr int64_t kMaxShrinkTiles = 4096;  // the shrink takes M <= 65536 per call
constexpr size_t kTileCounterOffset = kDoneOffset + (size_t)kDoneGroups * kDoneStride * 4;
constexpr size_t kZOffset = align256(kTileCounterOffset + 4 * (size_t)kMaxShrinkTiles);
constexpr size_t kZBytes = 64 * 512 * 4;  // M <= 64 tokens, up to 4 slices of rank 128
constexpr size_t kStateBytes = align256(kZOffset + kZBytes);

// ---- shrink -----------------------------------------------------------------
// A workgroup covers 16 consecutive tokens (64 for prefill batches, see
// below) and a range of 128-wide K steps; the K range is split over `splits`
// workgroups whose partial sums are combined in a fixed order by the last one
// to finish.  For 16-token tiles, splits give the chip about 1024 workgroups,
// but no fewer than one (step, rank block) pair per wave of a 4-wave
// workgroup; for 64-token tiles about 512, with at least two steps each (the
// next step's adapter rows load while the current one is multiplied).
constexpr int kShrinkTokens = 16;
constexpr int kShrinkStep = 128;

// Batches of more than kShrinkWideM tokens (prefill) take tiles of
// kShrinkWideTokens tokens whose adapter rows are shared through LDS.
constexpr int kShrinkWideM = 64;
constexpr int kShrinkWideTokens = 64;
inline int shrink_tokens(int64_t M) { return M > kShrinkWideM ? kShrinkWideTokens : kShrinkTokens; }

inline int shrink_splits(int64_t M, int64_t K, int32_t r) {
  const int64_t steps = cdiv(K, kShrinkStep);
  if (M > kShrinkWideM) {  // about 512 workgroups, at least two steps each
    const int64_t tiles = cdiv(M, kShrinkWideTokens);
    int64_t s = cdiv(512, tiles);
    const int64_t two = cdiv(steps, 2);
    if (s > two) s = two;
    if (s < 1) s = 1;
    return (int)s;
  }
  const int64_t tiles = cdiv(M, kShrinkTokens);
  const int64_t jb = r > 16 ? r / 16 : 1;
  int64_t s = steps;
  const int64_t want = cdiv(1024, tiles);
  if (s > want) s = want;
  const int64_t fill = cdiv(steps * jb, 4);
  if (s > fill) s = fill;
  if (s < 1) s = 1;
  return (int)s;
}

struct ShrinkWs {
  size_t counters;  // int32 [tiles], at the fixed tile-counter offset
  size_t partials;  // float [splits][M][r]
  size_t total;
};

// `base`: where the shrink's data region may start (at least kStateBytes).
// r is the slot width of one slice; S slices each keep their own partials.
// The tile counters ([tiles][S] words) hold at most kMaxShrinkTiles.
inline ShrinkWs shrink_ws(size_t base, int64_t M, int64_t K, int32_t r, int32_t S = 1) {
  ShrinkWs w;
  const int s = shrink_splits(M, K, r);
  w.counters = kTileCounterOffset;
  w.partials = align256(base);
  w.total = align256(w.partials + (s > 1 ? (size_t)s * M * r * 4 * S : 0));
  return w;
}

// ---- fused decode path ------------------------------------------------------
struct DecodeWs {
  size_t xq;     // uint8 [M][K] (when the caller keeps no copy)
  size_t sx;     // float [M]
  size_t z;      // float [M][r]
  ShrinkWs shrink;
  size_t total;
};

inline DecodeWs decode_ws(int64_t M, int64_t K, int32_t r, int32_t S = 1) {
  DecodeWs w;
  w.xq = kStateBytes;
  w.sx = align256(w.xq + (size_t)M * K);
  w.z = align256(w.sx + 4 * (size_t)M);
  w.shrink = shrink_ws(align256(w.z + 4 * (size_t)M * r * S), M, K, r, S);
  w.total = w.shrink.total;
  return w;
}

}  // namespace epilora
