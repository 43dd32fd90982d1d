// Per-token adapter resolution shared by the shrink, the GEMM epilogues and
// the fused path.
#pragma once

#include "../../include/epilora.h"
#include "device.h"
#include "kernels.h"

namespace epilora {

// Resolve token t: returns the adapter slot (or -1) and its rank.  A token is
// adapted when idx[t] is in [0, L), its mask byte (if any) is nonzero and the
// slot's rank (ranks[a] clamped to r, or r) is positive.  An index outside
// [-1, L) counts as -1; when `report` is set it raises the device error bit.
__device__ __forceinline__ int resolve_token(int64_t t, int64_t M, const AdapterArgs& ad, int* err,
                                             bool report, int& rank) {
  rank = 0;
  if (t >= M || ad.idx == nullptr) return -1;
  int a = ad.idx[t];
  if (a < -1 || a >= ad.L) {
    if (report) atomic_or_relaxed(err, EPILORA_DEV_BAD_INDEX);
    return -1;
  }
  if (a < 0) return -1;
  if (ad.mask != nullptr && ad.mask[t] == 0) return -1;
  int rk = ad.ranks != nullptr ? ad.ranks[a] : ad.r;
  rk = rk < ad.r ? rk : ad.r;
  if (rk <= 0) return -1;
  rank = rk;
  return a;
}

}  // namespace epilora
