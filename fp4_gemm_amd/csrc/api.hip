// The C ABI (include/epilora.h): host-side validation, workspace sizing and
// dispatch to the kernels.  No entry point allocates memory or synchronizes
// the stream, except the diagnostic epilora_device_error.
#include <atomic>
#include <climits>
#include <cmath>

#include "../../include/epilora.h"
#include "kernels.h"
#include "layout.h"

using namespace epilora;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? EPILORA_OK : EPILORA_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Checks shared by the quantizers: sizes, pointers, alignment.
int check_rows(const void* src, int64_t rows, int64_t K, int64_t ld_src, const void* dst, int64_t ld_dst,
               const void* scale) {
  if (rows < 0 || K < 0) return EPILORA_ERR_INVALID_ARG;
  if (rows == 0) return EPILORA_OK;
  if (src == nullptr || dst == nullptr || scale == nullptr) return EPILORA_ERR_INVALID_ARG;
  if (ld_src < K || ld_dst < K) return EPILORA_ERR_INVALID_ARG;
  if (K % 16 != 0 || ld_src % 16 != 0 || ld_dst % 16 != 0) return EPILORA_ERR_UNSUPPORTED;
  if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(scale, 4)) return EPILORA_ERR_UNSUPPORTED;
  return EPILORA_OK;
}

// Adapter arguments: slot geometry and pointers (A only where needed).
int check_adapters(int32_t L, int32_t r, const void* A, bool need_A, const void* B, bool need_B,
                   const int32_t* ranks, const int32_t* idx) {
  if (L < 0 || r <= 0 || idx == nullptr) return EPILORA_ERR_INVALID_ARG;
  if (r > EPILORA_MAX_RANK || r % 16 != 0) return EPILORA_ERR_UNSUPPORTED;
  if (L > 0 && ((need_A && A == nullptr) || (need_B && B == nullptr))) return EPILORA_ERR_INVALID_ARG;
  if ((A && !aligned(A, 16)) || (B && !aligned(B, 16)) || !aligned(idx, 4) || (ranks && !aligned(ranks, 4)))
    return EPILORA_ERR_UNSUPPORTED;
  return EPILORA_OK;
}

int check_ws(const void* ws, size_t have, size_t need) {
  if (ws == nullptr || have < need) return EPILORA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return EPILORA_ERR_UNSUPPORTED;
  return EPILORA_OK;
}

int check_weights(const epilora_layer_args* a) {
  if (a->w == nullptr) return EPILORA_ERR_INVALID_ARG;
  if (a->wfmt == EPILORA_W_FP8) {
    if (a->sw == nullptr) return EPILORA_ERR_INVALID_ARG;
    if (!aligned(a->w, 16) || !aligned(a->sw, 4)) return EPILORA_ERR_UNSUPPORTED;
  } else if (a->wfmt == EPILORA_W_FP4) {
    if (a->bs == nullptr || a->gs == nullptr) return EPILORA_ERR_INVALID_ARG;
    if (!aligned(a->w, 16) || !aligned(a->bs, 2) || !aligned(a->gs, 4)) return EPILORA_ERR_UNSUPPORTED;
  } else {
    return EPILORA_ERR_INVALID_ARG;
  }
  if (a->K % 32 != 0) return EPILORA_ERR_UNSUPPORTED;
  return EPILORA_OK;
}

WeightArgs weights_of(const epilora_layer_args* a) {
  WeightArgs w;
  w.fmt = a->wfmt; w.w = a->w; w.sw = a->sw; w.bs = a->bs; w.gs = a->gs;
  return w;
}

// Output slices with their own adapter pairs: nslices in [0, kMaxSlices]
// (0 and 1 mean one slice), widths positive and summing to N, each a
// multiple of `unit` (the output tile the kernels keep inside one slice).
int check_slices(int32_t nslices, const int64_t* slice_n, int64_t N, int64_t unit) {
  if (nslices < 0 || nslices > kMaxSlices) return EPILORA_ERR_INVALID_ARG;
  if (nslices <= 1) return EPILORA_OK;
  if (slice_n == nullptr) return EPILORA_ERR_INVALID_ARG;
  int64_t sum = 0;
  for (int i = 0; i < nslices; ++i) {
    if (slice_n[i] <= 0) return EPILORA_ERR_INVALID_ARG;
    if (slice_n[i] % unit != 0) return EPILORA_ERR_UNSUPPORTED;
    sum += slice_n[i];
  }
  return sum == N ? EPILORA_OK : EPILORA_ERR_INVALID_ARG;
}

void set_slices(AdapterArgs& d, int32_t nslices, const int64_t* slice_n) {
  d.S = nslices > 1 ? nslices : 1;
  d.zld = d.S * d.r;
  int64_t end = 0;
  for (int i = 0; i < kMaxSlices; ++i) {
    end += (i < d.S && d.S > 1) ? slice_n[i] : 0;
    d.slice_end[i] = i < d.S - 1 ? end : INT64_MAX;
  }
}

AdapterArgs adapters_of(const epilora_layer_args* a, bool on) {
  AdapterArgs d;
  d.A = a->A; d.B = a->B; d.ranks = a->ranks; d.mask = a->mask;
  d.idx = on ? a->idx : nullptr;
  d.L = a->L; d.r = a->r; d.scale = a->scale;
  if (!on) { d.r = 16; d.L = 0; }
  set_slices(d, on ? a->nslices : 1, a->slice_n);
  d.afmt = on ? a->afmt : EPILORA_A_BF16;
  d.sa = a->sa; d.sb = a->sb;
  return d;
}

// Adapter storage: bf16, or FP8 codes with row scales (sa for A where A is
// read, sb for B where B is read; 16-byte aligned).
int check_afmt(int32_t afmt, const float* sa, bool need_sa, const float* sb, bool need_sb) {
  if (afmt == EPILORA_A_BF16) return EPILORA_OK;
  if (afmt != EPILORA_A_FP8) return EPILORA_ERR_INVALID_ARG;
  if ((need_sa && sa == nullptr) || (need_sb && sb == nullptr)) return EPILORA_ERR_INVALID_ARG;
  if ((sa && !aligned(sa, 16)) || (sb && !aligned(sb, 16))) return EPILORA_ERR_UNSUPPORTED;
  return EPILORA_OK;
}

int32_t slices_of(const epilora_layer_args* a) { return a->nslices > 1 ? a->nslices : 1; }

// Host-side checks of a fused decode call (everything except the
// workspace); `r` receives the slot width the workspace is sized for.
int check_decode(const epilora_layer_args* a, int32_t& r) {
  if (a->M < 0 || a->N < 0 || a->K < 0) return EPILORA_ERR_INVALID_ARG;
  if (a->amode != EPILORA_ACT_FP8 && a->amode != EPILORA_ACT_BF16) return EPILORA_ERR_INVALID_ARG;
  if (a->amode == EPILORA_ACT_BF16 && (a->xq_out != nullptr || a->sx_out != nullptr)) return EPILORA_ERR_INVALID_ARG;
  if (a->M == 0 || a->N == 0) return EPILORA_OK;
  if (a->M > EPILORA_DECODE_MAX_M) return EPILORA_ERR_UNSUPPORTED;
  if (a->x == nullptr || a->y == nullptr) return EPILORA_ERR_INVALID_ARG;
  int st = check_weights(a);
  if (st != EPILORA_OK) return st;
  if (a->amode == EPILORA_ACT_BF16 && a->wfmt != EPILORA_W_FP8) return EPILORA_ERR_UNSUPPORTED;
  if (a->ldx < a->K || a->ldy < a->N) return EPILORA_ERR_INVALID_ARG;
  if (a->ldx % 16 != 0 || !aligned(a->x, 16) || !aligned(a->y, 2)) return EPILORA_ERR_UNSUPPORTED;
  if (a->xq_out != nullptr) {
    if (a->ldq_out < a->K) return EPILORA_ERR_INVALID_ARG;
    if (a->ldq_out % 16 != 0 || !aligned(a->xq_out, 16)) return EPILORA_ERR_UNSUPPORTED;
  }
  if (a->sx_out != nullptr && !aligned(a->sx_out, 4)) return EPILORA_ERR_UNSUPPORTED;
  r = 16;
  if (a->idx != nullptr) {
    st = check_adapters(a->L, a->r, a->A, true, a->B, true, a->ranks, a->idx);
    if (st != EPILORA_OK) return st;
    st = check_slices(a->nslices, a->slice_n, a->N, 16);
    if (st != EPILORA_OK) return st;
    st = check_afmt(a->afmt, a->sa, true, a->sb, true);
    if (st != EPILORA_OK) return st;
    r = a->r;
  }
  return EPILORA_OK;
}

// Workspace bytes of a fused decode call that passed check_decode.
size_t decode_need(const epilora_layer_args* a, int32_t r) {
  return decode_ws(a->M, a->K, r, a->idx != nullptr ? slices_of(a) : 1).total;
}

// ---- the fixed scratch of epilora_decode_lora_noalloc ------------------------
// One array per GPU, for the life of the process.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address on each
// GPU comes from hipGetSymbolAddress (with that GPU current) and only that
// address is ever passed to kernels or fill launches.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

int scratch_of_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EPILORA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return EPILORA_ERR_UNSUPPORTED;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {  // first call on this device: look the address up once
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return EPILORA_ERR_HIP;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return EPILORA_OK;
}

}  // namespace

extern "C" {

int epilora_version(void) { return EPILORA_VERSION; }

const char* epilora_strerror(int status) {
  switch (status) {
    case EPILORA_OK: return "ok";
    case EPILORA_ERR_INVALID_ARG: return "invalid argument";
    case EPILORA_ERR_UNSUPPORTED: return "unsupported shape, alignment or batch size";
    case EPILORA_ERR_WORKSPACE: return "workspace missing or too small";
    case EPILORA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

size_t epilora_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t r) {
  (void)N;
  if (M < 0 || K < 0 || r < 0) return 0;
  switch (op) {
    case EPILORA_OP_SHRINK: return shrink_ws(kStateBytes, M, K, r).total;
    case EPILORA_OP_GEMM:
    case EPILORA_OP_EXPAND:
    case EPILORA_OP_QUANT_W4: return kCtrlBytes;
    case EPILORA_OP_DECODE: return decode_ws(M, K, r).total;
    default: return 0;
  }
}

int epilora_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (ws == nullptr || ws_bytes < kCtrlBytes) return EPILORA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return EPILORA_ERR_UNSUPPORTED;
  return hip_status(launch_fill_u32(ws, 0u, (int64_t)(ws_bytes / 4), as_stream(stream)));
}

int epilora_workspace_force_timeout(void* ws, size_t ws_bytes, int32_t on, void* stream) {
  if (ws == nullptr || ws_bytes < kCtrlBytes) return EPILORA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return EPILORA_ERR_UNSUPPORTED;
  int* word = reinterpret_cast<int*>(ws) + kCtrlForceTimeout;
  return hip_status(launch_fill_u32(word, on != 0 ? 1u : 0u, 1, as_stream(stream)));
}

int epilora_device_error(void* ws, int32_t clear, int32_t* out_code, void* stream) {
  if (ws == nullptr || out_code == nullptr) return EPILORA_ERR_INVALID_ARG;
  hipStream_t s = as_stream(stream);
  int32_t word = 0;
  if (hipMemcpyAsync(&word, ws, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess) return EPILORA_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return EPILORA_ERR_HIP;
  *out_code = word;
  if (clear) return hip_status(launch_fill_u32(ws, 0u, 1, s));
  return EPILORA_OK;
}

int epilora_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* xq, int64_t ldq, float* sx,
                      void* stream) {
  const int st = check_rows(x, M, K, ldx, xq, ldq, sx);
  if (st != EPILORA_OK || M == 0) return st;
  return hip_status(launch_quant_rows(x, M, K, ldx, xq, ldq, sx, as_stream(stream)));
}

int epilora_quant_weight_fp8(const uint16_t* w, int64_t N, int64_t K, uint8_t* wq, float* sw, void* stream) {
  const int st = check_rows(w, N, K, K, wq, K, sw);
  if (st != EPILORA_OK || N == 0) return st;
  return hip_status(launch_quant_rows(w, N, K, K, wq, K, sw, as_stream(stream)));
}

int epilora_quant_weight_fp4(const uint16_t* w, int64_t N, int64_t K, uint8_t* wc, uint8_t* bs, float* gs,
                             void* ws, size_t ws_bytes, void* stream) {
  if (N < 0 || K < 0) return EPILORA_ERR_INVALID_ARG;
  if (N == 0 || K == 0) return EPILORA_OK;
  if (w == nullptr || wc == nullptr || bs == nullptr || gs == nullptr) return EPILORA_ERR_INVALID_ARG;
  if (K % 32 != 0) return EPILORA_ERR_UNSUPPORTED;
  if (!aligned(w, 16) || !aligned(wc, 8) || !aligned(gs, 4)) return EPILORA_ERR_UNSUPPORTED;
  const int st = check_ws(ws, ws_bytes, kCtrlBytes);
  if (st != EPILORA_OK) return st;
  return hip_status(launch_quant_weight_fp4(w, N, K, wc, bs, gs, ws, as_stream(stream)));
}

int epilora_lora_shrink_ex(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const void* A, int32_t afmt,
                           const float* sa, int32_t L, int32_t nslices, int32_t r, const int32_t* ranks,
                           const int32_t* idx, const uint8_t* mask, float* z, void* ws, size_t ws_bytes,
                           void* stream) {
  if (M < 0 || K < 0) return EPILORA_ERR_INVALID_ARG;
  if (nslices < 1 || nslices > kMaxSlices) return EPILORA_ERR_INVALID_ARG;
  int st = check_afmt(afmt, sa, true, nullptr, false);
  if (st != EPILORA_OK) return st;
  if (M == 0) return EPILORA_OK;
  if (x == nullptr || z == nullptr) return EPILORA_ERR_INVALID_ARG;
  st = check_adapters(L, r, A, true, nullptr, false, ranks, idx);
  if (st != EPILORA_OK) return st;
  if (ldx < K) return EPILORA_ERR_INVALID_ARG;
  if (K % 16 != 0 || ldx % 16 != 0 || !aligned(x, 16) || !aligned(z, 16)) return EPILORA_ERR_UNSUPPORTED;
  if (cdiv(M, kShrinkTokens) * nslices > kMaxShrinkTiles) return EPILORA_ERR_UNSUPPORTED;
  st = check_ws(ws, ws_bytes, shrink_ws(kStateBytes, M, K, r, nslices).total);
  if (st != EPILORA_OK) return st;
  AdapterArgs ad;
  ad.A = reinterpret_cast<const uint16_t*>(A); ad.B = nullptr; ad.ranks = ranks; ad.idx = idx; ad.mask = mask;
  ad.L = L; ad.r = r; ad.scale = 1.0f;
  ad.S = nslices; ad.zld = nslices * r;
  for (int i = 0; i < kMaxSlices; ++i) ad.slice_end[i] = INT64_MAX;
  ad.afmt = afmt; ad.sa = sa; ad.sb = nullptr;
  return hip_status(launch_shrink(x, M, K, ldx, ad, z, ws, as_stream(stream)));
}

int epilora_rmsnorm_quant_shrink(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                                 float eps, uint16_t* xn, int64_t ldn, uint8_t* xq, int64_t ldq, float* sx,
                                 const void* A, int32_t afmt, const float* sa, int32_t L, int32_t nslices, int32_t r,
                                 const int32_t* ranks, const int32_t* idx, const uint8_t* mask, float* z, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (M < 0 || K < 0) return EPILORA_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || eps == INFINITY) return EPILORA_ERR_INVALID_ARG;
  if (M == 0) return EPILORA_OK;
  if (x == nullptr || gamma == nullptr || (xq == nullptr) != (sx == nullptr)) return EPILORA_ERR_INVALID_ARG;
  if (ldx < K || (xq != nullptr && ldq < K) || (xn != nullptr && ldn < K)) return EPILORA_ERR_INVALID_ARG;
  if (K == 0 || K % 16 != 0 || ldx % 16 != 0 || !aligned(x, 16) || !aligned(gamma, 16)) return EPILORA_ERR_UNSUPPORTED;
  if (xq != nullptr && (ldq % 16 != 0 || !aligned(xq, 16) || !aligned(sx, 4))) return EPILORA_ERR_UNSUPPORTED;
  if (xn != nullptr && (ldn % 16 != 0 || !aligned(xn, 16))) return EPILORA_ERR_UNSUPPORTED;
  AdapterArgs ad{};
  ad.S = 1; ad.r = 16; ad.zld = 16;
  for (int i = 0; i < kMaxSlices; ++i) ad.slice_end[i] = INT64_MAX;
  if (A != nullptr) {  // the shrink too
    if (nslices < 1 || nslices > kMaxSlices || z == nullptr) return EPILORA_ERR_INVALID_ARG;
    int st = check_afmt(afmt, sa, true, nullptr, false);
    if (st != EPILORA_OK) return st;
    st = check_adapters(L, r, A, true, nullptr, false, ranks, idx);
    if (st != EPILORA_OK) return st;
    if (!aligned(z, 16)) return EPILORA_ERR_UNSUPPORTED;
    if (cdiv(M, kShrinkTokens) * nslices > kMaxShrinkTiles) return EPILORA_ERR_UNSUPPORTED;
    st = check_ws(ws, ws_bytes, shrink_ws(kStateBytes, M, K, r, nslices).total);
    if (st != EPILORA_OK) return st;
    ad.A = reinterpret_cast<const uint16_t*>(A); ad.ranks = ranks; ad.idx = idx; ad.mask = mask;
    ad.L = L; ad.r = r; ad.scale = 1.0f; ad.S = nslices; ad.zld = nslices * r;
    ad.afmt = afmt; ad.sa = sa;
  }
  return hip_status(launch_norm_quant_shrink(x, M, K, ldx, gamma, eps, xn, ldn, xq, ldq, sx, ad, z, ws,
                                             as_stream(stream)));
}

int epilora_lora_shrink(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* A, int32_t L,
                        int32_t r, const int32_t* ranks, const int32_t* idx, const uint8_t* mask, float* z,
                        void* ws, size_t ws_bytes, void* stream) {
  return epilora_lora_shrink_ex(x, M, K, ldx, A, EPILORA_A_BF16, nullptr, L, 1, r, ranks, idx, mask, z, ws, ws_bytes,
                                stream);
}

int epilora_gemm_lora(const epilora_layer_args* a, void* stream) {
  if (a == nullptr) return EPILORA_ERR_INVALID_ARG;
  if (a->M < 0 || a->N < 0 || a->K < 0) return EPILORA_ERR_INVALID_ARG;
  if (a->amode != EPILORA_ACT_FP8 && a->amode != EPILORA_ACT_BF16) return EPILORA_ERR_INVALID_ARG;
  if (a->M == 0 || a->N == 0) return EPILORA_OK;
  const bool a16 = a->amode == EPILORA_ACT_BF16;
  if (a->y == nullptr) return EPILORA_ERR_INVALID_ARG;
  int st = check_weights(a);
  if (st != EPILORA_OK) return st;
  if (a16) {  // the W8A16 GEMM reads the bf16 rows
    if (a->x == nullptr) return EPILORA_ERR_INVALID_ARG;
    if (a->ldx < a->K || a->ldy < a->N) return EPILORA_ERR_INVALID_ARG;
    if (a->wfmt != EPILORA_W_FP8 || a->ldx % 16 != 0 || !aligned(a->x, 16) || !aligned(a->y, 2))
      return EPILORA_ERR_UNSUPPORTED;
  } else {
    if (a->xq == nullptr || a->sx == nullptr) return EPILORA_ERR_INVALID_ARG;
    if (a->ldq < a->K || a->ldy < a->N) return EPILORA_ERR_INVALID_ARG;
    if (a->ldq % 16 != 0 || !aligned(a->xq, 16) || !aligned(a->sx, 4) || !aligned(a->y, 2))
      return EPILORA_ERR_UNSUPPORTED;
  }
  const bool lora = a->z != nullptr;
  if (lora) {
    st = check_adapters(a->L, a->r, a->A, false, a->B, true, a->ranks, a->idx);
    if (st != EPILORA_OK) return st;
    st = check_afmt(a->afmt, a->sa, false, a->sb, true);
    if (st != EPILORA_OK) return st;
    // output tiles stay inside one slice: 16 rows (M <= 64), 128 (prefill)
    st = check_slices(a->nslices, a->slice_n, a->N, a->M <= EPILORA_DECODE_MAX_M ? 16 : 128);
    if (st != EPILORA_OK) return st;
    if (!aligned(a->z, 16)) return EPILORA_ERR_UNSUPPORTED;
    st = check_ws(a->ws, a->ws_bytes, kCtrlBytes);
    if (st != EPILORA_OK) return st;
  }
  return hip_status(launch_gemm_lora(a->xq, a->sx, a->ldq, a16 ? a->x : nullptr, a->ldx, a->M, a->N, a->K,
                                     weights_of(a), adapters_of(a, lora), a->z, a->y, a->ldy, a->ws,
                                     as_stream(stream)));
}

int epilora_lora_expand_add_ex(const float* z, int64_t M, int64_t N, const void* B, int32_t afmt, const float* sb,
                               int32_t L, int32_t r, int32_t nslices, const int64_t* slice_n, const int32_t* ranks,
                               const int32_t* idx, const uint8_t* mask, float scale, uint16_t* y, int64_t ldy,
                               void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || N < 0) return EPILORA_ERR_INVALID_ARG;
  int st = check_slices(nslices, slice_n, N, 1);
  if (st != EPILORA_OK) return st;
  st = check_afmt(afmt, nullptr, false, sb, true);
  if (st != EPILORA_OK) return st;
  if (M == 0 || N == 0) return EPILORA_OK;
  if (z == nullptr || y == nullptr) return EPILORA_ERR_INVALID_ARG;
  st = check_adapters(L, r, nullptr, false, B, true, ranks, idx);
  if (st != EPILORA_OK) return st;
  if (ldy < N) return EPILORA_ERR_INVALID_ARG;
  if (!aligned(z, 16) || !aligned(y, 2)) return EPILORA_ERR_UNSUPPORTED;
  st = check_ws(ws, ws_bytes, kCtrlBytes);
  if (st != EPILORA_OK) return st;
  AdapterArgs ad;
  ad.A = nullptr; ad.B = reinterpret_cast<const uint16_t*>(B); ad.ranks = ranks; ad.idx = idx; ad.mask = mask;
  ad.L = L; ad.r = r; ad.scale = scale;
  set_slices(ad, nslices, slice_n);
  ad.afmt = afmt; ad.sa = nullptr; ad.sb = sb;
  return hip_status(launch_expand_add(z, M, N, ad, y, ldy, ws, as_stream(stream)));
}

int epilora_lora_expand_add(const float* z, int64_t M, int64_t N, const uint16_t* B, int32_t L, int32_t r,
                            const int32_t* ranks, const int32_t* idx, const uint8_t* mask, float scale, uint16_t* y,
                            int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return epilora_lora_expand_add_ex(z, M, N, B, EPILORA_A_BF16, nullptr, L, r, 1, nullptr, ranks, idx, mask, scale, y,
                                    ldy, ws, ws_bytes, stream);
}

int epilora_decode_lora(const epilora_layer_args* a, void* stream) {
  int32_t r = 16;
  if (a == nullptr) return EPILORA_ERR_INVALID_ARG;
  const int st0 = check_decode(a, r);
  if (st0 != EPILORA_OK || a->M == 0 || a->N == 0) return st0;
  const int st = check_ws(a->ws, a->ws_bytes, decode_need(a, r));
  if (st != EPILORA_OK) return st;
  return hip_status(launch_decode_lora(a->x, a->ldx, a->M, a->N, a->K, weights_of(a), adapters_of(a, a->idx != nullptr),
                                       a->y, a->ldy, a->xq_out, a->sx_out, a->ldq_out, a->ws,
                                       a->amode == EPILORA_ACT_BF16, as_stream(stream)));
}

int epilora_decode_lora_noalloc(const epilora_layer_args* a, void* stream) {
  int32_t r = 16;
  if (a == nullptr) return EPILORA_ERR_INVALID_ARG;
  const int st0 = check_decode(a, r);
  if (st0 != EPILORA_OK || a->M == 0 || a->N == 0) return st0;
  if (decode_need(a, r) > kScratchBytes) return EPILORA_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = scratch_of_device(&ws);
  if (st != EPILORA_OK) return st;
  // The previous call on this device left its counters at zero and cleared
  // its z words, unless it timed out; clear the whole state region (control
  // block, counters, z) so that every call starts from zero regardless.
  hipStream_t s = as_stream(stream);
  if (launch_fill_u32(ws, 0u, (int64_t)(kStateBytes / 4), s) != hipSuccess) return EPILORA_ERR_HIP;
  return hip_status(launch_decode_lora(a->x, a->ldx, a->M, a->N, a->K, weights_of(a), adapters_of(a, a->idx != nullptr),
                                       a->y, a->ldy, a->xq_out, a->sx_out, a->ldq_out, ws,
                                       a->amode == EPILORA_ACT_BF16, s));
}

}  // extern "C"
