/*
 * epilora.h -- C ABI of a multi-tenant LoRA linear layer on a low-precision
 * (FP8 or 4-bit) base, for AMD Instinct MI355X (gfx950).
 *
 * For every token t with tenant index a_t the layer computes
 *
 *     Y[t] = bf16( dequant(W_q . quant(x_t)) + s * B[a_t] (A[a_t] x_t) )
 *
 * where a_t = -1 means "no adapter" and an optional per-token mask limits the
 * adapter to flagged (prefill) tokens.  The method is described in
 * "EpiLoRA: Fusing Many LoRA Adapters into Low-Precision GEMMs for Serving and
 * RL" (Background; Design, section "Multi-adapter kernels": K1 quantizes the
 * activations once and forms the down-projection from the bf16 activations,
 * K2 runs the low-precision GEMM and adds each adapter group's up-projection
 * in its epilogue; the decode path overlaps the down-projection with the
 * GEMM's main loop) and, for the mask, "PreFT: Prefill-only finetuning for
 * efficient inference" (abstract; Figure 6: a per-forward position mask
 * written outside the compiled region, adapter parameters at stable
 * addresses).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every buffer pointer is a DEVICE pointer owned by the caller.  The
 *   library never allocates, frees, retains or copies them, never
 *   synchronizes the stream, and keeps no global state: calls are reentrant
 *   and may be captured in a HIP graph.  (The pages' fused call is a custom
 *   operator captured in the engine's CUDA graphs and reads the engine's own
 *   adapter buffers and batching metadata in place: "The vLLM plugin".)
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 * - bf16 values are passed as their uint16_t bit patterns; FP8 is OCP E4M3FN
 *   (bias 7, max 448, no infinity); 4-bit weights are E2M1 codes.
 * - Matrices are row-major with the given leading dimension (in elements).
 *   The leading dimensions of inputs (ldx, ldq) must be multiples of 16 and
 *   input matrix pointers 16-byte aligned; outputs (y, ldy >= N) take any
 *   2-byte-aligned layout.  M = 0 or N = 0 is a valid call that does nothing.
 * - Host-side validation happens before any HIP call; a failing call
 *   launches nothing.  Content that lives on the device (indices, ranks) is
 *   checked in the kernels: an index outside [-1, L) is treated as -1 and
 *   raises EPILORA_DEV_BAD_INDEX in the workspace's device error word.
 * - Inputs must be finite.
 *
 * Status codes: EPILORA_OK, EPILORA_ERR_INVALID_ARG (a null pointer, a
 * negative size, a bad enum), EPILORA_ERR_UNSUPPORTED (a valid request this
 * library does not serve, e.g. an alignment or a batch too large for the
 * fused decode path: the caller's cue to fall back, as the pages' plugin
 * falls back to the engine's own path), EPILORA_ERR_WORKSPACE (workspace
 * missing or too small), EPILORA_ERR_HIP (a HIP launch failed).
 */
#ifndef EPILORA_H
#define EPILORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EPILORA_VERSION 10000 /* 1.0.0 */

enum epilora_status {
  EPILORA_OK = 0,
  EPILORA_ERR_INVALID_ARG = 1,
  EPILORA_ERR_UNSUPPORTED = 2,
  EPILORA_ERR_WORKSPACE = 3,
  EPILORA_ERR_HIP = 4
};

/* Bits of the device error word kept in a workspace (sticky until cleared). */
enum epilora_device_error_bits {
  EPILORA_DEV_BAD_INDEX = 1,   /* an index outside [-1, L) was treated as -1 */
  EPILORA_DEV_WAIT_TIMEOUT = 2, /* the fused path's bounded wait expired; the
                                   outputs of that call are not valid */
  EPILORA_DEV_INTERNAL = 4      /* a workgroup was given more output tiles
                                   than it can hold (a library bug, never
                                   expected); the outputs are not valid */
};

/* Weight formats. */
enum epilora_wfmt {
  EPILORA_W_FP8 = 0, /* w: E4M3 [N][K]; sw: fp32 [N] (per output channel) */
  EPILORA_W_FP4 = 1  /* w: packed E2M1 [N][K/2], element 2i in the low
                        nibble of byte i; bs: E4M3 [N][K/16], one scale per
                        16 consecutive elements along K; gs: one fp32 */
};

/* Adapter storage ("EpiLoRA ...", Design, "Multi-adapter kernels": adapters
 * may be stored in FP8 and dequantized in registers, halving the adapter
 * bytes the kernels read; "The vLLM plugin", Memory: low-precision adapters
 * in smaller slots). */
enum epilora_afmt {
  EPILORA_A_BF16 = 0, /* A and B hold bf16 values */
  EPILORA_A_FP8 = 1   /* A and B hold E4M3 codes of the same shapes (one byte
                         per element), each row with one fp32 scale: sa
                         [L][nslices][r] for A's rank rows, sb [L][N] for B's
                         output rows; a row's values are e4m3(code) * scale
                         (epilora_quant_weight_fp8 applied to the rows makes
                         them).  z_j = sa_j * sum_k e4m3(A_jk) x_k and the
                         output adds s * sb_n * sum_j e4m3(B_nj) z_j. */
};

/* Activation modes of the GEMM. */
enum epilora_amode {
  EPILORA_ACT_FP8 = 0, /* per-token FP8 activations (W8A8 / W4A8) */
  EPILORA_ACT_BF16 = 1 /* bf16 activations: the matched W8A16 GEMM */
};

/* Operations, for epilora_workspace_bytes. */
enum epilora_op {
  EPILORA_OP_SHRINK = 1,
  EPILORA_OP_GEMM = 2,
  EPILORA_OP_EXPAND = 3,
  EPILORA_OP_DECODE = 4,
  EPILORA_OP_QUANT_W4 = 5
};

/* Largest batch the fused decode path serves (the pages use the decode path
 * for batches of up to 32 tokens; this library's kernel takes up to 64). */
#define EPILORA_DECODE_MAX_M 64
/* Largest adapter rank (slot width r). */
#define EPILORA_MAX_RANK 128

/* Arguments of epilora_gemm_lora and epilora_decode_lora. */
typedef struct epilora_layer_args {
  int64_t M, N, K;          /* tokens, output features, input features */
  /* Activations. */
  const uint16_t* x;        /* bf16 [M][ldx]; read by epilora_decode_lora */
  int64_t ldx;
  const uint8_t* xq;        /* E4M3 [M][ldq]; read by epilora_gemm_lora */
  const float* sx;          /* fp32 [M] per-token scales (gemm_lora) */
  int64_t ldq;
  /* Base weights. */
  int32_t wfmt;             /* enum epilora_wfmt */
  const uint8_t* w;
  const float* sw;          /* EPILORA_W_FP8 */
  const uint8_t* bs;        /* EPILORA_W_FP4 */
  const float* gs;          /* EPILORA_W_FP4: device pointer to one float */
  /* Adapters, in the caller's stacked slots. */
  int32_t L, r;             /* slots, slot width (rank padded), r <= 128 */
  const uint16_t* A;        /* bf16 [L][r][K]; read by epilora_decode_lora */
  const uint16_t* B;        /* bf16 [L][N][r] */
  const int32_t* ranks;     /* [L] true ranks (<= r) or NULL (all r);
                               columns j >= rank are ignored, rank 0 means
                               the adapter is off */
  const int32_t* idx;       /* [M] tenant per token, -1 = none */
  const uint8_t* mask;      /* [M], nonzero = adapter applies; NULL = all */
  const float* z;           /* fp32 [M][r] down-projection from
                               epilora_lora_shrink (gemm_lora only);
                               NULL = base GEMM only */
  float scale;              /* LoRA scaling s */
  /* Output. */
  uint16_t* y;              /* bf16 [M][ldy] */
  int64_t ldy;
  /* epilora_decode_lora: where the quantized activations go (E4M3
     [M][ldq_out] and fp32 [M]); NULL = kept in the workspace only. */
  uint8_t* xq_out;
  float* sx_out;
  int64_t ldq_out;
  /* Scratch. */
  void* ws;
  size_t ws_bytes;
  /* Projections whose N outputs are several consecutive slices, each with
     its own adapter pair (attention's query / key / value, the MLP's gate /
     up: "EpiLoRA ...", Evaluation, the many-tenant results and the
     appendix's comparison of expand costs, Tables 14 and 15): nslices in
     0..4 (0 or 1: one slice, the plain layer), slice_n[s] the width of
     slice s (sum N).  Then A is [L][nslices][r][K] (slice s's
     down-projection of adapter a at A[a][s]), B stays [L][N][r] (the rows of
     slice s hold its up-projection) and z is [M][nslices * r] (slice s in
     columns s*r .. s*r+r).  Output n of slice s adds s * B[a][n] . z_s.
     Widths must be multiples of 16 (M <= 64) or 128 (M > 64), else
     EPILORA_ERR_UNSUPPORTED. */
  int32_t nslices;
  int64_t slice_n[4];
  /* Adapter storage (enum epilora_afmt) and, for EPILORA_A_FP8, the row
     scales (16-byte aligned): sa [L][nslices][r] (read where A is), sb
     [L][N] (read where B is). */
  int32_t afmt;
  const float* sa;
  const float* sb;
  /* Activation mode (enum epilora_amode).  EPILORA_ACT_BF16 selects the
     matched W8A16 GEMM: both calls read the bf16 activations x / ldx (not
     xq / sx), the FP8 weights are widened to bf16 exactly, the products
     accumulate in fp32 and base = acc * sw[n] ("EpiLoRA ...", Design, "LoRA
     RL on the same base": the matched engine computes with the trainer's
     arithmetic on the same FP8 weights).  FP8 weights only; xq_out and
     sx_out must be NULL. */
  int32_t amode;
} epilora_layer_args;

/* Library version (EPILORA_VERSION of the build). */
int epilora_version(void);

/* Static text for a status code. */
const char* epilora_strerror(int status);

/* Bytes of workspace `op` needs for a call of the given sizes (r = the row
 * width of z: the slot width, times the number of output slices for a
 * projection with per-slice adapters); each call checks its own need
 * against ws_bytes.  One workspace may
 * serve every call on one stream in turn (the pages' plugin shares its
 * scratch buffers across layers: "The vLLM plugin", Memory); calls that
 * overlap in time must not share one. */
size_t epilora_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K,
                               int32_t r);

/* Zero a workspace (a fill kernel, safe inside graph capture).  Required once
 * after allocation; every call leaves its counters at zero again. */
int epilora_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Test hook for the failure path of the fused decode path: with on != 0,
 * every bounded wait of epilora_decode_lora calls on this workspace gives up
 * at once, as if its wall-clock bound had expired (the kernels still run to
 * their end; the call raises EPILORA_DEV_WAIT_TIMEOUT and its outputs are
 * not valid).  Sets one word of the workspace's control block with a fill
 * kernel on `stream`; epilora_workspace_init clears it again. */
int epilora_workspace_force_timeout(void* ws, size_t ws_bytes, int32_t on,
                                    void* stream);

/* Read the device error word of a workspace into *out_code: enqueues a copy
 * on `stream` and waits for it (a synchronizing diagnostic, not for use
 * inside graph capture).  Then clears the word when `clear` is nonzero. */
int epilora_device_error(void* ws, int32_t clear, int32_t* out_code,
                         void* stream);

/* Per-token dynamic FP8 quantization ("Multi-adapter kernels", K1).
 * For each row t: amax = max_k |x[t][k]|; sx[t] = fp32(amax / 448) (IEEE
 * division; 1.0 for an all-zero row); xq[t][k] = E4M3(fp32(x[t][k] / sx[t]))
 * rounded to nearest even and saturated at +-448.  Bit-exact.
 * x: bf16 [M][ldx]; xq: [M][ldq]; sx: [M].  K % 16 == 0. */
int epilora_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                      uint8_t* xq, int64_t ldq, float* sx, void* stream);

/* The RMS normalization in front of the query / key / value and gate / up
 * projections, with the per-token FP8 quantizer and the shrink taken from
 * its output in the same kernel ("EpiLoRA ...", appendix "Discussion and
 * Limitations": computing the down-projection inside the normalization
 * kernel that already reads the input hides it for these projections; the
 * GEMM then finds z ready: epilora_gemm_lora).
 * Per token row t: ms = fp32(sum_k x_k^2 / K) (the squares summed in fp64),
 * inv = fp32(1 / fp32(sqrt(fp32(ms + eps)))) (correctly rounded),
 * xn_k = bf16(bf16(x_k * inv) * gamma_k) (round to nearest even);
 * xq, sx = the epilora_quant_act result for xn (bit for bit); with A != NULL,
 * z = the epilora_lora_shrink_ex result for xn (same arguments and rules).
 * x: bf16 [M][ldx]; gamma: bf16 [K]; xn: bf16 [M][ldn] or NULL (not
 * written); xq: [M][ldq] and sx: [M], or both NULL (no codes: the plain
 * normalization when xn is given); eps >= 0.  K % 16 == 0, ldx, ldq, ldn
 * multiples of 16, x, gamma, xn, xq 16-byte aligned.  A == NULL: no shrink
 * (the adapter arguments, z and the workspace are ignored); otherwise a
 * workspace of EPILORA_OP_SHRINK (r = nslices * r). */
int epilora_rmsnorm_quant_shrink(const uint16_t* x, int64_t M, int64_t K,
                                 int64_t ldx, const uint16_t* gamma, float eps,
                                 uint16_t* xn, int64_t ldn, uint8_t* xq,
                                 int64_t ldq, float* sx, const void* A,
                                 int32_t afmt, const float* sa, int32_t L,
                                 int32_t nslices, int32_t r,
                                 const int32_t* ranks, const int32_t* idx,
                                 const uint8_t* mask, float* z, void* ws,
                                 size_t ws_bytes, void* stream);

/* Load-time FP8 weight quantization, one scale per output channel (the
 * pages' FP8 bases are quantized when the model loads: Evaluation, Setup).
 * Same rule as epilora_quant_act applied to the rows of W.
 * w: bf16 [N][K]; wq: [N][K]; sw: [N].  K % 16 == 0. */
int epilora_quant_weight_fp8(const uint16_t* w, int64_t N, int64_t K,
                             uint8_t* wq, float* sw, void* stream);

/* Load-time 4-bit weight quantization in the NVFP4 layout.
 * gs = fp32(amax(W) / 2688) (1.0 if W is zero);
 * bs[n][b] = E4M3(fp32(amax(block) / fp32(6 * gs)));
 * code = E2M1(fp32(w / fp32(e4m3(bs) * gs))) (nearest even, saturated at 6;
 * 0 where that product is 0).  w: bf16 [N][K]; wc: [N][K/2]; bs: [N][K/16];
 * gs: one float.  K % 32 == 0.  Needs a workspace of EPILORA_OP_QUANT_W4. */
int epilora_quant_weight_fp4(const uint16_t* w, int64_t N, int64_t K,
                             uint8_t* wc, uint8_t* bs, float* gs, void* ws,
                             size_t ws_bytes, void* stream);

/* The shrink ("Multi-adapter kernels", K1: h = x A^T from the bf16
 * activations, the sum over K split across workgroups).
 * z[t][j] = sum_k A[idx[t]][j][k] * x[t][k] (fp32 accumulation) for active
 * tokens and j < rank; 0 elsewhere.  A token is active when idx[t] is in
 * [0, L), its mask byte (if any) is nonzero and its rank is positive.
 * Split-K partial sums are combined in a fixed order, so results are
 * deterministic ("The decode path").  x: bf16 [M][ldx]; A: bf16 [L][r][K];
 * z: fp32 [M][r].  K % 16 == 0, r % 16 == 0, r <= 128, M <= 65536 (else
 * EPILORA_ERR_UNSUPPORTED; longer batches go in several calls).
 * Needs a workspace of EPILORA_OP_SHRINK. */
int epilora_lora_shrink(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                        const uint16_t* A, int32_t L, int32_t r,
                        const int32_t* ranks, const int32_t* idx,
                        const uint8_t* mask, float* z, void* ws,
                        size_t ws_bytes, void* stream);

/* The shrink with every adapter option: per-slice adapters (see
 * epilora_layer_args.nslices: A is [L][nslices][r][K], z is
 * [M][nslices * r], slice s's z_s[t] = A[idx[t]][s] x[t] in columns
 * s*r .. s*r+r) and FP8-stored adapters (afmt EPILORA_A_FP8: A holds E4M3
 * codes, sa [L][nslices][r] their row scales, z = sa * sum of code times x).
 * Same activity rule, rank and determinism as epilora_lora_shrink, which is
 * this call with afmt EPILORA_A_BF16 and nslices 1.  nslices in 1..4;
 * cdiv(M, 16) * nslices <= 4096.  Needs a workspace of EPILORA_OP_SHRINK
 * with r = nslices * r. */
int epilora_lora_shrink_ex(const uint16_t* x, int64_t M, int64_t K,
                           int64_t ldx, const void* A, int32_t afmt,
                           const float* sa, int32_t L, int32_t nslices,
                           int32_t r, const int32_t* ranks,
                           const int32_t* idx, const uint8_t* mask, float* z,
                           void* ws, size_t ws_bytes, void* stream);

/* The low-precision GEMM with the multi-adapter epilogue
 * ("Multi-adapter kernels", K2; "Kernel details", one output tile of K2).
 * base[t][n] = (acc[t][n] * sx[t]) * sw[n] for FP8 weights, where
 * acc = sum_k e4m3(xq[t][k]) * e4m3(w[n][k]) in fp32; for 4-bit weights each
 * weight is first decoded to the FP8 byte E4M3(e2m1(code) * e4m3(bs) / 8)
 * and base = (acc * sx[t]) * (gs * 8).  Active rows (as in
 * epilora_lora_shrink) get y = base + s * sum_j B[idx[t]][n][j] * z[t][j];
 * the other rows get y = base with no add at all, so they are bitwise equal
 * to the base-only GEMM.  Y = bf16(y), round to nearest even.
 * Tokens may come in any order; runs of equal indices (tokens sorted by
 * adapter) make the epilogue cheaper.  K % 32 == 0.  With z == NULL the call
 * is the base GEMM only and needs no workspace. */
int epilora_gemm_lora(const epilora_layer_args* args, void* stream);

/* The separate up-projection used by the pages' baseline path (Background,
 * "The cost of the separate adapter path": the expand reads, adds to and
 * writes the output again).  y[t][n] = bf16(y[t][n] + s * sum_j
 * B[idx[t]][n][j] * z[t][j]) for active rows; other rows untouched.
 * Needs a workspace of EPILORA_OP_EXPAND (device error word). */
int epilora_lora_expand_add(const float* z, int64_t M, int64_t N,
                            const uint16_t* B, int32_t L, int32_t r,
                            const int32_t* ranks, const int32_t* idx,
                            const uint8_t* mask, float scale, uint16_t* y,
                            int64_t ldy, void* ws, size_t ws_bytes,
                            void* stream);

/* The separate up-projection with every adapter option: per-slice adapters
 * (z [M][nslices * r]; output n of slice s uses z_s; slice widths slice_n,
 * a host array of nslices entries summing to N, or NULL with nslices <= 1)
 * and FP8-stored B (afmt EPILORA_A_FP8, row scales sb [L][N]). */
int epilora_lora_expand_add_ex(const float* z, int64_t M, int64_t N,
                               const void* B, int32_t afmt, const float* sb,
                               int32_t L, int32_t r, int32_t nslices,
                               const int64_t* slice_n, const int32_t* ranks,
                               const int32_t* idx, const uint8_t* mask,
                               float scale, uint16_t* y, int64_t ldy,
                               void* ws, size_t ws_bytes, void* stream);

/* The fused small-batch (decode) path ("Multi-adapter kernels", The decode
 * path): quantization, shrink and the GEMM with its epilogue in ONE launch.
 * The lowest workgroups compute z (and quantize x where the GEMM workgroups
 * do not do it themselves) and publish z in place, with device-coherent
 * stores into a workspace region that reads zero until written; the GEMM
 * workgroups stream their weights meanwhile, hold finished tiles in LDS and
 * poll z only before the epilogues.  HIP has no programmatic dependent
 * launch; this persistent split replaces it.  Inputs must be finite (a z
 * word that is a NaN with an all-ones payload would never count as
 * written: the wait would time out).
 * After a call that raised EPILORA_DEV_WAIT_TIMEOUT, re-initialise the
 * workspace (epilora_workspace_init) before using it again.
 * Same result as epilora_quant_act + epilora_lora_shrink +
 * epilora_gemm_lora.  Reads x (not xq/sx/z).  M <= EPILORA_DECODE_MAX_M,
 * else EPILORA_ERR_UNSUPPORTED.  Every wait is bounded; on expiry the
 * kernel sets EPILORA_DEV_WAIT_TIMEOUT and returns without the epilogue.
 * Needs a workspace of EPILORA_OP_DECODE. */
int epilora_decode_lora(const epilora_layer_args* args, void* stream);

/* The fused decode path for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels as epilora_decode_lora, but
 * the workspace is a fixed 16 MiB scratch array the library holds on each GPU
 * for the life of the process (a->ws and a->ws_bytes are ignored).  The call
 * allocates nothing: it enqueues a fill kernel that clears the scratch's
 * state region (so no call depends on how the previous one ended), then the
 * decode kernel.  A call whose workspace need, epilora_workspace_bytes(
 * EPILORA_OP_DECODE, M, N, K, r), exceeds 16 MiB returns
 * EPILORA_ERR_WORKSPACE and launches nothing.  Every call on one GPU shares
 * that GPU's scratch: calls that may overlap in time on one GPU (different
 * streams, or different host threads) race and must not be issued.  The
 * device error word lives in the scratch and is not readable by the caller:
 * an out-of-range index still counts as -1, and a wait timeout leaves that
 * call's outputs invalid. */
int epilora_decode_lora_noalloc(const epilora_layer_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EPILORA_H */
