// The fused decode kernels for the matched W8A16 GEMM (FP8 weights, bf16 activations).
#include "decode.h"

namespace epilora {

void decode_dispatch_a16(DecodeParams& p, bool want_xq, hipStream_t stream) { dispatch_decode<EPILORA_W_FP8, true>(p, want_xq, stream); }

}  // namespace epilora
