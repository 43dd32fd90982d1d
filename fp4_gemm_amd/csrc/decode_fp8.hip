// The fused decode kernels for FP8 weights, FP8 activations.
#include "decode.h"

namespace epilora {

void decode_dispatch_fp8(DecodeParams& p, bool want_xq, hipStream_t stream) { dispatch_decode<EPILORA_W_FP8, false>(p, want_xq, stream); }

}  // namespace epilora
