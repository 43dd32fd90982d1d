// The fused decode kernels for 4-bit weights folded to FP8, FP8 activations.
#include "decode.h"

namespace epilora {

void decode_dispatch_fp4(DecodeParams& p, bool want_xq, hipStream_t stream) { dispatch_decode<EPILORA_W_FP4, false>(p, want_xq, stream); }

}  // namespace epilora
