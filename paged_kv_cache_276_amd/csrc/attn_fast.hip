// attn_fast.hip -- placeholder until the bf16 fast path lands.
#include "launch.h"

namespace pkv {

bool fast_supports(int32_t, int32_t, int32_t, int32_t) { return false; }

hipError_t launch_decode_fast(const DecodeArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace pkv
