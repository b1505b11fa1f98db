// Decode path instantiation: bf16 activations, MXFP4 experts, bf16 shared expert.
#include "decode_impl.h"

namespace moe {
int launch_decode_fp4(Args A, hipStream_t st, bool route_only, const LaunchHook& hook) {
  return launch_decode_dt<MOE_BF16, MOE_MXFP4, MOE_BF16>(A, st, route_only, hook);
}
}  // namespace moe
