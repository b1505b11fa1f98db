// Decode path instantiation: bf16 activations, experts and shared expert.
#include "decode_impl.h"

namespace moe {
int launch_decode_bf16(Args A, hipStream_t st, bool route_only, const LaunchHook& hook) {
  return launch_decode_dt<MOE_BF16, MOE_BF16, MOE_BF16>(A, st, route_only, hook);
}
}  // namespace moe
