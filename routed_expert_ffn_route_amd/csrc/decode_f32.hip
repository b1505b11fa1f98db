// Decode path instantiation: fp32 activations, experts and shared expert.
#include "decode_impl.h"

namespace moe {
int launch_decode_f32(Args A, hipStream_t st, bool route_only, const LaunchHook& hook) {
  return launch_decode_dt<MOE_F32, MOE_F32, MOE_F32>(A, st, route_only, hook);
}
}  // namespace moe
