// Decode path (T <= 16) dispatch by dtype combination; the kernels are in decode_impl.h,
// instantiated once per combination in decode_{f32,bf16,fp4}.hip.
#include "kernels.h"

namespace moe {

int launch_decode_f32(Args A, hipStream_t st, bool route_only, const LaunchHook& hook);
int launch_decode_bf16(Args A, hipStream_t st, bool route_only, const LaunchHook& hook);
int launch_decode_fp4(Args A, hipStream_t st, bool route_only, const LaunchHook& hook);

int launch_decode(Args A, hipStream_t st, bool route_only, const LaunchHook& hook) {
  if (A.act == MOE_F32) return launch_decode_f32(A, st, route_only, hook);
  if (A.wdt == MOE_MXFP4) return launch_decode_fp4(A, st, route_only, hook);
  return launch_decode_bf16(A, st, route_only, hook);
}

}  // namespace moe
