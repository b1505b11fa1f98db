// Decode path (T <= 16) dispatch by dtype combination and token tile; the kernels are in
// decode_impl.h, instantiated per (combination, tile) by decode_inst.hip.
#include "kernels.h"

namespace moe {

#define MOE_DECL(n)                                                                            \
  int launch_decode_##n##_t1(Args, hipStream_t, bool, const LaunchHook&);                     \
  int launch_decode_##n##_t4(Args, hipStream_t, bool, const LaunchHook&);                     \
  int launch_decode_##n##_t8(Args, hipStream_t, bool, const LaunchHook&);                     \
  int launch_decode_##n##_t16(Args, hipStream_t, bool, const LaunchHook&);                    \
  static int launch_decode_##n(Args A, hipStream_t st, bool route_only, const LaunchHook& h) { \
    if (A.T <= 1) return launch_decode_##n##_t1(A, st, route_only, h);                        \
    if (A.T <= 4) return launch_decode_##n##_t4(A, st, route_only, h);                        \
    if (A.T <= 8) return launch_decode_##n##_t8(A, st, route_only, h);                        \
    return launch_decode_##n##_t16(A, st, route_only, h);                                     \
  }
MOE_DECL(f32)
MOE_DECL(bf16)
MOE_DECL(fp4)
MOE_DECL(i4)
#undef MOE_DECL

int launch_decode(Args A, hipStream_t st, bool route_only, const LaunchHook& hook) {
  if (A.act == MOE_F32) return launch_decode_f32(A, st, route_only, hook);
  if (A.wdt == MOE_MXFP4) return launch_decode_fp4(A, st, route_only, hook);
  if (A.wdt == MOE_INT4G64) return launch_decode_i4(A, st, route_only, hook);
  return launch_decode_bf16(A, st, route_only, hook);
}

}  // namespace moe
