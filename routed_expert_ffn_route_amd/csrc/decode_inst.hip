// Decode path instantiation unit: compiled once per (dtype combination, token tile) with
//   -DMOE_DEC_NAME=<f32|bf16|fp4|i4> -DMOE_DEC_TM=<1|4|8|16>
// so that the kernels of decode_impl.h build in parallel units.
#include "decode_impl.h"

#if !defined(MOE_DEC_NAME) || !defined(MOE_DEC_TM)
#error "decode_inst.hip is compiled with MOE_DEC_NAME and MOE_DEC_TM defined"
#endif

#define MOE_CAT4_(a, b, c, d) a##b##c##d
#define MOE_CAT4(a, b, c, d) MOE_CAT4_(a, b, c, d)
#define MOE_FN(n, t) MOE_CAT4(launch_decode_, n, _t, t)

namespace moe {
namespace {
constexpr int kDecF32[3] = {MOE_F32, MOE_F32, MOE_F32};
constexpr int kDecBf16[3] = {MOE_BF16, MOE_BF16, MOE_BF16};
constexpr int kDecFp4[3] = {MOE_BF16, MOE_MXFP4, MOE_BF16};
constexpr int kDecI4[3] = {MOE_BF16, MOE_INT4G64, MOE_BF16};
#define MOE_DT_f32 kDecF32
#define MOE_DT_bf16 kDecBf16
#define MOE_DT_fp4 kDecFp4
#define MOE_DT_i4 kDecI4
#define MOE_DT2(n) MOE_DT_##n
#define MOE_DT(n) MOE_DT2(n)
}  // namespace

int MOE_FN(MOE_DEC_NAME, MOE_DEC_TM)(Args A, hipStream_t st, bool route_only, const LaunchHook& hook) {
  return launch_decode_t<MOE_DT(MOE_DEC_NAME)[0], MOE_DT(MOE_DEC_NAME)[1], MOE_DT(MOE_DEC_NAME)[2],
                         MOE_DEC_TM>(A, st, route_only, hook);
}
}  // namespace moe
