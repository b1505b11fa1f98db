// Measurement support: the sustained HBM read rate of the access pattern the decode kernels use
// (16-byte loads streamed once over the whole chip), the ceiling a weight-streaming kernel is
// judged against ("Optimizing on-device inference for Apple Silicon", section "Limits of further
// optimization": the MoE kernels are compared with the fastest sustained weight-read rate for
// their access pattern, and removing their arithmetic changed the rate by 0.2%).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;  // 16-byte loads per thread in flight per pass

// Every 16-byte unit of [buf, buf + n16 * 16) is loaded once (grid-stride, kReadUnroll loads per
// thread issued before any is used) and folded into an xor; a block stores its fold only when it
// equals a constant no sane input produces, so the loads cannot be dropped and nothing is
// written in practice.
__global__ __launch_bounds__(kReadThreads) void read_stream(const uint4* buf, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads * kReadUnroll;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * kReadThreads * kReadUnroll + threadIdx.x; base < n16; base += stride) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) {
      const size_t i = base + (size_t)j * kReadThreads;
      v[j] = i < n16 ? ldnt16(buf + i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x & 63] = acc;
}

}  // namespace
}  // namespace moe

extern "C" int moe_read_ceiling(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  using namespace moe;
  if (!buf || !sink || bytes < 16) return MOE_EINVAL;
  if (((uintptr_t)buf & 15u) || ((uintptr_t)sink & 3u)) return MOE_EALIGN;
  const uint4* b = (const uint4*)buf;
  size_t n16 = bytes / 16;
  const int ncu = 256;  // blocks: eight per CU of a 256-CU part, enough loads in flight
  void* args[] = {&b, &n16, &sink};
  return launch(LaunchHook{}, "read_ceiling", (const void*)read_stream, dim3(8 * ncu), dim3(kReadThreads), args, 0,
                (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_EHIP;
}

extern "C" int moe_stage_rate(const void* buf, size_t region_bytes, int32_t seg_bytes, int32_t iters, uint32_t* sink,
                              void* stream) {
  using namespace moe;
  if (!buf || !sink || iters < 1) return MOE_EINVAL;
  if (region_bytes < 8192 || region_bytes > ((size_t)1 << 31) || (region_bytes & (region_bytes - 1))) return MOE_EINVAL;
  if (seg_bytes < 16 || seg_bytes > 1024 || (seg_bytes & (seg_bytes - 1))) return MOE_EINVAL;
  if (((uintptr_t)buf & 15u) || ((uintptr_t)sink & 3u)) return MOE_EALIGN;
  return launch_stage_probe(buf, (uint32_t)(region_bytes - 1), seg_bytes, iters, sink, (hipStream_t)stream);
}
