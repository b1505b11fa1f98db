// Per-token expert selection, shared by the decode and the any-T routing kernels.
#pragma once

#include <limits.h>

#include "common.h"

namespace moe {

// ------------------------------------------------------------------------------------------
// Selection: one wave per token.  Top-k on the fp32 logits (larger first, ties to the lower
// expert index), softmax over all E, renormalised over the k chosen.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void select_token(const float* lrow, int E, int k, int lane, int* ids_out,
                             float* w_out) {
  float v[MOE_MAX_E / kWave];
  unsigned avail = 0;
#pragma unroll
  for (int i = 0; i < MOE_MAX_E / kWave; ++i) {
    v[i] = 0.f;
    if (kWave * i < E) {
      int e = lane + kWave * i;
      if (e < E) {
        v[i] = lrow[e];
        avail |= 1u << i;
      }
    }
  }
  float lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < MOE_MAX_E / kWave; ++i)
    if ((avail >> i) & 1u) lmax = fmaxf(lmax, v[i]);
  const float m = wave_max(lmax);
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < MOE_MAX_E / kWave; ++i)
    if ((avail >> i) & 1u) z += expf(v[i] - m);
  z = group_sum<kWave>(z);

  unsigned taken = 0;
  int my_id = 0;
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < MOE_MAX_E / kWave; ++i) {
      if (((avail & ~taken) >> i) & 1u) {
        if (bi == INT_MAX || v[i] > bv) {
          bv = v[i];
          bi = lane + kWave * i;
        }
      }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o, kWave);
      int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == j) {
      my_id = bi;
      my_v = bv;
    }
  }
  float p = (lane < k) ? expf(my_v - m) / z : 0.f;
  float ps = group_sum<kWave>(p);
  if (lane < k) {
    ids_out[lane] = my_id;
    w_out[lane] = p / ps;
  }
}

}  // namespace moe
