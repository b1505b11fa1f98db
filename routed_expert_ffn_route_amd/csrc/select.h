// Per-token expert selection, shared by the decode and the any-T routing kernels.
//
// One wave selects for one token: the k largest fp32 logits, ties to the lower expert index,
// listed by descending logit; the combine weights are the softmax over all E renormalised
// over the k chosen ("Optimizing on-device inference for Apple Silicon", section "Qwen creates
// three distinct workload shapes": the router scores every expert and keeps eight).  The
// renormalised weights equal exp(l_j - m) / sum_{i<k} exp(l_i - m), m = the largest logit:
// the full-softmax denominator cancels, so it is never formed.
//
// Every (logit, expert) pair becomes one 64-bit key that orders exactly like the selection
// rule: the logit's bits mapped to an unsigned order in the high word, the complemented expert
// index in the low word (equal logits: lower index = larger key).  Each lane keeps its few
// keys sorted; a round takes the wave-wide maximum of the lanes' heads with DPP lane permutes
// (no LDS, no scalar round trips) and the winning lane pops its head.
#pragma once

#include <limits.h>

#include "common.h"

namespace moe {

__device__ __forceinline__ uint32_t f32_order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const uint32_t rlo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false);
  const uint32_t rhi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false);
  return ((uint64_t)rhi << 32) | rlo;
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t max_step(uint64_t v) {
  const uint64_t o = dpp_u64<CTRL, ROW_MASK>(v);
  return o > v ? o : v;
}
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// Wave-wide maximum of a 64-bit key; uniform result.  In-row butterfly (16 lanes), then
// row 0 -> row 1 and row 2 -> row 3 (row_bcast15), then rows 0-1 -> rows 2-3 (row_bcast31);
// lane 63 ends with the maximum of all 64 lanes.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_step<kDppXor1>(v);
  v = max_step<kDppXor2>(v);
  v = max_step<kDppHalfMirror>(v);
  v = max_step<kDppMirror>(v);
  v = max_step<kDppRowBcast15, 0xA>(v);
  v = max_step<kDppRowBcast31, 0xC>(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// NV = keys per lane (E <= 64 * NV).  Lanes 0..k-1 write ids_out[lane] and w_out[lane].
template <int NV>
__device__ __forceinline__ void select_token_nv(const float* lrow, int E, int k, int lane,
                                                int* ids_out, float* w_out) {
  uint64_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    const bool ok = e < E;
    const float l = lrow[ok ? e : 0];
    key[i] = ok ? (((uint64_t)f32_order_key(l) << 32) | (uint32_t)~e) : 0ull;
  }
  // sort the lane's keys, largest first (odd-even transposition; NV is 1..16)
#pragma unroll
  for (int r = 0; r < NV; ++r) {
#pragma unroll
    for (int i = r & 1; i + 1 < NV; i += 2) {
      const uint64_t a = key[i], b = key[i + 1];
      key[i] = a > b ? a : b;
      key[i + 1] = a > b ? b : a;
    }
  }
  uint64_t mine = 0;  // lane j keeps the j-th winner
  for (int j = 0; j < k; ++j) {
    const uint64_t w = wave_max_u64(key[0]);
    const bool pop = key[0] == w;
#pragma unroll
    for (int i = 0; i + 1 < NV; ++i) key[i] = pop ? key[i + 1] : key[i];
    key[NV - 1] = pop ? 0ull : key[NV - 1];
    mine = (lane == j) ? w : mine;
  }
  const float m = f32_from_order_key((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine >> 32), 0));
  const float v = f32_from_order_key((uint32_t)(mine >> 32));
  const float p = (lane < k) ? expf(v - m) : 0.f;
  const float ps = group_sum<16>(p);  // k <= 16: lanes 0..15 hold every selected term
  if (lane < k) {
    ids_out[lane] = (int)~(uint32_t)mine;
    w_out[lane] = p / ps;
  }
}

// One wave, one token; E <= MOE_MAX_E.
__device__ __forceinline__ void select_token(const float* lrow, int E, int k, int lane, int* ids_out,
                                             float* w_out) {
  if (E <= 64)
    select_token_nv<1>(lrow, E, k, lane, ids_out, w_out);
  else if (E <= 128)
    select_token_nv<2>(lrow, E, k, lane, ids_out, w_out);
  else if (E <= 256)
    select_token_nv<4>(lrow, E, k, lane, ids_out, w_out);
  else if (E <= 512)
    select_token_nv<8>(lrow, E, k, lane, ids_out, w_out);
  else
    select_token_nv<16>(lrow, E, k, lane, ids_out, w_out);
}

// The same selection as a SET, listed in ascending expert index (not by rank), for kernels
// that only need which experts a token uses and their weights.  The k-th largest key is
// found by a binary search over its bits with wave ballots (stopping as soon as exactly k
// keys pass), ties at the threshold go to the lowest indices, and every lane places its
// chosen experts by a prefix count of the chosen bits.  Lanes write ids_out[pos] and
// w_out[pos] for pos < k.
template <int NV>
__device__ __forceinline__ void select_set_nv(const float* lrow, int E, int k, int lane, int* ids_out,
                                              float* w_out) {
  uint32_t key[NV];
  float val[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    const bool ok = e < E;
    val[i] = lrow[ok ? e : 0];
    key[i] = ok ? f32_order_key(val[i]) : 0u;
  }
  // largest tau with count(key >= tau) >= k
  uint32_t tau = 0;
  int cnt_tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= k) {
      tau = cand;
      cnt_tau = cnt;
      if (cnt == k) break;  // exactly k keys at or above: no tie to resolve
    }
  }
  if (cnt_tau == 0) {  // tau stayed 0: every key qualifies
#pragma unroll
    for (int i = 0; i < NV; ++i) cnt_tau += __popcll(__ballot(lane + kWave * i < E));
  }
  // chosen: key > tau, plus the lowest-index keys == tau up to k in total
  int above = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) above += __popcll(__ballot(key[i] > tau && lane + kWave * i < E));
  int quota = k - above;
  uint64_t chosen[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const bool valid = lane + kWave * i < E;
    const uint64_t eq = __ballot(valid && key[i] == tau);
    const int my_rank = __popcll(eq & ((1ull << lane) - 1ull));
    const bool pick = valid && (key[i] > tau || (key[i] == tau && my_rank < quota));
    chosen[i] = __ballot(pick);
    quota -= __popcll(eq);
    quota = quota < 0 ? 0 : quota;
  }
  (void)cnt_tau;
  // weights: exp(l - m) / sum over the chosen, m = the largest logit
  float lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if ((chosen[i] >> lane) & 1ull) lmax = fmaxf(lmax, val[i]);
  const float m = wave_max(lmax);
  float psum = 0.f, p[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    p[i] = ((chosen[i] >> lane) & 1ull) ? expf(val[i] - m) : 0.f;
    psum += p[i];
  }
  const float ps = group_sum<kWave>(psum);
  int base = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if ((chosen[i] >> lane) & 1ull) {
      const int pos = base + __popcll(chosen[i] & ((1ull << lane) - 1ull));
      ids_out[pos] = lane + kWave * i;
      w_out[pos] = p[i] / ps;
    }
    base += __popcll(chosen[i]);
  }
}

__device__ __forceinline__ void select_set(const float* lrow, int E, int k, int lane, int* ids_out,
                                           float* w_out) {
  if (E <= 64)
    select_set_nv<1>(lrow, E, k, lane, ids_out, w_out);
  else if (E <= 128)
    select_set_nv<2>(lrow, E, k, lane, ids_out, w_out);
  else if (E <= 256)
    select_set_nv<4>(lrow, E, k, lane, ids_out, w_out);
  else if (E <= 512)
    select_set_nv<8>(lrow, E, k, lane, ids_out, w_out);
  else
    select_set_nv<16>(lrow, E, k, lane, ids_out, w_out);
}

}  // namespace moe
