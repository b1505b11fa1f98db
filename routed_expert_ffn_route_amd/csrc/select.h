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

// Inclusive prefix sum over the 64 lanes: a 16-lane Hillis-Steele scan on DPP row shifts,
// then each row adds the last lane of the rows below it (row_bcast 15 and 31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
  return v;
}

// The same selection as a SET, listed in ascending expert index (not by rank), for kernels
// that only need which experts a token uses and their weights.  The k-th largest 32-bit
// order key is found by a radix select, eight bits per pass from the top: each pass counts
// the candidates' next digit in a 256-bin LDS histogram (hist: 512 words private to the
// wave), a prefix sum over the bins taken from the largest digit down locates the digit that
// holds the k-th key, and the candidates narrow to that digit; the search stops as soon as
// that digit's whole bin is taken.  Ties at the threshold go to the lowest indices; the
// chosen experts are placed in ascending id by a prefix count of the chosen bits.  Lane
// l < k writes ids_out[l] and w_out[l].
template <int NV>
__device__ __forceinline__ void select_set_nv(const float* lrow, int E, int k, int lane, unsigned* hist,
                                              int* ids_out, float* w_out) {
  uint32_t key[NV];
  float val[NV];
  bool ok[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    ok[i] = e < E;
    val[i] = lrow[ok[i] ? e : 0];
    key[i] = f32_order_key(val[i]);
  }
  // hist[b] counts digit 255 - b, so lane l's four words hold digits 255-4l down to 252-4l.
  // Two histograms alternate; each is cleared right after it is read, off the critical path.
  ((uint4*)hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
  ((uint4*)hist)[kWave + lane] = make_uint4(0u, 0u, 0u, 0u);
  uint32_t prefix = 0;
  int need = k;  // rank of the wanted key among the remaining candidates
  int shift = 24;  // after the loop: the shift of the last digit taken (0 after all four)
  for (int p = 0; p < 4; ++p) {
    shift = 24 - 8 * p;
    unsigned* hp = hist + 256 * (p & 1);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const bool cand = ok[i] && (p == 0 || (key[i] >> (shift + 8)) == prefix);
      if (cand) atomicAdd(&hp[255u - ((key[i] >> shift) & 255u)], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    const uint4 h = ((const uint4*)hp)[lane];
    ((uint4*)hp)[lane] = make_uint4(0u, 0u, 0u, 0u);
    const int sum = (int)(h.x + h.y + h.z + h.w);
    const int incl = wave_incl_scan(sum);
    const uint64_t hit = __ballot(incl >= need);
    const int L = __builtin_ctzll(hit);  // the wanted key's digit is in lane L's bins
    int above = __builtin_amdgcn_readlane(incl - sum, L);
    const int c0 = __builtin_amdgcn_readlane((int)h.x, L), c1 = __builtin_amdgcn_readlane((int)h.y, L);
    const int c2 = __builtin_amdgcn_readlane((int)h.z, L), c3 = __builtin_amdgcn_readlane((int)h.w, L);
    int j = 0, c = c0;
    if (above + c0 < need) {
      above += c0;
      j = 1;
      c = c1;
      if (above + c1 < need) {
        above += c1;
        j = 2;
        c = c2;
        if (above + c2 < need) {
          above += c2;
          j = 3;
          c = c3;
        }
      }
    }
    need -= above;
    prefix = (prefix << 8) | (uint32_t)(255 - (4 * L + j));
    if (c == need) break;  // the whole bin is taken: no tie inside it to resolve
  }
  // chosen: (key >> shift) above prefix, plus the lowest-index `need` keys equal to it (one
  // ballot each; a per-lane rank only when the threshold's ties outnumber the keys still wanted)
  int quota = need;
  uint64_t chosen[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint32_t kh = key[i] >> shift;
    const uint64_t gt = __ballot(ok[i] && kh > prefix);
    const uint64_t eq = __ballot(ok[i] && kh == prefix);
    const int ne = __popcll(eq);
    uint64_t take = eq;
    if (ne > quota) {  // uniform
      const int my_rank = __popcll(eq & ((1ull << lane) - 1ull));
      take = __ballot(((eq >> lane) & 1ull) && my_rank < quota);
    }
    chosen[i] = gt | take;
    quota = quota > ne ? quota - ne : 0;
  }
  // the k chosen (value, id) pairs, in ascending id, gathered into lanes 0..k-1 through the
  // (now free) histogram words; weights exp(l - m) / sum over the chosen, m = the largest,
  // reduced over those k <= 16 lanes
  float* gv = (float*)hist;
  int* gid = (int*)hist + kWave;
  int base = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if ((chosen[i] >> lane) & 1ull) {
      const int pos = base + __popcll(chosen[i] & ((1ull << lane) - 1ull));
      gv[pos] = val[i];
      gid[pos] = lane + kWave * i;
    }
    base += __popcll(chosen[i]);
  }
  __builtin_amdgcn_wave_barrier();
  const bool act = lane < k;
  const float v = act ? gv[lane] : -INFINITY;
  const int id = act ? gid[lane] : 0;
  float m = v;  // maximum over the 16-lane row holding them
  m = fmaxf(m, dpp_f<kDppXor1>(m));
  m = fmaxf(m, dpp_f<kDppXor2>(m));
  m = fmaxf(m, dpp_f<kDppHalfMirror>(m));
  m = fmaxf(m, dpp_f<kDppMirror>(m));
  const float pe = act ? expf(v - m) : 0.f;
  const float ps = group_sum<16>(pe);
  if (act) {
    ids_out[lane] = id;
    w_out[lane] = pe / ps;
  }
}

__device__ __forceinline__ void select_set(const float* lrow, int E, int k, int lane, unsigned* hist,
                                           int* ids_out, float* w_out) {
  if (E <= 64)
    select_set_nv<1>(lrow, E, k, lane, hist, ids_out, w_out);
  else if (E <= 128)
    select_set_nv<2>(lrow, E, k, lane, hist, ids_out, w_out);
  else if (E <= 256)
    select_set_nv<4>(lrow, E, k, lane, hist, ids_out, w_out);
  else if (E <= 512)
    select_set_nv<8>(lrow, E, k, lane, hist, ids_out, w_out);
  else
    select_set_nv<16>(lrow, E, k, lane, hist, ids_out, w_out);
}

}  // namespace moe
