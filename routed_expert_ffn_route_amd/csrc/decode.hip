// Decode path (T <= 16): the layer as three bandwidth-bound kernels.
//
//  stage 1  router GEMV (fp32 router rows, all T tokens) in some blocks, the shared expert's
//           gate/up GEMV + SwiGLU in the others (it needs no routing, so it hides the
//           router); the last router block to finish selects top-k per token and writes
//           the decode plan ("Optimizing on-device inference for Apple Silicon", sections
//           "Overlap independent GPU work" and "Keep expert routing on the GPU").
//  gate/up  one lane group per (distinct expert, intermediate row): streams the gate and up
//           rows once with 16-byte loads and dots them with every token routed to that
//           expert, SwiGLU in registers (same page, sections "Optimize the one-row weight
//           path" and "Reduce intermediate and state traffic"; the window of several tokens
//           touching up to 32 experts is "Three ways to boost mixture-of-experts inference on
//           NVIDIA DGX Spark", section "Optimization 3").
//  down     one lane group per output row h: sum over the T*k slots of w * (Wd[e][h] . a) plus
//           the shared expert's Wd_s[h] . a_s, the four waves of a block splitting the slots
//           and reducing through LDS in a fixed order (deterministic).
#include <limits.h>

#include "common.h"
#include "kernels.h"
#include "select.h"

namespace moe {

// Exclusive scan of one int per thread over a 256-thread block.
__device__ int block_excl_scan256(int v, int* s_tmp) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += n;
  }
  if (lane == kWave - 1) s_tmp[wave] = incl;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += s_tmp[w];
  __syncthreads();
  return off + incl - v;
}

// Runs in the last router block (256 threads): selection for all T tokens, then the plan.
__device__ void select_and_plan(const Args& A) {
  __shared__ int s_ids[kDecodeMaxT * MOE_MAX_K];
  __shared__ float s_w[kDecodeMaxT * MOE_MAX_K];
  __shared__ int s_d[kDecodeMaxT * MOE_MAX_K];
  __shared__ unsigned s_bits[MOE_MAX_E / 32];
  __shared__ int s_pref[MOE_MAX_E / 32];
  __shared__ unsigned s_mask[kDecodeMaxT * MOE_MAX_K];
  __shared__ int s_tmp[4];
  __shared__ int s_nd;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int T = A.T, k = A.k, E = A.E, S = T * k;
  DecodePlan P(A.plan, min(S, E), T, S);

  if (tid < MOE_MAX_E / 32) s_bits[tid] = 0;
  s_mask[tid] = 0;  // 256 == kDecodeMaxT * MOE_MAX_K entries
  for (int t = wave; t < T; t += 4)
    select_token(A.logits + (size_t)t * E, E, k, lane, s_ids + t * k, s_w + t * k);
  __syncthreads();
  if (tid < S) atomicOr(&s_bits[s_ids[tid] >> 5], 1u << (s_ids[tid] & 31));
  __syncthreads();
  if (wave == 0) {
    const int nw = (E + 31) / 32;
    int p = (lane < nw) ? __popc(s_bits[lane]) : 0;
    int incl = p;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      int n = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += n;
    }
    if (lane < MOE_MAX_E / 32) s_pref[lane] = incl - p;
    if (lane == kWave - 1) s_nd = incl;
  }
  __syncthreads();
  const int nd = s_nd;
  if (tid < S) {
    const int e = s_ids[tid], t = tid / k;
    const int d = s_pref[e >> 5] + __popc(s_bits[e >> 5] & ((1u << (e & 31)) - 1u));
    s_d[tid] = d;
    atomicOr(&s_mask[d], 1u << t);
    P.dexp()[d] = e;
    P.dslot()[d * T + t] = tid;
    P.dw()[d * T + t] = s_w[tid];
    A.ids[tid] = e;
    A.cw[tid] = s_w[tid];
    if (A.o_ids) {
      A.o_ids[tid] = e;
      A.o_w[tid] = s_w[tid];
    }
  }
  __syncthreads();
  const int cnt = (tid < nd) ? __popc(s_mask[tid]) : 0;
  const int base = block_excl_scan256(cnt, s_tmp);
  __shared__ int s_base[kDecodeMaxT * MOE_MAX_K];
  s_base[tid] = base;
  if (tid < nd) P.dmask()[tid] = s_mask[tid];
  __syncthreads();
  if (tid < S) {
    const int d = s_d[tid], t = tid / k;
    const int pos = s_base[d] + __popc(s_mask[d] & ((1u << t) - 1u));
    P.sl_exp()[pos] = s_ids[tid];
    P.sl_tok()[pos] = t;
    P.sl_slot()[pos] = tid;
    P.sl_w()[pos] = s_w[tid];
  }
  if (tid == 0) *P.nd() = nd;
}

// ------------------------------------------------------------------------------------------
// Gate/up chunk arithmetic.  A chunk is 16 bytes of one weight row: 4 fp32, 8 bf16 or 32
// e2m1 elements (one MX block, one scale byte).
// ------------------------------------------------------------------------------------------
template <int WT> struct GU;
template <> struct GU<MOE_F32> { static constexpr int EPC = 4; };
template <> struct GU<MOE_BF16> { static constexpr int EPC = 8; };
template <> struct GU<MOE_MXFP4> { static constexpr int EPC = 32; };

template <int XT> struct XS;
template <> struct XS<MOE_F32> { static constexpr int BYTES = 4; };
template <> struct XS<MOE_BF16> { static constexpr int BYTES = 2; };

// acc + w . x over one chunk (c = chunk index within the row; xrow = token row of x).
template <int WT, int XT>
__device__ __forceinline__ float chunk_dot(uint4 w, const uint8_t* xrow, int c, float acc);

template <>
__device__ __forceinline__ float chunk_dot<MOE_BF16, MOE_BF16>(uint4 w, const uint8_t* xrow, int c,
                                                               float acc) {
  uint4 xv = ldg16(xrow + (size_t)c * 16);
  acc = dot2_bf16(w.x, xv.x, acc);
  acc = dot2_bf16(w.y, xv.y, acc);
  acc = dot2_bf16(w.z, xv.z, acc);
  acc = dot2_bf16(w.w, xv.w, acc);
  return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<MOE_F32, MOE_F32>(uint4 w, const uint8_t* xrow, int c,
                                                             float acc) {
  float4 xv = *(const float4*)(xrow + (size_t)c * 16);
  acc = fmaf(__uint_as_float(w.x), xv.x, acc);
  acc = fmaf(__uint_as_float(w.y), xv.y, acc);
  acc = fmaf(__uint_as_float(w.z), xv.z, acc);
  acc = fmaf(__uint_as_float(w.w), xv.w, acc);
  return acc;
}

__device__ __forceinline__ float fp4_dword_dot(uint32_t q, uint4 xv, float acc) {
  acc = dot2_bf16(fp4x2_to_bf16x2<0>(q), xv.x, acc);
  acc = dot2_bf16(fp4x2_to_bf16x2<1>(q), xv.y, acc);
  acc = dot2_bf16(fp4x2_to_bf16x2<2>(q), xv.z, acc);
  acc = dot2_bf16(fp4x2_to_bf16x2<3>(q), xv.w, acc);
  return acc;
}

// Unscaled: the caller multiplies by the block's e8m0 scale (a power of two, exact).
template <>
__device__ __forceinline__ float chunk_dot<MOE_MXFP4, MOE_BF16>(uint4 w, const uint8_t* xrow, int c,
                                                                float acc) {
  const uint8_t* xp = xrow + (size_t)c * 64;
  acc = fp4_dword_dot(w.x, ldg16(xp), acc);
  acc = fp4_dword_dot(w.y, ldg16(xp + 16), acc);
  acc = fp4_dword_dot(w.z, ldg16(xp + 32), acc);
  acc = fp4_dword_dot(w.w, ldg16(xp + 48), acc);
  return acc;
}

// One lane group of G lanes computes gate and up row `row` (K = H reduction) for every token
// in `mask` and writes a[slot][row] = silu(g) * u.  Rows are byte pointers to the row
// starts; `xb` is x as bytes with row stride xstride.  Rows longer than G*NCH chunks are
// walked in slices.
template <int XT, int WT, int G, int NCH, int TM>
__device__ __forceinline__ void gateup_row(const uint8_t* grow, const uint8_t* urow,
                                           const uint8_t* gsrow, const uint8_t* usrow,
                                           int nchunks, const uint8_t* xb, size_t xstride,
                                           unsigned mask, const int* slots, float* out,
                                           int out_ld, int row, int gl, bool valid) {
  float ag[TM], au[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) ag[t] = au[t] = 0.f;
  for (int c0 = 0; c0 < nchunks; c0 += G * NCH) {
    uint4 wg[NCH], wu[NCH];
    float sg[NCH], su[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = c0 + gl + G * m;
      const bool ok = valid && c < nchunks;
      const int cc = ok ? c : 0;
      wg[m] = ldg16(grow + (size_t)cc * 16);
      wu[m] = ldg16(urow + (size_t)cc * 16);
      if constexpr (WT == MOE_MXFP4) {
        sg[m] = ok ? e8m0_to_f32(gsrow[cc]) : 0.f;
        su[m] = ok ? e8m0_to_f32(usrow[cc]) : 0.f;
      } else {
        if (!ok) {
          wg[m] = make_uint4(0, 0, 0, 0);
          wu[m] = make_uint4(0, 0, 0, 0);
        }
        sg[m] = su[m] = 1.f;
      }
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (!((mask >> t) & 1u)) continue;
      const uint8_t* xrow = xb + (size_t)t * xstride;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        const int c = c0 + gl + G * m;
        const int cc = (valid && c < nchunks) ? c : 0;
        if constexpr (WT == MOE_MXFP4) {
          ag[t] = fmaf(sg[m], chunk_dot<WT, XT>(wg[m], xrow, cc, 0.f), ag[t]);
          au[t] = fmaf(su[m], chunk_dot<WT, XT>(wu[m], xrow, cc, 0.f), au[t]);
        } else {
          ag[t] = chunk_dot<WT, XT>(wg[m], xrow, cc, ag[t]);
          au[t] = chunk_dot<WT, XT>(wu[m], xrow, cc, au[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (!((mask >> t) & 1u)) continue;
    const float g = group_sum<G>(ag[t]);
    const float u = group_sum<G>(au[t]);
    if (gl == 0 && valid) out[(size_t)slots[t] * out_ld + row] = silu(g) * u;
  }
}

// ------------------------------------------------------------------------------------------
// Down chunk arithmetic.  A chunk is 4 (fp32) or 8 (bf16, e2m1) consecutive elements of one
// Wd row; the activation chunk is the same elements of a (fp32).
// ------------------------------------------------------------------------------------------
template <int WT> struct DN;
template <> struct DN<MOE_F32> {
  static constexpr int EPC = 4;
  typedef uint4 W;
  static __device__ __forceinline__ W load(const uint8_t* row, int c) { return ldg16(row + (size_t)c * 16); }
  static __device__ __forceinline__ W zero() { return make_uint4(0, 0, 0, 0); }
  static __device__ __forceinline__ float dot(W w, const float* a, int c, float acc) {
    float4 x = ldf4(a + (size_t)c * 4);
    acc = fmaf(__uint_as_float(w.x), x.x, acc);
    acc = fmaf(__uint_as_float(w.y), x.y, acc);
    acc = fmaf(__uint_as_float(w.z), x.z, acc);
    acc = fmaf(__uint_as_float(w.w), x.w, acc);
    return acc;
  }
};
template <> struct DN<MOE_BF16> {
  static constexpr int EPC = 8;
  typedef uint4 W;
  static __device__ __forceinline__ W load(const uint8_t* row, int c) { return ldg16(row + (size_t)c * 16); }
  static __device__ __forceinline__ W zero() { return make_uint4(0, 0, 0, 0); }
  static __device__ __forceinline__ float dot(W w, const float* a, int c, float acc) {
    float4 x0 = ldf4(a + (size_t)c * 8), x1 = ldf4(a + (size_t)c * 8 + 4);
    acc = fmaf(bf16lo(w.x), x0.x, acc);
    acc = fmaf(bf16hi(w.x), x0.y, acc);
    acc = fmaf(bf16lo(w.y), x0.z, acc);
    acc = fmaf(bf16hi(w.y), x0.w, acc);
    acc = fmaf(bf16lo(w.z), x1.x, acc);
    acc = fmaf(bf16hi(w.z), x1.y, acc);
    acc = fmaf(bf16lo(w.w), x1.z, acc);
    acc = fmaf(bf16hi(w.w), x1.w, acc);
    return acc;
  }
};
template <> struct DN<MOE_MXFP4> {
  static constexpr int EPC = 8;
  typedef uint32_t W;
  static __device__ __forceinline__ W load(const uint8_t* row, int c) { return ldg4(row + (size_t)c * 4); }
  static __device__ __forceinline__ W zero() { return 0u; }
  // unscaled; caller applies the e8m0 scale of block c/4
  static __device__ __forceinline__ float dot(W w, const float* a, int c, float acc) {
    float4 x0 = ldf4(a + (size_t)c * 8), x1 = ldf4(a + (size_t)c * 8 + 4);
    f32x2_t p0 = fp4x2_to_f32x2<0>(w), p1 = fp4x2_to_f32x2<1>(w);
    f32x2_t p2 = fp4x2_to_f32x2<2>(w), p3 = fp4x2_to_f32x2<3>(w);
    acc = fmaf(p0.x, x0.x, acc);
    acc = fmaf(p0.y, x0.y, acc);
    acc = fmaf(p1.x, x0.z, acc);
    acc = fmaf(p1.y, x0.w, acc);
    acc = fmaf(p2.x, x1.x, acc);
    acc = fmaf(p2.y, x1.y, acc);
    acc = fmaf(p3.x, x1.z, acc);
    acc = fmaf(p3.y, x1.w, acc);
    return acc;
  }
};

template <int WT>
__device__ __forceinline__ size_t row_bytes(int K) {
  return WT == MOE_F32 ? (size_t)K * 4 : WT == MOE_BF16 ? (size_t)K * 2 : (size_t)K / 2;
}

// ------------------------------------------------------------------------------------------
// Kernels
// ------------------------------------------------------------------------------------------
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int XT, int SWT, int G, int NCH, int TM>
__global__ __launch_bounds__(kThreads) void dec_stage1(Args A) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if ((int)blockIdx.x < A.router_blocks) {
    // ---- router GEMV: one wave per expert row, all tokens ----
    const int e = blockIdx.x * kWaves + wave;
    if (e < A.E) {
      if (A.logits_in) {
        if (lane < A.T) {
          float l = A.logits_in[(size_t)lane * A.E + e];
          A.logits[(size_t)lane * A.E + e] = l;
          if (A.o_logits) A.o_logits[(size_t)lane * A.E + e] = l;
        }
      } else {
        const float* wr = A.rw + (size_t)e * A.H;
        const uint8_t* xb = (const uint8_t*)A.x;
        const size_t xstride = (size_t)A.H * XS<XT>::BYTES;
        float acc[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) acc[t] = 0.f;
        const int nch = A.H / 4;
#pragma unroll 4
        for (int c = lane; c < nch; c += kWave) {
          float4 w = ldf4(wr + (size_t)c * 4);
#pragma unroll
          for (int t = 0; t < TM; ++t) {
            if (t < A.T) {
              float x0, x1, x2, x3;
              if constexpr (XT == MOE_F32) {
                float4 xv = *(const float4*)(xb + t * xstride + (size_t)c * 16);
                x0 = xv.x; x1 = xv.y; x2 = xv.z; x3 = xv.w;
              } else {
                uint2 xv = ldg8(xb + t * xstride + (size_t)c * 8);
                x0 = bf16lo(xv.x); x1 = bf16hi(xv.x); x2 = bf16lo(xv.y); x3 = bf16hi(xv.y);
              }
              acc[t] = fmaf(w.x, x0, acc[t]);
              acc[t] = fmaf(w.y, x1, acc[t]);
              acc[t] = fmaf(w.z, x2, acc[t]);
              acc[t] = fmaf(w.w, x3, acc[t]);
            }
          }
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          if (t < A.T) {
            float s = group_sum<kWave>(acc[t]);
            if (lane == 0) {
              if (A.rbias) s += A.rbias[(size_t)t * A.bias_stride + e];
              A.logits[(size_t)t * A.E + e] = s;
              if (A.o_logits) A.o_logits[(size_t)t * A.E + e] = s;
            }
          }
        }
      }
    }
    // ---- completion count; the last router block selects and plans ----
    __threadfence();
    __syncthreads();
    __shared__ int s_last;
    if (threadIdx.x == 0) {
      unsigned old = atomicAdd(A.ctr, 1u);
      s_last = (old == (unsigned)A.router_blocks - 1u);
      if (s_last) atomicExch(A.ctr, 0u);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    select_and_plan(A);
  } else {
    // ---- shared expert gate/up + SwiGLU for all tokens ----
    constexpr int RB = kWave / G;
    const int grp = lane / G, gl = lane % G;
    const int row = (blockIdx.x - A.router_blocks) * (kWaves * RB) + wave * RB + grp;
    const bool valid = row < A.Is;
    const int r = valid ? row : 0;
    const size_t rb = row_bytes<SWT>(A.H);
    int slots[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) slots[t] = t;
    const unsigned mask = (A.T >= 32) ? 0xffffffffu : ((1u << A.T) - 1u);
    gateup_row<XT, SWT, G, NCH, TM>((const uint8_t*)A.sgate + r * rb, (const uint8_t*)A.sup + r * rb,
                                    nullptr, nullptr, A.H / GU<SWT>::EPC, (const uint8_t*)A.x,
                                    (size_t)A.H * XS<XT>::BYTES, mask, slots, A.a_sh, A.Is, row, gl,
                                    valid);
  }
}

template <int XT, int WT, int G, int NCH, int TM>
__global__ __launch_bounds__(kThreads) void dec_gateup(Args A, int tiles_per_d) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int S = A.T * A.k;
  DecodePlan P(A.plan, min(S, A.E), A.T, S);
  const int d = blockIdx.x / tiles_per_d, tile = blockIdx.x - d * tiles_per_d;
  if (d >= *P.nd()) return;
  const int e = P.dexp()[d];
  const unsigned mask = P.dmask()[d];
  int slots[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) slots[t] = ((mask >> t) & 1u) ? P.dslot()[d * A.T + t] : 0;
  constexpr int RB = kWave / G;
  const int grp = lane / G, gl = lane % G;
  const int row = tile * (kWaves * RB) + wave * RB + grp;
  const bool valid = row < A.I;
  const size_t r = (size_t)e * A.I + (valid ? row : 0);
  const size_t rb = row_bytes<WT>(A.H);
  const uint8_t *gsr = nullptr, *usr = nullptr;
  if constexpr (WT == MOE_MXFP4) {
    gsr = A.gs + r * (A.H / 32);
    usr = A.us + r * (A.H / 32);
  }
  gateup_row<XT, WT, G, NCH, TM>((const uint8_t*)A.gate + r * rb, (const uint8_t*)A.up + r * rb, gsr,
                                 usr, A.H / GU<WT>::EPC, (const uint8_t*)A.x,
                                 (size_t)A.H * XS<XT>::BYTES, mask, slots, A.a, A.I, row, gl, valid);
}

template <int WT, int SWT, int G, int NCH, int TM, int US>
__global__ __launch_bounds__(kThreads) void dec_down(Args A) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  constexpr int RB = kWave / G;
  const int grp = lane / G, gl = lane % G;
  const int h = blockIdx.x * RB + grp;
  const bool valid = h < A.H;
  const int hh = valid ? h : 0;
  const int S = A.T * A.k;
  DecodePlan P(A.plan, min(S, A.E), A.T, S);
  const int nch = A.I / DN<WT>::EPC;
  const size_t rb = row_bytes<WT>(A.I);
  float acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = 0.f;

  for (int s0 = wave; s0 < S; s0 += kWaves * US) {
    typename DN<WT>::W wv[US][NCH];
    float sc[US][NCH];
#pragma unroll
    for (int u = 0; u < US; ++u) {
      const int s = min(s0 + kWaves * u, S - 1);
      const int e = P.sl_exp()[s];
      const uint8_t* row = (const uint8_t*)A.down + ((size_t)e * A.H + hh) * rb;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        const int c = gl + G * m;
        const bool ok = c < nch;
        wv[u][m] = DN<WT>::load(row, ok ? c : 0);
        if (!ok) wv[u][m] = DN<WT>::zero();
        if constexpr (WT == MOE_MXFP4) {
          sc[u][m] = ok ? e8m0_to_f32(A.ds[((size_t)e * A.H + hh) * (A.I / 32) + c / 4]) : 0.f;
        } else {
          sc[u][m] = 1.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < US; ++u) {
      const int s = s0 + kWaves * u;
      if (s < S) {
        const int t = P.sl_tok()[s];
        const float wt = P.sl_w()[s];
        const float* arow = A.a + (size_t)P.sl_slot()[s] * A.I;
        float part = 0.f;
#pragma unroll
        for (int m = 0; m < NCH; ++m) {
          const int c = gl + G * m;
          const int cc = c < nch ? c : 0;
          if constexpr (WT == MOE_MXFP4)
            part = fmaf(sc[u][m], DN<WT>::dot(wv[u][m], arow, cc, 0.f), part);
          else
            part = DN<WT>::dot(wv[u][m], arow, cc, part);
        }
        part *= wt;
#pragma unroll
        for (int tt = 0; tt < TM; ++tt) acc[tt] += (tt == t) ? part : 0.f;
      }
    }
  }
  // shared expert: its chunks are split over the block's waves
  if (A.Is > 0) {
    const int nchs = A.Is / DN<SWT>::EPC;
    const uint8_t* srow = (const uint8_t*)A.sdown + (size_t)hh * row_bytes<SWT>(A.Is);
    for (int cb = wave * G; cb < nchs; cb += kWaves * G) {
      const int c = cb + gl;
      if (c < nchs) {
        typename DN<SWT>::W w = DN<SWT>::load(srow, c);
#pragma unroll
        for (int t = 0; t < TM; ++t)
          if (t < A.T) acc[t] = DN<SWT>::dot(w, A.a_sh + (size_t)t * A.Is, c, acc[t]);
      }
    }
  }
  __shared__ float s_part[kWaves][TM][RB];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    float v = group_sum<G>(acc[t]);
    if (gl == 0) s_part[wave][t][grp] = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < TM * RB; i += kThreads) {
    const int t = i / RB, g = i % RB;
    const int ho = blockIdx.x * RB + g;
    if (t < A.T && ho < A.H) {
      float v = s_part[0][t][g];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += s_part[w][t][g];
      if (A.odt == MOE_BF16)
        ((uint16_t*)A.y)[(size_t)t * A.H + ho] = f32_to_bf16(v);
      else
        ((float*)A.y)[(size_t)t * A.H + ho] = v;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Host-side dispatch
// ------------------------------------------------------------------------------------------
namespace {

// (G, NCH) shapes a lane group can cover: G lanes x NCH chunks per lane.
struct GN { int G, NCH; };
constexpr GN kGN[] = {{64, 1}, {64, 2}, {64, 4}, {64, 5}, {64, 8}, {32, 3}, {16, 4}, {16, 5}, {8, 3}};
constexpr int kNGN = sizeof(kGN) / sizeof(kGN[0]);

// Pick the (G, NCH) with the least idle chunk slots, preferring wider groups on ties;
// rows longer than 512 chunks use (64, 8) with a slice loop.
int pick_gn(int nchunks) {
  int best = -1, waste = INT_MAX;
  for (int i = 0; i < kNGN; ++i) {
    int cap = kGN[i].G * kGN[i].NCH;
    if (cap < nchunks) continue;
    int w = cap - nchunks;
    if (w < waste || (w == waste && kGN[i].G > kGN[best].G)) {
      best = i;
      waste = w;
    }
  }
  return best < 0 ? 4 : best;
}

int pick_tm(int T) { return T <= 1 ? 1 : T <= 4 ? 4 : 16; }

template <int XT, int SWT, int TM>
void* stage1_fn(int gi) {
  switch (gi) {
#define C(i) case i: return (void*)dec_stage1<XT, SWT, kGN[i].G, kGN[i].NCH, TM>;
    C(0) C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8)
#undef C
  }
  return nullptr;
}
template <int XT, int WT, int TM>
void* gateup_fn(int gi) {
  switch (gi) {
#define C(i) case i: return (void*)dec_gateup<XT, WT, kGN[i].G, kGN[i].NCH, TM>;
    C(0) C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8)
#undef C
  }
  return nullptr;
}
template <int WT, int SWT, int TM>
void* down_fn(int gi) {
  switch (gi) {
#define C(i) case i: return (void*)dec_down<WT, SWT, kGN[i].G, kGN[i].NCH, TM, (kGN[i].NCH >= 3 ? 1 : 2)>;
    C(0) C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8)
#undef C
  }
  return nullptr;
}

template <int TM>
void pick_fns(const Args& A, int g1, int g2, int g3, void** f1, void** f2, void** f3) {
  if (A.act == MOE_F32) {  // all-fp32 layer
    *f1 = stage1_fn<MOE_F32, MOE_F32, TM>(g1);
    *f2 = gateup_fn<MOE_F32, MOE_F32, TM>(g2);
    *f3 = down_fn<MOE_F32, MOE_F32, TM>(g3);
  } else if (A.wdt == MOE_BF16) {
    *f1 = stage1_fn<MOE_BF16, MOE_BF16, TM>(g1);
    *f2 = gateup_fn<MOE_BF16, MOE_BF16, TM>(g2);
    *f3 = down_fn<MOE_BF16, MOE_BF16, TM>(g3);
  } else {
    *f1 = stage1_fn<MOE_BF16, MOE_BF16, TM>(g1);
    *f2 = gateup_fn<MOE_BF16, MOE_MXFP4, TM>(g2);
    *f3 = down_fn<MOE_MXFP4, MOE_BF16, TM>(g3);
  }
}

int gu_epc(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 8 : 32; }
int dn_epc(int dt) { return dt == MOE_F32 ? 4 : 8; }

}  // namespace

int launch_decode(Args A, hipStream_t st, bool route_only, const LaunchHook& hook) {
  const int TM = pick_tm(A.T);
  const int S = A.T * A.k, D = S < A.E ? S : A.E;
  // stage 1 grid: router rows (one wave each) + shared gate/up rows
  const int g1 = pick_gn(A.H / gu_epc(A.sdt));
  const int rb1 = kWaves * (kWave / kGN[g1].G);
  A.router_blocks = (A.E + kWaves - 1) / kWaves;
  A.shared_blocks = (route_only || A.Is == 0) ? 0 : (A.Is + rb1 - 1) / rb1;
  const int g2 = pick_gn(A.H / gu_epc(A.wdt));
  const int rb2 = kWaves * (kWave / kGN[g2].G);
  const int tiles_per_d = (A.I + rb2 - 1) / rb2;
  const int g3 = pick_gn(A.I / dn_epc(A.wdt));
  const int rb3 = kWave / kGN[g3].G;

  void *f1, *f2, *f3;
  if (TM == 1)
    pick_fns<1>(A, g1, g2, g3, &f1, &f2, &f3);
  else if (TM == 4)
    pick_fns<4>(A, g1, g2, g3, &f1, &f2, &f3);
  else
    pick_fns<16>(A, g1, g2, g3, &f1, &f2, &f3);

  void* args1[] = {&A};
  hook.pre("dec_router_shared", st);
  hipError_t err = hipLaunchKernel(f1, dim3(A.router_blocks + A.shared_blocks), dim3(kThreads), args1, 0, st);
  hook.post(st);
  if (err != hipSuccess) return MOE_EHIP;
  if (route_only) return MOE_OK;

  int tpd = tiles_per_d;
  void* args2[] = {&A, &tpd};
  hook.pre("dec_gateup", st);
  err = hipLaunchKernel(f2, dim3(D * tiles_per_d), dim3(kThreads), args2, 0, st);
  hook.post(st);
  if (err != hipSuccess) return MOE_EHIP;

  void* args3[] = {&A};
  hook.pre("dec_down", st);
  err = hipLaunchKernel(f3, dim3((A.H + rb3 - 1) / rb3), dim3(kThreads), args3, 0, st);
  hook.post(st);
  if (err != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

}  // namespace moe
