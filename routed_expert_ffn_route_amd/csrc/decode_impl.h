// Decode path (T <= 16): the layer as three bandwidth-bound kernels with no cross-block
// synchronisation inside any of them.
//
//  stage 1  router GEMV (fp32 router rows x all T tokens, one wave per expert row) in some
//           blocks; the shared expert's gate/up GEMV + SwiGLU in the others -- it needs no
//           routing, so it runs beside the router ("Optimizing on-device inference for Apple
//           Silicon", section "Overlap independent GPU work").
//  gate/up  every block first re-derives the (tiny) selection of all T tokens from the logits,
//           one wave per token, then takes one (token, rank) slot: the block owning the first
//           occurrence of an expert streams that expert's gate and up rows once with 16-byte
//           loads, dots them with every token routed to it and applies SwiGLU in registers
//           (same page, sections "Optimize the one-row weight path" and "Reduce intermediate
//           and state traffic"; a window of several tokens touching up to 32 experts is
//           "Three ways to boost mixture-of-experts inference on NVIDIA DGX Spark", section
//           "Optimization 3").  Block 0 publishes ids and weights for the next kernel.
//  down     one lane group per output row h: y[t][h] = sum over t's k slots of
//           w * (Wd[e][h] . a_slot) + Wd_s[h] . a_s[t]; the block's waves split the slots and
//           reduce through LDS in a fixed order, so results are deterministic.
#pragma once

#include "common.h"
#include "kernels.h"
#include "select.h"

// Everything here has internal linkage: each decode_*.hip instantiates its own copies.
namespace moe {
namespace {

// ------------------------------------------------------------------------------------------
// Gate/up chunk arithmetic.  A chunk is 16 bytes of one weight row: 4 fp32, 8 bf16 or 32
// e2m1 elements (one MX block, one scale byte).  chunk_dot returns the chunk's partial dot
// product (MXFP4: before the block scale).
// ------------------------------------------------------------------------------------------
template <int WT> struct GU;
template <> struct GU<MOE_F32> { static constexpr int EPC = 4; };
template <> struct GU<MOE_BF16> { static constexpr int EPC = 8; };
template <> struct GU<MOE_MXFP4> { static constexpr int EPC = 32; };

template <int XT> struct XS;
template <> struct XS<MOE_F32> { static constexpr int BYTES = 4; };
template <> struct XS<MOE_BF16> { static constexpr int BYTES = 2; };

template <int WT, int XT>
__device__ __forceinline__ float chunk_dot(uint4 w, const uint8_t* xrow, int c);

template <>
__device__ __forceinline__ float chunk_dot<MOE_BF16, MOE_BF16>(uint4 w, const uint8_t* xrow, int c) {
  const uint4 xv = ldg16(xrow + (size_t)c * 16);
  float acc = dot2_bf16(w.x, xv.x, 0.f);
  acc = dot2_bf16(w.y, xv.y, acc);
  acc = dot2_bf16(w.z, xv.z, acc);
  return dot2_bf16(w.w, xv.w, acc);
}

template <>
__device__ __forceinline__ float chunk_dot<MOE_F32, MOE_F32>(uint4 w, const uint8_t* xrow, int c) {
  const float4 xv = *(const float4*)(xrow + (size_t)c * 16);
  float acc = __uint_as_float(w.x) * xv.x;
  acc = fmaf(__uint_as_float(w.y), xv.y, acc);
  acc = fmaf(__uint_as_float(w.z), xv.z, acc);
  return fmaf(__uint_as_float(w.w), xv.w, acc);
}

__device__ __forceinline__ float fp4_dword_dot(uint32_t q, uint4 xv, float acc) {
  acc = dot2_bf16(fp4x2_to_bf16x2<0>(q), xv.x, acc);
  acc = dot2_bf16(fp4x2_to_bf16x2<1>(q), xv.y, acc);
  acc = dot2_bf16(fp4x2_to_bf16x2<2>(q), xv.z, acc);
  return dot2_bf16(fp4x2_to_bf16x2<3>(q), xv.w, acc);
}

template <>
__device__ __forceinline__ float chunk_dot<MOE_MXFP4, MOE_BF16>(uint4 w, const uint8_t* xrow, int c) {
  const uint8_t* xp = xrow + (size_t)c * 64;
  float acc = fp4_dword_dot(w.x, ldg16(xp), 0.f);
  acc = fp4_dword_dot(w.y, ldg16(xp + 16), acc);
  acc = fp4_dword_dot(w.z, ldg16(xp + 32), acc);
  return fp4_dword_dot(w.w, ldg16(xp + 48), acc);
}

// One lane group (G lanes) computes gate and up row `row` (reduction over K = H) for every
// token in `mask` and writes out[slot][row] = silu(g) * u.  All loads of a K-slice are issued
// before any is consumed; lanes past the row end load a valid chunk and scale it by 0.
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
    int cc[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = c0 + gl + G * m;
      const bool ok = valid && c < nchunks;
      cc[m] = ok ? c : 0;
      wg[m] = ldg16(grow + (size_t)cc[m] * 16);
      wu[m] = ldg16(urow + (size_t)cc[m] * 16);
      if constexpr (WT == MOE_MXFP4) {
        sg[m] = e8m0_to_f32(gsrow[cc[m]]);
        su[m] = e8m0_to_f32(usrow[cc[m]]);
      } else {
        sg[m] = su[m] = 1.f;
      }
      if (!ok) sg[m] = su[m] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (!((mask >> t) & 1u)) continue;  // uniform
      const uint8_t* xrow = xb + (size_t)t * xstride;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        ag[t] = fmaf(sg[m], chunk_dot<WT, XT>(wg[m], xrow, cc[m]), ag[t]);
        au[t] = fmaf(su[m], chunk_dot<WT, XT>(wu[m], xrow, cc[m]), au[t]);
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
  static __device__ __forceinline__ float dot(W w, const float* a, int c) {
    const float4 x = ldf4(a + (size_t)c * 4);
    float acc = __uint_as_float(w.x) * x.x;
    acc = fmaf(__uint_as_float(w.y), x.y, acc);
    acc = fmaf(__uint_as_float(w.z), x.z, acc);
    return fmaf(__uint_as_float(w.w), x.w, acc);
  }
};
template <> struct DN<MOE_BF16> {
  static constexpr int EPC = 8;
  typedef uint4 W;
  static __device__ __forceinline__ W load(const uint8_t* row, int c) { return ldg16(row + (size_t)c * 16); }
  static __device__ __forceinline__ float dot(W w, const float* a, int c) {
    const float4 x0 = ldf4(a + (size_t)c * 8), x1 = ldf4(a + (size_t)c * 8 + 4);
    float acc = bf16lo(w.x) * x0.x;
    acc = fmaf(bf16hi(w.x), x0.y, acc);
    acc = fmaf(bf16lo(w.y), x0.z, acc);
    acc = fmaf(bf16hi(w.y), x0.w, acc);
    acc = fmaf(bf16lo(w.z), x1.x, acc);
    acc = fmaf(bf16hi(w.z), x1.y, acc);
    acc = fmaf(bf16lo(w.w), x1.z, acc);
    return fmaf(bf16hi(w.w), x1.w, acc);
  }
};
template <> struct DN<MOE_MXFP4> {
  static constexpr int EPC = 8;
  typedef uint32_t W;
  static __device__ __forceinline__ W load(const uint8_t* row, int c) { return ldg4(row + (size_t)c * 4); }
  static __device__ __forceinline__ float dot(W w, const float* a, int c) {
    const float4 x0 = ldf4(a + (size_t)c * 8), x1 = ldf4(a + (size_t)c * 8 + 4);
    const f32x2_t p0 = fp4x2_to_f32x2<0>(w), p1 = fp4x2_to_f32x2<1>(w);
    const f32x2_t p2 = fp4x2_to_f32x2<2>(w), p3 = fp4x2_to_f32x2<3>(w);
    float acc = p0.x * x0.x;
    acc = fmaf(p0.y, x0.y, acc);
    acc = fmaf(p1.x, x0.z, acc);
    acc = fmaf(p1.y, x0.w, acc);
    acc = fmaf(p2.x, x1.x, acc);
    acc = fmaf(p2.y, x1.y, acc);
    acc = fmaf(p3.x, x1.z, acc);
    return fmaf(p3.y, x1.w, acc);
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

// Router logits (blocks [0, router_blocks)) and shared-expert gate/up (the rest).
template <int XT, int SWT, int G, int NCH, int TM>
__global__ __launch_bounds__(kThreads) void dec_stage1(Args A) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if ((int)blockIdx.x < A.router_blocks) {
    const int e = blockIdx.x * kWaves + wave;
    if (e >= A.E) return;
    if (A.logits_in) {  // moe_route on given logits: copy, no router
      for (int t = lane; t < A.T; t += kWave) {
        const float l = A.logits_in[(size_t)t * A.E + e];
        A.logits[(size_t)t * A.E + e] = l;
        if (A.o_logits) A.o_logits[(size_t)t * A.E + e] = l;
      }
      return;
    }
    const float* wr = A.rw + (size_t)e * A.H;
    const uint8_t* xb = (const uint8_t*)A.x;
    const size_t xstride = (size_t)A.H * XS<XT>::BYTES;
    float acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = 0.f;
    const int nch = A.H / 4;
#pragma unroll 8
    for (int c = lane; c < nch; c += kWave) {
      const float4 w = ldf4(wr + (size_t)c * 4);
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        if (t < A.T) {
          float x0, x1, x2, x3;
          if constexpr (XT == MOE_F32) {
            const float4 xv = *(const float4*)(xb + t * xstride + (size_t)c * 16);
            x0 = xv.x; x1 = xv.y; x2 = xv.z; x3 = xv.w;
          } else {
            const uint2 xv = ldg8(xb + t * xstride + (size_t)c * 8);
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
  } else {
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
__global__ __launch_bounds__(kThreads) void dec_gateup(Args A, int tiles) {
  __shared__ int s_ids[kDecodeMaxT * MOE_MAX_K];
  __shared__ float s_w[kDecodeMaxT * MOE_MAX_K];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int s = blockIdx.x / tiles, tile = blockIdx.x - s * tiles;
  const int T = A.T, k = A.k, S = T * k;
  // selection of every token (one wave per token), identical in every block; each token's
  // experts are listed in ascending index, which is also the slot order the down kernel reads
  for (int t = wave; t < T; t += kWaves)
    select_set(A.logits + (size_t)t * A.E, A.E, k, lane, s_ids + t * k, s_w + t * k);
  __syncthreads();
  if (blockIdx.x == 0) {  // publish the routing for the down kernel
    for (int i = threadIdx.x; i < S; i += kThreads) {
      A.ids[i] = s_ids[i];
      A.cw[i] = s_w[i];
    }
  }
  // this block's expert and the tokens routed to it; only the first token's slot works
  const int t0 = s / k, e = s_ids[s];
  unsigned mask = 0;
  int slots[TM];
  bool owner = true;
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    slots[t] = 0;
    if (t < T) {
      for (int j = 0; j < k; ++j) {
        if (s_ids[t * k + j] == e) {
          if (t < t0) owner = false;
          mask |= 1u << t;
          slots[t] = t * k + j;
        }
      }
    }
  }
  if (!owner) return;
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
  const int nch = A.I / DN<WT>::EPC;
  const size_t rb = row_bytes<WT>(A.I);
  float acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = 0.f;

  for (int c0 = 0; c0 < nch; c0 += G * NCH) {
    int cc[NCH];
    float okf[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = c0 + gl + G * m;
      cc[m] = c < nch ? c : 0;
      okf[m] = c < nch ? 1.f : 0.f;
    }
    for (int s0 = wave; s0 < S; s0 += kWaves * US) {
      typename DN<WT>::W wv[US][NCH];
      float sc[US][NCH];
      int eu[US];
#pragma unroll
      for (int u = 0; u < US; ++u) eu[u] = A.ids[min(s0 + kWaves * u, S - 1)];
#pragma unroll
      for (int u = 0; u < US; ++u) {
        const uint8_t* row = (const uint8_t*)A.down + ((size_t)eu[u] * A.H + hh) * rb;
#pragma unroll
        for (int m = 0; m < NCH; ++m) {
          wv[u][m] = DN<WT>::load(row, cc[m]);
          float scale = 1.f;
          if constexpr (WT == MOE_MXFP4)
            scale = e8m0_to_f32(A.ds[((size_t)eu[u] * A.H + hh) * (A.I / 32) + cc[m] / 4]);
          sc[u][m] = okf[m] * scale;
        }
      }
#pragma unroll
      for (int u = 0; u < US; ++u) {
        const int s = s0 + kWaves * u;
        if (s < S) {  // uniform
          const int t = s / A.k;
          const float* arow = A.a + (size_t)s * A.I;
          float part = 0.f;
#pragma unroll
          for (int m = 0; m < NCH; ++m) part = fmaf(sc[u][m], DN<WT>::dot(wv[u][m], arow, cc[m]), part);
          part *= A.cw[s];
#pragma unroll
          for (int tt = 0; tt < TM; ++tt) acc[tt] += (tt == t) ? part : 0.f;
        }
      }
    }
  }
  // shared expert: its chunks are split over the block's waves
  if (A.Is > 0) {
    const int nchs = A.Is / DN<SWT>::EPC;
    const uint8_t* srow = (const uint8_t*)A.sdown + (size_t)hh * row_bytes<SWT>(A.Is);
    for (int cb = wave * G; cb < nchs; cb += kWaves * G) {
      const int c = cb + gl;
      const int ccs = c < nchs ? c : 0;
      const float okf = c < nchs ? 1.f : 0.f;
      const typename DN<SWT>::W w = DN<SWT>::load(srow, ccs);
#pragma unroll
      for (int t = 0; t < TM; ++t)
        if (t < A.T) acc[t] = fmaf(okf, DN<SWT>::dot(w, A.a_sh + (size_t)t * A.Is, ccs), acc[t]);
    }
  }
  __shared__ float s_part[kWaves][TM][RB];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const float v = group_sum<G>(acc[t]);
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
// Launch: (G, NCH) chosen per kernel from a preference list, TM from T.
// ------------------------------------------------------------------------------------------
struct GN { int G, NCH; };
// gate/up (reduction over H): two rows per wave with 8 chunks per lane for one token;
// wider groups when several tokens share the x registers
constexpr GN kGU1[] = {{32, 8}, {64, 4}, {64, 5}, {16, 5}, {16, 4}, {32, 1}, {16, 1}, {64, 1}, {64, 2}, {64, 8}};
constexpr GN kGUn[] = {{64, 4}, {64, 5}, {16, 5}, {16, 4}, {64, 1}, {64, 2}, {32, 1}, {16, 1}, {32, 8}, {64, 8}};
// down (reduction over I): four rows per wave
constexpr GN kDN[] = {{16, 4}, {16, 6}, {16, 5}, {16, 3}, {16, 8}, {16, 2}, {16, 1}, {64, 8}};
constexpr int kNGU = sizeof(kGU1) / sizeof(kGU1[0]);
constexpr int kNDN = sizeof(kDN) / sizeof(kDN[0]);

// First entry with the fewest idle chunk slots; the last entry (64, 8) walks long rows in
// slices when nothing covers the row.
template <int N>
int pick_gn(const GN (&list)[N], int nchunks) {
  int best = N - 1, waste = 1 << 30;
  for (int i = 0; i < N; ++i) {
    const int cap = list[i].G * list[i].NCH;
    if (cap < nchunks) continue;
    if (cap - nchunks < waste) {
      best = i;
      waste = cap - nchunks;
    }
  }
  return best;
}

template <int XT, int SWT, int TM, const GN* L>
void* stage1_fn(int gi) {
  switch (gi) {
#define C(i) case i: return (void*)dec_stage1<XT, SWT, L[i].G, L[i].NCH, TM>;
    C(0) C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8) C(9)
#undef C
  }
  return nullptr;
}
template <int XT, int WT, int TM, const GN* L>
void* gateup_fn(int gi) {
  switch (gi) {
#define C(i) case i: return (void*)dec_gateup<XT, WT, L[i].G, L[i].NCH, TM>;
    C(0) C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8) C(9)
#undef C
  }
  return nullptr;
}
template <int WT, int SWT, int TM>
void* down_fn(int gi) {
  switch (gi) {
#define C(i) case i: return (void*)dec_down<WT, SWT, kDN[i].G, kDN[i].NCH, TM, (kDN[i].NCH >= 6 ? 1 : 2)>;
    C(0) C(1) C(2) C(3) C(4) C(5) C(6) C(7)
#undef C
  }
  return nullptr;
}

int gu_epc(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 8 : 32; }
int dn_epc(int dt) { return dt == MOE_F32 ? 4 : 8; }

template <int XT, int WT, int SWT, int TM>
int launch_decode_t(Args A, hipStream_t st, bool route_only, const LaunchHook& hook) {
  constexpr const GN* GUL = TM == 1 ? kGU1 : kGUn;
  const int S = A.T * A.k;
  const int g1 = pick_gn(TM == 1 ? kGU1 : kGUn, A.H / gu_epc(SWT));
  const int rb1 = kWaves * (kWave / GUL[g1].G);
  A.router_blocks = (A.E + kWaves - 1) / kWaves;
  A.shared_blocks = (route_only || A.Is == 0) ? 0 : (A.Is + rb1 - 1) / rb1;
  const int g2 = pick_gn(TM == 1 ? kGU1 : kGUn, A.H / gu_epc(WT));
  const int rb2 = kWaves * (kWave / GUL[g2].G);
  const int tiles = (A.I + rb2 - 1) / rb2;
  const int g3 = pick_gn(kDN, A.I / dn_epc(WT));
  const int rb3 = kWave / kDN[g3].G;
  void* f1 = stage1_fn<XT, SWT, TM, GUL>(g1);
  void* f2 = gateup_fn<XT, WT, TM, GUL>(g2);
  void* f3 = down_fn<WT, SWT, TM>(g3);

  void* args1[] = {&A};
  hook.pre("dec_router_shared", st);
  hipError_t err = hipLaunchKernel(f1, dim3(A.router_blocks + A.shared_blocks), dim3(kThreads), args1, 0, st);
  hook.post(st);
  if (err != hipSuccess) return MOE_EHIP;
  if (route_only) return MOE_OK;

  int tl = tiles;
  void* args2[] = {&A, &tl};
  hook.pre("dec_gateup", st);
  err = hipLaunchKernel(f2, dim3(S * tiles), dim3(kThreads), args2, 0, st);
  hook.post(st);
  if (err != hipSuccess) return MOE_EHIP;

  void* args3[] = {&A};
  hook.pre("dec_down", st);
  err = hipLaunchKernel(f3, dim3((A.H + rb3 - 1) / rb3), dim3(kThreads), args3, 0, st);
  hook.post(st);
  if (err != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

template <int XT, int WT, int SWT>
int launch_decode_dt(Args A, hipStream_t st, bool route_only, const LaunchHook& hook) {
  if (A.T <= 1) return launch_decode_t<XT, WT, SWT, 1>(A, st, route_only, hook);
  if (A.T <= 4) return launch_decode_t<XT, WT, SWT, 4>(A, st, route_only, hook);
  return launch_decode_t<XT, WT, SWT, 16>(A, st, route_only, hook);
}

}  // namespace
}  // namespace moe
