// Decode path (T <= 16): the layer as four kernels with no cross-block synchronisation
// inside any of them (a kernel boundary is the cheapest device-wide barrier).
//
//  router   router GEMV: one block per expert row (fp32) x all T tokens.
//  select   (T > 1) one block: top-k + renormalised softmax per token (one wave each), then
//           the distinct experts of the window with their tokens, slots and weights (the
//           plan).  A window of several tokens touches up to T*k experts ("Three ways to boost
//           mixture-of-experts inference on NVIDIA DGX Spark", section "Optimization 3").
//           The other blocks of the launch compute the shared expert's gate/up + SwiGLU,
//           which needs no routing ("Optimizing on-device inference for Apple Silicon",
//           section "Overlap independent GPU work").
//  gate/up  block (distinct expert, row tile): streams the expert's gate and up rows once
//           with 16-byte loads, dots them with every token routed to it and applies SwiGLU
//           in registers (Apple Silicon page, sections "Optimize the one-row weight path" and
//           "Reduce intermediate and state traffic").  At T = 1 every block selects the
//           token's experts itself and the shared gate/up blocks run here instead.
//  down     one lane group per output row h: y[t][h] = Wd_s[h] . a_s[t] + sum over t's
//           experts of w * (Wd[e][h] . a); the block's waves split the shared rows' slices and
//           the distinct experts and reduce through LDS in a fixed order, so results are
//           deterministic.
#pragma once

#include <algorithm>
#include <mutex>
#include <type_traits>

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
template <> struct GU<MOE_INT4G64> { static constexpr int EPC = 32; };

template <int XT> struct XS;
template <> struct XS<MOE_F32> { static constexpr int BYTES = 4; };
template <> struct XS<MOE_BF16> { static constexpr int BYTES = 2; };

// GUC<WT, XT>: the gate and up chunks of one row pair, unpacked once (deq), then dotted
// with each routed token's x chunk; the x chunk is read once for both rows.
template <int WT, int XT> struct GUC;
template <> struct GUC<MOE_BF16, MOE_BF16> {
  typedef uint4 D;
  static __device__ __forceinline__ D deq(uint4 w) { return w; }
  static __device__ __forceinline__ void dot(const D& g, const D& u, const uint8_t* xrow, int c,
                                             float sg, float su, float& ag, float& au) {
    const uint4 xv = ldg16(xrow + (size_t)c * 16);
    float a = dot2_bf16(g.x, xv.x, 0.f), b = dot2_bf16(u.x, xv.x, 0.f);
    a = dot2_bf16(g.y, xv.y, a);
    b = dot2_bf16(u.y, xv.y, b);
    a = dot2_bf16(g.z, xv.z, a);
    b = dot2_bf16(u.z, xv.z, b);
    a = dot2_bf16(g.w, xv.w, a);
    b = dot2_bf16(u.w, xv.w, b);
    ag = fmaf(sg, a, ag);
    au = fmaf(su, b, au);
  }
};
template <> struct GUC<MOE_F32, MOE_F32> {
  typedef uint4 D;
  static __device__ __forceinline__ D deq(uint4 w) { return w; }
  static __device__ __forceinline__ void dot(const D& g, const D& u, const uint8_t* xrow, int c,
                                             float sg, float su, float& ag, float& au) {
    const float4 xv = *(const float4*)(xrow + (size_t)c * 16);
    float a = __uint_as_float(g.x) * xv.x, b = __uint_as_float(u.x) * xv.x;
    a = fmaf(__uint_as_float(g.y), xv.y, a);
    b = fmaf(__uint_as_float(u.y), xv.y, b);
    a = fmaf(__uint_as_float(g.z), xv.z, a);
    b = fmaf(__uint_as_float(u.z), xv.z, b);
    a = fmaf(__uint_as_float(g.w), xv.w, a);
    b = fmaf(__uint_as_float(u.w), xv.w, b);
    ag = fmaf(sg, a, ag);
    au = fmaf(su, b, au);
  }
};
// 32 e2m1 codes (one MX block) -> 16 bf16 pairs, exact at unit scale; the block scale is
// applied to the chunk's dot product.
template <> struct GUC<MOE_MXFP4, MOE_BF16> {
  struct D { uint32_t v[16]; };
  static __device__ __forceinline__ void deq4(uint32_t q, uint32_t* o) {
    o[0] = fp4x2_to_bf16x2<0>(q);
    o[1] = fp4x2_to_bf16x2<1>(q);
    o[2] = fp4x2_to_bf16x2<2>(q);
    o[3] = fp4x2_to_bf16x2<3>(q);
  }
  static __device__ __forceinline__ D deq(uint4 w) {
    D d;
    deq4(w.x, d.v);
    deq4(w.y, d.v + 4);
    deq4(w.z, d.v + 8);
    deq4(w.w, d.v + 12);
    return d;
  }
  // CS: bytes from one 32-element chunk of x to the next (64, or 80 in the padded LDS layout)
  template <int CS = 64>
  static __device__ __forceinline__ void dot(const D& g, const D& u, const uint8_t* xrow, int c,
                                             float sg, float su, float& ag, float& au) {
    const uint8_t* xp = xrow + (size_t)c * CS;
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 xv = ldg16(xp + 16 * q);
      a = dot2_bf16(g.v[4 * q + 0], xv.x, a);
      b = dot2_bf16(u.v[4 * q + 0], xv.x, b);
      a = dot2_bf16(g.v[4 * q + 1], xv.y, a);
      b = dot2_bf16(u.v[4 * q + 1], xv.y, b);
      a = dot2_bf16(g.v[4 * q + 2], xv.z, a);
      b = dot2_bf16(u.v[4 * q + 2], xv.z, b);
      a = dot2_bf16(g.v[4 * q + 3], xv.w, a);
      b = dot2_bf16(u.v[4 * q + 3], xv.w, b);
    }
    ag = fmaf(sg, a, ag);
    au = fmaf(su, b, au);
  }
};

// Group-wise affine 4-bit (a code q in 0..15 per weight, a bf16 scale s and bias b per 64):
// a chunk is 32 codes, half a group.  Each code pair becomes the bf16 pair (128 + q0, 128 + q1)
// (exact: bf16 holds the integers 128..143), so one dot2 per pair gives D = sum x (128 + q),
// and sum x (s q + b) = s D + (b - 128 s) X with X = sum x over the chunk.
template <> struct GUC<MOE_INT4G64, MOE_BF16> {
  struct D { uint32_t v[16]; };
  // code pair j of dword w (elements 2j, 2j + 1) -> bf16 pair 128 + q: byte j of w and byte j
  // of w >> 4 (whose low nibble is the high code) land in the two halves, then the exponent
  static __device__ __forceinline__ void deq4(uint32_t w, uint32_t* o) {
    const uint32_t w4 = w >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t sel = (uint32_t)j | 0x0C00u | ((uint32_t)(4 + j) << 16) | 0x0C000000u;
      o[j] = (__builtin_amdgcn_perm(w4, w, sel) & 0x000F000Fu) | 0x43004300u;
    }
  }
  static __device__ __forceinline__ D deq(uint4 w) {
    D d;
    deq4(w.x, d.v);
    deq4(w.y, d.v + 4);
    deq4(w.z, d.v + 8);
    deq4(w.w, d.v + 12);
    return d;
  }
  // sg, su: the scales (0 for a masked chunk); cg, cu: b - 128 s
  template <int CS = 64>
  static __device__ __forceinline__ void dot(const D& g, const D& u, const uint8_t* xrow, int c, float sg,
                                             float cg, float su, float cu, float& ag, float& au) {
    const uint8_t* xp = xrow + (size_t)c * CS;
    float a = 0.f, b = 0.f, x = 0.f;
    constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 xv = ldg16(xp + 16 * q);
      a = dot2_bf16(g.v[4 * q + 0], xv.x, a);
      b = dot2_bf16(u.v[4 * q + 0], xv.x, b);
      x = dot2_bf16(kOnes, xv.x, x);
      a = dot2_bf16(g.v[4 * q + 1], xv.y, a);
      b = dot2_bf16(u.v[4 * q + 1], xv.y, b);
      x = dot2_bf16(kOnes, xv.y, x);
      a = dot2_bf16(g.v[4 * q + 2], xv.z, a);
      b = dot2_bf16(u.v[4 * q + 2], xv.z, b);
      x = dot2_bf16(kOnes, xv.z, x);
      a = dot2_bf16(g.v[4 * q + 3], xv.w, a);
      b = dot2_bf16(u.v[4 * q + 3], xv.w, b);
      x = dot2_bf16(kOnes, xv.w, x);
    }
    ag = fmaf(sg, a, fmaf(cg, x, ag));
    au = fmaf(su, b, fmaf(cu, x, au));
  }
};

// Copying x rows into LDS: the block's threads take 16-byte units of the rows of the tokens in
// `mask` (compacted: unit i lies in the (i / rw)-th token of the mask), kXB units per thread
// per pass, all loads of a pass issued before any store (a load-store loop would wait a full
// round trip per unit).
constexpr int kXB = 4;
__device__ __forceinline__ int nth_token(unsigned mask, int q) {
  int t = 0;
  for (;; ++t) {  // mask has more than q bits set
    if ((mask >> t) & 1u) {
      if (q == 0) return t;
      --q;
    }
  }
}
__device__ __forceinline__ void x_rows_load(uint4 (&xr)[kXB], int base, int n, int rw, unsigned mask,
                                            const uint8_t* xg, size_t xstride) {
#pragma unroll
  for (int j = 0; j < kXB; ++j) {
    const int i = base + j * (int)blockDim.x;
    if (i < n) {
      const int q = i / rw, t = nth_token(mask, q);
      xr[j] = ldg16(xg + (size_t)t * xstride + (size_t)(i - q * rw) * 16);
    }
  }
}
// XP (x of 4-bit experts): every 64-byte chunk (32 bf16) is followed by 16 bytes of padding in
// LDS, so that the G lanes of a group, which read chunks c, c + 1, ..., start 20 banks apart
// instead of 16 (64-byte strides put every fourth lane on the same banks).
template <bool XP>
__device__ __forceinline__ void x_rows_store(const uint4 (&xr)[kXB], int base, int n, int rw,
                                             unsigned mask, uint4* xs) {
  const int rwl = XP ? rw / 4 * 5 : rw;
#pragma unroll
  for (int j = 0; j < kXB; ++j) {
    const int i = base + j * (int)blockDim.x;
    if (i < n) {
      const int q = i / rw, t = nth_token(mask, q), u = i - q * rw;
      xs[t * rwl + (XP ? (u >> 2) * 5 + (u & 3) : u)] = xr[j];
    }
  }
}

// One lane group (G lanes) computes gate and up row `row` (reduction over K = H) for every
// token in `mask` and writes out[slot][row] = silu(g) * u.  All loads of a K-slice are issued
// before any is consumed; lanes past the row end load a valid chunk and scale it by 0.
// XL: the block copies the rows of x of the tokens in `mask` from xg into LDS at xs (row t at
// t * xstride) and reads x from there; the first pass of x loads is issued before the weight
// loads, so that waiting for x does not wait for the weights.  Every thread of the block must
// call this function with the same mask.
template <int XT, int WT, int G, int NCH, int TM, bool XL>
__device__ __forceinline__ void gateup_row(const uint8_t* grow, const uint8_t* urow,
                                           const void* gsrow, const void* usrow, const void* gbrow,
                                           const void* ubrow, int nchunks, const uint8_t* xg, uint4* xs, int xbytes,
                                           size_t xstride, unsigned mask, const int* slots,
                                           float* out, int out_ld, int row, int gl, bool valid) {
  typedef GUC<WT, XT> C;
  constexpr bool XP = XL && (WT == MOE_MXFP4 || WT == MOE_INT4G64);  // padded x rows in LDS
  float ag[TM], au[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) ag[t] = au[t] = 0.f;
  uint4 xr[kXB];
  const int rw = (int)(xstride / 16), xn = XL ? __popc(mask) * rw : 0;
  if constexpr (XL) x_rows_load(xr, threadIdx.x, xn, rw, mask, xg, xstride);
  for (int c0 = 0; c0 < nchunks; c0 += G * NCH) {
    uint4 wg[NCH], wu[NCH];
    uint32_t bg[NCH], bu[NCH];  // raw scales (e8m0 byte; int4: bf16 bias << 16 | bf16 scale), converted
                                // when the chunk is used
    float okf[NCH];
    int cc[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = c0 + gl + G * m;
      const bool ok = valid && c < nchunks;
      cc[m] = ok ? c : 0;
      okf[m] = ok ? 1.f : 0.f;
      wg[m] = ldg16(grow + (size_t)cc[m] * 16);
      wu[m] = ldg16(urow + (size_t)cc[m] * 16);
      if constexpr (WT == MOE_MXFP4) {
        bg[m] = ((const uint8_t*)gsrow)[cc[m]];
        bu[m] = ((const uint8_t*)usrow)[cc[m]];
      } else if constexpr (WT == MOE_INT4G64) {  // the chunk's group: two chunks per 64 codes
        bg[m] = ((const uint16_t*)gsrow)[cc[m] >> 1] | (uint32_t)((const uint16_t*)gbrow)[cc[m] >> 1] << 16;
        bu[m] = ((const uint16_t*)usrow)[cc[m] >> 1] | (uint32_t)((const uint16_t*)ubrow)[cc[m] >> 1] << 16;
      }
    }
    // keep every weight load of the slice ahead of the arithmetic: left to itself the
    // scheduler reuses registers and waits for each chunk before loading the next
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XL) {
      if (c0 == 0) {  // the rows of the tokens in `mask` only
        x_rows_store<XP>(xr, threadIdx.x, xn, rw, mask, xs);
        for (int base = threadIdx.x + kXB * blockDim.x; base < xn; base += kXB * blockDim.x) {
          x_rows_load(xr, base, xn, rw, mask, xg, xstride);
          x_rows_store<XP>(xr, base, xn, rw, mask, xs);
        }
        __syncthreads();
      }
    }
    const uint8_t* xb = XL ? (const uint8_t*)xs : xg;
    const size_t xrs = XP ? (size_t)(rw / 4 * 5) * 16 : xstride;  // bytes per x row where it is read
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const typename C::D dg = C::deq(wg[m]), du = C::deq(wu[m]);
      float sg = okf[m], su = okf[m];
      if constexpr (WT == MOE_MXFP4) {  // select, not multiply: a NaN scale must not leak
        sg = okf[m] != 0.f ? e8m0_to_f32(bg[m]) : 0.f;
        su = okf[m] != 0.f ? e8m0_to_f32(bu[m]) : 0.f;
      }
      float cg = 0.f, cu = 0.f;
      if constexpr (WT == MOE_INT4G64) {
        const float s_g = bf16lo(bg[m]), s_u = bf16lo(bu[m]);
        sg = okf[m] != 0.f ? s_g : 0.f;
        su = okf[m] != 0.f ? s_u : 0.f;
        cg = okf[m] != 0.f ? fmaf(-128.f, s_g, bf16hi(bg[m])) : 0.f;
        cu = okf[m] != 0.f ? fmaf(-128.f, s_u, bf16hi(bu[m])) : 0.f;
      }
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        if (!((mask >> t) & 1u)) continue;  // uniform
        if constexpr (WT == MOE_INT4G64)
          C::template dot<XP ? 80 : 64>(dg, du, xb + (size_t)t * xrs, cc[m], sg, cg, su, cu, ag[t], au[t]);
        else if constexpr (WT == MOE_MXFP4)
          C::template dot<XP ? 80 : 64>(dg, du, xb + (size_t)t * xrs, cc[m], sg, su, ag[t], au[t]);
        else
          C::dot(dg, du, xb + (size_t)t * xrs, cc[m], sg, su, ag[t], au[t]);
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
// Down chunk arithmetic.  A chunk is 16 bytes of one Wd row: 4 fp32, 8 bf16 or 32 e2m1
// elements; the activation chunk is the same elements of a (fp32).
// ------------------------------------------------------------------------------------------
template <int WT> struct DN;
template <> struct DN<MOE_F32> {
  static constexpr int EPC = 4;
  typedef uint4 W;
  static __device__ __forceinline__ W load(const uint8_t* row, int c) { return ldg16(row + (size_t)c * 16); }
  static __device__ __forceinline__ float dot_regs(W w, const float4* x) {
    float acc = __uint_as_float(w.x) * x[0].x;
    acc = fmaf(__uint_as_float(w.y), x[0].y, acc);
    acc = fmaf(__uint_as_float(w.z), x[0].z, acc);
    return fmaf(__uint_as_float(w.w), x[0].w, acc);
  }
  static __device__ __forceinline__ float dot(W w, const float* a, int c) {
    const float4 x[1] = {ldf4(a + (size_t)c * 4)};
    return dot_regs(w, x);
  }
};
template <> struct DN<MOE_BF16> {
  static constexpr int EPC = 8;
  typedef uint4 W;
  static __device__ __forceinline__ W load(const uint8_t* row, int c) { return ldg16(row + (size_t)c * 16); }
  static __device__ __forceinline__ float dot_regs(W w, const float4* x) {
    float acc = bf16lo(w.x) * x[0].x;
    acc = fmaf(bf16hi(w.x), x[0].y, acc);
    acc = fmaf(bf16lo(w.y), x[0].z, acc);
    acc = fmaf(bf16hi(w.y), x[0].w, acc);
    acc = fmaf(bf16lo(w.z), x[1].x, acc);
    acc = fmaf(bf16hi(w.z), x[1].y, acc);
    acc = fmaf(bf16lo(w.w), x[1].z, acc);
    return fmaf(bf16hi(w.w), x[1].w, acc);
  }
  static __device__ __forceinline__ float dot(W w, const float* a, int c) {
    const float4 x[2] = {ldf4(a + (size_t)c * 8), ldf4(a + (size_t)c * 8 + 4)};
    return dot_regs(w, x);
  }
};
template <> struct DN<MOE_MXFP4> {
  static constexpr int EPC = 32;  // one MX block: 16 bytes of codes, one scale byte
  typedef uint4 W;
  static __device__ __forceinline__ W load(const uint8_t* row, int c) { return ldg16(row + (size_t)c * 16); }
  static __device__ __forceinline__ float dword_dot(uint32_t q, float4 x0, float4 x1, float acc) {
    const f32x2_t p0 = fp4x2_to_f32x2<0>(q), p1 = fp4x2_to_f32x2<1>(q);
    const f32x2_t p2 = fp4x2_to_f32x2<2>(q), p3 = fp4x2_to_f32x2<3>(q);
    acc = fmaf(p0.x, x0.x, acc);
    acc = fmaf(p0.y, x0.y, acc);
    acc = fmaf(p1.x, x0.z, acc);
    acc = fmaf(p1.y, x0.w, acc);
    acc = fmaf(p2.x, x1.x, acc);
    acc = fmaf(p2.y, x1.y, acc);
    acc = fmaf(p3.x, x1.z, acc);
    return fmaf(p3.y, x1.w, acc);
  }
  static __device__ __forceinline__ float dot_regs(W w, const float4* x) {
    float acc = dword_dot(w.x, x[0], x[1], 0.f);
    acc = dword_dot(w.y, x[2], x[3], acc);
    acc = dword_dot(w.z, x[4], x[5], acc);
    return dword_dot(w.w, x[6], x[7], acc);
  }
  // CS: floats from one chunk's activations to the next (32, or 36 in the padded LDS layout)
  template <int CS = 32>
  static __device__ __forceinline__ float dot(W w, const float* a, int c) {
    const float* p = a + (size_t)c * CS;
    float acc = dword_dot(w.x, ldf4(p), ldf4(p + 4), 0.f);
    acc = dword_dot(w.y, ldf4(p + 8), ldf4(p + 12), acc);
    acc = dword_dot(w.z, ldf4(p + 16), ldf4(p + 20), acc);
    return dword_dot(w.w, ldf4(p + 24), ldf4(p + 28), acc);
  }
};

// Group-wise affine 4-bit: 32 codes (half a group of 64) per chunk, each weight s * q + b with
// the group's bf16 scale and bias, formed in fp32 (exact: a bf16 scale times a 4-bit integer has
// 12 significant bits) and multiplied by the fp32 activation.
template <> struct DN<MOE_INT4G64> {
  static constexpr int EPC = 32;
  typedef uint4 W;
  static __device__ __forceinline__ W load(const uint8_t* row, int c) { return ldg16(row + (size_t)c * 16); }
  // elements 8j .. 8j + 7: codes of even elements in the bytes of q & 0x0F0F0F0F, odd ones in
  // the bytes of (q >> 4) & 0x0F0F0F0F
  static __device__ __forceinline__ float dword_dot(uint32_t q, float4 x0, float4 x1, float s, float b, float acc) {
    const uint32_t ev = q & 0x0F0F0F0Fu, od = (q >> 4) & 0x0F0F0F0Fu;
    const float xe[4] = {x0.x, x0.z, x1.x, x1.z}, xo[4] = {x0.y, x0.w, x1.y, x1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(fmaf(s, (float)((ev >> (8 * i)) & 0xFFu), b), xe[i], acc);
      acc = fmaf(fmaf(s, (float)((od >> (8 * i)) & 0xFFu), b), xo[i], acc);
    }
    return acc;
  }
  template <int CS = 32>
  static __device__ __forceinline__ float dot_affine(W w, const float* a, int c, float s, float b) {
    const float* p = a + (size_t)c * CS;
    float acc = dword_dot(w.x, ldf4(p), ldf4(p + 4), s, b, 0.f);
    acc = dword_dot(w.y, ldf4(p + 8), ldf4(p + 12), s, b, acc);
    acc = dword_dot(w.z, ldf4(p + 16), ldf4(p + 20), s, b, acc);
    return dword_dot(w.w, ldf4(p + 24), ldf4(p + 28), s, b, acc);
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

// Router logits: block e computes logits[t][e] = Wr[e] . x[t] (+ bias) for every token.  Its
// four waves take contiguous quarters of H (up to four 16-byte chunks per lane in flight per
// pass, fewer for more tokens) and meet in LDS, where wave 0 adds the four partial sums in a
// fixed order.  One block per expert spreads the fp32 router rows over the whole chip.  The
// x chunks of a pass are loaded into registers before any is used (loads consumed as they
// are issued would wait one L2 round trip each).
template <int XT, int TM>
__device__ __forceinline__ void router_block(const Args& A, int e) {
  constexpr int RC = TM <= 4 ? 4 : TM <= 8 ? 2 : 1;  // 16-byte weight chunks per lane per pass
  typedef typename std::conditional<XT == MOE_F32, float4, uint2>::type XV;
  __shared__ float s_p[kWaves][TM];
  const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (A.logits_in) {  // routing on given logits: copy them, no router
    for (int t = threadIdx.x; t < A.T; t += blockDim.x) {
      const float l = A.logits_in[(size_t)t * A.E + e];
      A.logits[(size_t)t * A.E + e] = l;
      if (A.o_logits) A.o_logits[(size_t)t * A.E + e] = l;
    }
    return;
  }
  const float* wr = A.rw + (size_t)e * A.H;
  const uint8_t* xb = (const uint8_t*)A.x;
  const size_t xstride = (size_t)A.H * XS<XT>::BYTES;
  const int nch = A.H / 4;  // float4 chunks of the row
  const int per = (nch + kWaves - 1) / kWaves;
  const int cb = wave * per, ce = min(nch, cb + per);
  float acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = 0.f;
  for (int c0 = cb; c0 < ce; c0 += kWave * RC) {
    float4 w[RC];
    XV xv[RC][TM];
    int cc[RC];
    float okf[RC];  // chunks past the quarter's end load chunk 0 and count 0 times
#pragma unroll
    for (int m = 0; m < RC; ++m) {
      const int c = c0 + lane + kWave * m;
      const bool ok = c < ce;
      cc[m] = ok ? c : 0;
      okf[m] = ok ? 1.f : 0.f;
      w[m] = ldf4(wr + (size_t)cc[m] * 4);
    }
#pragma unroll
    for (int m = 0; m < RC; ++m) {
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        // no branch around the x loads; rows past T read row 0 and are never stored
        const int tt = t < A.T ? t : 0;
        xv[m][t] = *(const XV*)(xb + tt * xstride + (size_t)cc[m] * sizeof(XV));
      }
    }
#pragma unroll
    for (int m = 0; m < RC; ++m) {
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        float x0, x1, x2, x3;
        if constexpr (XT == MOE_F32) {
          x0 = xv[m][t].x; x1 = xv[m][t].y; x2 = xv[m][t].z; x3 = xv[m][t].w;
        } else {
          x0 = bf16lo(xv[m][t].x); x1 = bf16hi(xv[m][t].x); x2 = bf16lo(xv[m][t].y); x3 = bf16hi(xv[m][t].y);
        }
        float d = w[m].x * x0;
        d = fmaf(w[m].y, x1, d);
        d = fmaf(w[m].z, x2, d);
        d = fmaf(w[m].w, x3, d);
        acc[t] = fmaf(okf[m], d, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const float v = group_sum<kWave>(acc[t]);
    if (lane == 0) s_p[wave][t] = v;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < A.T) {
    float s = s_p[0][t];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += s_p[w][t];
    if (A.rbias) s += A.rbias[(size_t)t * A.bias_stride + e];
    A.logits[(size_t)t * A.E + e] = s;
    if (A.o_logits) A.o_logits[(size_t)t * A.E + e] = s;
  }
}

template <int XT, int TM>
__global__ __launch_bounds__(kThreads) void dec_router(Args A) {
  router_block<XT, TM>(A, blockIdx.x);
}

// The shared expert's gate/up + SwiGLU for every token: one wave per shared row (the 64 lanes
// split K = H, kShNch chunks each per pass), a_sh[t][row] = silu(g) * u.  It needs no routing,
// so it runs in the blocks of a kernel that would otherwise leave HBM idle while it selects
// ("Optimizing on-device inference for Apple Silicon", section "Overlap independent GPU
// work").  Every thread of the block must call it (XL stages x in LDS behind a barrier).
constexpr int kShNch = 5;
template <int XT, int SWT, int TM, bool XL>
__device__ __forceinline__ void shared_gateup_block(const Args& A, int blk, int lane, int wave,
                                                    uint4* s_x) {
  const int nw = blockDim.x / kWave;
  const int row = blk * nw + wave;
  const bool valid = row < A.Is;
  const size_t r = valid ? row : 0;
  const size_t rb = row_bytes<SWT>(A.H);
  int slots[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) slots[t] = t;
  const unsigned mask = (A.T >= 32) ? 0xffffffffu : ((1u << A.T) - 1u);
  const size_t xstride = (size_t)A.H * XS<XT>::BYTES;
  gateup_row<XT, SWT, kWave, kShNch, TM, XL>((const uint8_t*)A.sgate + r * rb,
                                             (const uint8_t*)A.sup + r * rb, nullptr, nullptr, nullptr,
                                             nullptr, A.H / GU<SWT>::EPC, (const uint8_t*)A.x, s_x,
                                             (int)(A.T * xstride), xstride, mask, slots, A.a_sh,
                                             A.Is, row, lane, valid);
}

// Selection and the decode plan (T > 1): the last block; wave t selects token t (select_set:
// the k largest logits, ties to the lower index, renormalised softmax weights), then the
// distinct experts are compacted in ascending id with one ballot per 64 experts.  The nsh
// blocks before it (none when the gate/up kernel takes the shared expert) compute the shared
// expert's gate/up (shared_gateup_block), which keeps HBM busy while the selection runs.
// Block size 64 * TM (TM >= T).
template <int XT, int SWT, int TM, bool XL>
__global__ __launch_bounds__(kWave * TM) void dec_select(Args A, int nsh) {
  extern __shared__ uint4 s_xs[];
  const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if ((int)blockIdx.x < nsh) {
    shared_gateup_block<XT, SWT, TM, XL>(A, blockIdx.x, lane, wave, s_xs);
    return;
  }
  __shared__ int s_ids[TM * MOE_MAX_K];
  __shared__ float s_w[TM * MOE_MAX_K];
  __shared__ unsigned s_flag[MOE_MAX_E];
  __shared__ int s_pos[MOE_MAX_E];
  __shared__ int s_dslot[TM * MOE_MAX_K * TM];
  __shared__ float s_dw[TM * MOE_MAX_K * TM];
  __shared__ unsigned s_hist[TM][512];
  __shared__ int s_nd;
  const int nth = blockDim.x;
  const int T = A.T, k = A.k, E = A.E, S = T * k, D = S < E ? S : E;
  const DecodePlan P(A.plan, D, T);
  for (int i = threadIdx.x; i < E; i += nth) s_flag[i] = 0u;
  for (int i = threadIdx.x; i < D * T; i += nth) {
    s_dslot[i] = 0;
    s_dw[i] = 0.f;
  }
  if (wave < T)
    select_set(A.logits + (size_t)wave * E, E, k, lane, s_hist[wave], s_ids + wave * k, s_w + wave * k);
  __syncthreads();
  for (int i = threadIdx.x; i < S; i += nth) atomicOr(&s_flag[s_ids[i]], 1u << (i / k));
  __syncthreads();
  if (wave == 0) {
    int cnt = 0;
    for (int b = 0; b < E; b += kWave) {
      const int e = b + lane;
      const unsigned f = e < E ? s_flag[e] : 0u;
      const uint64_t bal = __ballot(f != 0u);
      const int pos = cnt + __popcll(bal & ((1ull << lane) - 1ull));
      if (f) {
        s_pos[e] = pos;
        P.dexp()[pos] = e;
        P.dmask()[pos] = f;
      }
      cnt += __popcll(bal);
    }
    if (lane == 0) {
      s_nd = cnt;
      *P.nd() = cnt;
    }
  }
  __syncthreads();
  // the selection itself, for inspection through the workspace (ascending id per token)
  for (int i = threadIdx.x; i < S; i += nth) {
    A.ids[i] = s_ids[i];
    A.cw[i] = s_w[i];
  }
  // a token's k experts are distinct, so every (distinct expert, token) cell has one writer
  for (int i = threadIdx.x; i < S; i += nth) {
    const int c = s_pos[s_ids[i]] * T + i / k;
    s_dslot[c] = i;
    s_dw[c] = s_w[i];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < D * T; i += nth) {
    P.dslot()[i] = s_dslot[i];
    P.dw()[i] = s_dw[i];
  }
  for (int i = s_nd + threadIdx.x; i < D; i += nth) {
    P.dexp()[i] = 0;
    P.dmask()[i] = 0u;
  }
}

// Copies n 16-byte units from global memory to LDS with the whole block, B loads per thread
// in flight before the first store.
template <int B>
__device__ __forceinline__ void stage16(uint4* dst, const uint4* src, int n) {
  for (int base = threadIdx.x; base < n; base += B * blockDim.x) {
    uint4 r[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = base + j * (int)blockDim.x;
      if (i < n) r[j] = src[i];
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = base + j * (int)blockDim.x;
      if (i < n) dst[i] = r[j];
    }
  }
}

// Streams np steps of a wave with two register buffers used in turn: step p + 1 is loaded
// before step p is consumed, and no buffer is ever copied into the other (a register copy
// would wait for the copied loads).  At the end the last step is loaded once more (cache-
// resident) instead of branching around the load, which keeps the wait counts exact.
// stream_loaded: buffer a already holds step 0.
template <class Buf, class Load, class Consume>
__device__ __forceinline__ void stream_loaded(int np, Buf& a, Buf& b, Load load, Consume consume) {
  if (np <= 0) return;  // uniform
  for (int p = 0;; p += 2) {
    const bool more1 = p + 1 < np;
    load(more1 ? p + 1 : p, b);
    consume(p, a);
    if (!more1) break;
    const bool more2 = p + 2 < np;
    load(more2 ? p + 2 : p + 1, a);
    consume(p + 1, b);
    if (!more2) break;
  }
}

// Gate/up + SwiGLU: block (u, tile) streams RB rows per wave of distinct expert u's gate and
// up matrices once and dots them with every token routed to u.  XL: x is staged in LDS
// (dynamic shared memory of T * H * sizeof(x) bytes).  SEL1 (T = 1, no selection kernel):
// wave 0 of every block selects the token's experts from the logits itself -- the k experts
// are then the distinct experts, in ascending id -- and block 0 publishes the plan for the
// down kernel; the first sh_blocks blocks compute the shared expert's gate/up meanwhile.
template <int XT, int WT, int SWT, int G, int NCH, int TM, bool XL, bool SEL1>
__global__ __launch_bounds__(kThreads) void dec_gateup(Args A, int tiles, int sh_blocks) {
  extern __shared__ uint4 s_x[];
  const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if ((int)blockIdx.x < sh_blocks) {
    shared_gateup_block<XT, SWT, TM, XL>(A, blockIdx.x, lane, wave, s_x);
    return;
  }
  const int blk = blockIdx.x - sh_blocks;
  const int u = blk / tiles, tile = blk - u * tiles;
  const int T = A.T, S = T * A.k, D = S < A.E ? S : A.E;
  const DecodePlan P(A.plan, D, T);
  int e;
  unsigned mask;
  int slots[TM];
  if constexpr (SEL1) {
    __shared__ int s_ids[MOE_MAX_K];
    __shared__ float s_w[MOE_MAX_K];
    __shared__ unsigned s_hist[512];
    if (wave == 0) select_set(A.logits, A.E, A.k, lane, s_hist, s_ids, s_w);
    __syncthreads();
    if (blk == 0 && threadIdx.x < A.k) {
      const int i = threadIdx.x;
      if (i == 0) *P.nd() = A.k;
      A.ids[i] = s_ids[i];
      A.cw[i] = s_w[i];
      P.dexp()[i] = s_ids[i];
      P.dmask()[i] = 1u;
      P.dslot()[i] = i;
      P.dw()[i] = s_w[i];
    }
    e = s_ids[u];
    mask = 1u;
#pragma unroll
    for (int t = 0; t < TM; ++t) slots[t] = u;
  } else {
    if (u >= *P.nd()) return;
    e = P.dexp()[u];
    mask = P.dmask()[u];
#pragma unroll
    for (int t = 0; t < TM; ++t) slots[t] = t < T ? P.dslot()[u * T + t] : 0;
  }
  constexpr int RB = kWave / G;
  const int grp = lane / G, gl = lane % G;
  const int row = tile * (kWaves * RB) + wave * RB + grp;
  const bool valid = row < A.I;
  const size_t r = (size_t)e * A.I + (valid ? row : 0);
  const size_t rb = row_bytes<WT>(A.H);
  const void *gsr = nullptr, *usr = nullptr, *gbr = nullptr, *ubr = nullptr;
  if constexpr (WT == MOE_MXFP4) {
    gsr = (const uint8_t*)A.gs + r * (A.H / 32);
    usr = (const uint8_t*)A.us + r * (A.H / 32);
  } else if constexpr (WT == MOE_INT4G64) {
    gsr = (const uint16_t*)A.gs + r * (A.H / 64);
    usr = (const uint16_t*)A.us + r * (A.H / 64);
    gbr = (const uint16_t*)A.gb + r * (A.H / 64);
    ubr = (const uint16_t*)A.ub + r * (A.H / 64);
  }
  const size_t xstride = (size_t)A.H * XS<XT>::BYTES;
  gateup_row<XT, WT, G, NCH, TM, XL>((const uint8_t*)A.gate + r * rb, (const uint8_t*)A.up + r * rb,
                                     gsr, usr, gbr, ubr, A.H / GU<WT>::EPC, (const uint8_t*)A.x, s_x,
                                     (int)(T * xstride), xstride, mask, slots, A.a, A.I, row, gl,
                                     valid);
}

// Down + combine: y[t][h] = Wd_s[h] . a_s[t] + sum over t's experts of w * (Wd[e][h] . a).
// Output rows come in groups of RB (one lane group of G lanes per row); a block takes row
// groups blockIdx.x, blockIdx.x + gridDim.x, ... and its NW waves share the work items round
// robin: first (row group, K-slice) of the shared expert, then (row group, K-slice, distinct
// expert) of the routed ones.  The plan and -- when they fit (ALDS) -- every routed and shared
// activation row are staged in LDS once per block.  Each wave streams its items' 16-byte
// weight chunks with the next item's loads in flight while it consumes the current one.  Per
// (row group, wave) partial sums are added up in LDS and summed over the waves in a fixed
// order at the end, so the result is deterministic.
// PH (several tokens, when all routed rows do not fit): the distinct experts are taken in
// phases, each as many consecutive experts as their token rows fit act_rows staged rows; a
// phase stages its rows (expert u's tokens at rows s_base[u] + the token's rank in u's mask),
// runs its items, and the next one restages behind a barrier.  The shared items and rows stay
// for the whole kernel (phase 0 runs the shared items).
// Dynamic LDS (4-byte words): plan (2D + 2DT; PH: + D expert bases + act_rows row slots),
// partials [nrgb_max][NW][TM][RB], then ALDS activations [T*k][I] (PH: [act_rows][I]) at
// act_off and [T][Is] at ash_off.
template <int WT, int SWT, int G, int NCH, int TM, bool ALDS, bool PH = false>
__global__ __launch_bounds__(1024) void dec_down(Args A, int nrg, int nrgb_max, int act_off, int ash_off,
                                                 int act_rows) {
  extern __shared__ float s_f[];
  static_assert(sizeof(typename DN<WT>::W) == 16 && sizeof(typename DN<SWT>::W) == 16, "16-byte chunks");
  constexpr int RB = kWave / G;
  const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int NW = blockDim.x / kWave;
  const int grp = lane / G, gl = lane % G;
  const int T = A.T, S = T * A.k, D = S < A.E ? S : A.E;
  const DecodePlan P(A.plan, D, T);
  int* s_e = (int*)s_f;
  unsigned* s_m = (unsigned*)(s_f + D);
  int* s_sl = (int*)(s_f + 2 * D);
  float* s_w = s_f + 2 * D + D * T;
  int* s_base = (int*)(s_f + 2 * D + 2 * D * T);  // PH
  int* s_rowslot = s_base + D;                     // PH
  float* s_part = s_f + 2 * D + 2 * D * T + (PH ? D + act_rows : 0);
  float* s_act = s_f + act_off;
  float* s_ash = s_f + ash_off;

  const int nch = A.I / DN<WT>::EPC;
  // 4-bit experts with activations in LDS: 4 floats of padding after every 32-float chunk, so
  // that the G lanes of a group (chunks c, c + 1, ...) start 36 banks apart rather than 32
  constexpr bool AP = ALDS && DN<WT>::EPC == 32;
  constexpr int kCS = AP ? 36 : DN<WT>::EPC;  // floats per chunk where the routed rows are read
  const int ldr = ALDS ? nch * kCS : A.I;     // floats per routed activation row there
  const int nsl = (nch + G * NCH - 1) / (G * NCH);
  const int nchs = A.Is / DN<SWT>::EPC;
  const int nsls = (nchs + G * NCH - 1) / (G * NCH);
  const int nrgb = (nrg - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;
  const int nqs = nrgb * nsls;  // shared items
  const size_t rb = row_bytes<WT>(A.I), rbs = row_bytes<SWT>(A.Is);
  const float* abase = ALDS ? s_act : A.a;
  const float* asbase = ALDS ? s_ash : A.a_sh;

  float acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = 0.f;
  int cur_j = -1;
  int nd = 0, per_rg = 0;  // routed items per row group, known once the plan is read
  int u0 = 0, nup = 0, qs = nqs;  // the phase's first expert, its expert count, its shared items
  struct Buf {
    uint4 w[NCH];
    uint32_t sb[NCH];
  };
  auto row_of = [&](int j) { return ((int)blockIdx.x + j * (int)gridDim.x) * RB + grp; };
  auto load = [&](int q, Buf& bf) {
    if (q < qs) {  // uniform: shared item (row group j, slice sl)
      const int j = q / nsls, sl = q - j * nsls;
      const int h = row_of(j), hh = h < A.H ? h : 0;
      const uint8_t* row = (const uint8_t*)A.sdown + (size_t)hh * rbs;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        const int c = sl * G * NCH + gl + G * m;
        bf.w[m] = DN<SWT>::load(row, c < nchs ? c : 0);
        if constexpr (WT == MOE_MXFP4) bf.sb[m] = 127u;     // unit scale (never used for shared rows)
        if constexpr (WT == MOE_INT4G64) bf.sb[m] = 0x3F80u;  // scale 1, bias 0 (never used either)
      }
      return;
    }
    const int r = q - qs;
    const int j = r / per_rg, r2 = r - j * per_rg;
    const int sl = r2 / nup, u = u0 + r2 - sl * nup;
    const int h = row_of(j), hh = h < A.H ? h : 0;
    const int e = s_e[u];
    const uint8_t* row = (const uint8_t*)A.down + ((size_t)e * A.H + hh) * rb;
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = sl * G * NCH + gl + G * m;
      const int cc = c < nch ? c : 0;
      bf.w[m] = DN<WT>::load(row, cc);
      if constexpr (WT == MOE_MXFP4) bf.sb[m] = ((const uint8_t*)A.ds)[((size_t)e * A.H + hh) * (A.I / 32) + cc];
      if constexpr (WT == MOE_INT4G64) {  // bf16 bias << 16 | bf16 scale of the chunk's group
        const size_t gi = ((size_t)e * A.H + hh) * (A.I / 64) + (cc >> 1);
        bf.sb[m] = ((const uint16_t*)A.ds)[gi] | (uint32_t)((const uint16_t*)A.db)[gi] << 16;
      }
    }
  };
  auto flush = [&]() {
    if (cur_j < 0) return;  // uniform
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const float v = group_sum<G>(acc[t]);
      // a wave meets a row group at most twice (shared, then routed items): accumulate
      if (gl == 0) s_part[((cur_j * NW + wave) * TM + t) * RB + grp] += v;
      acc[t] = 0.f;
    }
  };
  // one body for both kinds of item (two copies of the token loop would double the live
  // registers): a shared item is every token with weight 1 over a_sh's rows
  const unsigned all_t = (T >= 32) ? 0xffffffffu : ((1u << T) - 1u);
  auto consume = [&](int q, const Buf& bf) {
    const bool sh = q < qs;  // uniform
    int j, sl, u = 0;
    if (sh) {
      j = q / nsls;
      sl = q - j * nsls;
    } else {
      const int r = q - qs;
      j = r / per_rg;
      const int r2 = r - j * per_rg;
      sl = r2 / nup;
      u = u0 + r2 - sl * nup;
    }
    if (j != cur_j) {  // uniform
      flush();
      cur_j = j;
    }
    const int lim = sh ? nchs : nch;
    int cc[NCH];
    float sc[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = sl * G * NCH + gl + G * m;
      cc[m] = c < lim ? c : 0;
      if constexpr (WT == MOE_MXFP4) {  // select, not multiply: a NaN scale must not leak
        const float s = e8m0_to_f32(bf.sb[m]);
        sc[m] = c < lim ? (sh ? 1.f : s) : 0.f;
      }
      else
        sc[m] = c < lim ? 1.f : 0.f;
    }
    const unsigned mask = sh ? all_t : s_m[u];
    const float* ab = sh ? asbase : abase;
    const int ld = sh ? A.Is : ldr;
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (!((mask >> t) & 1u)) continue;  // uniform
      const int ar = sh ? t : PH ? s_base[u] + __popc(mask & ((1u << t) - 1u)) : s_sl[u * T + t];
      const float* arow = ab + (size_t)ar * ld;
      const float wt = sh ? 1.f : s_w[u * T + t];
      float part = 0.f;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        float d;
        if constexpr (WT == SWT)
          d = DN<WT>::dot(bf.w[m], arow, cc[m]);
        else if constexpr (WT == MOE_INT4G64)
          d = sh ? DN<SWT>::dot(bf.w[m], arow, cc[m])
                 : DN<WT>::template dot_affine<kCS>(bf.w[m], arow, cc[m], bf16lo(bf.sb[m]), bf16hi(bf.sb[m]));
        else if constexpr (WT == MOE_MXFP4)
          d = sh ? DN<SWT>::dot(bf.w[m], arow, cc[m]) : DN<WT>::template dot<kCS>(bf.w[m], arow, cc[m]);
        else
          d = sh ? DN<SWT>::dot(bf.w[m], arow, cc[m]) : DN<WT>::dot(bf.w[m], arow, cc[m]);
        part = fmaf(sc[m], d, part);
      }
      acc[t] = fmaf(wt, part, acc[t]);
    }
  };

  // Prologue.  The plan words and the first pass of activations are loaded into registers
  // first; then, when this wave's first item belongs to the shared expert (its weights need no
  // plan), that item's weight loads are issued; only then is the staged data stored to LDS.
  // Loads complete in issue order, so the stores wait for the staging loads alone and the
  // shared weights are in flight across the staging barrier.
  const int tid = threadIdx.x, bd = blockDim.x;
  constexpr int kPl = 4;  // plan cells per thread: D * T <= 16 * 16 * 16 = 4096 with 1024 threads
  constexpr int kStg = 4;  // activation float4 per thread in the first staging pass
  int r_e = 0, r_sl[kPl];
  unsigned r_m = 0;
  float r_w[kPl];
  if (tid < D) {
    r_e = P.dexp()[tid];
    r_m = P.dmask()[tid];
  }
#pragma unroll
  for (int j = 0; j < kPl; ++j) {
    const int i = tid + j * bd;
    r_sl[j] = i < D * T ? P.dslot()[i] : 0;
    r_w[j] = i < D * T ? P.dw()[i] : 0.f;
  }
  const int n4 = ALDS && !PH ? S * A.I / 4 : 0, n4s = ALDS ? T * A.Is / 4 : 0;
  float4 sv[kStg];
#pragma unroll
  for (int j = 0; j < kStg; ++j) {
    const int i = tid + j * bd;
    if (i < n4 + n4s) sv[j] = i < n4 ? ldf4(A.a + (size_t)i * 4) : ldf4(A.a_sh + (size_t)(i - n4) * 4);
  }
  Buf a, b;
  const bool early = wave < nqs;  // uniform: the first item is a shared one
  if (early) load(wave, a);
  if (tid < D) {
    s_e[tid] = r_e;
    s_m[tid] = r_m;
  }
#pragma unroll
  for (int j = 0; j < kPl; ++j) {
    const int i = tid + j * bd;
    if (i < D * T) {
      s_sl[i] = r_sl[j];
      s_w[i] = r_w[j];
    }
  }
  for (int i = tid; i < nrgb_max * NW * TM * RB; i += bd) s_part[i] = 0.f;
  // staging unit i: routed activations [S][I] for i < n4 (AP: into the padded rows), then the
  // shared ones [T][I_s]
  const int q4 = A.I / 4;  // float4 units per routed row
  auto stage_dst = [&](int i) {
    if (i >= n4) return (float4*)s_ash + (i - n4);
    if constexpr (!AP) return (float4*)s_act + i;
    const int r = i / q4, q = i - r * q4;
    return (float4*)(s_act + (size_t)r * ldr + (q >> 3) * kCS) + (q & 7);
  };
#pragma unroll
  for (int j = 0; j < kStg; ++j) {
    const int i = tid + j * bd;
    if (i < n4 + n4s) *stage_dst(i) = sv[j];
  }
  for (int i = tid + kStg * bd; i < n4 + n4s; i += bd)  // larger windows: the rest, pass by pass
    *stage_dst(i) = i < n4 ? ldf4(A.a + (size_t)i * 4) : ldf4(A.a_sh + (size_t)(i - n4) * 4);
  nd = *P.nd();
  nup = nd;
  __syncthreads();
  for (int ph = 0;; ++ph) {
    if constexpr (PH) {
      // the phase's experts: from u0 on while their token rows fit the staged rows (the
      // launcher makes act_rows >= T, so every phase takes at least one expert)
      int rows = 0, u1 = u0;
      while (u1 < nd && rows + __popc(s_m[u1]) <= act_rows) rows += __popc(s_m[u1++]);
      if (u1 == u0) {  // not reached (act_rows >= T): one expert, its first act_rows rows
        u1 = u0 + 1;
        rows = act_rows;
      }
      nup = u1 - u0;
      qs = ph == 0 ? nqs : 0;
      if (ph > 0) __syncthreads();  // every wave is done with the previous phase's rows
      if (threadIdx.x == 0) {
        int r = 0;
        for (int u = u0; u < u1; ++u) {
          s_base[u] = r;
          r += __popc(s_m[u]);
        }
      }
      __syncthreads();
      for (int i = tid; i < nup * T; i += bd) {
        const int u = u0 + i / T, t = i - (i / T) * T;
        const unsigned m = s_m[u];
        const int r = s_base[u] + __popc(m & ((1u << t) - 1u));
        if (((m >> t) & 1u) && r < act_rows) s_rowslot[r] = s_sl[u * T + t];
      }
      __syncthreads();
      for (int i = tid; i < rows * q4; i += bd) {
        const int r = i / q4, q = i - r * q4;
        const float4 v = ldf4(A.a + (size_t)s_rowslot[r] * A.I + (size_t)q * 4);
        if constexpr (AP)
          *((float4*)(s_act + (size_t)r * ldr + (q >> 3) * kCS) + (q & 7)) = v;
        else
          *((float4*)s_act + (size_t)r * q4 + q) = v;
      }
      __syncthreads();
    }
    per_rg = nsl * nup;
    const int nq = qs + nrgb * per_rg;
    const int nmine = wave < nq ? (nq - 1 - wave) / NW + 1 : 0;
    if (nmine > 0) {  // uniform; this wave's items are q = wave + NW * step
      if (!early || ph > 0) load(wave, a);
      stream_loaded<Buf>(nmine, a, b, [&](int st, Buf& bf) { load(wave + NW * st, bf); },
                         [&](int st, const Buf& bf) { consume(wave + NW * st, bf); });
    }
    if constexpr (!PH) break;
    u0 += nup;
    if (u0 >= nd) break;
  }
  flush();
  __syncthreads();
  for (int i = threadIdx.x; i < nrgb * TM * RB; i += blockDim.x) {
    const int j = i / (TM * RB), r = i - j * (TM * RB);
    const int t = r / RB, g = r - t * RB;
    const int h = ((int)blockIdx.x + j * (int)gridDim.x) * RB + g;
    if (t < T && h < A.H) {
      float v = 0.f;
      for (int w = 0; w < NW; ++w) v += s_part[((j * NW + w) * TM + t) * RB + g];
      if (A.odt == MOE_BF16)
        ((uint16_t*)A.y)[(size_t)t * A.H + h] = f32_to_bf16(v);
      else
        ((float*)A.y)[(size_t)t * A.H + h] = v;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Launch: (G, NCH) chosen per kernel from a preference list, TM from T.
// ------------------------------------------------------------------------------------------
struct GN { int G, NCH; };
// gate/up (reduction over H): two rows per wave with 8 chunks per lane for one token;
// wider groups when several tokens share the x registers
// (no two entries of a list have the same capacity G * NCH: the picker takes the first of
// equal capacities, so a later one would never run)
constexpr GN kGU1[] = {{32, 8}, {64, 5}, {16, 5}, {16, 4}, {32, 1}, {16, 1}, {64, 2}, {64, 8}};
constexpr GN kGUn[] = {{64, 4}, {64, 5}, {16, 5}, {16, 4}, {64, 2}, {32, 1}, {16, 1}, {64, 8}};
// down (reduction over I): activations come from LDS, so several chunks per lane are cheap;
// the launcher prefers the entry that spreads the output rows most evenly over the CUs
constexpr GN kDN[] = {{8, 3}, {8, 2}, {16, 4}, {32, 3}, {16, 3}, {8, 4}, {16, 2}, {32, 2},
                      {16, 1}, {32, 1}, {8, 1}, {64, 4}};
constexpr int kNGU = sizeof(kGU1) / sizeof(kGU1[0]);
static_assert(kNGU == 8 && sizeof(kGUn) / sizeof(kGUn[0]) == 8, "gateup_fn instantiates 8 entries");
constexpr int kNDN = sizeof(kDN) / sizeof(kDN[0]);

struct DevInfo { int ncu, max_lds; };
DevInfo dev_info() {
  static DevInfo cache[64];
  static bool have[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!have[dev]) {
    int ncu = 0, lds = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) ncu = 256;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || lds <= 0) lds = 65536;
    cache[dev] = DevInfo{ncu, lds};
    have[dev] = true;
  }
  return cache[dev];
}

// First entry with the fewest idle chunk slots; the last entry walks long rows in slices
// when nothing covers the row.
// first_fit: the first entry that leaves at most a quarter of its chunk slots idle.
template <int N>
int pick_gn(const GN (&list)[N], int nchunks, bool first_fit = false) {
  if (first_fit)
    for (int i = 0; i < N; ++i) {
      const int cap = list[i].G * list[i].NCH;
      if (cap >= nchunks && 4 * (cap - nchunks) <= cap) return i;
    }
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

// Down config: among entries leaving at most a quarter of their chunk slots idle, the one
// whose busiest block has the fewest rounds of work items over its 16 waves (a wave keeps
// two items in flight, so rounds, not rows, set the latency chain), counting D distinct
// experts' and the shared expert's items; ties go to fewer idle chunk slots (idle lanes
// still execute the dot products, which bound the 4-bit kernels), then to more chunks per
// lane (more bytes in flight), then list order.  Else the fewest idle slots.
int pick_down(int nch, int nchs, int H, int D, int ncu) {
  int best = -1, score = 1 << 30, bidle = 0, bnch = 0;
  for (int i = 0; i < kNDN; ++i) {
    const int cap = kDN[i].G * kDN[i].NCH;
    if (cap < nch || 4 * (cap - nch) > cap) continue;
    const int rb = kWave / kDN[i].G, nrg = (H + rb - 1) / rb, nrgb = (nrg + ncu - 1) / ncu;
    const int items = nrgb * (((nch + cap - 1) / cap) * D + (nchs + cap - 1) / cap);
    const int sc = (items + 15) / 16, idle = cap - nch;
    if (best < 0 || sc < score || (sc == score && (idle < bidle || (idle == bidle && kDN[i].NCH > bnch)))) {
      best = i;
      score = sc;
      bidle = idle;
      bnch = kDN[i].NCH;
    }
  }
  return best >= 0 ? best : pick_gn(kDN, nch);
}

// The router's token tile is T itself up to 8 (its x loads are not masked per token), else 16.
template <int XT>
void* router_fn(int T) {
  switch (T) {
    case 1: return (void*)dec_router<XT, 1>;
    case 2: return (void*)dec_router<XT, 2>;
    case 3: return (void*)dec_router<XT, 3>;
    case 4: return (void*)dec_router<XT, 4>;
    case 5: return (void*)dec_router<XT, 5>;
    case 6: return (void*)dec_router<XT, 6>;
    case 7: return (void*)dec_router<XT, 7>;
    case 8: return (void*)dec_router<XT, 8>;
    default: return (void*)dec_router<XT, 16>;
  }
}

template <int XT, int WT, int SWT, int TM, const GN* L, bool XL, bool SEL1>
void* gateup_fn(int gi) {
  switch (gi) {
#define C(i) case i: return (void*)dec_gateup<XT, WT, SWT, L[i].G, L[i].NCH, TM, XL, SEL1>;
    C(0) C(1) C(2) C(3) C(4) C(5) C(6) C(7)
#undef C
  }
  return nullptr;
}
template <int WT, int SWT, int TM, bool ALDS, bool PH = false>
void* down_fn(int gi) {
  switch (gi) {
#define C(i) case i: return (void*)dec_down<WT, SWT, kDN[i].G, kDN[i].NCH, TM, ALDS, PH>;
    C(0) C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8) C(9) C(10) C(11)
#undef C
  }
  return nullptr;
}

int gu_epc(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 8 : 32; }  // MXFP4, INT4G64: 32
int dn_epc(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 8 : 32; }
constexpr int kMaxLdsX = 64 * 1024;       // one token's x always fits in LDS
constexpr int kMaxLdsXMulti = 40 * 1024;  // several tokens' x staged in LDS up to this size

template <int XT, int WT, int SWT, int TM>
int launch_decode_t(Args A, hipStream_t st, bool route_only, const LaunchHook& hook) {
  constexpr const GN* GUL = TM == 1 ? kGU1 : kGUn;
  const DevInfo dv = dev_info();
  const int S = A.T * A.k, D = S < A.E ? S : A.E;
  // x goes through LDS (its loads issued ahead of the weights, read back at LDS latency); one
  // token's row always fits (H <= MOE_MAX_H fp32 values are 64 KiB).  Several tokens' rows
  // only up to 40 KiB: beyond that the LDS they take costs the gate/up kernel more occupancy
  // than the staging saves, and x is read through the L1 instead
  const size_t xbytes = (size_t)A.T * A.H * (XT == MOE_F32 ? 4 : 2);
  static_assert((size_t)MOE_MAX_H * 4 <= (size_t)kMaxLdsX, "a single token's x fits in LDS");
  const bool xl = TM == 1 || xbytes <= kMaxLdsXMulti;
  // 4-bit experts read x from padded LDS rows (16 bytes after every 64)
  constexpr bool w4 = WT == MOE_MXFP4 || WT == MOE_INT4G64;
  const size_t xbytes_gu = w4 ? xbytes / 4 * 5 : xbytes;
  // shared expert gate/up: one row per wave, in the selection kernel's blocks while a long
  // selection (T = 2..4 tokens over E >= 512 experts) leaves time to stream it there, else
  // beside the routed rows of the gate/up kernel (T = 1; T > 4, where the selection kernel's
  // blocks of 8 or 16 waves would be too few; a short selection over fewer experts)
  const bool sh_in_sel = TM > 1 && TM <= 4 && A.E >= 512;
  const int sh_waves = sh_in_sel ? TM : kWaves;
  int nsh = A.Is > 0 ? (A.Is + sh_waves - 1) / sh_waves : 0;
  void* args1[] = {&A};
  hipError_t err = launch(hook, "dec_router", router_fn<XT>(A.T), dim3(A.E), dim3(kThreads), args1, 0, st);
  if (err != hipSuccess) return MOE_EHIP;
  if (route_only) return MOE_OK;
  if (TM > 1) {
    void* fs = xl ? (void*)dec_select<XT, SWT, TM, true> : (void*)dec_select<XT, SWT, TM, false>;
    int nsel = sh_in_sel ? nsh : 0;
    void* args_s[] = {&A, &nsel};
    err = launch(hook, "dec_select", fs, dim3(nsel + 1), dim3(kWave * TM), args_s, xl ? xbytes : 0, st);
    if (err != hipSuccess) return MOE_EHIP;
  }

  // gate/up: (shared gate/up blocks first unless the selection kernel has them, then)
  // (distinct expert, row tile) blocks
  const int g2 = TM == 1 ? pick_gn(kGU1, A.H / gu_epc(WT)) : pick_gn(kGUn, A.H / gu_epc(WT));
  const int rb2 = kWaves * (kWave / GUL[g2].G);
  int tiles = (A.I + rb2 - 1) / rb2;
  int sh_blocks = sh_in_sel ? 0 : nsh;
  void* f2;
  if constexpr (TM == 1)
    f2 = gateup_fn<XT, WT, SWT, TM, GUL, true, true>(g2);
  else
    f2 = xl ? gateup_fn<XT, WT, SWT, TM, GUL, true, false>(g2) : gateup_fn<XT, WT, SWT, TM, GUL, false, false>(g2);
  void* args2[] = {&A, &tiles, &sh_blocks};
  err = launch(hook, "dec_gateup", f2, dim3(sh_blocks + D * tiles), dim3(kThreads), args2, xl ? xbytes_gu : 0, st);
  if (err != hipSuccess) return MOE_EHIP;

  // down: at most one block per CU, each over an even share of the row groups
  const int g3 = pick_down(A.I / dn_epc(WT), A.Is / dn_epc(SWT), A.H, D, dv.ncu);
  const int rb3 = kWave / kDN[g3].G;
  int nrg = (A.H + rb3 - 1) / rb3;
  int nrgb = (nrg + dv.ncu - 1) / dv.ncu;
  const int grid3 = (nrg + nrgb - 1) / nrgb;
  constexpr int nw = 16;
  const size_t plan_w = 2 * (size_t)D + 2 * (size_t)D * A.T;
  int act_off = (int)((plan_w + (size_t)nrgb * nw * TM * rb3 + 3) / 4 * 4);
  // routed activations in LDS; 4-bit experts pad each 32-float chunk to 36 floats
  const size_t act_floats = w4 ? (size_t)S * (A.I / 32) * 36 : (size_t)S * A.I;
  int ash_off = (int)(act_off + (act_floats + 3) / 4 * 4);
  const size_t lds_act = (size_t)ash_off * 4 + (size_t)A.T * A.Is * 4;
  const bool alds = lds_act <= (size_t)dv.max_lds;
  size_t lds3 = alds ? lds_act : (size_t)act_off * 4;
  void* f3 = alds ? down_fn<WT, SWT, TM, true>(g3) : down_fn<WT, SWT, TM, false>(g3);
  int act_rows = 0;
  if constexpr (TM >= 8 && w4) {
    // 4-bit experts, several tokens whose routed rows do not all fit: stage them in phases of
    // act_rows rows (at least T, one expert's worst case), the most that fit beside the shared
    // rows.  (Read from the L2 instead, each 16-byte weight chunk would pull 128 bytes of
    // activations per token; bf16 chunks pull 32, and they are faster without the phases.)
    if (!alds) {
      const size_t ldr = w4 ? (size_t)(A.I / 32) * 36 : (size_t)A.I;  // floats per staged row
      const size_t part = (size_t)nrgb * nw * TM * rb3;
      auto need = [&](int rows, int* ao, int* so) {
        const size_t ao_ = (plan_w + D + rows + part + 3) / 4 * 4;
        const size_t so_ = ao_ + ((size_t)rows * ldr + 3) / 4 * 4;
        *ao = (int)ao_;
        *so = (int)so_;
        return so_ * 4 + (size_t)A.T * A.Is * 4;
      };
      int ao, so;
      int rows = (int)std::min<size_t>((size_t)S, (size_t)dv.max_lds / 4 / (ldr + 1));
      while (rows >= A.T && need(rows, &ao, &so) > (size_t)dv.max_lds) --rows;
      if (rows >= A.T) {
        act_rows = rows;
        act_off = ao;
        ash_off = so;
        lds3 = need(rows, &ao, &so);
        f3 = down_fn<WT, SWT, TM, true, true>(g3);
      }
    }
  }
  void* args3[] = {&A, &nrg, &nrgb, &act_off, &ash_off, &act_rows};
  err = launch(hook, "dec_down", f3, dim3(grid3), dim3(kWave * nw), args3, lds3, st);
  if (err != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

}  // namespace
}  // namespace moe
