// Device helpers and the argument block shared by the libmoe kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kDecodeMaxT = 16;     // T at or below this takes the decode (GEMV) path

// ---------------------------------------------------------------------------------------
// Argument block for every kernel of one call.  Passed by value (kernarg segment).
// ---------------------------------------------------------------------------------------
struct Args {
  int T, H, E, k, I, Is;
  int act, wdt, sdt, odt;             // moe_dtype_t of x, experts, shared, y
  int aq;                             // act_quant: MOE_QNONE | MOE_QMXFP8
  const void* x;
  const float* rw;
  const float* rbias;
  long long bias_stride;
  const void *gate, *up, *down;
  const void *gs, *us, *ds;           // MXFP4: e8m0 bytes; INT4G64: bf16 group scales
  const void *sgate, *sup, *sdown;
  const void *gb, *ub, *db;           // INT4G64: bf16 group biases
  void* y;
  // route-only inputs/outputs (moe_route); null in moe_forward
  const float* logits_in;
  int* o_ids;
  float* o_w;
  float* o_logits;
  int* o_count;
  int* o_offset;
  int* o_sorted;
  // workspace sections
  float* logits;        // [T][E]
  int* ids;             // [T][k]
  float* cw;            // [T][k]
  int* plan;            // decode plan, see DecodePlan
  float* a_sh;          // [T][Is]   decode: shared-expert activations (fp32)
  float* a;             // [T*k][I]  decode: routed activations (fp32)
  // prefill sections
  int* pf_count;        // [E+1]   (index E = shared expert group)
  int* pf_offset;       // [E+2]
  int* pf_rows;         // [T*k + T]   grouped rows: slot ids (shared group: T*k + t)
  int* pf_tiles;        // tile map entries
  uint16_t* pf_act;     // [T*k + T][max(I,Is)] bf16 gate/up activations
  uint16_t* pf_out;     // [T*k + T][H]  bf16 per-row expert outputs (weighted)
  int tiles_cap;        // capacity of pf_tiles
};

// Decode plan, written by the selection kernel and read by both expert kernels: the
// distinct experts of the T*k assignments in ascending expert id (nd of them), the tokens
// routed to each (bitmask), and per (distinct expert, token) the slot s = t*k + j that holds
// that token's activations and its combine weight (slot 0 and weight 0 where the token does
// not use the expert).  Every distinct expert's weights are then streamed exactly once.
// Layout (4-byte words): nd, pad[63], dexp[D], dmask[D], dslot[D][T], dw[D][T], D = min(T*k, E).
struct DecodePlan {
  int* base;
  int D, T;
  __host__ __device__ DecodePlan(int* b, int D_, int T_) : base(b), D(D_), T(T_) {}
  __host__ __device__ int* nd() const { return base; }
  __host__ __device__ int* dexp() const { return base + 64; }
  __host__ __device__ unsigned* dmask() const { return (unsigned*)(base + 64 + D); }
  __host__ __device__ int* dslot() const { return base + 64 + 2 * D; }
  __host__ __device__ float* dw() const { return (float*)(base + 64 + 2 * D + D * T); }
  __host__ __device__ static size_t bytes(int D, int T) {
    return sizeof(int) * (64 + 2 * (size_t)D + 2 * (size_t)D * T);
  }
};

// ---------------------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; NaN stays NaN.
// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// e8m0 scale byte -> fp32 power of two (0xFF -> NaN, 0x00 -> 2^-127 subnormal).  Branch
// free, so that a scale still in flight does not hold up the loads issued after it.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  uint32_t b = s << 23;
  b = s == 0u ? 0x00400000u : b;
  b = s == 0xffu ? 0x7fc00000u : b;
  return __uint_as_float(b);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two e2m1 codes in byte `sel` of v -> two bf16 values (exact; unit scale).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t v) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, r);
}
// Two e2m1 codes in byte `sel` of v -> two fp32 values (exact; unit scale).
template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32x2(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, SEL);
}

// ---------------------------------------------------------------------------------------
// Wave / lane-group reductions.  Within a 16-lane row the butterfly runs on DPP lane
// permutes (xor 1, xor 2 by quad_perm, xor 4 by row_half_mirror, xor 8 by row_mirror),
// which cost no LDS traffic; the 16-lane row results are combined with readlane.  Every
// lane of a group gets the group's result.
// ---------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
constexpr int kDppXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ __forceinline__ float rl(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "G");
  if constexpr (G >= 2) v += dpp_f<kDppXor1>(v);
  if constexpr (G >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (G >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (G >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (G == 32) {
    const float a = rl(v, 0) + rl(v, 16), b = rl(v, 32) + rl(v, 48);
    v = ((int)__lane_id() < 32) ? a : b;
  } else if constexpr (G == 64) {
    v = (rl(v, 0) + rl(v, 16)) + (rl(v, 32) + rl(v, 48));
  }
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return fmaxf(fmaxf(rl(v, 0), rl(v, 16)), fmaxf(rl(v, 32), rl(v, 48)));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ uint4 ldg16(const void* p) { return *(const uint4*)p; }
__device__ __forceinline__ uint2 ldg8(const void* p) { return *(const uint2*)p; }
__device__ __forceinline__ uint32_t ldg4(const void* p) { return *(const uint32_t*)p; }
__device__ __forceinline__ float4 ldf4(const float* p) { return *(const float4*)p; }

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Nontemporal 16-byte load for weight streams that are read exactly once per call.
__device__ __forceinline__ uint4 ldnt16(const void* p) {
  u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace moe
