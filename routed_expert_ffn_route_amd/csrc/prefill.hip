// Prefill path (T > 16): the layer as grouped GEMMs on MFMA.
//
//  router   logits = x . Wr^T on bf16 MFMA: x is bf16 exactly and every fp32 router weight is
//           split into three bf16 parts (hi + mid + lo == w), so each product is exact and the
//           sum is accumulated in fp32 -- fp32-accurate logits at bf16 matrix-core rates.
//  select   one wave per token (descending rank, ties to the lower index).
//  permute  histogram of assignments per expert -> prefix scan -> scatter of slots into expert
//           groups -> block map of fixed-size row tiles ("Optimizing on-device inference for
//           Apple Silicon", section "Keep expert routing on the GPU"; the shared expert is one
//           more group holding every token).  No host synchronisation anywhere.
//  gate/up  per tile: gather the tile's token rows of x, stream the group's gate and up rows
//           through LDS, MFMA, SwiGLU in the epilogue, bf16 activations in grouped order
//           (same page, sections "Decode weights during matrix multiplication" and "Match tile
//           size to expert load").
//  down     per tile: activations x Wd^T, scaled by the slot's routing weight in the
//           epilogue, one bf16 row per slot.
//  combine  y[t] = sum_j out[t*k + j] + out_shared[t], a fixed order (deterministic).
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPfBM = 128;     // rows per tile (gate/up and down)
constexpr int kPfBNI = 64;     // intermediate columns per gate/up block (x2: gate and up)
constexpr int kPfBNH = 128;    // hidden columns per down block
constexpr int kPfBK = 64;      // reduction step staged through LDS
constexpr int kPfLDK = kPfBK + 8;  // padded LDS row (bf16 elements)

size_t prefill_ws_bytes(int T, int H, int E, int k, int I, int Is) {
  const size_t S = (size_t)T * k, R = S + T;
  const size_t Imax = I > Is ? I : Is;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  return up(sizeof(int) * (E + 2)) * 2 + up(sizeof(int) * R) +
         up(sizeof(int) * 2 * (size_t)prefill_tiles_cap(T, E, k)) + up(256) + up(2 * R * Imax) +
         up(2 * R * (size_t)H);
}

// Upper bound of sum over the E+1 groups of ceil(rows / kPfBM).
int prefill_tiles_cap(int T, int E, int k) {
  return (int)(((size_t)T * k + T + kPfBM - 1) / kPfBM + E + 1);
}

namespace {

struct PfLayout {
  int* count;   // [E+1]
  int* offset;  // [E+2]
  int* rows;    // [S+T]
  int* tiles;   // [2*cap]
  int* ntiles;  // [1]
  uint16_t* act;  // [S+T][Imax]
  uint16_t* out;  // [S+T][H]
};

PfLayout pf_layout(const Args& A) {
  const size_t S = (size_t)A.T * A.k, R = S + A.T;
  const size_t Imax = A.I > A.Is ? A.I : A.Is;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  uint8_t* b = (uint8_t*)A.plan;
  PfLayout L;
  L.count = (int*)b;
  b += up(sizeof(int) * (A.E + 2));
  L.offset = (int*)b;
  b += up(sizeof(int) * (A.E + 2));
  L.rows = (int*)b;
  b += up(sizeof(int) * R);
  L.tiles = (int*)b;
  b += up(sizeof(int) * 2 * (size_t)prefill_tiles_cap(A.T, A.E, A.k));
  L.ntiles = (int*)b;
  b += up(256);
  L.act = (uint16_t*)b;
  b += up(2 * R * Imax);
  L.out = (uint16_t*)b;
  return L;
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *(const uint4*)p);
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Blocks are dispatched to the 8 XCDs round-robin; remap so that consecutive logical blocks
// (same tile / same expert, which share operands) run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_swizzle(int b, int nblocks) {
  const int per = nblocks / 8;
  return (b % 8) * per + b / 8;
}

// ------------------------------------------------------------------------------------------
// Router: logits[T][E] = x . Wr^T (+ bias), Wr split into three bf16 parts on the fly.
// Block: 64 tokens x 128 experts; 4 waves 2x2, wave tile 32 x 64 (two 32x32 MFMA tiles).
// ------------------------------------------------------------------------------------------
constexpr int kRtBT = 64, kRtBE = 128, kRtBK = 32, kRtLDK = kRtBK + 8;

__global__ __launch_bounds__(256) void pf_router(Args A) {
  __shared__ __attribute__((aligned(16))) uint16_t sx[kRtBT * kRtLDK];
  __shared__ __attribute__((aligned(16))) uint16_t sw[3][kRtBE * kRtLDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * kRtBT, e0 = blockIdx.y * kRtBE;
  f32x16_t acc[2] = {};
  // loaders: x tile 64 rows x 32 k = 256 chunks of 8 bf16 (one per thread);
  // Wr tile 128 rows x 32 k fp32 = 1024 chunks of 4 floats (four per thread)
  const int xr = tid >> 2, xc = tid & 3;
  const bool xok = t0 + xr < A.T;
  const uint16_t* xp = (const uint16_t*)A.x + (size_t)(xok ? t0 + xr : 0) * A.H + xc * 8;
  for (int k0 = 0; k0 < A.H; k0 += kRtBK) {
    uint4 xv = xok ? *(const uint4*)(xp + k0) : make_uint4(0, 0, 0, 0);
    *(uint4*)&sx[xr * kRtLDK + xc * 8] = xv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = tid + 256 * q, r = c >> 3, kc = c & 7;
      const bool ok = e0 + r < A.E;
      float4 w = ok ? *(const float4*)(A.rw + (size_t)(e0 + r) * A.H + k0 + kc * 4) : make_float4(0, 0, 0, 0);
      float wv[4] = {w.x, w.y, w.z, w.w};
      uint16_t hi[4], mid[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t u = __float_as_uint(wv[j]);
        const uint32_t uh = u & 0xffff0000u;               // truncation: exact leading part
        const float r1 = wv[j] - __uint_as_float(uh);       // exact remainder
        const uint32_t um = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(um);          // exact; fits in bf16
        hi[j] = (uint16_t)(uh >> 16);
        mid[j] = (uint16_t)(um >> 16);
        lo[j] = f32_to_bf16(r2);
      }
      uint2 vh = make_uint2(hi[0] | (uint32_t)hi[1] << 16, hi[2] | (uint32_t)hi[3] << 16);
      uint2 vm = make_uint2(mid[0] | (uint32_t)mid[1] << 16, mid[2] | (uint32_t)mid[3] << 16);
      uint2 vl = make_uint2(lo[0] | (uint32_t)lo[1] << 16, lo[2] | (uint32_t)lo[3] << 16);
      *(uint2*)&sw[0][r * kRtLDK + kc * 4] = vh;
      *(uint2*)&sw[1][r * kRtLDK + kc * 4] = vm;
      *(uint2*)&sw[2][r * kRtLDK + kc * 4] = vl;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kRtBK; ks += 16) {
      const int kk = ks + (lane >> 5) * 8;
      const bf16x8_t a = lds_frag(&sx[(wm * 32 + (lane & 31)) * kRtLDK + kk]);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int er = wn * 64 + n * 32 + (lane & 31);
#pragma unroll
        for (int p = 0; p < 3; ++p) acc[n] = mfma32(a, lds_frag(&sw[p][er * kRtLDK + kk]), acc[n]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int e = e0 + wn * 64 + n * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + wm * 32 + 8 * (r >> 2) + (lane >> 5) * 4 + (r & 3);
      if (t < A.T && e < A.E) {
        float l = acc[n][r];
        if (A.rbias) l += A.rbias[(size_t)t * A.bias_stride + e];
        A.logits[(size_t)t * A.E + e] = l;
      }
    }
  }
}

__global__ __launch_bounds__(256) void pf_select(Args A) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= A.T) return;
  const float* src = A.logits_in ? A.logits_in : A.logits;
  int* ids = A.ids + (size_t)t * A.k;
  float* w = A.cw + (size_t)t * A.k;
  select_token(src + (size_t)t * A.E, A.E, A.k, lane, ids, w);
  if (A.o_logits)
    for (int e = lane; e < A.E; e += 64) A.o_logits[(size_t)t * A.E + e] = src[(size_t)t * A.E + e];
  if (A.o_ids && lane < A.k) {  // each lane re-reads only what it wrote itself
    A.o_ids[(size_t)t * A.k + lane] = ids[lane];
    A.o_w[(size_t)t * A.k + lane] = w[lane];
  }
}

// ------------------------------------------------------------------------------------------
// Grouped GEMM main loop shared by gate/up and down.  A block stages a 128-row A tile and a
// 128-row B tile (rows = output columns, K contiguous) per K-step of 64 through two LDS
// buffers, with the next step's global loads held in registers: one barrier per step.  Each
// thread loads four 16-byte chunks of A and four of B per step; every load is unconditional
// (clamped to a valid address) and masked by selecting zero, so nothing branches in the loop.
// Four waves in a 2x2 grid each own a 64 x 64 corner = 2 x 2 MFMA 32x32 tiles.
// ------------------------------------------------------------------------------------------
struct TileOperands {
  const uint16_t* ap[4];  // A row chunk pointers (clamped)
  const uint16_t* bp[4];  // B row chunk pointers (clamped)
  bool aok[4], bok[4];    // row validity
  int K;                  // reduction length (multiple of 32)
};

__device__ __forceinline__ uint4 sel4(bool ok, uint4 v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

__device__ __forceinline__ void tile_load(const TileOperands& op, int k0, int kc, uint4* ra, uint4* rb) {
  const bool kok = k0 + kc * 8 < op.K;
  const int ko = kok ? k0 : 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ra[q] = sel4(kok && op.aok[q], *(const uint4*)(op.ap[q] + ko));
    rb[q] = sel4(kok && op.bok[q], *(const uint4*)(op.bp[q] + ko));
  }
}

__device__ __forceinline__ void tile_store(uint16_t* sa, uint16_t* sb, int tid, const uint4* ra,
                                           const uint4* rb) {
  const int kc = tid & 7;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = (tid >> 3) + 32 * q;
    *(uint4*)&sa[r * kPfLDK + kc * 8] = ra[q];
    *(uint4*)&sb[r * kPfLDK + kc * 8] = rb[q];
  }
}

__device__ __forceinline__ void tile_mma(const uint16_t* sa, const uint16_t* sb, int lane, int wm, int wn,
                                         f32x16_t (&acc)[2][2]) {
#pragma unroll
  for (int ks = 0; ks < kPfBK; ks += 16) {
    const int kk = ks + (lane >> 5) * 8;
    bf16x8_t af[2], bfr[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) af[m] = lds_frag(&sa[(wm * 64 + m * 32 + (lane & 31)) * kPfLDK + kk]);
#pragma unroll
    for (int n = 0; n < 2; ++n) bfr[n] = lds_frag(&sb[(wn * 64 + n * 32 + (lane & 31)) * kPfLDK + kk]);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n) acc[m][n] = mfma32(af[m], bfr[n], acc[m][n]);
  }
}

__device__ __forceinline__ void tile_gemm(const TileOperands& op, uint16_t (*sa)[kPfBM * kPfLDK],
                                          uint16_t (*sb)[kPfBM * kPfLDK], f32x16_t (&acc)[2][2]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, kc = tid & 7;
  const int nk = (op.K + kPfBK - 1) / kPfBK;
  uint4 r0a[4], r0b[4], r1a[4], r1b[4];
  tile_load(op, 0, kc, r0a, r0b);
  tile_load(op, kPfBK, kc, r1a, r1b);
  tile_store(sa[0], sb[0], tid, r0a, r0b);
  for (int kt = 0; kt < nk; kt += 2) {
    __syncthreads();
    if (kt + 1 < nk) tile_store(sa[1], sb[1], tid, r1a, r1b);
    if (kt + 2 < nk) tile_load(op, (kt + 2) * kPfBK, kc, r0a, r0b);
    tile_mma(sa[0], sb[0], lane, wm, wn, acc);
    if (kt + 1 < nk) {
      __syncthreads();
      if (kt + 2 < nk) tile_store(sa[0], sb[0], tid, r0a, r0b);
      if (kt + 3 < nk) tile_load(op, (kt + 3) * kPfBK, kc, r1a, r1b);
      tile_mma(sa[1], sb[1], lane, wm, wn, acc);
    }
  }
}

// Gate/up: block = (tile, 64 intermediate columns).  B rows 0..63 are gate rows n0..n0+63,
// rows 64..127 the matching up rows, so wave column half wn=0 holds gate and wn=1 holds up
// for the same 64 columns -> exchanged through LDS for the SwiGLU epilogue.
__global__ __launch_bounds__(256, 2) void pf_gateup(Args A, PfLayout L, int nb_per_tile, int nblocks) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][kPfBM * kPfLDK];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][kPfBM * kPfLDK];
  const int b = xcd_swizzle(blockIdx.x, nblocks);
  const int ti = b / nb_per_tile, nb = b - ti * nb_per_tile;
  if (ti >= *L.ntiles) return;
  const int g = L.tiles[2 * ti], it = L.tiles[2 * ti + 1];
  const bool shared = g == A.E;
  const int N = shared ? A.Is : A.I;
  const int n0 = nb * kPfBNI;
  if (n0 >= N) return;
  const int r0 = it * kPfBM, nrows = min(kPfBM, L.count[g] - r0);
  const int pos0 = L.offset[g] + r0;
  const int S = A.T * A.k;
  const size_t Imax = A.I > A.Is ? A.I : A.Is;
  const uint16_t* wg = shared ? (const uint16_t*)A.sgate : (const uint16_t*)A.gate + (size_t)g * A.I * A.H;
  const uint16_t* wu = shared ? (const uint16_t*)A.sup : (const uint16_t*)A.up + (size_t)g * A.I * A.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, kc = tid & 7;
  TileOperands op;
  op.K = A.H;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = (tid >> 3) + 32 * q;
    op.aok[q] = r < nrows;
    const int slot = L.rows[pos0 + (op.aok[q] ? r : 0)];
    const int t = slot < S ? slot / A.k : slot - S;
    op.ap[q] = (const uint16_t*)A.x + (size_t)t * A.H + kc * 8;
    const int n = n0 + (r & 63);
    op.bok[q] = n < N;
    op.bp[q] = (r < 64 ? wg : wu) + (size_t)(op.bok[q] ? n : 0) * A.H + kc * 8;
  }
  f32x16_t acc[2][2] = {};
  tile_gemm(op, sa, sb, acc);
  // SwiGLU epilogue: the wn=1 waves (up) hand their tiles to the wn=0 waves (gate) via LDS
  __syncthreads();
  // [wm][m][n][r][lane]: consecutive lanes hit consecutive banks
  float* xch = (float*)&sa[0][0];  // 2 x 64 floats x 64 lanes = 32 KB (fits in sa)
  if (wn == 1) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(((wm * 2 + m) * 2 + n) * 16 + r) * 64 + lane] = acc[m][n][r];
  }
  __syncthreads();
  if (wn == 0) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int col = n0 + n * 32 + (lane & 31);
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + m * 32 + 8 * (r >> 2) + (lane >> 5) * 4 + (r & 3);
          const float up = xch[(((wm * 2 + m) * 2 + n) * 16 + r) * 64 + lane];
          if (row < nrows) L.act[(size_t)(pos0 + row) * Imax + col] = f32_to_bf16(silu(acc[m][n][r]) * up);
        }
      }
    }
  }
}

// Down: block = (tile, 128 hidden columns).  Each row's result is scaled by its slot's
// routing weight (shared expert: 1) and stored as bf16 at its slot index.
__global__ __launch_bounds__(256, 2) void pf_down(Args A, PfLayout L, int nb_per_tile, int nblocks) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][kPfBM * kPfLDK];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][kPfBM * kPfLDK];
  const int b = xcd_swizzle(blockIdx.x, nblocks);
  const int ti = b / nb_per_tile, nb = b - ti * nb_per_tile;
  if (ti >= *L.ntiles) return;
  const int g = L.tiles[2 * ti], it = L.tiles[2 * ti + 1];
  const bool shared = g == A.E;
  const int h0 = nb * kPfBNH;
  const int r0 = it * kPfBM, nrows = min(kPfBM, L.count[g] - r0);
  const int pos0 = L.offset[g] + r0;
  const size_t Imax = A.I > A.Is ? A.I : A.Is;
  const uint16_t* wd = shared ? (const uint16_t*)A.sdown : (const uint16_t*)A.down + (size_t)g * A.H * A.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, kc = tid & 7;
  TileOperands op;
  op.K = shared ? A.Is : A.I;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = (tid >> 3) + 32 * q;
    op.aok[q] = r < nrows;
    op.ap[q] = L.act + (size_t)(pos0 + (op.aok[q] ? r : 0)) * Imax + kc * 8;
    const int h = h0 + r;
    op.bok[q] = h < A.H;
    op.bp[q] = wd + (size_t)(op.bok[q] ? h : 0) * op.K + kc * 8;
  }
  f32x16_t acc[2][2] = {};
  tile_gemm(op, sa, sb, acc);
  const int S = A.T * A.k;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + m * 32 + 8 * (r >> 2) + (lane >> 5) * 4 + (r & 3);
      if (row >= nrows) continue;
      const int slot = L.rows[pos0 + row];
      const float w = slot < S ? A.cw[slot] : 1.f;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int h = h0 + wn * 64 + n * 32 + (lane & 31);
        if (h < A.H) L.out[(size_t)slot * A.H + h] = f32_to_bf16(w * acc[m][n][r]);
      }
    }
  }
}

// y[t][h] = sum_j out[t*k + j][h] (+ out[S + t][h]); 8 columns per thread.
__global__ __launch_bounds__(256) void pf_combine(Args A, PfLayout L) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = A.H / 8;
  if (i >= (size_t)A.T * per_row) return;
  const int t = (int)(i / per_row), c = (int)(i % per_row) * 8;
  const int S = A.T * A.k;
  float acc[8] = {};
  auto add = [&](int row) {
    const uint4 v = *(const uint4*)&L.out[(size_t)row * A.H + c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16lo(w[j]);
      acc[2 * j + 1] += bf16hi(w[j]);
    }
  };
  for (int j = 0; j < A.k; ++j) add(t * A.k + j);
  if (A.Is > 0) add(S + t);
  if (A.odt == MOE_BF16) {
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = f32_to_bf16(acc[2 * j]) | ((uint32_t)f32_to_bf16(acc[2 * j + 1]) << 16);
    *(uint4*)((uint16_t*)A.y + (size_t)t * A.H + c) = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    float* yp = (float*)A.y + (size_t)t * A.H + c;
    *(float4*)yp = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *(float4*)(yp + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

}  // namespace

__global__ __launch_bounds__(1024) void permute(const int* ids, int T, int k, int E, bool with_shared,
                                                int* counts, int* offsets, int* rows, int* tiles,
                                                int* tiles_n, int bm);

// Router logits + per-token selection for T > 16 with bf16 activations (also used by
// moe_route so that routing-only calls take the forward path's arithmetic).
int launch_pf_route(Args A, hipStream_t st, const LaunchHook& hook) {
  hipError_t err;
  if (!A.logits_in) {
    hook.pre("pf_router", st);
    pf_router<<<dim3((A.T + kRtBT - 1) / kRtBT, (A.E + kRtBE - 1) / kRtBE), 256, 0, st>>>(A);
    hook.post(st);
    if ((err = hipGetLastError()) != hipSuccess) return MOE_EHIP;
  }
  hook.pre("pf_select", st);
  pf_select<<<(A.T + 3) / 4, 256, 0, st>>>(A);
  hook.post(st);
  if ((err = hipGetLastError()) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

int launch_prefill(Args A, hipStream_t st, const LaunchHook& hook) {
  const PfLayout L = pf_layout(A);
  hipError_t err;
  int rc = launch_pf_route(A, st, hook);
  if (rc) return rc;
  hook.pre("pf_permute", st);
  permute<<<1, 1024, 0, st>>>(A.ids, A.T, A.k, A.E, A.Is > 0, L.count, L.offset, L.rows, L.tiles,
                              L.ntiles, kPfBM);
  hook.post(st);
  if ((err = hipGetLastError()) != hipSuccess) return MOE_EHIP;
  const int cap = prefill_tiles_cap(A.T, A.E, A.k);
  const int Imax = A.I > A.Is ? A.I : A.Is;
  {
    const int nbt = (Imax + kPfBNI - 1) / kPfBNI;
    const int nblocks = (cap * nbt + 7) / 8 * 8;
    hook.pre("pf_gateup", st);
    pf_gateup<<<nblocks, 256, 0, st>>>(A, L, nbt, nblocks);
    hook.post(st);
    if ((err = hipGetLastError()) != hipSuccess) return MOE_EHIP;
  }
  {
    const int nbt = (A.H + kPfBNH - 1) / kPfBNH;
    const int nblocks = (cap * nbt + 7) / 8 * 8;
    hook.pre("pf_down", st);
    pf_down<<<nblocks, 256, 0, st>>>(A, L, nbt, nblocks);
    hook.post(st);
    if ((err = hipGetLastError()) != hipSuccess) return MOE_EHIP;
  }
  hook.pre("pf_combine", st);
  pf_combine<<<(unsigned)(((size_t)A.T * (A.H / 8) + 255) / 256), 256, 0, st>>>(A, L);
  hook.post(st);
  if ((err = hipGetLastError()) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

}  // namespace moe
