// Prefill path (T > 16): the layer as grouped GEMMs on MFMA.
//
//  router   logits = x . Wr^T on bf16 MFMA: x is bf16 exactly and every fp32 router weight is
//           split into three bf16 parts (hi + mid + lo == w) by a small pass, so each product
//           is exact and the three partial sums are added in fp32 -- fp32-accurate logits at
//           bf16 matrix-core rates.
//  select   one wave per token: the K-split partial logits added in split order, then the k
//           largest (ties to the lower index; ranked when the routing is an output).
//  permute  histogram of assignments per expert -> prefix scan -> scatter of slots into expert
//           groups -> block map of fixed-size row tiles ("Optimizing on-device inference for
//           Apple Silicon", section "Keep expert routing on the GPU"; the shared expert is one
//           more group holding every token).  No host synchronisation anywhere.
//  gate/up  per tile: the tile's token rows of x against the group's gate and up rows, SwiGLU
//           in the epilogue, bf16 activations in grouped order (same page, sections "Decode
//           weights during matrix multiplication" and "Match tile size to expert load").
//  down     per tile: activations x Wd^T, scaled by the slot's routing weight in the
//           epilogue, one bf16 row per slot.
//  combine  y[t] = sum_j out[t*k + j] + out_shared[t], a fixed order (deterministic).
//
// MXFP4 and group-wise affine 4-bit experts take the precise variant (template flag P) of the same kernels: the gate/up
// epilogue stores each fp32 activation as two bf16 parts, hi = bf16(a) and lo = bf16(a - hi),
// the down GEMM multiplies both parts by the same weight fragment (two MFMAs accumulating in
// fp32, so the activations keep about 16 significant bits instead of 8), and the per-slot rows
// stay fp32 through the combine.  The MXFP4 layer is held to a relative L2 error of 1e-3
// against the exactly dequantised layer, which bf16 activations and bf16 slot rows (each
// rounding costs about 1e-3 on its own) would not meet.
//
// The router, gate/up and down GEMMs share one block body (pf_gemm_body): 128 x 256 block
// tiles, K-steps of 32 staged in a two- or three-deep LDS ring that the buffer unit fills
// directly (loads to LDS, no register staging), rows XOR-swizzled so that MFMA fragment reads
// are free of bank conflicts.  W4A8's routed tiles run their own body on the block-scaled
// fp8 x fp4 matrix cores.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "select.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPfBM = kPfTileRows;  // rows per tile
constexpr int kPfBN = 256;     // B rows per block (gate/up: 128 activation columns x 2)
constexpr int kPfBK = 32;      // reduction step per LDS stage
constexpr int kPfNS = 3;       // LDS ring depth (two 256-thread blocks per CU)
constexpr int kPfNSG = 2;      // bf16 down GEMM: two stages, three blocks per CU (short K)

// The router GEMM splits K over this many blocks per output tile when the tiles alone would
// leave CUs idle (about 512 blocks wanted, at least four 32-deep K-steps per split); the
// selection kernel adds the partial logits in split order.
int pf_router_splits(int T, int H, int E) {
  const int tiles = ((T + kPfBM - 1) / kPfBM) * ((E + 63) / 64);
  const int want = (512 + tiles - 1) / tiles, most = std::max(1, H / kPfBK / 4);
  return std::max(1, std::min(want, most));
}

// W4A8: row strides of the MXFP8 scale arrays (one byte per 32 elements, padded to 16 bytes
// so that a row's scales stage into LDS with 16-byte loads)
inline int mx8_scale_ld(int K) { return (K / 32 + 15) / 16 * 16; }

size_t prefill_ws_bytes(int T, int H, int E, int k, int I, int Is, bool precise, bool w4a8) {
  const size_t S = (size_t)T * k, R = S + T;
  const size_t Imax = I > Is ? I : Is;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const int ks = pf_router_splits(T, H, E);
  const size_t np = precise ? 2 : 1;  // activation parts; slot rows fp32 instead of bf16
  return up(sizeof(int) * (E + 2)) * 2 + up(sizeof(int) * R) +
         up(sizeof(int) * 4 * (size_t)prefill_tiles_cap(T, E, k)) + up(256) + np * up(2 * R * Imax) +
         up(2 * np * R * (size_t)H) + up(2 * 3 * (size_t)E * H) +
         (ks > 1 ? up(sizeof(float) * (size_t)ks * T * E) : 0) +
         up(sizeof(int) * (size_t)permute_blocks(T, k) * E) +
         (w4a8 ? up((size_t)T * H) + up((size_t)T * mx8_scale_ld(H)) + up(R * Imax) + up(R * mx8_scale_ld((int)Imax))
               : 0);
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
  int* tiles;   // [cap] x {group, first row, rows, 0}
  int* ntiles;  // [1]
  uint16_t* act;     // [S+T][Imax] bf16 activations (precise: their hi parts)
  uint16_t* act_lo;  // precise: [S+T][Imax] the lo parts, else null
  uint16_t* out;     // [S+T][H] bf16 weighted slot rows (precise: null)
  float* outf;       // precise: [S+T][H] fp32 weighted slot rows, else null
  uint16_t* planes;  // [3][E][H] bf16 parts of the router weights
  float* rpart;      // [ks][T][E] partial router logits (K split ks > 1 ways), else null
  int ks;
  int* bcnt;         // [permute_blocks][E] per-block expert counts of the permutation
  // W4A8 (MXFP8 activations): x and the routed activations as E4M3 codes + e8m0 scales
  uint8_t* xq;       // [T][H]
  uint8_t* xs;       // [T][xs_ld]
  uint8_t* aq;       // [S+T][Imax] grouped order (routed rows)
  uint8_t* as;       // [S+T][as_ld]
  int xs_ld, as_ld;
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
  b += up(sizeof(int) * 4 * (size_t)prefill_tiles_cap(A.T, A.E, A.k));
  L.ntiles = (int*)b;
  b += up(256);
  const bool precise = A.wdt == MOE_MXFP4 || A.wdt == MOE_INT4G64;
  L.act = (uint16_t*)b;
  b += up(2 * R * Imax);
  L.act_lo = nullptr;
  if (precise) {
    L.act_lo = (uint16_t*)b;
    b += up(2 * R * Imax);
  }
  L.out = precise ? nullptr : (uint16_t*)b;
  L.outf = precise ? (float*)b : nullptr;
  b += up((precise ? 4 : 2) * R * (size_t)A.H);
  L.planes = (uint16_t*)b;
  b += up(2 * 3 * (size_t)A.E * A.H);
  L.ks = pf_router_splits(A.T, A.H, A.E);
  L.rpart = L.ks > 1 ? (float*)b : nullptr;
  if (L.ks > 1) b += up(sizeof(float) * (size_t)L.ks * A.T * A.E);
  L.bcnt = (int*)b;
  b += up(sizeof(int) * (size_t)permute_blocks(A.T, A.k) * A.E);
  L.xs_ld = mx8_scale_ld(A.H);
  L.as_ld = mx8_scale_ld((int)Imax);
  L.xq = L.xs = L.aq = L.as = nullptr;
  if (A.aq == MOE_QMXFP8) {
    L.xq = b;
    b += up((size_t)A.T * A.H);
    L.xs = b;
    b += up((size_t)A.T * L.xs_ld);
    L.aq = b;
    b += up(R * Imax);
    L.as = b;
  }
  return L;
}

// silu with the hardware exp and reciprocal (about 1 ulp each); its result is rounded to bf16.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Lanes l, l^1 hold column c, c^1 of rows R (a) and R + 1 (b).  The even lane returns row R's
// pair (c, c + 1) and the odd lane row R + 1's pair (c - 1, c), packed as two bf16.
__device__ __forceinline__ uint32_t pair_pack(float a, float b, bool odd) {
  const float send = odd ? a : b;
  const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false));
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const f2 v = {odd ? recv : a, odd ? b : recv};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Blocks are dispatched to the 8 XCDs round-robin; remap the first n blocks so that
// consecutive logical blocks (same tile / same expert, which share operands) run on the same
// XCD and share its L2.  A bijection on [0, n) for any n: XCD x takes a contiguous range of
// n / 8 (+1 for the first n % 8 XCDs) logical blocks.
__device__ __forceinline__ int xcd_swizzle(int h, int n) {
  const int x = h % 8, j = h / 8, q = n / 8, r = n % 8;
  return x * q + min(x, r) + j;
}

// Router weights -> three bf16 parts per element: hi = w truncated to bf16, mid = the
// remainder truncated, lo = what is left rounded (it fits exactly); hi + mid + lo == w.
__global__ __launch_bounds__(256) void pf_split_router(Args A, uint16_t* planes) {
  const size_t n = (size_t)A.E * A.H;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n / 4; i += (size_t)gridDim.x * 256) {
    const float4 w = ((const float4*)A.rw)[i];
    const float wv[4] = {w.x, w.y, w.z, w.w};
    uint16_t hi[4], mid[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t uh = __float_as_uint(wv[j]) & 0xffff0000u;
      const float r1 = wv[j] - __uint_as_float(uh);
      const uint32_t um = __float_as_uint(r1) & 0xffff0000u;
      const float r2 = r1 - __uint_as_float(um);
      hi[j] = (uint16_t)(uh >> 16);
      mid[j] = (uint16_t)(um >> 16);
      lo[j] = f32_to_bf16(r2);
    }
    auto pack = [](const uint16_t* v) {
      return make_uint2(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16);
    };
    ((uint2*)planes)[i] = pack(hi);
    ((uint2*)(planes + n))[i] = pack(mid);
    ((uint2*)(planes + 2 * n))[i] = pack(lo);
  }
}

// ------------------------------------------------------------------------------------------
// Grouped GEMM.  A block computes a BM-row x 256-column tile of C = A . B^T (B rows are
// output columns, K contiguous); BM / 32 waves in a (BM / 64) x 2 grid own 64 x 128 each
// (2 x 4 MFMA 32x32x16 tiles), except with 4-bit weights, where each of the four waves owns all
// 128 rows and 64 B rows of its own (4 x 2 tiles), so that every weight fragment is unpacked
// by one wave.  Operands are read through buffer resources: an offset at or past a
// resource's size reads as zero (kOOB), which masks rows past the tile or matrix end.
// Each K-step of 32 lands in one of NS LDS stages via buffer loads to LDS (every lane
// writes its 16 bytes at stage base + 16 * lane); 16-byte chunk c of row r sits at unit
// r * 4 + (c ^ (((r >> 1) ^ (r >> 2)) & 3)), which puts any 16 consecutive rows' copies of
// one chunk in distinct 16-byte bank slots of a 256-byte bank row (and any 8 in a 128-byte
// one), so fragment reads are free of bank conflicts.  Step s + NS - 1 is requested before
// step s is multiplied: one barrier per step.
//
// MODE 0 gate/up: A = gathered token rows of x; the B rows of column half h are 64 gate rows
//        and then 64 up rows of the activation columns n0 + 64 h ... + 63; the epilogue
//        applies SwiGLU in registers and stores bf16 activations.
// MODE 1 down: A = activation rows of the tile; B = Wd rows n0 ...; the epilogue scales by
//        the slot's routing weight and stores bf16 at the slot's row.
// MODE 2 router: A = token rows t0 ...; B rows per wave column half are the hi / mid / lo
//        parts of experts e0 + 32 wn ... (fourth group unused); the epilogue adds the three.
// ------------------------------------------------------------------------------------------
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kBufWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
typedef __attribute__((address_space(3))) void lds_void_t;


typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource: base address, stride 0, size in bytes (capped below kOOB), format word.
__device__ __forceinline__ i32x4_t buf_rsrc(const void* base, size_t bytes) {
  const uint64_t a = (uint64_t)base;
  return i32x4_t{(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xffff,
                 (int)(bytes < (size_t)kOOB ? bytes : (size_t)kOOB - 1), kBufWord3};
}

// 16 bytes per lane from buffer offset voff into LDS at lds_off + 16 * lane.  Written as
// inline assembly so that the compiler does not treat the pending write to LDS as a reason to
// wait for every outstanding load before each LDS read: the waits are placed by hand.  M0
// (the LDS base the load reads when it issues) is saved and put back around it.
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t voff, uint32_t lds_off) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(voff), "s"(rsrc), "s"(lds_off)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_t*)p;
}

__device__ __forceinline__ int swz_unit(int r, int c) { return r * 4 + (c ^ (((r >> 1) ^ (r >> 2)) & 3)); }

// s_waitcnt with only the vector-memory count constrained (expcnt and lgkmcnt left at max)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS sizes of one pf_gemm instance (16-byte units); the host sizes dynamic LDS from them.
template <int MODE, int BM, int NS, int WT, bool P>
struct PfCfg {
  static constexpr bool F4 = WT == MOE_MXFP4 || WT == MOE_INT4G64;  // 4-bit codes, 16 bytes per row per step
  static constexpr bool I4 = WT == MOE_INT4G64;                     // + a bf16 bias block per wave
  static constexpr bool AHL = P && MODE == 1;                    // A = activation hi and lo parts
  static constexpr int kUnitsA = BM * kPfBK * 2 / 16;             // one A part per stage
  static constexpr int kStageA = kUnitsA * (AHL ? 2 : 1);
  static constexpr int kStage = kStageA + (F4 ? kPfBN : kPfBN * kPfBK * 2 / 16);
  static constexpr int kNA = AHL ? 4 : 2;                         // A load instructions per wave per step
  static constexpr int kNB = F4 ? 1 : 512 / BM;                   // B load instructions per wave per step
  static constexpr bool kDyn = F4 || P;                           // LDS sized at launch
  static constexpr size_t ring_bytes = (size_t)NS * kStage * 16;
};

// The body of one GEMM block; bid: the block's index among the launch's blocks of this kind.
template <int MODE, int BM, int NS, int WT, bool P>
__device__ __forceinline__ void pf_gemm_body(const Args& A, const PfLayout& L, int nb_per_tile, int nblocks,
                                             int part, int bid) {
  typedef PfCfg<MODE, BM, NS, WT, P> C;
  constexpr bool F4 = C::F4, I4 = C::I4;
  constexpr int kStageA = C::kStageA, kStage = C::kStage, kNA = C::kNA, kNB = C::kNB;
  extern __shared__ __attribute__((aligned(16))) uint4 smem_dyn[];
  __shared__ __attribute__((aligned(16))) uint4 smem_st[C::kDyn ? 1 : NS * kStage];
  uint4* smem = C::kDyn ? smem_dyn : smem_st;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // the grouped GEMMs' real blocks are the first ntiles * nb_per_tile (the grid is sized for
  // the worst case); the rest leave at once.  part 1: the routed groups' tiles only, part 2:
  // the shared expert's tiles only (the last ceil(T / BM) of the map).
  const int shtiles = A.Is > 0 ? (A.T + BM - 1) / BM : 0;
  const int ntl = MODE == 2 ? 0 : *L.ntiles - (part == 1 ? shtiles : 0);
  const int nreal = MODE == 2 || part == 2 ? nblocks : min(nblocks, ntl * nb_per_tile);
  if (bid >= nreal) return;
  const int b = xcd_swizzle(bid, nreal);
  const int tb = b / nb_per_tile, ti = tb + (part == 2 ? *L.ntiles - shtiles : 0);
  int nb = b - tb * nb_per_tile, ksp = 0;  // router: nb_per_tile counts (group, K split) pairs
  if constexpr (MODE == 2) {
    ksp = nb % L.ks;
    nb /= L.ks;
  }
  const int S = A.T * A.k;
  const size_t Imax = A.I > A.Is ? A.I : A.Is;

  // ---- the tile
  int nrows, pos0 = 0, g = 0, K, N;
  if constexpr (MODE == 2) {
    nrows = min(BM, A.T - ti * BM);
    if (nrows <= 0) return;
    K = A.H;
    N = A.E;
  } else {
    if (ti >= *L.ntiles) return;
    const int4 tl = ((const int4*)L.tiles)[ti];  // {group, first row, rows, 0}
    g = tl.x;
    pos0 = tl.y;
    nrows = tl.z;
    K = MODE == 0 ? A.H : (g == A.E ? A.Is : A.I);
    N = MODE == 0 ? (g == A.E ? A.Is : A.I) : A.H;
  }
  const int n0 = MODE == 0 ? nb * (kPfBN / 2) : MODE == 1 ? nb * kPfBN : nb * 64;
  if (n0 >= N) return;

  // ---- per-lane load slots: 2 A (precise down: 2 hi + 2 lo) and kNB B 16-byte chunks per K-step
  i32x4_t ra, ra_lo, rb[kNB];
  uint32_t ao[2], bo[kNB];
  if constexpr (MODE == 0) ra = buf_rsrc(A.x, (size_t)A.T * A.H * 2);
  if constexpr (MODE == 1) ra = buf_rsrc(L.act + (size_t)pos0 * Imax, (size_t)nrows * Imax * 2);
  if constexpr (C::AHL) ra_lo = buf_rsrc(L.act_lo + (size_t)pos0 * Imax, (size_t)nrows * Imax * 2);
  if constexpr (MODE == 2) ra = buf_rsrc((const uint16_t*)A.x + (size_t)ti * BM * A.H, (size_t)nrows * A.H * 2);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = (wave * 2 + j) * 64 + lane, r = p >> 2, c = (p & 3) ^ (((r >> 1) ^ (r >> 2)) & 3);
    uint32_t rowb = kOOB;
    if (r < nrows) {
      if constexpr (MODE == 0) {
        const int slot = L.rows[pos0 + r];
        const int t = slot < S ? slot / A.k : slot - S;
        rowb = (uint32_t)t * A.H * 2u;
      } else if constexpr (MODE == 1) {
        rowb = (uint32_t)r * (uint32_t)Imax * 2u;
      } else {
        rowb = (uint32_t)r * A.H * 2u;
      }
    }
    ao[j] = rowb == kOOB ? kOOB : rowb + c * 16u;
  }
  // 4-bit B: row r of the tile is lane r % 64 of wave r / 64, one 16-byte chunk (32 codes) per
  // step.  The scales of a wave's 64 rows -- MXFP4: one e8m0 byte per 32; INT4G64: one bf16 per
  // 64, so sb = K / 32 bytes per row either way -- are one contiguous, 16-byte aligned block of
  // the scale matrix (64 sb is a multiple of 16), staged in LDS for the whole tile at wstr bytes
  // per wave; INT4G64 stages the bias block of the same rows right after it (wtot bytes per wave).
  const int sb = F4 ? K / 32 : 0, sbi = (64 * sb + 1023) / 1024, wstr = sbi * 1024, wtot = (I4 ? 2 : 1) * wstr;
  i32x4_t rs, rbi;
  uint32_t so = kOOB;  // the wave's first scale row's offset (uniform)
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    // bf16: instruction j of this wave covers B rows 16 (kNB wave + j) ... + 15
    int r, c;
    if constexpr (F4) {
      r = wave * 64 + lane;
      c = 0;
    } else {
      const int p = (wave * kNB + j) * 64 + lane;
      r = p >> 2;
      c = (p & 3) ^ (((r >> 1) ^ (r >> 2)) & 3);
    }
    const int half = r >> 7, jj = r & 127;
    uint32_t rowb = kOOB;
    if constexpr (MODE == 0) {
      // rows 64 half + 0..63 gate, 64 half + 64..127 up, of columns n0 + 64 half ... + 63
      const bool up = jj >> 6;  // uniform per instruction
      const bool sh = g == A.E;
      const int col = n0 + half * 64 + (jj & 63);
      if constexpr (F4) {
        const uint8_t* base = (const uint8_t*)(up ? A.up : A.gate) + (size_t)g * A.I * (A.H / 2);
        rb[j] = buf_rsrc(base, (size_t)N * (A.H / 2));
        if (col < N) rowb = (uint32_t)col * (A.H / 2);
        rs = buf_rsrc((const uint8_t*)(up ? A.us : A.gs) + (size_t)g * A.I * (A.H / 32), (size_t)N * (A.H / 32));
        if constexpr (I4)
          rbi = buf_rsrc((const uint8_t*)(up ? A.ub : A.gb) + (size_t)g * A.I * (A.H / 32), (size_t)N * (A.H / 32));
        so = (uint32_t)(n0 + half * 64) * (A.H / 32);
      } else {
        const uint16_t* base = up ? (sh ? (const uint16_t*)A.sup : (const uint16_t*)A.up + (size_t)g * A.I * A.H)
                                  : (sh ? (const uint16_t*)A.sgate : (const uint16_t*)A.gate + (size_t)g * A.I * A.H);
        rb[j] = buf_rsrc(base, (size_t)N * A.H * 2);
        if (col < N) rowb = (uint32_t)col * A.H * 2u;
      }
    } else if constexpr (MODE == 1) {
      const int h = n0 + r;
      if constexpr (F4) {
        rb[j] = buf_rsrc((const uint8_t*)A.down + (size_t)g * A.H * (A.I / 2), (size_t)A.H * (K / 2));
        if (h < A.H) rowb = (uint32_t)h * (K / 2);
        rs = buf_rsrc((const uint8_t*)A.ds + (size_t)g * A.H * (A.I / 32), (size_t)A.H * (K / 32));
        if constexpr (I4) rbi = buf_rsrc((const uint8_t*)A.db + (size_t)g * A.H * (A.I / 32), (size_t)A.H * (K / 32));
        so = (uint32_t)(n0 + wave * 64) * (K / 32);
      } else {
        const uint16_t* base = g == A.E ? (const uint16_t*)A.sdown : (const uint16_t*)A.down + (size_t)g * A.H * A.I;
        rb[j] = buf_rsrc(base, (size_t)A.H * K * 2);
        if (h < A.H) rowb = (uint32_t)h * K * 2u;
      }
    } else {
      rb[j] = buf_rsrc(L.planes, (size_t)3 * A.E * A.H * 2);
      const int plane = jj >> 5, e = n0 + half * 32 + (jj & 31);
      if (plane < 3 && e < A.E) rowb = ((uint32_t)plane * A.E + e) * A.H * 2u;
    }
    bo[j] = rowb == kOOB ? kOOB : rowb + c * 16u;
  }

  // K-steps [s0, s0 + nk) of this block (the router may split K)
  const int nk_all = K / kPfBK;
  const int s0 = MODE == 2 ? ksp * nk_all / L.ks : 0;
  const int nk = MODE == 2 ? (ksp + 1) * nk_all / L.ks - s0 : nk_all;
  constexpr int kNL = kNA + kNB;  // load instructions per wave per step
  // load li of step st (A, then the precise A's lo parts, then B) into its stage
  auto issue_one = [&](int st, uint4* stage, int li) {
    const uint32_t ks = (uint32_t)(s0 + (st < nk ? st : nk - 1));
    const uint32_t kb = ks * kPfBK * 2u, kbb = F4 ? ks * 16u : kb;
    if (li < 2) {
      dma16(ra, ao[li] + kb, lds_addr(stage + (wave * 2 + li) * 64));
    } else if (C::AHL && li < 4) {
      dma16(ra_lo, ao[li - 2] + kb, lds_addr(stage + C::kUnitsA + (wave * 2 + li - 2) * 64));
    } else {
      const int j = li - (C::AHL ? 4 : 2);
      dma16(rb[j], bo[j] + kbb, lds_addr(stage + kStageA + (wave * kNB + j) * 64));
    }
  };
  auto issue = [&](int st, uint4* stage) {
    const uint32_t ks = (uint32_t)(s0 + (st < nk ? st : nk - 1));
    const uint32_t kb = ks * kPfBK * 2u, kbb = F4 ? ks * 16u : kb;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(ra, ao[j] + kb, lds_addr(stage + (wave * 2 + j) * 64));
    if constexpr (C::AHL) {
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16(ra_lo, ao[j] + kb, lds_addr(stage + C::kUnitsA + (wave * 2 + j) * 64));
    }
#pragma unroll
    for (int j = 0; j < kNB; ++j) dma16(rb[j], bo[j] + kbb, lds_addr(stage + kStageA + (wave * kNB + j) * 64));
  };
  // MXFP4: the tile's scale rows, wave w's 64 rows by wave w, before the first stages (so the
  // first stage's wait covers them); they sit after the ring
  uint8_t* s_sc = (uint8_t*)(smem + NS * kStage);
  if constexpr (F4) {
    for (int i = 0; i < sbi; ++i)
      dma16(rs, so + (uint32_t)(i * 64 + lane) * 16u, lds_addr((uint4*)(s_sc + (size_t)wave * wtot) + i * 64));
    if constexpr (I4)
      for (int i = 0; i < sbi; ++i)
        dma16(rbi, so + (uint32_t)(i * 64 + lane) * 16u,
              lds_addr((uint4*)(s_sc + (size_t)wave * wtot + wstr) + i * 64));
  }

  // down: the tile's slots and routing weights, staged in LDS while the operands stream
  __shared__ int s_slot[BM];
  __shared__ float s_wt[BM];
  if constexpr (MODE == 1) {
    if (tid < nrows) {
      const int slot = L.rows[pos0 + tid];
      s_slot[tid] = slot;
      s_wt[tid] = slot < S ? A.cw[slot] : 1.f;
    }
  }
  // router: this lane's bias column when the bias is shared by all tokens
  float bias_e = 0.f;
  if constexpr (MODE == 2) {
    const int e = n0 + wn * 32 + (lane & 31);
    if (A.rbias && A.bias_stride == 0 && e < A.E) bias_e = A.rbias[e];
  }

  // 4-bit weights: every wave takes all 128 rows and its own 64 B rows (gate/up: the gate and
  // up tiles of 32 activation columns; down: 64 output columns), so each B fragment is
  // unpacked by one wave instead of two
  constexpr bool W14 = F4;
  constexpr int MT = W14 ? 4 : 2, NTW = W14 ? 2 : 4;  // MFMA tiles per wave: rows, columns
  const int mrow0 = W14 ? 0 : wm * 64;
  // rows of this wave that hold data (uniform): skip MFMA tiles wholly past the tile end
  const int mlive = min(MT, max(0, (nrows - mrow0 + 31) / 32));
  f32x16_t acc[MT][NTW] = {};
  // One K-step: wait for its stage, refill the ring, then the fragment reads of the step (both
  // 16-deep halves, or one half at a time with a two-stage ring) before their MFMAs, so that
  // the reads' latency overlaps the first MFMAs.  The precise down GEMM (two MFMAs per tile)
  // issues the refill loads one at a time between its MFMAs instead: a load waits in the
  // buffer unit's queue while the MFMAs issued before it run (its precise 4-bit downs measured
  // 4-5% faster that way; the one-MFMA GEMMs are slower with it).  ML = the wave's live 32-row groups, a constant inside the loop (the loop is
  // instantiated per value), so nothing branches between the MFMAs.
  auto step = [&](auto ml_c, int s) {
    constexpr int ML = decltype(ml_c)::value;
    wait_vm<(kNA + kNB) * (NS - 2)>();  // this wave's loads of step s have landed (later ones in flight)
    __syncthreads();          // ... and every other wave's; all are done with step s - 1's stage
    uint4* const nst = smem + ((s + NS - 1) % NS) * kStage;
    constexpr bool kSpread = C::AHL && ML > 0;
    if constexpr (!kSpread) issue(s + NS - 1, nst);
    if constexpr (ML == 0) return;
    int li = 0;  // spread refill loads issued so far
    const uint4* st = smem + (s % NS) * kStage;
    // two-stage rings run three blocks per CU: one half's fragments at a time
    constexpr int KB = NS >= 3 ? 2 : 1;
#pragma unroll
    for (int kb = 0; kb < 2; kb += KB) {
    bf16x8_t af[2][MT], afl[2][MT], bfr[2][NTW];
#pragma unroll
    for (int ks = kb; ks < kb + KB; ++ks) {
      const int c = ks * 2 + (lane >> 5);
#pragma unroll
      for (int m = 0; m < ML; ++m) {
        af[ks][m] = __builtin_bit_cast(bf16x8_t, st[swz_unit(mrow0 + m * 32 + (lane & 31), c)]);
        if constexpr (C::AHL)
          afl[ks][m] = __builtin_bit_cast(bf16x8_t, st[C::kUnitsA + swz_unit(mrow0 + m * 32 + (lane & 31), c)]);
      }
#pragma unroll
      for (int n = 0; n < NTW; ++n) {
        // W14 gate/up: the wave's gate rows (n = 0) and up rows (n = 1) of activation columns
        // n0 + 32 wave ... + 31, which sit in B rows 128 (wave / 2) + 32 (wave % 2) + 64 n + i;
        // W14 down: B rows 64 wave + 32 n + i
        const int br = !W14 ? wn * 128 + n * 32 + (lane & 31)
                       : MODE == 0 ? (wave >> 1) * 128 + (wave & 1) * 32 + n * 64 + (lane & 31)
                                   : wave * 64 + n * 32 + (lane & 31);
        if constexpr (I4) {  // 8 codes -> bf16(s * q + b), the group's scale and bias (one group per 2 steps)
          const uint32_t q = ((const uint32_t*)(st + kStageA + br))[c];
          const uint8_t* sp = s_sc + (br >> 6) * wtot + (br & 63) * sb + 2 * ((s0 + s) >> 1);
          const float gs = bf16_to_f32(*(const uint16_t*)sp), gb = bf16_to_f32(*(const uint16_t*)(sp + wstr));
          const uint32_t ev = q & 0x0F0F0F0Fu, od = (q >> 4) & 0x0F0F0F0Fu;
          uint32_t v[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            typedef float f2 __attribute__((ext_vector_type(2)));
            typedef __bf16 b2 __attribute__((ext_vector_type(2)));
            const f2 w2 = {fmaf(gs, (float)((ev >> (8 * p)) & 0xFFu), gb), fmaf(gs, (float)((od >> (8 * p)) & 0xFFu), gb)};
            v[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w2, b2));
          }
          bfr[ks][n] = __builtin_bit_cast(bf16x8_t, make_uint4(v[0], v[1], v[2], v[3]));
        } else if constexpr (F4) {  // 8 codes of this lane's K range, scaled while unpacked to bf16
          const uint32_t q = ((const uint32_t*)(st + kStageA + br))[c];
          const float sc = e8m0_to_f32(s_sc[(br >> 6) * wtot + (br & 63) * sb + s0 + s]);
          uint32_t v[4];
          v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 0));
          v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 1));
          v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 2));
          v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 3));
          bfr[ks][n] = __builtin_bit_cast(bf16x8_t, make_uint4(v[0], v[1], v[2], v[3]));
        } else {
          bfr[ks][n] = __builtin_bit_cast(bf16x8_t, st[kStageA + swz_unit(br, c)]);
        }
      }
    }
    // every read of the batch is issued before its first MFMA (two-stage rings: left to the
    // scheduler, which keeps the registers within three blocks per CU)
    if constexpr (NS >= 3) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = kb; ks < kb + KB; ++ks)
#pragma unroll
      for (int m = 0; m < ML; ++m)
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
          acc[m][n] = mfma32(af[ks][m], bfr[ks][n], acc[m][n]);
          if constexpr (C::AHL) acc[m][n] = mfma32(afl[ks][m], bfr[ks][n], acc[m][n]);
          if constexpr (kSpread) {  // kNL loads evenly over the step's 2 NTW ML tile groups
            const int mi = (ks * ML + m) * NTW + n;
            if ((mi + 1) * kNL / (2 * NTW * ML) > li) {  // constant once unrolled
              __builtin_amdgcn_sched_barrier(0);
              issue_one(s + NS - 1, nst, li);
              ++li;
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
    }
    if constexpr (kSpread)
      while (li < kNL) issue_one(s + NS - 1, nst, li++);
  };
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) issue(i, smem + i * kStage);
  typedef std::integral_constant<int, 0> ML0;
  typedef std::integral_constant<int, 1> ML1;
  typedef std::integral_constant<int, 2> ML2;
  typedef std::integral_constant<int, 3> ML3;
  typedef std::integral_constant<int, 4> ML4;
  auto run_k = [&](auto ml_c) {
    for (int s = 0; s < nk; ++s) step(ml_c, s);
  };
  if constexpr (W14) {
    if (mlive == 4)  // uniform
      run_k(ML4{});
    else if (mlive == 3)
      run_k(ML3{});
    else if (mlive == 2)
      run_k(ML2{});
    else if (mlive == 1)
      run_k(ML1{});
    else
      run_k(ML0{});
  } else {
    if (mlive == 2)  // uniform
      run_k(ML2{});
    else if (mlive == 1)
      run_k(ML1{});
    else
      run_k(ML0{});
  }
  wait_vm<0>();  // no load may still write this block's LDS after it retires

  // ---- epilogue; C row = wm * 64 + m * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4
  if constexpr (MODE == 2) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + m * 32 + 8 * (r >> 2) + (lane >> 5) * 4 + (r & 3);
        if (row >= nrows) continue;
        const int e = n0 + wn * 32 + (lane & 31), t = ti * BM + row;
        if (e < A.E) {
          float l = (acc[m][0][r] + acc[m][1][r]) + acc[m][2][r];
          if (L.ks > 1) {  // partial over this K split; the selection kernel adds bias and parts
            L.rpart[((size_t)ksp * A.T + t) * A.E + e] = l;
          } else {
            if (A.rbias) l += A.bias_stride == 0 ? bias_e : A.rbias[(size_t)t * A.bias_stride + e];
            A.logits[(size_t)t * A.E + e] = l;
          }
        }
      }
    }
  } else if constexpr (MODE == 1 && P) {
    // precise down: fp32 weighted rows straight from the accumulators; lanes 0-31 and 32-63
    // of a store hold 32 consecutive columns of two rows, two whole 128-byte pieces
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mrow0 + m * 32 + 8 * (r >> 2) + (lane >> 5) * 4 + (r & 3);
        if (row >= nrows) continue;
        const float wt = s_wt[row];
        float* orow = L.outf + (size_t)s_slot[row] * A.H;
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
          const int col = n0 + (W14 ? wave * 64 : wn * 128) + n * 32 + (lane & 31);
          if (col < N) orow[col] = wt * acc[m][n][r];
        }
      }
    }
  } else {
    // The bf16 tile goes through LDS (the operand ring is free now), so that the global
    // stores are whole 16-byte row pieces instead of one 2-byte element per lane; when the
    // ring is smaller than the tile, the two 64-row halves (wm = 0, 1) go one after the other.
    // Precise gate/up stores two planes, the activations' bf16 hi parts and then their lo
    // parts (a - hi, rounded to bf16), one pass each.
    constexpr int CW = MODE == 0 ? kPfBN / 2 : kPfBN;  // output columns of the tile
    constexpr int LDW = CW + 8;                          // padded LDS row (bf16)
    constexpr int kHalves = (C::kDyn || BM * LDW * 2 <= NS * kStage * 16) ? 1 : 2;
    static_assert(C::kDyn || (BM / kHalves) * LDW * 2 <= NS * kStage * 16, "the output rows fit in the ring");
    constexpr int HR = BM / kHalves;  // tile rows per pass
    constexpr int kPlanes = P ? 2 : 1;
    uint16_t* ct = (uint16_t*)smem;
    // A lane holds one column of rows R and R + 1 (r even, r + 1); lane pairs swap one value
    // so that the even lane stores (R, c..c+1) and the odd lane (R + 1, c-1..c) as one dword.
    const bool odd = lane & 1;
#pragma unroll
    for (int pl = 0; pl < kPlanes; ++pl) {
#pragma unroll
    for (int hp = 0; hp < kHalves; ++hp) {
      __syncthreads();  // every wave is done with the ring (or with the previous pass)
      if (kHalves == 1 || wm == hp) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const int row0 = mrow0 + m * 32 + 8 * (r >> 2) + (lane >> 5) * 4 + (r & 3);
            const int row = row0 + (odd ? 1 : 0);
            uint32_t* crow = (uint32_t*)(ct + (row - hp * HR) * LDW) + ((lane & 31) >> 1);
            if constexpr (MODE == 0) {
              // gate tile pr, up tile NTW / 2 + pr; W14: one pair at columns 32 wave ...
#pragma unroll
              for (int pr = 0; pr < NTW / 2; ++pr) {
                float a = silu_fast(acc[m][pr][r]) * acc[m][NTW / 2 + pr][r];
                float b = silu_fast(acc[m][pr][r + 1]) * acc[m][NTW / 2 + pr][r + 1];
                if (P && pl == 1) {  // the lo parts: what bf16 rounding left out (exact in fp32)
                  a -= bf16_to_f32(f32_to_bf16(a));
                  b -= bf16_to_f32(f32_to_bf16(b));
                }
                crow[((W14 ? wave * 32 : wn * 64) + pr * 32) / 2] = pair_pack(a, b, odd);
              }
            } else {
              const float wa = row0 < nrows ? s_wt[row0] : 0.f, wb = row0 + 1 < nrows ? s_wt[row0 + 1] : 0.f;
#pragma unroll
              for (int n = 0; n < NTW; ++n)
                crow[((W14 ? wave * 64 : wn * 128) + n * 32) / 2] =
                    pair_pack(wa * acc[m][n][r], wb * acc[m][n][r + 1], odd);
            }
          }
        }
      }
      __syncthreads();
      constexpr int UPR = CW / 8;  // 16-byte units per tile row
      const int prow = min(HR, nrows - hp * HR);
      uint16_t* const dst = MODE == 0 ? (pl == 0 ? L.act : L.act_lo) : L.out;
      for (int u = tid; u < prow * UPR; u += 2 * BM) {
        const int rr = u / UPR, cu = u - rr * UPR, col = n0 + cu * 8, row = hp * HR + rr;
        if (col >= N) continue;
        const uint4 v = *(const uint4*)&ct[rr * LDW + cu * 8];
        if constexpr (MODE == 0)
          *(uint4*)&dst[(size_t)(pos0 + row) * Imax + col] = v;
        else
          *(uint4*)&dst[(size_t)s_slot[row] * A.H + col] = v;
      }
    }
    }
  }
}

template <int MODE, int BM, int NS, int WT, bool P>
__global__ __launch_bounds__(2 * BM, BM == 128 ? (NS == 2 ? 3 : 2) : 1)
void pf_gemm(Args A, PfLayout L, int nb_per_tile, int nblocks, int part) {
  pf_gemm_body<MODE, BM, NS, WT, P>(A, L, nb_per_tile, nblocks, part, blockIdx.x);
}

// ------------------------------------------------------------------------------------------
// W4A8: MXFP8 activations against MXFP4 weights on gfx950's block-scaled matrix cores
// ("Three ways to boost mixture-of-experts inference on NVIDIA DGX Spark", section "Why
// decoding was slow in the first place": MXFP4 expert weights with 8-bit activations).  MXFP8
// per OCP MX v1.0: per 32 elements a scale 2^(floor(log2 amax) - 8) (8: the largest exponent of
// an E4M3 value), clamped to the e8m0 range, and E4M3 elements rounded to nearest even,
// saturated at +-448 (the input is clamped first; the hardware conversion then rounds to
// nearest even).
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ int mx8_exp(float amax) {
  if (!(amax > 0.f)) return -127;  // a block of zeros
  const int e = __builtin_amdgcn_frexp_expf(amax) - 9;  // frexp: amax = m 2^p, m in [0.5, 1)
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
__device__ __forceinline__ float mx8_clamp(float v) { return fminf(fmaxf(v, -448.f), 448.f); }
// four values (already divided by the block scale) -> four E4M3 codes, first in the low byte
__device__ __forceinline__ uint32_t mx8_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(mx8_clamp(a), mx8_clamp(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(mx8_clamp(c), mx8_clamp(d), w, true);
}

// x [T][H] bf16 -> E4M3 codes xq [T][H] and e8m0 scales xs [T][xs_ld]; one 32-element block per
// thread.
__global__ __launch_bounds__(256) void pf_quant_x(Args A, PfLayout L) {
  const int nb = A.H / 32;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)A.T * nb) return;
  const int t = (int)(i / nb), blk = (int)(i % nb);
  const uint4* src = (const uint4*)((const uint16_t*)A.x + (size_t)t * A.H + (size_t)blk * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 u = src[q];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * q + 2 * j] = bf16lo(w[j]);
      v[8 * q + 2 * j + 1] = bf16hi(w[j]);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const int xe = mx8_exp(amax);
  uint32_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    c[j] = mx8_pack4(ldexpf(v[4 * j], -xe), ldexpf(v[4 * j + 1], -xe), ldexpf(v[4 * j + 2], -xe),
                     ldexpf(v[4 * j + 3], -xe));
  uint4* dst = (uint4*)(L.xq + (size_t)t * A.H + (size_t)blk * 32);
  dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
  dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
  L.xs[(size_t)t * L.xs_ld + blk] = (uint8_t)(xe + 127);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// The grouped GEMM for W4A8, routed tiles only: 128 x 256 block tiles as pf_gemm, K-steps of 64
// (one v_mfma_scale_f32_32x32x64_f8f6f4 per 32 x 32 tile), a three-deep LDS ring filled by
// buffer loads to LDS: A = 128 rows x 64 E4M3 codes (the row XOR swizzle of pf_gemm, 64-byte
// rows), B = 256 rows x 64 e2m1 codes (32 bytes).  The e8m0 scales of the tile's A rows and of
// each wave's 64 B rows are staged once per tile.  Operand layout of the instruction: A lane
// (row, h) holds K [16h, 16h + 16) and [32 + 16h, 32 + 16h + 16), B lane (column, h) holds K
// [32h, 32h + 32), and lane (row or column, h) supplies the scale of the 32-block h.
// MODE 0 gate/up: A = the tile's token rows of xq, epilogue SwiGLU -> MXFP8 activations (aq, as).
// MODE 1 down: A = the tile's rows of aq; epilogue: fp32 rows weighted by the routing weight.
template <int MODE, int NS>
__device__ __forceinline__ void pf_gemm_w4a8_body(const Args& A, const PfLayout& L, int nb_per_tile, int nblocks,
                                                  int bid) {  // the routed tiles only
  constexpr int BM = kPfBM;
  constexpr int kUA = BM * 64 / 16;        // 16-byte units of A per stage (128 rows x 64 bytes)
  constexpr int kUB = kPfBN * 32 / 16;     // of B (256 rows x 32 bytes)
  constexpr int kStage = kUA + kUB;
  extern __shared__ __attribute__((aligned(16))) uint4 smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5;
  const int shtiles = A.Is > 0 ? (A.T + BM - 1) / BM : 0;
  const int ntl = *L.ntiles - shtiles;  // the routed groups' tiles come first in the map
  const int nreal = min(nblocks, ntl * nb_per_tile);
  if (bid >= nreal) return;
  const int b = xcd_swizzle(bid, nreal);
  const int ti = b / nb_per_tile, nb = b - ti * nb_per_tile;
  const int4 tl = ((const int4*)L.tiles)[ti];  // {group, first row, rows, 0}
  const int g = tl.x, pos0 = tl.y, nrows = tl.z;
  const int K = MODE == 0 ? A.H : A.I, N = MODE == 0 ? A.I : A.H;
  const int n0 = MODE == 0 ? nb * (kPfBN / 2) : nb * kPfBN;
  if (n0 >= N) return;
  const int S = A.T * A.k;
  const size_t Imax = A.I > A.Is ? A.I : A.Is;
  const int ald = MODE == 0 ? L.xs_ld : L.as_ld;  // A scale bytes per row (padded)

  // ---- A: per lane two 16-byte units per step (rows r = p / 4, chunk (p % 4) ^ swizzle)
  i32x4_t ra, ras;
  uint32_t ao[2];
  if constexpr (MODE == 0) {
    ra = buf_rsrc(L.xq, (size_t)A.T * A.H);
    ras = buf_rsrc(L.xs, (size_t)A.T * L.xs_ld);
  } else {
    ra = buf_rsrc(L.aq + (size_t)pos0 * Imax, (size_t)nrows * Imax);
    ras = buf_rsrc(L.as + (size_t)pos0 * L.as_ld, (size_t)nrows * L.as_ld);
  }
  auto a_row = [&](int r) -> int {  // the A row of tile row r in its array (-1: past the tile)
    if (r >= nrows) return -1;
    if constexpr (MODE == 0) {
      const int slot = L.rows[pos0 + r];
      return slot / A.k;  // routed tiles only: slot < S
    }
    return r;
  };
  const uint32_t a_ld = MODE == 0 ? (uint32_t)A.H : (uint32_t)Imax;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = (wave * 2 + j) * 64 + lane, r = p >> 2, c = (p & 3) ^ (((r >> 1) ^ (r >> 2)) & 3);
    const int ar = a_row(r);
    ao[j] = ar < 0 ? kOOB : (uint32_t)ar * a_ld + c * 16u;
  }
  // ---- B: per lane two 16-byte units per step (row p / 2, half p % 2)
  i32x4_t rb[2];
  uint32_t bo[2];
  i32x4_t rs;
  uint32_t so = 0;  // the wave's first B scale row's offset (uniform)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = (wave * 2 + j) * 64 + lane, r = p >> 1, c = p & 1;
    uint32_t rowb = kOOB;
    if constexpr (MODE == 0) {
      const int half = r >> 7, jj = r & 127;
      const bool up = jj >> 6;  // uniform per instruction
      const int col = n0 + half * 64 + (jj & 63);
      rb[j] = buf_rsrc((const uint8_t*)(up ? A.up : A.gate) + (size_t)g * A.I * (A.H / 2), (size_t)N * (A.H / 2));
      if (col < N) rowb = (uint32_t)col * (A.H / 2);
    } else {
      const int hh = n0 + r;
      rb[j] = buf_rsrc((const uint8_t*)A.down + (size_t)g * A.H * (A.I / 2), (size_t)A.H * (K / 2));
      if (hh < A.H) rowb = (uint32_t)hh * (K / 2);
    }
    bo[j] = rowb == kOOB ? kOOB : rowb + c * 16u;
  }
  const int sb = K / 32, sbi = (64 * sb + 1023) / 1024, wstr = sbi * 1024;  // B scale bytes per row / per wave
  if constexpr (MODE == 0) {
    const bool up = wave & 1;  // wave w stages B rows 64 w ... : half w / 2, gate (w even) or up
    rs = buf_rsrc((const uint8_t*)(up ? A.us : A.gs) + (size_t)g * A.I * (A.H / 32), (size_t)N * (A.H / 32));
    so = (uint32_t)(n0 + (wave >> 1) * 64) * (A.H / 32);
  } else {
    rs = buf_rsrc((const uint8_t*)A.ds + (size_t)g * A.H * (A.I / 32), (size_t)A.H * (K / 32));
    so = (uint32_t)(n0 + wave * 64) * (K / 32);
  }
  uint8_t* s_bs = (uint8_t*)(smem + NS * kStage);      // [4 waves][wstr]
  uint8_t* s_as = s_bs + 4 * wstr;                     // [BM rows][ald]
  const int nk = K / 64;
  auto issue = [&](int st, uint4* stage) {
    const uint32_t ks = (uint32_t)(st < nk ? st : nk - 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(ra, ao[j] + ks * 64u, lds_addr(stage + (wave * 2 + j) * 64));
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(rb[j], bo[j] + ks * 32u, lds_addr(stage + kUA + (wave * 2 + j) * 64));
  };
  // scales first (the first stage's wait covers them): the wave's 64 B rows, then the tile's A rows
  for (int i = 0; i < sbi; ++i)
    dma16(rs, so + (uint32_t)(i * 64 + lane) * 16u, lds_addr((uint4*)(s_bs + (size_t)wave * wstr) + i * 64));
  {
    const int upr = ald / 16, nu = BM * upr;  // 16-byte units per A scale row / per tile
    for (int u0 = wave * 64; u0 < nu; u0 += 4 * 64) {  // uniform trip count per wave
      const int u = u0 + lane, r = u / upr, cu = u - r * upr;
      const int ar = u < nu ? a_row(r) : -1;
      const uint32_t off = ar < 0 ? kOOB : (uint32_t)ar * (uint32_t)ald + cu * 16u;
      dma16(ras, off, lds_addr((uint4*)s_as + u0));
    }
  }
  __shared__ int s_slot[BM];
  __shared__ float s_wt[BM];
  if constexpr (MODE == 1) {
    if (tid < nrows) {
      const int slot = L.rows[pos0 + tid];
      s_slot[tid] = slot;
      s_wt[tid] = A.cw[slot];
    }
  }
  const int mlive = min(2, max(0, (nrows - wm * 64 + 31) / 32));
  f32x16_t acc[2][4] = {};
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) issue(i, smem + i * kStage);
  // one K-step: ML = the wave's live 32-row groups, a constant inside the loop (instantiated per
  // value); every operand read of the step is issued before its first MFMA
  auto step = [&](auto ml_c, int s) {
    constexpr int ML = decltype(ml_c)::value;
    wait_vm<4 * (NS - 2)>();  // this wave's loads of step s (and the scales) have landed
    __syncthreads();
    issue(s + NS - 1, smem + ((s + NS - 1) % NS) * kStage);
    if constexpr (ML == 0) return;
    const uint4* st = smem + (s % NS) * kStage;
    i32x8_t af[2], bfr[4];
    int sa[2], sbv[4];
#pragma unroll
    for (int m = 0; m < ML; ++m) {
      const int row = wm * 64 + m * 32 + (lane & 31);
      const uint4 u0 = st[swz_unit(row, h)], u1 = st[swz_unit(row, 2 + h)];
      af[m] = i32x8_t{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
      sa[m] = s_as[row * ald + 2 * s + h];
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int br = wn * 128 + n * 32 + (lane & 31);
      const uint4 u = st[kUA + br * 2 + h];
      bfr[n] = i32x8_t{(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
      sbv[n] = s_bs[(br >> 6) * wstr + (br & 63) * sb + 2 * s + h];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int m = 0; m < ML; ++m)
        acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[m], bfr[n], acc[m][n], 0, 4, 0, sa[m], 0, sbv[n]);
  };
  typedef std::integral_constant<int, 0> ML0;
  typedef std::integral_constant<int, 1> ML1;
  typedef std::integral_constant<int, 2> ML2;
  if (mlive == 2)  // uniform
    for (int s = 0; s < nk; ++s) step(ML2{}, s);
  else if (mlive == 1)
    for (int s = 0; s < nk; ++s) step(ML1{}, s);
  else
    for (int s = 0; s < nk; ++s) step(ML0{}, s);
  wait_vm<0>();

  // ---- epilogue; C row = wm * 64 + m * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4, column lane % 32
  if constexpr (MODE == 0) {
    // SwiGLU, then MXFP8 per 32 activation columns of a row: the 32 lanes of a half-wave hold one
    // such block, so its amax is a reduction over them; codes go through LDS for 16-byte stores
    constexpr int LDB = kPfBN / 2 + 16;  // bytes per LDS row
    uint8_t* ct = (uint8_t*)smem;
    __syncthreads();  // every wave is done with the ring
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + m * 32 + 8 * (r >> 2) + (lane >> 5) * 4 + (r & 3);
          const float v = silu_fast(acc[m][pr][r]) * acc[m][2 + pr][r];
          float am = fabsf(v);
          am = fmaxf(am, dpp_f<kDppXor1>(am));
          am = fmaxf(am, dpp_f<kDppXor2>(am));
          am = fmaxf(am, dpp_f<kDppHalfMirror>(am));
          am = fmaxf(am, dpp_f<kDppMirror>(am));
          am = fmaxf(am, __shfl_xor(am, 16, 64));
          const int xe = mx8_exp(am);
          const int code = __builtin_amdgcn_cvt_pk_fp8_f32(mx8_clamp(ldexpf(v, -xe)), 0.f, 0, false) & 0xFF;
          const int colb = wn * 64 + pr * 32;  // the block's first column in the tile
          ct[row * LDB + colb + (lane & 31)] = (uint8_t)code;
          if ((lane & 31) == 0 && row < nrows && n0 + colb < N)
            L.as[(size_t)(pos0 + row) * L.as_ld + (n0 + colb) / 32] = (uint8_t)(xe + 127);
        }
      }
    }
    __syncthreads();
    constexpr int UPR = (kPfBN / 2) / 16;  // 16-byte units per tile row
    for (int u = tid; u < nrows * UPR; u += 2 * BM) {
      const int rr = u / UPR, cu = u - rr * UPR, col = n0 + cu * 16;
      if (col >= N) continue;
      *(uint4*)&L.aq[(size_t)(pos0 + rr) * Imax + col] = *(const uint4*)&ct[rr * LDB + cu * 16];
    }
  } else {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + m * 32 + 8 * (r >> 2) + (lane >> 5) * 4 + (r & 3);
        if (row >= nrows) continue;
        const float wt = s_wt[row];
        float* orow = L.outf + (size_t)s_slot[row] * A.H;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int col = n0 + wn * 128 + n * 32 + (lane & 31);
          if (col < N) orow[col] = wt * acc[m][n][r];
        }
      }
    }
  }
  (void)S;
}

template <int MODE, int NS>
__global__ __launch_bounds__(2 * kPfBM, 2) void pf_gemm_w4a8(Args A, PfLayout L, int nb_per_tile, int nblocks, int) {
  pf_gemm_w4a8_body<MODE, NS>(A, L, nb_per_tile, nblocks, blockIdx.x);
}

// One launch for the two kinds of tile of a layer with 4-bit experts: the shared expert's
// (bf16, precise) tiles take the first nblk_s blocks, the routed groups' tiles (WT; MOE_MXFP4
// with W8 = W4A8) the rest.  The shared tiles then share the machine with the routed ones
// instead of running alone at low occupancy after them.  The shared down tiles keep a
// two-stage ring, so that their LDS (bf16 weight rows and two activation parts per stage) stays
// within the routed tiles' and two blocks fit per CU.
template <int MODE>
constexpr int kMixNsShared = MODE == 1 ? kPfNSG : kPfNS;
template <int MODE, int WT, bool W8>
__global__ __launch_bounds__(2 * kPfBM, 2) void pf_gemm_mix(Args A, PfLayout L, int nbt_s, int nblk_s, int nbt_r,
                                                             int nblk_r) {
  if ((int)blockIdx.x < nblk_s) {
    pf_gemm_body<MODE, kPfBM, kMixNsShared<MODE>, MOE_BF16, true>(A, L, nbt_s, nblk_s, 2, blockIdx.x);
  } else if constexpr (W8) {
    pf_gemm_w4a8_body<MODE, kPfNS>(A, L, nbt_r, nblk_r, (int)blockIdx.x - nblk_s);
  } else {
    pf_gemm_body<MODE, kPfBM, kPfNS, WT, true>(A, L, nbt_r, nblk_r, 1, (int)blockIdx.x - nblk_s);
  }
}

__global__ __launch_bounds__(256) void pf_select(Args A, const float* rpart, int ks) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= A.T) return;
  const float* src = A.logits_in ? A.logits_in : A.logits;
  if (rpart && !A.logits_in) {  // K-split router: logits = parts in split order + bias
    for (int e = lane; e < A.E; e += 64) {
      float l = rpart[(size_t)t * A.E + e];
      for (int p = 1; p < ks; ++p) l += rpart[((size_t)p * A.T + t) * A.E + e];
      if (A.rbias) l += A.rbias[(size_t)t * A.bias_stride + e];
      A.logits[(size_t)t * A.E + e] = l;  // select_token reads back only what this lane wrote
    }
  }
  int* ids = A.ids + (size_t)t * A.k;
  float* w = A.cw + (size_t)t * A.k;
  __shared__ unsigned s_hist[4][512];
  if (A.o_ids)  // routing outputs: listed by descending logit
    select_token(src + (size_t)t * A.E, A.E, A.k, lane, ids, w);
  else  // the forward pass only needs the set (radix select, fewer instructions)
    select_set(src + (size_t)t * A.E, A.E, A.k, lane, s_hist[threadIdx.x >> 6], ids, w);
  if (A.o_logits)
    for (int e = lane; e < A.E; e += 64) A.o_logits[(size_t)t * A.E + e] = src[(size_t)t * A.E + e];
  if (A.o_ids && lane < A.k) {  // each lane re-reads only what it wrote itself
    A.o_ids[(size_t)t * A.k + lane] = ids[lane];
    A.o_w[(size_t)t * A.k + lane] = w[lane];
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
    if (L.outf) {  // precise: fp32 slot rows
      const float4 a = *(const float4*)&L.outf[(size_t)row * A.H + c];
      const float4 b = *(const float4*)&L.outf[(size_t)row * A.H + c + 4];
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
      return;
    }
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

namespace {
// Operand-staging probe: the grouped GEMMs' load (16 bytes per lane from a buffer resource
// into LDS) with each instruction covering 64 * 16 / SEG rows of SEG contiguous bytes, rows
// 4 KiB apart in a region of mask + 1 bytes.  Every wave issues `iters` groups of six
// instructions and keeps six in flight; what lands is folded into a test that stores to sink
// only for a value no sane input produces.  Every offset stays inside the region: a row starts
// on a 4 KiB boundary below it and the segment ends within 2 KiB of that start.
template <int SEG>
__global__ __launch_bounds__(256) void stage_probe(const uint8_t* buf, uint32_t mask, int iters, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint4 s[2][4][6][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const i32x4_t rs = buf_rsrc(buf, (size_t)mask + 1);
  constexpr int LPR = SEG / 16, RPI = 64 / LPR;  // lanes per row, rows per instruction
  const uint32_t lr = (uint32_t)(lane / LPR), within = (uint32_t)(lane % LPR) * 16u;
  const uint32_t row0 = (uint32_t)(blockIdx.x * 4 + wave) * 37u;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const uint32_t g = (uint32_t)(it * 6 + j);
      const uint32_t seg0 = SEG >= 1024 ? 0u : (g * SEG) & 1023u;
      const uint32_t off = ((row0 + g * RPI + lr) * 4096u & mask & ~4095u) + seg0 + within;
      dma16(rs, off, lds_addr(&s[it & 1][wave][j][0]));
    }
    wait_vm<6>();
  }
  wait_vm<0>();
  __syncthreads();
  if (s[0][wave][0][lane].x == 0x9E3779B9u) sink[blockIdx.x & 63] = 1u;
}
}  // namespace

int launch_stage_probe(const void* buf, uint32_t mask, int seg, int iters, uint32_t* sink, hipStream_t st) {
  const void* f = nullptr;
  switch (seg) {
    case 16: f = (const void*)stage_probe<16>; break;
    case 32: f = (const void*)stage_probe<32>; break;
    case 64: f = (const void*)stage_probe<64>; break;
    case 128: f = (const void*)stage_probe<128>; break;
    case 256: f = (const void*)stage_probe<256>; break;
    case 512: f = (const void*)stage_probe<512>; break;
    case 1024: f = (const void*)stage_probe<1024>; break;
    default: return MOE_EINVAL;
  }
  const uint8_t* b = (const uint8_t*)buf;
  void* args[] = {&b, &mask, &iters, &sink};
  return launch(LaunchHook{}, "stage_probe", f, dim3(kStageProbeBlocks), dim3(256), args, 0, st) == hipSuccess
             ? MOE_OK
             : MOE_EHIP;
}

// Router logits + per-token selection for T > 16 with bf16 activations (also used by
// moe_route so that routing-only calls take the forward path's arithmetic).
int launch_pf_route(Args A, hipStream_t st, const LaunchHook& hook) {
  PfLayout L = pf_layout(A);
  if (!A.logits_in) {
    void* a1[] = {&A, &L.planes};
    if (launch(hook, "pf_router_split", (const void*)pf_split_router, dim3(256), dim3(256), a1, 0, st) != hipSuccess)
      return MOE_EHIP;
    int nbt = ((A.E + 63) / 64) * L.ks, nblocks = ((A.T + kPfBM - 1) / kPfBM) * nbt, part = 0;
    void* a2[] = {&A, &L, &nbt, &nblocks, &part};
    if (launch(hook, "pf_router", (const void*)pf_gemm<2, kPfBM, kPfNSG, MOE_BF16, false>, dim3(nblocks),
               dim3(2 * kPfBM), a2, 0, st) != hipSuccess)
      return MOE_EHIP;
  }
  const float* rp = A.logits_in ? nullptr : L.rpart;
  int ks = L.ks;
  void* a3[] = {&A, &rp, &ks};
  if (launch(hook, "pf_select", (const void*)pf_select, dim3((A.T + 3) / 4), dim3(256), a3, 0, st) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

namespace {
// Dynamic LDS of a pf_gemm instance for reduction length K: the operand ring plus, for MXFP4,
// the four waves' scale blocks (after the ring), or the bf16 output tile if that is larger.
template <int MODE, int NS, int WT, bool P>
size_t pf_lds(int K) {
  typedef PfCfg<MODE, kPfBM, NS, WT, P> C;
  if (!C::kDyn) return 0;
  const size_t sc = C::F4 ? (size_t)(C::I4 ? 2 : 1) * 4 * ((64 * (K / 32) + 1023) / 1024) * 1024 : 0;
  const size_t epi = (MODE == 1 && P) ? 0 : (size_t)kPfBM * ((MODE == 0 ? kPfBN / 2 : kPfBN) + 8) * 2;
  return std::max(C::ring_bytes + sc, epi);
}
// W4A8 LDS: the ring, the four waves' B scale blocks, the tile's A scale rows
size_t pf_w4a8_lds(int K) {
  const size_t ring = (size_t)kPfNS * (kPfBM * 64 + kPfBN * 32);
  return ring + (size_t)4 * ((64 * (K / 32) + 1023) / 1024) * 1024 + (size_t)kPfBM * mx8_scale_ld(K);
}
}  // namespace

size_t prefill_lds_bytes(int H, int I, int Is, int wdt, bool w4a8) {
  size_t gu = 0, dn = 0;
  if (w4a8 || wdt == MOE_MXFP4 || wdt == MOE_INT4G64) {  // one launch: shared (bf16 precise) + routed tiles
    gu = pf_lds<0, kMixNsShared<0>, MOE_BF16, true>(H);  // as the launches size it
    dn = pf_lds<1, kMixNsShared<1>, MOE_BF16, true>(Is);
    if (w4a8) {
      gu = std::max(gu, pf_w4a8_lds(H));
      dn = std::max(dn, pf_w4a8_lds(I));
    } else if (wdt == MOE_INT4G64) {
      gu = std::max(gu, pf_lds<0, kPfNS, MOE_INT4G64, true>(H));
      dn = std::max(dn, pf_lds<1, kPfNS, MOE_INT4G64, true>(I));
    } else {
      gu = std::max(gu, pf_lds<0, kPfNS, MOE_MXFP4, true>(H));
      dn = std::max(dn, pf_lds<1, kPfNS, MOE_MXFP4, true>(I));
    }
  }
  return std::max(gu, dn);  // bf16 experts: static LDS only (fixed by the tile, below the limit)
}

int launch_prefill(Args A, hipStream_t st, const LaunchHook& hook) {
  PfLayout L = pf_layout(A);
  int rc = launch_pf_route(A, st, hook);
  if (rc) return rc;
  rc = launch_permute_many(A.ids, A.T, A.k, A.E, A.Is > 0, L.bcnt, L.count, L.offset, L.rows, L.tiles,
                           L.ntiles, kPfBM, st, hook);
  if (rc) return rc;
  const int cap = prefill_tiles_cap(A.T, A.E, A.k);
  const int Imax = A.I > A.Is ? A.I : A.Is;
  const bool f4 = A.wdt == MOE_MXFP4, i4 = A.wdt == MOE_INT4G64, w4a8 = A.aq == MOE_QMXFP8;
  if (w4a8) {  // x -> MXFP8 for the routed gate/up GEMM
    void* aq[] = {&A, &L};
    if (launch(hook, "pf_quant_x", (const void*)pf_quant_x, dim3((unsigned)(((size_t)A.T * (A.H / 32) + 255) / 256)),
               dim3(256), aq, 0, st) != hipSuccess)
      return MOE_EHIP;
  }
  // MXFP4 experts: the routed groups' tiles run the MXFP4 kernel, the shared expert's tiles the
  // bf16 kernel, both in the precise variant (activation hi + lo parts, fp32 slot rows).
  // INT4G64 experts: the routed tiles run the int4 kernel (weights rebuilt in bf16 on the way
  // into the MFMA), the shared tiles the bf16 kernel, both precise as for MXFP4.  The weights'
  // own bf16 rounding stays (the page's reconstruction); the activations and slot rows keep
  // about 16 significant bits, so those roundings do not add to it.  W4A8: the routed tiles run
  // the block-scaled fp8 x fp4 kernel, the shared tiles the bf16 precise kernel.  With 4-bit
  // experts both kinds of tile go into one launch (pf_gemm_mix: shared tiles first).
  const int shtiles = A.Is > 0 ? (A.T + kPfBM - 1) / kPfBM : 0;
  auto run = [&](const char* name, const void* f, int nblocks, int nbt, int part, size_t lds) -> int {
    PfLayout Lc = L;
    void* args[] = {&A, &Lc, &nbt, &nblocks, &part};
    return launch(hook, name, f, dim3(nblocks), dim3(2 * kPfBM), args, lds, st) == hipSuccess ? MOE_OK : MOE_EHIP;
  };
  auto run_mix = [&](const char* name, const void* f, int nbt, size_t lds) -> int {
    PfLayout Lc = L;
    int nbs = nbt, nblk_s = shtiles * nbt, nbr = nbt, nblk_r = cap * nbt;
    void* args[] = {&A, &Lc, &nbs, &nblk_s, &nbr, &nblk_r};
    return launch(hook, name, f, dim3(nblk_s + nblk_r), dim3(2 * kPfBM), args, lds, st) == hipSuccess ? MOE_OK
                                                                                                     : MOE_EHIP;
  };
  {
    const int nbt = (Imax + kPfBN / 2 - 1) / (kPfBN / 2);
    const size_t lsh = pf_lds<0, kMixNsShared<0>, MOE_BF16, true>(A.H);
    if (w4a8)
      rc = run_mix("pf_gateup", (const void*)pf_gemm_mix<0, MOE_MXFP4, true>, nbt, std::max(pf_w4a8_lds(A.H), lsh));
    else if (i4)
      rc = run_mix("pf_gateup", (const void*)pf_gemm_mix<0, MOE_INT4G64, false>, nbt,
                   std::max(pf_lds<0, kPfNS, MOE_INT4G64, true>(A.H), lsh));
    else if (f4)
      rc = run_mix("pf_gateup", (const void*)pf_gemm_mix<0, MOE_MXFP4, false>, nbt,
                   std::max(pf_lds<0, kPfNS, MOE_MXFP4, true>(A.H), lsh));
    else
      rc = run("pf_gateup", (const void*)pf_gemm<0, kPfBM, kPfNS, MOE_BF16, false>, cap * nbt, nbt, 0, 0);
    if (rc) return rc;
  }
  {
    const int nbt = (A.H + kPfBN - 1) / kPfBN;
    const size_t lsh = pf_lds<1, kMixNsShared<1>, MOE_BF16, true>(A.Is);
    if (w4a8)
      rc = run_mix("pf_down", (const void*)pf_gemm_mix<1, MOE_MXFP4, true>, nbt, std::max(pf_w4a8_lds(A.I), lsh));
    else if (i4)
      rc = run_mix("pf_down", (const void*)pf_gemm_mix<1, MOE_INT4G64, false>, nbt,
                   std::max(pf_lds<1, kPfNS, MOE_INT4G64, true>(A.I), lsh));
    else if (f4)
      rc = run_mix("pf_down", (const void*)pf_gemm_mix<1, MOE_MXFP4, false>, nbt,
                   std::max(pf_lds<1, kPfNS, MOE_MXFP4, true>(A.I), lsh));
    else
      rc = run("pf_down", (const void*)pf_gemm<1, kPfBM, kPfNSG, MOE_BF16, false>, cap * nbt, nbt, 0, 0);
    if (rc) return rc;
  }
  void* ac[] = {&A, &L};
  if (launch(hook, "pf_combine", (const void*)pf_combine, dim3((unsigned)(((size_t)A.T * (A.H / 8) + 255) / 256)),
             dim3(256), ac, 0, st) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

}  // namespace moe
