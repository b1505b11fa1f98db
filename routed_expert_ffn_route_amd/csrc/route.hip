// Routing for any number of tokens: router logits, per-token selection, and the
// token-to-expert permutation ("Optimizing on-device inference for Apple Silicon", section
// "Keep expert routing on the GPU": a histogram counts the assignments per expert, a prefix
// scan turns the counts into start offsets, a scatter places the rows into their expert
// groups, and a block map lists the fixed-size row blocks a grouped GEMM walks).
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace moe {


// ------------------------------------------------------------------------------------------
// Router logits for many tokens: [T][H] x [E][H]^T on fp32 VALU FMAs, 64x64 output tiles,
// K staged through LDS in steps of 32.  (x bf16 or fp32, router fp32.)
// ------------------------------------------------------------------------------------------
template <int XT>
__global__ __launch_bounds__(256) void router_tiled(Args A) {
  constexpr int BT = 64, BE = 64, BK = 32;
  __shared__ float sx[BK][BT + 1];
  __shared__ float sw[BK][BE + 1];
  const int t0 = blockIdx.x * BT, e0 = blockIdx.y * BE;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;  // 16 x 16 threads, 4 x 4 each
  float acc[4][4] = {};
  for (int k0 = 0; k0 < A.H; k0 += BK) {
    // 64 rows x 32 k of x and of W: 2048 elements each, 8 per thread
    for (int i = threadIdx.x; i < BT * BK; i += 256) {
      const int r = i / BK, kk = i % BK;
      const int t = t0 + r, e = e0 + r;
      float xv = 0.f, wv = 0.f;
      if (t < A.T) {
        if constexpr (XT == MOE_F32)
          xv = ((const float*)A.x)[(size_t)t * A.H + k0 + kk];
        else
          xv = bf16_to_f32(((const uint16_t*)A.x)[(size_t)t * A.H + k0 + kk]);
      }
      if (e < A.E) wv = A.rw[(size_t)e * A.H + k0 + kk];
      sx[kk][r] = xv;
      sw[kk][r] = wv;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < BK; ++kk) {
      float xr[4], wr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xr[i] = sx[kk][ty * 4 + i];
        wr[i] = sw[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xr[i], wr[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= A.T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e >= A.E) continue;
      float l = acc[i][j];
      if (A.rbias) l += A.rbias[(size_t)t * A.bias_stride + e];
      A.logits[(size_t)t * A.E + e] = l;
      if (A.o_logits) A.o_logits[(size_t)t * A.E + e] = l;
    }
  }
}

// One wave per token: selection from ws logits (or logits_in), written to the workspace
// ids/weights and, when given, to the moe_route outputs.
__global__ __launch_bounds__(256) void select_tokens(Args A) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= A.T) return;
  const float* src = A.logits_in ? A.logits_in : A.logits;
  int* ids = A.ids + (size_t)t * A.k;
  float* w = A.cw + (size_t)t * A.k;
  select_token(src + (size_t)t * A.E, A.E, A.k, lane, ids, w);
  if (A.logits_in && A.o_logits) {
    for (int e = lane; e < A.E; e += kWave)
      A.o_logits[(size_t)t * A.E + e] = A.logits_in[(size_t)t * A.E + e];
  }
  if (A.o_ids && lane < A.k) {  // each lane re-reads only what it wrote itself
    A.o_ids[(size_t)t * A.k + lane] = ids[lane];
    A.o_w[(size_t)t * A.k + lane] = w[lane];
  }
}

// Exclusive scan of n (<= 1088) ints in LDS by one wave; returns the total in lane 0..63.
__device__ int wave_scan_lds(int* v, int n, int lane) {
  const int per = (n + kWave - 1) / kWave;
  const int b = lane * per, en = min(b + per, n);
  int local = 0;
  for (int i = b; i < en; ++i) local += v[i];
  int incl = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  int run = incl - local;
  for (int i = b; i < en; ++i) {
    int c = v[i];
    v[i] = run;
    run += c;
  }
  return __shfl(incl, kWave - 1, kWave);
}

// Histogram -> exclusive scan -> scatter, in one 1024-thread block.  Groups are the E
// experts plus, when with_shared, a final group E holding every token (the shared expert)
// as rows S + t.  Writes counts [G], offsets [G+1], rows [S (+T)], and when tiles != null the
// block map: for each group, ceil(count / bm) tiles {group, first row, rows, 0} (16 bytes
// each), their number in tiles_n.  The order inside a group is whatever the LDS atomics produce.
__global__ __launch_bounds__(1024) void permute(const int* ids, int T, int k, int E, bool with_shared,
                                                int* counts, int* offsets, int* rows, int* tiles,
                                                int* tiles_n, int bm) {
  __shared__ int s_cnt[MOE_MAX_E + 2];
  __shared__ int s_off[MOE_MAX_E + 2];
  __shared__ int s_til[MOE_MAX_E + 2];
  __shared__ int s_total, s_ntiles;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int S = T * k, G = E + (with_shared ? 1 : 0);
  for (int g = tid; g < G; g += 1024) s_cnt[g] = 0;
  __syncthreads();
  for (int s = tid; s < S; s += 1024) atomicAdd(&s_cnt[ids[s]], 1);
  __syncthreads();
  if (tid == 0 && with_shared) s_cnt[E] = T;
  __syncthreads();
  for (int g = tid; g < G; g += 1024) {
    s_off[g] = s_cnt[g];
    s_til[g] = (s_cnt[g] + bm - 1) / bm;
  }
  __syncthreads();
  if (tid < kWave) {
    int tot = wave_scan_lds(s_off, G, lane);
    if (lane == 0) s_total = tot;
  } else if (tid < 2 * kWave && tiles) {
    int tot = wave_scan_lds(s_til, G, lane);
    if (lane == 0) s_ntiles = tot;
  }
  __syncthreads();
  for (int g = tid; g < G; g += 1024) {
    if (counts) counts[g] = s_cnt[g];
    if (offsets) offsets[g] = s_off[g];
  }
  if (tid == 0) {
    if (offsets) offsets[G] = s_total;
    if (tiles_n) *tiles_n = tiles ? s_ntiles : 0;
  }
  if (tiles) {
    for (int g = tid; g < G; g += 1024) {
      const int nt = (s_cnt[g] + bm - 1) / bm;
      for (int i = 0; i < nt; ++i)
        ((int4*)tiles)[s_til[g] + i] = make_int4(g, s_off[g] + i * bm, min(bm, s_cnt[g] - i * bm), 0);
    }
  }
  __syncthreads();
  // s_cnt becomes the scatter cursor
  for (int g = tid; g < G; g += 1024) s_cnt[g] = s_off[g];
  __syncthreads();
  if (rows) {
    for (int s = tid; s < S; s += 1024) {
      const int pos = atomicAdd(&s_cnt[ids[s]], 1);
      rows[pos] = s;
    }
    if (with_shared)
      for (int t = tid; t < T; t += 1024) rows[s_off[E] + t] = S + t;
  }
}

// The same permutation over many blocks, for the forward pass's large T: the assignments are
// cut into chunks of kPermChunk; (1) each block counts its chunk's experts in LDS and writes
// its counts per expert, (2) one block adds them up per expert, turns each block's count into
// its start inside the expert's group (a prefix over blocks), scans the group sizes into
// offsets and writes the block map, (3) each block scatters its chunk from those starts with
// LDS cursors.  bcnt: [nblocks][E] ints of workspace.
constexpr int kPermChunk = 512;
__global__ __launch_bounds__(256) void permute_count(const int* ids, int S, int E, int* bcnt) {
  __shared__ int s_h[MOE_MAX_E];
  for (int g = threadIdx.x; g < E; g += blockDim.x) s_h[g] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * kPermChunk, s1 = min(S, s0 + kPermChunk);
  for (int s = s0 + threadIdx.x; s < s1; s += blockDim.x) atomicAdd(&s_h[ids[s]], 1);
  __syncthreads();
  for (int g = threadIdx.x; g < E; g += blockDim.x) bcnt[(size_t)blockIdx.x * E + g] = s_h[g];
}

__global__ __launch_bounds__(1024) void permute_plan(int* bcnt, int nb, int T, int k, int E, bool with_shared,
                                                     int* counts, int* offsets, int* rows, int* tiles,
                                                     int* tiles_n, int bm) {
  __shared__ int s_cnt[MOE_MAX_E + 2];
  __shared__ int s_off[MOE_MAX_E + 2];
  __shared__ int s_til[MOE_MAX_E + 2];
  __shared__ int s_total, s_ntiles;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int S = T * k, G = E + (with_shared ? 1 : 0);
  constexpr int kB = 16;  // counts read per pass before any is overwritten (one round trip)
  for (int g = tid; g < E; g += blockDim.x) {  // per expert: prefix over the blocks
    int run = 0;
    for (int b0 = 0; b0 < nb; b0 += kB) {
      int c[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) c[j] = b0 + j < nb ? bcnt[(size_t)(b0 + j) * E + g] : 0;
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (b0 + j < nb) bcnt[(size_t)(b0 + j) * E + g] = run;
        run += c[j];
      }
    }
    s_cnt[g] = run;
  }
  if (tid == 0 && with_shared) s_cnt[E] = T;
  __syncthreads();
  for (int g = tid; g < G; g += blockDim.x) {
    s_off[g] = s_cnt[g];
    s_til[g] = (s_cnt[g] + bm - 1) / bm;
  }
  __syncthreads();
  if (tid < kWave) {
    const int tot = wave_scan_lds(s_off, G, lane);
    if (lane == 0) s_total = tot;
  } else if (tid < 2 * kWave) {
    const int tot = wave_scan_lds(s_til, G, lane);
    if (lane == 0) s_ntiles = tot;
  }
  __syncthreads();
  for (int g = tid; g < G; g += blockDim.x) {
    counts[g] = s_cnt[g];
    offsets[g] = s_off[g];
    const int nt = (s_cnt[g] + bm - 1) / bm;
    for (int i = 0; i < nt; ++i)
      ((int4*)tiles)[s_til[g] + i] = make_int4(g, s_off[g] + i * bm, min(bm, s_cnt[g] - i * bm), 0);
  }
  if (tid == 0) {
    offsets[G] = s_total;
    *tiles_n = s_ntiles;
  }
  if (with_shared)
    for (int t = tid; t < T; t += blockDim.x) rows[s_off[E] + t] = S + t;
}

__global__ __launch_bounds__(256) void permute_scatter(const int* ids, int S, int E, const int* bcnt,
                                                       const int* offsets, int* rows) {
  __shared__ int s_cur[MOE_MAX_E];
  for (int g = threadIdx.x; g < E; g += blockDim.x) s_cur[g] = offsets[g] + bcnt[(size_t)blockIdx.x * E + g];
  __syncthreads();
  const int s0 = blockIdx.x * kPermChunk, s1 = min(S, s0 + kPermChunk);
  for (int s = s0 + threadIdx.x; s < s1; s += blockDim.x) rows[atomicAdd(&s_cur[ids[s]], 1)] = s;
}

int permute_blocks(int T, int k) { return (T * k + kPermChunk - 1) / kPermChunk; }

int launch_permute_many(const int* ids, int T, int k, int E, bool with_shared, int* bcnt, int* counts,
                        int* offsets, int* rows, int* tiles, int* tiles_n, int bm, hipStream_t st) {
  const int S = T * k, nb = permute_blocks(T, k);
  permute_count<<<nb, 256, 0, st>>>(ids, S, E, bcnt);
  permute_plan<<<1, 1024, 0, st>>>(bcnt, nb, T, k, E, with_shared, counts, offsets, rows, tiles, tiles_n, bm);
  permute_scatter<<<nb, 256, 0, st>>>(ids, S, E, bcnt, offsets, rows);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int launch_route_any(Args A, hipStream_t st, bool decode_sized, const LaunchHook& hook) {
  hipError_t err;
  if (!decode_sized && A.act == MOE_BF16) {  // the prefill path's router and selection
    const int rc = launch_pf_route(A, st, hook);
    if (rc) return rc;
  } else {
    if (!A.logits_in) {
      if (decode_sized) {  // the decode path's router kernel (no shared-expert blocks)
        const int rc = launch_decode(A, st, /*route_only=*/true, hook);
        if (rc) return rc;
      } else {
        dim3 grid((A.T + 63) / 64, (A.E + 63) / 64);
        hook.pre("route_logits", st);
        router_tiled<MOE_F32><<<grid, 256, 0, st>>>(A);
        hook.post(st);
        if ((err = hipGetLastError()) != hipSuccess) return MOE_EHIP;
      }
    }
    hook.pre("route_select", st);
    select_tokens<<<(A.T + 3) / 4, 256, 0, st>>>(A);
    hook.post(st);
    if ((err = hipGetLastError()) != hipSuccess) return MOE_EHIP;
  }
  if (A.o_count || A.o_offset || A.o_sorted) {
    hook.pre("route_permute", st);
    permute<<<1, 1024, 0, st>>>(A.ids, A.T, A.k, A.E, false, A.o_count, A.o_offset, A.o_sorted,
                                nullptr, nullptr, 1);
    hook.post(st);
    if ((err = hipGetLastError()) != hipSuccess) return MOE_EHIP;
  }
  return MOE_OK;
}

}  // namespace moe
