// Routing for any number of tokens: router logits, per-token selection, and the
// token-to-expert permutation ("Optimizing on-device inference for Apple Silicon", section
// "Keep expert routing on the GPU": a histogram counts the assignments per expert, a prefix
// scan turns the counts into start offsets, a scatter places the rows into their expert
// groups, and a block map lists the fixed-size row blocks a grouped GEMM walks).
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace moe {


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

// Stable placement of the assignments [s0, s1) (at most kPermChunk of them) by a block of
// kPermThreads threads: slot s goes to cursor[e] + the number of earlier slots of the range
// routed to the same expert e, so each expert group lists its slots in ascending order (the
// stable counting sort of the page's histogram / scan / scatter, "Optimizing on-device
// inference for Apple Silicon", section "Keep expert routing on the GPU").  Wave w takes
// slots s0 + 128 w ... in two passes of 64 lanes; the lanes of a pass that share an expert
// are found with one ballot per bit of the expert id, so no LDS atomic decides an order.
// cursor[E] (LDS) advances by the range's count of each expert.  s_wh: LDS [4][E] ints, zero
// on entry and on exit.
constexpr int kPermChunk = 512;
constexpr int kPermThreads = 256;

__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    m &= bit ? ones : ~ones;
  }
  return valid ? m : 0ull;
}

__device__ void stable_place(const int* ids, int s0, int s1, int E, int* cursor, int* s_wh, int* rows) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt = (1ull << lane) - 1ull;
  int e[2], rank[2], cnt[2];
  bool ok[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {  // counts per (wave, expert): one writer per group of lanes
    const int s = s0 + 128 * w + 64 * p + lane;
    ok[p] = s < s1;
    e[p] = ok[p] ? ids[s] : 0;
    const uint64_t m = same_expert_lanes(e[p], ok[p], nbits);
    rank[p] = __popcll(m & lt);
    cnt[p] = __popcll(m);
    if (ok[p] && rank[p] == 0) s_wh[w * E + e[p]] += cnt[p];
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int g = threadIdx.x; g < E; g += blockDim.x) {  // start of each wave's run of expert g
    int run = cursor[g];
#pragma unroll
    for (int ww = 0; ww < kPermThreads / kWave; ++ww) {
      const int c = s_wh[ww * E + g];
      s_wh[ww * E + g] = run;
      run += c;
    }
    cursor[g] = run;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int s = s0 + 128 * w + 64 * p + lane;
    const int start = ok[p] ? s_wh[w * E + e[p]] : 0;
    __builtin_amdgcn_wave_barrier();  // every lane has read its start before the leader moves it
    if (ok[p]) {
      rows[start + rank[p]] = s;
      if (rank[p] == 0) s_wh[w * E + e[p]] = start + cnt[p];
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int i = threadIdx.x; i < (kPermThreads / kWave) * E; i += blockDim.x) s_wh[i] = 0;
  __syncthreads();
}

// Histogram -> exclusive scan -> stable scatter in one block (the routing outputs of
// moe_route): counts [E], offsets [E+1], sorted slots [S] (nullable each).
__global__ __launch_bounds__(kPermThreads) void permute(const int* ids, int T, int k, int E, int* counts,
                                                       int* offsets, int* rows) {
  __shared__ int s_cnt[MOE_MAX_E + 1];
  __shared__ int s_off[MOE_MAX_E + 1];
  __shared__ int s_wh[(kPermThreads / kWave) * MOE_MAX_E];
  __shared__ int s_total;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int S = T * k;
  for (int g = tid; g < E; g += blockDim.x) s_cnt[g] = 0;
  for (int i = tid; i < (kPermThreads / kWave) * E; i += blockDim.x) s_wh[i] = 0;
  __syncthreads();
  for (int s = tid; s < S; s += blockDim.x) atomicAdd(&s_cnt[ids[s]], 1);  // counts: order-free
  __syncthreads();
  for (int g = tid; g < E; g += blockDim.x) s_off[g] = s_cnt[g];
  __syncthreads();
  if (tid < kWave) {
    const int tot = wave_scan_lds(s_off, E, lane);
    if (lane == 0) s_total = tot;
  }
  __syncthreads();
  for (int g = tid; g < E; g += blockDim.x) {
    if (counts) counts[g] = s_cnt[g];
    if (offsets) offsets[g] = s_off[g];
  }
  if (tid == 0 && offsets) offsets[E] = s_total;
  if (!rows) return;  // uniform
  // s_cnt becomes the scatter cursor
  for (int g = tid; g < E; g += blockDim.x) s_cnt[g] = s_off[g];
  __syncthreads();
  for (int s0 = 0; s0 < S; s0 += kPermChunk) stable_place(ids, s0, min(S, s0 + kPermChunk), E, s_cnt, s_wh, rows);
}

// The same permutation over many blocks, for the forward pass's large T: the assignments are
// cut into chunks of kPermChunk; (1) each block counts its chunk's experts in LDS and writes
// its counts per expert, (2) one block adds them up per expert, turns each block's count into
// its start inside the expert's group (a prefix over blocks), scans the group sizes into
// offsets and writes the block map, (3) each block places its chunk stably from those starts.
// bcnt: [nblocks][E] ints of workspace.
__global__ __launch_bounds__(kPermThreads) void permute_count(const int* ids, int S, int E, int* bcnt) {
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

__global__ __launch_bounds__(kPermThreads) void permute_scatter(const int* ids, int S, int E, const int* bcnt,
                                                                 const int* offsets, int* rows) {
  __shared__ int s_cur[MOE_MAX_E];
  __shared__ int s_wh[(kPermThreads / kWave) * MOE_MAX_E];
  for (int g = threadIdx.x; g < E; g += blockDim.x) s_cur[g] = offsets[g] + bcnt[(size_t)blockIdx.x * E + g];
  for (int i = threadIdx.x; i < (kPermThreads / kWave) * E; i += blockDim.x) s_wh[i] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * kPermChunk;
  stable_place(ids, s0, min(S, s0 + kPermChunk), E, s_cur, s_wh, rows);
}

int permute_blocks(int T, int k) { return (T * k + kPermChunk - 1) / kPermChunk; }

int launch_permute_many(const int* ids, int T, int k, int E, bool with_shared, int* bcnt, int* counts,
                        int* offsets, int* rows, int* tiles, int* tiles_n, int bm, hipStream_t st,
                        const LaunchHook& hook) {
  int S = T * k, nb = permute_blocks(T, k);
  void* a1[] = {&ids, &S, &E, &bcnt};
  if (launch(hook, "pf_permute_count", (const void*)permute_count, dim3(nb), dim3(kPermThreads), a1, 0, st) !=
      hipSuccess)
    return MOE_EHIP;
  void* a2[] = {&bcnt, &nb, &T, &k, &E, &with_shared, &counts, &offsets, &rows, &tiles, &tiles_n, &bm};
  if (launch(hook, "pf_permute_plan", (const void*)permute_plan, dim3(1), dim3(1024), a2, 0, st) != hipSuccess)
    return MOE_EHIP;
  void* a3[] = {&ids, &S, &E, &bcnt, &offsets, &rows};
  if (launch(hook, "pf_permute_scatter", (const void*)permute_scatter, dim3(nb), dim3(kPermThreads), a3, 0, st) !=
      hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

int launch_route_any(Args A, hipStream_t st, bool decode_sized, const LaunchHook& hook) {
  if (!decode_sized) {  // the prefill path's router and selection (bf16 activations)
    const int rc = launch_pf_route(A, st, hook);
    if (rc) return rc;
  } else {
    if (!A.logits_in) {  // the decode path's router kernel (no shared-expert blocks)
      const int rc = launch_decode(A, st, /*route_only=*/true, hook);
      if (rc) return rc;
    }
    void* as[] = {&A};
    if (launch(hook, "route_select", (const void*)select_tokens, dim3((A.T + 3) / 4), dim3(256), as, 0, st) !=
        hipSuccess)
      return MOE_EHIP;
  }
  if (A.o_count || A.o_offset || A.o_sorted) {
    void* ap[] = {&A.ids, &A.T, &A.k, &A.E, &A.o_count, &A.o_offset, &A.o_sorted};
    if (launch(hook, "route_permute", (const void*)permute, dim3(1), dim3(kPermThreads), ap, 0, st) != hipSuccess)
      return MOE_EHIP;
  }
  return MOE_OK;
}

}  // namespace moe
