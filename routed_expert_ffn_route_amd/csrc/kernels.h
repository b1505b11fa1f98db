// Host-side launchers of the libmoe kernels (one per path) and the per-launch timing hook.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace moe {

// Called around every kernel launch; the API layer records HIP events here when kernel
// timing is on (moe_timing_begin), and does nothing otherwise.
struct LaunchHook {
  void (*pre_fn)(const char* name, hipStream_t st) = nullptr;
  void (*post_fn)(hipStream_t st) = nullptr;
  void pre(const char* name, hipStream_t st) const {
    if (pre_fn) pre_fn(name, st);
  }
  void post(hipStream_t st) const {
    if (post_fn) post_fn(st);
  }
};

// Decode path (T <= kDecodeMaxT): router, selection/plan + shared gate/up, routed gate/up,
// down + combine (shared and routed).  route_only stops after the router.
int launch_decode(Args A, hipStream_t st, bool route_only, const LaunchHook& hook);

// Routing for any T: router logits (or logits_in), per-token selection, and the
// histogram / scan / scatter plan written to the moe_route outputs.
int launch_route_any(Args A, hipStream_t st, bool decode_sized, const LaunchHook& hook);

// Token-to-expert permutation over many blocks (count, plan, scatter) for the forward pass;
// bcnt: workspace of permute_blocks(T, k) * E ints.
int permute_blocks(int T, int k);
int launch_permute_many(const int* ids, int T, int k, int E, bool with_shared, int* bcnt, int* counts,
                        int* offsets, int* rows, int* tiles, int* tiles_n, int bm, hipStream_t st);

// Router (MFMA, bf16 activations) + selection for T > kDecodeMaxT.
int launch_pf_route(Args A, hipStream_t st, const LaunchHook& hook);

// Prefill path (T > kDecodeMaxT): grouped GEMMs on MFMA.
int launch_prefill(Args A, hipStream_t st, const LaunchHook& hook);

// Workspace bytes needed by the prefill path's sections; precise: MXFP4 experts (activations
// as bf16 hi + lo parts, fp32 slot rows).
size_t prefill_ws_bytes(int T, int H, int E, int k, int I, int Is, bool precise);
int prefill_tiles_cap(int T, int E, int k);
constexpr int kPfTileRows = 128;  // rows per grouped-GEMM tile (the block map's unit)

}  // namespace moe
