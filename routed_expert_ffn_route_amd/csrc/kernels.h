// Host-side launchers of the libmoe kernels (one per path) and the per-launch timing hook.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "common.h"

namespace moe {

// Kernel timing: while moe_timing_begin's events last, `events` hands each launch a pair of
// HIP events and the kernel is launched with hipExtLaunchKernel, which ties them to the
// kernel's own start and end (no marker packets between kernels, so the durations are the
// kernels' alone).  Otherwise events is null and launches are plain.
struct LaunchHook {
  bool (*events)(const char* name, hipEvent_t* start, hipEvent_t* stop) = nullptr;
};

// Every kernel of the library is launched here (`name` labels it in the timing records).
// Dynamic LDS above 64 KiB is enabled for the kernel first.
inline hipError_t launch(const LaunchHook& hook, const char* name, const void* f, dim3 grid, dim3 block,
                         void** args, size_t lds, hipStream_t st) {
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hook.events && hook.events(name, &e0, &e1))
    return hipExtLaunchKernel(f, grid, block, args, lds, st, e0, e1, 0);
  return hipLaunchKernel(f, grid, block, args, lds, st);
}

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
                        int* offsets, int* rows, int* tiles, int* tiles_n, int bm, hipStream_t st,
                        const LaunchHook& hook);

// Router (MFMA, bf16 activations) + selection for T > kDecodeMaxT.
int launch_pf_route(Args A, hipStream_t st, const LaunchHook& hook);

// Prefill path (T > kDecodeMaxT): grouped GEMMs on MFMA.
int launch_prefill(Args A, hipStream_t st, const LaunchHook& hook);

// Operand-staging probe (measurement): kStageProbeBlocks blocks of four waves, each wave
// moving iters * 6 KiB from a region of mask + 1 bytes (a power of two >= 8 KiB) into LDS in
// rows of seg bytes (16 .. 1024, a power of two).
constexpr int kStageProbeBlocks = 512;
int launch_stage_probe(const void* buf, uint32_t mask, int seg, int iters, uint32_t* sink, hipStream_t st);

// Workspace bytes needed by the prefill path's sections; precise: MXFP4 or INT4G64 experts
// (activations as bf16 hi + lo parts, fp32 slot rows).
size_t prefill_ws_bytes(int T, int H, int E, int k, int I, int Is, bool precise, bool w4a8);
// Largest dynamic LDS of the prefill GEMM launches for these sizes (4-bit experts stage one
// scale block per wave and tile, which grows with the reduction length); shapes whose launches
// would not fit kCuLdsBytes are rejected before anything is launched.
size_t prefill_lds_bytes(int H, int I, int Is, int wdt, bool w4a8);
constexpr size_t kCuLdsBytes = 160 * 1024;  // LDS per CU (gfx950)
int prefill_tiles_cap(int T, int E, int k);
constexpr int kPfTileRows = 128;  // rows per grouped-GEMM tile (the block map's unit)

}  // namespace moe
