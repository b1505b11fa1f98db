// libmoe C ABI: argument validation, workspace layout, path selection and the kernel-timing
// hook.  Everything here runs on the host; the kernels live in decode.hip, route.hip and
// prefill.hip.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const moe_shape_t* s) {
  if (!s) return MOE_EINVAL;
  if (s->T < 1 || s->H < 1 || s->E < 1 || s->k < 1 || s->I < 1 || s->I_shared < 0) return MOE_EINVAL;
  if (s->k > s->E) return MOE_EINVAL;
  if (s->E > MOE_MAX_E || s->k > MOE_MAX_K || s->H > MOE_MAX_H || s->I > MOE_MAX_I ||
      s->I_shared > MOE_MAX_I)
    return MOE_EUNSUPPORTED;
  if (s->H % 32 || s->I % 32 || s->I_shared % 32) return MOE_EUNSUPPORTED;
  const bool f32 = s->act_dtype == MOE_F32 && s->expert_dtype == MOE_F32 && s->shared_dtype == MOE_F32;
  const bool b16 = s->act_dtype == MOE_BF16 &&
                   (s->expert_dtype == MOE_BF16 || s->expert_dtype == MOE_MXFP4 ||
                    s->expert_dtype == MOE_INT4G64) &&
                   s->shared_dtype == MOE_BF16;
  if (!f32 && !b16) return MOE_EUNSUPPORTED;
  if (s->expert_dtype == MOE_INT4G64 && (s->H % 64 || s->I % 64)) return MOE_EUNSUPPORTED;
  if (s->out_dtype != MOE_F32 && s->out_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (s->act_quant != MOE_QNONE && s->act_quant != MOE_QMXFP8) return MOE_EUNSUPPORTED;
  if (s->act_quant == MOE_QMXFP8 && (s->expert_dtype != MOE_MXFP4 || s->T <= kDecodeMaxT)) return MOE_EUNSUPPORTED;
  if (s->T > kDecodeMaxT) {  // prefill path
    if (s->act_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
    // MXFP4 / INT4G64 experts: the scale (and bias) rows of a weight tile are staged in LDS
    if ((s->expert_dtype == MOE_MXFP4 || s->expert_dtype == MOE_INT4G64) && (s->H > 8192 || s->I > 8192))
      return MOE_EUNSUPPORTED;
    if ((size_t)s->T * s->H * 2 >= ((size_t)1 << 31)) return MOE_EUNSUPPORTED;  // 32-bit row offsets
    // the GEMM launches' LDS (4-bit experts: the ring plus one scale block per wave), with the
    // down kernels' 2 KiB of static LDS (a tile's slots and routing weights)
    if (prefill_lds_bytes(s->H, s->I, s->I_shared, s->expert_dtype, s->act_quant == MOE_QMXFP8) + 2048 > kCuLdsBytes)
      return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

struct Layout {
  size_t logits, ids, cw, plan, a_sh, a, pf, total;
};

Layout layout(const moe_shape_t* s) {
  Layout L{};
  const size_t T = s->T, E = s->E, k = s->k, S = T * k;
  const size_t D = S < E ? S : E;
  size_t off = 0;
  L.logits = off;
  off += up(T * E * 4);
  L.ids = off;
  off += up(S * 4);
  L.cw = off;
  off += up(S * 4);
  if (s->T <= kDecodeMaxT) {
    L.plan = off;
    off += up(DecodePlan::bytes((int)D, (int)T));
    L.a_sh = off;
    off += up(T * (size_t)s->I_shared * 4);
    L.a = off;
    off += up(S * (size_t)s->I * 4);
  } else {
    L.pf = off;
    off += up(prefill_ws_bytes(s->T, s->H, s->E, s->k, s->I, s->I_shared,
                               s->expert_dtype == MOE_MXFP4 || s->expert_dtype == MOE_INT4G64,
                               s->act_quant == MOE_QMXFP8));
  }
  L.total = off;
  return L;
}

Args make_args(const moe_shape_t* s, const void* x, const moe_weights_t* w, void* ws) {
  Args A;
  memset(&A, 0, sizeof A);
  A.T = s->T;
  A.H = s->H;
  A.E = s->E;
  A.k = s->k;
  A.I = s->I;
  A.Is = s->I_shared;
  A.act = s->act_dtype;
  A.wdt = s->expert_dtype;
  A.sdt = s->shared_dtype;
  A.odt = s->out_dtype;
  A.aq = s->act_quant;
  A.x = x;
  A.rw = w->router_w;
  A.rbias = w->router_bias;
  A.bias_stride = w->bias_t_stride;
  A.gate = w->gate;
  A.up = w->up;
  A.down = w->down;
  A.gs = w->gate_s;
  A.us = w->up_s;
  A.ds = w->down_s;
  A.sgate = w->sh_gate;
  A.sup = w->sh_up;
  A.sdown = w->sh_down;
  A.gb = w->gate_b;
  A.ub = w->up_b;
  A.db = w->down_b;
  const Layout L = layout(s);
  uint8_t* b = (uint8_t*)ws;
  A.logits = (float*)(b + L.logits);
  A.ids = (int*)(b + L.ids);
  A.cw = (float*)(b + L.cw);
  if (s->T <= kDecodeMaxT) {
    A.plan = (int*)(b + L.plan);
    A.a_sh = (float*)(b + L.a_sh);
    A.a = (float*)(b + L.a);
  } else {
    A.plan = (int*)(b + L.pf);  // prefill sections are carved by the prefill launcher
  }
  return A;
}

int check_weights(const moe_shape_t* s, const moe_weights_t* w, bool experts) {
  if (!w || !w->router_w) return MOE_EINVAL;
  if (w->router_bias && !(w->bias_t_stride == 0 || w->bias_t_stride == s->E)) return MOE_EINVAL;
  if (!aligned16(w->router_w)) return MOE_EALIGN;
  if (!experts) return MOE_OK;
  if (!w->gate || !w->up || !w->down) return MOE_EINVAL;
  if ((s->expert_dtype == MOE_MXFP4 || s->expert_dtype == MOE_INT4G64) && (!w->gate_s || !w->up_s || !w->down_s))
    return MOE_EINVAL;
  if (s->expert_dtype == MOE_INT4G64 && (!w->gate_b || !w->up_b || !w->down_b)) return MOE_EINVAL;
  if (s->I_shared > 0 && (!w->sh_gate || !w->sh_up || !w->sh_down)) return MOE_EINVAL;
  const void* ptrs[] = {w->gate, w->up, w->down, w->sh_gate, w->sh_up, w->sh_down};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_EALIGN;
  if (s->expert_dtype == MOE_MXFP4 || s->expert_dtype == MOE_INT4G64) {
    // the grouped GEMM stages scale (and bias) rows with 16-byte loads
    const void* sc[] = {w->gate_s, w->up_s, w->down_s};
    for (const void* p : sc)
      if (!aligned16(p)) return MOE_EALIGN;
  }
  if (s->expert_dtype == MOE_INT4G64) {
    const void* bi[] = {w->gate_b, w->up_b, w->down_b};
    for (const void* p : bi)
      if (!aligned16(p)) return MOE_EALIGN;
  }
  return MOE_OK;
}

// ---- kernel timing -------------------------------------------------------------------------
struct Timing {
  bool on = false;
  std::vector<hipEvent_t> ev;  // 2 per launch
  std::vector<std::string> names;
  size_t used = 0;  // launches recorded
} g_timing;

// The next event pair for a launch (hipExtLaunchKernel records the kernel's start and end in
// them), or false once the pairs are used up.
bool timing_events(const char* name, hipEvent_t* e0, hipEvent_t* e1) {
  if (!g_timing.on || g_timing.used >= g_timing.names.size()) return false;
  g_timing.names[g_timing.used] = name;
  *e0 = g_timing.ev[2 * g_timing.used];
  *e1 = g_timing.ev[2 * g_timing.used + 1];
  ++g_timing.used;
  return true;
}

LaunchHook hook() {
  LaunchHook h;
  if (g_timing.on) h.events = timing_events;
  return h;
}

// ---- static scratch for moe_forward_static ----------------------------------------------
// One array per GPU the library runs on, held until the process ends.  In host code the name
// `scratch` stands for the symbol, not for its device address: every kernel argument, fill or
// copy uses the pointer hipGetSymbolAddress returned for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up once per device, with that device current),
// or null if the lookup fails.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moe_workspace_size(const moe_shape_t* shape, size_t* bytes) {
  if (!bytes) return MOE_EINVAL;
  int rc = check_shape(shape);
  if (rc) return rc;
  *bytes = layout(shape).total;
  return MOE_OK;
}

int moe_route(const moe_shape_t* shape, const void* x, const moe_weights_t* w, const float* logits_in,
              const moe_route_out_t* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!out || !out->topk_ids || !out->topk_w) return MOE_EINVAL;
  if (!logits_in) {
    if (!x) return MOE_EINVAL;
    if (!aligned16(x)) return MOE_EALIGN;
    rc = check_weights(shape, w, false);
    if (rc) return rc;
  } else if (!aligned16(logits_in)) {
    return MOE_EALIGN;
  }
  if (!ws || ws_bytes < layout(shape).total) return MOE_EWORKSPACE;
  if (!aligned16(ws)) return MOE_EALIGN;
  moe_weights_t none;
  memset(&none, 0, sizeof none);
  Args A = make_args(shape, x, w ? w : &none, ws);
  if (logits_in) {  // selection only: the router (and its bias) is not applied
    A.rw = nullptr;
    A.rbias = nullptr;
  }
  A.logits_in = logits_in;
  A.o_ids = out->topk_ids;
  A.o_w = out->topk_w;
  A.o_logits = out->logits;
  A.o_count = out->expert_count;
  A.o_offset = out->expert_offset;
  A.o_sorted = out->sorted_slot;
  return launch_route_any(A, (hipStream_t)stream, shape->T <= kDecodeMaxT, hook());
}

int moe_forward(const moe_shape_t* shape, const void* x, const moe_weights_t* w, void* y, void* ws,
                size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!x || !y) return MOE_EINVAL;
  rc = check_weights(shape, w, true);
  if (rc) return rc;
  if (!aligned16(x) || !aligned16(y)) return MOE_EALIGN;
  if (!ws || ws_bytes < layout(shape).total) return MOE_EWORKSPACE;
  if (!aligned16(ws)) return MOE_EALIGN;
  Args A = make_args(shape, x, w, ws);
  A.y = y;
  if (shape->T <= kDecodeMaxT) return launch_decode(A, (hipStream_t)stream, false, hook());
  return launch_prefill(A, (hipStream_t)stream, hook());
}

int moe_forward_static(const moe_shape_t* shape, const void* x, const moe_weights_t* w, void* y,
                       void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (layout(shape).total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ESCRATCH;  // before any device call
  if (!x || !y) return MOE_EINVAL;
  rc = check_weights(shape, w, true);
  if (rc) return rc;
  if (!aligned16(x) || !aligned16(y)) return MOE_EALIGN;
  void* ws = scratch_ptr();
  if (!ws) return MOE_EHIP;
  // the kernels of moe_forward; the workspace needs no clearing (nothing carries across calls)
  return moe_forward(shape, x, w, y, ws, (size_t)MOE_STATIC_SCRATCH_BYTES, stream);
}

int moe_workspace_routing(const moe_shape_t* shape, size_t* logits_off, size_t* ids_off, size_t* w_off) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!logits_off || !ids_off || !w_off) return MOE_EINVAL;
  const Layout L = layout(shape);
  *logits_off = L.logits;
  *ids_off = L.ids;
  *w_off = L.cw;
  return MOE_OK;
}

const char* moe_path_name(const moe_shape_t* shape) {
  if (check_shape(shape)) return "invalid";
  const bool dec = shape->T <= kDecodeMaxT;
  switch (shape->expert_dtype) {
    case MOE_F32: return dec ? "decode.f32" : "prefill.f32";
    case MOE_BF16: return dec ? "decode.bf16" : "prefill.bf16";
    case MOE_MXFP4: return dec ? "decode.mxfp4" : shape->act_quant == MOE_QMXFP8 ? "prefill.mxfp4.w4a8" : "prefill.mxfp4";
    case MOE_INT4G64: return dec ? "decode.int4g64" : "prefill.int4g64";
  }
  return "invalid";
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer, size or k out of range)";
    case MOE_EUNSUPPORTED: return "unsupported dtype combination or shape";
    case MOE_EALIGN: return "pointer not 16-byte aligned";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EHIP: return "HIP runtime error or kernel launch failure";
    case MOE_ESCRATCH: return "shape needs more workspace than the static scratch (MOE_STATIC_SCRATCH_BYTES)";
  }
  return "unknown error code";
}

int moe_timing_begin(int32_t max_launches) {
  if (max_launches < 1) return MOE_EINVAL;
  if (g_timing.on) return MOE_EINVAL;
  g_timing.ev.assign(2 * (size_t)max_launches, nullptr);
  g_timing.names.assign((size_t)max_launches, std::string());
  for (auto& e : g_timing.ev)
    if (hipEventCreate(&e) != hipSuccess) return MOE_EHIP;
  g_timing.used = 0;
  g_timing.on = true;
  return MOE_OK;
}

int moe_timing_end(moe_kernel_time_t* out, int32_t max_out, int32_t* n_out) {
  if (!g_timing.on) return MOE_EINVAL;
  g_timing.on = false;
  int rc = MOE_OK;
  std::vector<moe_kernel_time_t> agg;
  for (size_t i = 0; i < g_timing.used; ++i) {
    if (hipEventSynchronize(g_timing.ev[2 * i + 1]) != hipSuccess) {
      rc = MOE_EHIP;
      break;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]) != hipSuccess) {
      rc = MOE_EHIP;
      break;
    }
    moe_kernel_time_t* slot = nullptr;
    for (auto& a : agg)
      if (g_timing.names[i] == a.name) slot = &a;
    if (!slot) {
      moe_kernel_time_t t;
      memset(&t, 0, sizeof t);
      snprintf(t.name, sizeof t.name, "%s", g_timing.names[i].c_str());
      agg.push_back(t);
      slot = &agg.back();
    }
    slot->launches += 1;
    slot->total_ms += ms;
  }
  for (auto& e : g_timing.ev) (void)hipEventDestroy(e);
  g_timing.ev.clear();
  g_timing.names.clear();
  g_timing.used = 0;
  int n = 0;
  for (auto& a : agg)
    if (out && n < max_out) out[n++] = a;
  if (n_out) *n_out = n;
  return rc;
}

}  // extern "C"
