/*
 * libmoe -- routed-expert FFN layer (sparse mixture of experts) on MI355X.
 *
 * C ABI.  Every array argument is a plain pointer to caller-owned DEVICE
 * memory (HBM of the current HIP device); every size is in elements unless a
 * name ends in _bytes.  The library allocates nothing on the device and
 * never synchronises the host inside a call: calls enqueue kernels on the
 * given HIP stream and return.
 *
 * What the layer computes, per token t (sources are the pages this project
 * follows; readings taken where they are silent are marked "reading"):
 *   l[t][e] = sum_h x[t][h] * Wr[e][h] + bias[t][e]                (router)
 *   S_t     = the k experts with the largest l[t][e]; ties go to the lower
 *             expert index; listed by descending logit             (reading)
 *   w[t][j] = softmax_e(l[t])[e_j] / sum_{i<k} softmax_e(l[t])[e_i] (reading)
 *   FFN_e(v) = Wd_e ( silu(Wg_e v) * (Wu_e v) ),  silu(z) = z/(1+exp(-z))
 *   y[t]    = sum_j w[t][j] * FFN_{e_j}(x[t]) + FFN_shared(x[t])
 * "Optimizing on-device inference for Apple Silicon" (Perplexity), sections
 * "Qwen creates three distinct workload shapes" (a router scores every
 * routed expert and picks eight; one shared expert sees every token) and
 * "Reduce intermediate and state traffic" (gate/up projections with a gated
 * activation; output projection combined with the routing score and the
 * shared expert's result).  "Three ways to boost mixture-of-experts
 * inference on NVIDIA DGX Spark", sections "Why decoding was slow in the
 * first place" and "Optimization 1" (512 experts, top-8, a shared expert,
 * MXFP4 expert weights).
 *
 * Layouts (reading: nn.Linear [out][in], reduction index contiguous):
 *   x        [T][H]          act_dtype
 *   router_w [E][H]          fp32
 *   gate, up [E][I][H]       expert_dtype   (MXFP4: codes [E][I][H/2])
 *   down     [E][H][I]       expert_dtype   (MXFP4: codes [E][H][I/2])
 *   MXFP4    two e2m1 codes per byte, element 2i in the low nibble; one e8m0
 *            scale byte per 32 consecutive elements of a row:
 *            gate_s, up_s [E][I][H/32], down_s [E][H][I/32]  (OCP MX v1.0)
 *   INT4G64  group-wise affine 4-bit ("Optimizing on-device inference for
 *            Apple Silicon", section "Decode weights during matrix
 *            multiplication": a 4-bit integer code per weight, a bfloat16
 *            scale and bias per 64 weights): unsigned codes q in 0..15 packed
 *            like MXFP4; per 64 consecutive elements of a row one bf16 scale s
 *            and one bf16 bias b, weight = s * q + b:
 *            gate_s/gate_b, up_s/up_b [E][I][H/64], down_s/down_b [E][H][I/64]
 *   sh_gate, sh_up [I_shared][H], sh_down [H][I_shared]   shared_dtype
 *   y        [T][H]          out_dtype
 *
 * Error behaviour: every entry point validates all arguments before it
 * enqueues anything, so MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EALIGN and
 * MOE_EWORKSPACE mean that nothing was launched and no output was written.
 * MOE_EHIP means a kernel launch failed; kernels of the same call enqueued
 * before it may still run, so the outputs and the workspace are then
 * undefined.  NaN/Inf inputs are not checked; they propagate.
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MOE_OK 0
#define MOE_EINVAL (-1)        /* null required pointer, bad size, k > E ...   */
#define MOE_EUNSUPPORTED (-2)  /* dtype combination or shape outside limits    */
#define MOE_EALIGN (-3)        /* a pointer is not 16-byte aligned (MXFP4 scale
                                  arrays included)                              */
#define MOE_EWORKSPACE (-4)    /* workspace null or smaller than required      */
#define MOE_EHIP (-5)          /* a HIP runtime call or kernel launch failed   */
#define MOE_ESCRATCH (-6)      /* moe_forward_static: the shape's workspace is
                                  larger than MOE_STATIC_SCRATCH_BYTES          */

/* Element encodings. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2, MOE_INT4G64 = 3 } moe_dtype_t;

/* Limits checked by every entry point. */
#define MOE_MAX_E 1024     /* routed experts                                   */
#define MOE_MAX_K 16       /* experts per token                                */
#define MOE_MAX_H 16384    /* hidden size                                      */
#define MOE_MAX_I 8192     /* intermediate sizes                               */
/* T > 16 (grouped-GEMM path) additionally needs bf16 activations, T * H * 2 < 2^31 bytes
   of x and, with 4-bit experts, GEMM launches whose LDS fits the CU's 160 KiB: each wave
   stages its weight rows' scale block (INT4G64: and bias block) for the whole reduction, so
   MXFP4 (and W4A8) take H, I <= 8192 and INT4G64 H <= 7680, I <= 6144. */

typedef struct {
  int32_t T;            /* tokens, >= 1                                        */
  int32_t H;            /* hidden size, multiple of 32 (INT4G64: of 64)        */
  int32_t E;            /* routed experts, 1..MOE_MAX_E                        */
  int32_t k;            /* experts per token, 1..min(E, MOE_MAX_K)             */
  int32_t I;            /* routed intermediate size, multiple of 32 (INT4G64: of 64) */
  int32_t I_shared;     /* shared intermediate size, multiple of 32; 0 = none  */
  int32_t act_dtype;    /* x:          MOE_F32 | MOE_BF16                      */
  int32_t expert_dtype; /* gate/up/down: MOE_F32 | MOE_BF16 | MOE_MXFP4 | MOE_INT4G64 */
  int32_t shared_dtype; /* shared expert: MOE_F32 | MOE_BF16                   */
  int32_t out_dtype;    /* y:          MOE_F32 | MOE_BF16                      */
  int32_t act_quant;    /* MOE_QNONE, or MOE_QMXFP8: W4A8 numerics             */
} moe_shape_t;

/* act_quant.  MOE_QMXFP8 ("Three ways to boost mixture-of-experts inference
 * on NVIDIA DGX Spark", section "Why decoding was slow in the first place":
 * MXFP4 expert weights with 8-bit activations): the input of each routed
 * expert's two GEMMs -- x before gate/up, the SwiGLU activations before down --
 * is quantised to MXFP8 (OCP MX v1.0: per 32 consecutive elements along the
 * reduction index an e8m0 scale 2^(floor(log2 amax) - 8), clamped to the e8m0
 * range, and E4M3 elements rounded to nearest even, saturated at +-448), and
 * both GEMMs run on gfx950's block-scaled fp8 x fp4 matrix cores.  The router
 * and the shared expert stay unquantised.  Needs MXFP4 experts, bf16
 * activations and T > 16 (the grouped-GEMM path); else MOE_EUNSUPPORTED. */
#define MOE_QNONE 0
#define MOE_QMXFP8 1

typedef struct {
  const float *router_w;     /* [E][H], required                               */
  const float *router_bias;  /* nullable; [E] if bias_t_stride == 0,
                                [T][E] if bias_t_stride == E                   */
  int64_t bias_t_stride;
  const void *gate, *up, *down;          /* required                           */
  const void *gate_s, *up_s, *down_s;    /* MXFP4: e8m0 scale bytes; INT4G64:
                                            bf16 group scales; else unused     */
  const void *sh_gate, *sh_up, *sh_down; /* required iff I_shared > 0          */
  const void *gate_b, *up_b, *down_b;    /* INT4G64: bf16 group biases; else
                                            unused                             */
} moe_weights_t;

typedef struct {          /* outputs of moe_route; ids and w required         */
  int32_t *topk_ids;      /* [T][k] chosen experts, descending logit           */
  float *topk_w;          /* [T][k] combine weights (sum to 1 per token)       */
  float *logits;          /* nullable; [T][E] biased router logits             */
  int32_t *expert_count;  /* nullable; [E] assignments per expert (histogram)  */
  int32_t *expert_offset; /* nullable; [E+1] exclusive prefix scan of counts   */
  int32_t *sorted_slot;   /* nullable; [T*k] slots s = t*k + j grouped by
                             expert: group e is sorted_slot[offset[e] ..
                             offset[e+1]); the order inside a group is not
                             specified                                         */
} moe_route_out_t;

/*
 * Workspace bytes that moe_route / moe_forward need for this shape: the router logits, the
 * per-token selection, the token-to-expert plan and the intermediate activations of the
 * layer ("Optimizing on-device inference for Apple Silicon", sections "Keep expert routing
 * on the GPU" and "Reduce intermediate and state traffic": routing stays on the device and
 * the intermediates the fused steps hand over are the only extra traffic).  The caller
 * allocates that many bytes of device memory (16-byte aligned; hipMalloc's 256-byte
 * alignment is fine) and passes it to every call.  Its contents need no initialisation
 * and carry nothing from one call to the next.  One workspace must not be used by two
 * calls that may run concurrently (e.g. on two streams).
 * Returns MOE_OK, MOE_EINVAL (null pointer) or a shape-validation error.
 */
int moe_workspace_size(const moe_shape_t *shape, size_t *bytes);

/*
 * Routing only: router logits, top-k selection, combine weights, and the
 * token-to-expert permutation (histogram of assignments per expert, prefix
 * scan to start offsets, scatter of slots into expert groups) --
 * "Optimizing on-device inference for Apple Silicon", section "Keep expert
 * routing on the GPU".
 *   x          [T][H] act_dtype; ignored when logits_in is given
 *   logits_in  nullable [T][E] fp32: if given, selection runs on these
 *              logits (bias is NOT added again) instead of the router
 *   out        output pointers, see moe_route_out_t
 *   ws         workspace of ws_bytes >= moe_workspace_size()
 *   stream     hipStream_t (NULL = default stream)
 * Only gate/up/down-independent fields of `w` are read (router_w, bias).
 */
int moe_route(const moe_shape_t *shape, const void *x, const moe_weights_t *w,
              const float *logits_in, const moe_route_out_t *out, void *ws,
              size_t ws_bytes, void *stream);

/*
 * The whole layer: y = routed experts combined with their weights + shared
 * expert, for all T tokens ("Optimizing on-device inference for Apple
 * Silicon", sections "Qwen creates three distinct workload shapes" and
 * "Reduce intermediate and state traffic"; the formulas at the top of this
 * file).  No host synchronisation, no allocation; the launch configuration
 * depends on the shape only, so the call can be captured into a HIP graph.
 * y must not alias x, the weights or ws.
 *   x [T][H] act_dtype, y [T][H] out_dtype, ws/ws_bytes as above,
 *   stream hipStream_t (NULL = default stream).
 */
int moe_forward(const moe_shape_t *shape, const void *x, const moe_weights_t *w,
                void *y, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_forward without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is a
 * static device array of MOE_STATIC_SCRATCH_BYTES that each GPU the library
 * runs on holds until the process ends; shapes whose moe_workspace_size
 * exceeds it are rejected with MOE_ESCRATCH before anything touches the
 * device (every decode shape fits; prefill fits up to a few hundred tokens at
 * the Qwen and Ling shapes).  Same kernels and results as moe_forward.  All
 * calls on one GPU share its array: calls that may overlap on one GPU (two
 * streams, two threads) race and must not be issued.  Nothing carries over
 * from one call to the next.  Arguments, layouts and errors as moe_forward.
 */
#define MOE_STATIC_SCRATCH_BYTES (32u << 20)
int moe_forward_static(const moe_shape_t *shape, const void *x,
                       const moe_weights_t *w, void *y, void *stream);

/*
 * Where moe_forward leaves the routing it used, as byte offsets into its
 * workspace: the biased router logits [T][E] fp32 at *logits_off, each token's
 * k experts in ascending expert id [T][k] int32 at *ids_off, and their
 * combine weights [T][k] fp32 (same order) at *w_off.  Valid once the
 * stream has run the moe_forward call and until the workspace is used again;
 * for inspection and tests (the selection the expert kernels consumed, checked
 * against an independent implementation, "Optimizing on-device inference for
 * Apple Silicon", section "Keep expert routing on the GPU").
 * Returns MOE_OK, MOE_EINVAL (null pointer) or a shape-validation error.
 */
int moe_workspace_routing(const moe_shape_t *shape, size_t *logits_off,
                          size_t *ids_off, size_t *w_off);

/*
 * Name of the kernel path moe_forward takes for this shape, e.g.
 * "decode.bf16" or "prefill.bf16" ("Three ways to boost mixture-of-experts
 * inference on NVIDIA DGX Spark", section "What this means for your
 * deployment": check at start-up that the intended path is the active one).
 * Returns "invalid" for a shape that fails validation.  Static string.
 */
const char *moe_path_name(const moe_shape_t *shape);

/* Static text for a return code (the codes above; "unknown error code" for
 * any other value).  Needs no device. */
const char *moe_strerror(int code);

/*
 * Kernel timing for measurement.  moe_timing_begin(n) creates n pairs of
 * HIP events (an allocation: call it outside any timed or captured region);
 * afterwards every kernel that moe_route / moe_forward launch takes the next
 * pair and is launched with hipExtLaunchKernel, which records the kernel's own
 * start and end in them (no marker packets between kernels), until the pairs
 * run out.  moe_timing_end() synchronises those events, writes for each
 * distinct kernel its name, the number of timed launches and their summed
 * duration in milliseconds (up to max_out entries, *n_out set to the count),
 * destroys the events and turns timing off.  Not thread-safe; for
 * benchmarks only ("Optimizing on-device inference for Apple Silicon",
 * section "Limits of further optimization": each kernel is measured against
 * the rate its access pattern can sustain).
 */
typedef struct {
  char name[64];
  int32_t launches;
  double total_ms;
} moe_kernel_time_t;

int moe_timing_begin(int32_t max_launches);
int moe_timing_end(moe_kernel_time_t *out, int32_t max_out, int32_t *n_out);

/*
 * Read-rate probe for measurement: streams bytes (>= 16; the tail below a
 * multiple of 16 is not read) of buf once with 16-byte loads spread over the
 * whole chip, the access pattern of the decode kernels, and returns.  Timing
 * it gives the sustained read ceiling the weight-streaming kernels are
 * compared with ("Optimizing on-device inference for Apple Silicon", section
 * "Limits of further optimization").  sink: 64 writable uint32 of device
 * memory the kernel may write to (in practice it does not).  buf 16-byte
 * aligned (MOE_EALIGN), null pointers MOE_EINVAL.
 */
int moe_read_ceiling(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/*
 * Operand-staging probe for measurement: the prefill GEMMs' way of feeding
 * their matrix cores (16 bytes per lane loaded from memory straight into LDS)
 * with each load instruction covering rows of seg_bytes contiguous bytes, rows
 * 4 KiB apart inside the first region_bytes of buf.  512 blocks of four
 * waves; each wave moves iters * 6144 bytes with six loads in flight, so one
 * call moves 512 * 4 * iters * 6144 bytes.  Timing it for seg_bytes 16, 64 and
 * 128 over a region that fits the L2 gives the rate at which the 4-bit weight
 * rows (16 bytes per 32-deep step), the bf16 operand rows (64) and full cache
 * lines (128) can be staged ("Optimizing on-device inference for Apple
 * Silicon", section "Limits of further optimization": kernels are compared
 * with the fastest rate their access pattern sustains).  region_bytes a power
 * of two in [8 KiB, 2 GiB], seg_bytes a power of two in [16, 1024], iters >= 1,
 * null pointers: MOE_EINVAL; buf not 16-byte or sink not 4-byte aligned:
 * MOE_EALIGN.  sink: 64 writable uint32 of device memory (in practice not
 * written).
 */
int moe_stage_rate(const void *buf, size_t region_bytes, int32_t seg_bytes, int32_t iters, uint32_t *sink,
                   void *stream);

#ifdef __cplusplus
}
#endif
#endif
