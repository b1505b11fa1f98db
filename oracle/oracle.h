/*
 * Reference ("oracle") implementation of the routed-expert FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This code is a plain, slow, single-threaded
 * restatement of what the layer computes, used to check the GPU library.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no source, header, table or helper with the GPU
 * library, and the GPU library never calls it.
 *
 * What the layer computes (sources are the three web pages this project
 * follows):
 *  - "Optimizing on-device inference for Apple Silicon" (Perplexity),
 *    section "Qwen creates three distinct workload shapes": a router scores
 *    every routed expert and picks eight of them per token; one shared expert
 *    processes every token.
 *  - same page, section "Reduce intermediate and state traffic": an expert is
 *    two input projections followed by a gated activation (gate/up), then an
 *    output projection whose result is scaled by the routing score and added
 *    to the shared expert's result.
 *  - same page, section "Keep expert routing on the GPU": after selection the
 *    assignments are counted per expert (histogram), the counts are turned
 *    into start offsets (prefix scan) and the rows are scattered into
 *    per-expert groups.
 *  - "Three ways to boost mixture-of-experts inference on NVIDIA DGX Spark",
 *    sections "Why decoding was slow in the first place" and "Optimization 1":
 *    512 routed experts, eight per token, a shared expert, hidden size 2560,
 *    expert intermediate size 768, expert weights in MXFP4.
 *
 * Readings taken where the pages are silent (each is also listed with the
 * design notes of the repository):
 *  R1 logits l[t][e] = sum_h x[t][h] * Wr[e][h] + bias[t][e], computed in
 *     double and rounded once to fp32; selection is taken on these fp32 keys.
 *  R2 top-k = the k largest logits, ties to the lower expert index, listed in
 *     descending logit order (ascending index among equals).
 *  R3 p = softmax over all E logits (double); the k combine weights are the
 *     selected p renormalised to sum 1.
 *  R4 expert FFN (SwiGLU): g = Wg x, u = Wu x, a_i = silu(g_i) * u_i with
 *     silu(z) = z / (1 + exp(-z)), o = Wd a.  No biases, no clamp.
 *  R5 y = sum_j w_j * o_j (in rank order j = 0..k-1) + S(x), where S is the
 *     shared expert's FFN with weight 1 (no shared gate).  I_shared = 0 means
 *     no shared expert.
 *  R6 weight layout is [out][in] (rows along the output, the reduction index
 *     contiguous).  MXFP4: two e2m1 codes per byte, the even element in the
 *     low nibble; one e8m0 scale byte per 32 consecutive elements of a row.
 *     e2m1 and e8m0 follow the OCP Microscaling (MX) v1.0 specification.
 *  R6b group-wise affine 4-bit weights (same page, section "Decode weights
 *     during matrix multiplication": each weight is a 4-bit integer code and
 *     every group of 64 weights shares a bfloat16 scale and bias that
 *     reconstruct its values): the code q is unsigned, 0..15, two per byte
 *     with the even element in the low nibble; the groups are 64 consecutive
 *     elements of a row along the reduction index; the weight is s*q + b,
 *     taken exactly (the page's kernel rounds it to bfloat16 before its
 *     multiply; that rounding belongs to the kernel, not to the weight).
 *  R6c W4A8 numerics ("Three ways to boost mixture-of-experts inference on
 *     NVIDIA DGX Spark", section "Why decoding was slow in the first place":
 *     the baseline serves MXFP4 expert weights with 8-bit activations): with
 *     act_quant = 1 the input of each routed expert's two GEMMs (x before
 *     gate/up, a before down) is replaced by its MXFP8 quantisation (OCP MX
 *     v1.0): per 32 consecutive elements along the reduction index a shared
 *     scale X = 2^(floor(log2(amax)) - 8) (8 = the largest exponent of an E4M3
 *     element; clamped to the e8m0 range 2^-127 .. 2^127, a block of zeros
 *     takes 2^-127) and elements P = E4M3(v / X), rounded to nearest even and
 *     saturated to +-448 (OCP FP8 E4M3: bias 7, no infinities, S.1111.111 is
 *     NaN).  The router and the shared expert are not quantised.
 *  R7 routing plan: per-expert counts, exclusive offsets, and slots
 *     (slot = t*k + j) ordered by expert by a stable counting sort.
 *
 * All arithmetic is double precision.  Inputs (fp32, bf16, MXFP4) are decoded
 * exactly to double.
 */
#ifndef ORACLE_MOE_H
#define ORACLE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element encodings understood by the oracle. */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_MXFP4 = 2, ORC_INT4G64 = 3 };

typedef struct {
  int32_t T, H, E, k, I, I_shared;
  int32_t act_dtype;    /* ORC_F32 | ORC_BF16 */
  int32_t expert_dtype; /* ORC_F32 | ORC_BF16 | ORC_MXFP4 | ORC_INT4G64 */
  int32_t shared_dtype; /* ORC_F32 | ORC_BF16 */
  int32_t act_quant;    /* 0: none; 1: MXFP8 inputs of the routed experts' GEMMs (R6c) */
} orc_shape;

typedef struct {
  const float *router_w;     /* [E][H] */
  const float *router_bias;  /* NULL, [E] (stride 0) or [T][E] (stride E) */
  int64_t bias_t_stride;
  const void *gate, *up, *down;          /* [E][I][H], [E][I][H], [E][H][I] */
  const void *gate_s, *up_s, *down_s;    /* MXFP4: e8m0 bytes [E][I][H/32] ...;
                                            INT4G64: bf16 scales [E][I][H/64] ... */
  const void *sh_gate, *sh_up, *sh_down; /* [Is][H], [Is][H], [H][Is] */
  const void *gate_b, *up_b, *down_b;    /* INT4G64: bf16 biases [E][I][H/64] ... */
} orc_weights;

/* Scalar decoders (exact). */
double orc_bf16_to_double(uint16_t bits);
double orc_e2m1_to_double(uint8_t nibble);   /* low 4 bits used */
double orc_e8m0_to_double(uint8_t bits);     /* 2^(bits-127); NaN for 0xFF */
double orc_e4m3_to_double(uint8_t bits);     /* OCP FP8 E4M3; NaN for S.1111.111 */
uint8_t orc_e4m3_from_double(double v);      /* round to nearest even, saturating */

/* R6c: MXFP8 quantisation of n (a multiple of 32) values: codes[n] E4M3,
 * scales[n/32] e8m0.  And its inverse. */
int orc_mxfp8_quantize(const double *v, int n, uint8_t *codes, uint8_t *scales);
int orc_mxfp8_dequantize(const uint8_t *codes, const uint8_t *scales, int n, double *v);

/* Element (row r, column c) of matrix `mat` of a stacked [n_mat][rows][cols]
 * weight array in the given encoding (cols is the reduction dimension). */
double orc_weight(const void *base, const void *scales, const void *biases,
                  int dtype, int64_t mat, int64_t rows, int64_t cols, int64_t r,
                  int64_t c);

/* R1: router logits for all tokens, fp32 [T][E]. */
int orc_logits(const orc_shape *s, const void *x, const orc_weights *w,
               float *logits);

/* R2 + R3 for one token: ids[k] and combine weights w[k] from fp32 logits. */
int orc_select(const float *logits_row, int E, int k, int32_t *ids, double *w);

/* R3 for a given set of k distinct experts ids[k] (any order): the softmax over
 * all E logits, renormalised over the set; w[j] belongs to ids[j].  Used to
 * state the output of every valid selection of a token whose k-th and
 * (k+1)-th logits are nearly equal. */
int orc_set_weights(const float *logits_row, int E, int k, const int32_t *ids,
                    double *w);

/* R7: counts[E], offsets[E+1], sorted_slot[T*k] from ids[T][k]. */
int orc_plan(const int32_t *ids, int T, int k, int E, int32_t *counts,
             int32_t *offsets, int32_t *sorted_slot);

/* One SwiGLU FFN (R4) on one token vector: rows Wg/Wu [I][H], Wd [H][I]. */
int orc_ffn(const double *xv, int H, int I, const void *g, const void *u,
            const void *d, const void *gs, const void *us, const void *ds,
            const void *gb, const void *ub, const void *db, int dtype,
            int64_t mat, int act_quant, double *out);

/* R4 + R5 with the routing given: y[T][H] (double). */
int orc_forward_with_routing(const orc_shape *s, const void *x,
                             const orc_weights *w, const int32_t *ids,
                             const double *cw, double *y);

/* Whole layer: R1..R5.  ids/cw/logits may be NULL. */
int orc_forward(const orc_shape *s, const void *x, const orc_weights *w,
                double *y, int32_t *ids, double *cw, float *logits);

#ifdef __cplusplus
}
#endif
#endif
