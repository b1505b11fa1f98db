/*
 * Reference ("oracle") implementation of the routed-expert FFN layer.
 * TEST INFRASTRUCTURE ONLY -- see oracle.h for what is computed, the sources
 * it follows and the readings taken.  Plain loops, double precision, one
 * thread; nothing here is blocked, fused or reordered beyond the definition.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the upper half of an IEEE binary32 value. */
double orc_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* e2m1 (OCP MX v1.0): 1 sign bit, 2 exponent bits with bias 1, 1 mantissa
 * bit; exponent field 0 is subnormal (0.5 * mantissa). */
double orc_e2m1_to_double(uint8_t nibble) {
  int sign = (nibble >> 3) & 1;
  int ex = (nibble >> 1) & 3;
  int man = nibble & 1;
  double mag;
  if (ex == 0)
    mag = 0.5 * man;
  else
    mag = ldexp(1.0 + 0.5 * man, ex - 1);
  return sign ? -mag : mag;
}

/* e8m0 (OCP MX v1.0): unsigned biased exponent, 2^(bits-127); 0xFF is NaN. */
double orc_e8m0_to_double(uint8_t bits) {
  if (bits == 0xFF) return NAN;
  return ldexp(1.0, (int)bits - 127);
}

/* The 16 e2m1 values and the 256 e8m0 values, filled once when the library is
 * loaded by calling the two decoders above: orc_weight reads an MXFP4 element
 * from these tables (the same values, without a libm call per element). */
static double e2m1_table[16];
static double e8m0_table[256];

__attribute__((constructor)) static void fill_mx_tables(void) {
  for (int c = 0; c < 16; ++c) e2m1_table[c] = orc_e2m1_to_double((uint8_t)c);
  for (int b = 0; b < 256; ++b) e8m0_table[b] = orc_e8m0_to_double((uint8_t)b);
}

/* OCP FP8 E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 is subnormal (mantissa * 2^-9); S.1111.111 is NaN. */
double orc_e4m3_to_double(uint8_t bits) {
  int sign = bits >> 7, ex = (bits >> 3) & 15, man = bits & 7;
  double mag;
  if (ex == 15 && man == 7) return NAN;
  if (ex == 0)
    mag = ldexp((double)man, -9);
  else
    mag = ldexp(1.0 + man / 8.0, ex - 7);
  return sign ? -mag : mag;
}

/* Nearest E4M3 value, ties to the even mantissa, magnitudes beyond the largest
 * finite value (448) saturating to it.  rint rounds half to even in the
 * default rounding mode. */
uint8_t orc_e4m3_from_double(double v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) /* subnormal steps of 2^-9; 8 steps is the smallest normal */
    return sign | (uint8_t)rint(a * 512.0);
  int e;
  double m = frexp(a, &e); /* a = m 2^e, m in [0.5, 1): a = (1 + f) 2^(e-1) */
  int E = e - 1;
  double q = rint((2.0 * m - 1.0) * 8.0); /* the 3-bit mantissa, 8 = carry */
  if (q == 8.0) {
    q = 0.0;
    E += 1;
  }
  return sign | (uint8_t)(((E + 7) << 3) | (int)q);
}

int orc_mxfp8_quantize(const double *v, int n, uint8_t *codes, uint8_t *scales) {
  if (n % 32) return -1;
  for (int b = 0; b < n / 32; ++b) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i)
      if (fabs(v[32 * b + i]) > amax) amax = fabs(v[32 * b + i]);
    int xe = -127; /* shared exponent: floor(log2 amax) - 8, in the e8m0 range */
    if (amax > 0.0) {
      int p;
      frexp(amax, &p); /* amax = m 2^p, m in [0.5, 1): floor(log2 amax) = p - 1 */
      xe = p - 1 - 8;
      if (xe < -127) xe = -127;
      if (xe > 127) xe = 127;
    }
    scales[b] = (uint8_t)(xe + 127);
    for (int i = 0; i < 32; ++i) codes[32 * b + i] = orc_e4m3_from_double(ldexp(v[32 * b + i], -xe));
  }
  return 0;
}

int orc_mxfp8_dequantize(const uint8_t *codes, const uint8_t *scales, int n, double *v) {
  if (n % 32) return -1;
  for (int i = 0; i < n; ++i) v[i] = orc_e4m3_to_double(codes[i]) * orc_e8m0_to_double(scales[i / 32]);
  return 0;
}

/* v[0..n) replaced by its MXFP8 quantisation, dequantised (R6c). */
static int mxfp8_round_trip(double *v, int n) {
  uint8_t *c = (uint8_t *)malloc((size_t)n);
  uint8_t *s = (uint8_t *)malloc((size_t)(n / 32 + 1));
  int rc = (c && s) ? orc_mxfp8_quantize(v, n, c, s) : -2;
  if (rc == 0) rc = orc_mxfp8_dequantize(c, s, n, v);
  free(c);
  free(s);
  return rc;
}

double orc_weight(const void *base, const void *scales, const void *biases,
                  int dtype, int64_t mat, int64_t rows, int64_t cols, int64_t r,
                  int64_t c) {
  int64_t row = mat * rows + r;
  if (dtype == ORC_F32) {
    return (double)((const float *)base)[row * cols + c];
  } else if (dtype == ORC_BF16) {
    return orc_bf16_to_double(((const uint16_t *)base)[row * cols + c]);
  }
  const uint8_t *codes = (const uint8_t *)base;
  uint8_t byte = codes[row * (cols / 2) + c / 2];
  uint8_t nib = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
  if (dtype == ORC_MXFP4) {
    uint8_t sc = ((const uint8_t *)scales)[row * (cols / 32) + c / 32];
    return e2m1_table[nib] * e8m0_table[sc];
  }
  /* ORC_INT4G64: s * q + b with the group's bf16 scale and bias */
  int64_t g = row * (cols / 64) + c / 64;
  double s = orc_bf16_to_double(((const uint16_t *)scales)[g]);
  double b = orc_bf16_to_double(((const uint16_t *)biases)[g]);
  return s * (double)nib + b;
}

static double act_value(const orc_shape *s, const void *x, int t, int h) {
  if (s->act_dtype == ORC_F32) return (double)((const float *)x)[(int64_t)t * s->H + h];
  return orc_bf16_to_double(((const uint16_t *)x)[(int64_t)t * s->H + h]);
}

static int shape_ok(const orc_shape *s) {
  if (s->T < 0 || s->H < 1 || s->E < 1 || s->k < 1 || s->k > s->E || s->I < 1 || s->I_shared < 0)
    return 0;
  if (s->expert_dtype == ORC_MXFP4 && (s->H % 32 != 0 || s->I % 32 != 0)) return 0;
  if (s->expert_dtype == ORC_INT4G64 && (s->H % 64 != 0 || s->I % 64 != 0)) return 0;
  if (s->act_quant && (s->H % 32 != 0 || s->I % 32 != 0)) return 0;
  return 1;
}

int orc_logits(const orc_shape *s, const void *x, const orc_weights *w,
               float *logits) {
  if (!shape_ok(s)) return -1;
  for (int t = 0; t < s->T; ++t) {
    for (int e = 0; e < s->E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < s->H; ++h)
        acc += act_value(s, x, t, h) * (double)w->router_w[(int64_t)e * s->H + h];
      if (w->router_bias)
        acc += (double)w->router_bias[(int64_t)t * w->bias_t_stride + e];
      logits[(int64_t)t * s->E + e] = (float)acc;
    }
  }
  return 0;
}

/* "a ranks before b": larger logit first, lower index among equal logits. */
static int ranks_before(float la, int a, float lb, int b) {
  if (la > lb) return 1;
  if (la < lb) return 0;
  return a < b;
}

int orc_select(const float *lrow, int E, int k, int32_t *ids, double *w) {
  if (E < 1 || k < 1 || k > E) return -1;
  char *taken = (char *)calloc((size_t)E, 1);
  if (!taken) return -2;
  /* k rounds of "best remaining expert". */
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || ranks_before(lrow[e], e, lrow[best], best)) best = e;
    }
    taken[best] = 1;
    ids[j] = best;
  }
  free(taken);
  /* softmax over all E logits, then renormalise the selected ones. */
  double m = -INFINITY;
  for (int e = 0; e < E; ++e)
    if ((double)lrow[e] > m) m = (double)lrow[e];
  double z = 0.0;
  for (int e = 0; e < E; ++e) z += exp((double)lrow[e] - m);
  double sel = 0.0;
  for (int j = 0; j < k; ++j) {
    w[j] = exp((double)lrow[ids[j]] - m) / z;
    sel += w[j];
  }
  for (int j = 0; j < k; ++j) w[j] = w[j] / sel;
  return 0;
}

int orc_set_weights(const float *lrow, int E, int k, const int32_t *ids,
                    double *w) {
  if (E < 1 || k < 1 || k > E) return -1;
  for (int j = 0; j < k; ++j) {
    if (ids[j] < 0 || ids[j] >= E) return -1;
    for (int i = 0; i < j; ++i)
      if (ids[i] == ids[j]) return -1;
  }
  /* p_e = exp(l_e - m) / sum over all E of exp(l - m); then w_j = p_{ids[j]} / sum of the set's p. */
  double m = -INFINITY;
  for (int e = 0; e < E; ++e)
    if ((double)lrow[e] > m) m = (double)lrow[e];
  double z = 0.0;
  for (int e = 0; e < E; ++e) z += exp((double)lrow[e] - m);
  double sel = 0.0;
  for (int j = 0; j < k; ++j) {
    w[j] = exp((double)lrow[ids[j]] - m) / z;
    sel += w[j];
  }
  for (int j = 0; j < k; ++j) w[j] = w[j] / sel;
  return 0;
}

int orc_plan(const int32_t *ids, int T, int k, int E, int32_t *counts,
             int32_t *offsets, int32_t *sorted_slot) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int s = 0; s < T * k; ++s) {
    if (ids[s] < 0 || ids[s] >= E) return -1;
    counts[ids[s]] += 1; /* histogram */
  }
  offsets[0] = 0; /* exclusive prefix scan */
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  if (!next) return -2;
  for (int e = 0; e < E; ++e) next[e] = offsets[e];
  for (int s = 0; s < T * k; ++s) sorted_slot[next[ids[s]]++] = s; /* scatter */
  free(next);
  return 0;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

int orc_ffn(const double *xv, int H, int I, const void *g, const void *u,
            const void *d, const void *gs, const void *us, const void *ds,
            const void *gb, const void *ub, const void *db, int dtype,
            int64_t mat, int act_quant, double *out) {
  double *a = (double *)malloc(sizeof(double) * (size_t)I);
  double *xq = (double *)malloc(sizeof(double) * (size_t)H);
  if (!a || !xq) {
    free(a);
    free(xq);
    return -2;
  }
  int rc = 0;
  for (int h = 0; h < H; ++h) xq[h] = xv[h];
  if (act_quant) rc = mxfp8_round_trip(xq, H); /* R6c: the gate/up input */
  for (int i = 0; i < I && rc == 0; ++i) {
    double gi = 0.0, ui = 0.0;
    for (int h = 0; h < H; ++h) {
      gi += orc_weight(g, gs, gb, dtype, mat, I, H, i, h) * xq[h];
      ui += orc_weight(u, us, ub, dtype, mat, I, H, i, h) * xq[h];
    }
    a[i] = silu(gi) * ui;
  }
  if (rc == 0 && act_quant) rc = mxfp8_round_trip(a, I); /* R6c: the down input */
  for (int h = 0; h < H && rc == 0; ++h) {
    double o = 0.0;
    for (int i = 0; i < I; ++i) o += orc_weight(d, ds, db, dtype, mat, H, I, h, i) * a[i];
    out[h] = o;
  }
  free(a);
  free(xq);
  return rc;
}

int orc_forward_with_routing(const orc_shape *s, const void *x,
                             const orc_weights *w, const int32_t *ids,
                             const double *cw, double *y) {
  if (!shape_ok(s)) return -1;
  int H = s->H;
  double *xv = (double *)malloc(sizeof(double) * (size_t)H);
  double *o = (double *)malloc(sizeof(double) * (size_t)H);
  if (!xv || !o) {
    free(xv);
    free(o);
    return -2;
  }
  int rc = 0;
  for (int t = 0; t < s->T && rc == 0; ++t) {
    for (int h = 0; h < H; ++h) xv[h] = act_value(s, x, t, h);
    double *yt = y + (int64_t)t * H;
    for (int h = 0; h < H; ++h) yt[h] = 0.0;
    for (int j = 0; j < s->k && rc == 0; ++j) {
      int e = ids[(int64_t)t * s->k + j];
      if (e < 0 || e >= s->E) {
        rc = -1;
        break;
      }
      rc = orc_ffn(xv, H, s->I, w->gate, w->up, w->down, w->gate_s, w->up_s,
                   w->down_s, w->gate_b, w->up_b, w->down_b, s->expert_dtype, e,
                   s->act_quant, o);
      for (int h = 0; h < H; ++h) yt[h] += cw[(int64_t)t * s->k + j] * o[h];
    }
    if (rc == 0 && s->I_shared > 0) {
      rc = orc_ffn(xv, H, s->I_shared, w->sh_gate, w->sh_up, w->sh_down, NULL,
                   NULL, NULL, NULL, NULL, NULL, s->shared_dtype, 0, 0, o);
      for (int h = 0; h < H; ++h) yt[h] += o[h];
    }
  }
  free(xv);
  free(o);
  return rc;
}

int orc_forward(const orc_shape *s, const void *x, const orc_weights *w,
                double *y, int32_t *ids_out, double *cw_out, float *logits_out) {
  if (!shape_ok(s)) return -1;
  size_t TE = (size_t)s->T * s->E, Tk = (size_t)s->T * s->k;
  float *lg = (float *)malloc(sizeof(float) * (TE ? TE : 1));
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (Tk ? Tk : 1));
  double *cw = (double *)malloc(sizeof(double) * (Tk ? Tk : 1));
  int rc = (lg && ids && cw) ? 0 : -2;
  if (rc == 0) rc = orc_logits(s, x, w, lg);
  for (int t = 0; t < s->T && rc == 0; ++t)
    rc = orc_select(lg + (int64_t)t * s->E, s->E, s->k, ids + (int64_t)t * s->k,
                    cw + (int64_t)t * s->k);
  if (rc == 0) rc = orc_forward_with_routing(s, x, w, ids, cw, y);
  if (rc == 0) {
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * Tk);
    if (cw_out) memcpy(cw_out, cw, sizeof(double) * Tk);
    if (logits_out) memcpy(logits_out, lg, sizeof(float) * TE);
  }
  free(lg);
  free(ids);
  free(cw);
  return rc;
}
