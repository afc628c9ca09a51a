/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.  A plain CPU reference of one
 * routed-MoE layer over block-quantized experts; see oracle.h for the block
 * formats and the pages cited as [P2], [P3], [P5].
 *
 * Written for a reader checking it against the definitions by eye: no
 * blocking, no fusion, no decode-once.  Every block a column touches is
 * decoded again for that column.  All arithmetic is double; the layer output
 * is rounded to fp32 once at the end.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- scalars */

int orc_block_bytes(int fmt) {
  /* [P3] "ROCmFPX": FP2 is 10 bytes per 32-weight block (2.50 bit/weight),
   * FP3 about 3.50 bit/weight (14 bytes), FP4 about 4.25 bit/weight
   * (17 bytes). */
  switch (fmt) {
    case ORC_FP2: return 10;
    case ORC_FP3: return 14;
    case ORC_FP4: return 17;
    default: return 0;
  }
}

double orc_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 31;
  int man = h & 1023;
  double v;
  if (ex == 0) {
    v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
  } else if (ex == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + man), ex - 25); /* (1 + man/1024) * 2^(ex-15) */
  }
  return sign ? -v : v;
}

double orc_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

uint16_t orc_double_to_half_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7E00;
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex);     /* a = m * 2^ex, m in [0.5, 1) */
  int E = ex - 1;    /* a = (1.f) * 2^E */
  if (E < -14) {
    /* subnormal range: multiples of 2^-24; nearbyint rounds half to even */
    double r = nearbyint(ldexp(a, 24));
    return (uint16_t)(sign | (uint16_t)r); /* r == 1024 is the smallest normal */
  }
  double r = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
  if (r == 2048.0) {
    r = 1024.0;
    E += 1;
  }
  if (E > 15) return (uint16_t)(sign | 0x7C00);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(r - 1024.0));
}

/* ----------------------------------------------------------- block decode */

/* Read bits [pos, pos+n) of a little-endian byte string, one bit at a time. */
static int read_bits(const uint8_t *b, int pos, int n) {
  int v = 0;
  for (int i = 0; i < n; ++i) {
    int bit = (b[(pos + i) / 8] >> ((pos + i) % 8)) & 1;
    v |= bit << i;
  }
  return v;
}

void orc_block_codes(int fmt, const uint8_t *blk, int codes[32],
                     double *scale) {
  switch (fmt) {
    case ORC_FP2:
      for (int j = 0; j < 32; ++j) codes[j] = read_bits(blk, 2 * j, 2);
      *scale = orc_half_to_double((uint16_t)(blk[8] | (blk[9] << 8)));
      break;
    case ORC_FP3:
      for (int j = 0; j < 32; ++j) codes[j] = read_bits(blk, 3 * j, 3);
      *scale = orc_half_to_double((uint16_t)(blk[12] | (blk[13] << 8)));
      break;
    case ORC_FP4:
      for (int j = 0; j < 32; ++j) codes[j] = read_bits(blk, 4 * j, 4);
      *scale = ldexp(1.0, (int)blk[16] - 127); /* E8M0: 2^(e-127) */
      break;
    default:
      for (int j = 0; j < 32; ++j) codes[j] = 0;
      *scale = NAN;
  }
}

/* Code offset: the codebook is symmetric about zero, value = code - offset. */
static double code_offset(int fmt) {
  switch (fmt) {
    case ORC_FP2: return 1.5; /* {-1.5, -0.5, 0.5, 1.5} */
    case ORC_FP3: return 3.5; /* {-3.5 .. 3.5} */
    case ORC_FP4: return 7.5; /* {-7.5 .. 7.5} */
    default: return NAN;
  }
}

static int code_bits(int fmt) { return fmt; /* FP2 -> 2, FP3 -> 3, FP4 -> 4 */ }

void orc_decode_block(int fmt, const uint8_t *blk, double w[32]) {
  int c[32];
  double s;
  orc_block_codes(fmt, blk, c, &s);
  double o = code_offset(fmt);
  for (int j = 0; j < 32; ++j) w[j] = ((double)c[j] - o) * s;
}

void orc_unpack(int fmt, const uint8_t *bytes, int rows, int cols, double *w) {
  int bb = orc_block_bytes(fmt);
  int nb = cols / 32;
  for (int r = 0; r < rows; ++r)
    for (int b = 0; b < nb; ++b)
      orc_decode_block(fmt, bytes + ((size_t)r * nb + b) * bb,
                       w + (size_t)r * cols + 32 * b);
}

/* ------------------------------------------------------------ block encode */

static void write_bits(uint8_t *b, int pos, int n, int v) {
  for (int i = 0; i < n; ++i)
    if ((v >> i) & 1) b[(pos + i) / 8] |= (uint8_t)(1u << ((pos + i) % 8));
}

static void pack_one(int fmt, const int codes[32], uint16_t scale_bits,
                     uint8_t *blk) {
  int bb = orc_block_bytes(fmt);
  memset(blk, 0, (size_t)bb);
  int nbits = code_bits(fmt);
  for (int j = 0; j < 32; ++j) write_bits(blk, nbits * j, nbits, codes[j]);
  if (fmt == ORC_FP4) {
    blk[16] = (uint8_t)scale_bits;
  } else {
    blk[bb - 2] = (uint8_t)(scale_bits & 0xFF);
    blk[bb - 1] = (uint8_t)(scale_bits >> 8);
  }
}

void orc_pack_codes(int fmt, const uint8_t *codes, const uint16_t *scale_bits,
                    int rows, int cols, uint8_t *out) {
  int bb = orc_block_bytes(fmt);
  size_t nblk = (size_t)rows * (cols / 32);
  for (size_t i = 0; i < nblk; ++i) {
    int c[32];
    for (int j = 0; j < 32; ++j) c[j] = codes[32 * i + j];
    pack_one(fmt, c, scale_bits[i], out + i * bb);
  }
}

static double clampd(double v, double lo, double hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

/* Quantizer for one block: absmax scaling.  The largest magnitude a maps to
 * the outermost code value (offset o), the scale is rounded once (fp16 round
 * to nearest even, or a power of two for FP4), and every code is the nearest
 * (ties to even) integer to w/s + o computed from that rounded scale. */
static void quantize_block(int fmt, const float *w, uint8_t *blk) {
  int bb = orc_block_bytes(fmt);
  double o = code_offset(fmt);
  double cmax = (double)((1 << code_bits(fmt)) - 1);
  double a = 0.0;
  for (int j = 0; j < 32; ++j)
    if (fabs((double)w[j]) > a) a = fabs((double)w[j]);
  memset(blk, 0, (size_t)bb);
  if (a == 0.0) return; /* all-zero block */
  int c[32];
  if (fmt == ORC_FP4) {
    int ex;
    double m = frexp(a / o, &ex); /* a/o = m * 2^ex, m in [0.5, 1) */
    int ceil_log2 = (m == 0.5) ? ex - 1 : ex;
    int e = 127 + ceil_log2;
    if (e < 1) e = 1;
    if (e > 254) e = 254;
    for (int j = 0; j < 32; ++j)
      c[j] = (int)clampd(nearbyint(ldexp((double)w[j], 127 - e) + o), 0.0, cmax);
    pack_one(fmt, c, (uint16_t)e, blk);
    return;
  }
  uint16_t s16 = orc_double_to_half_rne(a / o);
  if ((s16 & 0x7FFF) == 0x7C00) s16 = 0x7BFF; /* overflow clamps to 65504 */
  double s = orc_half_to_double(s16);
  if (s == 0.0) return; /* the rounded scale vanished: all-zero block */
  for (int j = 0; j < 32; ++j)
    c[j] = (int)clampd(nearbyint((double)w[j] / s + o), 0.0, cmax);
  pack_one(fmt, c, s16, blk);
}

void orc_pack(int fmt, const float *w, int rows, int cols, uint8_t *out) {
  int bb = orc_block_bytes(fmt);
  int nb = cols / 32;
  for (int r = 0; r < rows; ++r)
    for (int b = 0; b < nb; ++b)
      quantize_block(fmt, w + (size_t)r * cols + 32 * b,
                     out + ((size_t)r * nb + b) * bb);
}

/* Importance-weighted quantizer ([P3] "ROCmFPX": the weights are quantized
 * with an importance matrix).  The pages do not give the search; the one
 * here is the plainest that uses a per-column importance:
 *   error(block, s) = sum_j imp_j * (w_j - (c_j - o) * s)^2,
 * codes c_j nearest (ties to even) to w_j / s + o, clamped, from the scale
 * s as stored; the stored scale is the candidate of least error, the first
 * one listed winning a tie.  Candidates, for a = max_j |w_j|:
 *   FP2/FP3: s = fp16(a / (o * t)) for t = 1, 1 + 1/16, 1 - 1/16, 1 + 2/16,
 *            1 - 2/16, ..., 1 + 8/16, 1 - 8/16 (t = 1 is the absmax scale);
 *            a scale that overflows fp16 clamps to 65504, a scale of 0 or one
 *            already listed is skipped;
 *   FP4:     e = e0, e0 - 1, e0 + 1 with e0 the absmax exponent of
 *            quantize_block, each clamped to [1, 254], repeats skipped.
 * For a fixed scale the nearest code minimizes each weight's term on its
 * own (the terms are independent and imp_j >= 0), so only the scale is
 * searched.  a = 0 (or no candidate left) gives the all-zero block. */
static double block_error(int fmt, const float *w, const float *imp,
                          const int c[32], double s) {
  double o = code_offset(fmt), err = 0.0;
  for (int j = 0; j < 32; ++j) {
    double d = (double)w[j] - ((double)c[j] - o) * s;
    err += (double)imp[j] * (d * d);
  }
  return err;
}

static void codes_for_scale(int fmt, const float *w, double s, int c[32]) {
  double o = code_offset(fmt);
  double cmax = (double)((1 << code_bits(fmt)) - 1);
  for (int j = 0; j < 32; ++j)
    c[j] = (int)clampd(nearbyint((double)w[j] / s + o), 0.0, cmax);
}

static void quantize_block_weighted(int fmt, const float *w, const float *imp,
                                    uint8_t *blk) {
  int bb = orc_block_bytes(fmt);
  double o = code_offset(fmt);
  double a = 0.0;
  for (int j = 0; j < 32; ++j)
    if (fabs((double)w[j]) > a) a = fabs((double)w[j]);
  memset(blk, 0, (size_t)bb);
  if (a == 0.0) return;
  int c[32], best_c[32];
  double best = INFINITY;
  int have = 0;
  uint16_t best_bits = 0, seen[17];
  int nseen = 0;
  if (fmt == ORC_FP4) {
    int ex;
    double m = frexp(a / o, &ex);
    int e0 = 127 + ((m == 0.5) ? ex - 1 : ex);
    int cand[3] = {e0, e0 - 1, e0 + 1};
    for (int i = 0; i < 3; ++i) {
      int e = cand[i] < 1 ? 1 : (cand[i] > 254 ? 254 : cand[i]);
      int dup = 0;
      for (int k = 0; k < nseen; ++k) dup |= seen[k] == (uint16_t)e;
      if (dup) continue;
      seen[nseen++] = (uint16_t)e;
      double s = ldexp(1.0, e - 127);
      codes_for_scale(fmt, w, s, c);
      double err = block_error(fmt, w, imp, c, s);
      if (!have || err < best) {
        have = 1;
        best = err;
        best_bits = (uint16_t)e;
        memcpy(best_c, c, sizeof c);
      }
    }
  } else {
    for (int i = 0; i < 17; ++i) {
      int k = (i + 1) / 2 * ((i & 1) ? 1 : -1); /* 0, 1, -1, 2, -2, ... */
      double t = 1.0 + (double)k / 16.0;
      uint16_t s16 = orc_double_to_half_rne(a / (o * t));
      if ((s16 & 0x7FFF) == 0x7C00) s16 = 0x7BFF;
      double s = orc_half_to_double(s16);
      if (s == 0.0) continue;
      int dup = 0;
      for (int n = 0; n < nseen; ++n) dup |= seen[n] == s16;
      if (dup) continue;
      seen[nseen++] = s16;
      codes_for_scale(fmt, w, s, c);
      double err = block_error(fmt, w, imp, c, s);
      if (!have || err < best) {
        have = 1;
        best = err;
        best_bits = s16;
        memcpy(best_c, c, sizeof c);
      }
    }
  }
  if (have) pack_one(fmt, best_c, best_bits, blk);
}

void orc_pack_weighted(int fmt, const float *w, const float *imp, int rows,
                       int cols, uint8_t *out) {
  int bb = orc_block_bytes(fmt);
  int nb = cols / 32;
  for (int r = 0; r < rows; ++r)
    for (int b = 0; b < nb; ++b)
      quantize_block_weighted(fmt, w + (size_t)r * cols + 32 * b, imp + 32 * b,
                              out + ((size_t)r * nb + b) * bb);
}

/* ------------------------------------------------------------------ router */

void orc_router_scores(const double *x, int q, int d, const float *wr, int E,
                       double *s) {
  for (int c = 0; c < q; ++c)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i)
        acc += (double)wr[(size_t)e * d + i] * x[(size_t)c * d + i];
      s[(size_t)c * E + e] = acc;
    }
}

/* qsort has no context argument; one pointer per calling thread */
static _Thread_local const double *g_sort_scores;

static int by_score_desc_then_index(const void *pa, const void *pb) {
  int a = *(const int *)pa, b = *(const int *)pb;
  double sa = g_sort_scores[a], sb = g_sort_scores[b];
  if (sa > sb) return -1;
  if (sa < sb) return 1;
  return (a > b) - (a < b);
}

void orc_topk(const double *s, int E, int k, int32_t *ids) {
  /* [P2] "Lucebox 的优化三板斧": routing selects experts with TOP-K/ARGSORT;
   * [P5] "MoE 专家并行": 6 of 256 routed experts per layer.  Ties go to the
   * lower index. */
  int *order = (int *)malloc(sizeof(int) * (size_t)E);
  for (int e = 0; e < E; ++e) order[e] = e;
  g_sort_scores = s;
  qsort(order, (size_t)E, sizeof(int), by_score_desc_then_index);
  for (int j = 0; j < k; ++j) ids[j] = order[j];
  free(order);
}

void orc_gating(const double *s, const int32_t *ids, int k,
                double routed_scale, double *w) {
  double s0 = s[ids[0]], z = 0.0;
  for (int j = 0; j < k; ++j) z += exp(s[ids[j]] - s0);
  for (int j = 0; j < k; ++j) w[j] = exp(s[ids[j]] - s0) / z * routed_scale;
}

/* ------------------------------------------------------------------ expert */

/* y[rows] = M x for a block-quantized rows x cols matrix, decoding block by
 * block. */
static void qmatvec(int fmt, const uint8_t *m, int rows, int cols,
                    const double *x, double *y) {
  int bb = orc_block_bytes(fmt);
  int nb = cols / 32;
  double w[32];
  for (int r = 0; r < rows; ++r) {
    double acc = 0.0;
    for (int b = 0; b < nb; ++b) {
      orc_decode_block(fmt, m + ((size_t)r * nb + b) * bb, w);
      for (int j = 0; j < 32; ++j) acc += w[j] * x[32 * b + j];
    }
    y[r] = acc;
  }
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

void orc_expert_forward(const uint8_t *gate, int fmt_gate, const uint8_t *up,
                        int fmt_up, const uint8_t *down, int fmt_down, int d,
                        int f, const double *x, double *o) {
  double *g = (double *)malloc(sizeof(double) * (size_t)f);
  double *u = (double *)malloc(sizeof(double) * (size_t)f);
  qmatvec(fmt_gate, gate, f, d, x, g);
  qmatvec(fmt_up, up, f, d, x, u);
  for (int i = 0; i < f; ++i) g[i] = silu(g[i]) * u[i]; /* h, SiLU-gated */
  qmatvec(fmt_down, down, d, f, g, o);
  free(g);
  free(u);
}

void orc_dense_forward(int fmt, const uint8_t *w, int rows, int cols,
                       const void *x, int xtype, int q, float *y) {
  /* [P2] "Lucebox 的优化三板斧": in the q-column verify step each packed
   * dense weight is decoded once and applied to every column; the result is
   * q independent products y_c = W x_c, which is what is computed here
   * (decoding again for every column). */
  double *xc = (double *)malloc(sizeof(double) * (size_t)cols);
  double *yc = (double *)malloc(sizeof(double) * (size_t)rows);
  for (int c = 0; c < q; ++c) {
    if (xtype == 1)
      orc_load_x((const uint16_t *)x + (size_t)c * cols, 1, cols, xc);
    else
      orc_load_x((const float *)x + (size_t)c * cols, 0, cols, xc);
    qmatvec(fmt, w, rows, cols, xc, yc);
    for (int r = 0; r < rows; ++r) y[(size_t)c * rows + r] = (float)yc[r];
  }
  free(xc);
  free(yc);
}

void orc_load_x(const void *x, int xtype, int n, double *out) {
  if (xtype == 1) {
    const uint16_t *b = (const uint16_t *)x;
    for (int i = 0; i < n; ++i) out[i] = orc_bf16_to_double(b[i]);
  } else {
    const float *f = (const float *)x;
    for (int i = 0; i < n; ++i) out[i] = (double)f[i];
  }
}

void orc_layer_forward(int d, int f, int E, int k, double routed_scale,
                       const float *wr, const uint8_t *const *mats,
                       const int *fmts, const void *x, int xtype, int q,
                       float *y, int32_t *ids_out, double *w_out) {
  double *xc = (double *)malloc(sizeof(double) * (size_t)d);
  double *s = (double *)malloc(sizeof(double) * (size_t)E);
  double *o = (double *)malloc(sizeof(double) * (size_t)d);
  double *acc = (double *)malloc(sizeof(double) * (size_t)d);
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
  double *w = (double *)malloc(sizeof(double) * (size_t)k);
  for (int c = 0; c < q; ++c) {
    if (xtype == 1)
      orc_load_x((const uint16_t *)x + (size_t)c * d, 1, d, xc);
    else
      orc_load_x((const float *)x + (size_t)c * d, 0, d, xc);
    orc_router_scores(xc, 1, d, wr, E, s);
    orc_topk(s, E, k, ids);
    orc_gating(s, ids, k, routed_scale, w);
    for (int i = 0; i < d; ++i) acc[i] = 0.0;
    for (int j = 0; j < k; ++j) {
      int e = ids[j];
      orc_expert_forward(mats[3 * e], fmts[3 * e], mats[3 * e + 1],
                         fmts[3 * e + 1], mats[3 * e + 2], fmts[3 * e + 2], d,
                         f, xc, o);
      for (int i = 0; i < d; ++i) acc[i] += w[j] * o[i];
    }
    /* the shared expert is applied to every column with weight 1
     * ([P5] "MoE 专家并行": 256 routed experts, top-6, plus 1 shared) */
    orc_expert_forward(mats[3 * E], fmts[3 * E], mats[3 * E + 1],
                       fmts[3 * E + 1], mats[3 * E + 2], fmts[3 * E + 2], d, f,
                       xc, o);
    for (int i = 0; i < d; ++i) y[(size_t)c * d + i] = (float)(acc[i] + o[i]);
    if (ids_out)
      for (int j = 0; j < k; ++j) ids_out[(size_t)c * k + j] = ids[j];
    if (w_out)
      for (int j = 0; j < k; ++j) w_out[(size_t)c * k + j] = w[j];
  }
  free(xc);
  free(s);
  free(o);
  free(acc);
  free(ids);
  free(w);
}
