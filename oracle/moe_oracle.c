/*
 * moe_oracle.c -- plain, slow CPU oracle of the routed-expert MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h for who may call it and for the
 * source key [tcti], [dpshk], [muninn], [OCP-MX] used below).
 *
 * Written for a reader who checks it by eye: no blocking, no fusion, no
 * reordering beyond what each definition states.  Built with
 * -ffp-contract=off and without fast-math so every fp32 step is a single
 * IEEE operation.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ======================================================================= */
/* Element codecs [OCP-MX; tcti "DeepSeek-V4-Flash的可能性": experts FP4]   */
/* ======================================================================= */

/* E2M1: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0.
 * exponent 0 is subnormal: 0.5 * m.  Code 0x8 is -0. */
double orc_e2m1_value(unsigned code4) {
  unsigned s = (code4 >> 3) & 1u, e = (code4 >> 1) & 3u, m = code4 & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -mag : mag;
}

/* UE8M0: an unsigned biased exponent, value 2^(b-127); 0xFF is NaN. */
double orc_ue8m0_value(unsigned byte) {
  if ((byte & 0xFFu) == 0xFFu) return NAN;
  return ldexp(1.0, (int)(byte & 0xFFu) - 127);
}

/* E4M3 ("FN"): sign bit 7, exponent bits 6-3 (bias 7), mantissa bits 2-0.
 * exponent 0 is subnormal: 2^-6 * m/8.  S.1111.111 is NaN; no infinities;
 * largest finite value 1.75 * 2^8 = 448. */
double orc_e4m3_value(unsigned byte) {
  unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  if (e == 15u && m == 7u) return NAN;
  double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

/* bfloat16 = the upper 16 bits of an IEEE binary32. */
double orc_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static float bf16_to_f32(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a non-negative real r to the nearest integer, ties to even. */
static double round_half_even(double r) {
  double fl = floor(r);
  double d = r - fl;
  if (d > 0.5) return fl + 1.0;
  if (d < 0.5) return fl;
  return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* fp32 -> E4M3 code: round to nearest, ties to the even mantissa,
 * saturating to +-448 (reading: no value of the layer may become NaN),
 * sign kept (so -0 and tiny negatives give 0x80). */
unsigned orc_e4m3_encode(float v) {
  unsigned sign = signbit(v) ? 0x80u : 0x00u;
  double a = fabs((double)v);
  if (isnan(v)) return 0x7Fu | sign;
  if (a >= 448.0) return 0x7Eu | sign;
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9; m = 8 is the smallest normal,
     * whose code is also 8 (exponent field 1, mantissa 0). */
    double m = round_half_even(a * 512.0);
    return (unsigned)m | sign;
  }
  int ex;
  double f = frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;           /* a = (2f) * 2^e, 2f in [1, 2) */
  double mm = round_half_even((2.0 * f - 1.0) * 8.0);
  if (mm == 8.0) {
    mm = 0.0;
    e += 1;
  }
  unsigned code = ((unsigned)(e + 7) << 3) | (unsigned)mm;
  if (code > 0x7Eu) code = 0x7Eu; /* unreachable below 448, kept as a guard */
  return code | sign;
}

void orc_e4m3_encode_n(const float* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e4m3_encode(v[i]);
}

/* ======================================================================= */
/* S3: act_quant [tcti "补齐软件栈缺失": activation quantisation feeding the */
/* FP8/FP4 linears; dpshk "核心实现四": quantised once, shared by gate and  */
/* up].  Per row, per block of 128: a = max|x| (exact), s = fl32(a / 448),  */
/* q_i = E4M3(fl32(x_i / s)) with IEEE fp32 division.  a = 0 -> s = 0 and   */
/* every code 0x00 (reading for the silent zero-block case).               */
/* ======================================================================= */

void orc_act_quant_f32(const float* x, int64_t rows, int32_t cols, uint8_t* q, float* s) {
  const int32_t nb = cols / 128;
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t b = 0; b < nb; ++b) {
      const float* xb = x + r * cols + (int64_t)b * 128;
      uint8_t* qb = q + r * cols + (int64_t)b * 128;
      float amax = 0.0f;
      for (int i = 0; i < 128; ++i) {
        float a = fabsf(xb[i]);
        if (a > amax) amax = a;
      }
      float sc = amax / 448.0f;
      s[r * nb + b] = sc;
      for (int i = 0; i < 128; ++i) {
        if (amax == 0.0f) {
          qb[i] = 0x00;
        } else {
          float t = xb[i] / sc;
          qb[i] = (uint8_t)orc_e4m3_encode(t);
        }
      }
    }
  }
}

void orc_act_quant_bf16(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* q, float* s) {
  float* xf = (float*)malloc(sizeof(float) * (size_t)cols);
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t i = 0; i < cols; ++i) xf[i] = bf16_to_f32(x[r * cols + i]);
    orc_act_quant_f32(xf, 1, cols, q + r * cols, s + r * (cols / 128));
  }
  free(xf);
}

/* ======================================================================= */
/* S1: router logits [dpshk "核心实现一": the router runs first and picks   */
/* the token's experts].  z[t][e] = sum_h x[t][h] * Wr[h][e] in fp32, in    */
/* one fixed order (reading; dpshk "核心实现四" keeps each row's            */
/* accumulation order fixed, but the pages do not say which order): chunk   */
/* partials P_c over h = 64c..64c+63, each a chain of multiply-adds from +0 */
/* in ascending h (a bf16 x bf16 product is exact in fp32, so fusing the    */
/* multiply and the add changes nothing); then one chain over the partials  */
/* in ascending c: z = ((P_0 + P_1) + P_2) + ... + P_{H/64-1}.              */
/* ======================================================================= */

void orc_router_logits(const uint16_t* x, const uint16_t* wr, int32_t T, int32_t H, int32_t E,
                       float* z) {
  const int32_t nc = H / 64;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int32_t c = 0; c < nc; ++c) {
        float p = 0.0f;
        for (int32_t h = 64 * c; h < 64 * c + 64; ++h) {
          p = fmaf(bf16_to_f32(x[(int64_t)t * H + h]), bf16_to_f32(wr[(int64_t)h * E + e]), p);
        }
        acc = (c == 0) ? p : acc + p;
      }
      z[(int64_t)t * E + e] = acc;
    }
  }
}

/* ======================================================================= */
/* S2: top-k + renormalisation [muninn: 6 of 256 experts per token; tcti   */
/* "DeepSeek-V4-Flash的可能性": top-6].  Experts ordered by (z descending,  */
/* id ascending); the first k are kept in that rank order.  Scores are     */
/* sigmoids (fp64 here), w_j = s_j / sum_{i<k} s_i.  Selection is on the    */
/* fp32 logit (the sigmoid is increasing, so the order is the same).       */
/* The pages define no order for a NaN logit (reading: it ranks below every */
/* number, -inf included, lower id first among NaNs); -0 and +0 are equal.  */
/* ======================================================================= */

/* Logit a ranks strictly before logit b (ties leave the lower id first). */
static int ranks_before(float a, float b) {
  if (isnan(a)) return 0;
  if (isnan(b)) return 1;
  return a > b;
}

/* Weights of a given selection: s_j = sigmoid(z[t][ids_j]) in fp64 and
 * w_j = s_j / sum_{i<k} s_i, slots in the order given. */
void orc_topk_weights(const float* z, int32_t T, int32_t E, int32_t k, const int32_t* ids,
                      double* w) {
  for (int32_t t = 0; t < T; ++t) {
    const float* zt = z + (int64_t)t * E;
    double sum = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      double zz = (double)zt[ids[(int64_t)t * k + j]];
      double sg = 1.0 / (1.0 + exp(-zz));
      w[(int64_t)t * k + j] = sg;
      sum += sg;
    }
    for (int32_t j = 0; j < k; ++j) w[(int64_t)t * k + j] /= sum;
  }
}

void orc_topk(const float* z, int32_t T, int32_t E, int32_t k, int32_t* ids, double* w) {
  char* taken = (char*)malloc((size_t)E);
  for (int32_t t = 0; t < T; ++t) {
    const float* zt = z + (int64_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || ranks_before(zt[e], zt[best])) best = e; /* ties keep the lower id */
      }
      taken[best] = 1;
      ids[(int64_t)t * k + j] = best;
    }
  }
  free(taken);
  orc_topk_weights(z, T, E, k, ids, w);
}

/* ======================================================================= */
/* S4: permutation [dpshk "核心实现三": each expert's weights are read once */
/* for all of the tokens routed to it].  A stable counting sort of the T*k */
/* (t, j) pairs by expert, tokens ascending inside each expert; then the   */
/* shared-expert group (slot E) holding every token in order.             */
/*   offsets[E+2]: group g occupies rows offsets[g] .. offsets[g+1]-1       */
/*   row_token[r]: the token of row r                                      */
/*   row_of[t][j]: the row of (t, slot j); row_of[t][k] = the shared row    */
/* An id outside [0, E) is dropped: row_of = -1.  Returns the number of    */
/* dropped pairs.                                                          */
/* ======================================================================= */

int orc_permute(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t* offsets,
                int32_t* row_token, int32_t* row_of) {
  int dropped = 0;
  int32_t* count = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
  for (int64_t p = 0; p < (int64_t)T * k; ++p) {
    int32_t e = ids[p];
    if (e >= 0 && e < E) count[e]++;
  }
  count[E] = T;
  offsets[0] = 0;
  for (int32_t g = 0; g <= E; ++g) offsets[g + 1] = offsets[g] + count[g];
  int32_t* fill = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = ids[(int64_t)t * k + j];
      if (e < 0 || e >= E) {
        row_of[(int64_t)t * (k + 1) + j] = -1;
        dropped++;
        continue;
      }
      int32_t r = offsets[e] + fill[e]++;
      row_token[r] = t;
      row_of[(int64_t)t * (k + 1) + j] = r;
    }
    int32_t rs = offsets[E] + t;
    row_token[rs] = t;
    row_of[(int64_t)t * (k + 1) + k] = rs;
  }
  /* rows left unfilled by dropped pairs (none: counts skip them) */
  free(fill);
  free(count);
  return dropped;
}

/* ======================================================================= */
/* S5/S6: one expert [tcti "补齐软件栈缺失": fp4_gemm = FP8-quantised act x */
/* FP4 packed weight, fp8_gemm = FP8 x FP8; dpshk "核心实现四": weights are */
/* dequantised inside the product, never expanded first].                  */
/* ======================================================================= */

/* Dequantised weight element: mat 0 = gate [I][H], 1 = up [I][H],
 * 2 = down [H][I]; (row, col) = (out, in). */
double orc_weight(const orc_weights* w, int mat, int32_t e, int32_t row, int32_t col) {
  const int32_t rows = (mat == 2) ? w->H : w->I;
  const int32_t cols = (mat == 2) ? w->I : w->H;
  const uint8_t* q = (mat == 0) ? w->gate_q : (mat == 1) ? w->up_q : w->down_q;
  const void* s = (mat == 0) ? w->gate_s : (mat == 1) ? w->up_s : w->down_s;
  if (w->format == ORC_FMT_FP4) {
    int64_t qi = ((int64_t)e * rows + row) * (cols / 2) + col / 2;
    unsigned byte = q[qi];
    unsigned nib = (col % 2 == 0) ? (byte & 0xFu) : (byte >> 4);
    int64_t si = ((int64_t)e * rows + row) * (cols / 32) + col / 32;
    unsigned sb = ((const uint8_t*)s)[si];
    return orc_e2m1_value(nib) * orc_ue8m0_value(sb);
  } else {
    int64_t qi = ((int64_t)e * rows + row) * cols + col;
    int64_t si = ((int64_t)e * (rows / 128) + row / 128) * (cols / 128) + col / 128;
    return orc_e4m3_value(q[qi]) * (double)((const float*)s)[si];
  }
}

/* g_n = sum_kb xs[kb] * sum_{i in kb} E4M3(xq_i) * Wg[e][n][i], u likewise;
 * fp64 throughout.  Gate and up read the same quantised row. */
void orc_gate_up(const orc_weights* w, int32_t e, const uint8_t* xq, const float* xs, double* g,
                 double* u) {
  const int32_t H = w->H, I = w->I;
  for (int32_t n = 0; n < I; ++n) {
    double gs = 0.0, us = 0.0;
    for (int32_t kb = 0; kb < H / 128; ++kb) {
      double gb = 0.0, ub = 0.0;
      for (int32_t i = 128 * kb; i < 128 * kb + 128; ++i) {
        double a = orc_e4m3_value(xq[i]);
        gb += a * orc_weight(w, 0, e, n, i);
        ub += a * orc_weight(w, 1, e, n, i);
      }
      gs += (double)xs[kb] * gb;
      us += (double)xs[kb] * ub;
    }
    g[n] = gs;
    u[n] = us;
  }
}

/* SwiGLU (workload definition: silu(gate) * up, no clamp): h = fl32(silu(g) * u),
 * silu(v) = v / (1 + e^-v) in fp64. */
void orc_swiglu(const double* g, const double* u, int32_t n, float* h) {
  for (int32_t i = 0; i < n; ++i) {
    double sv = g[i] / (1.0 + exp(-g[i]));
    h[i] = (float)(sv * u[i]);
  }
}

/* y_m = sum_kb hs[kb] * sum_{n in kb} E4M3(hq_n) * Wd[e][m][n], fp64. */
void orc_down(const orc_weights* w, int32_t e, const uint8_t* hq, const float* hs, double* y) {
  const int32_t H = w->H, I = w->I;
  for (int32_t m = 0; m < H; ++m) {
    double acc = 0.0;
    for (int32_t kb = 0; kb < I / 128; ++kb) {
      double b = 0.0;
      for (int32_t n = 128 * kb; n < 128 * kb + 128; ++n) {
        b += orc_e4m3_value(hq[n]) * orc_weight(w, 2, e, m, n);
      }
      acc += (double)hs[kb] * b;
    }
    y[m] = acc;
  }
}

/* One routed row through expert e: gate+up, SwiGLU, requantise h to E4M3
 * per 128 exactly as S3 does (reading: every FP4/FP8 linear takes an
 * FP8-quantised activation), then down.  h, hq, hs, y are outputs. */
void orc_expert_row(const orc_weights* w, int32_t e, const uint8_t* xq, const float* xs, float* h,
                    uint8_t* hq, float* hs, double* y) {
  const int32_t I = w->I;
  double* g = (double*)malloc(sizeof(double) * (size_t)I);
  double* u = (double*)malloc(sizeof(double) * (size_t)I);
  orc_gate_up(w, e, xq, xs, g, u);
  orc_swiglu(g, u, I, h);
  orc_act_quant_f32(h, 1, I, hq, hs);
  orc_down(w, e, hq, hs, y);
  free(g);
  free(u);
}

/* ======================================================================= */
/* Whole layer for a list of tokens (all T when tokens == NULL):          */
/*   out[t] = y_shared + sum_{j<k} w_j * y_{e_j}   (fp64, this order)       */
/* [tcti "DeepSeek-V4-Flash的可能性": the shared expert sits beside the     */
/* routed ones; reading: added with weight 1, gate weights applied after   */
/* down].  ids_in/w_in (nullable) inject routing; otherwise the router of  */
/* S1/S2 runs on x.  out is [n_tokens][H].  Returns 0, or -1 on bad ids.   */
/* ======================================================================= */

int orc_moe_forward(const orc_weights* w, const uint16_t* wr, const uint16_t* x, int32_t T,
                    int32_t k, const int32_t* ids_in, const float* w_in, const int32_t* tokens,
                    int32_t n_tokens, double* out, int32_t n_threads) {
  const int32_t H = w->H, I = w->I, E = w->E;
  int bad = 0;
  if (tokens == NULL) n_tokens = T;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int32_t it = 0; it < n_tokens; ++it) {
    const int32_t t = tokens ? tokens[it] : it;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    double* wt = (double*)malloc(sizeof(double) * (size_t)k);
    if (ids_in) {
      for (int32_t j = 0; j < k; ++j) {
        ids[j] = ids_in[(int64_t)t * k + j];
        wt[j] = (double)w_in[(int64_t)t * k + j];
      }
    } else {
      float* z = (float*)malloc(sizeof(float) * (size_t)E);
      orc_router_logits(x + (int64_t)t * H, wr, 1, H, E, z);
      orc_topk(z, 1, E, k, ids, wt);
      free(z);
    }
    uint8_t* xq = (uint8_t*)malloc((size_t)H);
    float* xs = (float*)malloc(sizeof(float) * (size_t)(H / 128));
    orc_act_quant_bf16(x + (int64_t)t * H, 1, H, xq, xs);
    float* h = (float*)malloc(sizeof(float) * (size_t)I);
    uint8_t* hq = (uint8_t*)malloc((size_t)I);
    float* hs = (float*)malloc(sizeof(float) * (size_t)(I / 128));
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    double* o = out + (int64_t)it * H;
    orc_expert_row(w, E, xq, xs, h, hq, hs, y);
    for (int32_t m = 0; m < H; ++m) o[m] = y[m];
    for (int32_t j = 0; j < k; ++j) {
      if (ids[j] < 0 || ids[j] >= E) {
        bad = 1;
        continue;
      }
      orc_expert_row(w, ids[j], xq, xs, h, hq, hs, y);
      for (int32_t m = 0; m < H; ++m) o[m] += wt[j] * y[m];
    }
    free(ids);
    free(wt);
    free(xq);
    free(xs);
    free(h);
    free(hq);
    free(hs);
    free(y);
  }
  return bad ? -1 : 0;
}
