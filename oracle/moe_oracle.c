/*
 * Plain CPU oracle for the routed MXFP4 Mixture-of-Experts feed-forward at decode.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link, load or call this file:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no code,
 * header, table or constant with the HIP library; it is written directly from the definitions below.
 *
 * Arithmetic is IEEE fp64 throughout (no fused multiply-add contraction, no fast-math), which makes it
 * an upper-precision reference for a GPU path that accumulates in fp32.
 *
 * What is computed, step by step, and where each step comes from:
 *   - MXFP4 decoding follows the OCP Microscaling Formats (MX) v1.0 specification: an MXFP4 block is
 *     32 E2M1 elements sharing one E8M0 scale. The pages name MXFP4 as the weight format of the routed
 *     expert GEMMs (vllm.cpp PR #52 title and body; b70-optimization-lab "MTP1 Post-Portfolio
 *     Eager-Cycle Profile", Purpose And Identity: "MXFP4 N64 policy") without defining it.
 *   - Router logits: the token's hidden state projected onto one vector per expert. The pages time
 *     only the router's select/normalize kernel (next item) and do not define the projection; the
 *     plainest reading is a dense bf16 matrix W_router[E, H], logits = x . W_router^T.
 *   - Routing: per token, score the experts, select the top k, normalise the selected weights
 *     ("Native router select/normalize" row of the Post-Portfolio Device Attribution table).
 *   - Grouping: the pairs (token, slot) are remapped into per-expert order ("Direct M=2 route remap"
 *     row of the same table).
 *   - Expert FFN: gate and up projections, (clamped) SwiGLU, down projection ("Compact routed MXFP4
 *     GEMM" and "Routed clamp-SwiGLU" rows of the same table; the gate_up fusion discussed in
 *     vllm.cpp PR #52 changes only how the work is launched, not the values).
 *   - Combine: each token's output is the routing-weighted sum of its k expert outputs.
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *   - element kk of a packed row sits in byte kk/2, low nibble for even kk;
 *   - the 32-element scale blocks run along the reduction dimension (H for w13, I for w2);
 *   - w13 holds the I gate rows first, then the I up rows;
 *   - SwiGLU is silu(gate) * up with silu(g) = g / (1 + exp(-g)); the optional clamp limits both gate
 *     and up to [-c, c] before the activation;
 *   - the experts are ranked on the raw logits (both score functions are strictly increasing), ties
 *     going to the lower expert index; renormalisation divides each selected score by the sum of the
 *     selected scores;
 *   - within one expert, pairs keep ascending flat pair order p = t*k + j;
 *   - the routing weight is applied after the down projection, and the sum over j runs in j order;
 *   - the output is rounded once, to nearest-even, to bfloat16.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- scalar formats ------------------------------------------------------------------------- */

/* E2M1 (OCP MX v1.0): bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa. An exponent field
 * of zero is the subnormal 0.m * 2^(1-1). There is no Inf or NaN encoding. */
double oracle_e2m1_value(int code) {
  int sign = (code >> 3) & 1;
  int expo = (code >> 1) & 3;
  int mant = code & 1;
  double mag;
  if (expo == 0)
    mag = 0.5 * (double)mant;
  else
    mag = ldexp(1.0 + 0.5 * (double)mant, expo - 1);
  return sign ? -mag : mag;
}

/* E8M0 (OCP MX v1.0): an unsigned biased exponent, value 2^(byte - 127); 0xFF encodes NaN. */
double oracle_e8m0_value(int byte) {
  if (byte == 255) return NAN;
  return ldexp(1.0, byte - 127);
}

/* bfloat16 bits -> value: the 16 bits are the upper half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a double once to the nearest bfloat16 (ties to even) and return its bits. bfloat16 has
 * binary32's exponent range and 8 significant bits; values past the largest finite bfloat16 after
 * rounding become infinities, tiny values round onto the subnormal grid of spacing 2^-133. */
uint16_t oracle_double_to_bf16(double v) {
  if (isnan(v)) return (uint16_t)0x7FC0;
  if (v == 0.0) return signbit(v) ? (uint16_t)0x8000 : (uint16_t)0x0000;
  double a = fabs(v);
  int e;
  frexp(a, &e); /* a = f * 2^e with f in [0.5, 1) */
  int q = e - 8; /* unit in the last place for 8 significant bits */
  if (q < -133) q = -133;
  double r = ldexp(nearbyint(ldexp(a, -q)), q); /* nearbyint: current mode = ties to even */
  const double max_bf16 = ldexp(255.0, 127 - 7); /* (2 - 2^-7) * 2^127 */
  float f;
  if (r > max_bf16)
    f = INFINITY;
  else
    f = (float)r; /* exact: r has at most 8 significant bits and is in binary32 range */
  if (signbit(v)) f = -f;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* Element (n, kk) of one expert's MXFP4 matrix with K columns: codes packed two per byte along K
 * (row stride K/2 bytes, low nibble = even kk), one E8M0 scale per 32 consecutive elements of a row
 * (row stride K/32 bytes). */
double oracle_mxfp4_element(const uint8_t* q, const uint8_t* s, int K, long n, long kk) {
  uint8_t byte = q[n * (long)(K / 2) + kk / 2];
  int code = (kk & 1) ? (byte >> 4) : (byte & 0xF);
  return oracle_e2m1_value(code) * oracle_e8m0_value(s[n * (long)(K / 32) + kk / 32]);
}

/* ---- activation formats (MX) --------------------------------------------------------------- */

/* E4M3 (the OCP 8-bit floating point format MXFP8 uses, "FN": no infinities): bit 7 sign, bits 6..3
 * exponent with bias 7, bits 2..0 mantissa. An exponent field of zero is the subnormal 0.m * 2^-6;
 * S.1111.111 is NaN; the largest finite magnitude is 1.75 * 2^8 = 448. */
double oracle_e4m3_value(int code) {
  int sign = (code >> 7) & 1;
  int expo = (code >> 3) & 15;
  int mant = code & 7;
  double mag;
  if (expo == 15 && mant == 7) return NAN;
  if (expo == 0)
    mag = ldexp((double)mant / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)mant / 8.0, expo - 7);
  return sign ? -mag : mag;
}

/* The nearest representable magnitude of |v| (ties to even) on a grid with `mbits` mantissa bits,
 * smallest normal exponent emin and largest finite magnitude vmax (saturating there). */
static double round_to_grid(double a, int mbits, int emin, double vmax) {
  int e;
  if (a == 0.0) return 0.0;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int ex = e - 1;
  if (ex < emin) ex = emin; /* subnormal range: the spacing of the smallest binade */
  double ulp = ldexp(1.0, ex - mbits);
  double r = nearbyint(a / ulp) * ulp; /* default rounding: ties to even */
  return r > vmax ? vmax : r;
}

/* E4M3 code nearest to a finite v (ties to even), saturating at +-448. */
int oracle_e4m3_encode(double v) {
  double r = round_to_grid(fabs(v), 3, -6, 448.0);
  int code = 0;
  for (int c = 0; c < 127; ++c)  /* the non-negative codes in increasing value; 127 is NaN */
    if (oracle_e4m3_value(c) == r) code = c;
  return (signbit(v) ? 0x80 : 0) | code;
}

/* E2M1 code nearest to a finite v (ties to even), saturating at +-6. */
int oracle_e2m1_encode(double v) {
  double r = round_to_grid(fabs(v), 1, 0, 6.0);
  int code = 0;
  for (int c = 0; c < 8; ++c)
    if (oracle_e2m1_value(c) == r) code = c;
  return (signbit(v) ? 8 : 0) | code;
}

double oracle_mx_element(int fmt, int code) {
  return fmt == ORACLE_ACT_MXFP8 ? oracle_e4m3_value(code) : oracle_e2m1_value(code);
}

/* One 32-value block quantised to an MX format (OCP MX v1.0, the shared-scale computation): with
 * amax the largest magnitude, the shared exponent is floor(log2(amax)) - emax_elem, where emax_elem
 * is the exponent of the element format's largest normal (8 for E4M3, 2 for E2M1), clamped to the
 * E8M0 range [-127, 127]; each element is v / 2^shared_exp converted to the element format, nearest
 * with ties to even, saturating at its largest finite magnitude. A block of zeros gets the scale
 * byte 0 and zero elements. Returns the E8M0 scale byte; codes[0..31] receive the elements. */
int oracle_mx_quantize_block(const double* v, int fmt, uint8_t* codes) {
  double amax = 0.0;
  for (int i = 0; i < 32; ++i)
    if (fabs(v[i]) > amax) amax = fabs(v[i]);
  if (amax == 0.0) {
    for (int i = 0; i < 32; ++i) codes[i] = 0;
    return 0;
  }
  int e;
  frexp(amax, &e);
  int shared = (e - 1) - (fmt == ORACLE_ACT_MXFP8 ? 8 : 2);
  if (shared < -127) shared = -127;
  if (shared > 127) shared = 127;
  for (int i = 0; i < 32; ++i) {
    double q = ldexp(v[i], -shared); /* exact: a power-of-two scaling */
    codes[i] = (uint8_t)(fmt == ORACLE_ACT_MXFP8 ? oracle_e4m3_encode(q) : oracle_e2m1_encode(q));
  }
  return shared + 127;
}

/* Replace v[0 .. 32*nblocks) by its MX-quantised values (the dequantised blocks). */
static void mx_fake_quantize(double* v, long nblocks, int fmt) {
  uint8_t codes[32];
  for (long b = 0; b < nblocks; ++b) {
    int s = oracle_mx_quantize_block(v + 32 * b, fmt, codes);
    for (int i = 0; i < 32; ++i) v[32 * b + i] = oracle_mx_element(fmt, codes[i]) * oracle_e8m0_value(s);
  }
}

/* ---- routing -------------------------------------------------------------------------------- */

int oracle_route_topk(const float* logits, int T, int E, int k, int score_fn, int renorm,
                      int32_t* topk_ids, double* topk_w) {
  if (T < 0 || E < 1 || k < 1 || k > E) return -2;
  double* score = (double*)malloc(sizeof(double) * (size_t)E);
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  if (!score || !taken) {
    free(score);
    free(taken);
    return -3;
  }
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (long)t * E;
    /* scores: softmax over all E experts, or an independent sigmoid per expert */
    if (score_fn == ORACLE_SCORE_SOFTMAX) {
      double m = -INFINITY;
      for (int e = 0; e < E; ++e)
        if ((double)l[e] > m) m = (double)l[e];
      double z = 0.0;
      for (int e = 0; e < E; ++e) {
        score[e] = exp((double)l[e] - m);
        z += score[e];
      }
      for (int e = 0; e < E; ++e) score[e] /= z;
    } else {
      for (int e = 0; e < E; ++e) score[e] = 1.0 / (1.0 + exp(-(double)l[e]));
    }
    /* selection: k rounds, each taking the untaken expert with the largest logit (lower index on ties) */
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      topk_ids[(long)t * k + j] = best;
    }
    /* weights: the selected scores, divided by their sum when renormalising */
    double sel = 0.0;
    for (int j = 0; j < k; ++j) sel += score[topk_ids[(long)t * k + j]];
    for (int j = 0; j < k; ++j) {
      double sc = score[topk_ids[(long)t * k + j]];
      topk_w[(long)t * k + j] = renorm ? sc / sel : sc;
    }
  }
  free(score);
  free(taken);
  return 0;
}

/* ---- grouping ------------------------------------------------------------------------------- */

int oracle_group_tokens(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                        int32_t* n_active) {
  if (T < 0 || E < 1 || k < 1) return -2;
  long P = (long)T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (long p = 0; p < P; ++p) {
    int e = topk_ids[p];
    if (e < 0 || e >= E) return -2;
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  /* stable placement: pairs are visited in ascending p, each goes to the next free row of its expert */
  int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!next) return -3;
  for (int e = 0; e < E; ++e) next[e] = offsets[e];
  for (long p = 0; p < P; ++p) {
    int r = next[topk_ids[p]]++;
    sorted_pair[r] = (int32_t)p;
    pair_pos[p] = r;
  }
  free(next);
  int na = 0;
  for (int e = 0; e < E; ++e)
    if (counts[e] > 0) active[na++] = e;
  *n_active = na;
  return 0;
}

/* ---- expert feed-forward and combine -------------------------------------------------------- */

int oracle_mxfp4_ffn(const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                     const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                     const uint8_t* w2_s, const int32_t* topk_ids, const double* topk_w,
                     double clamp_limit, int nthreads, double* y_pairs, double* out_ref,
                     uint16_t* out_bf16) {
  return oracle_mxfp4_ffn_act(x_bf16, T, H, I, E, k, w13_q, w13_s, w2_q, w2_s, topk_ids, topk_w, clamp_limit,
                              ORACLE_ACT_NONE, nthreads, y_pairs, NULL, out_ref, out_bf16);
}

/* The FFN with the activations of both GEMMs quantised to an MX format (act_fmt ORACLE_ACT_MXFP8 or
 * ORACLE_ACT_MXFP4; ORACLE_ACT_NONE computes the plain FFN): each token's x is quantised per 32-value
 * block along H before the gate/up projection, and each pair's h, rounded to binary32 first (the
 * precision in which a GPU computes it, so that both take each element's rounding decision from a
 * binary32 value), per 32-value block along I before the down projection. Everything else is as
 * oracle_mxfp4_ffn, in fp64. */
int oracle_mxfp4_ffn_act(const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                         const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                         const uint8_t* w2_s, const int32_t* topk_ids, const double* topk_w,
                         double clamp_limit, int act_fmt, int nthreads, double* y_pairs, double* h_pairs,
                         double* out_ref, uint16_t* out_bf16) {
  if (T < 0 || H < 32 || I < 32 || H % 32 || I % 32 || E < 1 || k < 1) return -2;
  if (act_fmt != ORACLE_ACT_NONE && act_fmt != ORACLE_ACT_MXFP8 && act_fmt != ORACLE_ACT_MXFP4) return -2;
  long P = (long)T * k;
  const long w13_qe = (long)2 * I * (H / 2), w13_se = (long)2 * I * (H / 32);
  const long w2_qe = (long)H * (I / 2), w2_se = (long)H * (I / 32);
  double* y = y_pairs;
  int own_y = 0;
  if (!y) {
    y = (double*)malloc(sizeof(double) * (size_t)(P * H > 0 ? P * H : 1));
    if (!y) return -3;
    own_y = 1;
  }
  int bad = 0;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : bad)
#endif
  for (long p = 0; p < P; ++p) {
    long t = p / k;
    int e = topk_ids[p];
    if (e < 0 || e >= E) {
      bad |= 1;
      continue;
    }
    double* xd = (double*)malloc(sizeof(double) * (size_t)H);
    double* hv = (double*)malloc(sizeof(double) * (size_t)I);
    if (!xd || !hv) {
      free(xd);
      free(hv);
      bad |= 1;
      continue;
    }
    for (int hh = 0; hh < H; ++hh) xd[hh] = oracle_bf16_to_double(x_bf16[t * H + hh]);
    if (act_fmt != ORACLE_ACT_NONE) mx_fake_quantize(xd, H / 32, act_fmt);
    const uint8_t* q13 = w13_q + e * w13_qe;
    const uint8_t* s13 = w13_s + e * w13_se;
    for (int i = 0; i < I; ++i) {
      double g = 0.0, u = 0.0;
      for (int hh = 0; hh < H; ++hh) {
        g += xd[hh] * oracle_mxfp4_element(q13, s13, H, i, hh);
        u += xd[hh] * oracle_mxfp4_element(q13, s13, H, (long)I + i, hh);
      }
      if (clamp_limit > 0.0) {
        g = fmin(fmax(g, -clamp_limit), clamp_limit);
        u = fmin(fmax(u, -clamp_limit), clamp_limit);
      }
      hv[i] = g / (1.0 + exp(-g)) * u;
    }
    if (act_fmt != ORACLE_ACT_NONE)
      for (int i = 0; i < I; ++i) hv[i] = (double)(float)hv[i];
    if (h_pairs)
      for (int i = 0; i < I; ++i) h_pairs[p * (long)I + i] = hv[i];
    if (act_fmt != ORACLE_ACT_NONE)
      mx_fake_quantize(hv, I / 32, act_fmt);
    const uint8_t* q2 = w2_q + e * w2_qe;
    const uint8_t* s2 = w2_s + e * w2_se;
    for (int n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int i = 0; i < I; ++i) acc += hv[i] * oracle_mxfp4_element(q2, s2, I, n, i);
      y[p * H + n] = acc;
    }
    free(xd);
    free(hv);
  }
  if (!bad) {
    for (long t = 0; t < T; ++t) {
      for (int n = 0; n < H; ++n) {
        double acc = 0.0;
        for (int j = 0; j < k; ++j) acc += topk_w[t * k + j] * y[(t * k + j) * H + n];
        if (out_ref) out_ref[t * H + n] = acc;
        if (out_bf16) out_bf16[t * H + n] = oracle_double_to_bf16(acc);
      }
    }
  }
  if (own_y) free(y);
  return bad ? -2 : 0;
}

/* ---- router logits ------------------------------------------------------------------------ */

/* logits[t][e] = sum over h of x[t][h] * w[e][h] for bfloat16 x[T, H] and w[E, H], in fp64 with h
 * ascending (a product of two bfloat16 values is exact in fp64). Tokens are independent, so the
 * thread count changes no result. */
int oracle_router_logits(const uint16_t* x_bf16, const uint16_t* w_bf16, int T, int H, int E,
                         int nthreads, double* logits) {
  if (T < 0 || H < 1 || E < 1 || (T > 0 && (!x_bf16 || !w_bf16 || !logits))) return -2;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#else
  (void)nthreads;
#endif
  for (long t = 0; t < T; ++t) {
    const uint16_t* xr = x_bf16 + t * (long)H;
    for (long e = 0; e < E; ++e) {
      const uint16_t* wr = w_bf16 + e * (long)H;
      double acc = 0.0;
      for (long h = 0; h < H; ++h) acc += oracle_bf16_to_double(xr[h]) * oracle_bf16_to_double(wr[h]);
      logits[t * (long)E + e] = acc;
    }
  }
  return 0;
}

int oracle_num_threads(int nthreads) {
#ifdef _OPENMP
  return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}
