/*
 * moe_oracle.c -- plain, slow, double-precision CPU reference of the routed
 * mixture-of-experts FFN step of a 4-bit MoE decoder.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, import or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * Sources (the three diskformer engine pages):
 *   [FLINT] diskformer 0.5.4 -> 0.6.4, package/engines/flint_moe_ssd.js
 *   [LING]  diskformer 0.5.3 -> 0.6.4, package/engines/ling_moe_ssd.js
 *   [LFM]   diskformer 0.5.4 -> 0.6.6, package/engines/lfm2_moe_ssd.js
 *
 * Every value is computed in IEEE double.  The only single-precision steps are
 * the routing DECISIONS (which experts and which groups win): the pages score
 * and compare in f32, so the oracle rounds its double logit to f32 once, forms
 * the f32 score sigmoid(l)+bias from it and compares f32 values with the pages'
 * tie rules.  The routing WEIGHTS are values and stay in double.
 *
 * Parity pins: every function here is pinned by tests under tests/ against
 * closed forms, brute force or an independent library routine; none is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MO_Q4_0 0
#define MO_Q4_1 1
#define MO_Q8_0 2

/* Clamp on the sum of the picked sigmoids: 2^-14 in both router kernels
 * ([LFM] TOPK_SIG_BODY; [LING] routeLing). */
#define MO_WSUM_MIN 6.103515625e-5

typedef struct {
  int32_t hidden, n_experts, top_k;
  int32_t n_groups, groups_used;
  int32_t expert_ff, shared_ff;
  int32_t qtype;
  double weights_scale;
  double wsum_min;
  double swiglu_limit;         /* routed experts' SwiGLU clamp L; 0 = none */
  double swiglu_limit_shared;  /* the shared expert's; 0 = none */
  double norm_eps;             /* RMSNorm epsilon, used when a norm weight is given */
} mo_cfg;

/* ---------------------------------------------------------------- f16 ---- */

/* IEEE binary16 -> double, exact, subnormals included (1 sign bit, 5 exponent
 * bits with bias 15, 10 fraction bits).  Inf/NaN map to inf/nan. */
double mo_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 31;
  int fr = h & 1023;
  double v;
  if (ex == 0)
    v = ldexp((double)fr, -24); /* subnormal: fr * 2^-14 * 2^-10 */
  else if (ex == 31)
    v = fr ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + fr), ex - 25); /* (1 + fr/1024) * 2^(ex-15) */
  return sign ? -v : v;
}

/* --------------------------------------------------------- Q4 blocks ---- */

int mo_block_bytes(int qtype) { return qtype == MO_Q4_1 ? 20 : (qtype == MO_Q8_0 ? 34 : 18); }

/* One block of 32 weights -> 32 doubles.
 * Q4_1 ([FLINT] file header comment and the Q41DOT comment): 20 bytes, f16 d,
 * f16 m, then 16 bytes of nibbles; byte i holds element i in its low nibble and
 * element i+16 in its high nibble; value = d*q + m.
 * Q4_0: 18 bytes, f16 d then the same 16 nibble bytes; value = d*(q-8).  The
 * formula and the 18-byte block are the GGUF definition named for the
 * decoder; the pages only show Q4_0's split into a nibble plane and an f16
 * scale plane ([LFM] planLayoutLfm2Moe), with the nibble bytes copied
 * unchanged, so the same nibble order is read.
 * Q8_0 ([LFM] planLayoutLfm2Moe: an int8 plane of 32 bytes per 32 values and
 * the same f16 scale plane; Q8_BLOCK): 34 bytes, f16 d then 32 signed bytes,
 * element i = byte i; value = d*q. */
void mo_dequant_block(int qtype, const uint8_t *blk, double *out) {
  uint16_t dbits = (uint16_t)(blk[0] | (blk[1] << 8));
  double d = mo_f16(dbits);
  if (qtype == MO_Q8_0) {
    for (int i = 0; i < 32; i++) out[i] = d * (double)(int8_t)blk[2 + i];
    return;
  }
  const uint8_t *qs;
  double m = 0.0;
  if (qtype == MO_Q4_1) {
    uint16_t mbits = (uint16_t)(blk[2] | (blk[3] << 8));
    m = mo_f16(mbits);
    qs = blk + 4;
  } else {
    qs = blk + 2;
  }
  for (int i = 0; i < 16; i++) {
    int lo = qs[i] & 15, hi = qs[i] >> 4;
    if (qtype == MO_Q4_1) {
      out[i] = d * lo + m;
      out[i + 16] = d * hi + m;
    } else {
      out[i] = d * (lo - 8);
      out[i + 16] = d * (hi - 8);
    }
  }
}

/* A row of n = 32*nb weights stored as nb consecutive blocks. */
void mo_dequant_row(int qtype, const uint8_t *row, int32_t nb, double *out) {
  int bs = mo_block_bytes(qtype);
  for (int b = 0; b < nb; b++) mo_dequant_block(qtype, row + (size_t)b * bs, out + 32 * b);
}

/* sum_h deq(row)[h] * x[h], dequantise first, then a plain ascending sum. */
double mo_row_dot(int qtype, const uint8_t *row, int32_t nb, const double *x) {
  double w[32], acc = 0.0;
  int bs = mo_block_bytes(qtype);
  for (int b = 0; b < nb; b++) {
    mo_dequant_block(qtype, row + (size_t)b * bs, w);
    for (int i = 0; i < 32; i++) acc += w[i] * x[32 * b + i];
  }
  return acc;
}

/* ------------------------------------------------------------ router ---- */

/* Router logits l[e] = sum_h W[e][h] x[h]; W is the F32 ffn_gate_inp matrix,
 * E rows of H ([LFM] and [FLINT]: matmulF32 with uniform [E, H]). */
void mo_router_logits(const float *W, const float *x, int32_t E, int32_t H, double *logits) {
  for (int e = 0; e < E; e++) {
    double acc = 0.0;
    for (int h = 0; h < H; h++) acc += (double)W[(size_t)e * H + h] * (double)x[h];
    logits[e] = acc;
  }
}

double mo_sigmoid(double l) { return 1.0 / (1.0 + exp(-l)); }

/* f32 selection score of one expert from its f32 logit: p rounded to f32, then
 * the f32 sum p + bias (the bias only steers selection: [LFM] router comment,
 * [LING] routeLing). */
static float score32(float l32, const float *bias, int e) {
  float p32 = (float)mo_sigmoid((double)l32);
  float b = bias ? bias[e] : 0.0f;
  volatile float s = p32 + b; /* one f32 rounding, as the pages' kernels */
  return s;
}

/* Group-limited selection ([LING] routeLing and its file header: groups are
 * ranked by the sum of their two best selection scores and only the
 * groups_used best groups stay selectable).  Written from that rule:
 *   gscore[g] = f32 sum of the two largest values of group g's scores (a
 *               sorted copy; an equal value counts as the second);
 *   the kept groups are the first groups_used of the groups ordered by
 *   (gscore descending, group index ascending), i.e. the lower index wins a
 *   tie.
 * keep[g] = 1 for kept groups. */
static int desc_f32(const void *a, const void *b) {
  float x = *(const float *)a, y = *(const float *)b;
  return (x < y) - (x > y);
}
static const float *g_order_scores; /* (qsort has no context argument) */
static int by_score_then_index(const void *a, const void *b) {
  int i = *(const int *)a, j = *(const int *)b;
  float x = g_order_scores[i], y = g_order_scores[j];
  if (x != y) return x > y ? -1 : 1;
  return (i > j) - (i < j);
}
void mo_group_keep(const float *s32, int32_t E, int32_t G, int32_t Gu, int32_t *keep, float *gscore) {
  int P = E / G;
  float *copy = (float *)malloc(sizeof(float) * (size_t)P);
  int *order = (int *)malloc(sizeof(int) * (size_t)G);
  for (int g = 0; g < G; g++) {
    memcpy(copy, s32 + (size_t)g * P, sizeof(float) * (size_t)P);
    qsort(copy, (size_t)P, sizeof(float), desc_f32);
    volatile float sum = copy[0] + copy[1]; /* one f32 rounding, as the page's kernel */
    gscore[g] = sum;
    keep[g] = 0;
    order[g] = g;
  }
  g_order_scores = gscore;
  qsort(order, (size_t)G, sizeof(int), by_score_then_index);
  for (int r = 0; r < Gu; r++) keep[order[r]] = 1;
  free(copy);
  free(order);
}

/* Top-k over the allowed experts: k rounds, each picking the largest f32
 * score not yet picked, lowest index on ties; picks are reported in pick order
 * ([LFM] TOPK_SIG_BODY, [LING] routeLing). */
void mo_topk(const float *s32, const int32_t *allowed, int32_t E, int32_t k, int32_t *ids) {
  char *taken = (char *)calloc((size_t)E, 1);
  for (int j = 0; j < k; j++) {
    int best = -1;
    float bv = -INFINITY;
    for (int e = 0; e < E; e++) {
      if (taken[e] || (allowed && !allowed[e])) continue;
      if (best < 0 || s32[e] > bv) {
        bv = s32[e];
        best = e;
      }
    }
    ids[j] = best;
    if (best >= 0) taken[best] = 1;
  }
  free(taken);
}

/* Routing of one token.
 *   logit32[E]: the f32 logits that drive the decisions;
 *   logit64[E]: the same logits in double (NULL -> use logit32) for weights.
 * Weights: w_j = p_j / max(sum_j p_j, wsum_min) * scale with p = sigmoid of the
 * logit, no bias; the sum runs in pick order ([LFM] TOPK_SIG_BODY, [LING]
 * routeLing).  Outputs ids[k] and w[k].  Returns 0, or -1 on a config that
 * leaves fewer than k selectable experts. */
int mo_route(const mo_cfg *c, const float *logit32, const double *logit64, const float *bias,
             int32_t *ids, double *w) {
  int E = c->n_experts, k = c->top_k, G = c->n_groups > 0 ? c->n_groups : 1;
  int Gu = c->groups_used > 0 ? c->groups_used : G;
  if (E <= 0 || k <= 0 || k > 32 || E > 512) return -1;
  float *s32 = (float *)malloc(sizeof(float) * (size_t)E);
  int32_t *allowed = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  for (int e = 0; e < E; e++) {
    s32[e] = score32(logit32[e], bias, e);
    allowed[e] = 1;
  }
  if (Gu < G) {
    int32_t keep[512];
    float gs[512];
    int P = E / G;
    mo_group_keep(s32, E, G, Gu, keep, gs);
    for (int e = 0; e < E; e++) allowed[e] = keep[e / P];
  }
  int n_allowed = 0;
  for (int e = 0; e < E; e++) n_allowed += allowed[e];
  if (n_allowed < k) {
    free(s32);
    free(allowed);
    return -1;
  }
  mo_topk(s32, allowed, E, k, ids);
  double S = 0.0;
  double p[32];
  for (int j = 0; j < k; j++) {
    double l = logit64 ? logit64[ids[j]] : (double)logit32[ids[j]];
    p[j] = mo_sigmoid(l);
    S += p[j];
  }
  double den = S > c->wsum_min ? S : c->wsum_min;
  for (int j = 0; j < k; j++) w[j] = p[j] / den * c->weights_scale;
  free(s32);
  free(allowed);
  return 0;
}

/* ----------------------------------------------------------- experts ---- */

/* SwiGLU activation silu(g)*u with silu(g) = g / (1 + e^-g) ([LING] swiglu;
 * [LFM] siluSplitB).  With a clamp L > 0 ([LING] swiglu kernel and the FFN
 * line of its file header: some layers clamp the SwiGLU), u is clamped to
 * [-L, L] and silu(g) is capped at L from above only; L = 0 is no clamp. */
double mo_swiglu(double g, double u, double L) {
  double sg = g / (1.0 + exp(-g));
  if (L > 0.0) {
    u = u < -L ? -L : (u > L ? L : u);
    sg = sg > L ? L : sg;
  }
  return sg * u;
}

/* One SwiGLU expert on one token (double throughout):
 *   g_f = sum_h Wg[f][h] x_h,  u_f = sum_h Wu[f][h] x_h,  a_f = silu(g_f) u_f,
 *   y_h = sum_f Wd[h][f] a_f  (a_f clamped as in mo_swiglu when limit > 0).
 * gate/up hold F rows of H/32 blocks, down holds H rows of F/32 blocks (GGUF
 * ffn_{gate,up}_exps [H, F] and ffn_down_exps [F, H] per expert, rows of the
 * first dimension). */
void mo_expert_ffn(int qtype, const uint8_t *gate, const uint8_t *up, const uint8_t *down,
                   int32_t H, int32_t F, double limit, const double *x, double *y) {
  int bs = mo_block_bytes(qtype);
  int nbH = H / 32, nbF = F / 32;
  double *a = (double *)malloc(sizeof(double) * (size_t)F);
  for (int f = 0; f < F; f++) {
    double g = mo_row_dot(qtype, gate + (size_t)f * nbH * bs, nbH, x);
    double u = mo_row_dot(qtype, up + (size_t)f * nbH * bs, nbH, x);
    a[f] = mo_swiglu(g, u, limit);
  }
  for (int h = 0; h < H; h++) y[h] = mo_row_dot(qtype, down + (size_t)h * nbF * bs, nbF, a);
  free(a);
}

/* ------------------------------------------------------------- layer ---- */

/* Pre-FFN RMSNorm of one token: xn_h = f32(x_h * s * g_h) with
 * s = 1 / sqrt(mean_h(x_h^2) + eps) in double, h ascending ([FLINT], [LFM]
 * file headers: the FFN input is rms_norm(x) * ffn_norm; the Ling page's
 * normalising kernels divide by sqrt(sum(x^2) / n + eps) and then multiply by
 * the weight; eps is the model's attention.layer_norm_rms_epsilon).  The
 * result is rounded once to f32, as the pages keep the normalised input in an
 * f32 buffer. */
void mo_rmsnorm(const float *x, const float *g, int32_t H, double eps, float *xn) {
  double ss = 0.0;
  for (int h = 0; h < H; h++) ss += (double)x[h] * (double)x[h];
  const double s = 1.0 / sqrt(ss / (double)H + eps);
  for (int h = 0; h < H; h++) xn[h] = (float)((double)x[h] * s * (double)g[h]);
}

/* The whole MoE FFN step for T tokens:
 *   out[t][h] = resid[t][h] + sum_j w_tj * FFN_{id_tj}(x_t)[h] + FFN_shared(x_t)[h]
 * ([LING] moeAccum; [LFM] moeAccumB and the shared-expert addInPlace; the
 * shared expert is always on, ungated, weight 1).
 *   gate_exps/up_exps: E experts of F rows x H/32 blocks, down_exps: E experts
 *   of H rows x F/32 blocks, shared tensors likewise with SF (NULL if SF = 0).
 *   logits_in: NULL -> logits from the router weights in double; else [T][E]
 *   f32 logits used for both decisions and weights.
 * ffn_norm: NULL -> x is the FFN input; else x is the residual stream and
 * the FFN input is mo_rmsnorm(x) with that weight (x may alias resid).
 * A dense SwiGLU FFN layer is E = k = 0: no routing, out = resid +
 * FFN_shared(x) ([FLINT] and [LING] file headers: a dense SwiGLU FFN of 6144
 * on the first two layers; [LFM] likewise with 11776).
 * Outputs out[T][H] (double), ids[T][k], w[T][k].  Returns 0 or -1. */
int mo_layer(const mo_cfg *c, const float *router_w, const float *bias, const uint8_t *gate_exps,
             const uint8_t *up_exps, const uint8_t *down_exps, const uint8_t *gate_sh,
             const uint8_t *up_sh, const uint8_t *down_sh, const float *ffn_norm, const float *x, int32_t T,
             const float *resid, const float *logits_in, double *out, int32_t *ids, double *w) {
  int H = c->hidden, E = c->n_experts, k = c->top_k, F = c->expert_ff, SF = c->shared_ff;
  int bs = mo_block_bytes(c->qtype);
  size_t exp_gu = (size_t)F * (H / 32) * bs, exp_dn = (size_t)H * (F / 32) * bs;
  double *l64 = (double *)malloc(sizeof(double) * (size_t)E);
  float *l32 = (float *)malloc(sizeof(float) * (size_t)E);
  double *xd = (double *)malloc(sizeof(double) * (size_t)H);
  float *xn = (float *)malloc(sizeof(float) * (size_t)H);
  double *y = (double *)malloc(sizeof(double) * (size_t)H);
  int rc = 0;
  for (int t = 0; t < T && rc == 0; t++) {
    const float *xt = x + (size_t)t * H;
    if (ffn_norm) {
      mo_rmsnorm(x + (size_t)t * H, ffn_norm, H, c->norm_eps, xn);
      xt = xn;
    }
    for (int h = 0; h < H; h++) xd[h] = xt[h];
    const double *lv = NULL;
    if (E == 0) {
      /* a dense layer: no router, only the FFN held in the shared tensors */
    } else if (logits_in) {
      for (int e = 0; e < E; e++) l32[e] = logits_in[(size_t)t * E + e];
    } else {
      mo_router_logits(router_w, xt, E, H, l64);
      for (int e = 0; e < E; e++) l32[e] = (float)l64[e];
      lv = l64;
    }
    if (E > 0) {
      rc = mo_route(c, l32, lv, bias, ids + (size_t)t * k, w + (size_t)t * k);
      if (rc) break;
    }
    double *o = out + (size_t)t * H;
    for (int h = 0; h < H; h++) o[h] = resid ? (double)resid[(size_t)t * H + h] : 0.0;
    for (int j = 0; j < k; j++) {
      int e = ids[(size_t)t * k + j];
      mo_expert_ffn(c->qtype, gate_exps + (size_t)e * exp_gu, up_exps + (size_t)e * exp_gu,
                    down_exps + (size_t)e * exp_dn, H, F, c->swiglu_limit, xd, y);
      double wj = w[(size_t)t * k + j];
      for (int h = 0; h < H; h++) o[h] += wj * y[h];
    }
    if (SF > 0 && gate_sh && up_sh && down_sh) {
      mo_expert_ffn(c->qtype, gate_sh, up_sh, down_sh, H, SF, c->swiglu_limit_shared, xd, y);
      for (int h = 0; h < H; h++) o[h] += y[h];
    }
  }
  free(l64);
  free(l32);
  free(xd);
  free(xn);
  free(y);
  return rc;
}

/* ----------------------------------------------------- sort by expert ---- */

/* Stable grouping of the T*k (token, pick) pairs by expert id: pair p = t*k+j
 * has expert ids[p]; perm lists the pairs ordered by (expert, p), so tokens
 * ascend within an expert, and offsets[e]..offsets[e+1] is expert e's range.
 * Definition only: a counting pass and a placement pass in pair order. */
void mo_sort_by_expert(const int32_t *ids, int32_t npairs, int32_t E, int32_t *offsets, int32_t *perm) {
  int32_t *cursor = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
  for (int e = 0; e <= E; e++) offsets[e] = 0;
  for (int p = 0; p < npairs; p++) offsets[ids[p] + 1]++;
  for (int e = 0; e < E; e++) offsets[e + 1] += offsets[e];
  for (int e = 0; e < E; e++) cursor[e] = offsets[e];
  for (int p = 0; p < npairs; p++) perm[cursor[ids[p]]++] = p;
  free(cursor);
}
