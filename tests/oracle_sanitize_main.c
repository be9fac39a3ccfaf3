/*
 * Drives every function of the C oracle on small inputs so that a build with
 * -fsanitize=address,undefined can catch out-of-bounds accesses, leaks,
 * signed overflow and other undefined behaviour in it (tests only; the
 * library never links the oracle).  Inputs come from a fixed xorshift
 * stream.  Exit status 0 when every call returned its success code and every
 * output is finite; the sanitizers abort on their own findings.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../oracle/moe_oracle.c"

static uint64_t st = 0x9e3779b97f4a7c15ull;
static uint32_t rnd(void) {
  st ^= st << 13;
  st ^= st >> 7;
  st ^= st << 17;
  return (uint32_t)(st >> 32);
}
static float unif(float a, float b) { return a + (b - a) * (float)(rnd() >> 8) / 16777216.0f; }

/* f16 bits of a value of magnitude below 1 (truncated; subnormal below 2^-14) */
static uint16_t f16_bits(float v) {
  int neg = v < 0;
  if (neg) v = -v;
  if (v < 6.103515625e-5f) return (uint16_t)((neg << 15) | (uint16_t)(v * 16777216.0f));
  int e;
  float m = frexpf(v, &e); /* v = m 2^e, m in [0.5, 1) */
  int ex = e - 1 + 15;
  uint16_t frac = (uint16_t)((m * 2.0f - 1.0f) * 1024.0f);
  return (uint16_t)((neg << 15) | (ex << 10) | frac);
}

static uint8_t *blocks(int qtype, size_t n) {
  int bs = mo_block_bytes(qtype);
  uint8_t *b = (uint8_t *)malloc((size_t)bs * n);
  for (size_t i = 0; i < n; i++) {
    uint8_t *p = b + (size_t)bs * i;
    for (int j = 0; j < bs; j++) p[j] = (uint8_t)rnd();
    uint16_t d = f16_bits(unif(0.001f, 0.02f) * (rnd() & 1 ? 1.f : -1.f));
    if (i % 17 == 0) d = (uint16_t)(1 + rnd() % 1023); /* a subnormal scale */
    p[0] = (uint8_t)d;
    p[1] = (uint8_t)(d >> 8);
    if (qtype == MO_Q4_1) {
      uint16_t m = f16_bits(unif(-0.02f, 0.02f));
      p[2] = (uint8_t)m;
      p[3] = (uint8_t)(m >> 8);
    }
  }
  return b;
}
static float *floats(size_t n, float sd) {
  float *f = (float *)malloc(sizeof(float) * n);
  for (size_t i = 0; i < n; i++) f[i] = unif(-1.7f, 1.7f) * sd;
  return f;
}

static int all_finite(const double *v, size_t n) {
  for (size_t i = 0; i < n; i++)
    if (!isfinite(v[i])) return 0;
  return 1;
}

static int run_layer(int H, int E, int k, int G, int Gu, int F, int SF, int qtype, int T, int bias, int norm,
                     double lim, int given_logits) {
  mo_cfg c = {H, E, k, G, Gu, F, SF, qtype, 2.5, MO_WSUM_MIN, lim, lim, 1e-5};
  size_t nbH = (size_t)H / 32, nbF = (size_t)F / 32, nbS = (size_t)SF / 32;
  float *rw = E ? floats((size_t)E * H, 0.05f) : NULL;
  float *b = bias && E ? floats((size_t)E, 0.1f) : NULL;
  uint8_t *ge = E ? blocks(qtype, (size_t)E * F * nbH) : NULL, *ue = E ? blocks(qtype, (size_t)E * F * nbH) : NULL;
  uint8_t *de = E ? blocks(qtype, (size_t)E * H * nbF) : NULL;
  uint8_t *gs = SF ? blocks(qtype, (size_t)SF * nbH) : NULL, *us = SF ? blocks(qtype, (size_t)SF * nbH) : NULL;
  uint8_t *ds = SF ? blocks(qtype, (size_t)H * nbS) : NULL;
  float *gn = norm ? floats((size_t)H, 1.0f) : NULL;
  float *x = floats((size_t)T * H, 1.0f), *r = floats((size_t)T * H, 1.0f);
  float *li = given_logits && E ? floats((size_t)T * E, 3.0f) : NULL;
  double *out = (double *)malloc(sizeof(double) * (size_t)T * H);
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * (k ? k : 1));
  double *w = (double *)malloc(sizeof(double) * (size_t)T * (k ? k : 1));
  int rc = mo_layer(&c, rw, b, ge, ue, de, gs, us, ds, gn, x, T, r, li, out, ids, w);
  int ok = rc == 0 && all_finite(out, (size_t)T * H);
  if (ok && E) {
    int32_t *off = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *perm = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * k);
    ids[0] = ids[k - 1]; /* a repeated id: the sort takes any ids in [0, E) */
    mo_sort_by_expert(ids, T * k, E, off, perm);
    ok = off[E] == T * k;
    free(off);
    free(perm);
  }
  free(rw); free(b); free(ge); free(ue); free(de); free(gs); free(us); free(ds); free(gn);
  free(x); free(r); free(li); free(out); free(ids); free(w);
  if (!ok) fprintf(stderr, "layer H=%d E=%d k=%d G=%d/%d F=%d SF=%d q=%d T=%d: rc %d\n", H, E, k, G, Gu, F, SF, qtype,
                   T, rc);
  return ok;
}

int main(void) {
  int ok = 1;
  for (uint32_t h = 0; h < 65536; h++) (void)mo_f16((uint16_t)h);
  ok &= run_layer(64, 8, 2, 1, 1, 32, 32, MO_Q4_1, 3, 0, 0, 0.0, 0);
  ok &= run_layer(96, 16, 3, 4, 2, 64, 0, MO_Q4_0, 4, 1, 1, 3.0, 0);
  ok &= run_layer(64, 12, 12, 1, 1, 32, 64, MO_Q8_0, 2, 1, 0, 0.0, 1);
  ok &= run_layer(128, 32, 5, 8, 3, 96, 32, MO_Q4_1, 5, 1, 1, 0.0, 0);
  ok &= run_layer(64, 0, 0, 1, 1, 0, 96, MO_Q4_0, 3, 0, 1, 2.0, 0); /* a dense FFN layer */
  /* selection pieces on their own */
  float s[40];
  int32_t keep[8], ids[32];
  float gs[8];
  for (int i = 0; i < 40; i++) s[i] = unif(0.f, 1.f);
  int32_t allowed[40];
  mo_group_keep(s, 40, 8, 3, keep, gs);
  for (int e = 0; e < 40; e++) allowed[e] = keep[e / 5];
  mo_topk(s, NULL, 40, 32, ids);
  mo_topk(s, allowed, 40, 1, ids);
  double y = mo_swiglu(1.5, -2.0, 1.0) + mo_sigmoid(-800.0) + mo_sigmoid(800.0);
  ok &= isfinite(y);
  printf("oracle sanitizer run: %s\n", ok ? "ok" : "FAILED");
  return ok ? 0 : 1;
}
