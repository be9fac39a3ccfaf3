// router.hip -- router logits and top-k selection (gfx950, wave64).
//
// What is computed follows the router of the diskformer pages: sigmoid of the
// F32 router logits, an optional bias that only steers selection, optional
// group-limited selection (groups ranked by the sum of their two best scores),
// k rounds of argmax with lowest-index ties, and weights = picked sigmoids
// over their sum clamped at wsum_min, times weights_scale (lfm2_moe_ssd.js
// page: router comment and TOPK_SIG_BODY; ling_moe_ssd.js page: routeLing).
//
// MI355X design:
//  * logits: each wave owns one router row (decode) and streams it with
//    16-byte loads; products and sums in f64 (full-rate on gfx950), one
//    rounding to f32 at the end.  Large T uses an LDS-tiled f64 kernel.
//  * selection: one wave per token; expert e sits in lane e%64, slot e/64, so
//    every comparison is in registers and every reduction is a 6-step
//    butterfly -- no LDS, no barriers.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

// ---------------------------------------------------------------- logits --

// T <= 8 tokens: one 64-thread block per router row e; logits[t][e].
template <int TT>
__global__ __launch_bounds__(64) void k_router_rows(const float *__restrict__ W, const float *__restrict__ x,
                                                    int H, int E, int T, float *__restrict__ logits) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const float4 *w4 = reinterpret_cast<const float4 *>(W + (size_t)e * H);
  const int n4 = H >> 2;
  double acc[TT];
#pragma unroll
  for (int t = 0; t < TT; t++) acc[t] = 0.0;
  for (int c = lane; c < n4; c += 64) {
    float4 w = w4[c];
#pragma unroll
    for (int t = 0; t < TT; t++) {
      if (t < T) {
        float4 v = reinterpret_cast<const float4 *>(x + (size_t)t * H)[c];
        acc[t] = __builtin_fma((double)w.x, (double)v.x, acc[t]);
        acc[t] = __builtin_fma((double)w.y, (double)v.y, acc[t]);
        acc[t] = __builtin_fma((double)w.z, (double)v.z, acc[t]);
        acc[t] = __builtin_fma((double)w.w, (double)v.w, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; t++) {
    if (t < T) {
      double s = group_sum_d(acc[t], 64);
      if (lane == 0) logits[(size_t)t * E + e] = (float)s;
    }
  }
}

// Any T: 16 router rows x 16 tokens per 256-thread block, K staged through
// LDS in chunks of 64; thread (r, t) accumulates one logit in f64.
__global__ __launch_bounds__(256) void k_router_tiled(const float *__restrict__ W, const float *__restrict__ x,
                                                      int H, int E, int T, float *__restrict__ logits) {
  __shared__ float ws[16][65];
  __shared__ float xs[16][65];
  const int tid = threadIdx.x;
  const int r = tid >> 4, tt = tid & 15;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  double acc = 0.0;
  for (int k0 = 0; k0 < H; k0 += 64) {
    // 16 rows x 64 columns of W and of x: 1024 floats each, 4 per thread.
    for (int i = tid; i < 1024; i += 256) {
      int rr = i >> 6, kk = i & 63;
      int e = e0 + rr, t = t0 + rr, k = k0 + kk;
      ws[rr][kk] = (e < E && k < H) ? W[(size_t)e * H + k] : 0.f;
      xs[rr][kk] = (t < T && k < H) ? x[(size_t)t * H + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 16
    for (int kk = 0; kk < 64; kk++) acc = __builtin_fma((double)ws[r][kk], (double)xs[tt][kk], acc);
    __syncthreads();
  }
  const int e = e0 + r, t = t0 + tt;
  if (e < E && t < T) logits[(size_t)t * E + e] = (float)acc;
}

// ---------------------------------------------------------------- select --

// Wave-wide arg-max with lowest index on equal values; all lanes get it.
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float ov = __shfl_xor(v, m, 64);
    int oi = __shfl_xor(i, m, 64);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

// Wave-wide top-2 multiset (a >= b) of per-lane pairs; all lanes get it.
__device__ __forceinline__ void wave_top2(float &a, float &b) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float oa = __shfl_xor(a, m, 64), ob = __shfl_xor(b, m, 64);
    float na = fmaxf(a, oa);
    float nb = fmaxf(fminf(a, oa), fmaxf(b, ob));
    a = na;
    b = nb;
  }
}

constexpr float NEG = -3.402823466e38f;  // below every score (scores are >= -|bias| - 0)

// One wave per token.  Expert e = lane + 64*s for slot s < S = ceil(E/64).
template <int S>
__global__ __launch_bounds__(256) void k_select(const float *__restrict__ logits, const float *__restrict__ bias,
                                                int T, int E, int k, int G, int Gu, float scale, float wsum_min,
                                                int32_t *__restrict__ ids, float *__restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *l = logits + (size_t)t * E;
  float p[S], s[S];
#pragma unroll
  for (int j = 0; j < S; j++) {
    int e = lane + 64 * j;
    if (e < E) {
      // sigmoid of the f32 logit, evaluated in double, rounded once to f32
      double pd = 1.0 / (1.0 + exp(-(double)l[e]));
      p[j] = (float)pd;
      s[j] = p[j] + (bias ? bias[e] : 0.f);
    } else {
      p[j] = 0.f;
      s[j] = NEG;
    }
  }
  if (Gu < G) {
    // Group g covers experts [g*P, (g+1)*P).  Lane g ends up holding the
    // score of group g (its two best selection scores, summed in f32).
    const int P = E / G;
    float gscore = NEG;
    for (int g = 0; g < G; g++) {
      float a = NEG, b = NEG;
#pragma unroll
      for (int j = 0; j < S; j++) {
        int e = lane + 64 * j;
        if (e < E && e / P == g) {
          float v = s[j];
          if (v > a) {
            b = a;
            a = v;
          } else if (v > b) {
            b = v;
          }
        }
      }
      wave_top2(a, b);
      if (lane == g) gscore = a + b;
    }
    // Keep Gu groups: Gu rounds of arg-max over lanes < G (lowest g on ties).
    bool kept = false;
    float gv = (lane < G) ? gscore : NEG;
    for (int r = 0; r < Gu; r++) {
      float v = (lane < G && !kept) ? gv : NEG;
      int i = lane;
      wave_argmax(v, i);
      if (lane == i) kept = true;
    }
    // Drop the experts of the other groups.
#pragma unroll
    for (int j = 0; j < S; j++) {
      int e = lane + 64 * j;
      int g = (e < E) ? e / P : 0;
      bool keep_e = __shfl(kept ? 1 : 0, g, 64) != 0;
      if (!keep_e) s[j] = NEG;
    }
  }
  // k rounds of arg-max; the winner is removed.  Lane j keeps pick j.
  float wsum = 0.f, my_p = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; j++) {
    float v = NEG;
    int i = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < S; q++) {
      int e = lane + 64 * q;
      if (e < E && (s[q] > v || (s[q] == v && e < i))) {
        v = s[q];
        i = e;
      }
    }
    wave_argmax(v, i);
    // the owner of expert i drops it and broadcasts its sigmoid
    float pi = 0.f;
#pragma unroll
    for (int q = 0; q < S; q++) {
      if (lane + 64 * q == i) {
        pi = p[q];
        s[q] = NEG;
      }
    }
    pi = __shfl(pi, i & 63, 64);
    if (lane == j) {
      my_p = pi;
      my_e = i;
    }
    wsum += pi;  // f32 sum in pick order (identical on every lane)
  }
  wsum = fmaxf(wsum, wsum_min);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    wts[(size_t)t * k + lane] = my_p / wsum * scale;
  }
}

// ---------------------------------------------------------------- launch --

hipError_t launch_router_logits(const float *W, const float *x, int H, int E, int T, float *logits,
                                hipStream_t st) {
  if (T <= 8) {
    dim3 grid(E);
    if (T == 1)
      k_router_rows<1><<<grid, 64, 0, st>>>(W, x, H, E, T, logits);
    else if (T <= 2)
      k_router_rows<2><<<grid, 64, 0, st>>>(W, x, H, E, T, logits);
    else if (T <= 4)
      k_router_rows<4><<<grid, 64, 0, st>>>(W, x, H, E, T, logits);
    else
      k_router_rows<8><<<grid, 64, 0, st>>>(W, x, H, E, T, logits);
  } else {
    dim3 grid((E + 15) / 16, (T + 15) / 16);
    k_router_tiled<<<grid, 256, 0, st>>>(W, x, H, E, T, logits);
  }
  return hipGetLastError();
}

hipError_t launch_select(const float *logits, const float *bias, int T, int E, int k, int G, int Gu,
                         float scale, float wsum_min, int32_t *ids, float *wts, hipStream_t st) {
  dim3 grid((T + 3) / 4);
  int S = (E + 63) / 64;
#define MOE_SEL(n) k_select<n><<<grid, 256, 0, st>>>(logits, bias, T, E, k, G, Gu, scale, wsum_min, ids, wts)
  switch (S) {
    case 1: MOE_SEL(1); break;
    case 2: MOE_SEL(2); break;
    case 3: MOE_SEL(3); break;
    case 4: MOE_SEL(4); break;
    case 5: MOE_SEL(5); break;
    case 6: MOE_SEL(6); break;
    case 7: MOE_SEL(7); break;
    default: MOE_SEL(8); break;
  }
#undef MOE_SEL
  return hipGetLastError();
}

}  // namespace moe
