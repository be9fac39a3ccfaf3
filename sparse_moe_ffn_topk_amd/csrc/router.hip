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
#include "select_block.h"

namespace moe {

// ---------------------------------------------------------------- logits --

// T <= 8 tokens: one 64-thread block per router row e; logits[t][e].  A lane
// holds up to RCH float4 of the row in registers (all loads in flight at once),
// then runs the tokens over them; products and sums in f64.
constexpr int RCH = 16;
template <int TT>
__global__ __launch_bounds__(64) void k_router_rows(const float *__restrict__ W, const float *__restrict__ x,
                                                    int H, int E, int T, float *__restrict__ logits) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const float4 *w4 = reinterpret_cast<const float4 *>(W + (size_t)e * H);
  const int n4 = H >> 2;
  double acc[TT];
#pragma unroll
  for (int t = 0; t < TT; t++) acc[t] = 0.0;
  for (int c0 = 0; c0 < n4; c0 += 64 * RCH) {
    float4 w[RCH];
#pragma unroll
    for (int i = 0; i < RCH; i++) {
      const int c = c0 + lane + 64 * i;
      w[i] = c < n4 ? w4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int t = 0; t < TT; t++) {
      if (t < T) {
        const float4 *x4 = reinterpret_cast<const float4 *>(x + (size_t)t * H);
#pragma unroll
        for (int i = 0; i < RCH; i++) {
          const int c = c0 + lane + 64 * i;
          if (c < n4) {
            const float4 v = x4[c];
            acc[t] = __builtin_fma((double)w[i].x, (double)v.x, acc[t]);
            acc[t] = __builtin_fma((double)w[i].y, (double)v.y, acc[t]);
            acc[t] = __builtin_fma((double)w[i].z, (double)v.z, acc[t]);
            acc[t] = __builtin_fma((double)w[i].w, (double)v.w, acc[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; t++) {
    if (t < T) {
      const double s = wave_sum_d(acc[t]);
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

// One block of 256 threads per token.
__global__ __launch_bounds__(256) void k_select(const float *__restrict__ logits, const float *__restrict__ bias,
                                                int T, SelParams P, int32_t *__restrict__ ids,
                                                float *__restrict__ wts) {
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  select_block(logits + (size_t)t * P.E, bias, P, sh, wts + (size_t)t * P.k);
  if (threadIdx.x < P.k) ids[(size_t)t * P.k + threadIdx.x] = sh.pick[threadIdx.x];
}

// ---------------------------------------------------------------- launch --

hipError_t launch_router_logits(const float *W, const float *x, int H, int E, int T, float *logits,
                                hipStream_t st) {
  if (T <= 8) {
    dim3 grid(E);
    if (T == 1)
      MOE_LAUNCH(1, (k_router_rows<1>), grid, dim3(64), 0u, st, W, x, H, E, T, logits);
    else if (T <= 2)
      MOE_LAUNCH(1, (k_router_rows<2>), grid, dim3(64), 0u, st, W, x, H, E, T, logits);
    else if (T <= 4)
      MOE_LAUNCH(1, (k_router_rows<4>), grid, dim3(64), 0u, st, W, x, H, E, T, logits);
    else
      MOE_LAUNCH(1, (k_router_rows<8>), grid, dim3(64), 0u, st, W, x, H, E, T, logits);
  } else {
    dim3 grid((E + 15) / 16, (T + 15) / 16);
    MOE_LAUNCH(1, k_router_tiled, grid, dim3(256), 0u, st, W, x, H, E, T, logits);
  }
  return hipGetLastError();
}

hipError_t launch_select(const float *logits, const float *bias, int T, int E, int k, int G, int Gu,
                         float scale, float wsum_min, int32_t *ids, float *wts, hipStream_t st) {
  const SelParams P{E, k, G, Gu, scale, wsum_min};
  MOE_LAUNCH(2, k_select, dim3(T), dim3(256), 0u, st, logits, bias, T, P, ids, wts);
  return hipGetLastError();
}

}  // namespace moe
