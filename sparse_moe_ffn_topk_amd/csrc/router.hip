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
//  * logits: each wave owns one router row (T <= 8) and streams it with
//    16-byte buffer loads, all issued before the first product; products and
//    sums in f64 (full-rate on gfx950), one rounding to f32 at the end.  Larger
//    T uses an LDS-tiled f64 kernel.
//  * selection: one 256-thread block per token ranks the experts (a score's
//    rank is the number of experts that beat it), which gives the k argmax
//    rounds' picks at once.
#include "moe_common.h"
#include "moe_launch.h"
#include "select_block.h"

namespace moe {

// ---------------------------------------------------------------- logits --

// T <= 8 tokens: one 64-thread block per router row e; logits[t][e].  A lane
// takes NC 16-byte chunks of the row per pass and, per token, the matching NC
// chunks of x; every load of a pass is issued before the first product (buffer
// loads with an out-of-range offset past the row end read zeros, so there are
// no branches between them).  Products and sums in f64, one f32 rounding.
constexpr uint32_t ROUTER_OOB = 0x7ffffff0u;
template <int TT, int NC>
__global__ __launch_bounds__(64) void k_router_rows(const float *__restrict__ W, const float *__restrict__ x,
                                                    int H, int E, int T, float *__restrict__ logits) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const uint32_t rowbytes = (uint32_t)H * 4u;
  const rsrc_t rw = make_rsrc(W + (size_t)e * H, rowbytes);
  const rsrc_t rx = make_rsrc(x, (uint32_t)T * rowbytes);
  double acc[TT][2];
#pragma unroll
  for (int t = 0; t < TT; t++) acc[t][0] = acc[t][1] = 0.0;
  for (uint32_t c0 = 0; c0 < rowbytes; c0 += 1024u * NC) {
    uint32_t off[NC];
    u32x4 w[NC];
#pragma unroll
    for (int i = 0; i < NC; i++) {
      const uint32_t o = c0 + 16u * (uint32_t)(lane + 64 * i);
      off[i] = o < rowbytes ? o : ROUTER_OOB;
      w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off[i], 0, 0);
    }
#pragma unroll
    for (int t = 0; t < TT; t++) {
      if (t < T) {
        u32x4 v[NC];
#pragma unroll
        for (int i = 0; i < NC; i++)
          v[i] = __builtin_amdgcn_raw_buffer_load_b128(
              rx, (int)(off[i] == ROUTER_OOB ? ROUTER_OOB : (uint32_t)t * rowbytes + off[i]), 0, 0);
#pragma unroll
        for (int i = 0; i < NC; i++) {
          acc[t][0] = __builtin_fma((double)__uint_as_float(w[i][0]), (double)__uint_as_float(v[i][0]), acc[t][0]);
          acc[t][1] = __builtin_fma((double)__uint_as_float(w[i][1]), (double)__uint_as_float(v[i][1]), acc[t][1]);
          acc[t][0] = __builtin_fma((double)__uint_as_float(w[i][2]), (double)__uint_as_float(v[i][2]), acc[t][0]);
          acc[t][1] = __builtin_fma((double)__uint_as_float(w[i][3]), (double)__uint_as_float(v[i][3]), acc[t][1]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; t++) {
    if (t < T) {
      const double s = wave_sum_d(acc[t][0] + acc[t][1]);
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
    // Chunks per lane and pass: the whole row in one pass up to H = 4096.
    const int n16 = (H + 3) / 4;
    const int nc = (n16 + 63) / 64;
    const dim3 grid(E);
#define MOE_ROUTER_ROWS(TT)                                                                              \
  do {                                                                                                   \
    if (nc <= 2)                                                                                         \
      MOE_LAUNCH(1, (k_router_rows<TT, 2>), grid, dim3(64), 0u, st, W, x, H, E, T, logits);              \
    else if (nc <= 4)                                                                                    \
      MOE_LAUNCH(1, (k_router_rows<TT, 4>), grid, dim3(64), 0u, st, W, x, H, E, T, logits);              \
    else if (nc <= 8)                                                                                    \
      MOE_LAUNCH(1, (k_router_rows<TT, 8>), grid, dim3(64), 0u, st, W, x, H, E, T, logits);              \
    else if (nc <= 12)                                                                                   \
      MOE_LAUNCH(1, (k_router_rows<TT, 12>), grid, dim3(64), 0u, st, W, x, H, E, T, logits);             \
    else                                                                                                 \
      MOE_LAUNCH(1, (k_router_rows<TT, 16>), grid, dim3(64), 0u, st, W, x, H, E, T, logits);             \
  } while (0)
    if (T == 1)
      MOE_ROUTER_ROWS(1);
    else if (T <= 2)
      MOE_ROUTER_ROWS(2);
    else if (T <= 4)
      MOE_ROUTER_ROWS(4);
    else
      MOE_ROUTER_ROWS(8);
#undef MOE_ROUTER_ROWS
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
