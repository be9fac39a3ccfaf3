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
//  * logits: one block owns one router row (T <= 8), its waves splitting the
//    tokens (or, for one token, the row), and streams it with 16-byte buffer
//    loads, all issued before the first product; products and sums in f64 (full-rate on gfx950), one
//    rounding to f32 at the end.  Larger T runs on the f64 matrix cores
//    (v_mfma_f64_16x16x4f64).
//  * selection: one 256-thread block per token ranks the experts (a score's
//    rank is the number of experts that beat it), which gives the k argmax
//    rounds' picks at once.
#include "moe_common.h"
#include "moe_launch.h"
#include "select_block.h"

namespace moe {

// ---------------------------------------------------------------- logits --

// T <= 8 tokens: one block of NW = min(T, 4) waves per router row e;
// logits[t][e].  Wave w takes tokens w, w + NW (TPW of them), so a wave's
// serial path is at most two tokens long.  A lane takes NC 16-byte chunks of
// the row per pass and, per token, the matching NC chunks of x; every load of
// a pass is issued before the first product (buffer loads with an
// out-of-range offset past the row end read zeros, so there are no branches
// between them).  Products and sums in f64, one f32 rounding.
constexpr uint32_t ROUTER_OOB = 0x7ffffff0u;
//
// With gnorm != NULL (one pass: H <= 256 * NC) x is the residual stream and
// each token is first normalised in registers: the wave's lanes hold the whole
// row, so the sum of squares (f64) reduces across the wave, and the lanes form
// xn = f32(x * s * g), s = 1/sqrt(ss/H + eps), before the dot; block 0 writes
// xn for the FFN kernels.  Every block computes the same xn the same way.
template <int TPW, int NC>
__global__ __launch_bounds__(512) void k_router_rows(const float *__restrict__ W, const float *__restrict__ x,
                                                     int H, int E, int T, float *__restrict__ logits,
                                                     const float *__restrict__ gnorm, float eps,
                                                     float *__restrict__ xn_out) {
  const int e = blockIdx.x, lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), NW = blockDim.x >> 6;
  const uint32_t rowbytes = (uint32_t)H * 4u;
  const rsrc_t rw = make_rsrc(W + (size_t)e * H, rowbytes);
  const rsrc_t rx = make_rsrc(x, (uint32_t)T * rowbytes);
  const rsrc_t rg = make_rsrc(gnorm, rowbytes);
  double acc[TPW][2];
#pragma unroll
  for (int i = 0; i < TPW; i++) acc[i][0] = acc[i][1] = 0.0;
  for (uint32_t c0 = 0; c0 < rowbytes; c0 += 1024u * NC) {
    uint32_t off[NC];
    u32x4 wr[NC];
#pragma unroll
    for (int i = 0; i < NC; i++) {
      const uint32_t o = c0 + 16u * (uint32_t)(lane + 64 * i);
      off[i] = o < rowbytes ? o : ROUTER_OOB;
      wr[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off[i], 0, 0);
    }
    u32x4 gv[NC];
    if (gnorm) {
#pragma unroll
      for (int i = 0; i < NC; i++) gv[i] = __builtin_amdgcn_raw_buffer_load_b128(rg, (int)off[i], 0, 0);
    }
#pragma unroll
    for (int ti = 0; ti < TPW; ti++) {
      const int t = w + NW * ti;
      if (t < T) {
        u32x4 v[NC];
#pragma unroll
        for (int i = 0; i < NC; i++)
          v[i] = __builtin_amdgcn_raw_buffer_load_b128(
              rx, (int)(off[i] == ROUTER_OOB ? ROUTER_OOB : (uint32_t)t * rowbytes + off[i]), 0, 0);
        if (gnorm) {
          double ss = 0.0;
#pragma unroll
          for (int i = 0; i < NC; i++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
              const double f = (double)__uint_as_float(v[i][c]);
              ss = __builtin_fma(f, f, ss);
            }
          const double sc = 1.0 / sqrt(wave_sum_d(ss) / (double)H + (double)eps);
#pragma unroll
          for (int i = 0; i < NC; i++) {
#pragma unroll
            for (int c = 0; c < 4; c++)
              v[i][c] = __float_as_uint(
                  (float)((double)__uint_as_float(v[i][c]) * sc * (double)__uint_as_float(gv[i][c])));
            if (e == 0 && off[i] != ROUTER_OOB)
              *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(xn_out) + (size_t)t * rowbytes + off[i]) = v[i];
          }
        }
#pragma unroll
        for (int i = 0; i < NC; i++) {
          acc[ti][0] = __builtin_fma((double)__uint_as_float(wr[i][0]), (double)__uint_as_float(v[i][0]), acc[ti][0]);
          acc[ti][1] = __builtin_fma((double)__uint_as_float(wr[i][1]), (double)__uint_as_float(v[i][1]), acc[ti][1]);
          acc[ti][0] = __builtin_fma((double)__uint_as_float(wr[i][2]), (double)__uint_as_float(v[i][2]), acc[ti][0]);
          acc[ti][1] = __builtin_fma((double)__uint_as_float(wr[i][3]), (double)__uint_as_float(v[i][3]), acc[ti][1]);
        }
      }
    }
  }
#pragma unroll
  for (int ti = 0; ti < TPW; ti++) {
    const int t = w + NW * ti;
    if (t < T) {
      const double s = wave_sum_d(acc[ti][0] + acc[ti][1]);
      if (lane == 0) logits[(size_t)t * E + e] = (float)s;
    }
  }
}

// T = 1: one block of 256 threads per router row e; thread i takes the row's
// 16-byte chunks i, i + 256, ... (NCB of them, every load issued up front), so
// a wave's serial f64 work is a quarter of a row.  Partial sums reduce per
// wave, then over the four waves in LDS in wave order (fixed: reproducible).
// With gnorm the same two-level reduction first gives the sum of squares;
// every block normalises its chunks the same way and block 0 writes xn.
template <int NCB>
__global__ __launch_bounds__(256) void k_router_row1(const float *__restrict__ W, const float *__restrict__ x, int H,
                                                     float *__restrict__ logits, const float *__restrict__ gnorm,
                                                     float eps, float *__restrict__ xn_out) {
  __shared__ double red[2][4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t rowbytes = (uint32_t)H * 4u;
  const rsrc_t rw = make_rsrc(W + (size_t)e * H, rowbytes);
  const rsrc_t rx = make_rsrc(x, rowbytes);
  const rsrc_t rg = make_rsrc(gnorm, rowbytes);
  uint32_t off[NCB];
  u32x4 wr[NCB], xv[NCB], gv[NCB];
#pragma unroll
  for (int i = 0; i < NCB; i++) {
    const uint32_t o = 16u * (uint32_t)(tid + 256 * i);
    off[i] = o < rowbytes ? o : ROUTER_OOB;
    wr[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off[i], 0, 0);
  }
#pragma unroll
  for (int i = 0; i < NCB; i++) xv[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off[i], 0, 0);
  if (gnorm) {
#pragma unroll
    for (int i = 0; i < NCB; i++) gv[i] = __builtin_amdgcn_raw_buffer_load_b128(rg, (int)off[i], 0, 0);
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NCB; i++)
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const double f = (double)__uint_as_float(xv[i][c]);
        ss = __builtin_fma(f, f, ss);
      }
    ss = wave_sum_d(ss);
    if (lane == 0) red[0][w] = ss;
    __syncthreads();
    const double sc = 1.0 / sqrt(((red[0][0] + red[0][1]) + (red[0][2] + red[0][3])) / (double)H + (double)eps);
#pragma unroll
    for (int i = 0; i < NCB; i++) {
#pragma unroll
      for (int c = 0; c < 4; c++)
        xv[i][c] = __float_as_uint(
            (float)((double)__uint_as_float(xv[i][c]) * sc * (double)__uint_as_float(gv[i][c])));
      if (e == 0 && off[i] != ROUTER_OOB) *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(xn_out) + off[i]) = xv[i];
    }
  }
  double a0 = 0.0, a1 = 0.0;
#pragma unroll
  for (int i = 0; i < NCB; i++) {
    a0 = __builtin_fma((double)__uint_as_float(wr[i][0]), (double)__uint_as_float(xv[i][0]), a0);
    a1 = __builtin_fma((double)__uint_as_float(wr[i][1]), (double)__uint_as_float(xv[i][1]), a1);
    a0 = __builtin_fma((double)__uint_as_float(wr[i][2]), (double)__uint_as_float(xv[i][2]), a0);
    a1 = __builtin_fma((double)__uint_as_float(wr[i][3]), (double)__uint_as_float(xv[i][3]), a1);
  }
  const double s = wave_sum_d(a0 + a1);
  if (lane == 0) red[1][w] = s;
  __syncthreads();
  if (tid == 0) logits[e] = (float)((red[1][0] + red[1][1]) + (red[1][2] + red[1][3]));
}

// T > 8: logits = x W^T on v_mfma_f64_16x16x4f64 (f32 inputs are exact in
// f64, so products are exact and sums are f64, as in the row kernel).  A block
// takes 16 router rows x 32 tokens with eight waves: wave w the tokens
// 16 (w & 1) .. +15 over the quarter w >> 1 of every chunk's columns (split
// K: two waves per SIMD of the chip), with four accumulator chains per wave.  Lane l feeds A =
// x[token l%16][h + l/16] and B = W[row l%16][h + l/16] and holds
// D[token l/16 + 4i][row l%16], i < 4.  The four quarters' sums are added in
// a fixed order (reproducible).  W and x are staged through LDS in chunks of RKT
// columns (16-byte loads, next chunk prefetched into registers); columns past
// H, rows past E and tokens past T read as zeros.
constexpr int RKT = 128;
typedef double f64x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(512) void k_router_mfma(const float *__restrict__ W, const float *__restrict__ x, int H,
                                                     int E, int T, float *__restrict__ logits) {
  __shared__ __attribute__((aligned(16))) float ws[16][RKT + 4];
  __shared__ __attribute__((aligned(16))) float xs[32][RKT + 4];
  __shared__ f64x4 red[3][2][64];  // quarters 1..3
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tg = wave & 1, kh = wave >> 1;  // token group, K quarter
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 32;
  const int ne = min(16, E - e0), nt = min(32, T - t0);
  const rsrc_t rW = make_rsrc(W + (size_t)e0 * H, (uint32_t)ne * (uint32_t)H * 4u);
  const rsrc_t rX = make_rsrc(x + (size_t)t0 * H, (uint32_t)nt * (uint32_t)H * 4u);
  // staging roles: piece q = tid + 512 i of a chunk is row q / 32, 16-byte
  // column q % 32 (W: i < 1, rows 0..15; x: i < 2, rows 0..31)
  constexpr int CPR = RKT / 4;  // 16-byte columns per staged row
  constexpr int NT = 512;
  u32x4 wr[16 * CPR / NT], xr[32 * CPR / NT];
  auto issue = [&](int h0) {
#pragma unroll
    for (int i = 0; i < 16 * CPR / NT; i++) {
      const int q = tid + NT * i, r = q / CPR, h = h0 + 4 * (q % CPR);
      wr[i] = __builtin_amdgcn_raw_buffer_load_b128(rW, (int)(h < H ? (uint32_t)(r * H + h) * 4u : 0x7ffffff0u), 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 32 * CPR / NT; i++) {
      const int q = tid + NT * i, r = q / CPR, h = h0 + 4 * (q % CPR);
      xr[i] = __builtin_amdgcn_raw_buffer_load_b128(rX, (int)(h < H ? (uint32_t)(r * H + h) * 4u : 0x7ffffff0u), 0, 0);
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int i = 0; i < 16 * CPR / NT; i++) {
      const int q = tid + NT * i;
      *reinterpret_cast<u32x4 *>(&ws[q / CPR][4 * (q % CPR)]) = wr[i];
    }
#pragma unroll
    for (int i = 0; i < 32 * CPR / NT; i++) {
      const int q = tid + NT * i;
      *reinterpret_cast<u32x4 *>(&xs[q / CPR][4 * (q % CPR)]) = xr[i];
    }
  };
  f64x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; j++) acc[j] = f64x4{0.0, 0.0, 0.0, 0.0};
  const int m = lane & 15, kq = lane >> 4;
  const float *xrow = xs[16 * tg + m];
  const float *wrow = ws[m];
  issue(0);
  for (int h0 = 0; h0 < H; h0 += RKT) {
    put();
    __syncthreads();
    if (h0 + RKT < H) issue(h0 + RKT);
#pragma unroll
    for (int kk = kh * (RKT / 4); kk < (kh + 1) * (RKT / 4); kk += 16) {
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xrow[kk + 4 * j + kq], (double)wrow[kk + 4 * j + kq],
                                                      acc[j], 0, 0, 0);
    }
    __syncthreads();
  }
  const f64x4 sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  if (kh > 0) red[kh - 1][tg][lane] = sum;
  __syncthreads();
  if (kh == 0) {
    const f64x4 tot = ((sum + red[0][tg][lane]) + red[1][tg][lane]) + red[2][tg][lane];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int t = 16 * tg + kq + 4 * i, e = m;
      if (t < nt && e < ne) logits[(size_t)(t0 + t) * E + e0 + e] = (float)tot[i];
    }
  }
}

// --------------------------------------------------------------- rmsnorm --

// One 256-thread block per token: the sum of squares in f64 (fixed order:
// per-thread strided partials, wave sums, then the four waves in order),
// s = 1/sqrt(ss/H + eps), xn = f32(x * s * g).  H % 32 == 0.
__global__ __launch_bounds__(256) void k_rmsnorm(const float *__restrict__ x, const float *__restrict__ g, int H,
                                                 float eps, float *__restrict__ xn) {
  __shared__ double part[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const float4 *x4 = reinterpret_cast<const float4 *>(x + (size_t)t * H);
  const float4 *g4 = reinterpret_cast<const float4 *>(g);
  float4 *o4 = reinterpret_cast<float4 *>(xn + (size_t)t * H);
  const int n4 = H >> 2;
  double ss = 0.0;
  for (int i = tid; i < n4; i += 256) {
    const float4 v = x4[i];
    ss = __builtin_fma((double)v.x, (double)v.x, ss);
    ss = __builtin_fma((double)v.y, (double)v.y, ss);
    ss = __builtin_fma((double)v.z, (double)v.z, ss);
    ss = __builtin_fma((double)v.w, (double)v.w, ss);
  }
  ss = wave_sum_d(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const double s = 1.0 / sqrt(((part[0] + part[1]) + (part[2] + part[3])) / (double)H + (double)eps);
  for (int i = tid; i < n4; i += 256) {
    const float4 v = x4[i], w = g4[i];
    o4[i] = make_float4((float)((double)v.x * s * (double)w.x), (float)((double)v.y * s * (double)w.y),
                        (float)((double)v.z * s * (double)w.z), (float)((double)v.w * s * (double)w.w));
  }
}

hipError_t launch_rmsnorm(const float *x, const float *g, int H, int T, float eps, float *xn, hipStream_t st) {
  MOE_LAUNCH(9, k_rmsnorm, dim3(T), dim3(256), 0u, st, x, g, H, eps, xn);
  return hipGetLastError();
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

int router_fuses_norm(int H, int T) { return T <= 8 && H <= 4096; }

hipError_t launch_router_logits(const float *W, const float *x, int H, int E, int T, float *logits,
                                hipStream_t st, const float *gnorm, float eps, float *xn) {
  if (gnorm && !router_fuses_norm(H, T)) return hipErrorInvalidValue;
  if (T == 1 && H <= 4096) {
    const int ncb = (H / 4 + 255) / 256;  // 16-byte chunks per thread
    const dim3 grid(E), block(256);
    if (ncb <= 1)
      MOE_LAUNCH(1, (k_router_row1<1>), grid, block, 0u, st, W, x, H, logits, gnorm, eps, xn);
    else if (ncb == 2)
      MOE_LAUNCH(1, (k_router_row1<2>), grid, block, 0u, st, W, x, H, logits, gnorm, eps, xn);
    else if (ncb == 3)
      MOE_LAUNCH(1, (k_router_row1<3>), grid, block, 0u, st, W, x, H, logits, gnorm, eps, xn);
    else
      MOE_LAUNCH(1, (k_router_row1<4>), grid, block, 0u, st, W, x, H, logits, gnorm, eps, xn);
  } else if (T <= 8) {
    // Chunks per lane and pass: the whole row in one pass up to H = 4096.
    const int n16 = (H + 3) / 4;
    const int nc = (n16 + 63) / 64;
    const dim3 grid(E), block(64 * T);  // one wave per token
#define MOE_ROUTER_ROWS(TPW)                                                                             \
  do {                                                                                                   \
    if (nc <= 2)                                                                                         \
      MOE_LAUNCH(1, (k_router_rows<TPW, 2>), grid, block, 0u, st, W, x, H, E, T, logits, gnorm, eps, xn); \
    else if (nc <= 4)                                                                                    \
      MOE_LAUNCH(1, (k_router_rows<TPW, 4>), grid, block, 0u, st, W, x, H, E, T, logits, gnorm, eps, xn); \
    else if (nc <= 8)                                                                                    \
      MOE_LAUNCH(1, (k_router_rows<TPW, 8>), grid, block, 0u, st, W, x, H, E, T, logits, gnorm, eps, xn); \
    else if (nc <= 12)                                                                                   \
      MOE_LAUNCH(1, (k_router_rows<TPW, 12>), grid, block, 0u, st, W, x, H, E, T, logits, gnorm, eps, xn);\
    else                                                                                                 \
      MOE_LAUNCH(1, (k_router_rows<TPW, 16>), grid, block, 0u, st, W, x, H, E, T, logits, gnorm, eps, xn);\
  } while (0)
    MOE_ROUTER_ROWS(1);
#undef MOE_ROUTER_ROWS
  } else {
    const dim3 grid((E + 15) / 16, (T + 31) / 32);
    MOE_LAUNCH(1, k_router_mfma, grid, dim3(512), 0u, st, W, x, H, E, T, logits);
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
