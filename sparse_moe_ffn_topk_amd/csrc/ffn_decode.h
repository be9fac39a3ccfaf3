// ffn_decode.h -- expert FFNs for small T (decode): fused dequant-GEMVs
// read straight from GGUF Q4_0 / Q4_1 blocks (gfx950, wave64).
//
// Computes, per token t and pick j (plus the always-on shared expert):
//   act[f] = silu(g_f) * u_f,  g = Wg x_t, u = Wu x_t        (gate || up)
//   resid[t][h] += sum_j w_tj * (Wd_j act_j)[h] + (Wd_sh act_sh)[h]
// as the swiglu and moeAccum kernels of the diskformer ling_moe_ssd.js page
// and moeAccumB of the lfm2_moe_ssd.js page state it (no SwiGLU clamp).
//
// MI355X design:
//  * a "lane group" of LPR lanes (a power of two <= 16 dividing the row's
//    block count) owns one output row; lane i reads blocks i, i+LPR, ... with
//    one 16-byte and one 4-byte buffer load per 20-byte block, so a group's
//    loads cover consecutive bytes of the row and rows stay whole per group;
//  * nibbles are unpacked in registers (mask, v_cvt_f32_ubyte*, FMA) against
//    the input block staged in LDS; the Q4_1 offset term m*sum(x) uses the
//    per-block input sums staged beside it;
//  * gate and up rows of the same f are streamed by the same lanes so the
//    SwiGLU is applied in registers and act is written once;
//  * the down kernel gives each output h one owner that loops over the
//    token's picks and the shared expert, so the routing weight is applied in
//    registers and resid is read and written once: no atomics, bitwise
//    reproducible.
#pragma once
#include "moe_common.h"
#include "moe_launch.h"
#include "select_block.h"

namespace moe {

// Blocks per lane held in registers per chunk (two chunks in flight).
constexpr int NCH = 4;
// Offset past every buffer resource's range: loads there return zeros without
// touching memory, and an all-zero block contributes exactly 0 to a dot.
constexpr uint32_t OOB = 0x7ffffff0u;

// Input staging in two halves so its loads are issued before the weight
// loads and its LDS writes happen after them.  stage_load() reads the n floats
// of src into registers (XR float4 per thread; loads past n return zeros);
// stage_store() writes them as blocks of 32 (stride XSTRIDE) and each block's
// sum to sx[].  n % 32 == 0, n <= 1024 * XR.
template <int XR>
struct Stage {
  float4 v[XR];
};
template <int XR>
__device__ __forceinline__ void stage_load(Stage<XR> &st, const float *src, int n) {
  const rsrc_t r = make_rsrc(src, (uint32_t)n * 4u);
#pragma unroll
  for (int i = 0; i < XR; i++) {
    // (element-wise: __builtin_bit_cast of an ext-vector element reads element 0 with this compiler)
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)((threadIdx.x + 256 * i) * 16), 0, 0);
    const uint32_t a0 = v.x, a1 = v.y, a2 = v.z, a3 = v.w;
    st.v[i] = make_float4(__uint_as_float(a0), __uint_as_float(a1), __uint_as_float(a2), __uint_as_float(a3));
  }
}
template <int XR>
__device__ __forceinline__ void stage_store(const Stage<XR> &st, int n, float *xs, float *sx) {
  const int n4 = n >> 2;
#pragma unroll
  for (int i = 0; i < XR; i++) {
    const int q = threadIdx.x + 256 * i;
    const int b = q >> 3, c = q & 7;
    const float4 v = st.v[i];
    if (q < n4) *reinterpret_cast<float4 *>(xs + b * XSTRIDE + 4 * c) = v;
    // 8 consecutive lanes hold one block; the last of them gets its sum
    const float s = group_sum_last<8>((v.x + v.y) + (v.z + v.w));
    if (q < n4 && c == 7) sx[b] = s;
  }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// grid.x: row tiles of 256/LPR rows; grid.y: pair p (T*k routed, then T shared).
// act row of token t: its k routed rows of F, then the shared row of SF.
// With logits != NULL the routed blocks first route their token with the whole
// block (select_block) while their x loads are in flight; block (0, t*k+k-1)
// writes the token's ids and weights.  Otherwise ids are read from `ids`.
template <int QT, int LPR, int XR>
__global__ __launch_bounds__(256) void k_gateup_swiglu(
    const float *__restrict__ x, int32_t *__restrict__ ids, float *__restrict__ wts,
    const float *__restrict__ logits, const float *__restrict__ bias, SelParams P, int T, int H, int k, int F,
    int SF, const uint8_t *__restrict__ gate_exps, const uint8_t *__restrict__ up_exps,
    const uint8_t *__restrict__ gate_sh, const uint8_t *__restrict__ up_sh, float *__restrict__ act) {
  extern __shared__ float smem[];
  constexpr int BS = QBlock<QT>::bytes;
  constexpr int ROWS = 256 / LPR;
  const int nbH = H >> 5;
  const int p = blockIdx.y;
  const int nroute = T * k;
  const size_t arow = (size_t)k * F + SF;
  const bool routed = p < nroute;
  const int t = routed ? p / k : p - nroute;
  const int rows = routed ? F : SF;
  const int f0 = blockIdx.x * ROWS;
  if (f0 >= rows) return;

  Stage<XR> xst;
  int e = 0;
  if (routed && logits) {
    // route the token with the whole block; x is already in flight
    __shared__ SelShared sh;
    stage_load(xst, x + (size_t)t * H, H);
    const int j = p - t * k;
    const bool writer = j == k - 1 && blockIdx.x == 0;
    select_block(logits + (size_t)t * P.E, bias, P, sh, writer ? wts + (size_t)t * k : nullptr);
    e = sh.pick[j];
    if (writer && threadIdx.x < k) ids[(size_t)t * k + threadIdx.x] = sh.pick[threadIdx.x];
  } else {
    if (routed) e = ids[p];
    stage_load(xst, x + (size_t)t * H, H);  // input first: its loads retire first
  }
  const uint8_t *gbase, *ubase;
  float *out;
  if (routed) {
    const size_t mat = (size_t)F * nbH * BS;
    gbase = gate_exps + (size_t)e * mat;
    ubase = up_exps + (size_t)e * mat;
    out = act + (size_t)t * arow + (size_t)(p - t * k) * F;
  } else {
    gbase = gate_sh;
    ubase = up_sh;
    out = act + (size_t)t * arow + (size_t)k * F;
  }

  const int gi = threadIdx.x / LPR, li = threadIdx.x % LPR;
  const int f = f0 + gi;
  const bool live = f < rows;
  const uint32_t mbytes = (uint32_t)((size_t)rows * nbH * BS);
  const rsrc_t rg = make_rsrc(gbase, mbytes), ru = make_rsrc(ubase, mbytes);
  const uint32_t rowoff = (uint32_t)f * nbH * BS;
  const int nch = (nbH / LPR + NCH - 1) / NCH;  // LPR divides nbH

  Raw5 ga[NCH], ua[NCH], gb[NCH], ub[NCH];
  auto offset = [&](int c, int i) {
    const int b = li + LPR * (c * NCH + i);
    return (live && b < nbH) ? rowoff + (uint32_t)b * BS : OOB;
  };
  auto load = [&](Raw5 *G, Raw5 *U, int c) {
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const uint32_t off = offset(c, i);
      G[i] = QBlock<QT>::load(rg, off);
      U[i] = QBlock<QT>::load(ru, off);
    }
  };
  float *xs = smem, *sx = smem + nbH * XSTRIDE;
  float g = 0.f, u = 0.f;
  auto compute = [&](const Raw5 *G, const Raw5 *U, int c) {
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const uint32_t off = offset(c, i);
      const int b = min(li + LPR * (c * NCH + i), nbH - 1);
      const float *xb = xs + b * XSTRIDE;
      const float s = sx[b];
      g += block_dot<QT>(G[i], off, xb, s);
      u += block_dot<QT>(U[i], off, xb, s);
    }
  };

  load(ga, ua, 0);
  if (nch > 1) load(gb, ub, 1);
  stage_store(xst, H, xs, sx);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    compute(ga, ua, c);
    if (c + 2 < nch) load(ga, ua, c + 2);
    if (c + 1 < nch) {
      compute(gb, ub, c + 1);
      if (c + 3 < nch) load(gb, ub, c + 3);
    }
  }
  g = group_sum_last<LPR>(g);
  u = group_sum_last<LPR>(u);
  if (li == LPR - 1 && live) out[f] = silu_mul(g, u);
}

// grid.x: tiles of 256/LPR outputs h; grid.y: token t.  Each lane walks a flat
// list of (pick j, block) tasks -- the token's k routed rows h, then the shared
// row h -- two register chunks at a time.
template <int QT, int LPR, int XR>
__global__ __launch_bounds__(256) void k_down_accum(
    const float *__restrict__ act, const int32_t *__restrict__ ids, const float *__restrict__ wts, int T,
    int H, int k, int F, int SF, const uint8_t *__restrict__ down_exps, const uint8_t *__restrict__ down_sh,
    float *__restrict__ resid) {
  extern __shared__ float smem[];
  constexpr int BS = QBlock<QT>::bytes;
  constexpr int ROWS = 256 / LPR;
  const int t = blockIdx.y;
  const int nbF = F >> 5, nbS = SF >> 5;
  const int nbAll = k * nbF + nbS;
  float *xs = smem, *sx = smem + nbAll * XSTRIDE;
  const int gi = threadIdx.x / LPR, li = threadIdx.x % LPR;
  const int h = blockIdx.x * ROWS + gi;
  const bool live = h < H;
  const int bplF = nbF / LPR, bplS = nbS / LPR;  // LPR divides both
  const int nqF = k * bplF, nq = nqF + bplS;
  const int nch = (nq + NCH - 1) / NCH;
  const size_t mat = (size_t)H * nbF * BS;
  const uint32_t rowF = (uint32_t)h * nbF * BS;
  const uint32_t rowS = (uint32_t)h * nbS * BS;
  const int32_t *tid_ids = ids + (size_t)t * k;
  const float *tw = wts + (size_t)t * k;

  Stage<XR> ast;  // the token's act row: its k routed rows, then the shared row
  stage_load(ast, act + (size_t)t * (k * F + SF), k * F + SF);

  // task q: routed pick j = q / bplF (block li + LPR*(q % bplF)), then the shared row
  auto pick = [&](int q) { return q < nqF ? q / bplF : k; };
  auto block = [&](int q, int j) { return li + LPR * (q < nqF ? q - j * bplF : q - nqF); };
  auto rsrc_for = [&](int j) {
    return j < k ? make_rsrc(down_exps + (size_t)tid_ids[j] * mat, (uint32_t)mat)
                 : make_rsrc(down_sh, (uint32_t)((size_t)H * nbS * BS));
  };
  auto offset = [&](int q, int j) {
    return (live && q < nq) ? (j < k ? rowF : rowS) + (uint32_t)block(q, j) * BS : OOB;
  };
  Raw5 A[NCH], B[NCH];
  auto load = [&](Raw5 *W, int c) {
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const int q = c * NCH + i, j = pick(q);
      W[i] = QBlock<QT>::load(rsrc_for(j), offset(q, j));
    }
  };
  float acc = 0.f;
  auto compute = [&](const Raw5 *W, int c) {
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const int q = c * NCH + i, j = pick(q);
      const int ab = min(j * nbF + block(q, j), nbAll - 1);  // staged act block (shared row after routed)
      const float d = block_dot<QT>(W[i], offset(q, j), xs + ab * XSTRIDE, sx[ab]);
      acc = __builtin_fmaf(j < k ? tw[min(j, k - 1)] : 1.0f, d, acc);
    }
  };

  load(A, 0);
  if (nch > 1) load(B, 1);
  stage_store(ast, k * F + SF, xs, sx);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    compute(A, c);
    if (c + 2 < nch) load(A, c + 2);
    if (c + 1 < nch) {
      compute(B, c + 1);
      if (c + 3 < nch) load(B, c + 3);
    }
  }
  acc = group_sum_last<LPR>(acc);
  if (li == LPR - 1 && live) resid[(size_t)t * H + h] += acc;
}

// ---------------------------------------------------------------- launch --

static inline int lanes_for(int nb) {
  int l = nb & -nb;  // largest power of two dividing nb
  return l > 16 ? 16 : l;
}
static inline int xr_for(int n) {  // float4s per thread to stage n floats with 256 threads
  int need = (n / 4 + 255) / 256, xr = 1;
  while (xr < need) xr <<= 1;
  return xr;
}

template <int QT, int LPR, int XR>
static void gateup_launch(const DecodeArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  MOE_LAUNCH(3, (k_gateup_swiglu<QT, LPR, XR>), grid, dim3(256), (uint32_t)lds, st, a.x, a.ids, a.wts, a.logits,
             a.bias, a.sel, a.T, a.H, a.k, a.F, a.SF, a.gate_exps, a.up_exps, a.gate_sh, a.up_sh, a.act);
}
template <int QT, int LPR, int XR>
static void down_launch(const DecodeArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  MOE_LAUNCH(4, (k_down_accum<QT, LPR, XR>), grid, dim3(256), (uint32_t)lds, st, (const float *)a.act,
             (const int32_t *)a.ids, (const float *)a.wts, a.T, a.H, a.k, a.F, a.SF, a.down_exps, a.down_sh, a.resid);
}

#define MOE_XR_SWITCH(FN, QT, LPR)                  \
  switch (xr) {                                      \
    case 1: FN<QT, LPR, 1>(a, grid, lds, st); break;  \
    case 2: FN<QT, LPR, 2>(a, grid, lds, st); break;  \
    case 4: FN<QT, LPR, 4>(a, grid, lds, st); break;  \
    case 8: FN<QT, LPR, 8>(a, grid, lds, st); break;  \
    default: FN<QT, LPR, 16>(a, grid, lds, st); break; \
  }
#define MOE_LPR_SWITCH(FN, QT)                        \
  switch (lpr) {                                       \
    case 1: MOE_XR_SWITCH(FN, QT, 1) break;            \
    case 2: MOE_XR_SWITCH(FN, QT, 2) break;            \
    case 4: MOE_XR_SWITCH(FN, QT, 4) break;            \
    case 8: MOE_XR_SWITCH(FN, QT, 8) break;            \
    default: MOE_XR_SWITCH(FN, QT, 16) break;          \
  }

template <int QT>
static hipError_t gateup_q(const DecodeArgs &a, hipStream_t st) {
  const int nbH = a.H / 32;
  const int lpr = lanes_for(nbH);
  const int rows = 256 / lpr;
  const int maxrows = a.F > a.SF ? a.F : a.SF;
  const dim3 grid((maxrows + rows - 1) / rows, a.T * a.k + (a.SF > 0 ? a.T : 0));
  const size_t lds = (size_t)nbH * (XSTRIDE + 1) * sizeof(float);
  const int xr = xr_for(a.H);
  MOE_LPR_SWITCH(gateup_launch, QT)
  return hipGetLastError();
}

template <int QT>
static hipError_t down_q(const DecodeArgs &a, hipStream_t st) {
  const int nbF = a.F / 32, nbS = a.SF / 32;
  int lpr = lanes_for(nbF);
  if (nbS > 0 && lanes_for(nbS) < lpr) lpr = lanes_for(nbS);
  const int rows = 256 / lpr;
  const dim3 grid((a.H + rows - 1) / rows, a.T);
  const size_t lds = (size_t)(a.k * nbF + nbS) * (XSTRIDE + 1) * sizeof(float);
  const int xr = xr_for(a.k * a.F + a.SF);
  MOE_LPR_SWITCH(down_launch, QT)
  return hipGetLastError();
}

}  // namespace moe
