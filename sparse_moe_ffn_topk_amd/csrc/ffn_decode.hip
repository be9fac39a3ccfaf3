// ffn_decode.hip -- expert FFNs for small T (decode): fused dequant-GEMVs
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
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

// Stage n floats of `src` into LDS as blocks of 32 (stride XSTRIDE) and write
// each block's sum to sx[]. Block-wide; n % 32 == 0.
__device__ __forceinline__ void stage_blocks(const float *__restrict__ src, int n, float *xs, float *sx) {
  const int tid = threadIdx.x, nt = blockDim.x;
  // 8 consecutive threads load one block as float4s and sum it.
  const int nb = n >> 5;
  for (int base = 0; base < nb * 8; base += nt) {
    int idx = base + tid;  // float4 index
    int b = idx >> 3, c = idx & 7;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (b < nb) {
      v = reinterpret_cast<const float4 *>(src)[idx];
      *reinterpret_cast<float4 *>(xs + b * XSTRIDE + 4 * c) = v;
    }
    float s = (v.x + v.y) + (v.z + v.w);
    s = group_sum(s, 8);
    if (b < nb && c == 0) sx[b] = s;
  }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// grid.x: row tiles of 256/LPR rows; grid.y: pair p (T*k routed, then T shared).
template <int QT, int LPR>
__global__ __launch_bounds__(256) void k_gateup_swiglu(
    const float *__restrict__ x, const int32_t *__restrict__ ids, int T, int H, int k, int F, int SF,
    const uint8_t *__restrict__ gate_exps, const uint8_t *__restrict__ up_exps,
    const uint8_t *__restrict__ gate_sh, const uint8_t *__restrict__ up_sh, float *__restrict__ act) {
  extern __shared__ float smem[];
  constexpr int BS = QBlock<QT>::bytes;
  constexpr int ROWS = 256 / LPR;
  const int nbH = H >> 5;
  const int p = blockIdx.y;
  const int nroute = T * k;
  int t, rows;
  const uint8_t *gbase, *ubase;
  float *out;
  if (p < nroute) {
    t = p / k;
    const int e = ids[p];
    rows = F;
    const size_t mat = (size_t)F * nbH * BS;
    gbase = gate_exps + (size_t)e * mat;
    ubase = up_exps + (size_t)e * mat;
    out = act + (size_t)p * F;
  } else {
    t = p - nroute;
    rows = SF;
    gbase = gate_sh;
    ubase = up_sh;
    out = act + (size_t)nroute * F + (size_t)t * SF;
  }
  const int f0 = blockIdx.x * ROWS;
  if (f0 >= rows) return;

  float *xs = smem, *sx = smem + nbH * XSTRIDE;
  stage_blocks(x + (size_t)t * H, H, xs, sx);
  __syncthreads();

  const uint32_t mbytes = (uint32_t)((size_t)rows * nbH * BS);
  const rsrc_t rg = make_rsrc(gbase, mbytes), ru = make_rsrc(ubase, mbytes);
  const int gi = threadIdx.x / LPR, li = threadIdx.x % LPR;
  const int f = f0 + gi;
  float g = 0.f, u = 0.f;
  if (f < rows) {
    const uint32_t rowoff = (uint32_t)f * nbH * BS;
#pragma unroll 2
    for (int b = li; b < nbH; b += LPR) {
      const uint32_t off = rowoff + (uint32_t)b * BS;
      Raw5 wg = QBlock<QT>::load(rg, off);
      Raw5 wu = QBlock<QT>::load(ru, off);
      const float *xb = xs + b * XSTRIDE;
      const float s = sx[b];
      g += block_dot<QT>(wg, off, xb, s);
      u += block_dot<QT>(wu, off, xb, s);
    }
  }
  g = group_sum(g, LPR);
  u = group_sum(u, LPR);
  if (li == 0 && f < rows) out[f] = silu_mul(g, u);
}

// grid.x: tiles of 256/LPR outputs h; grid.y: token t.
template <int QT, int LPR>
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
  // the token's k act rows are contiguous; the shared act row follows them
  stage_blocks(act + (size_t)t * k * F, k * F, xs, sx);
  if (SF > 0)
    stage_blocks(act + (size_t)T * k * F + (size_t)t * SF, SF, xs + k * nbF * XSTRIDE, sx + k * nbF);
  __syncthreads();

  const int gi = threadIdx.x / LPR, li = threadIdx.x % LPR;
  const int h = blockIdx.x * ROWS + gi;
  float acc = 0.f;
  if (h < H) {
    const size_t mat = (size_t)H * nbF * BS;
    const uint32_t rowoff = (uint32_t)h * nbF * BS;
    for (int j = 0; j < k; j++) {
      const int e = ids[(size_t)t * k + j];
      const float w = wts[(size_t)t * k + j];
      const rsrc_t rd = make_rsrc(down_exps + (size_t)e * mat, (uint32_t)mat);
      float part = 0.f;
#pragma unroll 2
      for (int b = li; b < nbF; b += LPR) {
        const uint32_t off = rowoff + (uint32_t)b * BS;
        Raw5 wd = QBlock<QT>::load(rd, off);
        const int ab = j * nbF + b;
        part += block_dot<QT>(wd, off, xs + ab * XSTRIDE, sx[ab]);
      }
      acc = __builtin_fmaf(w, part, acc);
    }
    if (SF > 0) {
      const uint32_t smat = (uint32_t)((size_t)H * nbS * BS);
      const rsrc_t rs = make_rsrc(down_sh, smat);
      const uint32_t srow = (uint32_t)h * nbS * BS;
#pragma unroll 2
      for (int b = li; b < nbS; b += LPR) {
        const uint32_t off = srow + (uint32_t)b * BS;
        Raw5 wd = QBlock<QT>::load(rs, off);
        const int ab = k * nbF + b;
        acc += block_dot<QT>(wd, off, xs + ab * XSTRIDE, sx[ab]);
      }
    }
  }
  acc = group_sum(acc, LPR);
  if (li == 0 && h < H) resid[(size_t)t * H + h] += acc;
}

// ---------------------------------------------------------------- launch --

static int lanes_for(int nb) {
  int l = nb & -nb;  // largest power of two dividing nb
  return l > 16 ? 16 : l;
}

template <int QT>
static hipError_t gateup_q(const DecodeArgs &a, hipStream_t st) {
  const int nbH = a.H / 32;
  const int lpr = lanes_for(nbH);
  const int rows = 256 / lpr;
  const int maxrows = a.F > a.SF ? a.F : a.SF;
  dim3 grid((maxrows + rows - 1) / rows, a.T * a.k + (a.SF > 0 ? a.T : 0));
  const size_t lds = (size_t)nbH * (XSTRIDE + 1) * sizeof(float);
#define MOE_GU(L)                                                                                         \
  k_gateup_swiglu<QT, L><<<grid, 256, lds, st>>>(a.x, a.ids, a.T, a.H, a.k, a.F, a.SF, a.gate_exps, \
                                                   a.up_exps, a.gate_sh, a.up_sh, a.act)
  switch (lpr) {
    case 1: MOE_GU(1); break;
    case 2: MOE_GU(2); break;
    case 4: MOE_GU(4); break;
    case 8: MOE_GU(8); break;
    default: MOE_GU(16); break;
  }
#undef MOE_GU
  return hipGetLastError();
}

template <int QT>
static hipError_t down_q(const DecodeArgs &a, hipStream_t st) {
  const int nbF = a.F / 32, nbS = a.SF / 32;
  int lpr = lanes_for(nbF);
  if (nbS > 0 && lanes_for(nbS) < lpr) lpr = lanes_for(nbS);
  const int rows = 256 / lpr;
  dim3 grid((a.H + rows - 1) / rows, a.T);
  const size_t lds = (size_t)(a.k * nbF + nbS) * (XSTRIDE + 1) * sizeof(float);
#define MOE_DN(L)                                                                                   \
  k_down_accum<QT, L><<<grid, 256, lds, st>>>(a.act, a.ids, a.wts, a.T, a.H, a.k, a.F, a.SF, \
                                                a.down_exps, a.down_sh, a.resid)
  switch (lpr) {
    case 1: MOE_DN(1); break;
    case 2: MOE_DN(2); break;
    case 4: MOE_DN(4); break;
    case 8: MOE_DN(8); break;
    default: MOE_DN(16); break;
  }
#undef MOE_DN
  return hipGetLastError();
}

size_t decode_down_lds_bytes(int k, int F, int SF) {
  return (size_t)(k * (F / 32) + SF / 32) * (XSTRIDE + 1) * sizeof(float);
}

hipError_t launch_decode_ffn(const DecodeArgs &a, hipStream_t st) {
  hipError_t e = a.qtype == MOE_Q4_1 ? gateup_q<MOE_Q4_1>(a, st) : gateup_q<MOE_Q4_0>(a, st);
  if (e != hipSuccess) return e;
  return a.qtype == MOE_Q4_1 ? down_q<MOE_Q4_1>(a, st) : down_q<MOE_Q4_0>(a, st);
}

}  // namespace moe
