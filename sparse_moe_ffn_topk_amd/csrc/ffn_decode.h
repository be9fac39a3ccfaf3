// ffn_decode.h -- expert FFNs for small T (decode): fused dequant-GEMVs
// read straight from GGUF Q4_0 / Q4_1 / Q8_0 blocks (gfx950, wave64).
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
//  * nibbles are unpacked in registers against the input block staged in
//    LDS: each goes to a byte of its own, two bytes convert to exact f16 q in
//    one E4M3 conversion, and each product is a mixed f16 x f32 fma (Q8_0
//    bytes: v_cvt_f32_ubyte*, FMA); the Q4_1 offset term m*sum(x) uses the
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

// Blocks per lane held in registers per chunk, two chunks in flight.  In the
// gate||up kernel 1 (95 registers against 138 at 2: five waves per SIMD
// instead of three for launches of a thousand blocks and more, and for one
// token a lane's two blocks of a 32-lane row go out as two chunks, so the
// first is computed while the second arrives), except 2 for one token of
// Q4_0 blocks and for one token of a dense layer, where 2 measured faster.  In
// the down kernel 4 where a row's task list is split over waves (one token),
// and 1 where it is not (several tokens: a launch of a thousand blocks then
// stays resident at once, which at 4 per chunk and 204 registers took two
// rounds; 2 per chunk measured 1 % slower at eight tokens); a split list whose
// waves' task counts are not a multiple of 4 takes one block per chunk
// (down_launch_nt).
constexpr int NCH_GU = 1;
constexpr int NCH_GU_PAIR = 2;
constexpr int NCHD = 4;
constexpr int NCHD_UNSPLIT = 1;
// Offset past every buffer resource's range: loads there return zeros without
// touching memory, and an all-zero block contributes exactly 0 to a dot.
constexpr uint32_t OOB = 0x7ffffff0u;

// Input staging in two halves so its loads are issued before the weight
// loads and its LDS writes happen after them.  stage_load() reads the n floats
// of src into registers (XR float4 per thread of NT; loads past n return
// zeros); stage_store() writes them as blocks of 32 (stride XSTRIDE) and each
// block's sum to sx[].  n % 32 == 0, n <= 4 * NT * XR.
template <int XR>
struct Stage {
  float4 v[XR];
};
template <int NT, int XR>
__device__ __forceinline__ void stage_load(Stage<XR> &st, const float *src, int n) {
  const rsrc_t r = make_rsrc(src, (uint32_t)n * 4u);
#pragma unroll
  for (int i = 0; i < XR; i++) {
    // (element-wise: __builtin_bit_cast of an ext-vector element reads element 0 with this compiler)
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)((threadIdx.x + NT * i) * 16), 0, 0);
    const uint32_t a0 = v.x, a1 = v.y, a2 = v.z, a3 = v.w;
    st.v[i] = make_float4(__uint_as_float(a0), __uint_as_float(a1), __uint_as_float(a2), __uint_as_float(a3));
  }
}
template <int NT, int XR>
__device__ __forceinline__ void stage_store(const Stage<XR> &st, int n, float *xs, float *sx) {
  const int n4 = n >> 2;
#pragma unroll
  for (int i = 0; i < XR; i++) {
    const int q = threadIdx.x + NT * i;
    const int b = q >> 3, c = q & 7;
    const float4 v = st.v[i];
    if (q < n4) *reinterpret_cast<float4 *>(xs + b * XSTRIDE + 4 * c) = v;
    // 8 consecutive lanes hold one block; the last of them gets its sum
    const float s = group_sum_last<8>((v.x + v.y) + (v.z + v.w));
    if (q < n4 && c == 7) sx[b] = s;
  }
}

// silu(g) * u, with the SwiGLU clamp when L > 0: min(silu(g), L) * clamp(u, -L, L)
// (the ling_moe_ssd.js page's swiglu kernel).
__device__ __forceinline__ float silu_mul(float g, float u, float L) {
  float sg = g / (1.0f + __expf(-g));
  if (L > 0.f) {
    u = fminf(fmaxf(u, -L), L);
    sg = fminf(sg, L);
  }
  return sg * u;
}

// grid.x: NB blocks per token; grid.y: token t.  A wave task is RW = 64/LPR
// rows (one per lane group) of a gate/up matrix pair.  Token t's tasks are the
// shared expert's rows first, then pick j's rows for j = 0..k-1; task u runs
// on wave u / NB of block u % NB.  So the first waves of every block stream
// shared rows, whose loads are issued before routing, and the routed waves
// issue theirs as soon as the block has routed the token.
// act row of token t: its k routed rows of F, then the shared row of SF.
// With logits != NULL every block routes its token (select_load/select_rank)
// and block (0, t) writes the token's ids and weights; otherwise ids are read.
template <int QT, int LPR, int XR, int CH>
__global__ __launch_bounds__(256, 2) void k_gateup_swiglu(
    const float *__restrict__ x, int32_t *__restrict__ ids, float *__restrict__ wts,
    const float *__restrict__ logits, const float *__restrict__ bias, SelParams P, int H, int k, int F, int SF,
    int sf_tasks, const uint8_t *__restrict__ gate_exps, const uint8_t *__restrict__ up_exps,
    const uint8_t *__restrict__ gate_sh, const uint8_t *__restrict__ up_sh, float lim, float lim_sh,
    float *__restrict__ act) {
  extern __shared__ float smem[];
  __shared__ SelShared sh;
  constexpr int BS = QBlock<QT>::bytes;
  constexpr int RW = 64 / LPR;
  const int nbH = H >> 5;
  const int t = blockIdx.y, NB = gridDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, gi = lane / LPR, li = lane % LPR;
  const int nsw = (sf_tasks + RW - 1) / RW, nfw = (F + RW - 1) / RW;  // (sf_tasks: SF, or 0 when done elsewhere)
  const int u = wave * NB + blockIdx.x;
  const bool is_sh = u < nsw;
  const bool wlive = u < nsw + k * nfw;
  const int j = (is_sh || k == 0) ? 0 : min((u - nsw) / nfw, k - 1);  // (no routed tasks when k == 0)
  const int row = (is_sh ? u : u - nsw - j * nfw) * RW + gi;
  const bool live = wlive && row < (is_sh ? SF : F);
  const uint32_t rowbytes = (uint32_t)nbH * BS;
  const uint32_t rowoff = live ? (uint32_t)row * rowbytes : 0u;
  float *out = act + (size_t)t * ((size_t)k * F + SF) + (is_sh ? (size_t)k * F : (size_t)j * F);

  // input, then router inputs, then (shared waves) weights: in-order retirement
  // lets routing wait for the first two only
  Stage<XR> xst;
  stage_load<256, XR>(xst, x + (size_t)t * H, H);
  SelIn in{};
  int e = 0;
  if (logits)
    select_load(logits + (size_t)t * P.E, bias, P, in);
  else if (!is_sh && wlive)
    e = ids[(size_t)t * k + j];

  const int nch = (nbH / LPR + CH - 1) / CH;  // LPR divides nbH
  typedef typename QBlock<QT>::Raw Raw;
  Raw ga[CH], ua[CH], gb[CH], ub[CH];
  rsrc_t rg = make_rsrc(gate_sh, (uint32_t)SF * rowbytes), ru = make_rsrc(up_sh, (uint32_t)SF * rowbytes);
  auto offset = [&](int c, int i) {
    const int b = li + LPR * (c * CH + i);
    return (live && b < nbH) ? rowoff + (uint32_t)b * BS : OOB;
  };
  // early: every wave issues the same loads (routed waves at the out-of-range
  // offset, which moves no data), so each wave has the same count in flight and
  // routing waits for exactly its own inputs
  auto load = [&](Raw *G, Raw *U, int c, bool early) {
#pragma unroll
    for (int i = 0; i < CH; i++) {
      const uint32_t off = (early && !is_sh) ? OOB : offset(c, i);
      G[i] = QBlock<QT>::load(rg, off);
      U[i] = QBlock<QT>::load(ru, off);
    }
  };
  load(ga, ua, 0, true);
  load(gb, ub, 1, true);  // (past the row end: out of range, no data moves)
  if (logits) {
    const bool writer = blockIdx.x == 0;
    select_rank(in, P, sh, writer ? wts + (size_t)t * k : nullptr);
    if (writer && threadIdx.x < k) ids[(size_t)t * k + threadIdx.x] = sh.pick[threadIdx.x];
    e = __builtin_amdgcn_readfirstlane(sh.pick[j]);
  }
  if (!is_sh) {  // the routed loads go out first: the input's LDS stores are off their path
    const size_t mat = (size_t)F * rowbytes;
    rg = make_rsrc(gate_exps + (size_t)e * mat, (uint32_t)mat);
    ru = make_rsrc(up_exps + (size_t)e * mat, (uint32_t)mat);
    load(ga, ua, 0, false);
    if (nch > 1) load(gb, ub, 1, false);
  }
  float *xs = smem, *sx = smem + nbH * XSTRIDE;
  stage_store<256, XR>(xst, H, xs, sx);
  __syncthreads();

  float g = 0.f, v = 0.f;
  auto compute = [&](const Raw *G, const Raw *U, int c) {
#pragma unroll
    for (int i = 0; i < CH; i++) {
      const uint32_t off = offset(c, i);
      const int b = min(li + LPR * (c * CH + i), nbH - 1);
      const float *xb = xs + b * XSTRIDE;
      const float s = sx[b];
      g += block_dot<QT>(G[i], off, xb, s);
      v += block_dot<QT>(U[i], off, xb, s);
    }
  };
  for (int c = 0; c < nch; c += 2) {
    compute(ga, ua, c);
    if (c + 2 < nch) load(ga, ua, c + 2, false);
    if (c + 1 < nch) {
      compute(gb, ub, c + 1);
      if (c + 3 < nch) load(gb, ub, c + 3, false);
    }
  }
  g = group_sum_last<LPR>(g);
  v = group_sum_last<LPR>(v);
  if (li == LPR - 1 && live) out[row] = silu_mul(g, v, is_sh ? lim_sh : lim);
}

// Sum of a float over the whole wave (row sums, then the four rows in a fixed
// order); the result is uniform.
__device__ __forceinline__ float wave_sum_f(float v) {
  v = group_sum_last<16>(v);
  auto rl = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  return (rl(15) + rl(31)) + (rl(47) + rl(63));
}

// Prelude of a decode step of several tokens, in one launch.  Blocks
// [0, nsel) route token blockIdx.x (select_block: ids and weights).  The other
// blocks compute the shared expert's gate||up rows for groups of up to TG
// tokens, so its weights stream once per group rather than once per token:
// shared block s takes rows 4 (s % nrg) + wave (nrg = SF/4 rounded up) for the
// tokens of group s / nrg.  A wave's 64 lanes split the row's blocks (lane i:
// blocks i and i + 64, so H <= 4096); each block is unpacked once and dotted
// with every token's input staged in LDS.  Writes act[t][k*F + f].
template <int QT, int XR, int TG>
__global__ __launch_bounds__(256) void k_decode_prelude(
    const float *__restrict__ logits, const float *__restrict__ bias, SelParams P, int nsel,
    int32_t *__restrict__ ids, float *__restrict__ wts, const float *__restrict__ x, int T, int H, int k, int F,
    int SF, const uint8_t *__restrict__ gate_sh, const uint8_t *__restrict__ up_sh, float lim_sh,
    float *__restrict__ act) {
  __shared__ SelShared sh;
  extern __shared__ float smem[];
  if ((int)blockIdx.x < nsel) {
    const int t = blockIdx.x;
    select_block(logits + (size_t)t * P.E, bias, P, sh, wts + (size_t)t * P.k);
    if ((int)threadIdx.x < P.k) ids[(size_t)t * P.k + threadIdx.x] = sh.pick[threadIdx.x];
    return;
  }
  constexpr int BS = QBlock<QT>::bytes;
  constexpr int NBL = 2;  // blocks per lane
  const int nbH = H >> 5;
  const int nrg = (SF + 3) >> 2;
  const int s = (int)blockIdx.x - nsel;
  const int t0 = (s / nrg) * TG, nt = min(TG, T - t0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row = (s % nrg) * 4 + wave;
  const bool live = row < SF;
  const uint32_t rowbytes = (uint32_t)nbH * BS;

  // the group's inputs (tokens past T read as zeros), then the weights, then
  // the LDS stores: the weight loads are in flight while the inputs land
  Stage<XR> xst[TG];
#pragma unroll
  for (int tt = 0; tt < TG; tt++)
    stage_load<256, XR>(xst[tt], x + (size_t)min(t0 + tt, T - 1) * H, tt < nt ? H : 0);
  typedef typename QBlock<QT>::Raw Raw;
  Raw gw[NBL], uw[NBL];
  const rsrc_t rg = make_rsrc(gate_sh, (uint32_t)SF * rowbytes), ru = make_rsrc(up_sh, (uint32_t)SF * rowbytes);
  auto offset = [&](int i) {
    const int b = lane + 64 * i;
    return (live && b < nbH) ? (uint32_t)row * rowbytes + (uint32_t)b * BS : OOB;
  };
#pragma unroll
  for (int i = 0; i < NBL; i++) {
    gw[i] = QBlock<QT>::load(rg, offset(i));
    uw[i] = QBlock<QT>::load(ru, offset(i));
  }
  float *xs = smem, *sx = smem + TG * nbH * XSTRIDE;  // token tt: blocks at tt*nbH*XSTRIDE, sums at tt*nbH
#pragma unroll
  for (int tt = 0; tt < TG; tt++) stage_store<256, XR>(xst[tt], H, xs + tt * nbH * XSTRIDE, sx + tt * nbH);
  __syncthreads();

  float ga[TG], ua[TG];
#pragma unroll
  for (int tt = 0; tt < TG; tt++) ga[tt] = ua[tt] = 0.f;
  // 2-byte-aligned blocks (Q4_0, Q8_0) are shifted once so that every block
  // starts at byte 0 of its first dword (offset 0 below): the accessors then
  // select nothing per lane
  auto realign = [&](Raw &r, uint32_t off) {
    if constexpr (QT != MOE_Q4_1) {
      constexpr int NW = sizeof(Raw) / 4;
      const bool odd = (off & 2u) != 0u;
#pragma unroll
      for (int j = 0; j < NW; j++) {
        const uint32_t nx = j + 1 < NW ? r.w[j + 1] : 0u;
        r.w[j] = odd ? __builtin_amdgcn_alignbyte(nx, r.w[j], 2) : r.w[j];
      }
    }
  };
#pragma unroll
  for (int i = 0; i < NBL; i++) {
    realign(gw[i], offset(i));
    realign(uw[i], offset(i));
  }
#pragma unroll
  for (int i = 0; i < NBL; i++) {
    if (64 * i >= nbH) break;  // (uniform: no lane has a block i)
    const int b = min(lane + 64 * i, nbH - 1);  // (blocks past the row are zeros: they add 0)
    float q[32], d, m;
    // (a scheduling barrier per token pair keeps the pair's 64 input reads next
    // to its FMAs instead of all tokens' inputs live at once)
    block_unpack<QT>(gw[i], 0u, q, d, m);
#pragma unroll
    for (int tt = 0; tt < TG; tt++) {
      ga[tt] += unpacked_dot(q, d, m, xs + (tt * nbH + b) * XSTRIDE, sx[tt * nbH + b]);
      if (tt & 1) __builtin_amdgcn_sched_barrier(0);
    }
    block_unpack<QT>(uw[i], 0u, q, d, m);
#pragma unroll
    for (int tt = 0; tt < TG; tt++) {
      ua[tt] += unpacked_dot(q, d, m, xs + (tt * nbH + b) * XSTRIDE, sx[tt * nbH + b]);
      if (tt & 1) __builtin_amdgcn_sched_barrier(0);
    }
  }
  float gv = 0.f, uv = 0.f;
#pragma unroll
  for (int tt = 0; tt < TG; tt++) {
    const float g = wave_sum_f(ga[tt]), u = wave_sum_f(ua[tt]);
    if (lane == tt) {
      gv = g;
      uv = u;
    }
  }
  if (live && lane < nt) act[(size_t)(t0 + lane) * ((size_t)k * F + SF) + (size_t)k * F + row] = silu_mul(gv, uv, lim_sh);
}

// grid.x: tiles of outputs h; grid.y: token t.  Each lane of a row's lane
// group walks a flat list of (row, block) tasks -- the shared row h first (its
// loads need no routing and go out at once), then the token's k routed rows h
// -- two register chunks at a time.  With S > 1 the list of a row is split
// over S waves of the block (wave s takes tasks s, s + S, ...), so long lists
// keep all their loads in flight; the S partial sums of a row are added in
// LDS in split order (fixed: bitwise reproducible).  A block is (NT/64)/S row
// groups of 64/LPR rows (SPLIT == false: S is 1).  The token's ids and
// weights are fetched into lanes 0..k-1 ahead of everything else.
template <int QT, int LPR, int XR, int NT, bool SPLIT, int CH>
__global__ __launch_bounds__(NT) void k_down_accum(
    const float *__restrict__ act, const int32_t *__restrict__ ids, const float *__restrict__ wts, int H, int k,
    int F, int SF, const uint8_t *__restrict__ down_exps, const uint8_t *__restrict__ down_sh,
    float *__restrict__ resid, int S_arg) {
  extern __shared__ float smem[];
  __shared__ float part[SPLIT ? NT / LPR : 1];  // [split][row of the block]
  const int S = SPLIT ? S_arg : 1;
  constexpr int BS = QBlock<QT>::bytes;
  constexpr int RPW = 64 / LPR;  // rows per wave
  const int rows = (NT / 64 / S) * RPW;
  const int t = blockIdx.y;
  const int nbF = F >> 5, nbS = SF >> 5;
  const int nbAll = k * nbF + nbS;
  float *xs = smem, *sx = smem + nbAll * XSTRIDE;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ws = wave % S, rg = wave / S;  // task split, row group
  const int gi = (threadIdx.x & 63) / LPR, li = threadIdx.x % LPR;
  const int rb = rg * RPW + gi;  // row within the block
  const int h = blockIdx.x * rows + rb;
  const bool live = h < H;
  const int bplF = nbF / LPR, bplS = nbS / LPR;  // LPR divides both
  const int nq = bplS + k * bplF;
  const int nqw = (nq - ws + S - 1) / S;  // this wave's tasks: q = ws + S * i
  const int nch = (nqw + CH - 1) / CH;
  const size_t mat = (size_t)H * nbF * BS;
  const uint32_t rowF = (uint32_t)h * nbF * BS;
  const uint32_t rowS = (uint32_t)h * nbS * BS;

  const uint32_t lane = threadIdx.x & 63;
  const rsrc_t rid = make_rsrc(ids + (size_t)t * k, (uint32_t)k * 4u);
  const rsrc_t rwt = make_rsrc(wts + (size_t)t * k, (uint32_t)k * 4u);
  const int id_v = (int)__builtin_amdgcn_raw_buffer_load_b32(rid, (int)(lane * 4u), 0, 0);
  const float wt_v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rwt, (int)(lane * 4u), 0, 0));
  Stage<XR> ast;  // the token's act row: its k routed rows, then the shared row
  stage_load<NT, XR>(ast, act + (size_t)t * (k * F + SF), k * F + SF);
  // the residual values this block updates, loaded now: the end of the kernel
  // then adds to them without another memory round trip
  const int hb = blockIdx.x * rows + (int)threadIdx.x;  // (SPLIT: thread i finishes row i of the block)
  const bool writer = SPLIT ? ((int)threadIdx.x < rows && hb < H) : (li == LPR - 1 && live);
  const float r_in = writer ? resid[(size_t)t * H + (SPLIT ? hb : h)] : 0.f;

  // task q: the shared row (j = k) for q < bplS, then pick j = (q - bplS) / bplF
  auto pick = [&](int q) { return (q < bplS || bplF == 0) ? k : (q - bplS) / bplF; };  // (k == 0: shared only)
  auto block = [&](int q, int j) { return li + LPR * (q < bplS ? q : q - bplS - j * bplF); };
  auto rsrc_for = [&](int j) {
    return j < k ? make_rsrc(down_exps + (size_t)__builtin_amdgcn_readlane(id_v, j) * mat, (uint32_t)mat)
                 : make_rsrc(down_sh, (uint32_t)((size_t)H * nbS * BS));
  };
  auto offset = [&](int q, int j) {
    return (live && q < nq) ? (j < k ? rowF : rowS) + (uint32_t)block(q, j) * BS : OOB;
  };
  typedef typename QBlock<QT>::Raw Raw;
  Raw A[CH], B[CH];
  auto load = [&](Raw *W, int c) {
#pragma unroll
    for (int i = 0; i < CH; i++) {
      const int q = ws + S * (c * CH + i), j = min(pick(q), k);
      W[i] = QBlock<QT>::load(rsrc_for(j), offset(q, j));
    }
  };
  float acc = 0.f;
  auto compute = [&](const Raw *W, int c) {
#pragma unroll
    for (int i = 0; i < CH; i++) {
      const int q = ws + S * (c * CH + i), j = min(pick(q), k);
      const int ab = min(j * nbF + block(q, j), nbAll - 1);  // staged act block (shared row after routed)
      const float d = block_dot<QT>(W[i], offset(q, j), xs + ab * XSTRIDE, sx[ab]);
      const int wbits = j < k ? __builtin_amdgcn_readlane(__float_as_int(wt_v), j) : __float_as_int(1.0f);
      acc = __builtin_fmaf(__int_as_float(wbits), d, acc);
    }
  };

  load(A, 0);
  if (nch > 1) load(B, 1);
  stage_store<NT, XR>(ast, k * F + SF, xs, sx);
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
  if constexpr (!SPLIT) {
    if (writer) resid[(size_t)t * H + h] = r_in + acc;
  } else {
    if (li == LPR - 1) part[ws * rows + rb] = acc;
    __syncthreads();
    if (writer) {
      float y = part[threadIdx.x];
      for (int s2 = 1; s2 < S; s2++) y += part[s2 * rows + threadIdx.x];
      resid[(size_t)t * H + hb] = r_in + y;
    }
  }
}

// ---------------------------------------------------------------- launch --

static inline int lanes_for(int nb) {
  int l = nb & -nb;  // largest power of two dividing nb
  return l > 16 ? 16 : l;
}
static inline int xr_for(int n, int nt) {  // float4s per thread to stage n floats with nt threads
  int need = (n / 4 + nt - 1) / nt, xr = 1;
  while (xr < need) xr <<= 1;
  return xr;
}

template <int QT, int LPR, int XR, int CH>
static void gateup_launch_ch(const DecodeArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  MOE_LAUNCH(3, (k_gateup_swiglu<QT, LPR, XR, CH>), grid, dim3(256), (uint32_t)lds, st, a.x, a.ids, a.wts, a.logits,
             a.bias, a.sel, a.H, a.k, a.F, a.SF, a.sf_tasks, a.gate_exps, a.up_exps, a.gate_sh, a.up_sh, a.lim,
             a.lim_sh, a.act);
}
template <int QT, int LPR, int XR>
static void gateup_launch(const DecodeArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  if (a.T == 1 && (QT == MOE_Q4_0 || a.k == 0))
    gateup_launch_ch<QT, LPR, XR, NCH_GU_PAIR>(a, grid, lds, st);
  else
    gateup_launch_ch<QT, LPR, XR, NCH_GU>(a, grid, lds, st);
}
template <int QT, int LPR, int XR, int NT, bool SPLIT, int CH>
static void down_launch_ch(const DecodeArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  MOE_LAUNCH(4, (k_down_accum<QT, LPR, XR, NT, SPLIT, CH>), grid, dim3(NT), (uint32_t)lds, st, (const float *)a.act,
             (const int32_t *)a.ids, (const float *)a.wts, a.H, a.k, a.F, a.SF, a.down_exps, a.down_sh, a.resid,
             a.down_split);
}
// Split task lists: NCHD blocks per chunk when a wave's task count is a
// multiple of it (every chunk full) in a 256-thread block, else one (chunks
// then follow each other two in flight; 512-thread blocks always take one, so
// that two of them fit a CU).  Measured per layer step against NCHD
// throughout: LFM2.5 (3 tasks a wave) 17.2 -> 16.3 us, with Q8_0 experts
// 22.6 -> 20.2, Ling (7) 24.0-24.4 -> 23.8; Flint (4) keeps NCHD (one block
// per chunk: 14.8 against 14.3).
template <int QT, int LPR, int XR, int NT, bool SPLIT>
static void down_launch_nt(const DecodeArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  if constexpr (SPLIT) {
    const int nq = a.k * ((a.F / 32) / LPR) + (a.SF / 32) / LPR;
    const int per_wave = (nq + a.down_split - 1) / a.down_split;
    if (NT == 512 || per_wave % NCHD != 0) {
      down_launch_ch<QT, LPR, XR, NT, true, 1>(a, grid, lds, st);
      return;
    }
  }
  down_launch_ch<QT, LPR, XR, NT, SPLIT, SPLIT ? NCHD : NCHD_UNSPLIT>(a, grid, lds, st);
}
template <int QT, int LPR, int XR>
static void down_launch_128(const DecodeArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  down_launch_nt<QT, LPR, XR, 128, false>(a, grid, lds, st);
}
template <int QT, int LPR, int XR>
static void down_launch_256(const DecodeArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  down_launch_nt<QT, LPR, XR, 256, false>(a, grid, lds, st);
}
template <int QT, int LPR, int XR>
static void down_launch_split(const DecodeArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  down_launch_nt<QT, LPR, XR, 256, true>(a, grid, lds, st);
}
template <int QT, int LPR, int XR>
static void down_launch_split512(const DecodeArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  down_launch_nt<QT, LPR, XR, 512, true>(a, grid, lds, st);
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

// Multi-token prelude.  Tokens per shared-expert group: 4, or 2 when T <= 2
// or when 4 tokens' inputs do not fit the LDS left beside the select state
// (0: the shared rows stay in the gate||up kernel, per token).
int prelude_token_group(int T, int H);
template <int QT, int XR, int TG>
static void prelude_launch(const DecodeArgs &a, int nsel, int nsh, size_t lds, hipStream_t st) {
  MOE_LAUNCH(10, (k_decode_prelude<QT, XR, TG>), dim3(nsel + nsh), dim3(256), (uint32_t)lds, st, a.logits, a.bias,
             a.sel, nsel, a.ids, a.wts, a.x, a.T, a.H, a.k, a.F, a.SF, a.gate_sh, a.up_sh, a.lim_sh, a.act);
}
// With several tokens: route each token once (when logits are given) and run
// the shared expert's gate||up for all tokens, in one launch; a is updated so
// the gate||up kernel then reads the ids and skips the shared rows.
template <int QT>
static hipError_t prelude_q(DecodeArgs &a, hipStream_t st) {
  a.sf_tasks = a.SF;
  if (a.T < 2) return hipSuccess;
  const int nsel = a.logits ? a.T : 0;
  const int tg = a.SF > 0 ? prelude_token_group(a.T, a.H) : 0;
  if (nsel == 0 && tg == 0) return hipSuccess;
  const int nsh = tg ? ((a.SF + 3) / 4) * ((a.T + tg - 1) / tg) : 0;
  const size_t lds = tg ? (size_t)tg * (a.H / 32) * (XSTRIDE + 1) * sizeof(float) : 0;
  const int xr = xr_for(a.H, 256);
#define MOE_PRELUDE_XR(TG)                                             \
  switch (xr) {                                                        \
    case 1: prelude_launch<QT, 1, TG>(a, nsel, nsh, lds, st); break;   \
    case 2: prelude_launch<QT, 2, TG>(a, nsel, nsh, lds, st); break;   \
    default: prelude_launch<QT, 4, TG>(a, nsel, nsh, lds, st); break;  \
  }
  if (tg >= 4) {
    MOE_PRELUDE_XR(4)
  } else {
    MOE_PRELUDE_XR(2)
  }
#undef MOE_PRELUDE_XR
  const hipError_t e = hipGetLastError();
  if (nsel) a.logits = nullptr;
  if (tg) a.sf_tasks = 0;
  return e;
}

#define MOE_LPR32_SWITCH(FN, QT)             \
  if (lpr == 32) {                            \
    MOE_XR_SWITCH(FN, QT, 32)                 \
  } else {                                    \
    MOE_LPR_SWITCH(FN, QT)                    \
  }
template <int QT>
static hipError_t gateup_q(const DecodeArgs &a, hipStream_t st) {
  const int nbH = a.H / 32;
  int lpr = lanes_for(nbH);
  // one token: 32 lanes per row where they divide the row and leave a lane at
  // most two blocks (all in flight at once, and the launch has twice the
  // blocks; for Q8_0 blocks 19.9 against 20.15 us per LFM2.5 layer step)
  if (a.T == 1 && lpr == 16 && nbH % 32 == 0 && nbH / 32 <= 2) lpr = 32;
  const int rw = 64 / lpr;  // rows per wave task
  const int tasks = (a.sf_tasks + rw - 1) / rw + a.k * ((a.F + rw - 1) / rw);
  if (tasks == 0) return hipSuccess;  // (a dense layer whose rows the prelude computed)
  const dim3 grid((tasks + 3) / 4, a.T);
  const size_t lds = (size_t)nbH * (XSTRIDE + 1) * sizeof(float);
  const int xr = xr_for(a.H, 256);
  MOE_LPR32_SWITCH(gateup_launch, QT)
  return hipGetLastError();
}

// Down launch shape.  The split S (waves per row group) is the smallest power
// of two <= 4 that leaves each lane at most one register chunk of blocks, as
// long as the launch stays within 512 blocks (two per CU: more waves and
// shorter serial chains); beyond that, at most two chunks (more blocks would
// each stage the act row again).  S > 1 runs 256-thread blocks, except that a
// split of 4 that still leaves a wave more than two tasks becomes a split of
// 8 in 512-thread blocks (as many blocks, each wave half the tasks: Ling 23.0-
// 23.3 -> 22.9 us per layer step, LFM2.5 16.0-16.2 -> 15.9, dense LFM2.5
// layers 22.0 -> 20.8).  Unsplit blocks are 256 threads, or 128 where 256
// would leave fewer than 256 blocks (so the launch covers the 256 CUs) and the
// act row still stages in 16 float4 per thread.
static inline int down_split(int nq, int per_lane) {
  int S = 1;
  while (S < 4 && (nq + S - 1) / S > per_lane) S <<= 1;
  return S;
}
template <int QT>
static hipError_t down_q(DecodeArgs a, hipStream_t st) {
  const int nbF = a.k > 0 ? a.F / 32 : 0, nbS = a.SF / 32;
  int lpr = nbF > 0 ? lanes_for(nbF) : 16;  // (a dense layer has only the shared row)
  if (nbS > 0 && lanes_for(nbS) < lpr) lpr = lanes_for(nbS);
  const size_t lds = (size_t)(a.k * nbF + nbS) * (XSTRIDE + 1) * sizeof(float);
  const int n = a.k * nbF * 32 + a.SF;
  const int nq = a.k * (nbF / lpr) + nbS / lpr;  // blocks per lane of a whole row
  int S = down_split(nq, NCHD);
  if (S > 1 && (size_t)((a.H + (4 / S) * (64 / lpr) - 1) / ((4 / S) * (64 / lpr))) * a.T > 512)
    S = down_split(nq, 2 * NCHD);
  const bool split8 = S == 4 && (nq + 3) / 4 > 2;
  if (split8) S = 8;
  auto rows_for = [&](int nt) { return (nt / 64 / S) * (64 / lpr); };
  const bool wide = S > 1 || (size_t)((a.H + rows_for(256) - 1) / rows_for(256)) * a.T >= 256 || n > 4 * 128 * 16;
  const int nt = split8 ? 512 : (wide ? 256 : 128);
  const dim3 grid((a.H + rows_for(nt) - 1) / rows_for(nt), a.T);
  const int xr = xr_for(n, nt);
  a.down_split = S;
  if (split8) {
    MOE_LPR_SWITCH(down_launch_split512, QT)
  } else if (S > 1) {
    MOE_LPR_SWITCH(down_launch_split, QT)
  } else if (wide) {
    MOE_LPR_SWITCH(down_launch_256, QT)
  } else {
    MOE_LPR_SWITCH(down_launch_128, QT)
  }
  return hipGetLastError();
}

}  // namespace moe
