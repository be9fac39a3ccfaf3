// prefill.hip -- expert FFNs for many tokens (chunked prefill): the (token,
// pick) pairs are grouped by expert and every expert runs as a small dense
// GEMM on the MFMA units (gfx950, v_mfma_f32_16x16x32_f16).
//
// What is computed is the same MoE FFN as the decode path (swiglu, moeAccum
// and moeAccumB of the diskformer ling_moe_ssd.js / lfm2_moe_ssd.js pages):
//   act[p][f] = silu(g) * u,  g = Wg_e x_t,  u = Wu_e x_t     (pair p = (t, j))
//   resid[t][h] += sum_j w_tj * (Wd_e act_p)[h] + shared(x_t)[h]
// The pages run one GEMV per (token, pick) pair with no grouping; grouping
// the pairs by expert is this library's design, so every expert's weights
// are read once per chunk.
//
// Steps:
//  1. k_sort_by_expert (block 0): a stable counting sort of the pairs by
//     expert, pair order (tokens ascending) within an expert: per-expert
//     token bit sets, popcount prefixes, an exclusive scan (wave shuffles) -> offsets, pos[p],
//     perm[pos], and the list of 16-token tiles of every expert.  Its other
//     blocks take the input rows' largest exponents (below), which do not
//     depend on the sort, so both share one launch.
//  2. k_group_gemm<GATEUP>: per (tile, 256-row slice): g and u for 16 tokens
//     x 256 rows, SwiGLU in registers, act rows written in sorted order; the
//     shared expert runs as extra tiles over all tokens.
//  3. k_group_gemm<DOWN>: Y[pos] = w_p * (Wd_e act_pos), shared Ysh[t].
//  4. k_combine: resid[t] += sum_j Y[pos(t, j)] + Ysh[t], fixed order: no
//     atomics, bitwise reproducible.
//
// Numerics of the GEMM: a Q4 block's nibbles q (and a Q8_0 block's bytes as
// q + 128) are exact in f16, so each
// block's MFMA partial sum_k q_k x_k is exact up to f32 accumulation once x
// is split as x = hi + lo (two f16, about 22 significant bits); the block's
// f32 scale d and offset term m * sum_k x_k are applied per block in f32
// (value d*q + m; Q4_0 is m = -8d).  The nibbles enter the MFMA as exact f16
// values: in the row-streaming kernels through the E4M3 conversion
// (nibbles_e4m3), in k_group_gemm by a mask-or that builds the f16 1024 + q
// and a packed f16 subtract that removes the 1024.  The row-streaming kernels
// add the offset term on the matrix cores too (two MFMAs per tile and chunk).
//
// f16 has a narrow exponent range, so every input row (a token's x, a pair's
// or a token's act) is first scaled by a power of two that puts its largest
// |value| in [2^14, 2^15): the hi + lo split then neither overflows nor drops
// into f16 subnormals at the top of the row, at any input scale.  The scale
// is exact; each tile's result is scaled back before the epilogue.  The
// exponents come from k_row_exp (x) and from the gate||up epilogue
// (atomicMax over the act values it writes).
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {


// Biased f32 exponent field of v.
__device__ __forceinline__ int bexp(float v) { return (int)((__float_as_uint(v) >> 23) & 0xffu); }

// The power-of-two shift that puts a row whose largest biased exponent is eb
// in [2^14, 2^15) (2^(eb - 127) <= max < 2^(eb - 126)).
__device__ __forceinline__ int row_shift(int eb) { return 141 - eb; }

// Largest biased f32 exponent of each of nrows rows of K floats (one wave per
// row: rows r = wpb * b + wave of block b of nb), and nzero ints zeroed.
// Where xhl is not NULL the row is also written scaled by 2^row_shift: each
// octet of values as its 8 f16 hi parts, then the 8 f16 lo parts (v - hi),
// 32 bytes, and each 32-value block's sum into xsum, added in the order the
// grouped gate||up kernel needs (each octet in order, then (octet 0 + octet 1)
// + (octet 2 + octet 3)).
__device__ __forceinline__ void row_exp_part(const float *__restrict__ rows, int nrows, int K, int32_t *__restrict__ eb,
                                             int32_t *__restrict__ zero, int nzero, int b, int nb,
                                             uint16_t *__restrict__ xhl, float *__restrict__ xsum) {
  const int nt = (int)blockDim.x, wpb = nt >> 6;
  for (int i = b * nt + (int)threadIdx.x; i < nzero; i += nb * nt) zero[i] = 0;
  const int r = b * wpb + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= nrows) return;
  const float4 *p = reinterpret_cast<const float4 *>(rows + (size_t)r * K);
  // octet o of the row (values 8 o .. 8 o + 7) scaled by 2^sh: its f16 hi and
  // lo parts, and its block's sum from the four octets' lanes (K / 8 octets,
  // a multiple of 4: the lanes that take a last, partial round hold whole
  // blocks, so the shuffles stay within active lanes)
  auto convert = [&](int o, int sh, float4 v0, float4 v1) {
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    half8 h, l;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float s = __builtin_ldexpf(v[i], sh);
      h[i] = (_Float16)s;
      l[i] = (_Float16)(s - (float)h[i]);
      sum += s;
    }
    half8 *dst = reinterpret_cast<half8 *>(xhl + ((size_t)r * K + 8 * (size_t)o) * 2);
    dst[0] = h;
    dst[1] = l;
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    if ((o & 3) == 0) xsum[(size_t)r * (K / 32) + (o >> 2)] = sum;
  };
  constexpr int RC = 8;  // octet rounds a lane holds in registers: rows of up to 4096 values
  if (xhl != nullptr && K <= 512 * RC) {
    float4 v[RC][2];
    int m = 0;
#pragma unroll
    for (int it = 0; it < RC; it++) {
      const int o = lane + 64 * it;
      if (o < K / 8) {
        v[it][0] = p[2 * o];
        v[it][1] = p[2 * o + 1];
        const float4 a = v[it][0], c = v[it][1];
        m = max(m, max(max(max(bexp(a.x), bexp(a.y)), max(bexp(a.z), bexp(a.w))),
                       max(max(bexp(c.x), bexp(c.y)), max(bexp(c.z), bexp(c.w)))));
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = max(m, __shfl_xor(m, d, 64));
    if (lane == 0) eb[r] = m;
    const int sh = row_shift(m);
#pragma unroll
    for (int it = 0; it < RC; it++) {
      const int o = lane + 64 * it;
      if (o < K / 8) convert(o, sh, v[it][0], v[it][1]);
    }
    return;
  }
  int m = 0;
  for (int i = lane; i < K / 4; i += 64) {
    const float4 v = p[i];
    m = max(m, max(max(bexp(v.x), bexp(v.y)), max(bexp(v.z), bexp(v.w))));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = max(m, __shfl_xor(m, d, 64));
  if (lane == 0) eb[r] = m;
  if (xhl == nullptr) return;
  const int sh = row_shift(m);
  for (int o = lane; o < K / 8; o += 64) convert(o, sh, p[2 * o], p[2 * o + 1]);
}

// ------------------------------------------------------------------ sort --

// One block of 1024 threads; T <= PREFILL_CHUNK, E <= 512.  The rank of pair
// p = (t, j) of expert e is the number of pairs of e that come before it in
// pair order: those of earlier tokens, then token t's own earlier picks of e.
//   bits[e][w]: bit t%32 of word w = t/32 set when token t picked e at all;
//   pre[e][w]:  pairs of e in the words before w.
// A token that lists an expert more than once (only ids a caller passes in
// can: the router never does) has one bit but several pairs; when the chunk
// holds such a token, the prefix and the rank add each earlier token's extra
// picks (a slower path).
template <typename P>
__device__ __forceinline__ int earlier_picks(P ids, int t, int k, int j, int e) {
  int n = 0;
  for (int i = 0; i < j; i++) n += ids[t * k + i] == e;
  return n;
}

// STAGE: the ids are first copied to LDS (after bits and pre) and read there.
// Block 0 sorts; blocks 1.. take the T input rows' largest exponents (H floats
// each, into xexp), their f16 hi + lo form and block sums (xhl, xsum; where
// xhl is not NULL), and zero nzero words at aexp, as k_row_exp does.
template <bool STAGE>
__global__ __launch_bounds__(1024) void k_sort_by_expert(const int32_t *__restrict__ gids, int T, int k, int E,
                                                         int32_t *__restrict__ offsets, int32_t *__restrict__ pos,
                                                         int32_t *__restrict__ perm, int32_t *__restrict__ tiles,
                                                         int32_t *__restrict__ ntiles, const float *__restrict__ x,
                                                         int H, int32_t *__restrict__ xexp,
                                                         int32_t *__restrict__ aexp, int nzero,
                                                         uint16_t *__restrict__ xhl, float *__restrict__ xsum) {
  if (blockIdx.x > 0) {
    row_exp_part(x, T, H, xexp, aexp, nzero, (int)blockIdx.x - 1, (int)gridDim.x - 1, xhl, xsum);
    return;
  }
  extern __shared__ uint32_t lds[];
  const int W = (T + 31) >> 5;
  uint32_t *bits = lds;                       // [E][W]
  uint16_t *pre = (uint16_t *)(lds + E * W);  // [E][W] (T * k <= 16384 pairs)
  int32_t *sids = (int32_t *)(lds + E * W + (E * W + 1) / 2);  // [T * k] (STAGE)
  __shared__ int cnt[512], off[513], toff[513];
  __shared__ int repeats;
  const int tid = threadIdx.x;
  const int np = T * k;
  for (int i = tid; i < E * W; i += 1024) bits[i] = 0u;
  if constexpr (STAGE)
    for (int i = tid; i < np; i += 1024) sids[i] = gids[i];
  if (tid == 0) repeats = 0;
  __syncthreads();
  const int32_t *ids = STAGE ? sids : gids;
  // (k <= SORT_KR: one thread per token with its ids in registers, so the
  // duplicate checks and the ranks below need no reloads)
  constexpr int SORT_KR = 8;
  const bool by_token = k <= SORT_KR;
  int te[SORT_KR];
  if (by_token) {
    if (tid < T) {
#pragma unroll
      for (int j = 0; j < SORT_KR; j++) te[j] = j < k ? ids[tid * k + j] : -1;
      bool dup = false;
#pragma unroll
      for (int j = 0; j < SORT_KR; j++) {
        bool first = true;
#pragma unroll
        for (int i = 0; i < j; i++) first = first && te[i] != te[j];
        if (j < k && first) atomicOr(&bits[te[j] * W + (tid >> 5)], 1u << (tid & 31));
        dup = dup || (j < k && !first);
      }
      if (dup) repeats = 1;
    }
  } else {
    for (int p = tid; p < np; p += 1024) {
      const int e = ids[p], t = p / k;
      if (earlier_picks(ids, t, k, p - t * k, e) == 0)
        atomicOr(&bits[e * W + (t >> 5)], 1u << (t & 31));
      else
        repeats = 1;
    }
  }
  __syncthreads();
  const bool rep = repeats != 0;
  if (tid < E) {
    int c = 0;
    if (!rep && W <= 16) {
      // all of the expert's words first (pre shares the LDS array, so a load
      // after a store could not be moved ahead of it)
      uint32_t bw[16];
#pragma unroll
      for (int w = 0; w < 16; w++) bw[w] = w < W ? bits[tid * W + w] : 0u;
#pragma unroll
      for (int w = 0; w < 16; w++)
        if (w < W) {
          pre[tid * W + w] = (uint16_t)c;
          c += __popc(bw[w]);
        }
    } else {
      for (int w = 0; w < W; w++) {
        pre[tid * W + w] = (uint16_t)c;
        const uint32_t b = bits[tid * W + w];
        c += __popc(b);
        if (rep)
          for (uint32_t m = b; m; m &= m - 1) c += earlier_picks(ids, 32 * w + __builtin_ctz(m), k, k, tid) - 1;
      }
    }
    cnt[tid] = c;
  }
  __syncthreads();
  // exclusive scans of the pair counts and of the 16-token tile counts over
  // the E <= 512 experts: inclusive scans within each wave (shuffles), then
  // the totals of the waves before it
  __shared__ int wsum[8], wtsum[8];
  const int lane = tid & 63, wave = tid >> 6;
  int v = 0, tv = 0;
  if (tid < 512) {
    v = tid < E ? cnt[tid] : 0;
    tv = (v + 15) >> 4;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int nv = __shfl_up(v, d, 64), ntv = __shfl_up(tv, d, 64);
      if (lane >= d) {
        v += nv;
        tv += ntv;
      }
    }
    if (lane == 63) {
      wsum[wave] = v;
      wtsum[wave] = tv;
    }
  }
  __syncthreads();
  if (tid < 512) {
    int o = 0, to = 0;
    for (int w = 0; w < wave; w++) {
      o += wsum[w];
      to += wtsum[w];
    }
    const int c = tid < E ? cnt[tid] : 0;
    if (tid < E) {
      off[tid] = o + v - c;
      toff[tid] = to + tv - ((c + 15) >> 4);
    }
    if (tid == E - 1) {
      off[E] = o + v;
      toff[E] = to + tv;
      *ntiles = to + tv;
    }
  }
  __syncthreads();
  for (int e = tid; e <= E; e += 1024) offsets[e] = off[e];
  if (tid < E) {
    const int nt = (cnt[tid] + 15) >> 4;
    for (int i = 0; i < nt; i++) {
      tiles[2 * (toff[tid] + i)] = tid;
      tiles[2 * (toff[tid] + i) + 1] = 16 * i;
    }
  }
  if (by_token && !rep) {
    // no token lists an expert twice: pair (t, j) of expert e ranks after the
    // pairs of e of the tokens before t
    if (tid < T) {
#pragma unroll
      for (int j = 0; j < SORT_KR; j++)
        if (j < k) {
          const int e = te[j];
          const uint32_t below = bits[e * W + (tid >> 5)] & ((1u << (tid & 31)) - 1u);
          const int q = off[e] + pre[e * W + (tid >> 5)] + __popc(below);
          pos[tid * k + j] = q;
          perm[q] = tid * k + j;
        }
    }
    return;
  }
  for (int p = tid; p < np; p += 1024) {
    const int e = ids[p], t = p / k, j = p - t * k;
    const uint32_t below = bits[e * W + (t >> 5)] & ((1u << (t & 31)) - 1u);
    int r = pre[e * W + (t >> 5)] + __popc(below) + earlier_picks(ids, t, k, j, e);
    if (rep) {  // earlier tokens of the word that picked e more than once
      for (uint32_t m = below; m; m &= m - 1) {
        const int t2 = (t & ~31) + __builtin_ctz(m);
        r += earlier_picks(ids, t2, k, k, e) - 1;
      }
    }
    const int q = off[e] + r;
    pos[p] = q;
    perm[q] = p;
  }
}

// ------------------------------------------------------------- grouped GEMM --

// (w & mask) | bits in one v_and_or_b32.  A VOP3 form takes no literal and
// at most one scalar operand here, so the mask sits in a scalar register and
// the bits in a vector register (set once); the compiler's own selection
// emits a separate and + or instead.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t bits) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(bits));
  return r;
}

// 8 nibbles of 8 bytes (the low halves, or the high halves with sh = 4) as
// exact f16 q, in the order k = 0,2,1,3,4,6,5,7 of the bytes (one mask-or per
// f16 pair: 0x6400 | q is the f16 1024 + q).
__device__ __forceinline__ half8 nibbles_f16(u32x2 nb, uint32_t sh) {
  const uint32_t w0 = nb.x >> sh, w1 = nb.y >> sh;
  const uint32_t a = and_or(w0, 0x000F000Fu, 0x64006400u), b = and_or(w0 >> 8, 0x000F000Fu, 0x64006400u);
  const uint32_t c = and_or(w1, 0x000F000Fu, 0x64006400u), d = and_or(w1 >> 8, 0x000F000Fu, 0x64006400u);
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v v = {a, b, c, d};
  // (1024 + q) - 1024 = q, exact in f16
  return __builtin_bit_cast(half8, v) - (half8)(_Float16)1024.0f;
}
// Position, within a lane's 8 A values, of byte j of its 8 nibble bytes
// (matches nibbles_f16's order 0,2,1,3,4,6,5,7).
__device__ __forceinline__ int kperm(int j) { return (j & 4) | ((j & 1) << 1) | ((j >> 1) & 1); }

// 8 bytes (Q8_0 values, already as q + 128) as exact f16 q + 128 in the same
// order 0,2,1,3,4,6,5,7 (two mask-ors per dword: f16 1024 + b, minus 1024).
__device__ __forceinline__ half8 bytes_f16(u32x2 nb) {
  const uint32_t w0 = nb.x, w1 = nb.y;
  const uint32_t a = and_or(w0, 0x00FF00FFu, 0x64006400u), b = and_or(w0 >> 8, 0x00FF00FFu, 0x64006400u);
  const uint32_t c = and_or(w1, 0x00FF00FFu, 0x64006400u), d = and_or(w1 >> 8, 0x00FF00FFu, 0x64006400u);
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v v = {a, b, c, d};
  return __builtin_bit_cast(half8, v) - (half8)(_Float16)1024.0f;
}

enum { GG_GATEUP = 0, GG_DOWN = 1 };

struct GemmArgs {
  int T, k, H, F, SF, E;
  const float *x;            // [T][H]
  const float *act;          // sorted act [T*k][F]
  const float *act_sh;       // [T][SF]
  const float *wts;          // [T*k]
  const int32_t *offsets, *perm, *tiles, *ntiles;
  const uint8_t *w0, *w1;    // gate, up (GATEUP) or down (DOWN): routed experts
  const uint8_t *s0, *s1;    // same for the shared expert
  float *out;                // GATEUP: sorted act; DOWN: Y [T*k][H]
  float *out_sh;             // GATEUP: act_sh; DOWN: Ysh [T][H]
  int max_routed_tiles;      // grid.x = max_routed_tiles + shared tiles
  int runw[4];               // row-streaming GEMMs: run weights by dispatch order on the CU (run_bounds; {0}: equal)
  float lim, lim_sh;         // GATEUP: SwiGLU clamp of routed / shared experts (0: none)
  const int32_t *xexp;       // [T] largest biased f32 exponent of |x| per token (k_row_exp)
  const uint16_t *xhl;       // [T][H/8][16]: x scaled by 2^row_shift(xexp), f16 hi + lo per octet (row-streaming form)
  const float *xsum;         // [T][H/32]: the scaled values' block sums
  int32_t *aexp;             // [T*k] then [T]: the same for the act rows (sorted, then shared);
                             // GATEUP raises them with atomicMax, DOWN reads them
};

// Largest biased exponent of |x| over each of nrows rows of K floats (one
// wave per row), with the rows' f16 hi + lo form and block sums where xhl is
// not NULL; the grid also zeroes nzero words at zero (the act rows'
// exponents, raised later by atomicMax).  For a layer with no routed pairs;
// otherwise the sort's launch does this in its blocks past the first.
__global__ __launch_bounds__(256) void k_row_exp(const float *__restrict__ rows, int nrows, int K,
                                                 int32_t *__restrict__ eb, int32_t *__restrict__ zero, int nzero,
                                                 uint16_t *__restrict__ xhl, float *__restrict__ xsum) {
  row_exp_part(rows, nrows, K, eb, zero, nzero, blockIdx.x, gridDim.x, xhl, xsum);
}

// K is walked in chunks of KB blocks.  Per chunk a block stages, in LDS, the
// raw bytes of its 256 weight rows (brow<QT>() bytes each: 4 x 20; 4 x 18 or
// 4 x 34 plus 2 bytes of alignment slack, rounded up to 16) read with
// contiguous 16-byte loads, and its 16 tokens' inputs as f16 hi + lo in the
// MFMA lanes' k order.
constexpr int KB = 4;
template <int QT>
constexpr int brow() { return QT == MOE_Q8_0 ? 144 : 80; }
constexpr int APAD = KB * 32 + 8;      // f16 per staged input row (16-byte pad)

// A chunk: 16 threads per token, 8 consecutive k each.
struct AStage {
  float v[8];
};
// (buffer loads: past the row, or for no row, they read zeros -- no branches,
// so the loads stay in order behind the weight loads).  r covers all the
// input rows (one resource for the wave: the rows differ per lane).
__device__ __forceinline__ void a_load(AStage &st, rsrc_t r, int K, int row, int kc) {
  const int seg = threadIdx.x & 15;
  const uint32_t kb = (uint32_t)(kc * 32 + seg * 8);
  const uint32_t rowoff = (uint32_t)(row >= 0 ? row : 0) * (uint32_t)K * 4u;
#pragma unroll
  for (int i = 0; i < 8; i += 4) {
    const uint32_t off = (row >= 0 && kb + i < (uint32_t)K) ? rowoff + (kb + i) * 4u : 0x7ffffff0u;
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    const uint32_t a0 = v.x, a1 = v.y, a2 = v.z, a3 = v.w;
    st.v[i] = __uint_as_float(a0);
    st.v[i + 1] = __uint_as_float(a1);
    st.v[i + 2] = __uint_as_float(a2);
    st.v[i + 3] = __uint_as_float(a3);
  }
}
// k within the block kk = (seg%4)*8 + i; the lane holding it has k-octet
// (kk%16)/8 + 2*(kk/16) and slot kperm(kk%8).  asum[block][token].
// sh: the row's power-of-two shift (row_shift).
__device__ __forceinline__ void a_store(const AStage &st, int sh, _Float16 (*ahi)[APAD], _Float16 (*alo)[APAD],
                                        float (*asum)[16]) {
  const int m = threadIdx.x >> 4, seg = threadIdx.x & 15;
  const int blk = seg >> 2;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int kk = (seg & 3) * 8 + i;
    const int q8 = ((kk & 15) >> 3) + 2 * (kk >> 4);
    const int col = blk * 32 + q8 * 8 + kperm(kk & 7);
    const float v = __builtin_ldexpf(st.v[i], sh);
    const _Float16 h = (_Float16)v;
    ahi[m][col] = h;
    alo[m][col] = (_Float16)(v - (float)h);
    s += v;
  }
  s += __shfl_xor(s, 1, 64);  // the four threads of one block
  s += __shfl_xor(s, 2, 64);
  if ((seg & 3) == 0) asum[blk][m] = s;
}

// Scale, offset and the lane's MFMA B fragment (8 k values of block jb of a
// staged row as exact f16, in the order kperm() gives) for k-octet kq
// (w: the row's dwords; o0: byte offset of block 0 in them).  Q4: bytes 0..7
// or 8..15 of the nibbles (kq odd), low nibbles for kq < 2, high otherwise.
// Q8_0: bytes 8kq .. 8kq+7 as q + 128, with m = -128 d.
template <int QT> struct QStaged;
template <> struct QStaged<MOE_Q4_1> {
  static __device__ __forceinline__ half8 frag(const uint32_t *w, int, int jb, int kq, float &d, float &m) {
    const uint32_t dm = w[5 * jb];
    d = (float)__builtin_bit_cast(_Float16, (uint16_t)(dm & 0xffffu));
    m = (float)__builtin_bit_cast(_Float16, (uint16_t)(dm >> 16));
    const int half = kq & 1;
    u32x2 nb;
    nb.x = w[5 * jb + 1 + 2 * half];
    nb.y = w[5 * jb + 2 + 2 * half];
    return nibbles_f16(nb, (uint32_t)(kq & 2) << 1);
  }
};
template <> struct QStaged<MOE_Q4_0> {
  static __device__ __forceinline__ half8 frag(const uint32_t *w, int o0, int jb, int kq, float &d, float &m) {
    const int o = o0 + 18 * jb;  // even
    const uint32_t dw = w[o >> 2];
    d = (float)__builtin_bit_cast(_Float16, (uint16_t)((o & 2) ? (dw >> 16) : (dw & 0xffffu)));
    m = -8.0f * d;
    const int s = o + 2 + 8 * (kq & 1), a = s >> 2;
    const uint32_t w0 = w[a], w1 = w[a + 1], w2 = w[a + 2];
    u32x2 nb;
    if (s & 2) {
      nb.x = __builtin_amdgcn_alignbyte(w1, w0, 2);
      nb.y = __builtin_amdgcn_alignbyte(w2, w1, 2);
    } else {
      nb.x = w0;
      nb.y = w1;
    }
    return nibbles_f16(nb, (uint32_t)(kq & 2) << 1);
  }
};
template <> struct QStaged<MOE_Q8_0> {
  static __device__ __forceinline__ half8 frag(const uint32_t *w, int o0, int jb, int kq, float &d, float &m) {
    const int o = o0 + 34 * jb;  // even
    const uint32_t dw = w[o >> 2];
    d = (float)__builtin_bit_cast(_Float16, (uint16_t)((o & 2) ? (dw >> 16) : (dw & 0xffffu)));
    m = -128.0f * d;
    const int s = o + 2 + 8 * kq, a = s >> 2;
    const uint32_t w0 = w[a], w1 = w[a + 1], w2 = w[a + 2];
    u32x2 nb;
    if (s & 2) {
      nb.x = __builtin_amdgcn_alignbyte(w1, w0, 2);
      nb.y = __builtin_amdgcn_alignbyte(w2, w1, 2);
    } else {
      nb.x = w0;
      nb.y = w1;
    }
    nb.x ^= 0x80808080u;
    nb.y ^= 0x80808080u;
    return bytes_f16(nb);
  }
};

// Per-block factor of the input-sum term of a staged block: m for Q4_1
// (w = d q + m), d for Q4_0 (w = d q - 8 d: the term is -8 d sum(x), the -8
// applied by the caller).  factor_word() is the dword holding its f16 bits;
// factor_pair() packs the factors of blocks j - 1 (low half) and j (high half),
// j odd and the wave's first block even: Q4_1's m is the high half of its
// block's first dword, Q4_0's d the low half for an even block, the high half
// for an odd one (18-byte blocks).
template <int QT> struct QFactor;
template <> struct QFactor<MOE_Q4_1> {
  static __device__ __forceinline__ uint32_t word(const uint32_t *w, int jb) { return w[5 * jb]; }
  static __device__ __forceinline__ uint32_t pair(uint32_t wj, uint32_t wprev) {
    return __builtin_amdgcn_perm(wj, wprev, 0x07060302u);
  }
};
template <> struct QFactor<MOE_Q4_0> {
  static __device__ __forceinline__ uint32_t word(const uint32_t *w, int jb) { return w[(18 * jb) >> 2]; }
  static __device__ __forceinline__ uint32_t pair(uint32_t wj, uint32_t wprev) {
    return __builtin_amdgcn_perm(wj, wprev, 0x07060100u);
  }
};

// As QStaged, with the nibbles in the natural order (nibbles_e4m3): the A
// operand that meets them is in the same order.
template <int QT> struct QStagedNat;
template <> struct QStagedNat<MOE_Q4_1> {
  static __device__ __forceinline__ half8 frag(const uint32_t *w, int jb, int kq, float &d) {
    d = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[5 * jb] & 0xffffu));
    const int half = kq & 1;
    u32x2 nb;
    nb.x = w[5 * jb + 1 + 2 * half];
    nb.y = w[5 * jb + 2 + 2 * half];
    return nibbles_e4m3(nb, (uint32_t)(kq & 2) << 1);
  }
};
template <> struct QStagedNat<MOE_Q4_0> {
  static __device__ __forceinline__ half8 frag(const uint32_t *w, int jb, int kq, float &d) {
    const int o = 18 * jb;  // even
    const uint32_t dw = w[o >> 2];
    d = (float)__builtin_bit_cast(_Float16, (uint16_t)((o & 2) ? (dw >> 16) : (dw & 0xffffu)));
    const int s = o + 2 + 8 * (kq & 1), a = s >> 2;
    const uint32_t w0 = w[a], w1 = w[a + 1], w2 = w[a + 2];
    u32x2 nb;
    if (s & 2) {
      nb.x = __builtin_amdgcn_alignbyte(w1, w0, 2);
      nb.y = __builtin_amdgcn_alignbyte(w2, w1, 2);
    } else {
      nb.x = w0;
      nb.y = w1;
    }
    return nibbles_e4m3(nb, (uint32_t)(kq & 2) << 1);
  }
};

// grid.x: routed tiles (16 tokens of one expert) then shared tiles (16 tokens);
// grid.y: slices of 256 output rows; 4 waves x 64 rows (4 MFMA tiles of 16).
// Each chunk: registers -> LDS, barrier, issue the next chunk's loads, MFMAs
// from LDS, barrier.  Blocks past K get d = m = 0 (their inputs are 0 too).
template <int QT, int MODE>
__global__ __launch_bounds__(256) void k_group_gemm(GemmArgs a) {
  constexpr int BS = QBlock<QT>::bytes;
  constexpr int NM = MODE == GG_GATEUP ? 2 : 1;  // weight matrices
  constexpr int BRW = brow<QT>() / 4;            // staged dwords per row
  constexpr int PR = brow<QT>() / 16;            // 16-byte pieces per row
  __shared__ __attribute__((aligned(16))) uint32_t bst[NM][256][BRW];
  __shared__ __attribute__((aligned(16))) _Float16 ahi[16][APAD], alo[16][APAD];
  __shared__ __attribute__((aligned(16))) float asum[KB][16];
  __shared__ int rowid[16];  // A row per tile token (-1: none)
  __shared__ int outid[16];  // output row per tile token
  __shared__ float outw[16];
  __shared__ int rsh[16];    // the A row's power-of-two shift

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bx = blockIdx.x;
  const bool shared = bx >= a.max_routed_tiles;
  // tile parameters first, all wave-uniform and with no divergent code in
  // between, so the weight buffer resources stay in scalar registers
  int e = 0, first = 0, ntok, K, R;
  const uint8_t *m0p, *m1p;
  if (!shared) {
    if (bx >= __builtin_amdgcn_readfirstlane(*a.ntiles)) return;
    e = __builtin_amdgcn_readfirstlane(a.tiles[2 * bx]);
    first = __builtin_amdgcn_readfirstlane(a.offsets[e] + a.tiles[2 * bx + 1]);
    ntok = min(16, __builtin_amdgcn_readfirstlane(a.offsets[e + 1]) - first);
    K = MODE == GG_GATEUP ? a.H : a.F;
    R = MODE == GG_GATEUP ? a.F : a.H;
    const size_t mat = (size_t)R * (K / 32) * BS;
    m0p = a.w0 + (size_t)e * mat;
    m1p = MODE == GG_GATEUP ? a.w1 + (size_t)e * mat : nullptr;
  } else {
    first = 16 * (bx - a.max_routed_tiles);  // the tile's first token
    ntok = min(16, a.T - first);
    K = MODE == GG_GATEUP ? a.H : a.SF;
    R = MODE == GG_GATEUP ? a.SF : a.H;
    m0p = a.s0;
    m1p = a.s1;
  }
  if (tid < 16) {
    const bool ok = tid < ntok;
    if (!shared) {
      const int q = first + tid;
      rowid[tid] = ok ? (MODE == GG_GATEUP ? a.perm[q] / a.k : q) : -1;
      outid[tid] = ok ? q : -1;
      outw[tid] = ok && MODE == GG_DOWN ? a.wts[a.perm[q]] : 1.f;
    } else {
      rowid[tid] = ok ? first + tid : -1;
      outid[tid] = ok ? first + tid : -1;
      outw[tid] = 1.f;
    }
    const int ar = rowid[tid];
    const int32_t *ex = MODE == GG_GATEUP ? a.xexp : (shared ? a.aexp + (size_t)a.T * a.k : a.aexp);
    rsh[tid] = ar >= 0 ? row_shift(ex[ar]) : 0;
  }
  const int r0 = blockIdx.y * 256;
  if (r0 >= R) return;
  const int nbK = K / 32;
  const uint32_t rowbytes = (uint32_t)nbK * BS;
  const uint32_t mbytes = (uint32_t)((size_t)R * rowbytes);
  const rsrc_t rw0 = make_rsrc(m0p, mbytes);
  const rsrc_t rw1 = NM == 2 ? make_rsrc(m1p, mbytes) : rw0;
  const float *arows = MODE == GG_GATEUP ? a.x : (shared ? a.act_sh : a.act);
  const int nrows = (MODE == GG_GATEUP || shared) ? a.T : a.T * a.k;  // rows of arows, K floats each
  const rsrc_t ra = make_rsrc(arows, (uint32_t)nrows * (uint32_t)K * 4u);

  // weight pieces of this thread: p = tid + 256 i (i < PR) -> row p / PR, 16 bytes p % PR
  u32x4 breg[NM][PR];
  auto b_issue = [&](int kc) {
#pragma unroll
    for (int mt = 0; mt < NM; mt++) {
#pragma unroll
      for (int i = 0; i < PR; i++) {
        const int p = tid + 256 * i, row = p / PR, j = p - PR * row;
        const int grow = r0 + row;
        const uint32_t seg = (uint32_t)grow * rowbytes + (uint32_t)kc * BS;
        const uint32_t off = (grow < R && kc < nbK) ? (seg & ~3u) + 16u * j : 0x7ffffff0u;
        breg[mt][i] = __builtin_amdgcn_raw_buffer_load_b128(mt == 0 ? rw0 : rw1, (int)off, 0, 0);
      }
    }
  };
  auto b_store = [&]() {
#pragma unroll
    for (int mt = 0; mt < NM; mt++) {
#pragma unroll
      for (int i = 0; i < PR; i++) {
        const int p = tid + 256 * i, row = p / PR, j = p - PR * row;
        *reinterpret_cast<u32x4 *>(&bst[mt][row][4 * j]) = breg[mt][i];
      }
    }
  };

  // lane roles in the MFMA: token m = lane%16 (A) / column n = lane%16 (B),
  // k-octet kq = lane/16; D rows (tokens) 4*kq + i, column n
  const int n = lane & 15, kq = lane >> 4;
  f32x4 acc[NM][4];
#pragma unroll
  for (int mt = 0; mt < NM; mt++)
#pragma unroll
    for (int c = 0; c < 4; c++) acc[mt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // byte offset of block 0 within each of this lane's staged rows (Q4_0 rows
  // may start 2 bytes past a dword; chunks start at multiples of 4 blocks)
  int o0[4];
#pragma unroll
  for (int c = 0; c < 4; c++) o0[c] = (int)(((uint32_t)(r0 + wave * 64 + 16 * c + n) * rowbytes) & 3u);

  __syncthreads();  // rowid
  const int arow = rowid[tid >> 4], ash = rsh[tid >> 4];
  AStage ast;
  b_issue(0);
  a_load(ast, ra, K, arow, 0);

  for (int kc = 0; kc < nbK; kc += KB) {
    b_store();
    a_store(ast, ash, ahi, alo, asum);
    __syncthreads();
    if (kc + KB < nbK) {
      b_issue(kc + KB);
      a_load(ast, ra, K, arow, kc + KB);
    }
#pragma unroll
    for (int jb = 0; jb < KB; jb++) {
      const bool valid = kc + jb < nbK;
      const half8 xh = *reinterpret_cast<const half8 *>(&ahi[n][jb * 32 + kq * 8]);
      const half8 xl = *reinterpret_cast<const half8 *>(&alo[n][jb * 32 + kq * 8]);
      const float4 sx4 = *reinterpret_cast<const float4 *>(&asum[jb][4 * kq]);
      const float sx[4] = {sx4.x, sx4.y, sx4.z, sx4.w};
#pragma unroll
      for (int mt = 0; mt < NM; mt++) {
#pragma unroll
        for (int c = 0; c < 4; c++) {
          float d, m;
          const half8 q = QStaged<QT>::frag(bst[mt][wave * 64 + 16 * c + n], o0[c], jb, kq, d, m);
          if (!valid) d = m = 0.f;
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
          z = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, q, z, 0, 0, 0);
          z = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl, q, z, 0, 0, 0);
          // block value: d * sum(q x) + m * sum(x); the column (row) of D is
          // this lane's n, its tokens 4*kq + i
#pragma unroll
          for (int i = 0; i < 4; i++) acc[mt][c][i] = __builtin_fmaf(d, z[i], __builtin_fmaf(m, sx[i], acc[mt][c][i]));
        }
      }
    }
    __syncthreads();
  }

  // epilogue: this lane holds D[token 4*kq + i][row r0 + wave*64 + 16c + n]
  // (scaled by 2^rsh[token]: scaled back first)
  const int rbase = r0 + wave * 64;
  int emax[4] = {0, 0, 0, 0};  // GATEUP: largest exponent of the act values this lane writes, per token
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const int row = rbase + 16 * c + n;
    if (row >= R) continue;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int m = 4 * kq + i;
      const int o = outid[m];
      if (o < 0) continue;
      float v;
      if (MODE == GG_GATEUP) {
        // SwiGLU, clamped when L > 0 (the ling_moe_ssd.js page's swiglu kernel)
        const float g = __builtin_ldexpf(acc[0][c][i], -rsh[m]), L = shared ? a.lim_sh : a.lim;
        float u = __builtin_ldexpf(acc[NM - 1][c][i], -rsh[m]), sg = g / (1.0f + __expf(-g));
        if (L > 0.f) {
          u = fminf(fmaxf(u, -L), L);
          sg = fminf(sg, L);
        }
        v = sg * u;
        emax[i] = max(emax[i], bexp(v));
      } else {
        v = outw[m] * __builtin_ldexpf(acc[0][c][i], -rsh[m]);
      }
      float *dst = shared ? a.out_sh : a.out;
      dst[(size_t)o * R + row] = v;
    }
  }
  if constexpr (MODE == GG_GATEUP) {
    // the act rows' exponents: the 16 lanes of one k-octet share their tokens
#pragma unroll
    for (int i = 0; i < 4; i++) {
      int e = emax[i];
#pragma unroll
      for (int d = 8; d >= 1; d >>= 1) e = max(e, __shfl_xor(e, d, 64));
      const int o = outid[4 * kq + i];
      if (n == 0 && o >= 0) atomicMax(shared ? a.aexp + (size_t)a.T * a.k + o : a.aexp + o, e);
    }
  }
}

// Grouped gate||up, row-streaming form (Q4 blocks; K <= 64 blocks, rows a
// multiple of 16 bytes): a block walks a run of 16-token tiles' rows of gate
// and of up in chunks of 16 whole rows per matrix, so every chunk is one
// contiguous run of each matrix (the column-chunk form above reads 80 bytes
// from each of 512 rows per chunk, a pattern that a stream probe ran at
// 3.5 TB/s against 5.7 TB/s for these runs).  Wave w takes K blocks
// [w KQ, (w+1) KQ): its tokens' inputs for those blocks are held as MFMA A
// fragments (f16 hi + lo) in registers while the block stays on one tile.
// The four waves' partial tiles of a chunk are added in wave order (fixed:
// reproducible), each wave finishing a quarter of the tile's values (SwiGLU
// and store).  Its registers (about 250 per lane) allow two blocks per CU.
// The grid is resident (the kernel's occupancy, two blocks per CU, times the
// CUs) and splits the sequence of (tile, chunk) pairs -- the shared expert's
// tiles first, then the routed tiles the sort produced, each tile's chunks in
// row order -- into runs of equal cost, one per block (below), so the blocks
// finish together and each loads its inputs again only where its run crosses
// into another tile.  The runs are dealt to
// the XCDs in order (xcd_run): an XCD's blocks take one contiguous part of the
// sequence, so a tile's token rows and an expert's rows are fetched into one
// L2.
constexpr int RS_KQM = 16;   // max K blocks per wave
// Run weights of the row-streaming GEMMs' resident grids, by the order in
// which a CU's blocks were dispatched.  A per-block timing of gate||up at two
// blocks per CU showed the first block on each CU (the grid's first half)
// ending about 15 % before the second (its older waves issue first), which
// then finished alone on a half-idle CU; runs weighted 20 : 16 measured best
// (layer 192.3 -> 189.8 us; 18 : 16 and 22 : 16 gave 190.8).  The down
// kernel, at three blocks per CU, measured best with 20 : 16 : 12 (layer
// 193.1 -> 191.3 us; 18 : 16 : 14 gave 192.2-194.8).
constexpr int RS_RUNW2[2] = {20, 16};
constexpr int RS_RUNW3[3] = {20, 16, 12};

// Units [u0, u1) of run wk of the W runs (W blocks in XCD runs, xcd_run) over
// U units.  Where w[0] > 0 and the grid is resident at nw blocks per CU (W a
// multiple of 8 nw), block i was dispatched (i / (W / nw))-th to its CU and
// its run's length is in the proportion w of that order; otherwise the runs
// are equal.  The bounds are exact for the ends (0 and U) and the same
// expression for a run's end and the next run's start.
__device__ __forceinline__ void run_bounds(int U, int W, int wk, int nw, const int (&w)[4], int &u0, int &u1) {
  if (w[0] > 0 && nw > 0 && nw <= 4 && W % (8 * nw) == 0) {
    const int per = W >> 3, gp = per / nw, x = wk / per, j = wk - x * per, g = j / gp, jj = j - g * gp;
    int tot = 0, pre = 0;
    for (int h = 0; h < nw; h++) {
      tot += gp * w[h];
      if (h < g) pre += gp * w[h];
    }
    const int p0 = x * tot + pre + jj * w[g], p1 = p0 + w[g];
    u0 = (int)((double)U * (double)p0 / (double)(8 * tot));
    u1 = (int)((double)U * (double)p1 / (double)(8 * tot));
  } else {
    const int uq = U / W, ur = U - uq * W;  // run wk: units [wk uq + min(wk, ur), ...), uq or uq + 1 of them
    u0 = wk * uq + min(wk, ur);
    u1 = u0 + uq + (wk < ur ? 1 : 0);
  }
}

// Blocks are dealt to the chip's eight XCDs (each with its own L2) in turn:
// block i runs on XCD i % 8.  For i in [0, n) this returns a work index in
// [0, n), one to one, such that the blocks of XCD x take the contiguous run
// [x q + min(x, r), ...) of work indices (q = n / 8, r = n % 8), so tiles
// that read the same rows run behind one L2.
__device__ __forceinline__ int xcd_run(int i, int n) {
  const int x = i & 7, q = n >> 3, r = n & 7;
  return x * q + min(x, r) + (i >> 3);
}
template <int QT, int KQ>
__global__ __launch_bounds__(256, 2) void k_group_gateup_rows(GemmArgs a) {
  static_assert(KQ <= RS_KQM && KQ % 2 == 0, "K blocks per wave");
  constexpr int BS = QBlock<QT>::bytes;
  constexpr int MAXDW = KQ * 4 * BS / 4;       // dwords of a row
  constexpr int PADW = MAXDW + 4;              // staged row stride (a 16-byte pad spreads the banks)
  constexpr int nbK = 4 * KQ;
  constexpr uint32_t rowbytes = (uint32_t)nbK * BS;
  constexpr int ppr = (int)(rowbytes / 16u);  // 16-byte pieces per row
  constexpr int np = 16 * ppr;                // pieces per matrix and chunk
  constexpr int PMAX = (2 * np + 255) / 256;  // pieces per thread
  __shared__ __attribute__((aligned(16))) uint32_t bst[2][16][PADW];
  __shared__ __attribute__((aligned(16))) float red[4][2][64][4];  // [wave][gate, up][lane][element]
  // the input-sum MFMA operand of each wave, 2^-6 sum(x) of token lane % 16 over
  // the wave's K blocks 8 (lane / 16) + i, as f16 hi and lo parts
  __shared__ __attribute__((aligned(16))) half8 amt[4][2][64];
  __shared__ int rowid[16], outid[16], rsh[16];

  // this block's run [c, c1) of the (tile, chunk) sequence: the shared tiles'
  // nchS chunks each, then the nt routed tiles' nchR chunks each.  The runs
  // are equal in cost units: a chunk counts UC, a tile's input prologue UP
  // (its units come before the tile's chunks).  Almost every run starts inside
  // a tile, so every block pays one prologue the units do not count, and a run
  // that crosses into another tile is that much shorter in chunks.  (Measured:
  // runs equal in chunks left the kernel 2.5 % slower; a prologue of 10 units
  // beat 4 and 6.)
  const int shtiles = a.SF > 0 ? (a.T + 15) / 16 : 0;
  const int nchS = (a.SF + 15) / 16, nchR = (a.F + 15) / 16;
  const int nt = a.k > 0 && a.F > 0 ? __builtin_amdgcn_readfirstlane(*a.ntiles) : 0;
  const int CS = shtiles * nchS;
  constexpr int UC = 4, UP = 10;
  const int US = shtiles * (UP + UC * nchS), U = US + nt * (UP + UC * nchR);
  const int W = (int)gridDim.x, wk = xcd_run((int)blockIdx.x, W);
  auto chunk_of = [&](int u) {  // the number of chunks whose first unit lies below u
    if (u < US) {
      const int t = u / (UP + UC * nchS), o = u - t * (UP + UC * nchS);
      return t * nchS + (max(0, o - UP) + UC - 1) / UC;
    }
    const int v = u - US, t = v / (UP + UC * nchR), o = v - t * (UP + UC * nchR);
    return CS + t * nchR + (max(0, o - UP) + UC - 1) / UC;
  };
  int u0, u1;
  run_bounds(U, W, wk, 2, a.runw, u0, u1);
  int c = chunk_of(u0);
  const int c1 = chunk_of(u1);
  const int K = a.H;
  const rsrc_t rx = make_rsrc(a.xhl, (uint32_t)a.T * (uint32_t)K * 4u);
  const rsrc_t rs = make_rsrc(a.xsum, (uint32_t)a.T * (uint32_t)(K / 32) * 4u);
  const int tid0 = threadIdx.x;
  while (c < c1) {  // one pass per tile the run touches
    // (the thread index passes through an empty asm each pass, so nothing
    // derived from it is hoisted out of this loop and held live through the
    // input prologue, which then spilled; its range is restated)
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    __builtin_assume(tid >= 0 && tid < 256);
    const int lane = tid & 63, wave = tid >> 6, n = lane & 15, kq = lane >> 4;
    const bool shared = c < CS;
    int first, ntok, R, cc, tnch;
    const uint8_t *g0, *u0;
    if (shared) {
      const int t = c / nchS;
      cc = c - t * nchS;
      tnch = nchS;
      first = 16 * t;
      ntok = min(16, a.T - first);
      R = a.SF;
      g0 = a.s0;
      u0 = a.s1;
    } else {
      const int q = c - CS, t = q / nchR;
      cc = q - t * nchR;
      tnch = nchR;
      const int e = __builtin_amdgcn_readfirstlane(a.tiles[2 * t]);
      first = __builtin_amdgcn_readfirstlane(a.offsets[e] + a.tiles[2 * t + 1]);
      ntok = min(16, __builtin_amdgcn_readfirstlane(a.offsets[e + 1]) - first);
      R = a.F;
      const size_t mat = (size_t)R * (a.H / 32) * BS;
      g0 = a.w0 + (size_t)e * mat;
      u0 = a.w1 + (size_t)e * mat;
    }
    const int cend = cc + min(c1 - c, tnch - cc);  // this pass: the tile's chunks [cc, cend)
    c += cend - cc;
    __syncthreads();  // the previous pass's readers of rowid, outid, rsh
    int ar = -1;  // (threads tid < 16: token slot tid's input row)
    if (tid < 16) {
      const bool ok = tid < ntok;
      const int q = first + tid;
      ar = ok ? (shared ? q : a.perm[q] / a.k) : -1;
      rowid[tid] = ar;
      outid[tid] = ok ? q : -1;
    }
    const uint32_t mbytes = (uint32_t)((size_t)R * rowbytes);
    const rsrc_t rg = make_rsrc(g0, mbytes), ru = make_rsrc(u0, mbytes);
    __syncthreads();  // rowid

    // staged chunk ch: 16 rows of gate (m = 0) and of up (m = 1), row i at bst[m][i]
    u32x4 breg[PMAX];
    auto issue = [&](int ch) {
#pragma unroll
      for (int i = 0; i < PMAX; i++) {
        const int q = tid + 256 * i, m = q >= np, qq = q - m * np;  // (q < 2 np)
        const uint32_t off = (q < 2 * np && 16 * ch + qq / ppr < R)
                                 ? (uint32_t)(16 * ch) * rowbytes + 16u * (uint32_t)qq
                                 : 0x7ffffff0u;
        breg[i] = __builtin_amdgcn_raw_buffer_load_b128(m ? ru : rg, (int)off, 0, 0);
      }
    };
    auto stage = [&]() {
#pragma unroll
      for (int i = 0; i < PMAX; i++) {
        const int q = tid + 256 * i, m = q >= np, qq = q - m * np;
        if (q < 2 * np) {
          const int row = qq / ppr, pc = qq - row * ppr;
          *reinterpret_cast<u32x4 *>(&bst[m][row][4 * pc]) = breg[i];
        }
      }
    };

    // this wave's A fragments: token n, k = (wave KQ + j) 32 + 8 kq + i in slot
    // i (the order of QStagedNat), as f16 hi + lo, loaded as the sort's launch
    // wrote them; and the input-sum MFMA's A operand: lanes kq < 2 hold the
    // sums of the wave's blocks 8 kq + i, i < 8 (zero past KQ, and in lanes
    // kq >= 2), an invalid token's loads fall outside the buffer and read zero
    half8 xh[KQ], xl[KQ];
    {
      const int arow = rowid[n];
#pragma unroll
      for (int j = 0; j < KQ; j++) {
        const uint32_t k0 = (uint32_t)((wave * KQ + j) * 32 + 8 * kq);
        const uint32_t off = arow >= 0 ? ((uint32_t)arow * (uint32_t)K + k0) * 4u : 0x7ffffff0u;
        xh[j] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0));
        xl[j] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(arow >= 0 ? off + 16u : off), 0, 0));
      }
      issue(cc);  // (after the input loads: the prologue waits for those alone)
      const uint32_t so = ((uint32_t)arow * (uint32_t)(K / 32) + (uint32_t)(wave * KQ + 8 * kq)) * 4u;
      const u32x4 s0 = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(arow >= 0 && 8 * kq < KQ ? so : 0x7ffffff0u), 0, 0);
      const u32x4 s1 = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(arow >= 0 && 8 * kq + 4 < KQ ? so + 16u : 0x7ffffff0u), 0, 0);
      const float am[8] = {__uint_as_float(s0.x), __uint_as_float(s0.y), __uint_as_float(s0.z), __uint_as_float(s0.w),
                           __uint_as_float(s1.x), __uint_as_float(s1.y), __uint_as_float(s1.z), __uint_as_float(s1.w)};
      // |sum| < 32 * 2^15 (the row shift puts |x| below 2^15): 2^-6 sum fits f16;
      // hi + lo carry 22 of its bits
      half8 ah, al;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float v = __builtin_ldexpf(am[i], -6);
        const _Float16 h = (_Float16)v;
        ah[i] = h;
        al[i] = (_Float16)(v - (float)h);
      }
      amt[wave][0][lane] = ah;
      amt[wave][1][lane] = al;
    }

    // the rows' shifts, needed only from the first chunk's output on (the input
    // pairs come scaled), so their loads leave the chain before the input loads
    if (tid < 16) rsh[tid] = ar >= 0 ? row_shift(a.xexp[ar]) : 0;
    int emax = 0;  // largest exponent of the act values this lane writes (one token slot, every chunk)
    for (int ch = cc; ch < cend; ch++) {
      stage();
      __syncthreads();
      if (ch + 1 < cend) issue(ch + 1);
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      // B operand of the input-sum MFMA, per matrix: the blocks' f16 factors (m,
      // or d for Q4_0) of row n, blocks 8 (kq & 1) + i of the wave's K range
      // (lanes kq >= 2 meet zeros in A; two named vectors, not an array, which
      // was placed in LDS)
      u32x4 P0 = {0u, 0u, 0u, 0u}, P1 = P0;
      uint32_t fprev0 = 0u, fprev1 = 0u;
      const bool upper = (kq & 1) != 0;
#pragma unroll
      for (int j = 0; j < KQ; j++) {
        const int jb = wave * KQ + j;
#pragma unroll
        for (int m = 0; m < 2; m++) {
          float d;
          const half8 q = QStagedNat<QT>::frag(&bst[m][n][0], jb, kq, d);
          const uint32_t fw = QFactor<QT>::word(&bst[m][n][0], jb);
          uint32_t &fprev = m ? fprev1 : fprev0;
          u32x4 &Pv = m ? P1 : P0;
          const bool mine = ((j >> 3) != 0) == upper;  // (j >> 3: compile time)
          if (j & 1) Pv[(j & 7) >> 1] = mine ? QFactor<QT>::pair(fw, fprev) : Pv[(j & 7) >> 1];
          fprev = fw;
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
          z = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[j], q, z, 0, 0, 0);
          z = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[j], q, z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; i++) acc[m][i] = __builtin_fmaf(d, z[i], acc[m][i]);
        }
      }
      {
        // + the input-sum term sum_j f_j sum(x)_j on the matrix cores: acc is
        // scaled by 1/S (exact: S = 2^6, or -2^9 for Q4_0's -8 d), the two MFMAs
        // add 2^-6 sum(x) (hi, lo) times the factors, and the result is scaled back
        constexpr float S = QT == MOE_Q4_1 ? 64.0f : -512.0f;
        const half8 ah = amt[wave][0][lane], al = amt[wave][1][lane];
#pragma unroll
        for (int m = 0; m < 2; m++) {
          const half8 bq = __builtin_bit_cast(half8, m ? P1 : P0);
          f32x4 t = acc[m] * (1.0f / S);
          t = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bq, t, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bq, t, 0, 0, 0);
          acc[m] = t * S;
        }
      }
      *reinterpret_cast<f32x4 *>(red[wave][0][lane]) = acc[0];
      *reinterpret_cast<f32x4 *>(red[wave][1][lane]) = acc[1];
      __syncthreads();
      {
        // wave w finishes element w of every lane's tile values: D[token 4 (l/16) + w][row 16 ch + l%16],
        // the waves' partials added in order 0..3
        // (the tile values are scaled by 2^rsh[token]: scaled back first)
        const int l = lane, i = wave, slot = 4 * (l >> 4) + i;
        const int sh = rsh[slot];
        const float g = __builtin_ldexpf(((red[0][0][l][i] + red[1][0][l][i]) + red[2][0][l][i]) + red[3][0][l][i], -sh);
        const float u = __builtin_ldexpf(((red[0][1][l][i] + red[1][1][l][i]) + red[2][1][l][i]) + red[3][1][l][i], -sh);
        const int row = 16 * ch + (l & 15);
        const int o = outid[slot];
        if (o >= 0 && row < R) {
          const float L = shared ? a.lim_sh : a.lim;
          float sg = g / (1.0f + __expf(-g)), uu = u;
          if (L > 0.f) {
            uu = fminf(fmaxf(uu, -L), L);
            sg = fminf(sg, L);
          }
          const float v = sg * uu;
          (shared ? a.out_sh : a.out)[(size_t)o * R + row] = v;
          emax = max(emax, bexp(v));
        }
      }
    }
    // the act row's exponent: lane l served token slot 4 (l / 16) + wave in
    // every chunk; the 16 lanes of l / 16 share it
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) emax = max(emax, __shfl_xor(emax, d, 64));
    const int o = outid[4 * (lane >> 4) + wave];
    if ((lane & 15) == 0 && o >= 0) atomicMax(shared ? a.aexp + (size_t)a.T * a.k + o : a.aexp + o, emax);
  }
}

// N u32x4 registers indexed by a compile-time tile number (named members:
// an array here was placed in LDS).
template <int N> struct TileWords {
  u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = w0, w2 = w0, w3 = w0;
  static_assert(N >= 1 && N <= 4, "tiles per chunk");
  __device__ __forceinline__ u32x4 &at(int t) { return t == 0 ? w0 : (t == 1 ? w1 : (t == 2 ? w2 : w3)); }
};

// LDS of one k_group_down_rows tile (bytes; every part a multiple of 16).
template <int QT, int KQ>
struct DownRowsLds {
  static constexpr int TPC = KQ <= 4 ? 4 : (KQ <= 8 ? 2 : 1);  // 16-row tiles per chunk
  static constexpr int PADW = KQ * QBlock<QT>::bytes + 4;     // staged row stride, dwords
  static constexpr size_t bst = 4 * 16 * TPC * PADW;          // staged chunk
  static constexpr size_t red = 4 * 4 * TPC * 64 * 4;         // waves' partial tiles
  static constexpr size_t asum = 4 * 2 * 64 * 16;             // input-sum MFMA operands (as in k_group_gateup_rows)
  static constexpr size_t bytes = bst + red + asum + 4 * 4 * 16;  // + rowid, outid, outw, rsh
};

// Grouped down, row-streaming form (Q4 blocks; K = F or SF of 16..64 blocks,
// rows a multiple of 16 bytes): as k_group_gateup_rows for one matrix.  A
// block takes one 16-token tile x rb rows; a chunk is TPC 16-row tiles of
// whole rows (about 20 KB, one contiguous run); wave w takes K blocks
// [w KQ, (w+1) KQ) of every tile, with its tokens' act rows held as MFMA A
// fragments.  The waves' partial tiles are added in wave order and weighted
// by the pair's routing weight.  One pass runs tile bx (routed tiles first,
// then shared ones) over its chunks [cc, cend), rows [CR cc, CR cend); tid is
// the thread's index.

template <int QT, int KQ>
__device__ __forceinline__ void down_rows_pass(const GemmArgs &a, int bx, int cc, int cend, char *smem, int tid) {
  static_assert(KQ <= RS_KQM, "K blocks per wave");
  constexpr int BS = QBlock<QT>::bytes;
  constexpr int TPC = DownRowsLds<QT, KQ>::TPC;  // 16-row tiles per chunk
  constexpr int CR = 16 * TPC;                   // rows per chunk
  constexpr int ROWDW = KQ * 4 * BS / 4;         // dwords of a row
  constexpr int PADW = ROWDW + 4;                // staged row stride (a 16-byte pad spreads the banks)
  static_assert(PADW == DownRowsLds<QT, KQ>::PADW, "row stride");
  // LDS, carved from the kernel's buffer (16-byte aligned; every part a multiple of 16 bytes)
  auto &bst = *reinterpret_cast<uint32_t (*)[CR][PADW]>(smem);
  auto &red = *reinterpret_cast<float (*)[4][TPC][64][4]>(smem + DownRowsLds<QT, KQ>::bst);  // [wave][tile][lane][element]
  auto &amt = *reinterpret_cast<half8 (*)[4][2][64]>(smem + DownRowsLds<QT, KQ>::bst + DownRowsLds<QT, KQ>::red);
  int *rowid = reinterpret_cast<int *>(smem + DownRowsLds<QT, KQ>::bst + DownRowsLds<QT, KQ>::red +
                                       DownRowsLds<QT, KQ>::asum);
  int *outid = rowid + 16;
  float *outw = reinterpret_cast<float *>(rowid + 32);
  int *rsh = rowid + 48;
  static_assert(DownRowsLds<QT, KQ>::bst % 16 == 0 && DownRowsLds<QT, KQ>::red % 16 == 0, "alignment");

  const int lane = tid & 63, wave = tid >> 6;
  const bool shared = bx >= a.max_routed_tiles;
  int e = 0, first = 0, ntok, K;
  const int R = a.H;
  const uint8_t *m0p;
  if (!shared) {
    e = __builtin_amdgcn_readfirstlane(a.tiles[2 * bx]);
    first = __builtin_amdgcn_readfirstlane(a.offsets[e] + a.tiles[2 * bx + 1]);
    ntok = min(16, __builtin_amdgcn_readfirstlane(a.offsets[e + 1]) - first);
    K = a.F;
    m0p = a.w0 + (size_t)e * ((size_t)R * (K / 32) * BS);
  } else {
    first = 16 * (bx - a.max_routed_tiles);
    ntok = min(16, a.T - first);
    K = a.SF;
    m0p = a.s0;
  }
  __syncthreads();  // the previous pass's readers of this LDS (its parts may lie elsewhere)
  if (tid < 16) {
    const bool ok = tid < ntok;
    const int q = first + tid;
    rowid[tid] = ok ? q : -1;
    outid[tid] = ok ? q : -1;
    outw[tid] = ok && !shared ? a.wts[a.perm[q]] : 1.f;
    rsh[tid] = ok ? row_shift((shared ? a.aexp + (size_t)a.T * a.k : a.aexp)[q]) : 0;
  }
  const uint32_t rowbytes = (uint32_t)(4 * KQ) * BS;
  const rsrc_t rw = make_rsrc(m0p, (uint32_t)((size_t)R * rowbytes));
  const float *arows = shared ? a.act_sh : a.act;
  const int nrows = shared ? a.T : a.T * a.k;
  const rsrc_t ra = make_rsrc(arows, (uint32_t)nrows * (uint32_t)K * 4u);
  const int n = lane & 15, kq = lane >> 4;
  __syncthreads();  // rowid

  // staged chunk: CR whole rows, row i at bst[i]
  constexpr int PMAX = (CR * ROWDW / 4 + 255) / 256;
  constexpr int PPR = ROWDW / 4;  // 16-byte pieces per row
  u32x4 breg[PMAX];
  auto issue = [&](int c) {
#pragma unroll
    for (int i = 0; i < PMAX; i++) {
      const int q = tid + 256 * i;
      const uint32_t off = (q < CR * PPR && CR * c + q / PPR < R)
                               ? (uint32_t)(CR * c) * rowbytes + 16u * (uint32_t)q
                               : 0x7ffffff0u;
      breg[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off, 0, 0);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < PMAX; i++) {
      const int q = tid + 256 * i;
      if (q < CR * PPR) {
        const int row = q / PPR, pc = q - row * PPR;
        *reinterpret_cast<u32x4 *>(&bst[row][4 * pc]) = breg[i];
      }
    }
  };

  // this wave's A fragments and input-sum MFMA operand (as in k_group_gateup_rows)
  half8 xh[KQ], xl[KQ];
  {
    const int arow = rowid[n], ash = rsh[n];
    float am[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    u32x4 v0[2][2], v1[2][2];
    auto load_group = [&](int g, u32x4 (&a0)[2], u32x4 (&a1)[2]) {
#pragma unroll
      for (int jj = 0; jj < 2; jj++) {
        const uint32_t k0 = (uint32_t)((wave * KQ + 2 * g + jj) * 32 + 8 * kq);
        const uint32_t off = arow >= 0 ? ((uint32_t)arow * (uint32_t)K + k0) * 4u : 0x7ffffff0u;
        a0[jj] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0);
        a1[jj] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(arow >= 0 ? off + 16u : off), 0, 0);
      }
    };
    load_group(0, v0[0], v1[0]);
#pragma unroll
    for (int g = 0; g < KQ / 2; g++) {
      if (g + 1 < KQ / 2) load_group(g + 1, v0[(g + 1) & 1], v1[(g + 1) & 1]);
      if (g + 2 == KQ / 2) issue(cc);  // (after the last act loads: loads complete in order)
#pragma unroll
      for (int jj = 0; jj < 2; jj++) {
        const int j = 2 * g + jj;
        float xv[8];
        const u32x4 a0 = v0[g & 1][jj], a1 = v1[g & 1][jj];
        xv[0] = __uint_as_float(a0.x); xv[1] = __uint_as_float(a0.y); xv[2] = __uint_as_float(a0.z); xv[3] = __uint_as_float(a0.w);
        xv[4] = __uint_as_float(a1.x); xv[5] = __uint_as_float(a1.y); xv[6] = __uint_as_float(a1.z); xv[7] = __uint_as_float(a1.w);
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const float v = __builtin_ldexpf(xv[i], ash);
          const _Float16 h = (_Float16)v;
          xh[j][i] = h;
          xl[j][i] = (_Float16)(v - (float)h);
          sum += v;
        }
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        if ((j >> 3) == kq) am[j & 7] = sum;
      }
    }
    half8 ah, al;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float v = __builtin_ldexpf(am[i], -6);
      const _Float16 h = (_Float16)v;
      ah[i] = h;
      al[i] = (_Float16)(v - (float)h);
    }
    amt[wave][0][lane] = ah;
    amt[wave][1][lane] = al;
  }

  for (int c = cc; c < cend; c++) {
    stage();
    __syncthreads();
    if (c + 1 < cend) issue(c + 1);
    f32x4 acc[TPC];
#pragma unroll
    for (int t = 0; t < TPC; t++) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the input-sum MFMA's B operand per tile (as in k_group_gateup_rows;
    // with KQ <= 8 every block sits in the lanes kq & 1 == 0, and the others
    // meet zeros in A, so no lane selects)
    TileWords<TPC> P;
    uint32_t fprev[TPC];
    const bool upper = (kq & 1) != 0;
#pragma unroll
    for (int j = 0; j < KQ; j++) {
      const int jb = wave * KQ + j;
#pragma unroll
      for (int t = 0; t < TPC; t++) {
        float d;
        const half8 q = QStagedNat<QT>::frag(&bst[16 * t + n][0], jb, kq, d);
        const uint32_t fw = QFactor<QT>::word(&bst[16 * t + n][0], jb);
        if (j & 1) {
          const uint32_t pw = QFactor<QT>::pair(fw, fprev[t]);
          u32x4 &Pv = P.at(t);
          if constexpr (KQ > 8)
            Pv[(j & 7) >> 1] = (((j >> 3) != 0) == upper) ? pw : Pv[(j & 7) >> 1];
          else
            Pv[(j & 7) >> 1] = pw;
        }
        fprev[t] = fw;
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[j], q, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[j], q, z, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; i++) acc[t][i] = __builtin_fmaf(d, z[i], acc[t][i]);
      }
    }
    {
      constexpr float S = QT == MOE_Q4_1 ? 64.0f : -512.0f;  // (as in k_group_gateup_rows)
      const half8 ah = amt[wave][0][lane], al = amt[wave][1][lane];
#pragma unroll
      for (int t = 0; t < TPC; t++) {
        const half8 bq = __builtin_bit_cast(half8, P.at(t));
        f32x4 u = acc[t] * (1.0f / S);
        u = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bq, u, 0, 0, 0);
        u = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bq, u, 0, 0, 0);
        acc[t] = u * S;
      }
    }
#pragma unroll
    for (int t = 0; t < TPC; t++) *reinterpret_cast<f32x4 *>(red[wave][t][lane]) = acc[t];
    __syncthreads();
    {
      // wave w finishes element w: D[token 4 (l/16) + w][row CR c + 16 t + l%16], waves added in order
      const int l = lane, i = wave;
      const int slot = 4 * (l >> 4) + i, o = outid[slot], sh = rsh[slot];
      const float wgt = outw[slot];
      float *dst = shared ? a.out_sh : a.out;
#pragma unroll
      for (int t = 0; t < TPC; t++) {
        const float v = __builtin_ldexpf(((red[0][t][l][i] + red[1][t][l][i]) + red[2][t][l][i]) + red[3][t][l][i], -sh);
        const int row = CR * c + 16 * t + (l & 15);
        if (o >= 0 && row < R) dst[(size_t)o * R + row] = wgt * v;
      }
    }
  }
}

// Grouped down, both kinds of tile in one launch: K = SF for the shared
// tiles (KQS blocks per wave), K = F for the routed ones (KQF); KQF or KQS is 0
// where the layer has no routed or no shared expert.  As in
// k_group_gateup_rows the grid is resident and splits the sequence of (tile,
// chunk) pairs -- the shared tiles first, then the routed tiles the sort
// produced -- into runs equal in cost units (a chunk UC, a tile's act prologue
// UP), dealt to the XCDs in order (xcd_run), so a tile's act rows and an
// expert's rows are fetched into one L2.  A chunk of either kind is about
// 20 KB of weights and the same MFMA work (TPC 16-row tiles of K / 32 blocks).
template <int QT, int KQF, int KQS>
__global__ __launch_bounds__(256, 2) void k_group_down_rows(GemmArgs a, int shtiles) {
  constexpr size_t lf = KQF > 0 ? DownRowsLds<QT, KQF>::bytes : 0, ls = KQS > 0 ? DownRowsLds<QT, KQS>::bytes : 0;
  __shared__ __attribute__((aligned(16))) char smem[lf > ls ? lf : (ls > 0 ? ls : 16)];  // one tile's LDS, either kind
  constexpr int CRS = KQS > 0 ? 16 * DownRowsLds<QT, KQS>::TPC : 16;  // rows per chunk, shared tiles
  constexpr int CRF = KQF > 0 ? 16 * DownRowsLds<QT, KQF>::TPC : 16;  // rows per chunk, routed tiles
  constexpr int UC = 4, UP = 6;
  const int nchS = (a.H + CRS - 1) / CRS, nchR = (a.H + CRF - 1) / CRF;
  const int nts = KQS > 0 ? shtiles : 0;
  const int nt = KQF > 0 ? __builtin_amdgcn_readfirstlane(*a.ntiles) : 0;
  const int CS = nts * nchS;
  const int US = nts * (UP + UC * nchS), U = US + nt * (UP + UC * nchR);
  const int W = (int)gridDim.x, wk = xcd_run((int)blockIdx.x, W);
  auto chunk_of = [&](int u) {  // the number of chunks whose first unit lies below u
    if (u < US) {
      const int t = u / (UP + UC * nchS), o = u - t * (UP + UC * nchS);
      return t * nchS + (max(0, o - UP) + UC - 1) / UC;
    }
    const int v = u - US, t = v / (UP + UC * nchR), o = v - t * (UP + UC * nchR);
    return CS + t * nchR + (max(0, o - UP) + UC - 1) / UC;
  };
  int u0, u1;
  run_bounds(U, W, wk, 3, a.runw, u0, u1);
  int c = chunk_of(u0);
  const int c1 = chunk_of(u1);
  const int tid0 = threadIdx.x;
  while (c < c1) {  // one pass per tile the run touches
    // (the thread index passes through an empty asm each pass, as in
    // k_group_gateup_rows, so nothing derived from it is hoisted out of this loop)
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    __builtin_assume(tid >= 0 && tid < 256);
    if (c < CS) {
      const int t = c / nchS, cc = c - t * nchS, cend = cc + min(c1 - c, nchS - cc);
      c += cend - cc;
      if constexpr (KQS > 0) down_rows_pass<QT, KQS>(a, a.max_routed_tiles + t, cc, cend, smem, tid);
    } else {
      const int q = c - CS, t = q / nchR, cc = q - t * nchR, cend = cc + min(c1 - c, nchR - cc);
      c += cend - cc;
      if constexpr (KQF > 0) down_rows_pass<QT, KQF>(a, t, cc, cend, smem, tid);
    }
  }
}

// resid[t][h] += sum_j Y[pos(t, j)][h] + Ysh[t][h], the same order for every
// element; each thread takes four consecutive h (16-byte loads; H % 32 == 0).
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ Y, const float *__restrict__ Ysh,
                                                 const int32_t *__restrict__ pos, int T, int k, int H,
                                                 float *__restrict__ resid) {
  const int t = blockIdx.y, h = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (h >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; j++) {
    const float4 y = *reinterpret_cast<const float4 *>(Y + (size_t)pos[t * k + j] * H + h);
    acc.x += y.x;
    acc.y += y.y;
    acc.z += y.z;
    acc.w += y.w;
  }
  if (Ysh) {
    const float4 y = *reinterpret_cast<const float4 *>(Ysh + (size_t)t * H + h);
    acc.x += y.x;
    acc.y += y.y;
    acc.z += y.z;
    acc.w += y.w;
  }
  float4 *r = reinterpret_cast<float4 *>(resid + (size_t)t * H + h);
  float4 v = *r;
  v.x += acc.x;
  v.y += acc.y;
  v.z += acc.z;
  v.w += acc.w;
  *r = v;
}

// ---------------------------------------------------------------- launch --

size_t prefill_sort_lds_bytes(int T, int E) { return (size_t)E * ((T + 31) / 32) * (4 + 2) + 4; }
// The sort stages the ids in LDS while the whole stays within 56 KB.
static bool sort_stages_ids(int T, int k, int E) { return prefill_sort_lds_bytes(T, E) + (size_t)T * k * 4 <= 56 * 1024; }

// Compute units of the current device, looked up once per device.
static int cu_count() {
  static int counts[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] <= 0) {
    int n = 0;
    counts[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return counts[dev];
}

// Grid of a resident launch of a 256-thread kernel without dynamic LDS: its
// blocks per CU (occ caches them) times the CUs, at most cap and at least 1.
template <typename Kern>
static unsigned resident_grid(Kern kernel, int &occ, long long cap) {
  if (occ <= 0) {
    int nb = 0;
    occ = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, 256, 0) == hipSuccess && nb > 0 ? nb : 1;
  }
  return (unsigned)std::max(1LL, std::min(cap, (long long)occ * cu_count()));
}

// The down launch for routed and shared K blocks per wave KQF and KQS: one
// block per chunk of the layer at most, else resident.
template <int QT, int KQF, int KQS>
static void launch_down_rows_k(const GemmArgs &g, int shtiles, hipStream_t st) {
  static int occ = 0;
  constexpr int crs = 16 * DownRowsLds<QT, KQS>::TPC, crf = 16 * DownRowsLds<QT, KQF>::TPC;
  const long long cap = (KQS > 0 ? (long long)shtiles * ((g.H + crs - 1) / crs) : 0) +
                        (KQF > 0 ? (long long)g.max_routed_tiles * ((g.H + crf - 1) / crf) : 0);
  const unsigned grid = resident_grid(k_group_down_rows<QT, KQF, KQS>, occ, cap);
  GemmArgs gr = g;
  if (occ == 3 && grid == 3u * (unsigned)cu_count())
    for (int i = 0; i < 3; i++) gr.runw[i] = RS_RUNW3[i];
  MOE_LAUNCH(7, (k_group_down_rows<QT, KQF, KQS>), dim3(grid), dim3(256), 0u, st, gr, shtiles);
}

template <int QT, int KQF>
static void launch_down_rows_s(int kqs, const GemmArgs &g, int shtiles, hipStream_t st) {
  switch (kqs) {
    case 0: launch_down_rows_k<QT, KQF, 0>(g, shtiles, st); break;
    case 4: launch_down_rows_k<QT, KQF, 4>(g, shtiles, st); break;
    case 8: launch_down_rows_k<QT, KQF, 8>(g, shtiles, st); break;
    case 12: launch_down_rows_k<QT, KQF, 12>(g, shtiles, st); break;
    default: launch_down_rows_k<QT, KQF, 16>(g, shtiles, st); break;
  }
}

// K blocks per wave of the routed (kqf) and shared (kqs) down matrices: 0
// (none), 4, 8, 12 or 16.
template <int QT>
static void launch_down_rows(int kqf, int kqs, const GemmArgs &g, int shtiles, hipStream_t st) {
  switch (kqf) {
    case 0: launch_down_rows_s<QT, 0>(kqs, g, shtiles, st); break;
    case 4: launch_down_rows_s<QT, 4>(kqs, g, shtiles, st); break;
    case 8: launch_down_rows_s<QT, 8>(kqs, g, shtiles, st); break;
    case 12: launch_down_rows_s<QT, 12>(kqs, g, shtiles, st); break;
    default: launch_down_rows_s<QT, 16>(kqs, g, shtiles, st); break;
  }
}

hipError_t launch_prefill_ffn(const PrefillArgs &p, hipStream_t st) {
  const int T = p.T, k = p.k, E = p.E;
  hipError_t err;
  // gate||up in the row-streaming form: Q4 rows of 16, 32, 48 or 64 blocks
  // (whole 16-byte pieces); it reads x as the f16 hi + lo pairs made below
  const int nbH = p.H / 32;
  const bool rowform = p.qtype != MOE_Q8_0 && nbH % 16 == 0 && nbH <= 4 * RS_KQM;
  uint16_t *xhl = rowform ? p.xhl : nullptr;
  // the sort, and the rows' power-of-two scales: x now (with its f16 form),
  // the act rows' exponents zeroed for the gate||up epilogue (in the sort's
  // launch, blocks past the first)
  const int nzero = T * (k + 1);
  if (k > 0) {  // (a dense layer, k == 0, has no routed pairs to sort)
    const int nexp = max((T + 15) / 16, (nzero + 1023) / 1024);
    if (sort_stages_ids(T, k, E))
      MOE_LAUNCH(5, k_sort_by_expert<true>, dim3(1 + nexp), dim3(1024),
                 (uint32_t)(prefill_sort_lds_bytes(T, E) + T * k * 4), st, p.ids, T, k, E, p.offsets, p.pos, p.perm,
                 p.tiles, p.ntiles, p.x, p.H, p.xexp, p.aexp, nzero, xhl, p.xsum);
    else
      MOE_LAUNCH(5, k_sort_by_expert<false>, dim3(1 + nexp), dim3(1024), (uint32_t)prefill_sort_lds_bytes(T, E), st,
                 p.ids, T, k, E, p.offsets, p.pos, p.perm, p.tiles, p.ntiles, p.x, p.H, p.xexp, p.aexp, nzero, xhl,
                 p.xsum);
  } else {
    const int nblk = max((T + 3) / 4, (nzero + 255) / 256);
    MOE_LAUNCH(11, k_row_exp, dim3(nblk), dim3(256), 0u, st, p.x, T, p.H, p.xexp, p.aexp, nzero, xhl, p.xsum);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  GemmArgs g{};
  g.T = T;
  g.k = k;
  g.H = p.H;
  g.xexp = p.xexp;
  g.xhl = p.xhl;
  g.xsum = p.xsum;
  g.aexp = p.aexp;
  g.F = p.F;
  g.SF = p.SF;
  g.E = E;
  g.x = p.x;
  g.act = p.act;
  g.act_sh = p.act_sh;
  g.wts = p.wts;
  g.offsets = p.offsets;
  g.perm = p.perm;
  g.tiles = p.tiles;
  g.ntiles = p.ntiles;
  g.max_routed_tiles = (T * k + 15) / 16 + E;
  g.lim = p.lim;
  g.lim_sh = p.lim_sh;
  // (runw stays {0}: equal runs, unless a launch below sets its weights)
  const int shtiles = p.SF > 0 ? (T + 15) / 16 : 0;
  // gate || up
  g.w0 = p.gate_exps;
  g.w1 = p.up_exps;
  g.s0 = p.gate_sh;
  g.s1 = p.up_sh;
  g.out = p.act;
  g.out_sh = p.act_sh;
  {
    const int rows = p.F > p.SF ? p.F : p.SF;
    dim3 grid(g.max_routed_tiles + shtiles, (rows + 255) / 256);
    // (its grid: resident blocks, or one per chunk where the layer has fewer chunks)
    const long long cmax = (long long)shtiles * ((p.SF + 15) / 16) +
                           (k > 0 && p.F > 0 ? (long long)g.max_routed_tiles * ((p.F + 15) / 16) : 0);
#define MOE_RS_CASE(QT, KQ)                                                                              \
  {                                                                                                      \
    static int occ_ = 0;                                                                                 \
    const unsigned grid_ = resident_grid(k_group_gateup_rows<QT, KQ>, occ_, cmax);                    \
    GemmArgs gr_ = g;                                                                                    \
    if (occ_ == 2 && grid_ == 2u * (unsigned)cu_count())                                                 \
      for (int i_ = 0; i_ < 2; i_++) gr_.runw[i_] = RS_RUNW2[i_];                                        \
    MOE_LAUNCH(6, (k_group_gateup_rows<QT, KQ>), dim3(grid_), dim3(256), 0u, st, gr_);                  \
  }
#define MOE_RS_LAUNCH(QT)                                                                                \
  switch (nbH / 4) {                                                                                     \
    case 4: MOE_RS_CASE(QT, 4) break;                                                                    \
    case 8: MOE_RS_CASE(QT, 8) break;                                                                    \
    case 12: MOE_RS_CASE(QT, 12) break;                                                                  \
    default: MOE_RS_CASE(QT, 16) break;                                                                  \
  }
    if (rowform && p.qtype == MOE_Q4_1) {
      MOE_RS_LAUNCH(MOE_Q4_1)
    } else if (rowform) {
      MOE_RS_LAUNCH(MOE_Q4_0)
    } else if (p.qtype == MOE_Q4_1)
      MOE_LAUNCH(6, (k_group_gemm<MOE_Q4_1, GG_GATEUP>), grid, dim3(256), 0u, st, g);
    else if (p.qtype == MOE_Q8_0)
      MOE_LAUNCH(6, (k_group_gemm<MOE_Q8_0, GG_GATEUP>), grid, dim3(256), 0u, st, g);
    else
      MOE_LAUNCH(6, (k_group_gemm<MOE_Q4_0, GG_GATEUP>), grid, dim3(256), 0u, st, g);
#undef MOE_RS_LAUNCH
#undef MOE_RS_CASE
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // down, weighted
  g.w0 = p.down_exps;
  g.w1 = nullptr;
  g.s0 = p.down_sh;
  g.s1 = nullptr;
  g.out = p.Y;
  g.out_sh = p.Ysh;
  const int nbF = k > 0 ? p.F / 32 : 0, nbS = p.SF / 32;
  auto rowable = [](int nb) { return nb % 16 == 0 && nb <= 4 * RS_KQM; };
  if (p.qtype != MOE_Q8_0 && (nbF == 0 || rowable(nbF)) && (nbS == 0 || rowable(nbS))) {
    // row-streaming form: shared tiles, then routed tiles, in one resident launch
    const bool any = shtiles > 0 || nbF > 0;
    if (any && p.qtype == MOE_Q4_1)
      launch_down_rows<MOE_Q4_1>(nbF / 4, nbS / 4, g, shtiles, st);
    else if (any)
      launch_down_rows<MOE_Q4_0>(nbF / 4, nbS / 4, g, shtiles, st);
  } else {
    dim3 grid(g.max_routed_tiles + shtiles, (p.H + 255) / 256);
    if (p.qtype == MOE_Q4_1)
      MOE_LAUNCH(7, (k_group_gemm<MOE_Q4_1, GG_DOWN>), grid, dim3(256), 0u, st, g);
    else if (p.qtype == MOE_Q8_0)
      MOE_LAUNCH(7, (k_group_gemm<MOE_Q8_0, GG_DOWN>), grid, dim3(256), 0u, st, g);
    else
      MOE_LAUNCH(7, (k_group_gemm<MOE_Q4_0, GG_DOWN>), grid, dim3(256), 0u, st, g);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  MOE_LAUNCH(8, k_combine, dim3((p.H / 4 + 255) / 256, T), dim3(256), 0u, st, (const float *)p.Y,
             (const float *)(p.SF > 0 ? p.Ysh : nullptr), (const int32_t *)p.pos, T, k, p.H, p.resid);
  return hipGetLastError();
}

}  // namespace moe
