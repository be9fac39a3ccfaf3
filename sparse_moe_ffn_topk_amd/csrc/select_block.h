// select_block.h -- routing of one token by one 256-thread block (gfx950).
//
// Follows the router of the diskformer pages: p = sigmoid(logit); selection
// score s = p + bias (the bias only picks); optional group limit -- a group's
// score is the f32 sum of its two largest s (an equal value counts as the
// second), the groups_used best groups are kept with the lower group index
// winning ties; then the top k experts by s over the kept groups, the lower
// expert index winning ties, listed in pick order; weights = picked p over
// their f32 sum (pick order) clamped at wsum_min, times weights_scale
// (lfm2_moe_ssd.js page: router comment and TOPK_SIG_BODY; ling_moe_ssd.js
// page: routeLing).
//
// The pages pick with k sequential rounds of arg-max.  The outcome of those
// rounds is fixed by ranks: expert e is pick number
//   rank(e) = #{e' : s(e') > s(e), or s(e') == s(e) and e' < e}
// whenever rank(e) < k.  Here the threads rank experts in parallel, in two
// stages: each wave ranks the experts of its own segment (64 of every 256)
// and keeps its k best as candidates; the candidates (at most 4k) are then
// ranked against each other.  Every global top-k expert is a candidate of its
// segment, and every expert that beats it is one too, so the candidate ranks
// are the exact pick positions.  Kept groups use the same rank rule.
//
// The sigmoid of the f32 logit is evaluated in double and rounded once to
// f32, so equal f32 logits always give equal scores.
#pragma once
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr float NEG = -3.402823466e38f;  // below every score
constexpr int SEL_MAX_E = 512, SEL_MAX_K = 32, SEL_MAX_G = 64;

struct SelShared {
  float s[SEL_MAX_E];  // selection scores (NEG: padding or dropped group)
  float p[SEL_MAX_E];  // sigmoids
  float gs[SEL_MAX_G];
  int kept[SEL_MAX_G];
  float cs[4 * SEL_MAX_K];  // candidates: score and expert
  int ce[4 * SEL_MAX_K];
  int pick[SEL_MAX_K];
  float pp[SEL_MAX_K];
};

// a beats b: higher score, or equal score and lower index
__device__ __forceinline__ int beats(float sa, int ea, float sb, int eb) { return sa > sb || (sa == sb && ea < eb); }

// Route one token with the whole block (blockDim.x == 256; every thread must
// call it).  On return (after a barrier) sh.pick[0..k) holds the experts in
// pick order and sh.pp[0..k) their sigmoids; if w_out is given, threads
// 0..k-1 write the k weights to it.
__device__ __forceinline__ void select_block(const float *__restrict__ l, const float *__restrict__ bias,
                                             const SelParams &P, SelShared &sh, float *__restrict__ w_out) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const int R = (P.E + 255) >> 8;  // experts per thread (1 or 2)
  for (int r = 0; r < R; r++) {
    const int e = tid + 256 * r;
    float p = 0.f, s = NEG;
    if (e < P.E) {
      p = (float)(1.0 / (1.0 + exp(-(double)l[e])));
      s = p + (bias ? bias[e] : 0.f);
    }
    sh.s[e] = s;
    sh.p[e] = p;
  }
  if (tid < 4 * SEL_MAX_K) {
    sh.cs[tid] = NEG;
    sh.ce[tid] = 0x7fffffff;
  }
  __syncthreads();

  if (P.Gu < P.G) {
    const int PG = P.E / P.G;
    if (tid < P.G) {
      // the group's two largest scores, an equal value counting as the second
      float a = NEG, b = NEG;
      for (int e = tid * PG; e < (tid + 1) * PG; e++) {
        const float v = sh.s[e];
        if (v > a) {
          b = a;
          a = v;
        } else if (v > b) {
          b = v;
        }
      }
      sh.gs[tid] = a + b;
    }
    __syncthreads();
    if (tid < P.G) {
      const float mine = sh.gs[tid];
      int rank = 0;
      for (int g = 0; g < P.G; g++) rank += beats(sh.gs[g], g, mine, tid);
      sh.kept[tid] = rank < P.Gu;
    }
    __syncthreads();
    for (int r = 0; r < R; r++) {
      const int e = tid + 256 * r;
      if (e < P.E && !sh.kept[e / PG]) sh.s[e] = NEG;
    }
    __syncthreads();
  }

  // stage 1: rank within the wave's segment {64*wave + i + 256*r}
  for (int r = 0; r < R; r++) {
    const int e = tid + 256 * r;
    if (e < P.E) {
      const float mine = sh.s[e];
      int rank = 0;
      for (int r2 = 0; r2 < R; r2++) {
        const int e0 = 256 * r2 + 64 * wave;
        const float *seg = sh.s + e0;
#pragma unroll 4
        for (int i = 0; i < 64; i += 4) {
          const float4 v = *reinterpret_cast<const float4 *>(seg + i);
          rank += beats(v.x, e0 + i, mine, e) + beats(v.y, e0 + i + 1, mine, e) + beats(v.z, e0 + i + 2, mine, e) +
                  beats(v.w, e0 + i + 3, mine, e);
        }
      }
      if (rank < P.k) {
        sh.cs[wave * P.k + rank] = mine;
        sh.ce[wave * P.k + rank] = e;
      }
    }
  }
  __syncthreads();

  // stage 2: rank among the candidates
  const int C = 4 * P.k;
  if (tid < C && sh.ce[tid] != 0x7fffffff) {
    const float mine = sh.cs[tid];
    const int e = sh.ce[tid];
    int rank = 0;
    for (int c = 0; c < C; c++) rank += beats(sh.cs[c], sh.ce[c], mine, e);
    if (rank < P.k) {
      sh.pick[rank] = e;
      sh.pp[rank] = sh.p[e];
    }
  }
  __syncthreads();
  if (w_out && tid < P.k) {
    float wsum = 0.f;
    for (int j = 0; j < P.k; j++) wsum += sh.pp[j];  // f32, pick order
    wsum = fmaxf(wsum, P.wsum_min);
    w_out[tid] = sh.pp[tid] / wsum * P.scale;
  }
}

}  // namespace moe
