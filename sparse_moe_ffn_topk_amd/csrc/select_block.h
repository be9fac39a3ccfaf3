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
// stages: each wave finds the k best experts of its own segment (64 of every
// 256) -- after dropping, in registers, every expert that k others of its
// 16-lane row already beat -- and keeps them as candidates; the candidates
// (at most 4k) are then ranked against each other.  Every global top-k expert
// is a candidate of its segment, and every expert that beats it is one too,
// so the candidate ranks are the exact pick positions.  With E <= 64 only
// wave 0 holds experts, so its segment ranks are already the pick positions
// and stage 2 is skipped.  With two experts a thread (E > 256) a wave's k best
// are found instead by a bitwise search for its k-th largest score word (one
// ballot count per bit), which costs less than ranking the many survivors.  Experts are compared through 64-bit keys (sel_key)
// whose unsigned order is the beats order, so a comparison is one integer
// compare.  Kept groups use the same rank rule.
//
// The sigmoid of the f32 logit is evaluated in double and rounded once to
// f32, so equal f32 logits always give equal scores.
#pragma once
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr float NEG = -3.402823466e38f;  // below every score
constexpr int SEL_MAX_E = 512, SEL_MAX_K = 32, SEL_MAX_G = 64;

struct alignas(16) SelShared {
  unsigned long long sk[4][136];         // per wave: keys of its stage-1 survivors (zero-padded to 8)
  float s[SEL_MAX_E];                    // selection scores
  float p[SEL_MAX_E];                    // sigmoids
  float gs[SEL_MAX_G];
  int kept[SEL_MAX_G];
  unsigned long long ck[4 * SEL_MAX_K];  // candidate keys (0: empty slot)
  int pick[SEL_MAX_K];
  float pp[SEL_MAX_K];
};

// Ranking key: a beats b (higher score, or equal score and lower index) exactly
// when key(a) > key(b) as unsigned integers.  High word: the score's bits mapped
// so that unsigned order is float order (scores are never NaN; -0 is folded to
// +0 first, as float comparison treats them equal); low word: ~expert, so of
// two equal scores the lower index has the larger key.  Every real key is
// nonzero (the high word of any non-NaN float is).
__device__ __forceinline__ unsigned long long sel_key(float s, int e) {
  const uint32_t b = __float_as_uint(s + 0.0f);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)o << 32) | (uint32_t)~e;
}

// Number of the other 15 lanes of this lane's 16-lane row holding a larger h
// (DPP row rotations: register traffic only).
template <int N>
__device__ __forceinline__ int row_count_above(uint32_t h) {
  if constexpr (N == 0) {
    return 0;
  } else {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x120 + N, 0xF, 0xF, false);  // row_ror:N
    return (int)(o > h) + row_count_above<N - 1>(h);
  }
}

// a beats b: higher score, or equal score and lower index
__device__ __forceinline__ int beats(float sa, int ea, float sb, int eb) { return sa > sb || (sa == sb && ea < eb); }

// One token's router inputs for thread tid: experts tid and tid + 256.
struct SelIn {
  float l[2], b[2];
};

// Issue the loads of the logits (and bias) the calling thread ranks; split
// from select_rank() so a caller can put other loads behind them and still
// wait for these first (vector loads retire in order).  Experts past E read
// as 0 (buffer loads past the range return zeros).
__device__ __forceinline__ void select_load(const float *__restrict__ l, const float *__restrict__ bias,
                                            const SelParams &P, SelIn &in) {
  const uint32_t tid = threadIdx.x;
  const rsrc_t rl = make_rsrc(l, (uint32_t)P.E * 4u);
#pragma unroll
  for (int r = 0; r < 2; r++) in.l[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (int)((tid + 256u * r) * 4u), 0, 0));
  if (bias) {
    const rsrc_t rb = make_rsrc(bias, (uint32_t)P.E * 4u);
#pragma unroll
    for (int r = 0; r < 2; r++) in.b[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (int)((tid + 256u * r) * 4u), 0, 0));
  } else {
    in.b[0] = in.b[1] = 0.f;
  }
}

// Merge of two top-2 multisets (an equal value counts as the second).
__device__ __forceinline__ void top2_merge(float &a, float &b, float a2, float b2) {
  const float lo = fminf(a, a2);
  a = fmaxf(a, a2);
  b = fmaxf(lo, fmaxf(b, b2));
}
template <int N>
__device__ __forceinline__ float row_ror_f(float v) {  // DPP row_ror:N (register moves within a 16-lane row)
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}
// Top-2 of each 16-lane row, in every lane of the row: rotations by 8, 4, 2,
// 1 merge disjoint halves (max / min only, so exact in any order).
__device__ __forceinline__ void row_top2(float &a, float &b) {
  top2_merge(a, b, row_ror_f<8>(a), row_ror_f<8>(b));
  top2_merge(a, b, row_ror_f<4>(a), row_ror_f<4>(b));
  top2_merge(a, b, row_ror_f<2>(a), row_ror_f<2>(b));
  top2_merge(a, b, row_ror_f<1>(a), row_ror_f<1>(b));
}

// Top-2 of the PG scores held by each aligned run of PG lanes (PG a power of
// two <= 64), as a multiset (an equal value counts as the second); every lane
// of the run gets the pair.
__device__ __forceinline__ void run_top2(float &a, float &b, int PG) {
  for (int m = PG >> 1; m >= 1; m >>= 1) {
    const float a2 = __shfl_xor(a, m, 64), b2 = __shfl_xor(b, m, 64);
    const float lo = fminf(a, a2);
    a = fmaxf(a, a2);
    b = fmaxf(lo, fmaxf(b, b2));
  }
}

// Route one token with the whole block from inputs loaded by select_load()
// (blockDim.x == 256; every thread must call it).  On return (after a
// barrier) sh.pick[0..k) holds the experts in pick order and sh.pp[0..k) their
// sigmoids; if w_out is given, threads 0..k-1 write the k weights to it.
__device__ __forceinline__ void select_rank(const SelIn &in, const SelParams &P, SelShared &sh,
                                            float *__restrict__ w_out) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const int R = (P.E + 255) >> 8;  // experts per thread (1 or 2)
  float sv[2];
#pragma unroll
  for (int r = 0; r < 2; r++) {
    const int e = tid + 256 * r;
    float p = 0.f, s = NEG;
    if (e < P.E) {
      p = (float)(1.0 / (1.0 + exp(-(double)in.l[r])));
      s = p + in.b[r];
    }
    sv[r] = s;
    if (r < R) {
      sh.s[e] = s;
      sh.p[e] = p;
    }
  }
  if (R == 1 && tid < 4 * SEL_MAX_K) sh.ck[tid] = 0ull;  // (two experts a thread: each wave clears its own slots)

  const int PG = P.G > 1 ? P.E / P.G : P.E;  // experts per group
  const int pg_shift = (PG & (PG - 1)) == 0 ? __builtin_ctz(PG) : -1;  // (uniform)
  if (P.Gu < P.G) {
    if (PG == 64) {
      // a group is one wave's slice: each row's top-2 by DPP rotations, then
      // the four rows' pairs read out and merged (uniform)
#pragma unroll
      for (int r = 0; r < 2; r++) {
        if (r < R) {
          float a = sv[r], b = NEG;
          row_top2(a, b);
          auto rl = [&](float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
          float A = rl(a, 15), B = rl(b, 15);
          top2_merge(A, B, rl(a, 31), rl(b, 31));
          top2_merge(A, B, rl(a, 47), rl(b, 47));
          top2_merge(A, B, rl(a, 63), rl(b, 63));
          const int e = tid + 256 * r;
          if ((tid & 63) == 0 && e < P.E) sh.gs[e >> 6] = A + B;
        }
      }
      __syncthreads();
    } else if (pg_shift >= 0 && PG <= 64) {
      // a group is an aligned run of PG lanes of one wave: butterfly top-2
#pragma unroll
      for (int r = 0; r < 2; r++) {
        if (r < R) {
          float a = sv[r], b = NEG;
          run_top2(a, b, PG);
          const int e = tid + 256 * r;
          if (e < P.E && (e & (PG - 1)) == 0) sh.gs[e >> pg_shift] = a + b;
        }
      }
      __syncthreads();
    } else {
      __syncthreads();
      if (tid < P.G) {
        float a = NEG, b = NEG;
        for (int e = tid * PG; e < (tid + 1) * PG; e++) {
          const float v = sh.s[e];
          const float lo = fminf(a, v);
          a = fmaxf(a, v);
          b = fmaxf(b, lo);
        }
        sh.gs[tid] = a + b;
      }
      __syncthreads();
    }
    if (tid < P.G) {
      const float mine = sh.gs[tid];
      int rank = 0;
#pragma unroll 8
      for (int g = 0; g < P.G; g++) rank += beats(sh.gs[g], g, mine, tid);
      sh.kept[tid] = rank < P.Gu;
    }
    __syncthreads();
  }
  // keys; padding experts and dropped groups get 0, which beats nothing
  unsigned long long kr[2];
#pragma unroll
  for (int r = 0; r < 2; r++) {
    const int e = tid + 256 * r;
    const bool real = r < R && e < P.E && (P.Gu >= P.G || sh.kept[pg_shift >= 0 ? e >> pg_shift : e / PG]);
    kr[r] = real ? sel_key(sv[r], e) : 0ull;
  }

  const int lane = tid & 63;
  const bool one_wave = P.E <= 64;  // (uniform) every expert is in wave 0
  if (R == 1) {
    // stage 1: the k best of the wave's segment {64*wave + i + 256*r}.
    // (a) an expert with k or more strictly larger score words in its 16-lane
    // row has k experts beating it and is dropped; (b) the survivors' keys are
    // compacted per wave; (c) each survivor is ranked among them.  Everything
    // that beats a top-k expert of the segment survives (a), so the survivor
    // ranks below k are its exact ranks in the segment.
    bool surv[2];
#pragma unroll
    for (int r = 0; r < 2; r++) {
      surv[r] = false;
      if (r < R) {  // (uniform) every lane takes part in the row moves
        const int above = row_count_above<15>((uint32_t)(kr[r] >> 32));
        surv[r] = kr[r] != 0ull && above < P.k;
      }
    }
    int ns = 0;
#pragma unroll
    for (int r = 0; r < 2; r++) {
      const unsigned long long m = __ballot(surv[r]);
      if (surv[r]) {
        const int pos = ns + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        sh.sk[wave][pos] = kr[r];
      }
      ns += __popcll(m);
    }
    if (lane < 8 && ns + lane < ((ns + 7) & ~7)) sh.sk[wave][ns + lane] = 0ull;  // pad to 8
    // with E <= 64 every expert is in wave 0, so its segment ranks are the pick
    // positions: wave 0 writes the picks itself, and neither the block barrier
    // here nor stage 2 is needed (its own LDS writes are ordered by a wave fence)
    if (one_wave) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 2; r++) {
      if (surv[r]) {
        const unsigned long long mine = kr[r];
        int rank = 0;
        for (int c = 0; c < ns; c += 8) {  // four reads in flight per step
          const ulonglong2 *q = reinterpret_cast<const ulonglong2 *>(&sh.sk[wave][c]);
          const ulonglong2 v0 = q[0], v1 = q[1], v2 = q[2], v3 = q[3];
          rank += (v0.x > mine) + (v0.y > mine) + (v1.x > mine) + (v1.y > mine) + (v2.x > mine) + (v2.y > mine) +
                  (v3.x > mine) + (v3.y > mine);
        }
        if (rank < P.k) {
          if (one_wave) {
            const int e = (int)~(uint32_t)mine;
            sh.pick[rank] = e;
            sh.pp[rank] = sh.p[e];
          } else {
            sh.ck[wave * P.k + rank] = mine;
          }
        }
      }
    }
    __syncthreads();
  } else {
    // stage 1 with two experts a thread (E > 256): t = the k-th largest score
    // word of the wave's segment (the largest t with at least k words >= t),
    // found bit by bit from the top with ballots; the segment's k best are the
    // keys whose word is above t and, of those equal to t, the lowest-index
    // ones (lane order, experts tid before tid + 256).  Their keys go to the
    // wave's k candidate slots, unranked: stage 2 ranks them.
    const uint32_t hw0 = (uint32_t)(kr[0] >> 32), hw1 = (uint32_t)(kr[1] >> 32);
    uint32_t t = 0;
#pragma unroll
    for (int b = 31; b >= 0; b--) {
      const uint32_t trial = t | (1u << b);
      const int c = __popcll(__ballot(hw0 >= trial)) + __popcll(__ballot(hw1 >= trial));
      t = c >= P.k ? trial : t;
    }
    const unsigned long long gt0 = __ballot(hw0 > t), gt1 = __ballot(hw1 > t);
    const unsigned long long eq0 = __ballot(hw0 == t && kr[0] != 0ull), eq1 = __ballot(hw1 == t && kr[1] != 0ull);
    const int m = P.k - (__popcll(gt0) + __popcll(gt1));  // ties to take, lowest index first
    auto below = [&](unsigned long long msk) {
      return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(msk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0u));
    };
    const bool sel0 = ((gt0 >> lane) & 1ull) || (((eq0 >> lane) & 1ull) && below(eq0) < m);
    const bool sel1 = ((gt1 >> lane) & 1ull) || (((eq1 >> lane) & 1ull) && __popcll(eq0) + below(eq1) < m);
    const unsigned long long s0 = __ballot(sel0), s1 = __ballot(sel1);
    if (lane < P.k) sh.ck[wave * P.k + lane] = 0ull;  // (then the selected keys over them: one wave, in order)
    if (sel0) sh.ck[wave * P.k + below(s0)] = kr[0];
    if (sel1) sh.ck[wave * P.k + __popcll(s0) + below(s1)] = kr[1];
    if (tid >= 4 * P.k && tid < ((4 * P.k + 7) & ~7)) sh.ck[tid] = 0ull;  // stage 2 reads in steps of 8
    __syncthreads();
  }

  // stage 2: rank among the candidates (4k slots; a dropped expert's key and
  // an empty slot are 0 and are never picked: k <= the kept experts)
  const int C = 4 * P.k;
  if (!one_wave && tid < C) {
    const unsigned long long mine = sh.ck[tid];
    if (mine != 0ull) {
      int rank = 0;
      for (int c = 0; c < C; c += 8) {  // slots past C are 0; C <= 4 * SEL_MAX_K, a multiple of 8
        const ulonglong2 *q = reinterpret_cast<const ulonglong2 *>(sh.ck + c);
        const ulonglong2 v0 = q[0], v1 = q[1], v2 = q[2], v3 = q[3];
        rank += (v0.x > mine) + (v0.y > mine) + (v1.x > mine) + (v1.y > mine) + (v2.x > mine) + (v2.y > mine) +
                (v3.x > mine) + (v3.y > mine);
      }
      if (rank < P.k) {
        const int e = (int)~(uint32_t)mine;
        sh.pick[rank] = e;
        sh.pp[rank] = sh.p[e];
      }
    }
  }
  if (!one_wave) __syncthreads();
  if (w_out && tid < P.k) {
    float wsum = 0.f;
#pragma unroll 8
    for (int j = 0; j < P.k; j++) wsum += sh.pp[j];  // f32, pick order
    wsum = fmaxf(wsum, P.wsum_min);
    w_out[tid] = sh.pp[tid] / wsum * P.scale;
  }
}

// select_load() then select_rank().
__device__ __forceinline__ void select_block(const float *__restrict__ l, const float *__restrict__ bias,
                                             const SelParams &P, SelShared &sh, float *__restrict__ w_out) {
  SelIn in;
  select_load(l, bias, P, in);
  select_rank(in, P, sh, w_out);
}

}  // namespace moe
