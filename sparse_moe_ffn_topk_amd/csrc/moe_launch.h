// moe_launch.h -- host-side launchers of the MoE kernels (internal).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Router logits [T][E] f32 from W [E][H] and x [T][H] (f64 accumulation).
// With gnorm (only where router_fuses_norm(H, T)): x is the residual stream,
// normalised in the kernel (RMSNorm weight gnorm, eps), and the normalised
// input is written to xn [T][H].
int router_fuses_norm(int H, int T);
hipError_t launch_router_logits(const float *W, const float *x, int H, int E, int T, float *logits,
                                hipStream_t st, const float *gnorm = nullptr, float eps = 0.f,
                                float *xn = nullptr);

// Pre-FFN RMSNorm of T tokens: xn = f32(x * s * g), s = 1/sqrt(mean(x^2) + eps)
// with the sum of squares in f64; one block per token.
hipError_t launch_rmsnorm(const float *x, const float *g, int H, int T, float eps, float *xn, hipStream_t st);

// Scores, optional group limit, top-k, weights; one block per token.
hipError_t launch_select(const float *logits, const float *bias, int T, int E, int k, int G, int Gu,
                         float scale, float wsum_min, int32_t *ids, float *wts, hipStream_t st);

// Routing parameters: experts, top-k, groups, groups kept, weights scale,
// clamp on the picked-sigmoid sum.
struct SelParams {
  int E, k, G, Gu;
  float scale, wsum_min;
};

struct DecodeArgs {
  int qtype, T, H, k, F, SF;
  const float *x;
  int32_t *ids;     // [T][k]: written by the gate||up kernel when logits != NULL, else read
  float *wts;       // [T][k]: likewise
  const float *logits;  // [T][E] router logits to route in-kernel, or NULL
  const float *bias;    // selection bias or NULL
  SelParams sel;
  const uint8_t *gate_exps, *up_exps, *down_exps;
  const uint8_t *gate_sh, *up_sh, *down_sh;
  float *act;    // per token: [k][F] routed rows, then [SF] shared
  float *resid;  // [T][H] in/out
  float lim, lim_sh;  // SwiGLU clamp of the routed and of the shared experts (0: none)
  int down_split = 1;  // waves sharing one row group's task list in the down kernel (set by its launcher)
  int sf_tasks = 0;    // shared rows the gate||up kernel computes: SF, or 0 after the multi-token prelude
};

// gate||up + SwiGLU, then down + weighted per-token accumulate.
hipError_t launch_decode_ffn(const DecodeArgs &a, hipStream_t st);
size_t decode_down_lds_bytes(int k, int F, int SF);

// Many tokens (chunked prefill, T <= PREFILL_CHUNK): sort the pairs by expert,
// grouped MFMA GEMMs, combine.
constexpr int PREFILL_CHUNK = 512;
struct PrefillArgs {
  int qtype, T, H, k, F, SF, E;
  const float *x;          // [T][H]
  const int32_t *ids;      // [T][k]
  const float *wts;        // [T][k]
  const uint8_t *gate_exps, *up_exps, *down_exps;
  const uint8_t *gate_sh, *up_sh, *down_sh;
  int32_t *offsets, *pos, *perm, *tiles, *ntiles;  // sort results
  float *act, *act_sh;     // [T*k][F] sorted, [T][SF]
  float *Y, *Ysh;          // [T*k][H] sorted and weighted, [T][H]
  float *resid;            // [T][H] in/out
  float lim, lim_sh;       // SwiGLU clamp of the routed and of the shared experts (0: none)
  int32_t *xexp, *aexp;    // [T], [T*k + T]: the rows' largest f32 exponents (scales of the f16 MFMA inputs)
  uint16_t *xhl;           // [T][H/8][16]: each octet of x, scaled by its row's power of two, as 8 f16 hi then 8 f16 lo parts
  float *xsum;             // [T][H/32]: the scaled values' sum over each 32-value block
};
hipError_t launch_prefill_ffn(const PrefillArgs &p, hipStream_t st);
size_t prefill_sort_lds_bytes(int T, int E);

// Kernel timer (diagnostics, eager launches only): when armed for kernel `id`,
// timer_slot() hands out the next (start, stop) event pair, which the launch
// attaches to the kernel's own dispatch (hipExtLaunchKernelGGL), so the events
// time that kernel's execution on its stream; otherwise both are NULL.  With
// drain set (moe_kernel_timer_begin's mode 1) the stream is drained before a
// timed launch, so the interval also holds the dispatch from an idle queue.
struct TimerSlot {
  hipEvent_t start = nullptr, stop = nullptr;
  bool drain = false;
};
TimerSlot timer_slot(int id);

// Launch KERNEL (parenthesise template names) with the timer's events for ID.
#define MOE_LAUNCH(ID, KERNEL, GRID, BLOCK, LDS, ST, ...)                                                 \
  do {                                                                                                   \
    const ::moe::TimerSlot ts_ = ::moe::timer_slot(ID);                                                  \
    if (ts_.start && ts_.drain) (void)hipStreamSynchronize(ST);                                          \
    hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, ST, ts_.start, ts_.stop, 0, __VA_ARGS__);            \
  } while (0)

}  // namespace moe
