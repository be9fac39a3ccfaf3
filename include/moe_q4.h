/*
 * moe_q4.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts FFN step
 * with GGUF Q4_0 / Q4_1 experts.
 *
 * The layer these calls compute is the MoE FFN of the three diskformer engine
 * pages (Flint: diskformer 0.5.4->0.6.4 engines/flint_moe_ssd.js, file header;
 * Ling 3.0 flash: diskformer 0.5.3->0.6.4 engines/ling_moe_ssd.js, file header
 * and the routeLing / swiglu / moeAccum kernels; LFM2.5: diskformer
 * 0.5.4->0.6.6 engines/lfm2_moe_ssd.js, file header and the router comment
 * with TOPK_SIG_BODY and moeAccumB).  For each token t with FFN input x_t
 * (already RMS-normalised by the caller):
 *
 *   l_e   = sum_h Wr[e][h] x_t[h]                    router logits (F32 router)
 *   p_e   = 1 / (1 + exp(-l_e)),  s_e = p_e + b_e    sigmoid; bias b selects only
 *   [groups] keep the groups_used groups whose two largest s sum highest
 *   ids   = the top_k experts by s (lowest index wins ties), in pick order
 *   w_j   = p_{id_j} / max(sum_j p_{id_j}, wsum_min) * weights_scale
 *   resid_t += sum_j w_j * FFN_{id_j}(x_t) + FFN_shared(x_t)
 *   FFN(x) = Wd * (silu(Wg x) * (Wu x)),  silu(g) = g / (1 + exp(-g))
 *
 * Numerics.  Router logits accumulate in double and are rounded to f32; the
 * sigmoid of that f32 logit is evaluated in double and rounded to f32; scores,
 * group sums, comparisons and weights are f32 as on the pages.  Expert GEMVs
 * dequantise Q4 in registers and accumulate in f32.  Outputs are bitwise
 * reproducible run to run (no floating-point atomics).
 *
 * Conventions for every call:
 *   - every pointer is a DEVICE pointer unless stated; all work is enqueued on
 *     `stream` and the call returns without synchronising;
 *   - the caller owns every buffer; the library allocates nothing and keeps no
 *     pointer after returning; calls are reentrant for distinct workspaces;
 *   - x, resid, router_w, logits_in, the workspace and the Q4 tensors must be
 *     16-byte aligned; ids, routing weights and the bias 4-byte aligned; rows of Q4 tensors
 *     are whole blocks, consecutive (Q4_1 rows stay 4-byte aligned, Q4_0 rows
 *     may be 2-byte aligned, which the kernels handle);
 *   - T = 0 is a no-op returning MOE_OK;
 *   - on any error nothing is enqueued and moe_last_error() describes it;
 *     faults of the kernels themselves surface at the caller's next sync.
 */
#ifndef MOE_Q4_H
#define MOE_Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *moe_stream_t; /* a hipStream_t; NULL = default stream */

enum { MOE_Q4_0 = 0, MOE_Q4_1 = 1, MOE_Q8_0 = 2 };

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,     /* a configuration/shape rule below, or a NULL required pointer */
  MOE_EALIGN = -2,     /* a pointer is not 16-byte aligned */
  MOE_EWORKSPACE = -3, /* workspace NULL or smaller than moe_workspace_bytes() */
  MOE_ELAUNCH = -4     /* a kernel launch failed (hipGetLastError) */
};

/* Layer shape.  Limits (the pages cap E at 512 and k at 32):
 *   hidden H:      32 <= H <= 8192, H % 32 == 0
 *   n_experts E:   1 <= E <= 512, or 0 for a dense SwiGLU FFN layer (the
 *                  leading layers of the three pages' models: no router, the
 *                  FFN sits in the shared-expert tensors, shared_ff is its
 *                  size; then top_k = 0, n_groups = groups_used = 1, and
 *                  expert_ff and the routed tensors are ignored)
 *   top_k k:       1 <= k <= min(32, E)  (0 for a dense layer)
 *   n_groups G:    1 <= G <= 64, E % G == 0, E/G >= 2 when G > 1
 *   groups_used:   1 <= Gu <= G, k <= Gu * (E/G); Gu == G means no group limit
 *   expert_ff F:   32 <= F <= 8192, F % 32 == 0
 *   shared_ff SF:  0 (no shared expert) or 32 <= SF <= 16384, SF % 32 == 0
 *   qtype:         MOE_Q4_0, MOE_Q4_1 or MOE_Q8_0 (routed and shared experts
 *                  alike; Q8_0 = f16 d and 32 signed bytes, 34 B, value d*q,
 *                  as the lfm2_moe_ssd.js page's int8 expert plane)
 *   weights_scale: finite, > 0 (1 for Flint and LFM2.5, 2.5 for Ling)
 *   wsum_min:      finite, > 0 (2^-14 = 6.103515625e-5 on all three pages)
 *   swiglu_limit, swiglu_limit_shared: finite, >= 0.  SwiGLU clamp L of the
 *                  routed experts and of the shared expert (the ling_moe_ssd.js
 *                  page's swiglu kernel and per-layer clamp lists): with L > 0,
 *                  act = min(silu(g), L) * clamp(u, -L, L); 0 = no clamp.
 *                  A layer's own values; moe_stack_step applies one config
 *                  (and so one pair of limits) to all its layers.
 *   norm_eps:      RMSNorm epsilon (attention.layer_norm_rms_epsilon), used
 *                  when a layer's ffn_norm is given: finite, > 0 then.
 *
 * Pre-FFN RMSNorm: when moe_layer_weights.ffn_norm is not NULL, the x a call
 * takes is the residual stream h and the FFN input is xn = f32(h * s * w),
 * s = 1 / sqrt(mean(h^2) + eps) (the flint_moe_ssd.js and lfm2_moe_ssd.js
 * file headers: ffn(rms_norm(x) * ffn_norm)); x may then alias resid, which
 * is the chained form resid += FFN(rms_norm(resid) * w).  Without ffn_norm, x
 * is the (already normalised) FFN input and must not alias resid.          */
typedef struct {
  int32_t hidden, n_experts, top_k;
  int32_t n_groups, groups_used;
  int32_t expert_ff, shared_ff;
  int32_t qtype;
  float weights_scale;
  float wsum_min;
  float swiglu_limit;
  float swiglu_limit_shared;
  float norm_eps;
} moe_config;

/* Weights of one MoE layer (GGUF tensor names in brackets).  Block tensors
 * hold Q4 blocks: Q4_1 = 20 bytes (f16 d, f16 m, 16 nibble bytes; value
 * d*q + m), Q4_0 = 18 bytes (f16 d, 16 nibble bytes; value d*(q-8)); byte i of
 * the nibbles holds element i (low nibble) and element i+16 (high nibble). */
typedef struct {
  const float *router_w;      /* [E][H] f32                          (ffn_gate_inp)     */
  const float *router_bias;   /* [E] f32, selection only; NULL = none (exp_probs_b)     */
  const uint8_t *gate_exps;   /* [E][F][H/32] blocks                 (ffn_gate_exps)    */
  const uint8_t *up_exps;     /* [E][F][H/32] blocks                 (ffn_up_exps)      */
  const uint8_t *down_exps;   /* [E][H][F/32] blocks                 (ffn_down_exps)    */
  const uint8_t *gate_shexp;  /* [SF][H/32] blocks, NULL iff SF == 0 (ffn_gate_shexp)   */
  const uint8_t *up_shexp;    /* [SF][H/32] blocks, NULL iff SF == 0 (ffn_up_shexp)     */
  const uint8_t *down_shexp;  /* [H][SF/32] blocks, NULL iff SF == 0 (ffn_down_shexp)   */
  const float *ffn_norm;      /* [H] f32 pre-FFN RMSNorm weight, or NULL  (ffn_norm)    */
} moe_layer_weights;

/* Bytes of device workspace the calls below need for T tokens (16-byte
 * aligned, contents need not be initialised, not kept between calls).
 * Returns 0 for an invalid configuration or T < 0. */
size_t moe_workspace_bytes(const moe_config *cfg, int32_t T);

/* Router scoring and top-k selection for T tokens (the lfm2_moe_ssd.js page's
 * router comment and TOPK_SIG_BODY; group-limited selection from the
 * ling_moe_ssd.js page's routeLing).
 *   x:         [T][H] f32 FFN input (ignored when logits_in != NULL)
 *   logits_in: NULL = compute logits from router_w and x; else [T][E] f32
 *              logits used as given (selection-only path)
 *   ids:       [T][k] int32 out, pick order (descending score, lowest index
 *              first on ties)
 *   weights:   [T][k] f32 out, aligned with ids
 * router_w may be NULL when logits_in is given. */
int moe_router_topk(const moe_config *cfg, const moe_layer_weights *w, const float *x, int32_t T,
                    const float *logits_in, int32_t *ids, float *weights, void *workspace,
                    size_t workspace_bytes, moe_stream_t stream);

/* Expert FFNs for given routing: resid[t] += sum_j weights[t][j] *
 * FFN_{ids[t][j]}(x_t) + FFN_shared(x_t) (the ling_moe_ssd.js page's swiglu
 * and moeAccum; the lfm2_moe_ssd.js page's moeAccumB and shared-expert
 * addInPlace).  ids must be in [0, E) (not checked on the device; out-of-range
 * ids read out-of-bounds weights).  resid [T][H] f32 in/out, must not alias x.
 * Small T (decode) runs fused dequant-GEMV kernels; large T (chunked prefill)
 * groups the (token, pick) pairs by expert and runs per-expert MFMA GEMMs. */
int moe_expert_ffn_q4(const moe_config *cfg, const moe_layer_weights *w, const float *x, int32_t T,
                      const int32_t *ids, const float *weights, float *resid, void *workspace,
                      size_t workspace_bytes, moe_stream_t stream);

/* The whole step: moe_router_topk then moe_expert_ffn_q4 on the same
 * workspace.  ids_out / weights_out ([T][k]) are optional (NULL = keep in the
 * workspace). */
int moe_layer_step(const moe_config *cfg, const moe_layer_weights *w, const float *x, int32_t T,
                   float *resid, int32_t *ids_out, float *weights_out, void *workspace,
                   size_t workspace_bytes, moe_stream_t stream);

/* moe_layer_step without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array
 * of MOE_NOALLOC_SCRATCH_BYTES that each GPU holds until the process ends;
 * the call allocates nothing.  A T whose moe_workspace_bytes(cfg, T) exceeds
 * it is rejected with MOE_EWORKSPACE (16 MiB covers decode at every shape
 * and the grouped path up to 155 tokens at the Flint shape, 156 at the
 * LFM2.5 shape and 98 at the Ling shape).  Every call on one GPU uses that
 * GPU's one array, so calls that overlap on a GPU (other streams, other
 * threads) race and must be ordered by the caller.  No kernel needs the
 * array zeroed.  Otherwise as moe_layer_step. */
#define MOE_NOALLOC_SCRATCH_BYTES (16 << 20)
int moe_layer_step_noalloc(const moe_config *cfg, const moe_layer_weights *w, const float *x, int32_t T,
                           float *resid, int32_t *ids_out, float *weights_out, moe_stream_t stream);

/* L MoE layers of one shape run in order on one stream, each a
 * moe_layer_step: layer l reads x[l] and adds its FFN output to the shared
 * residual, so layer l+1's expert reads start only after layer l finished.
 *   layers:      host array of L weight sets
 *   x:           host array of L device pointers, each [T][H] f32
 *   ids_out / weights_out: [L][T][k] or NULL
 * The workspace is reused by every layer (moe_workspace_bytes(cfg, T)).
 * Every layer's arguments are checked before the first layer is enqueued, so
 * an invalid layer l returns an error naming it with nothing enqueued. */
int moe_stack_step(const moe_config *cfg, const moe_layer_weights *layers, int32_t L, const float *const *x,
                   int32_t T, float *resid, int32_t *ids_out, float *weights_out, void *workspace,
                   size_t workspace_bytes, moe_stream_t stream);

/* Message for the last non-zero return on this thread ("" if none).  This is
 * the C form of the pages' error convention: their engines refuse a model
 * shape or setting they do not implement by throwing an Error whose message
 * names the offending value (flint_moe_ssd.js page, configFromGgufFlint;
 * lfm2_moe_ssd.js page, initBuffers with its top-k and expert-count limits).
 * Here the call returns a MOE_E* code instead and this string carries the
 * message. */
const char *moe_last_error(void);

/* Diagnostics: where, in a workspace of moe_workspace_bytes(cfg, T) bytes, a
 * call over T tokens leaves an intermediate result (tests read them back).
 *   MOE_WS_IDS, MOE_WS_WEIGHTS: [T][k] routing of moe_layer_step when its
 *     ids_out / weights_out are NULL;
 *   grouped path only (T > moe_decode_max_tokens(), or shapes whose act row
 *   does not fit the decode kernels), for the last chunk of at most 512
 *   tokens: MOE_WS_OFFSETS [E+1] int32 (expert e's pairs are sorted positions
 *   offsets[e] .. offsets[e+1]-1), MOE_WS_PERM [Tc*k] int32 (the pair
 *   p = t*k + j at each sorted position; pairs ascend within an expert),
 *   MOE_WS_POS [Tc*k] int32 (the inverse of perm), MOE_WS_TILES [n][2] int32
 *   (expert, first position within it, of each 16-pair tile) and
 *   MOE_WS_NTILES (n, one int32).
 * Writes the byte offset and size; MOE_EINVAL if the region is not used for
 * this configuration and T. */
enum { MOE_WS_IDS = 1, MOE_WS_WEIGHTS = 2, MOE_WS_OFFSETS = 3, MOE_WS_PERM = 4, MOE_WS_POS = 5,
       MOE_WS_TILES = 6, MOE_WS_NTILES = 7 };
int moe_workspace_region(const moe_config *cfg, int32_t T, int32_t region, size_t *offset, size_t *bytes);

/* Largest T that takes the decode (GEMV) path; larger T takes the grouped
 * GEMM path. */
int32_t moe_decode_max_tokens(void);

/* Diagnostics: time launches of one kernel with HIP events recorded on the
 * stream each launch goes to (process-wide, not thread-safe; for benchmarks).
 * moe_kernel_timer_begin creates `capacity` event pairs and arms the timer
 * for `kernel`; every later launch of that kernel is bracketed until the
 * capacity is used.  moe_kernel_timer_end waits for the recorded events,
 * returns the number of timed launches in *count and the sum of their
 * durations in *total_ms, and releases the events. */
enum {
  MOE_KERNEL_ROUTER = 1,  /* router logits                              */
  MOE_KERNEL_SELECT = 2,  /* scores, group limit, top-k, weights         */
  MOE_KERNEL_GATEUP = 3,  /* gate||up GEMV + SwiGLU (decode)             */
  MOE_KERNEL_DOWN = 4,    /* down GEMV + weighted accumulate (decode)    */
  MOE_KERNEL_SORT = 5,    /* pairs grouped by expert (grouped path); the
                             same launch takes the input rows' scales and
                             their f16 hi + lo form                       */
  MOE_KERNEL_GROUP_GATEUP = 6, /* grouped gate||up MFMA GEMM + SwiGLU     */
  MOE_KERNEL_GROUP_DOWN = 7,   /* grouped down MFMA GEMM, weighted        */
  MOE_KERNEL_COMBINE = 8,      /* per-token sum into the residual         */
  MOE_KERNEL_RMSNORM = 9,      /* pre-FFN RMSNorm (when ffn_norm is given) */
  MOE_KERNEL_PRELUDE = 10,     /* decode of 2+ tokens: per-token select and
                                  the shared expert's gate||up for all tokens */
  MOE_KERNEL_ROW_SCALE = 11    /* grouped path of a layer without routed
                                  experts: the input rows' power-of-two
                                  scales and f16 hi + lo form for the MFMA
                                  operands                                  */
};
int moe_kernel_timer_begin(int32_t kernel, int32_t capacity);
/* Timer mode (before moe_kernel_timer_begin; kept until changed): drain 1
 * (the default) first waits for the stream to go idle, so the interval holds
 * the kernel and its dispatch from an idle queue; drain 0 records the events
 * in stream order, so the interval also holds the wait for the previous
 * kernel's end and the dispatch after it.  MOE_EINVAL while the timer is
 * armed. */
int moe_kernel_timer_drain(int32_t drain);
int moe_kernel_timer_end(int32_t *count, double *total_ms);

/* Probes of the chip (diagnostics; no part of the MoE step uses them).  They
 * measure what bounds the decode path: the rate of a plain streaming read,
 * the cost of a kernel boundary and the cost of an exchange between blocks
 * of one kernel across the XCDs.  Return MOE_OK, MOE_EINVAL or MOE_ELAUNCH.
 *   moe_probe_stream:   one launch of `blocks` x 256 threads reading `bytes`
 *                       (a multiple of 16, 16-byte aligned) of buf with
 *                       16-byte loads; sink (>= 256 words, or NULL) is
 *                       never written in practice.
 *   moe_probe_empty:    one launch of an empty kernel of `blocks` x 64.
 *   moe_probe_exchange: a cooperative launch of `blocks` x 256 threads that
 *                       run `rounds` all-to-all exchanges through slots
 *                       ([blocks] 64-bit words, zero before the launch):
 *                       each block publishes a word per round, then waits
 *                       until every block's word of that round is visible.
 *                       A wait that reads one slot spin_limit times gives up
 *                       and sets status[0] = 1.  cycles[0..1]: the 100 MHz
 *                       real-time counter at the start and end (block 0). */
int moe_probe_stream(const void *buf, size_t bytes, int32_t blocks, uint32_t *sink, moe_stream_t stream);
int moe_probe_empty(int32_t blocks, moe_stream_t stream);
int moe_probe_exchange(int32_t blocks, int32_t rounds, uint32_t spin_limit, void *slots, uint32_t *status,
                       unsigned long long *cycles, moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_Q4_H */
