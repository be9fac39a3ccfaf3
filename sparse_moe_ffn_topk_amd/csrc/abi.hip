// abi.hip -- the C ABI of the MoE step: argument checks, workspace layout and
// kernel sequencing on the caller's stream.  Nothing here allocates device
// memory or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <string>

#include "../../include/moe_q4.h"
#include "moe_launch.h"

// Workspace of moe_layer_step_noalloc: a fixed array in device memory that
// every GPU the library runs on holds from module load to process end.  In
// host code `scratch` names a host-side stand-in, not the device array: host
// code only ever uses the device address hipGetSymbolAddress returns for the
// current device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

constexpr int kDecodeMaxT = 8;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace regions (byte offsets, each 256-byte aligned).  Decode (T <= 8)
// uses logits/ids/wts/act; the grouped path works on chunks of at most
// PREFILL_CHUNK tokens and adds the sort results and its act and Y rows.
struct Layout {
  size_t logits, ids, wts, act, xn, offsets, pos, perm, tiles, ntiles, pact, pact_sh, Y, Ysh, xexp, aexp, xhl, xsum, total;
};

Layout layout(const moe_config &c, int32_t T) {
  Layout L;
  const size_t k = c.top_k, E = c.n_experts, SF = c.shared_ff, H = c.hidden;
  const size_t F = c.top_k > 0 ? c.expert_ff : 0;  // (a dense layer: no routed rows)
  const size_t Tc = T < moe::PREFILL_CHUNK ? (size_t)T : (size_t)moe::PREFILL_CHUNK;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += up256(bytes);
    return at;
  };
  L.logits = take((size_t)T * E * 4);
  L.ids = take((size_t)T * k * 4);
  L.wts = take((size_t)T * k * 4);
  L.act = take(((size_t)T * k * F + (size_t)T * SF) * 4);
  L.xn = take((size_t)T * H * 4);  // normalised FFN input (layers with ffn_norm)
  const bool grouped = T > kDecodeMaxT || moe::decode_down_lds_bytes(c.top_k, c.expert_ff, c.shared_ff) > 65536;
  if (grouped) {
    L.offsets = take((E + 1) * 4);
    L.pos = take(Tc * k * 4);
    L.perm = take(Tc * k * 4);
    L.tiles = take(((Tc * k + 15) / 16 + E) * 2 * 4);
    L.ntiles = take(4);
    L.pact = take(Tc * k * F * 4);
    L.pact_sh = take(Tc * SF * 4);
    L.Y = take(Tc * k * H * 4);
    L.Ysh = take(Tc * H * 4);
    L.xexp = take(Tc * 4);
    L.aexp = take(Tc * (k + 1) * 4);
    L.xhl = take(Tc * H * 4);          // the input rows as f16 hi + lo pairs
    L.xsum = take(Tc * (H / 32) * 4);  // and their 32-value block sums
  } else {
    L.offsets = L.pos = L.perm = L.tiles = L.ntiles = L.pact = L.pact_sh = L.Y = L.Ysh = L.xexp = L.aexp = 0;
    L.xhl = L.xsum = 0;
  }
  L.total = o;
  return L;
}

int check_cfg(const moe_config *c) {
  if (!c) return fail(MOE_EINVAL, "cfg is NULL");
  const int H = c->hidden, E = c->n_experts, k = c->top_k, G = c->n_groups, Gu = c->groups_used;
  if (H < 32 || H > 8192 || H % 32) return fail(MOE_EINVAL, "hidden %d: need 32 <= H <= 8192, H %% 32 == 0", H);
  if (E == 0) {
    // a dense SwiGLU FFN layer: no router, the shared-expert tensors hold the FFN
    if (k != 0) return fail(MOE_EINVAL, "top_k %d: a dense layer (n_experts 0) needs top_k 0", k);
    if (G != 1 || Gu != 1) return fail(MOE_EINVAL, "n_groups/groups_used: a dense layer needs 1 and 1");
    if (c->shared_ff == 0) return fail(MOE_EINVAL, "shared_ff 0: a dense layer (n_experts 0) needs its FFN size");
  } else {
    if (E < 1 || E > 512) return fail(MOE_EINVAL, "n_experts %d: need 0 (dense) or 1..512", E);
    if (k < 1 || k > 32 || k > E) return fail(MOE_EINVAL, "top_k %d: need 1 <= k <= min(32, E=%d)", k, E);
    if (G < 1 || G > 64 || E % G) return fail(MOE_EINVAL, "n_groups %d: need 1..64 dividing E=%d", G, E);
    if (G > 1 && E / G < 2) return fail(MOE_EINVAL, "groups of %d experts: need >= 2 per group", E / G);
    if (Gu < 1 || Gu > G) return fail(MOE_EINVAL, "groups_used %d: need 1..G=%d", Gu, G);
    if ((long)k > (long)Gu * (E / G)) return fail(MOE_EINVAL, "top_k %d exceeds the experts of %d kept groups", k, Gu);
    if (c->expert_ff < 32 || c->expert_ff > 8192 || c->expert_ff % 32)
      return fail(MOE_EINVAL, "expert_ff %d: need 32 <= F <= 8192, F %% 32 == 0", c->expert_ff);
  }
  if (c->shared_ff != 0 && (c->shared_ff < 32 || c->shared_ff > 16384 || c->shared_ff % 32))
    return fail(MOE_EINVAL, "shared_ff %d: need 0 or 32 <= SF <= 16384, SF %% 32 == 0", c->shared_ff);
  if (c->qtype != MOE_Q4_0 && c->qtype != MOE_Q4_1 && c->qtype != MOE_Q8_0)
    return fail(MOE_EINVAL, "qtype %d: need 0 (Q4_0), 1 (Q4_1) or 2 (Q8_0)", c->qtype);
  if (!(std::isfinite(c->weights_scale) && c->weights_scale > 0))
    return fail(MOE_EINVAL, "weights_scale must be finite and > 0");
  if (!(std::isfinite(c->wsum_min) && c->wsum_min > 0)) return fail(MOE_EINVAL, "wsum_min must be finite and > 0");
  if (!(std::isfinite(c->swiglu_limit) && c->swiglu_limit >= 0) ||
      !(std::isfinite(c->swiglu_limit_shared) && c->swiglu_limit_shared >= 0))
    return fail(MOE_EINVAL, "swiglu limits must be finite and >= 0");
  return MOE_OK;
}

int check_ptr(const void *p, const char *name, bool required) {
  if (!p) return required ? fail(MOE_EINVAL, "%s is NULL", name) : MOE_OK;
  if (!aligned16(p)) return fail(MOE_EALIGN, "%s is not 16-byte aligned", name);
  return MOE_OK;
}
// ids, routing weights and the bias are read and written element by element
int check_ptr4(const void *p, const char *name, bool required) {
  if (!p) return required ? fail(MOE_EINVAL, "%s is NULL", name) : MOE_OK;
  if ((uintptr_t)p & 3u) return fail(MOE_EALIGN, "%s is not 4-byte aligned", name);
  return MOE_OK;
}

int check_ws(const moe_config &c, int32_t T, void *ws, size_t bytes) {
  size_t need = layout(c, T).total;
  if (!ws) return fail(MOE_EWORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (!aligned16(ws)) return fail(MOE_EALIGN, "workspace is not 16-byte aligned");
  if (bytes < need) return fail(MOE_EWORKSPACE, "workspace has %zu bytes, need %zu", bytes, need);
  return MOE_OK;
}

int check_expert_ptrs(const moe_config &c, const moe_layer_weights *w) {
  int rc;
  const bool routed = c.n_experts > 0;
  if ((rc = check_ptr(w->gate_exps, "gate_exps", routed))) return rc;
  if ((rc = check_ptr(w->up_exps, "up_exps", routed))) return rc;
  if ((rc = check_ptr(w->down_exps, "down_exps", routed))) return rc;
  const bool sh = c.shared_ff > 0;
  if ((rc = check_ptr(w->gate_shexp, "gate_shexp", sh))) return rc;
  if ((rc = check_ptr(w->up_shexp, "up_shexp", sh))) return rc;
  if ((rc = check_ptr(w->down_shexp, "down_shexp", sh))) return rc;
  return MOE_OK;
}

// With a norm weight: check it and eps, and normalise x into the workspace.
// *xin is then the normalised input (else x itself).
int prologue_norm(const moe_config &c, const moe_layer_weights *w, const float *x, int32_t T, void *ws,
                  hipStream_t st, const float **xin);

int launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(MOE_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

int router_topk_impl(const moe_config &c, const moe_layer_weights *w, const float *x, int32_t T,
                     const float *logits_in, int32_t *ids, float *wts, void *ws, hipStream_t st) {
  const Layout L = layout(c, T);
  const float *logits = logits_in;
  if (!logits_in) {
    float *lg = (float *)((char *)ws + L.logits);
    int rc = launched(moe::launch_router_logits(w->router_w, x, c.hidden, c.n_experts, T, lg, st), "router logits");
    if (rc) return rc;
    logits = lg;
  }
  return launched(moe::launch_select(logits, w->router_bias, T, c.n_experts, c.top_k, c.n_groups, c.groups_used,
                                     c.weights_scale, c.wsum_min, ids, wts, st),
                  "top-k select");
}

// Expert FFNs.  With logits != NULL (decode path of moe_layer_step) the
// tokens are routed on the way (one token: in the gate||up kernel's prologue;
// more: in the decode prelude), which writes ids / wts.
int expert_ffn_impl(const moe_config &c, const moe_layer_weights *w, const float *x, int32_t T, int32_t *ids,
                    float *wts, const float *logits, float *resid, void *ws, hipStream_t st) {
  const Layout L = layout(c, T);
  moe::DecodeArgs a;
  a.qtype = c.qtype;
  a.T = T;
  a.H = c.hidden;
  a.k = c.top_k;
  a.F = c.top_k > 0 ? c.expert_ff : 0;  // (a dense layer: no routed rows)
  a.SF = c.shared_ff;
  a.x = x;
  a.ids = ids;
  a.wts = wts;
  a.logits = logits;
  a.bias = w->router_bias;
  a.sel = moe::SelParams{c.n_experts, c.top_k, c.n_groups, c.groups_used, c.weights_scale, c.wsum_min};
  a.lim = c.swiglu_limit;
  a.lim_sh = c.swiglu_limit_shared;
  a.gate_exps = w->gate_exps;
  a.up_exps = w->up_exps;
  a.down_exps = w->down_exps;
  a.gate_sh = w->gate_shexp;
  a.up_sh = w->up_shexp;
  a.down_sh = w->down_shexp;
  a.act = (float *)((char *)ws + L.act);
  a.resid = resid;
  return launched(moe::launch_decode_ffn(a, st), "decode expert FFN");
}

// Grouped (prefill) expert FFNs, chunk by chunk of at most PREFILL_CHUNK tokens.
int prefill_ffn_impl(const moe_config &c, const moe_layer_weights *w, const float *x, int32_t T, const int32_t *ids,
                     const float *wts, float *resid, void *ws, hipStream_t st) {
  const Layout L = layout(c, T);
  char *b = (char *)ws;
  for (int32_t t0 = 0; t0 < T; t0 += moe::PREFILL_CHUNK) {
    const int32_t Tc = T - t0 < moe::PREFILL_CHUNK ? T - t0 : moe::PREFILL_CHUNK;
    moe::PrefillArgs p;
    p.qtype = c.qtype;
    p.T = Tc;
    p.H = c.hidden;
    p.k = c.top_k;
    p.F = c.top_k > 0 ? c.expert_ff : 0;
    p.SF = c.shared_ff;
    p.E = c.n_experts;
    p.x = x + (size_t)t0 * c.hidden;
    p.ids = ids + (size_t)t0 * c.top_k;
    p.wts = wts + (size_t)t0 * c.top_k;
    p.gate_exps = w->gate_exps;
    p.up_exps = w->up_exps;
    p.down_exps = w->down_exps;
    p.gate_sh = w->gate_shexp;
    p.up_sh = w->up_shexp;
    p.down_sh = w->down_shexp;
    p.offsets = (int32_t *)(b + L.offsets);
    p.pos = (int32_t *)(b + L.pos);
    p.perm = (int32_t *)(b + L.perm);
    p.tiles = (int32_t *)(b + L.tiles);
    p.ntiles = (int32_t *)(b + L.ntiles);
    p.act = (float *)(b + L.pact);
    p.act_sh = (float *)(b + L.pact_sh);
    p.Y = (float *)(b + L.Y);
    p.Ysh = (float *)(b + L.Ysh);
    p.resid = resid + (size_t)t0 * c.hidden;
    p.xexp = (int32_t *)(b + L.xexp);
    p.aexp = (int32_t *)(b + L.aexp);
    p.xhl = (uint16_t *)(b + L.xhl);
    p.xsum = (float *)(b + L.xsum);
    p.lim = c.swiglu_limit;
    p.lim_sh = c.swiglu_limit_shared;
    int rc = launched(moe::launch_prefill_ffn(p, st), "grouped expert FFN");
    if (rc) return rc;
  }
  return MOE_OK;
}

int prologue_norm(const moe_config &c, const moe_layer_weights *w, const float *x, int32_t T, void *ws,
                  hipStream_t st, const float **xin) {
  *xin = x;
  if (!w->ffn_norm) return MOE_OK;
  float *xn = (float *)((char *)ws + layout(c, T).xn);
  *xin = xn;
  return launched(moe::launch_rmsnorm(x, w->ffn_norm, c.hidden, T, c.norm_eps, xn, st), "rmsnorm");
}

int check_norm(const moe_config &c, const moe_layer_weights *w) {
  int rc;
  if ((rc = check_ptr(w->ffn_norm, "ffn_norm", false))) return rc;
  if (w->ffn_norm && !(std::isfinite(c.norm_eps) && c.norm_eps > 0))
    return fail(MOE_EINVAL, "norm_eps must be finite and > 0 when ffn_norm is given");
  return MOE_OK;
}

// Decode kernels stage a token's whole act row in LDS; configurations whose
// row does not fit take the grouped path at any T.
bool decode_fits(const moe_config &c) { return moe::decode_down_lds_bytes(c.top_k, c.expert_ff, c.shared_ff) <= 65536; }

// Every argument rule of one moe_layer_step (cfg already checked); enqueues
// nothing.
int check_layer_args(const moe_config &c, const moe_layer_weights *w, const float *x, int32_t T, float *resid,
                     int32_t *ids_out, float *weights_out, void *workspace, size_t workspace_bytes) {
  int rc;
  if (T < 0) return fail(MOE_EINVAL, "T %d < 0", T);
  if (T == 0) return MOE_OK;
  if (!w) return fail(MOE_EINVAL, "weights is NULL");
  const bool dense = c.n_experts == 0;
  if ((rc = check_ptr(w->router_w, "router_w", !dense))) return rc;
  if ((rc = check_ptr4(w->router_bias, "router_bias", false))) return rc;
  if ((rc = check_expert_ptrs(c, w))) return rc;
  if ((rc = check_ptr(x, "x", true))) return rc;
  if ((rc = check_ptr(resid, "resid", true))) return rc;
  if ((rc = check_norm(c, w))) return rc;
  if (resid == x && !w->ffn_norm) return fail(MOE_EINVAL, "resid must not alias x (unless ffn_norm is given)");
  if ((rc = check_ptr4(ids_out, "ids_out", false))) return rc;
  if ((rc = check_ptr4(weights_out, "weights_out", false))) return rc;
  return check_ws(c, T, workspace, workspace_bytes);
}

// The layer step on checked arguments (T > 0).
int layer_step_impl(const moe_config &c, const moe_layer_weights *w, const float *x, int32_t T, float *resid,
                    int32_t *ids_out, float *weights_out, void *workspace, hipStream_t st) {
  int rc;
  const Layout L = layout(c, T);
  const bool dense = c.n_experts == 0;
  int32_t *ids = ids_out ? ids_out : (int32_t *)((char *)workspace + L.ids);
  float *wts = weights_out ? weights_out : (float *)((char *)workspace + L.wts);
  const bool decode = T <= kDecodeMaxT && decode_fits(c);
  if (decode && !dense && w->ffn_norm && moe::router_fuses_norm(c.hidden, T)) {
    // decode with a norm: the router kernel normalises x and writes xn; the
    // gate||up kernel routes a single token in its prologue, more tokens are
    // routed once each in the decode prelude
    float *lg = (float *)((char *)workspace + L.logits);
    float *xn = (float *)((char *)workspace + L.xn);
    if ((rc = launched(moe::launch_router_logits(w->router_w, x, c.hidden, c.n_experts, T, lg, st, w->ffn_norm,
                                                 c.norm_eps, xn),
                       "router logits + rmsnorm")))
      return rc;
    return expert_ffn_impl(c, w, xn, T, ids, wts, lg, resid, workspace, st);
  }
  if ((rc = prologue_norm(c, w, x, T, workspace, st, &x))) return rc;  // x: the FFN input from here on
  if (dense) {  // no router: only the FFN held in the shared-expert tensors
    if (decode) return expert_ffn_impl(c, w, x, T, ids, wts, nullptr, resid, workspace, st);
    return prefill_ffn_impl(c, w, x, T, ids, wts, resid, workspace, st);
  }
  if (decode) {
    // decode: router logits, then the gate||up kernel routes one token in its
    // prologue (more tokens: the decode prelude routes each once)
    float *lg = (float *)((char *)workspace + L.logits);
    if ((rc = launched(moe::launch_router_logits(w->router_w, x, c.hidden, c.n_experts, T, lg, st),
                       "router logits")))
      return rc;
    return expert_ffn_impl(c, w, x, T, ids, wts, lg, resid, workspace, st);
  }
  if ((rc = router_topk_impl(c, w, x, T, nullptr, ids, wts, workspace, st))) return rc;
  return prefill_ffn_impl(c, w, x, T, ids, wts, resid, workspace, st);
}

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int noalloc_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ELAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EINVAL, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ELAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

// ---- kernel timer (diagnostics) ----
struct Timer {
  int kernel = 0, capacity = 0, count = 0;
  bool drain = true;
  hipEvent_t *start = nullptr, *stop = nullptr;
} g_timer;

}  // namespace

namespace moe {
TimerSlot timer_slot(int id) {
  TimerSlot t;
  if (g_timer.kernel == id && g_timer.count < g_timer.capacity) {
    t.start = g_timer.start[g_timer.count];
    t.stop = g_timer.stop[g_timer.count++];
    t.drain = g_timer.drain;
  }
  return t;
}
}  // namespace moe

extern "C" {

int moe_kernel_timer_end(int32_t *count, double *total_ms);

int moe_kernel_timer_drain(int32_t drain) {
  g_err.clear();
  if (g_timer.kernel) return fail(MOE_EINVAL, "kernel timer: set the drain mode before moe_kernel_timer_begin");
  g_timer.drain = drain != 0;
  return MOE_OK;
}

int moe_kernel_timer_begin(int32_t kernel, int32_t capacity) {
  g_err.clear();
  if (g_timer.kernel) moe_kernel_timer_end(nullptr, nullptr);
  if (kernel < MOE_KERNEL_ROUTER || kernel > MOE_KERNEL_ROW_SCALE || capacity < 1 || capacity > (1 << 20))
    return fail(MOE_EINVAL, "kernel timer: bad kernel %d or capacity %d", kernel, capacity);
  g_timer.start = new hipEvent_t[capacity];
  g_timer.stop = new hipEvent_t[capacity];
  for (int i = 0; i < capacity; i++) {
    if (hipEventCreate(&g_timer.start[i]) != hipSuccess || hipEventCreate(&g_timer.stop[i]) != hipSuccess) {
      g_timer.capacity = i;
      moe_kernel_timer_end(nullptr, nullptr);
      return fail(MOE_ELAUNCH, "kernel timer: hipEventCreate failed");
    }
  }
  g_timer.kernel = kernel;
  g_timer.capacity = capacity;
  g_timer.count = 0;
  return MOE_OK;
}

int moe_kernel_timer_end(int32_t *count, double *total_ms) {
  double total = 0.0;
  int n = g_timer.count, rc = MOE_OK;
  for (int i = 0; i < n; i++) {
    float ms = 0.f;
    if (hipEventSynchronize(g_timer.stop[i]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timer.start[i], g_timer.stop[i]) != hipSuccess)
      rc = fail(MOE_ELAUNCH, "kernel timer: event %d not measurable", i);
    total += ms;
  }
  for (int i = 0; i < g_timer.capacity; i++) {
    (void)hipEventDestroy(g_timer.start[i]);
    (void)hipEventDestroy(g_timer.stop[i]);
  }
  delete[] g_timer.start;
  delete[] g_timer.stop;
  const bool drain = g_timer.drain;
  g_timer = Timer();
  g_timer.drain = drain;
  if (count) *count = n;
  if (total_ms) *total_ms = total;
  return rc;
}


size_t moe_workspace_bytes(const moe_config *cfg, int32_t T) {
  if (T < 0 || check_cfg(cfg) != MOE_OK) return 0;
  return layout(*cfg, T).total;
}

const char *moe_last_error(void) { return g_err.c_str(); }

int moe_workspace_region(const moe_config *cfg, int32_t T, int32_t region, size_t *offset, size_t *bytes) {
  g_err.clear();
  int rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (T < 1) return fail(MOE_EINVAL, "T %d < 1", T);
  if (!offset || !bytes) return fail(MOE_EINVAL, "offset or bytes is NULL");
  const Layout L = layout(*cfg, T);
  const bool grouped = L.offsets != 0;
  const size_t k = cfg->top_k, E = cfg->n_experts;
  const size_t Tc = T < moe::PREFILL_CHUNK ? (size_t)T : (size_t)moe::PREFILL_CHUNK;
  switch (region) {
    case MOE_WS_IDS: *offset = L.ids; *bytes = (size_t)T * k * 4; return MOE_OK;
    case MOE_WS_WEIGHTS: *offset = L.wts; *bytes = (size_t)T * k * 4; return MOE_OK;
    default: break;
  }
  if (!grouped || k == 0) return fail(MOE_EINVAL, "region %d: not used for T %d with this configuration", region, T);
  switch (region) {
    case MOE_WS_OFFSETS: *offset = L.offsets; *bytes = (E + 1) * 4; return MOE_OK;
    case MOE_WS_POS: *offset = L.pos; *bytes = Tc * k * 4; return MOE_OK;
    case MOE_WS_PERM: *offset = L.perm; *bytes = Tc * k * 4; return MOE_OK;
    case MOE_WS_NTILES: *offset = L.ntiles; *bytes = 4; return MOE_OK;
    case MOE_WS_TILES: *offset = L.tiles; *bytes = ((Tc * k + 15) / 16 + E) * 2 * 4; return MOE_OK;
    default: return fail(MOE_EINVAL, "region %d: unknown", region);
  }
}

int32_t moe_decode_max_tokens(void) { return kDecodeMaxT; }

int moe_router_topk(const moe_config *cfg, const moe_layer_weights *w, const float *x, int32_t T,
                    const float *logits_in, int32_t *ids, float *weights, void *workspace, size_t workspace_bytes,
                    moe_stream_t stream) {
  g_err.clear();
  int rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T %d < 0", T);
  if (T == 0 || cfg->n_experts == 0) return MOE_OK;  // (a dense layer routes nothing)
  if (!w) return fail(MOE_EINVAL, "weights is NULL");
  if ((rc = check_ptr(logits_in, "logits_in", false))) return rc;
  if (!logits_in) {
    if ((rc = check_ptr(w->router_w, "router_w", true))) return rc;
    if ((rc = check_ptr(x, "x", true))) return rc;
  }
  if ((rc = check_ptr4(w->router_bias, "router_bias", false))) return rc;
  if ((rc = check_ptr4(ids, "ids", true))) return rc;
  if ((rc = check_ptr4(weights, "weights", true))) return rc;
  if ((rc = check_norm(*cfg, w))) return rc;
  if ((rc = check_ws(*cfg, T, workspace, workspace_bytes))) return rc;
  const float *xin = x;
  if (!logits_in && (rc = prologue_norm(*cfg, w, x, T, workspace, (hipStream_t)stream, &xin))) return rc;
  return router_topk_impl(*cfg, w, xin, T, logits_in, ids, weights, workspace, (hipStream_t)stream);
}

int moe_expert_ffn_q4(const moe_config *cfg, const moe_layer_weights *w, const float *x, int32_t T,
                      const int32_t *ids, const float *weights, float *resid, void *workspace,
                      size_t workspace_bytes, moe_stream_t stream) {
  g_err.clear();
  int rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T %d < 0", T);
  if (T == 0) return MOE_OK;
  if (!w) return fail(MOE_EINVAL, "weights is NULL");
  if ((rc = check_expert_ptrs(*cfg, w))) return rc;
  if ((rc = check_ptr(x, "x", true))) return rc;
  if ((rc = check_ptr4(ids, "ids", cfg->top_k > 0))) return rc;
  if ((rc = check_ptr4(weights, "weights", cfg->top_k > 0))) return rc;
  if ((rc = check_ptr(resid, "resid", true))) return rc;
  if ((rc = check_norm(*cfg, w))) return rc;
  if (resid == x && !w->ffn_norm) return fail(MOE_EINVAL, "resid must not alias x (unless ffn_norm is given)");
  if ((rc = check_ws(*cfg, T, workspace, workspace_bytes))) return rc;
  const float *xin;
  if ((rc = prologue_norm(*cfg, w, x, T, workspace, (hipStream_t)stream, &xin))) return rc;
  if (T > kDecodeMaxT || !decode_fits(*cfg))
    return prefill_ffn_impl(*cfg, w, xin, T, ids, weights, resid, workspace, (hipStream_t)stream);
  return expert_ffn_impl(*cfg, w, xin, T, const_cast<int32_t *>(ids), const_cast<float *>(weights), nullptr, resid,
                         workspace, (hipStream_t)stream);
}

int moe_layer_step(const moe_config *cfg, const moe_layer_weights *w, const float *x, int32_t T, float *resid,
                   int32_t *ids_out, float *weights_out, void *workspace, size_t workspace_bytes,
                   moe_stream_t stream) {
  g_err.clear();
  int rc;
  if ((rc = check_cfg(cfg))) return rc;
  if ((rc = check_layer_args(*cfg, w, x, T, resid, ids_out, weights_out, workspace, workspace_bytes))) return rc;
  if (T == 0) return MOE_OK;
  return layer_step_impl(*cfg, w, x, T, resid, ids_out, weights_out, workspace, (hipStream_t)stream);
}

int moe_layer_step_noalloc(const moe_config *cfg, const moe_layer_weights *w, const float *x, int32_t T,
                           float *resid, int32_t *ids_out, float *weights_out, moe_stream_t stream) {
  g_err.clear();
  int rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T %d < 0", T);
  if (T == 0) return MOE_OK;
  const size_t need = layout(*cfg, T).total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_EWORKSPACE, "T %d needs %zu bytes of workspace, above the %d-byte static scratch of "
                "moe_layer_step_noalloc (use moe_layer_step with a workspace, or fewer tokens)",
                T, need, MOE_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if ((rc = noalloc_scratch(&ws))) return rc;
  if ((rc = check_layer_args(*cfg, w, x, T, resid, ids_out, weights_out, ws, need))) return rc;
  return layer_step_impl(*cfg, w, x, T, resid, ids_out, weights_out, ws, (hipStream_t)stream);
}

int moe_stack_step(const moe_config *cfg, const moe_layer_weights *layers, int32_t L, const float *const *x,
                   int32_t T, float *resid, int32_t *ids_out, float *weights_out, void *workspace,
                   size_t workspace_bytes, moe_stream_t stream) {
  g_err.clear();
  if (L < 0) return fail(MOE_EINVAL, "L %d < 0", L);
  if (L > 0 && (!layers || !x)) return fail(MOE_EINVAL, "layers or x is NULL");
  int rc;
  if ((rc = check_cfg(cfg))) return rc;
  const size_t per = (size_t)T * cfg->top_k;
  // every layer is checked before the first one is enqueued: on an error
  // nothing runs
  for (int32_t l = 0; l < L; l++) {
    rc = check_layer_args(*cfg, &layers[l], x[l], T, resid, ids_out ? ids_out + l * per : nullptr,
                          weights_out ? weights_out + l * per : nullptr, workspace, workspace_bytes);
    if (rc) {
      std::string m = g_err;
      return fail(rc, "layer %d: %s", l, m.c_str());
    }
  }
  if (T == 0) return MOE_OK;
  for (int32_t l = 0; l < L; l++) {
    rc = layer_step_impl(*cfg, &layers[l], x[l], T, resid, ids_out ? ids_out + l * per : nullptr,
                         weights_out ? weights_out + l * per : nullptr, workspace, (hipStream_t)stream);
    if (rc) {
      std::string m = g_err;
      return fail(rc, "layer %d: %s", l, m.c_str());
    }
  }
  return MOE_OK;
}

}  // extern "C"
