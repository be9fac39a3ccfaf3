"""Python binding of libmoe_q4.so: the routed MoE FFN step with Q4_0 / Q4_1
experts on MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
(include/moe_q4.h).  torch supplies device memory (tensor.data_ptr()) and the
current HIP stream.  There is no fallback: if the built library is missing,
load_library() raises.
"""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_q4.so")

MOE_Q4_0, MOE_Q4_1, MOE_Q8_0 = 0, 1, 2
WSUM_MIN = 6.103515625e-5  # 2^-14

_lib = None


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"moe error {code}: {msg}")
        self.code = code


class MoeConfig(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("n_groups", C.c_int32), ("groups_used", C.c_int32),
                ("expert_ff", C.c_int32), ("shared_ff", C.c_int32), ("qtype", C.c_int32),
                ("weights_scale", C.c_float), ("wsum_min", C.c_float),
                ("swiglu_limit", C.c_float), ("swiglu_limit_shared", C.c_float), ("norm_eps", C.c_float)]


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("router_w", "router_bias", "gate_exps", "up_exps", "down_exps",
                                          "gate_shexp", "up_shexp", "down_shexp", "ffn_norm")]


def load_library(path=LIB_PATH):
    """Load the built HIP library; raises if it is missing (no CPU fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is not built: run __graft_entry__.build() "
                                f"(or python sparse_moe_ffn_topk_amd/build.py) first")
    L = C.CDLL(path)
    P, S = C.c_void_p, C.c_size_t
    L.moe_workspace_bytes.restype = S
    L.moe_workspace_bytes.argtypes = [C.POINTER(MoeConfig), C.c_int32]
    L.moe_router_topk.restype = C.c_int
    L.moe_router_topk.argtypes = [C.POINTER(MoeConfig), C.POINTER(LayerWeights), P, C.c_int32, P, P, P, P, S, P]
    L.moe_expert_ffn_q4.restype = C.c_int
    L.moe_expert_ffn_q4.argtypes = [C.POINTER(MoeConfig), C.POINTER(LayerWeights), P, C.c_int32, P, P, P, P, S, P]
    L.moe_layer_step.restype = C.c_int
    L.moe_layer_step.argtypes = [C.POINTER(MoeConfig), C.POINTER(LayerWeights), P, C.c_int32, P, P, P, P, S, P]
    L.moe_last_error.restype = C.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_decode_max_tokens.restype = C.c_int32
    L.moe_decode_max_tokens.argtypes = []
    L.moe_stack_step.restype = C.c_int
    L.moe_stack_step.argtypes = [C.POINTER(MoeConfig), C.POINTER(LayerWeights), C.c_int32, C.POINTER(C.c_void_p),
                                 C.c_int32, P, P, P, P, S, P]
    L.moe_kernel_timer_begin.restype = C.c_int
    L.moe_kernel_timer_begin.argtypes = [C.c_int32, C.c_int32]
    L.moe_kernel_timer_drain.restype = C.c_int
    L.moe_kernel_timer_drain.argtypes = [C.c_int32]
    L.moe_kernel_timer_end.restype = C.c_int
    L.moe_kernel_timer_end.argtypes = [C.POINTER(C.c_int32), C.POINTER(C.c_double)]
    L.moe_workspace_region.restype = C.c_int
    L.moe_workspace_region.argtypes = [C.POINTER(MoeConfig), C.c_int32, C.c_int32, C.POINTER(C.c_size_t),
                                       C.POINTER(C.c_size_t)]
    L.moe_layer_step_noalloc.restype = C.c_int
    L.moe_layer_step_noalloc.argtypes = [C.POINTER(MoeConfig), C.POINTER(LayerWeights), P, C.c_int32, P, P, P, P]
    L.moe_probe_stream.restype = C.c_int
    L.moe_probe_stream.argtypes = [P, S, C.c_int32, P, P]
    L.moe_probe_empty.restype = C.c_int
    L.moe_probe_empty.argtypes = [C.c_int32, P]
    L.moe_probe_exchange.restype = C.c_int
    L.moe_probe_exchange.argtypes = [C.c_int32, C.c_int32, C.c_uint32, P, P, P, P]
    _lib = L
    return L


EXPORTED = ("moe_workspace_bytes", "moe_router_topk", "moe_expert_ffn_q4", "moe_layer_step", "moe_last_error",
            "moe_decode_max_tokens", "moe_kernel_timer_begin", "moe_kernel_timer_end", "moe_kernel_timer_drain", "moe_stack_step",
            "moe_workspace_region", "moe_probe_stream", "moe_probe_empty", "moe_probe_exchange",
            "moe_layer_step_noalloc")
NOALLOC_SCRATCH_BYTES = 16 << 20
WS_IDS, WS_WEIGHTS, WS_OFFSETS, WS_PERM, WS_POS, WS_TILES, WS_NTILES = 1, 2, 3, 4, 5, 6, 7
KERNEL_ROUTER, KERNEL_SELECT, KERNEL_GATEUP, KERNEL_DOWN = 1, 2, 3, 4
KERNEL_SORT, KERNEL_GROUP_GATEUP, KERNEL_GROUP_DOWN, KERNEL_COMBINE, KERNEL_RMSNORM = 5, 6, 7, 8, 9
KERNEL_PRELUDE, KERNEL_ROW_SCALE = 10, 11


def make_config(hidden, n_experts, top_k, expert_ff, shared_ff=0, qtype=MOE_Q4_1, n_groups=1, groups_used=None,
                weights_scale=1.0, wsum_min=WSUM_MIN, swiglu_limit=0.0, swiglu_limit_shared=0.0, norm_eps=1e-5):
    return MoeConfig(hidden, n_experts, top_k, n_groups, n_groups if groups_used is None else groups_used,
                     expert_ff, shared_ff, qtype, weights_scale, wsum_min, swiglu_limit, swiglu_limit_shared, norm_eps)


def config_for(wl):
    """MoeConfig of a moe_synth.Workload-like object."""
    return make_config(wl.hidden, wl.n_experts, wl.top_k, wl.expert_ff, wl.shared_ff, wl.qtype, wl.n_groups,
                       wl.groups_used, wl.weights_scale, swiglu_limit=getattr(wl, "swiglu_limit", 0.0),
                       swiglu_limit_shared=getattr(wl, "swiglu_limit_shared", 0.0),
                       norm_eps=getattr(wl, "norm_eps", 0.0) or 1e-5)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _keep_for(stream, *temps):
    """Temporaries allocated here on the current stream but used by kernels on `stream`: tell torch's caching
    allocator, so it does not hand their memory to other work before those kernels finish."""
    import torch
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in temps:
        if t is not None:
            t.record_stream(stream)


def _check(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def layer_weights(w):
    """LayerWeights from a dict of device tensors (keys as moe_synth.make_layer)."""
    import torch
    _check(w.get("router_w"), "router_w", torch.float32)
    _check(w.get("bias"), "bias", torch.float32)
    _check(w.get("ffn_norm"), "ffn_norm", torch.float32)
    for n in ("gate_exps", "up_exps", "down_exps", "gate_sh", "up_sh", "down_sh"):
        _check(w.get(n), n, torch.uint8)
    return LayerWeights(*[None if w.get(n) is None else w[n].data_ptr()
                          for n in ("router_w", "bias", "gate_exps", "up_exps", "down_exps",
                                    "gate_sh", "up_sh", "down_sh", "ffn_norm")])


def _raise(rc):
    if rc != 0:
        raise MoeError(rc, load_library().moe_last_error().decode())


def workspace_bytes(cfg, T):
    return load_library().moe_workspace_bytes(C.byref(cfg), T)


def workspace_region(cfg, T, region):
    """(byte offset, bytes) of a workspace region (diagnostics: WS_* constants)."""
    off, n = C.c_size_t(0), C.c_size_t(0)
    _raise(load_library().moe_workspace_region(C.byref(cfg), T, region, C.byref(off), C.byref(n)))
    return off.value, n.value


def alloc_workspace(cfg, T, device="cuda"):
    import torch
    n = workspace_bytes(cfg, T)
    if n == 0:
        raise MoeError(-1, "invalid configuration")
    return torch.empty(n, dtype=torch.uint8, device=device)


def router_topk(cfg, w, x, logits_in=None, ids=None, weights=None, workspace=None, stream=None, lw=None):
    import torch
    T = (logits_in if x is None else x).shape[0]
    dev = (logits_in if x is None else x).device
    _check(x, "x", torch.float32)
    _check(logits_in, "logits_in", torch.float32)
    temps = []
    if ids is None:
        ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
        temps.append(ids)
    if weights is None:
        weights = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
        temps.append(weights)
    if workspace is None:
        workspace = alloc_workspace(cfg, T, dev)
        temps.append(workspace)
    _keep_for(stream, *temps)
    lw = lw if lw is not None else layer_weights(w)
    _raise(load_library().moe_router_topk(C.byref(cfg), C.byref(lw), _ptr(x), T, _ptr(logits_in), _ptr(ids),
                                          _ptr(weights), _ptr(workspace), workspace.numel(), _stream(stream)))
    return ids, weights


def expert_ffn_q4(cfg, w, x, ids, weights, resid, workspace=None, stream=None, lw=None):
    import torch
    T = x.shape[0]
    _check(x, "x", torch.float32)
    _check(ids, "ids", torch.int32)
    _check(weights, "weights", torch.float32)
    _check(resid, "resid", torch.float32)
    if workspace is None:
        workspace = alloc_workspace(cfg, T, x.device)
        _keep_for(stream, workspace)
    lw = lw if lw is not None else layer_weights(w)
    _raise(load_library().moe_expert_ffn_q4(C.byref(cfg), C.byref(lw), _ptr(x), T, _ptr(ids), _ptr(weights),
                                            _ptr(resid), _ptr(workspace), workspace.numel(), _stream(stream)))
    return resid


def layer_step(cfg, w, x, resid, ids_out=None, weights_out=None, workspace=None, stream=None, lw=None):
    import torch
    T = x.shape[0]
    _check(x, "x", torch.float32)
    _check(resid, "resid", torch.float32)
    _check(ids_out, "ids_out", torch.int32)
    _check(weights_out, "weights_out", torch.float32)
    if workspace is None:
        workspace = alloc_workspace(cfg, T, x.device)
        _keep_for(stream, workspace)
    lw = lw if lw is not None else layer_weights(w)
    _raise(load_library().moe_layer_step(C.byref(cfg), C.byref(lw), _ptr(x), T, _ptr(resid), _ptr(ids_out),
                                         _ptr(weights_out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return resid


def layer_step_noalloc(cfg, w, x, resid, ids_out=None, weights_out=None, stream=None, lw=None):
    """moe_layer_step_noalloc: the layer step on the library's static device scratch (no workspace)."""
    import torch
    T = x.shape[0]
    _check(x, "x", torch.float32)
    _check(resid, "resid", torch.float32)
    _check(ids_out, "ids_out", torch.int32)
    _check(weights_out, "weights_out", torch.float32)
    lw = lw if lw is not None else layer_weights(w)
    _raise(load_library().moe_layer_step_noalloc(C.byref(cfg), C.byref(lw), _ptr(x), T, _ptr(resid), _ptr(ids_out),
                                                 _ptr(weights_out), _stream(stream)))
    return resid


class Stack:
    """L layers of one shape run in order by moe_stack_step (one native call per step)."""

    def __init__(self, cfg, layers, xs, resid, ids=None, wts=None, workspace=None):
        self.cfg, self.L, self.resid = cfg, len(layers), resid
        self.lws = (LayerWeights * self.L)(*[layer_weights(w) for w in layers])
        self.xs = (C.c_void_p * self.L)(*[x.data_ptr() for x in xs])
        self.T = xs[0].shape[0]
        self.ids, self.wts = ids, wts
        self.ws = workspace if workspace is not None else alloc_workspace(cfg, self.T, resid.device)
        self._keep = (layers, xs)

    def step(self, stream=None):
        _raise(load_library().moe_stack_step(C.byref(self.cfg), self.lws, self.L, self.xs, self.T, _ptr(self.resid),
                                             _ptr(self.ids), _ptr(self.wts), _ptr(self.ws), self.ws.numel(),
                                             _stream(stream)))


class KernelTimer:
    """Times every launch of one kernel with HIP events on its own stream (diagnostics).  drain (default): wait
    for the stream to go idle before each timed launch; otherwise the events are recorded in stream order."""

    def __init__(self, kernel, capacity, drain=True):
        self.kernel, self.capacity, self.drain = kernel, capacity, drain

    def __enter__(self):
        _raise(load_library().moe_kernel_timer_drain(1 if self.drain else 0))
        _raise(load_library().moe_kernel_timer_begin(self.kernel, self.capacity))
        return self

    def __exit__(self, *exc):
        n, ms = C.c_int32(0), C.c_double(0.0)
        rc = load_library().moe_kernel_timer_end(C.byref(n), C.byref(ms))
        self.count, self.total_ms = n.value, ms.value
        if exc[0] is None:
            _raise(rc)
        return False

    @property
    def mean_us(self):
        return 1000.0 * self.total_ms / max(self.count, 1)
