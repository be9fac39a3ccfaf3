"""Double-precision CPU oracle of the routed MoE FFN step (Q4_0 / Q4_1 experts).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg; the product library never imports it.

Thin ctypes marshalling over moe_oracle.c; every function there cites the page
passage it follows.  Arrays are numpy; results come back as float64 (values)
or int32 (ids, offsets, permutations).
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or (os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        L = C.CDLL(_build.LIB)
        P = C.c_void_p
        L.mo_f16.restype = C.c_double
        L.mo_f16.argtypes = [C.c_uint16]
        L.mo_dequant_row.argtypes = [C.c_int, P, C.c_int32, P]
        L.mo_row_dot.restype = C.c_double
        L.mo_row_dot.argtypes = [C.c_int, P, C.c_int32, P]
        L.mo_router_logits.argtypes = [P, P, C.c_int32, C.c_int32, P]
        L.mo_sigmoid.restype = C.c_double
        L.mo_sigmoid.argtypes = [C.c_double]
        L.mo_swiglu.restype = C.c_double
        L.mo_swiglu.argtypes = [C.c_double, C.c_double, C.c_double]
        L.mo_group_keep.argtypes = [P, C.c_int32, C.c_int32, C.c_int32, P, P]
        L.mo_topk.argtypes = [P, P, C.c_int32, C.c_int32, P]
        L.mo_route.restype = C.c_int
        L.mo_route.argtypes = [P, P, P, P, P, P]
        L.mo_expert_ffn.argtypes = [C.c_int, P, P, P, C.c_int32, C.c_int32, C.c_double, P, P]
        L.mo_layer.restype = C.c_int
        L.mo_layer.argtypes = [P] + [P] * 9 + [P, C.c_int32, P, P, P, P, P]
        L.mo_rmsnorm.argtypes = [P, P, C.c_int32, C.c_double, P]
        L.mo_sort_by_expert.argtypes = [P, C.c_int32, C.c_int32, P, P]
        _lib = L
    return _lib


class Cfg(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("n_groups", C.c_int32), ("groups_used", C.c_int32),
                ("expert_ff", C.c_int32), ("shared_ff", C.c_int32), ("qtype", C.c_int32),
                ("weights_scale", C.c_double), ("wsum_min", C.c_double),
                ("swiglu_limit", C.c_double), ("swiglu_limit_shared", C.c_double), ("norm_eps", C.c_double)]


Q4_0, Q4_1, Q8_0 = 0, 1, 2
WSUM_MIN = 6.103515625e-5


def make_cfg(hidden, n_experts, top_k, expert_ff, shared_ff=0, qtype=Q4_1, n_groups=1, groups_used=None,
             weights_scale=1.0, wsum_min=WSUM_MIN, swiglu_limit=0.0, swiglu_limit_shared=0.0, norm_eps=1e-5):
    return Cfg(hidden, n_experts, top_k, n_groups, groups_used if groups_used is not None else n_groups,
               expert_ff, shared_ff, qtype, weights_scale, wsum_min, swiglu_limit, swiglu_limit_shared, norm_eps)


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def f16(bits):
    return lib().mo_f16(int(bits))


def block_bytes(qtype):
    return {Q4_0: 18, Q4_1: 20, Q8_0: 34}[qtype]


def dequant_row(qtype, row_bytes):
    """row_bytes: uint8 array of nb whole blocks -> float64[32*nb]."""
    b = _c(row_bytes, np.uint8).reshape(-1)
    nb = b.size // block_bytes(qtype)
    out = np.empty(32 * nb, np.float64)
    lib().mo_dequant_row(qtype, _p(b), nb, _p(out))
    return out


def row_dot(qtype, row_bytes, x):
    b = _c(row_bytes, np.uint8).reshape(-1)
    nb = b.size // block_bytes(qtype)
    xd = _c(x, np.float64)
    return lib().mo_row_dot(qtype, _p(b), nb, _p(xd))


def router_logits(W, x):
    W = _c(W, np.float32)
    x = _c(x, np.float32)
    E, H = W.shape
    out = np.empty(E, np.float64)
    lib().mo_router_logits(_p(W), _p(x), E, H, _p(out))
    return out


def sigmoid(v):
    return lib().mo_sigmoid(float(v))


def swiglu(g, u, limit=0.0):
    return lib().mo_swiglu(float(g), float(u), float(limit))


def group_keep(s32, n_groups, groups_used):
    s = _c(s32, np.float32)
    keep = np.zeros(n_groups, np.int32)
    gs = np.zeros(n_groups, np.float32)
    lib().mo_group_keep(_p(s), s.size, n_groups, groups_used, _p(keep), _p(gs))
    return keep, gs


def topk(s32, k, allowed=None):
    s = _c(s32, np.float32)
    a = _c(allowed, np.int32)
    ids = np.empty(k, np.int32)
    lib().mo_topk(_p(s), _p(a), s.size, k, _p(ids))
    return ids


def route(cfg, logit32, logit64=None, bias=None):
    l32 = _c(logit32, np.float32)
    l64 = _c(logit64, np.float64)
    b = _c(bias, np.float32)
    ids = np.empty(cfg.top_k, np.int32)
    w = np.empty(cfg.top_k, np.float64)
    rc = lib().mo_route(C.byref(cfg), _p(l32), _p(l64), _p(b), _p(ids), _p(w))
    if rc:
        raise ValueError("oracle: fewer selectable experts than top_k")
    return ids, w


def expert_ffn(qtype, gate, up, down, H, F, x, limit=0.0):
    g, u, d = (_c(a, np.uint8) for a in (gate, up, down))
    xd = _c(x, np.float64)
    y = np.empty(H, np.float64)
    lib().mo_expert_ffn(qtype, _p(g), _p(u), _p(d), H, F, float(limit), _p(xd), _p(y))
    return y


def layer(cfg, w, x, resid=None, logits_in=None):
    """w: dict with router_w [E,H] f32, bias [E] f32 or None, gate_exps/up_exps/down_exps uint8,
    gate_sh/up_sh/down_sh uint8 or None, optional ffn_norm [H] f32 (then x is the residual stream and the
    FFN input is its RMSNorm).  x: [T,H] f32.  Returns (out f64 [T,H], ids [T,k], w [T,k])."""
    x = _c(x, np.float32)
    T, H = x.shape
    k = cfg.top_k
    rw = _c(w.get("router_w"), np.float32)
    bias = _c(w.get("bias"), np.float32)
    ge, ue, de = (_c(w[n], np.uint8) for n in ("gate_exps", "up_exps", "down_exps"))
    gs, us, ds = (_c(w.get(n), np.uint8) for n in ("gate_sh", "up_sh", "down_sh"))
    gn = _c(w.get("ffn_norm"), np.float32)
    r = _c(resid, np.float32)
    li = _c(logits_in, np.float32)
    out = np.empty((T, H), np.float64)
    ids = np.empty((T, k), np.int32)
    ww = np.empty((T, k), np.float64)
    rc = lib().mo_layer(C.byref(cfg), _p(rw), _p(bias), _p(ge), _p(ue), _p(de), _p(gs), _p(us), _p(ds), _p(gn),
                        _p(x), T, _p(r), _p(li), _p(out), _p(ids), _p(ww))
    if rc:
        raise ValueError("oracle: fewer selectable experts than top_k")
    return out, ids, ww


def rmsnorm(x, g, eps):
    """Pre-FFN RMSNorm of one token, rounded to f32 (mo_rmsnorm)."""
    xv, gv = _c(x, np.float32), _c(g, np.float32)
    out = np.empty(xv.size, np.float32)
    lib().mo_rmsnorm(_p(xv), _p(gv), xv.size, float(eps), _p(out))
    return out


def sort_by_expert(ids, n_experts):
    i = _c(ids, np.int32).reshape(-1)
    offsets = np.empty(n_experts + 1, np.int32)
    perm = np.empty(i.size, np.int32)
    lib().mo_sort_by_expert(_p(i), i.size, n_experts, _p(offsets), _p(perm))
    return offsets, perm
