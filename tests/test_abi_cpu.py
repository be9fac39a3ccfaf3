"""CPU checks of the C-ABI library: it loads, exports every symbol the public
header declares, and rejects invalid arguments before touching the GPU."""
import ctypes as C
import os
import re

import pytest

import sparse_moe_ffn_topk_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    L = moe.load_library()
    decl = _declared_symbols()
    assert set(decl) >= {"moe_workspace_bytes", "moe_router_topk", "moe_expert_ffn_q4", "moe_layer_step",
                         "moe_last_error"}
    for n in decl:
        assert hasattr(L, n), n
    assert set(moe.EXPORTED) == set(decl)


def test_struct_layouts_match_header():
    assert C.sizeof(moe.MoeConfig) == 13 * 4
    assert C.sizeof(moe.LayerWeights) == 9 * 8


def _cfg(**kw):
    base = dict(hidden=256, n_experts=8, top_k=2, expert_ff=128)
    base.update(kw)
    return moe.make_config(**base)


@pytest.mark.parametrize("kw,msg", [
    (dict(hidden=100), "hidden"), (dict(hidden=0), "hidden"), (dict(hidden=16384), "hidden"),
    (dict(n_experts=0), "n_experts"), (dict(n_experts=513), "n_experts"),
    (dict(top_k=0), "top_k"), (dict(top_k=9), "top_k"), (dict(n_experts=64, top_k=33), "top_k"),
    (dict(n_groups=3), "n_groups"), (dict(n_experts=8, n_groups=8), "groups of"),
    (dict(n_groups=4, groups_used=5), "groups_used"), (dict(n_groups=4, groups_used=0), "groups_used"),
    (dict(top_k=5, n_groups=4, groups_used=2), "exceeds"),
    (dict(expert_ff=100), "expert_ff"), (dict(shared_ff=16), "shared_ff"),
    (dict(qtype=3), "qtype"), (dict(weights_scale=0.0), "weights_scale"), (dict(wsum_min=-1.0), "wsum_min"),
    (dict(n_experts=0), "needs top_k 0"), (dict(n_experts=0, top_k=0), "needs its FFN size"),
    (dict(n_experts=0, top_k=0, shared_ff=64, n_groups=2, groups_used=1), "dense layer needs"),
    (dict(shared_ff=16416), "shared_ff"),
    (dict(swiglu_limit=-1.0), "swiglu"), (dict(swiglu_limit_shared=float("inf")), "swiglu"),
    (dict(swiglu_limit=float("nan")), "swiglu"),
])
def test_invalid_config_rejected(kw, msg):
    L = moe.load_library()
    cfg = _cfg(**kw)
    assert L.moe_workspace_bytes(C.byref(cfg), 1) == 0
    lw = moe.LayerWeights(*([0x1000] * 8 + [0]))
    rc = L.moe_layer_step(C.byref(cfg), C.byref(lw), C.c_void_p(0x1000), 1, C.c_void_p(0x2000), None, None,
                          C.c_void_p(0x3000), 1 << 30, None)
    assert rc == -1
    assert msg in L.moe_last_error().decode()


def test_dense_layer_config_accepted():
    # n_experts = top_k = 0: a dense SwiGLU FFN layer held in the shared tensors; expert_ff is ignored
    L = moe.load_library()
    for ff in (6144, 11776, 16384):
        cfg = _cfg(n_experts=0, top_k=0, expert_ff=0, shared_ff=ff)
        assert L.moe_workspace_bytes(C.byref(cfg), 1) > 0
        assert L.moe_workspace_bytes(C.byref(cfg), 600) > 0
    # routing a dense layer is a no-op that succeeds
    cfg = _cfg(n_experts=0, top_k=0, expert_ff=0, shared_ff=64)
    assert L.moe_router_topk(C.byref(cfg), None, None, 4, None, None, None, None, 0, None) == 0


def test_norm_rules():
    # with ffn_norm the eps must be > 0, and x may alias resid (the chained form); without it, it may not
    L = moe.load_library()
    lw = moe.LayerWeights(*([0x1000] * 8 + [0x4000]))
    bad = _cfg(norm_eps=0.0)
    rc = L.moe_layer_step(C.byref(bad), C.byref(lw), C.c_void_p(0x2000), 1, C.c_void_p(0x3000), None, None,
                          C.c_void_p(0x5000), 1 << 30, None)
    assert rc == -1 and "norm_eps" in L.moe_last_error().decode()
    ok = _cfg(norm_eps=1e-5)
    # x == resid with a norm passes the argument checks (then stops at the missing workspace)
    rc = L.moe_layer_step(C.byref(ok), C.byref(lw), C.c_void_p(0x2000), 1, C.c_void_p(0x2000), None, None,
                          None, 0, None)
    assert rc == -3, L.moe_last_error().decode()
    lw.ffn_norm = None
    rc = L.moe_layer_step(C.byref(ok), C.byref(lw), C.c_void_p(0x2000), 1, C.c_void_p(0x2000), None, None,
                          None, 0, None)
    assert rc == -1 and "alias" in L.moe_last_error().decode()


def test_workspace_bytes_grows_with_tokens():
    L = moe.load_library()
    cfg = _cfg(shared_ff=64)
    a, b = L.moe_workspace_bytes(C.byref(cfg), 1), L.moe_workspace_bytes(C.byref(cfg), 8)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0
    assert L.moe_workspace_bytes(C.byref(cfg), -1) == 0


def test_pointer_errors_are_reported_without_launching():
    L = moe.load_library()
    cfg = _cfg()
    ws = L.moe_workspace_bytes(C.byref(cfg), 2)
    good = [0x10000] * 8
    good[1] = 0  # no bias
    good[5] = good[6] = good[7] = 0  # no shared expert
    lw = moe.LayerWeights(*good)
    x, r, w = C.c_void_p(0x20000), C.c_void_p(0x30000), C.c_void_p(0x40000)
    # NULL x
    assert L.moe_layer_step(C.byref(cfg), C.byref(lw), None, 2, r, None, None, w, ws, None) == -1
    # misaligned resid
    assert L.moe_layer_step(C.byref(cfg), C.byref(lw), x, 2, C.c_void_p(0x30004), None, None, w, ws, None) == -2
    # resid aliases x
    assert L.moe_layer_step(C.byref(cfg), C.byref(lw), x, 2, x, None, None, w, ws, None) == -1
    # workspace too small / NULL
    assert L.moe_layer_step(C.byref(cfg), C.byref(lw), x, 2, r, None, None, w, ws - 1, None) == -3
    assert L.moe_layer_step(C.byref(cfg), C.byref(lw), x, 2, r, None, None, None, ws, None) == -3
    # shared expert pointers missing when shared_ff > 0
    cfg2 = _cfg(shared_ff=64)
    ws2 = L.moe_workspace_bytes(C.byref(cfg2), 2)
    assert L.moe_layer_step(C.byref(cfg2), C.byref(lw), x, 2, r, None, None, w, ws2, None) == -1
    assert "gate_shexp" in L.moe_last_error().decode()
    # T = 0 is a no-op that succeeds without a workspace
    assert L.moe_layer_step(C.byref(cfg), C.byref(lw), x, 0, r, None, None, None, 0, None) == 0
    assert L.moe_last_error().decode() == ""
    # negative T
    assert L.moe_router_topk(C.byref(cfg), C.byref(lw), x, -1, None, w, w, w, ws, None) == -1


def test_wide_configs_take_the_grouped_path_workspace():
    # k*F + SF beyond the decode kernels' LDS staging: such shapes run the
    # grouped path at any T, so even T = 1 reserves its regions
    L = moe.load_library()
    wide = moe.make_config(1024, 64, 32, 512)
    narrow = moe.make_config(1024, 64, 4, 512)
    assert L.moe_workspace_bytes(C.byref(wide), 1) > 0
    assert L.moe_workspace_bytes(C.byref(narrow), 1) > 0
    # many tokens: the grouped path's chunked regions
    assert L.moe_workspace_bytes(C.byref(narrow), 4096) > L.moe_workspace_bytes(C.byref(narrow), 8)


def _stack_args(n=3):
    good = [0x10000] * 8
    good[1] = 0  # no bias
    good[5] = good[6] = good[7] = 0  # no shared expert
    layers = (moe.LayerWeights * n)(*[moe.LayerWeights(*good) for _ in range(n)])
    xs = (C.c_void_p * n)(*([0x20000] * n))
    return layers, xs


def test_stack_checks_every_layer_before_enqueueing():
    # an invalid layer 1 of 3: the stack call fails naming layer 1 before it enqueues layer 0 (without a
    # GPU, enqueueing layer 0 would have failed first, with MOE_ELAUNCH)
    L = moe.load_library()
    cfg = _cfg()
    ws = L.moe_workspace_bytes(C.byref(cfg), 1)
    layers, xs = _stack_args()
    layers[1].down_exps = None
    rc = L.moe_stack_step(C.byref(cfg), layers, 3, xs, 1, C.c_void_p(0x30000), None, None, C.c_void_p(0x40000), ws,
                          None)
    msg = L.moe_last_error().decode()
    assert rc == -1 and msg.startswith("layer 1:") and "down_exps" in msg, (rc, msg)
    layers, xs = _stack_args()
    xs[2] = 0x20004  # misaligned input of layer 2
    rc = L.moe_stack_step(C.byref(cfg), layers, 3, xs, 1, C.c_void_p(0x30000), None, None, C.c_void_p(0x40000), ws,
                          None)
    msg = L.moe_last_error().decode()
    assert rc == -2 and msg.startswith("layer 2:"), (rc, msg)
    # T = 0: every layer is still checked, then nothing runs
    layers, xs = _stack_args()
    assert L.moe_stack_step(C.byref(cfg), layers, 3, xs, 0, C.c_void_p(0x30000), None, None, None, 0, None) == 0


def test_workspace_regions():
    L = moe.load_library()
    cfg = _cfg(shared_ff=64)
    for T in (9, 512, 700):
        total = L.moe_workspace_bytes(C.byref(cfg), T)
        seen = []
        for region in (moe.WS_IDS, moe.WS_WEIGHTS, moe.WS_OFFSETS, moe.WS_PERM, moe.WS_POS, moe.WS_TILES,
                       moe.WS_NTILES):
            off, n = moe.workspace_region(cfg, T, region)
            assert off % 256 == 0 and off + n <= total
            seen.append((off, off + n))
        seen.sort()
        assert all(a[1] <= b[0] for a, b in zip(seen, seen[1:])), "regions overlap"
    # the decode path keeps no sort results
    with pytest.raises(moe.MoeError):
        moe.workspace_region(cfg, 8, moe.WS_PERM)
    assert moe.workspace_region(cfg, 8, moe.WS_IDS)[1] == 8 * cfg.top_k * 4
