"""GPU parity of the HIP path (called through the C ABI) against the f64 oracle.

Each case prints what names it before the GPU work so a failing run can be
traced from its output.
"""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle as O
from moe_testlib import (REG_TOL, REL_TOL, oracle_cfg, oracle_given_routing, oracle_layer, row_rel_err,
                         run_layer_parity, to_device)

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _ok(err, what, guard=REG_TOL):
    """The 1e-3 gate, then the regression guard (see moe_testlib)."""
    print(f"[result] {what} max_row_rel_err={err:.3e}", flush=True)
    assert err <= REL_TOL, f"{what}: {err:.3e} above the 1e-3 gate"
    assert err <= guard, f"{what}: {err:.3e} above the regression guard {guard:g}"


def _layer(wl, seed=0, tokens=None, step=0):
    w = S.make_layer(wl, layer=seed, device="cpu")
    x = S.make_x(wl, tokens=tokens, layer=seed, step=step, device="cpu")
    return w, x


# ----------------------------------------------------------- selection only --

SEL_CASES = {
    "tiny": dict(E=8, k=2),
    "flint": dict(E=256, k=6),
    "lfm25": dict(E=64, k=4, bias=True),
    "ling": dict(E=512, k=8, G=8, Gu=4, bias=True, scale=2.5),
    "k_eq_E": dict(E=16, k=16),
    "groups_all_used": dict(E=128, k=8, G=8, Gu=8),
    "max": dict(E=512, k=32, G=64, Gu=7, bias=True),
    "odd_E": dict(E=97, k=5),
    "small_E_groups": dict(E=64, k=6, G=8, Gu=3, bias=True),  # one wave holds every expert, with a group limit
}


@pytest.mark.parametrize("name", sorted(SEL_CASES))
def test_select_from_given_logits_bit_exact(gpu, name):
    moe = gpu
    c = SEL_CASES[name]
    E, k, G, Gu = c["E"], c["k"], c.get("G", 1), c.get("Gu", c.get("G", 1))
    T = 37
    _say("select", name, f"E={E} k={k} G={G} Gu={Gu} T={T}")
    g = torch.Generator().manual_seed(1000 + E + k)
    logits = (torch.randn((T, E), generator=g) * 2.5).float()
    logits[3] = 0.7  # a token with all-equal logits: pure index tie-break
    logits[4, : E // 2] = -30.0  # part of the table deep in the clamp region
    logits[5] = -30.0  # every sigmoid tiny: the weight-sum clamp applies
    bias = (torch.randn(E, generator=g) * 0.1).float() if c.get("bias") else None
    cfg = moe.make_config(64, E, k, 32, n_groups=G, groups_used=Gu, weights_scale=c.get("scale", 1.0))
    w = {"router_w": None, "bias": None if bias is None else bias.cuda()}
    ids, wts = moe.router_topk(cfg, w, None, logits_in=logits.cuda())
    ids, wts = ids.cpu().numpy(), wts.cpu().numpy()
    ocfg = O.make_cfg(64, E, k, 32, n_groups=G, groups_used=Gu, weights_scale=c.get("scale", 1.0))
    for t in range(T):
        rid, rw = O.route(ocfg, logits[t].numpy(), bias=None if bias is None else bias.numpy())
        assert list(ids[t]) == list(rid), f"token {t}"
        assert np.allclose(wts[t], rw, rtol=2e-6, atol=0), f"token {t}"


def test_select_clamp_and_scale_exact(gpu):
    moe = gpu
    _say("select clamp ling")
    logits = torch.full((2, 512), -30.0)
    cfg = moe.make_config(64, 512, 8, 32, n_groups=8, groups_used=4, weights_scale=2.5)
    ids, wts = moe.router_topk(cfg, {"router_w": None, "bias": None}, None, logits_in=logits.cuda())
    assert ids.cpu().tolist() == [list(range(8))] * 2
    p32 = np.float32(1.0 / (1.0 + np.exp(30.0)))
    want = np.float32(p32 / np.float32(2.0 ** -14) * np.float32(2.5))
    assert np.all(wts.cpu().numpy() == want)


# ------------------------------------------------------------- whole layer --

LAYER_CASES = ["tiny", "flint", "flint8", "lfm25", "ling"]


@pytest.mark.parametrize("name", LAYER_CASES)
@pytest.mark.parametrize("composed", [False, True])
def test_layer_step_parity(gpu, name, composed):
    wl = S.WORKLOADS[name]
    T = wl.tokens
    _say("layer", name, f"T={T} composed={composed}")
    w, x = _layer(wl, seed=3)
    wd, xd = to_device(w), x.cuda()
    resid = xd.clone() if composed else None
    err, ties = run_layer_parity(wl, wd, xd, resid, wnp=S.to_numpy(w))
    _ok(err, f"{name} composed={composed} near_ties={ties}")


@pytest.mark.parametrize("name,T", [("ling", 5), ("ling", 40), ("lfm25", 5), ("lfm25", 40)])
def test_layer_several_tokens_full_shapes(gpu, name, T):
    # the Ling (512 experts in groups: each selection thread holds two experts) and LFM2.5 (64 experts: one
    # wave holds them all) layers at several tokens: the decode prelude's selection (T = 5) and the grouped
    # path's (T = 40), every token row against the oracle
    wl = S.WORKLOADS[name]
    _say("layer", name, f"T={T}")
    w, x = _layer(wl, seed=11 + T, tokens=T)
    err, ties = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"{name} T={T} near_ties={ties}")


def test_layer_prefill_chunk(gpu):
    # 512 tokens through one Flint-shaped layer (grouped MFMA path), every
    # token row against the oracle, and the sort of the pairs bit-exact
    wl = S.WORKLOADS["prefill"]
    _say("layer prefill T=512 (all rows)")
    w, x = _layer(wl, seed=7)
    err, ties = run_layer_parity(wl, to_device(w), x.cuda(), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"prefill near_ties={ties}")


@pytest.mark.parametrize("name,T", [("flint_dense", 1), ("flint_dense", 8), ("flint_dense", 40),
                                    ("lfm25_dense", 1), ("lfm25_dense", 3), ("lfm25_dense", 520)])
def test_dense_ffn_layer(gpu, name, T):
    # dense leading SwiGLU FFN layers (no router), decode and grouped paths
    wl = S.WORKLOADS[name]
    _say(f"dense layer {name} SF={wl.shared_ff} Q4_{wl.qtype} T={T}")
    w, x = _layer(wl, seed=17, tokens=T)
    err, ties = run_layer_parity(wl, to_device(w), x.cuda(), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"dense {name} T={T}")


@pytest.mark.parametrize("name,T", [("flint", 1), ("flint8", 8), ("prefill", 512), ("flint_dense", 2),
                                    ("lfm25", 1), ("ling", 1)])
def test_layer_rmsnorm(gpu, name, T):
    # pre-FFN RMSNorm given as ffn_norm (x is the residual stream; the FFN sees rms_norm(x) * w)
    import dataclasses
    wl = dataclasses.replace(S.WORKLOADS[name], norm_eps=1e-5)
    _say(f"layer {name} T={T} with ffn_norm")
    w, x = _layer(wl, seed=19, tokens=T)
    x = x * 3.0 + 0.5  # a residual stream that is not already normalised
    err, ties = run_layer_parity(wl, to_device(w), x.cuda(), None, wnp=S.to_numpy(w))
    _ok(err, f"rmsnorm {name} T={T} near_ties={ties}")


@pytest.mark.parametrize("name,centred", [("flint", False), ("flint8", False), ("flint", True), ("ling", True)])
def test_chained_stack_with_rmsnorm(gpu, name, centred):
    # the chained form: each layer's input is the running residual, resid += FFN(rms_norm(resid) * w);
    # per layer against the oracle given that layer's input, and one stack call against per-layer calls
    # (centred: the Q4_1 offsets of the chained benchmark stack)
    import dataclasses
    moe = gpu
    wl = dataclasses.replace(S.WORKLOADS[name], norm_eps=1e-5, centred=centred)
    L = 3
    _say(f"chained stack {name} L={L} centred={centred}")
    layers = [S.make_layer(wl, layer=100 + l, device="cpu") for l in range(L)]
    dev = [to_device(w) for w in layers]
    h0 = S.make_x(wl, layer=99, device="cpu") * 2.0
    cfg = moe.config_for(wl)
    resid = h0.cuda().clone()
    for l in range(L):
        before = resid.cpu().numpy().copy()
        moe.layer_step(cfg, dev[l], resid, resid)  # x aliases resid
        torch.cuda.synchronize()
        ref, _, _ = O.layer(oracle_cfg(wl), S.to_numpy(layers[l]), before, resid=before)
        err = row_rel_err(resid.cpu().numpy() - before, ref - before).max()
        _ok(err, f"chained {name} layer {l}")
    stacked = h0.cuda().clone()
    st = moe.Stack(cfg, dev, [stacked] * L, stacked)
    st.step()
    torch.cuda.synchronize()
    assert torch.equal(stacked, resid)


STACK_CASES = [("flint", "chained"), ("ling", "chained"), ("lfm25", "independent_norm"), ("tiny", "independent"),
               ("flint", "independent")]


@pytest.mark.parametrize("name,mode", STACK_CASES)
def test_stack_against_oracle_chain(gpu, name, mode):
    # one token through L layers in one stack call (chained: each layer's input is the running residual;
    # independent: given inputs, the residual accumulates), against the oracle run as the same chain on the
    # host: every layer's ids and weights, and the final residual
    import dataclasses
    moe = gpu
    norm = mode in ("chained", "independent_norm")
    wl = dataclasses.replace(S.WORKLOADS[name], norm_eps=1e-5 if norm else 0.0, centred=True, tokens=1)
    L, H, k = 4, wl.hidden, wl.top_k
    _say(f"stack with carried router {name} {mode} L={L}")
    layers = [S.make_layer(wl, layer=200 + l, device="cpu") for l in range(L)]
    dev = [to_device(w) for w in layers]
    cfg = moe.config_for(wl)
    ocfg = oracle_cfg(wl)
    ids = torch.empty((L, 1, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((L, 1, k), device="cuda")
    h0 = S.make_x(wl, 1, layer=199)
    if mode == "chained":
        resid = h0.cuda().clone()
        xs = [resid] * L
    else:
        resid = torch.zeros((1, H), device="cuda")
        xs = [S.make_x(wl, 1, layer=300 + l).cuda() for l in range(L)]
    moe.Stack(cfg, dev, xs, resid, ids, wts).step()
    torch.cuda.synchronize()
    # the oracle chain, each layer on the f32 input the GPU layer saw (f32 residual between layers)
    h = h0.numpy().astype(np.float32) if mode == "chained" else np.zeros((1, H), np.float32)
    tot = np.zeros((1, H))
    for l in range(L):
        wnp = S.to_numpy(layers[l])
        if mode == "chained":
            out, rid, rw = O.layer(ocfg, wnp, h, resid=h)
            tot = out
            h = out.astype(np.float32)
        else:
            out, rid, rw = O.layer(ocfg, wnp, xs[l].cpu().numpy())
            tot = tot + out
        gi = ids[l].cpu().numpy()
        assert np.array_equal(gi, rid), f"layer {l}: ids {gi} vs oracle {rid}"
        assert np.allclose(wts[l].cpu().numpy(), rw, rtol=2e-6, atol=1e-7), f"layer {l} weights"
    got = resid.cpu().numpy().astype(np.float64)
    base = h0.numpy() if mode == "chained" else 0.0
    _ok(row_rel_err(got - base, tot - base).max(), f"stack {name} {mode} final residual", guard=1e-5)


@pytest.mark.parametrize("name,T", [("flint", 1), ("flint8", 8), ("prefill", 512)])
def test_layer_swiglu_clamp(gpu, name, T):
    # SwiGLU clamp (ling_moe_ssd.js page: min(silu(g), L) * clamp(u, -L, L)),
    # distinct limits for the routed and the shared experts, at magnitudes where
    # both clamps are active (g, u ~ N(0, 4.5^2) for these weights)
    import dataclasses
    wl = dataclasses.replace(S.WORKLOADS[name], swiglu_limit=3.0, swiglu_limit_shared=2.0)
    _say(f"layer {name} T={T} with SwiGLU clamps 3.0 / 2.0")
    w, x = _layer(wl, seed=13)
    wnp = S.to_numpy(w)
    err, ties = run_layer_parity(wl, to_device(w), x.cuda(), None, wnp=wnp)
    # the clamps change the layer's output (so the test exercises them)
    rows = [0, T - 1]
    ref_c = O.layer(oracle_cfg(wl), wnp, x.numpy()[rows])[0]
    ref_u = O.layer(oracle_cfg(dataclasses.replace(wl, swiglu_limit=0.0, swiglu_limit_shared=0.0)), wnp,
                    x.numpy()[rows])[0]
    assert row_rel_err(ref_c, ref_u).max() > 0.05
    _ok(err, f"clamp {name} T={T} near_ties={ties}")


@pytest.mark.parametrize("T", [600, 1100])
def test_layer_prefill_multi_chunk(gpu, T):
    # more tokens than one chunk: the chunks run one after another
    wl = S.Workload("chunks", 256, 16, 3, 64, 96, S.Q4_1, has_bias=True)
    _say("prefill chunks T", T)
    w, x = _layer(wl, seed=T, tokens=T)
    err, _ = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"prefill chunks T={T}")


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8, 9, 13, 40])
def test_layer_token_counts_ragged(gpu, T):
    wl = S.Workload("ragged", 96 * 2, 24, 3, 160, 96, S.Q4_1, has_bias=True)
    _say("ragged T", T)
    w, x = _layer(wl, seed=T, tokens=T)
    err, _ = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"ragged T={T}")


@pytest.mark.parametrize("T", [3, 20])
@pytest.mark.parametrize("H,F,SF", [(96, 96, 0), (96, 160, 96), (288, 32, 64), (2080, 224, 0)])
def test_layer_q4_0_unaligned_rows(gpu, H, F, SF, T):
    # odd block counts give Q4_0 rows at 2-byte alignment (T=3 decode, T=20 grouped)
    wl = S.Workload("q40odd", H, 16, 3, F, SF, S.Q4_0, has_bias=True)
    _say("q4_0 odd rows", H, F, SF, "T", T)
    w, x = _layer(wl, seed=H + F, tokens=T)
    err, _ = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"q4_0 odd rows H={H} F={F} SF={SF} T={T}")


@pytest.mark.parametrize("qt", [S.Q4_1, S.Q4_0])
@pytest.mark.parametrize("H", [512, 1024, 1536, 2048])
def test_grouped_gateup_row_streaming_shapes(gpu, H, qt):
    # the grouped gate||up's row-streaming form: rows of 16, 32, 48 and 64 blocks
    # (one compile-time K split each), Q4_1 and Q4_0, routed tiles with 1..3
    # tiles per expert and a shared expert, a ragged token count, the SwiGLU
    # clamp active on both
    import dataclasses
    wl = S.Workload("rowstream", H, 12, 3, 160, 96, qt, has_bias=True)
    wl = dataclasses.replace(wl, swiglu_limit=3.0, swiglu_limit_shared=2.0)
    T = 37
    _say("grouped gate||up row-streaming", "H", H, "qtype", qt, "T", T)
    w, x = _layer(wl, seed=H + qt, tokens=T)
    err, ties = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"row-streaming H={H} q={qt} near_ties={ties}")


@pytest.mark.parametrize("qt", [S.Q4_1, S.Q4_0])
@pytest.mark.parametrize("F,SF", [(512, 0), (1536, 512), (2048, 1024)])
def test_grouped_down_row_streaming_shapes(gpu, F, SF, qt):
    # the grouped down's row-streaming form: routed rows of 16, 48 or 64 blocks
    # and shared rows of 16 or 32 (a launch each), Q4_1 and Q4_0, a ragged
    # token count; the gate||up runs its row-streaming form too (H = 512)
    wl = S.Workload("rowdown", 512, 10, 3, F, SF, qt, has_bias=True)
    T = 29
    _say("grouped down row-streaming", "F", F, "SF", SF, "qtype", qt, "T", T)
    w, x = _layer(wl, seed=F + SF + qt, tokens=T)
    err, ties = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"down row-streaming F={F} SF={SF} q={qt} near_ties={ties}")


@pytest.mark.parametrize("T", [100, 600])
def test_row_streaming_many_tiles_and_chunks(gpu, T):
    # the row-streaming grouped kernels with every token on two experts (a
    # selection bias forces them): 7 to 32 16-token tiles per expert, and
    # with T = 600 two chunks of the grouped path one after another
    wl = S.Workload("rowtiles", 512, 16, 2, 512, 512, S.Q4_1, has_bias=True)
    _say("row-streaming many tiles per expert, T", T)
    w, x = _layer(wl, seed=31 + T, tokens=T)
    w["bias"] = torch.zeros(16)
    w["bias"][[3, 11]] = 10.0
    err, ties = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"row-streaming many tiles T={T} near_ties={ties}")


@pytest.mark.parametrize("name,T", [("lfm25_q8", 1), ("lfm25_q8", 3), ("lfm25_q8", 520)])
def test_layer_q8_0(gpu, name, T):
    # Q8_0 experts (f16 d, 32 signed bytes; the lfm2_moe_ssd.js page's int8 expert plane), decode and grouped
    wl = S.WORKLOADS[name]
    _say(f"layer {name} Q8_0 T={T}")
    w, x = _layer(wl, seed=23, tokens=T)
    err, ties = run_layer_parity(wl, to_device(w), x.cuda(), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"q8_0 {name} T={T} near_ties={ties}")


@pytest.mark.parametrize("H,F,SF,T", [(96, 96, 64, 3), (96, 96, 64, 20), (2080, 160, 224, 1), (2080, 160, 224, 9)])
def test_layer_q8_0_odd_rows_and_shared(gpu, H, F, SF, T):
    # odd block counts give Q8_0 rows at 2-byte alignment; a shared expert too (T <= 8 decode, else grouped)
    wl = S.Workload("q80odd", H, 16, 3, F, SF, S.Q8_0, has_bias=True, scale_lo=0.0001, scale_hi=0.0004)
    _say("q8_0 odd rows", H, F, SF, "T", T)
    w, x = _layer(wl, seed=H + F + T, tokens=T)
    err, _ = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"q8_0 odd rows H={H} F={F} SF={SF} T={T}")


def test_layer_single_expert_and_k_equals_E(gpu):
    for E, k in ((1, 1), (6, 6)):
        wl = S.Workload("kE", 128, E, k, 64, 32, S.Q4_1)
        _say("k=E", E)
        w, x = _layer(wl, seed=E, tokens=4)
        err, _ = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
        _ok(err, f"k=E={E}")


def test_layer_all_tokens_on_one_expert(gpu):
    wl = S.Workload("one", 256, 32, 2, 64, 0, S.Q4_1, has_bias=True)
    _say("all tokens on one expert")
    w, x = _layer(wl, seed=9, tokens=8)
    w["bias"] = torch.zeros(32)
    w["bias"][[5, 17]] = 10.0  # bias forces experts 5 and 17 for every token
    wd = to_device(w)
    err, _ = run_layer_parity(wl, wd, x.cuda(), wnp=S.to_numpy(w))
    _ok(err, "all tokens on experts 5 and 17")


def test_layer_large_shape(gpu):
    # the ABI maxima for H and E with every group kept by a limit
    wl = S.Workload("big", 8192, 512, 32, 64, 128, S.Q4_1, n_groups=64, groups_used=8, weights_scale=1.5,
                    has_bias=True)
    _say("large H=8192 E=512 k=32")
    w, x = _layer(wl, seed=1, tokens=2)
    err, _ = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, "large H=8192 E=512 k=32")


def test_expert_ffn_zero_offsets_give_exact_zero(gpu):
    # Q4_0 blocks with every nibble 8 contribute exactly zero, bitwise on the GPU too
    moe = gpu
    wl = S.Workload("zero", 256, 8, 2, 64, 64, S.Q4_0)
    _say("q4_0 midpoint nibbles")
    w, x = _layer(wl, seed=2, tokens=3)
    for n in ("gate_exps", "up_exps", "down_exps", "gate_sh", "up_sh", "down_sh"):
        w[n].view(-1, 18)[:, 2:] = 0x88
    wd, xd = to_device(w), x.cuda()
    resid = torch.randn(3, 256, device="cuda")
    out = resid.clone()
    moe.layer_step(moe.config_for(wl), wd, xd, out)
    torch.cuda.synchronize()
    assert torch.equal(out, resid)


def test_determinism_and_token_independence(gpu):
    moe = gpu
    wl = S.WORKLOADS["flint8"]
    _say("determinism flint8")
    w, x = _layer(wl, seed=4)
    wd, xd = to_device(w), x.cuda()
    cfg = moe.config_for(wl)
    outs = []
    for _ in range(2):
        o = torch.zeros_like(xd)
        moe.layer_step(cfg, wd, xd, o)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    for t in range(xd.shape[0]):
        o1 = torch.zeros_like(xd[t:t + 1])
        moe.layer_step(cfg, wd, xd[t:t + 1].contiguous(), o1)
        torch.cuda.synchronize()
        err = row_rel_err(o1.cpu().numpy(), outs[0][t:t + 1].cpu().numpy())
        assert err.max() <= 1e-6


@pytest.mark.parametrize("name,T", [("ling", 1), ("flint8", 8), ("flint8", 5)])
def test_split_calls_equal_layer_step(gpu, name, T):
    # one token: routing inside the gate||up kernel vs the select kernel; several
    # tokens: the decode prelude routing and running the shared expert, vs
    # the select kernel then the prelude's shared half alone
    moe = gpu
    wl = S.WORKLOADS[name]
    _say("router_topk + expert_ffn_q4 == layer_step", name, f"T={T}")
    w, x = _layer(wl, seed=5, tokens=T)
    wd, xd = to_device(w), x.cuda()
    cfg = moe.config_for(wl)
    a = torch.zeros_like(xd)
    ids = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, wl.top_k), device="cuda")
    moe.layer_step(cfg, wd, xd, a, ids, wts)
    ids2, wts2 = moe.router_topk(cfg, wd, xd)
    b = torch.zeros_like(xd)
    moe.expert_ffn_q4(cfg, wd, xd, ids2, wts2, b)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(wts, wts2) and torch.equal(a, b)


# ------------------------------------------------- wide input distributions --

WIDE_CASES = [(qt, T) for qt in (S.Q4_0, S.Q4_1, S.Q8_0) for T in (1, 5, 40)]


@pytest.mark.parametrize("qt,T", WIDE_CASES)
def test_layer_wide_block_scales_and_outliers(gpu, qt, T):
    # block scales d of either sign, 5% of them f16 subnormals, Q4_1 offsets m of either sign, and 2% of the
    # inputs replaced by +-30: decode (T = 1, 5) and grouped (T = 40) paths, with a shared expert
    wl = S.Workload("wide", 512, 16, 3, 160, 96, qt, has_bias=True, signed_scales=True, subnormal_frac=0.05,
                    x_outlier_frac=0.02, x_outlier=30.0,
                    scale_lo=0.0001 if qt == S.Q8_0 else 0.001, scale_hi=0.0004 if qt == S.Q8_0 else 0.02)
    _say("wide scales and outliers", "qtype", qt, "T", T)
    w, x = _layer(wl, seed=41 + qt, tokens=T)
    err, ties = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"wide qtype={qt} T={T} near_ties={ties}")


@pytest.mark.parametrize("scale", [1e-4, 1e3])
@pytest.mark.parametrize("T", [1, 40])
def test_layer_input_scale(gpu, scale, T):
    # FFN inputs far from unit scale: 1e-4 puts the act values of the grouped path's f16 MFMA operands in
    # the f16 subnormal range unless they are rescaled; 1e3 tests the upper side
    wl = S.Workload("xscale", 512, 16, 3, 160, 96, S.Q4_1, has_bias=True, x_scale=scale)
    _say("input scale", scale, "T", T)
    w, x = _layer(wl, seed=43, tokens=T)
    err, ties = run_layer_parity(wl, to_device(w), x.cuda(), wnp=S.to_numpy(w))
    _ok(err, f"input scale {scale:g} T={T} near_ties={ties}")


@pytest.mark.parametrize("T", [8, 9, 40])
def test_expert_ffn_repeated_ids(gpu, T):
    # caller-given ids in which a token lists one expert twice (or three times): the decode path (T = 8)
    # and the grouped path (T = 9, 40) must both add every pick with its own weight, as the oracle does
    moe = gpu
    wl = S.Workload("rep", 256, 12, 4, 96, 64, S.Q4_1)
    _say("repeated ids", "T", T)
    w, x = _layer(wl, seed=47, tokens=T)
    g = torch.Generator().manual_seed(T)
    ids = torch.randint(0, 12, (T, 4), generator=g, dtype=torch.int32)
    ids[0, 1] = ids[0, 0]
    ids[T - 1, 3] = ids[T - 1, 2] = ids[T - 1, 0]
    ids[T // 2, 2] = ids[T // 2, 1]
    wts = torch.rand((T, 4), generator=g) + 0.1
    wd = to_device(w)
    out = torch.zeros((T, 256), device="cuda")
    moe.expert_ffn_q4(moe.config_for(wl), wd, x.cuda(), ids.cuda(), wts.cuda(), out)
    torch.cuda.synchronize()
    wnp = S.to_numpy(w)
    ref = np.stack([oracle_given_routing(wl, wnp, x[t].numpy(), ids[t].numpy(), wts[t].numpy())
                    for t in range(T)])
    _ok(row_rel_err(out.cpu().numpy(), ref).max(), f"repeated ids T={T}")


def test_grouped_sort_with_repeated_ids_bit_exact(gpu):
    # the grouped path's sort of caller-given ids with repeats, read back from the workspace
    from moe_testlib import check_sort
    moe = gpu
    wl = S.Workload("rep", 256, 12, 4, 96, 64, S.Q4_1)
    T = 70
    _say("sort with repeated ids T", T)
    w, x = _layer(wl, seed=53, tokens=T)
    g = torch.Generator().manual_seed(5)
    ids = torch.randint(0, 12, (T, 4), generator=g, dtype=torch.int32)
    ids[::3, 1] = ids[::3, 0]
    ids[::7, 3] = ids[::7, 0]
    cfg = moe.config_for(wl)
    ws = moe.alloc_workspace(cfg, T)
    out = torch.zeros((T, 256), device="cuda")
    moe.expert_ffn_q4(cfg, to_device(w), x.cuda(), ids.cuda(), torch.ones((T, 4), device="cuda"), out,
                      workspace=ws)
    torch.cuda.synchronize()
    check_sort(cfg, ws, ids.numpy(), T)


@pytest.mark.parametrize("T,E,k", [(512, 256, 6), (300, 64, 8), (45, 8, 1), (129, 40, 12)])
def test_grouped_sort_bit_exact(gpu, T, E, k):
    # the grouped path's sort of caller-given ids with k distinct experts per token (one thread per token holds
    # its ids for k <= 8; k = 12 takes the per-pair form), read back from the workspace
    from moe_testlib import check_sort
    moe = gpu
    wl = S.Workload("srt", 256, E, k, 96, 0, S.Q4_1)
    _say("sort T", T, "E", E, "k", k)
    w, x = _layer(wl, seed=61 + T, tokens=T)
    g = torch.Generator().manual_seed(T + E + k)
    ids = torch.argsort(torch.rand((T, E), generator=g), dim=1)[:, :k].to(torch.int32).contiguous()
    cfg = moe.config_for(wl)
    ws = moe.alloc_workspace(cfg, T)
    out = torch.zeros((T, 256), device="cuda")
    moe.expert_ffn_q4(cfg, to_device(w), x.cuda(), ids.cuda(), torch.ones((T, k), device="cuda"), out,
                      workspace=ws)
    torch.cuda.synchronize()
    check_sort(cfg, ws, ids.numpy(), T)


# ------------------------------------------------ one-token routing, exact ties --

TIE_CASES = {
    "flint": dict(E=256, k=6, G=1, Gu=1, bias=False),
    "lfm25": dict(E=64, k=4, G=1, Gu=1, bias=True),
    "ling": dict(E=512, k=8, G=8, Gu=4, bias=True),
    "odd_E": dict(E=100, k=5, G=1, Gu=1, bias=False),
    "k32": dict(E=64, k=32, G=1, Gu=1, bias=False),
    "groups_small": dict(E=128, k=6, G=16, Gu=5, bias=True),  # groups of 8: the block router
    "e64_groups": dict(E=64, k=5, G=4, Gu=2, bias=True),  # one wave holds every expert, groups of 16
}


@pytest.mark.parametrize("name", sorted(TIE_CASES))
def test_one_token_routing_exact_ties(gpu, name):
    # identical router rows give bitwise equal logits, so the lowest expert index (and, with groups, the lowest
    # group index) decides: the GPU's picks must equal the oracle's exactly (a near-tie certificate would accept
    # any order here, so the ids are compared strictly), and so must the layer output
    moe = gpu
    c = TIE_CASES[name]
    E, k = c["E"], c["k"]
    wl = S.Workload("ties", 256, E, k, 64, 32, S.Q4_1, n_groups=c["G"], groups_used=c["Gu"],
                    weights_scale=2.5 if c["G"] > 1 else 1.0, has_bias=c["bias"])
    _say("one-token routing with exact ties", name)
    w, x = _layer(wl, seed=71 + E, tokens=1)
    g = torch.Generator().manual_seed(E + k)
    tied = torch.randperm(E, generator=g)[: 2 * k + 3]
    v = x[0] / x[0].norm() * 0.25
    w["router_w"][tied] = v  # every tied expert scores above the rest, all equally
    if c["bias"]:
        w["bias"][tied] = 0.0  # the tied experts also tie on the selection bias
    wd = to_device(w)
    cfg = moe.config_for(wl)
    out = torch.zeros((1, 256), device="cuda")
    ids = torch.empty((1, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((1, k), dtype=torch.float32, device="cuda")
    moe.layer_step(cfg, wd, x.cuda(), out, ids, wts)
    torch.cuda.synchronize()
    ref, ids_ref, w_ref = O.layer(oracle_cfg(wl), S.to_numpy(w), x.numpy())
    assert np.array_equal(ids.cpu().numpy(), ids_ref), (ids.cpu().numpy(), ids_ref)
    assert np.allclose(wts.cpu().numpy(), w_ref, rtol=2e-6, atol=1e-7)
    _ok(row_rel_err(out.cpu().numpy(), ref).max(), f"ties {name}")
