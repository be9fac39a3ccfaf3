"""Pins of the double-precision oracle to facts outside itself: closed forms,
exact values of hand-built blocks, brute force on tiny inputs, independent
library routines.  CPU only.

Passages (the diskformer engine pages):
  flint_moe_ssd.js page: Q4_1 block layout (file header, Q41DOT comment).
  lfm2_moe_ssd.js page:  router comment + TOPK_SIG_BODY (sigmoid, selection
                         bias, top-k with lowest-index ties, weights over the
                         clamped sum times the scale); moeAccumB.
  ling_moe_ssd.js page:  routeLing (group top-2 sums, kept groups, scale 2.5),
                         swiglu, moeAccum (shared expert added with weight 1).
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_block_fixture(name):
    byts, vals = None, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("bytes:"):
                byts = np.array([int(t, 16) for t in line.split()[1:]], np.uint8)
            elif line.startswith("values:"):
                vals = np.array([float(t) for t in line.split()[1:]])
    return byts, vals


# ----------------------------------------------------------------- f16 ----

def test_f16_golden_patterns():
    with open(os.path.join(GOLDEN, "f16_patterns.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for h, v in rows:
        got = O.f16(int(h, 16))
        assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v)), h


def test_f16_all_finite_patterns_match_numpy():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    L = O.lib()
    got = np.array([L.mo_f16(int(p)) for p in pats])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.all(np.isinf(got[np.isinf(ref)])) and np.all(np.isnan(got[np.isnan(ref)]))


# ----------------------------------------------------------- dequant ----

def test_q4_1_handbuilt_block():
    b, v = _read_block_fixture("q4_1_block.txt")
    assert b.size == 20 and v.size == 32
    assert np.array_equal(O.dequant_row(O.Q4_1, b), v)


def test_q4_0_handbuilt_block():
    b, v = _read_block_fixture("q4_0_block.txt")
    assert b.size == 18 and v.size == 32
    assert np.array_equal(O.dequant_row(O.Q4_0, b), v)


def test_q8_0_handbuilt_block():
    b, v = _read_block_fixture("q8_0_block.txt")
    assert b.size == 34 and v.size == 32
    assert np.array_equal(O.dequant_row(O.Q8_0, b), v)


def test_q8_0_matches_numpy_views():
    # Q8_0 through numpy's own f16 and int8 views of random blocks (incl. subnormal and negative scales)
    rng = np.random.default_rng(5)
    nb = 64
    row = rng.integers(0, 256, size=(nb, 34), dtype=np.uint8)
    row[:, 0:2] = rng.uniform(-2.0, 2.0, size=nb).astype(np.float16)[:, None].view(np.uint8)
    row[0, 0:2] = np.array([np.float16(6e-7)]).view(np.uint8)  # a subnormal scale
    d = row[:, 0:2].copy().view(np.float16).astype(np.float64)
    q = row[:, 2:].copy().view(np.int8).astype(np.float64)
    assert np.array_equal(O.dequant_row(O.Q8_0, row.reshape(-1)), (d * q).reshape(-1))
    x = rng.integers(-4, 5, size=32 * nb).astype(np.float64)
    assert O.row_dot(O.Q8_0, row.reshape(-1), x) == pytest.approx(float(((d * q).reshape(-1) * x).sum()), rel=1e-15)


@pytest.mark.parametrize("nib,expect", [(8, 0.0), (0, -8.0), (15, 7.0)])
def test_q4_0_constant_nibbles(nib, expect):
    d = np.float16(0.375)
    blk = np.zeros(18, np.uint8)
    blk[0:2] = np.array([d]).view(np.uint8)
    blk[2:] = nib | (nib << 4)
    assert np.array_equal(O.dequant_row(O.Q4_0, blk), np.full(32, expect * 0.375))


def test_q4_1_scale_and_offset_are_distinct_fields():
    # d = 2, m = -3: element value 2q - 3; swapping d and m would give -3q + 2.
    blk = np.zeros(20, np.uint8)
    blk[0:2] = np.array([np.float16(2.0)]).view(np.uint8)
    blk[2:4] = np.array([np.float16(-3.0)]).view(np.uint8)
    blk[4:] = np.arange(16, dtype=np.uint8) | (np.uint8(1) << 4)
    v = O.dequant_row(O.Q4_1, blk)
    assert np.array_equal(v[:16], 2.0 * np.arange(16) - 3.0)
    assert np.array_equal(v[16:], np.full(16, -1.0))


def test_row_dot_block_identity_exact():
    # d*sum(q x) + m*sum(x) == sum((d q + m) x), exact for small integers x.
    rng = np.random.default_rng(1)
    nb = 5
    row = rng.integers(0, 256, size=(nb, 20), dtype=np.uint8)
    for b in range(nb):
        row[b, 0:2] = np.array([np.float16(rng.integers(1, 8) / 4)]).view(np.uint8)
        row[b, 2:4] = np.array([np.float16(-rng.integers(0, 8) / 8)]).view(np.uint8)
    x = rng.integers(-4, 5, size=32 * nb).astype(np.float64)
    q = np.zeros(32 * nb)
    for b in range(nb):
        qs = row[b, 4:]
        q[32 * b:32 * b + 16] = qs & 15
        q[32 * b + 16:32 * b + 32] = qs >> 4
    d = np.repeat([float(row[b, 0:2].view(np.float16)[0]) for b in range(nb)], 32)
    m = np.repeat([float(row[b, 2:4].view(np.float16)[0]) for b in range(nb)], 32)
    expect = sum(d[32 * b] * np.dot(q[32 * b:32 * b + 32], x[32 * b:32 * b + 32])
                 + m[32 * b] * x[32 * b:32 * b + 32].sum() for b in range(nb))
    assert O.row_dot(O.Q4_1, row, x) == expect
    assert np.array_equal(O.dequant_row(O.Q4_1, row), d * q + m)


# ------------------------------------------------------------ router ----

def test_router_logits_integer_exact():
    rng = np.random.default_rng(2)
    E, H = 13, 96
    W = rng.integers(-50, 51, size=(E, H)).astype(np.float32)
    x = rng.integers(-20, 21, size=H).astype(np.float32)
    ref = (W.astype(np.int64) @ x.astype(np.int64)).astype(np.float64)
    assert np.array_equal(O.router_logits(W, x), ref)


def test_router_logits_random_vs_longdouble():
    rng = np.random.default_rng(3)
    E, H = 16, 2048
    W = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    x = rng.standard_normal(H).astype(np.float32)
    ref = (W.astype(np.longdouble) * x.astype(np.longdouble)).sum(axis=1)
    assert np.allclose(O.router_logits(W, x), ref.astype(np.float64), rtol=0, atol=1e-12)


def test_sigmoid_closed_forms():
    assert O.sigmoid(0.0) == 0.5
    for v in (0.3, 1.7, 5.0, 20.0):
        assert abs(O.sigmoid(v) + O.sigmoid(-v) - 1.0) < 1e-15
        assert abs(O.sigmoid(v) - 1.0 / (1.0 + math.exp(-v))) < 1e-16
    assert O.sigmoid(-800.0) == 0.0


# -------------------------------------------------------------- top-k ----

def _bruteforce_topk(s, k, allowed=None):
    """The unique k-subset whose every member beats every non-member on (score, -index),
    listed in pick order (descending score, lowest index first on ties)."""
    E = len(s)
    cand = [e for e in range(E) if allowed is None or allowed[e]]
    key = lambda e: (float(s[e]), -e)
    winners = []
    for sub in itertools.combinations(cand, k):
        rest = [e for e in cand if e not in sub]
        if all(key(a) > key(b) for a in sub for b in rest):
            winners.append(sub)
    assert len(winners) == 1
    return sorted(winners[0], key=lambda e: (-float(s[e]), e))


@pytest.mark.parametrize("seed", range(12))
def test_topk_bruteforce_small(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 11))
    k = int(rng.integers(1, E + 1))
    # few distinct values -> many exact ties
    s = rng.integers(0, 4, size=E).astype(np.float32) / 4
    assert list(O.topk(s, k)) == _bruteforce_topk(s, k)


def test_topk_ties_go_to_lowest_index():
    s = np.full(10, 0.25, np.float32)
    assert list(O.topk(s, 4)) == [0, 1, 2, 3]
    s[7] = 0.5
    assert list(O.topk(s, 3)) == [7, 0, 1]


def _gscores32(s, G):
    P = len(s) // G
    out = []
    for g in range(G):
        v = np.sort(s[g * P:(g + 1) * P])[::-1]
        out.append(np.float32(v[0]) + np.float32(v[1]))
    return np.array(out, np.float32)


@pytest.mark.parametrize("seed", range(4))
def test_groups_bruteforce_ling_shape(seed):
    rng = np.random.default_rng(100 + seed)
    E, G, Gu, k = 512, 8, 4, 8
    s = (rng.random(E) + rng.standard_normal(E) * 0.1).astype(np.float32)
    if seed == 3:  # force equal group scores: lower group index must win
        s[64:128] = s[0:64]
        s[320:384] = s[0:64]
    gs = _gscores32(s, G)
    keep, gs_o = O.group_keep(s, G, Gu)
    assert np.array_equal(gs_o, gs)
    key = lambda g: (float(gs[g]), -g)
    sets = [sub for sub in itertools.combinations(range(G), Gu)
            if all(key(a) > key(b) for a in sub for b in range(G) if b not in sub)]
    assert len(sets) == 1
    assert set(np.nonzero(keep)[0]) == set(sets[0])
    allowed = np.repeat(keep, E // G)
    ids = O.topk(s, k, allowed)
    # top-k within the kept groups, checked against a sort
    cand = sorted([e for e in range(E) if allowed[e]], key=lambda e: (-float(s[e]), e))
    assert list(ids) == cand[:k]


def test_group_top2_sum_not_max():
    # group 0 holds the best single expert but a poor second; group 1 two good ones.
    E, G = 8, 4
    s = np.array([0.99, 0.01, 0.6, 0.6, 0.3, 0.3, 0.2, 0.2], np.float32)
    keep, gs = O.group_keep(s, G, 1)
    assert list(keep) == [0, 1, 0, 0]
    cfg = O.make_cfg(64, E, 2, 32, n_groups=G, groups_used=1)
    logits = np.log(s / (1 - s)).astype(np.float32)  # sigmoid(logit) == s (to f32)
    ids, _ = O.route(cfg, logits)
    assert sorted(ids) == [2, 3]


def test_group_duplicate_top_value_counts_twice():
    s = np.array([0.5, 0.5, 0.1, 0.1, 0.8, 0.1], np.float32)
    keep, gs = O.group_keep(s, 3, 1)
    assert gs[0] == np.float32(1.0) and list(keep) == [1, 0, 0]


def test_groups_all_used_reduces_to_plain_topk():
    rng = np.random.default_rng(7)
    E, k = 64, 6
    l = rng.standard_normal(E).astype(np.float32)
    a = O.make_cfg(64, E, k, 32, n_groups=8, groups_used=8)
    b = O.make_cfg(64, E, k, 32)
    assert np.array_equal(O.route(a, l)[0], O.route(b, l)[0])


def test_bias_selects_but_does_not_weight():
    E, k = 6, 2
    l = np.array([2.0, 1.0, 0.0, -1.0, -2.0, -3.0], np.float32)
    bias = np.array([0, 0, 0, 0, 5, 5], np.float32)
    cfg = O.make_cfg(64, E, k, 32)
    ids, w = O.route(cfg, l, bias=bias)
    assert list(ids) == [4, 5]
    p = 1 / (1 + np.exp(-l.astype(np.float64)))
    assert np.allclose(w, p[[4, 5]] / p[[4, 5]].sum(), rtol=1e-15)


# ------------------------------------------------------------- weights ----

@pytest.mark.parametrize("scale", [1.0, 2.5])
def test_weights_sum_to_scale(scale):
    rng = np.random.default_rng(9)
    cfg = O.make_cfg(64, 256, 6, 32, weights_scale=scale)
    for _ in range(20):
        l = (rng.standard_normal(256) * 2).astype(np.float32)
        ids, w = O.route(cfg, l)
        assert abs(w.sum() - scale) < 1e-14
        assert len(set(ids)) == 6


def test_k1_weight_is_scale():
    cfg = O.make_cfg(64, 16, 1, 32, weights_scale=2.5)
    l = np.linspace(-1, 1, 16).astype(np.float32)
    ids, w = O.route(cfg, l)
    assert ids[0] == 15 and w[0] == 2.5


def test_weight_clamp_ling_case():
    # all logits -30: the picked sigmoids sum to ~7.5e-13 < 2^-14, so w_j = p_j * 2.5 * 2^14
    cfg = O.make_cfg(2560, 512, 8, 768, n_groups=8, groups_used=4, weights_scale=2.5)
    l = np.full(512, -30.0, np.float32)
    ids, w = O.route(cfg, l)
    assert list(ids) == list(range(8))  # all tie: groups 0..3 kept, lowest indices
    p = 1.0 / (1.0 + math.exp(30.0))
    assert np.all(w == p / 2.0 ** -14 * 2.5)


@pytest.mark.parametrize("side", [-1, 1])
def test_weight_clamp_boundary(side):
    target = 2.0 ** -14 * (1 + side * 1e-3)  # S just below / above the clamp
    k = 2
    p = target / k
    l = math.log(p / (1 - p))
    cfg = O.make_cfg(64, 4, k, 32)
    logits = np.array([l, l, -60, -60], np.float32)
    ids, w = O.route(cfg, logits, logit64=np.array([l, l, -60, -60]))
    S = 2 * (1 / (1 + math.exp(-l)))
    if side < 0:
        assert np.allclose(w, (1 / (1 + math.exp(-l))) / 2.0 ** -14, rtol=1e-15) and w.sum() < 1
    else:
        assert abs(w.sum() - 1.0) < 1e-14 and S > 2.0 ** -14


# -------------------------------------------------------------- SwiGLU ----

def test_swiglu_closed_forms():
    assert O.swiglu(0.0, 5.0) == 0.0
    for g in (0.1, 1.0, 3.3, 12.0):
        # silu(g) - silu(-g) == g
        assert abs(O.swiglu(g, 1.0) - O.swiglu(-g, 1.0) - g) < 1e-14
        assert O.swiglu(g, 2.0) == 2.0 * O.swiglu(g, 1.0)


def _silu(g):
    return g / (1.0 + math.exp(-g))


def _const_q4_1_rows(n_rows, n_blocks, m):
    """Q4_1 rows whose every weight is m: d = 0 (so d*q = 0 for any nibble) and
    offset m, f16-encoded by numpy.  m must be exact in f16."""
    assert float(np.float16(m)) == m
    blk = np.zeros(20, np.uint8)
    blk[2:4] = np.frombuffer(np.float16(m).tobytes(), np.uint8)
    blk[4:] = 0x5A  # arbitrary nibbles: multiplied by d = 0
    return np.tile(blk, n_rows * n_blocks).reshape(n_rows, n_blocks * 20)


@pytest.mark.parametrize("g,u,L", [
    (10.0, -7.0, 5.0),    # silu(g) capped at L, u clamped at -L
    (-3.0, 2.0, 0.1),     # negative silu(g) is not raised to -L (the cap is one-sided), u clamped
    (0.25, 1.0, 0.2),     # silu(0.25) < L stays; the clamp is on silu(g), not on g before silu
    (10.0, -7.0, 0.0),    # L = 0: no clamp
    (1.5, 0.75, 100.0),   # inactive clamp
])
def test_swiglu_clamp_closed_forms(g, u, L):
    """ling_moe_ssd.js page, swiglu kernel and the FFN line of its file header:
    act = min(silu(g), L) * clamp(u, -L, L) when L > 0.  Checked on a whole
    expert whose rows are constant: with x = 1 and H = F = 32, every gate row
    gives g = 32 m_g, every up row u = 32 m_u, and y_h = 32 m_d act."""
    H = F = 32
    gate = _const_q4_1_rows(F, 1, g / 32)
    up = _const_q4_1_rows(F, 1, u / 32)
    down = _const_q4_1_rows(H, 1, 0.0625)
    sg = _silu(g)
    if L > 0:
        act = min(sg, L) * min(max(u, -L), L)
    else:
        act = sg * u
    y = O.expert_ffn(O.Q4_1, gate, up, down, H, F, np.ones(H), limit=L)
    assert np.allclose(y, 2.0 * act, rtol=1e-13, atol=0)
    assert O.swiglu(g, u, L) == pytest.approx(act, rel=1e-15)


def test_swiglu_clamp_routed_and_shared_limits_apply_to_their_experts():
    """The routed experts take the routed limit and the shared expert its own
    (ling_moe_ssd.js page: clampExp for the experts, clampShexp for the shared
    expert).  One pick with weight p/p = 1; constant-row experts as above."""
    H = F = SF = 32
    E = 2
    ge = np.stack([_const_q4_1_rows(F, 1, 10.0 / 32), _const_q4_1_rows(F, 1, 1.0 / 32)])
    ue = np.stack([_const_q4_1_rows(F, 1, -7.0 / 32), _const_q4_1_rows(F, 1, 1.0 / 32)])
    de = np.stack([_const_q4_1_rows(H, 1, 0.0625), _const_q4_1_rows(H, 1, 0.0625)])
    w = {"router_w": None, "bias": None, "gate_exps": ge, "up_exps": ue, "down_exps": de,
         "gate_sh": _const_q4_1_rows(SF, 1, -3.0 / 32), "up_sh": _const_q4_1_rows(SF, 1, 2.0 / 32),
         "down_sh": _const_q4_1_rows(H, 1, 0.0625)}
    cfg = O.make_cfg(H, E, 1, F, SF, O.Q4_1, swiglu_limit=5.0, swiglu_limit_shared=0.1)
    logits = np.array([[3.0, -3.0]], np.float32)  # picks expert 0
    out, ids, ww = O.layer(cfg, w, np.ones((1, H), np.float32), logits_in=logits)
    assert ids[0, 0] == 0 and ww[0, 0] == 1.0
    routed = 2.0 * (5.0 * -5.0)                       # min(silu(10), 5) * clamp(-7)
    shared = 2.0 * (_silu(-3.0) * 0.1)                # silu(-3) < 0.1 stays; clamp(2) = 0.1
    assert np.allclose(out[0], routed + shared, rtol=1e-13, atol=0)
    # the limits swapped give a clearly different answer
    swapped = 2.0 * (0.1 * -0.1) + 2.0 * (_silu(-3.0) * 2.0)
    assert abs((routed + shared) - swapped) > 1.0


def test_dense_layer_is_the_ffn_alone():
    """A dense SwiGLU FFN layer (the pages' leading layers: no router) is
    E = k = 0 with the FFN in the shared tensors: out = resid + FFN(x).
    Constant-row FFN as above: g = 10, u = -7, y_h = 32 * 0.0625 * act."""
    H = SF = 32
    w = {"router_w": None, "bias": None, "gate_exps": None, "up_exps": None, "down_exps": None,
         "gate_sh": _const_q4_1_rows(SF, 1, 10.0 / 32), "up_sh": _const_q4_1_rows(SF, 1, -7.0 / 32),
         "down_sh": _const_q4_1_rows(H, 1, 0.0625)}
    cfg = O.make_cfg(H, 0, 0, 0, SF, O.Q4_1)
    resid = np.linspace(-1, 1, H, dtype=np.float32)[None, :]
    out, ids, ww = O.layer(cfg, w, np.ones((1, H), np.float32), resid=resid)
    assert ids.shape == (1, 0) and ww.shape == (1, 0)
    assert np.allclose(out[0], resid[0].astype(np.float64) + 2.0 * _silu(10.0) * -7.0, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------- RMSNorm ----

def test_rmsnorm_closed_forms():
    """Pre-FFN RMSNorm, x / sqrt(mean(x^2) + eps) * g (flint/lfm2 page file
    headers: rms_norm(x) * ffn_norm; ling page: the normalising kernels divide
    by sqrt(sum/n + eps) before the weight), rounded once to f32."""
    # x = (3, 4): mean(x^2) = 12.5
    got = O.rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 1.0]), 0.0)
    assert np.allclose(got, np.float32(np.array([3.0, 4.0]) / math.sqrt(12.5)), rtol=0, atol=0)
    # constant c with eps = c^2: s = 1 / (c * sqrt(2)); a sum in place of the mean, or eps outside the
    # square root, would give 1 / (c sqrt(H + 1)) or 1 / (c + c^2)
    c, H = 0.5, 64
    g = np.linspace(-2.0, 2.0, H).astype(np.float32)  # the weight is an f32 tensor
    got = O.rmsnorm(np.full(H, c), g, c * c)
    want = g.astype(np.float64) / math.sqrt(2.0)
    assert np.allclose(got, want, rtol=1.2e-7, atol=0)  # one f32 rounding
    # weight 1 and eps 0: every element of a constant vector becomes 1 (sign kept)
    assert np.array_equal(O.rmsnorm(np.full(32, -7.25), np.ones(32), 0.0), -np.ones(32, np.float32))


def test_rmsnorm_chained_dense_layer():
    """With a norm weight the layer input is the residual stream h and the FFN
    sees rms_norm(h) * w; the chained form passes h as both x and resid:
    out = h + FFN(rms_norm(h) * w).  h = 2 * 1, w = 1, eps = 0: rms_norm(h) = 1,
    and the constant-row FFN of test_dense_layer_is_the_ffn_alone gives
    2 silu(10) (-7) on top."""
    H = SF = 32
    w = {"router_w": None, "bias": None, "gate_exps": None, "up_exps": None, "down_exps": None,
         "gate_sh": _const_q4_1_rows(SF, 1, 10.0 / 32), "up_sh": _const_q4_1_rows(SF, 1, -7.0 / 32),
         "down_sh": _const_q4_1_rows(H, 1, 0.0625), "ffn_norm": np.ones(H, np.float32)}
    cfg = O.make_cfg(H, 0, 0, 0, SF, O.Q4_1, norm_eps=0.0)
    h = np.full((1, H), 2.0, np.float32)
    out, _, _ = O.layer(cfg, w, h, resid=h)
    assert np.allclose(out[0], 2.0 + 2.0 * _silu(10.0) * -7.0, rtol=1e-13, atol=0)
    # without the norm the same h feeds the FFN directly: g = 20, u = -14
    w2 = dict(w, ffn_norm=None)
    out2, _, _ = O.layer(cfg, w2, h, resid=h)
    assert np.allclose(out2[0], 2.0 + 2.0 * _silu(20.0) * -14.0, rtol=1e-13, atol=0)


# -------------------------------------------------------------- experts ----

def _const_blocks(n_rows, cols, d, m, qtype=O.Q4_1, nib=0):
    nb = cols // 32
    bs = O.block_bytes(qtype)
    b = np.zeros((n_rows, nb, bs), np.uint8)
    b[:, :, 0:2] = np.array([np.float16(d)]).view(np.uint8)
    if qtype == O.Q4_1:
        b[:, :, 2:4] = np.array([np.float16(m)]).view(np.uint8)
        b[:, :, 4:] = nib | (nib << 4)
    else:
        b[:, :, 2:] = nib | (nib << 4)
    return b.reshape(n_rows, nb * bs)


def test_expert_closed_form_offsets_only():
    # d = 0, m = c everywhere: g_f = c_g X, u_f = c_u X (X = sum x), y_h = c_d F silu(c_g X) c_u X
    H, F = 96, 64
    cg, cu, cd = 0.125, -0.25, 0.0625
    rng = np.random.default_rng(11)
    x = rng.standard_normal(H)
    X = x.sum()
    y = O.expert_ffn(O.Q4_1, _const_blocks(F, H, 0.0, cg), _const_blocks(F, H, 0.0, cu),
                     _const_blocks(H, F, 0.0, cd), H, F, x)
    sg = cg * X / (1 + math.exp(-cg * X))
    expect = cd * F * sg * cu * X
    assert np.allclose(y, expect, rtol=1e-13, atol=0)


def test_expert_q4_0_midpoint_nibbles_give_zero():
    H, F = 64, 32
    x = np.random.default_rng(12).standard_normal(H)
    z = lambda r, c: _const_blocks(r, c, 0.5, 0, O.Q4_0, nib=8)
    assert np.all(O.expert_ffn(O.Q4_0, z(F, H), z(F, H), z(H, F), H, F, x) == 0.0)


def _dense_numpy_ffn(qtype, gate, up, down, H, F, x):
    """Independent composition: dequantise whole matrices (pinned above) and use numpy matmul."""
    dq = lambda M, rows: np.stack([O.dequant_row(qtype, M[r]) for r in range(rows)])
    g = dq(gate, F) @ x
    u = dq(up, F) @ x
    a = g / (1 + np.exp(-g)) * u
    return dq(down, H) @ a


@pytest.mark.parametrize("qtype", [O.Q4_0, O.Q4_1])
def test_expert_ffn_vs_numpy_composition(qtype):
    import moe_synth as S
    H, F = 128, 64
    gate = S.expert_tensor(1, F, H, qtype, "cpu", 5).numpy()[0]
    up = S.expert_tensor(1, F, H, qtype, "cpu", 6).numpy()[0]
    down = S.expert_tensor(1, H, F, qtype, "cpu", 7).numpy()[0]
    x = np.random.default_rng(13).standard_normal(H)
    y = O.expert_ffn(qtype, gate, up, down, H, F, x)
    assert np.allclose(y, _dense_numpy_ffn(qtype, gate, up, down, H, F, x), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- layer ----

def _tiny_layer(qtype=O.Q4_1, E=8, H=128, F=64, SF=0, bias=False, seed=0, name="pin"):
    import moe_synth as S
    wl = S.Workload(name, H, E, 2, F, SF, qtype, has_bias=bias)
    return wl, S.to_numpy(S.make_layer(wl, seed))


@pytest.mark.parametrize("SF,bias,qtype", [(0, False, O.Q4_1), (64, True, O.Q4_1), (96, True, O.Q4_0)])
def test_layer_dense_bruteforce_equals_gather(SF, bias, qtype):
    wl, w = _tiny_layer(qtype, SF=SF, bias=bias)
    cfg = O.make_cfg(wl.hidden, wl.n_experts, wl.top_k, wl.expert_ff, SF, qtype)
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, wl.hidden)).astype(np.float32)
    resid = rng.standard_normal((3, wl.hidden)).astype(np.float32)
    out, ids, ww = O.layer(cfg, w, x, resid)
    H, F = wl.hidden, wl.expert_ff
    for t in range(3):
        dense_w = np.zeros(wl.n_experts)
        dense_w[ids[t]] = ww[t]
        acc = resid[t].astype(np.float64).copy()
        for e in range(wl.n_experts):  # every expert computed, scaled by a sparse weight vector
            acc += dense_w[e] * _dense_numpy_ffn(qtype, w["gate_exps"][e], w["up_exps"][e], w["down_exps"][e],
                                                 H, F, x[t].astype(np.float64))
        if SF:
            acc += _dense_numpy_ffn(qtype, w["gate_sh"], w["up_sh"], w["down_sh"], H, SF, x[t].astype(np.float64))
        assert np.allclose(out[t], acc, rtol=1e-12, atol=1e-13)


def test_layer_router_and_ids_match_independent_route():
    wl, w = _tiny_layer(bias=True)
    cfg = O.make_cfg(wl.hidden, wl.n_experts, wl.top_k, wl.expert_ff)
    x = np.random.default_rng(22).standard_normal((4, wl.hidden)).astype(np.float32)
    _, ids, ww = O.layer(cfg, w, x)
    for t in range(4):
        l64 = w["router_w"].astype(np.float64) @ x[t].astype(np.float64)
        p = 1 / (1 + np.exp(-l64))
        s = (p.astype(np.float32) + w["bias"]).astype(np.float32)
        order = sorted(range(wl.n_experts), key=lambda e: (-float(s[e]), e))[:wl.top_k]
        assert list(ids[t]) == order
        assert np.allclose(ww[t], p[order] / p[order].sum(), rtol=1e-13)


def test_layer_identical_experts():
    import moe_synth as S
    wl, w = _tiny_layer(SF=64, bias=False)
    for n in ("gate_exps", "up_exps", "down_exps"):
        w[n] = np.repeat(w[n][:1], wl.n_experts, axis=0)
    scale = 2.5
    cfg = O.make_cfg(wl.hidden, wl.n_experts, wl.top_k, wl.expert_ff, 64, weights_scale=scale)
    x = np.random.default_rng(23).standard_normal((2, wl.hidden)).astype(np.float32)
    out, _, _ = O.layer(cfg, w, x)
    for t in range(2):
        xd = x[t].astype(np.float64)
        ffn = O.expert_ffn(O.Q4_1, w["gate_exps"][0], w["up_exps"][0], w["down_exps"][0], wl.hidden, wl.expert_ff, xd)
        sh = O.expert_ffn(O.Q4_1, w["gate_sh"], w["up_sh"], w["down_sh"], wl.hidden, 64, xd)
        assert np.allclose(out[t], scale * ffn + sh, rtol=1e-12, atol=1e-14)


def test_layer_permutation_invariance():
    wl, w = _tiny_layer(bias=True, SF=64)
    cfg = O.make_cfg(wl.hidden, wl.n_experts, wl.top_k, wl.expert_ff, 64)
    x = np.random.default_rng(24).standard_normal((3, wl.hidden)).astype(np.float32)
    out, ids, ww = O.layer(cfg, w, x)
    perm = np.random.default_rng(25).permutation(wl.n_experts)  # new slot i holds old expert perm[i]
    w2 = dict(w)
    for n in ("router_w", "bias", "gate_exps", "up_exps", "down_exps"):
        w2[n] = w[n][perm]
    out2, ids2, ww2 = O.layer(cfg, w2, x)
    assert np.array_equal(perm[ids2], ids)
    assert np.array_equal(ww2, ww)
    assert np.allclose(out2, out, rtol=1e-13, atol=1e-15)


def test_layer_token_independence():
    wl, w = _tiny_layer(SF=64)
    cfg = O.make_cfg(wl.hidden, wl.n_experts, wl.top_k, wl.expert_ff, 64)
    x = np.random.default_rng(26).standard_normal((4, wl.hidden)).astype(np.float32)
    out, ids, ww = O.layer(cfg, w, x)
    for t in range(4):
        o1, i1, w1 = O.layer(cfg, w, x[t:t + 1])
        assert np.array_equal(o1[0], out[t]) and np.array_equal(i1[0], ids[t]) and np.array_equal(w1[0], ww[t])


def test_layer_logits_in_drives_selection():
    wl, w = _tiny_layer()
    cfg = O.make_cfg(wl.hidden, wl.n_experts, wl.top_k, wl.expert_ff)
    x = np.random.default_rng(27).standard_normal((2, wl.hidden)).astype(np.float32)
    li = np.tile(np.arange(wl.n_experts, dtype=np.float32), (2, 1))
    _, ids, ww = O.layer(cfg, w, x, logits_in=li)
    assert np.array_equal(ids, [[7, 6], [7, 6]])
    p = 1 / (1 + np.exp(-np.array([7.0, 6.0])))
    assert np.allclose(ww[0], p / p.sum(), rtol=1e-15)


# ----------------------------------------------------------------- sort ----

@pytest.mark.parametrize("seed", range(3))
def test_sort_by_expert_vs_stable_argsort(seed):
    rng = np.random.default_rng(seed)
    T, k, E = 97, 6, 40
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    off, perm = O.sort_by_expert(ids, E)
    flat = ids.reshape(-1)
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
