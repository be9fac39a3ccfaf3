"""Helpers shared by the GPU parity tests: input placement, oracle runs on
copies of the exact device inputs, and the parity measures.

Tolerance (per token row, on the FFN delta or the composed residual):
    ||y_gpu - y_oracle||_inf / ||y_oracle||_inf <= 1e-3
(f32 accumulation on the GPU against the oracle's f64).  Selected expert ids
must match bit-exact, except where the oracle certifies a near-tie: the two
disputed experts' f64 selection scores differ by less than TIE_TAU.

REG_TOL is a regression guard beside that gate: the f32 paths land about
1e-6 from the oracle on these inputs, so an error above 1e-5 means the
arithmetic changed even where the 1e-3 gate would still pass.

Every token row is compared.  The oracle runs over chunks of tokens in a
thread pool (its C calls release the interpreter lock), at most 16 threads.
"""
import concurrent.futures as cf
import os

import numpy as np
import torch

import moe_synth as S
import oracle as O

REL_TOL = 1e-3
REG_TOL = 1e-5
TIE_TAU = 1e-6
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def oracle_layer(cfg, wnp, x, resid=None, logits_in=None):
    """O.layer over the rows of x, split into chunks run in parallel threads (rows are independent)."""
    T = x.shape[0]
    n = min(ORACLE_THREADS, max(1, T))
    if n == 1:
        return O.layer(cfg, wnp, x, resid, logits_in)
    O.lib()  # load once before the threads start
    bounds = np.linspace(0, T, n + 1).astype(int)

    def run(i):
        a, b = bounds[i], bounds[i + 1]
        return O.layer(cfg, wnp, x[a:b], None if resid is None else resid[a:b],
                       None if logits_in is None else logits_in[a:b])

    with cf.ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(run, range(n)))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(3))


def oracle_cfg(wl):
    return O.make_cfg(wl.hidden, wl.n_experts, wl.top_k, wl.expert_ff, wl.shared_ff, wl.qtype, wl.n_groups,
                      wl.groups_used, wl.weights_scale, swiglu_limit=wl.swiglu_limit,
                      swiglu_limit_shared=wl.swiglu_limit_shared,
                      norm_eps=float(np.float32(wl.norm_eps or 1e-5)))  # the GPU config holds eps in f32


def to_device(w, device="cuda"):
    return {k: (None if v is None else v.to(device).contiguous()) for k, v in w.items()}


def row_rel_err(got, ref):
    """Per-row max-norm relative error."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-300)


def scores64(wnp, x_t, bias):
    l = O.router_logits(wnp["router_w"], x_t)
    p = 1.0 / (1.0 + np.exp(-l))
    return p + (0.0 if bias is None else bias.astype(np.float64))


def ffn_input(wl, wnp, x_t):
    """The FFN input of one token: x itself, or its RMSNorm when the layer has a norm weight."""
    if wnp.get("ffn_norm") is None:
        return x_t
    return O.rmsnorm(x_t, wnp["ffn_norm"], float(np.float32(wl.norm_eps or 1e-5)))


def check_ids(wl, wnp, x, ids_gpu, ids_ref):
    """Return the list of tokens whose ids differ; assert each is a certified near-tie."""
    bad = []
    for t in range(ids_ref.shape[0]):
        if np.array_equal(ids_gpu[t], ids_ref[t]):
            continue
        s = scores64(wnp, ffn_input(wl, wnp, x[t]), wnp.get("bias"))
        a, b = set(ids_gpu[t].tolist()), set(ids_ref[t].tolist())
        disputed = sorted(a ^ b) if a != b else [int(i) for i, j in zip(ids_gpu[t], ids_ref[t]) if i != j]
        gap = max(s[disputed]) - min(s[disputed])
        assert gap < TIE_TAU, f"token {t}: ids {ids_gpu[t]} vs oracle {ids_ref[t]} (score gap {gap:.3g})"
        bad.append(t)
    return bad


def oracle_given_routing(wl, wnp, x_t, ids, wts, resid_t=None):
    """Oracle FFN output of one token for forced ids / weights (used for certified near-ties)."""
    H, F, SF = wl.hidden, wl.expert_ff, wl.shared_ff
    out = np.zeros(H) if resid_t is None else resid_t.astype(np.float64).copy()
    xd = ffn_input(wl, wnp, x_t).astype(np.float64)
    for e, wj in zip(ids, wts):
        out += float(wj) * O.expert_ffn(wl.qtype, wnp["gate_exps"][e], wnp["up_exps"][e], wnp["down_exps"][e],
                                        H, F, xd, limit=wl.swiglu_limit)
    if SF:
        out += O.expert_ffn(wl.qtype, wnp["gate_sh"], wnp["up_sh"], wnp["down_sh"], H, SF, xd,
                            limit=wl.swiglu_limit_shared)
    return out


def run_layer_parity(wl, w_dev, x_dev, resid_dev=None, wnp=None, workspace=None):
    """Run moe_layer_step on the device and the oracle on the same inputs, every token row.
    Returns (max row rel err, n near-ties); also checks the routing weights and, on the
    grouped path, the GPU's sort of the pairs by expert (bit-exact)."""
    import sparse_moe_ffn_topk_amd as moe
    cfg = moe.config_for(wl)
    T = x_dev.shape[0]
    resid_in = torch.zeros_like(x_dev) if resid_dev is None else resid_dev.clone()
    out = resid_in.clone()
    ids = torch.empty((T, wl.top_k), dtype=torch.int32, device=x_dev.device)
    wts = torch.empty((T, wl.top_k), dtype=torch.float32, device=x_dev.device)
    ws = moe.alloc_workspace(cfg, T, x_dev.device) if workspace is None else workspace
    moe.layer_step(cfg, w_dev, x_dev, out, ids, wts, workspace=ws)
    torch.cuda.synchronize()
    if wnp is None:
        wnp = S.to_numpy(w_dev)
    x = x_dev.cpu().numpy()
    r = resid_in.cpu().numpy()
    ref, ids_ref, w_ref = oracle_layer(oracle_cfg(wl), wnp, x, r)
    ids_g = ids.cpu().numpy()
    wts_g = wts.cpu().numpy()
    got = out.cpu().numpy()
    ties = check_ids(wl, wnp, x, ids_g, ids_ref)
    for t in ties:  # compare outputs under the GPU's own (certified) routing
        ref[t] = oracle_given_routing(wl, wnp, x[t], ids_g[t], wts_g[t], r[t])
    ok = [t for t in range(T) if t not in ties]
    if ok and wl.top_k > 0:
        assert np.allclose(wts_g[ok], w_ref[ok], rtol=2e-6, atol=1e-7), "routing weights differ"
    if wl.top_k > 0 and T > moe.load_library().moe_decode_max_tokens():
        check_sort(cfg, ws, ids_g, T)
    # delta parity: compare FFN contributions, not the residual they ride on
    err = row_rel_err(got - r, ref - r)
    return float(err.max()), len(ties)


def read_region(cfg, ws, T, region, dtype=np.int32):
    import sparse_moe_ffn_topk_amd as moe
    off, n = moe.workspace_region(cfg, T, region)
    return ws[off:off + n].cpu().numpy().view(dtype)


def check_sort(cfg, ws, ids, T):
    """The grouped path's sort of the (token, pick) pairs of the last chunk, read back from the
    workspace, bit-exact against the oracle's stable sort; the tile list and pos against their
    definitions from it."""
    import sparse_moe_ffn_topk_amd as moe
    chunk = 512
    t0 = ((T - 1) // chunk) * chunk
    last = ids[t0:]
    E, k = cfg.n_experts, cfg.top_k
    off_ref, perm_ref = O.sort_by_expert(last, E)
    offsets = read_region(cfg, ws, T, moe.WS_OFFSETS)
    perm = read_region(cfg, ws, T, moe.WS_PERM)[:last.size]
    pos = read_region(cfg, ws, T, moe.WS_POS)[:last.size]
    assert np.array_equal(offsets, off_ref), "sort offsets differ from the oracle"
    assert np.array_equal(perm, perm_ref), "sort permutation differs from the oracle"
    assert np.array_equal(pos[perm_ref], np.arange(last.size)), "pos is not the inverse of perm"
    tiles_ref = [(e, 16 * i) for e in range(E) for i in range((off_ref[e + 1] - off_ref[e] + 15) // 16)]
    ntiles = int(read_region(cfg, ws, T, moe.WS_NTILES)[0])
    tiles = read_region(cfg, ws, T, moe.WS_TILES).reshape(-1, 2)[:ntiles]
    assert ntiles == len(tiles_ref) and np.array_equal(tiles, np.array(tiles_ref, np.int32).reshape(-1, 2)), \
        "tile list differs"
