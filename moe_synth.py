"""Seeded synthetic inputs for the routed MoE FFN step (Q4_0 / Q4_1 experts).

Shared by the tests, the smoke check and the benchmark; used to feed BOTH the
HIP library and the CPU oracle.  It holds no arithmetic of the method: it only
draws random tensors and packs random numbers into the GGUF block byte layout.

Workload shapes follow the three diskformer engine pages (Flint: H 2048, 256
experts top-6, ff 512, shared ff 1024, Q4_1; LFM2.5-24B-A2B: H 2048, 64
experts top-4 with a selection bias, ff 1536, Q4_0; Ling 3.0 flash: H 2560,
512 experts in 8 groups, 4 groups kept, top-8, ff 768 + shared 768, weights
scale 2.5) plus a tiny layer.  Distributions (the pages give none):
  x ~ N(0, 1) f32;  router ~ N(0, 0.05) f32;  bias ~ N(0, 0.1) f32;
  Q4 block scales d (and Q4_1 offsets m) ~ U(0.001, 0.02) rounded to f16
  (round to nearest even);  nibbles i.i.d. uniform over 0..15.
Every tensor has its own torch.Generator seeded from a hash of
(master seed, workload, layer, tensor name), so any tensor of any layer can
be regenerated alone, on the CPU or on the GPU (same generator family per
device; the oracle always receives copies of the exact tensors the GPU used).
"""
import dataclasses
import hashlib

import torch

Q4_0, Q4_1, Q8_0 = 0, 1, 2
BLOCK_BYTES = {Q4_0: 18, Q4_1: 20, Q8_0: 34}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    n_experts: int
    top_k: int
    expert_ff: int
    shared_ff: int = 0
    qtype: int = Q4_1
    n_groups: int = 1
    groups_used: int = 1
    weights_scale: float = 1.0
    has_bias: bool = False
    swiglu_limit: float = 0.0         # SwiGLU clamp of the routed experts (0: none)
    swiglu_limit_shared: float = 0.0  # and of the shared expert
    norm_eps: float = 0.0             # > 0: layers carry a pre-FFN RMSNorm weight, 1 + N(0, norm_std)
    norm_std: float = 0.1
    tokens: int = 1
    layers: int = 1
    # distributions
    router_std: float = 0.05
    bias_std: float = 0.1
    scale_lo: float = 0.001
    scale_hi: float = 0.02
    # wide-range variants (off by default): d (and Q4_1 m) of either sign, m ~ U(-hi, hi); a fraction of
    # blocks with an f16-subnormal d; x scaled, and a fraction of x entries replaced by +-x_outlier
    signed_scales: bool = False
    subnormal_frac: float = 0.0
    x_scale: float = 1.0
    x_outlier_frac: float = 0.0
    x_outlier: float = 30.0
    # Q4_1 offsets centred on the block: m = -c * d, c ~ U(7, 8) (rounded to f16), so a block spans about
    # [-7.5 d, 7.5 d] as when zero-mean weights are quantised (m is the block minimum); off: m ~ U(lo, hi)
    centred: bool = False


WORKLOADS = {
    "tiny": Workload("tiny", 256, 8, 2, 128, 0, Q4_1, tokens=1, layers=1),
    "flint": Workload("flint", 2048, 256, 6, 512, 1024, Q4_1, tokens=1, layers=47),
    "flint8": Workload("flint8", 2048, 256, 6, 512, 1024, Q4_1, tokens=8, layers=47),
    "lfm25": Workload("lfm25", 2048, 64, 4, 1536, 0, Q4_0, has_bias=True, tokens=1, layers=38),
    "ling": Workload("ling", 2560, 512, 8, 768, 768, Q4_1, n_groups=8, groups_used=4, weights_scale=2.5,
                     has_bias=True, tokens=1, layers=1),
    "prefill": Workload("prefill", 2048, 256, 6, 512, 1024, Q4_1, tokens=512, layers=1),
    # LFM2.5 shape with Q8_0 experts (the lfm2_moe_ssd.js page's int8 expert plane); Q8_0 scales are a
    # row block's max |w| / 127, so they are drawn smaller
    "lfm25_q8": Workload("lfm25_q8", 2048, 64, 4, 1536, 0, Q8_0, has_bias=True, tokens=1, layers=38,
                         scale_lo=0.0001, scale_hi=0.0004),
    # dense leading SwiGLU FFN layers (no router): Flint and Ling 6144, LFM2.5 11776 (Q4_0 here).  The
    # models have two such layers; 16 generated copies are cycled so the weights exceed the 256 MB MALL.
    "flint_dense": Workload("flint_dense", 2048, 0, 0, 0, 6144, Q4_1, tokens=1, layers=16),
    "lfm25_dense": Workload("lfm25_dense", 2048, 0, 0, 0, 11776, Q4_0, tokens=1, layers=16),
}


def seed_for(master, workload, layer, tensor):
    h = hashlib.blake2b(f"{master}/{workload}/{layer}/{tensor}".encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std, device, seed):
    t = torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    return t * std if std != 1.0 else t


def q4_blocks(n_blocks, qtype, device, seed, lo=0.001, hi=0.02, chunk=1 << 24, signed=False, subnormal_frac=0.0,
              centred=False):
    """n_blocks random GGUF blocks as a uint8 tensor [n_blocks, 18|20|34].

    Byte layout: f16 d (little endian), for Q4_1 also f16 m, then 16 bytes of
    nibbles (Q4) or 32 signed bytes (Q8_0).  d, m ~ U(lo, hi) rounded to f16;
    nibble and int8 bytes uniform 0..255.  With signed: d takes a random sign
    and m ~ U(-hi, hi); with subnormal_frac > 0 that fraction of the blocks
    gets a d drawn uniformly from the nonzero f16 subnormals (either sign).
    With centred (Q4_1): m = -c d with c ~ U(7, 8), rounded to f16."""
    bs = BLOCK_BYTES[qtype]
    out = torch.empty((n_blocks, bs), dtype=torch.uint8, device=device)
    g = _gen(device, seed)
    for s in range(0, n_blocks, chunk):
        n = min(chunk, n_blocks - s)
        o = out[s:s + n]
        d = (torch.rand(n, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo).to(torch.float16)
        q0 = 2
        if qtype == Q4_1:
            m = (torch.rand(n, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo).to(torch.float16)
            q0 = 4
        o[:, q0:] = torch.randint(0, 256, (n, bs - q0), generator=g, device=device, dtype=torch.uint8)
        if signed:
            sign = torch.randint(0, 2, (n,), generator=g, device=device).to(torch.float16) * 2 - 1
            d = d * sign
            if qtype == Q4_1:
                m = ((torch.rand(n, generator=g, device=device, dtype=torch.float32) * 2 - 1) * hi).to(torch.float16)
        if centred and qtype == Q4_1:
            c = torch.rand(n, generator=g, device=device, dtype=torch.float32) + 7.0
            m = (-(c * d.to(torch.float32))).to(torch.float16)
        if subnormal_frac > 0:
            pick = torch.rand(n, generator=g, device=device) < subnormal_frac
            bits = torch.randint(1, 1024, (n,), generator=g, device=device, dtype=torch.int32)
            bits = bits | (torch.randint(0, 2, (n,), generator=g, device=device, dtype=torch.int32) << 15)
            sub = bits.to(torch.int16).view(torch.float16)
            d = torch.where(pick, sub, d)
        o[:, 0:2] = d.view(torch.uint8).view(n, 2)
        if qtype == Q4_1:
            o[:, 2:4] = m.view(torch.uint8).view(n, 2)
    return out


def expert_tensor(n_experts, rows, cols, qtype, device, seed, wl=None):
    """E experts of `rows` rows, each a row of cols/32 blocks: uint8 [E, rows, cols/32*bs]."""
    nb = cols // 32
    lo, hi = (wl.scale_lo, wl.scale_hi) if wl else (0.001, 0.02)
    signed = wl.signed_scales if wl else False
    subn = wl.subnormal_frac if wl else 0.0
    cen = wl.centred if wl else False
    b = q4_blocks(n_experts * rows * nb, qtype, device, seed, lo, hi, signed=signed, subnormal_frac=subn, centred=cen)
    return b.view(n_experts, rows, nb * BLOCK_BYTES[qtype])


def make_layer(wl, layer=0, device="cpu", master=0):
    """All weights of one MoE layer of workload `wl`, on `device`."""
    H, E, F, SF = wl.hidden, wl.n_experts, wl.expert_ff, wl.shared_ff
    s = lambda name: seed_for(master, wl.name, layer, name)
    routed = E > 0  # E == 0: a dense SwiGLU FFN layer, held in the shared tensors
    w = {
        "router_w": normal((E, H), wl.router_std, device, s("router_w")) if routed else None,
        "bias": normal((E,), wl.bias_std, device, s("bias")) if wl.has_bias and routed else None,
        "gate_exps": expert_tensor(E, F, H, wl.qtype, device, s("gate_exps"), wl) if routed else None,
        "up_exps": expert_tensor(E, F, H, wl.qtype, device, s("up_exps"), wl) if routed else None,
        "down_exps": expert_tensor(E, H, F, wl.qtype, device, s("down_exps"), wl) if routed else None,
        "gate_sh": None, "up_sh": None, "down_sh": None,
    }
    if wl.norm_eps > 0:
        w["ffn_norm"] = normal((H,), wl.norm_std, device, s("ffn_norm")) + 1.0
    if SF:
        w["gate_sh"] = expert_tensor(1, SF, H, wl.qtype, device, s("gate_sh"), wl)[0]
        w["up_sh"] = expert_tensor(1, SF, H, wl.qtype, device, s("up_sh"), wl)[0]
        w["down_sh"] = expert_tensor(1, H, SF, wl.qtype, device, s("down_sh"), wl)[0]
    return w


def make_x(wl, tokens=None, layer=0, step=0, device="cpu", master=0):
    """FFN input (already normalised by the caller's RMSNorm): [T, H] ~ N(0, 1)."""
    T = wl.tokens if tokens is None else tokens
    seed = seed_for(master, wl.name, layer, f"x/{step}/{T}")
    x = normal((T, wl.hidden), 1.0, device, seed)
    if wl.x_scale != 1.0:
        x = x * wl.x_scale
    if wl.x_outlier_frac > 0:
        g = _gen(device, seed ^ 0x5A5A5A5A)
        pick = torch.rand(x.shape, generator=g, device=device) < wl.x_outlier_frac
        sign = torch.randint(0, 2, x.shape, generator=g, device=device).to(torch.float32) * 2 - 1
        x = torch.where(pick, sign * wl.x_outlier, x)
    return x


def layer_weight_bytes(wl):
    """Resident bytes of one layer (router + bias + all experts + shared)."""
    bs = BLOCK_BYTES[wl.qtype]
    H, E, F, SF = wl.hidden, wl.n_experts, wl.expert_ff, wl.shared_ff
    per_exp = 3 * F * (H // 32) * bs
    return E * H * 4 + (E * 4 if wl.has_bias else 0) + E * per_exp + 3 * SF * (H // 32) * bs


def to_numpy(w):
    return {k: (None if v is None else v.detach().cpu().numpy()) for k, v in w.items()}
