#!/usr/bin/env python
"""Benchmark of the routed MoE FFN step (Q4 experts) on one MI355X.

Default workload: the Flint-shaped decode stack -- H 2048, 256 experts top-6
by sigmoid, SwiGLU experts ff 512 plus an always-on shared expert ff 1024, all
Q4_1, batch 1, 47 distinct MoE layers resident in HBM (23.9 GB).  One step =
one decode token through all 47 layers: router logits, top-k, gate||up +
SwiGLU, down + weighted residual accumulate, per layer, in layer order on one
stream (each layer's expert reads start after the previous layer finished).

The stack is chained by default (--stack chained): every layer carries a
pre-FFN RMSNorm weight (1 + N(0, 0.1)) and takes the running residual as its
input, resid += FFN(rms_norm(resid) * w), so each layer's routing depends on
the previous layer's output -- a real data-dependent chain, as in a decoder
(the attention between the FFNs is outside this path).  --stack independent
instead gives every layer its own synthetic, already normalised input
(x ~ N(0,1), 16 pre-generated steps cycled).  Other inputs are synthetic and
seeded (moe_synth): router N(0, 0.05); Q4 scales U(0.001, 0.02) in f16;
uniform nibbles.  Weights are generated directly on the GPU.

Timing: each step variant (one native moe_stack_step call) is captured once as
a HIP graph; W warm-up replays, then K timed replays between two
synchronisations give the headline.  A second timed region of eager native
steps measures kernel durations: the library attaches HIP start/stop events to
every dispatch of the kernel under test, on its stream; the dominant kernel
(gate||up + SwiGLU) gives the roofline line.  The CPU baseline times the f64
oracle on a bounded sample.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "MoE-layer decode tokens/s + achieved weight-stream GB/s (% of HBM peak), 1 GPU"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# Sources each dominant kernel is built from: its committed traffic counters
# are used only while these files are unchanged.
KERNEL_SOURCES = {
    "gateup_swiglu": ("moe_common.h", "select_block.h", "ffn_decode.h", "ffn_decode_q41.hip", "ffn_decode_q40.hip"),
    "group_gateup": ("moe_common.h", "prefill.hip"),
}
# (the grouped gate||up at the Flint prefill shape runs as the row-streaming kernel)
KERNEL_SYMBOLS = {"gateup_swiglu": "k_gateup_swiglu", "group_gateup": "k_group_gateup_rows"}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for fn in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sparse_moe_ffn_topk_amd", "csrc", fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(kernel, workload, ext):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.{ext}")


def load_traffic(kernel, workload):
    """HBM traffic per launch of the dominant kernel from committed rocprofv3 counter runs,
    only if they were taken on the current kernel source."""
    p = traffic_path(kernel, workload, "json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != kernel_source_hash(kernel):
        return None
    return d.get("bytes_per_launch")


def _pmc_means(run_dir, counter):
    """Mean per-dispatch value of one counter, per kernel name, from a rocprofv3 --pmc output folder."""
    import glob
    import sqlite3
    dbs = glob.glob(os.path.join(run_dir, "*.db")) + glob.glob(os.path.join(run_dir, "*", "*.db"))
    if not dbs:
        raise FileNotFoundError(f"no rocprofv3 database under {run_dir}")
    con = sqlite3.connect(dbs[0])
    acc = {}
    for name, val in con.execute("select name, counter_value from pmc_events where counter_name = ?", (counter,)):
        acc.setdefault(name, []).append(val)
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def write_traffic(args):
    """profiles/<kernel>_<workload>_traffic.{json,md} from four rocprofv3 --pmc runs: FETCH_SIZE and
    WRITE_SIZE of the workload, and of the copy calibration (a 1 GiB device copy)."""
    kernel = "group_gateup" if args.workload == "prefill" else "gateup_swiglu"
    fetch_dir, write_dir, copyf_dir, copyw_dir = args.write_traffic
    sym = KERNEL_SYMBOLS[kernel]

    def pick(d, want):
        hits = {k: v for k, v in d.items() if want(k)}
        if not hits:
            raise SystemExit(f"no matching kernel in {sorted(d)[:8]}")
        return max(hits.items(), key=lambda kv: kv[1][1])  # the most dispatched

    kname, (fetch, nd) = pick(_pmc_means(fetch_dir, "FETCH_SIZE"), lambda k: sym in k)
    _, (write, _) = pick(_pmc_means(write_dir, "WRITE_SIZE"), lambda k: sym in k)
    copy_bytes = (1 << 28) * 4
    _, (cf, _) = pick(_pmc_means(copyf_dir, "FETCH_SIZE"), lambda k: "copy" in k.lower() or "elementwise" in k.lower())
    _, (cw, _) = pick(_pmc_means(copyw_dir, "WRITE_SIZE"), lambda k: "copy" in k.lower() or "elementwise" in k.lower())
    fscale, wscale = copy_bytes / 1024.0 / cf, copy_bytes / 1024.0 / cw
    fscale, wscale = round(fscale, 3), round(wscale, 3)
    nbytes = int(round((fetch * fscale + write * wscale) * 1024))
    cmds = args.traffic_commands or []
    rec = {"kernel": kname.split("(")[0], "workload": args.workload, "kernel_source_sha": kernel_source_hash(kernel),
           "dispatches": nd, "fetch_kib_per_dispatch": round(fetch, 1), "write_kib_per_dispatch": round(write, 1),
           "fetch_scale": fscale, "write_scale": wscale, "bytes_per_launch": nbytes, "commands": cmds}
    with open(traffic_path(kernel, args.workload, "json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    with open(traffic_path(kernel, args.workload, "md"), "w") as f:
        f.write(f"# HBM traffic per dispatch: {rec['kernel']} ({args.workload})\n\n")
        f.write("Counter passes, each in its own run (repo root on the MI355X host, TMPDIR=/tmp):\n\n")
        for c in cmds:
            f.write(f"    {c}\n")
        f.write(f"\nCopy calibration: a {copy_bytes >> 20} MiB device copy reads FETCH_SIZE = {cf:.0f} KiB and "
                f"WRITE_SIZE = {cw:.0f} KiB per dispatch, so FETCH_SIZE is scaled by {fscale} and WRITE_SIZE by "
                f"{wscale}.\n\n")
        f.write("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes per launch |\n|---|---|---|---|---|\n")
        f.write(f"| {rec['kernel']} | {nd} | {fetch:.1f} | {write:.1f} | {nbytes:,} |\n\n")
        f.write(f"Kernel source hash {rec['kernel_source_sha']} (the bench reports this traffic only while the "
                f"sources are unchanged).  Written by `python bench.py --workload {args.workload} --write-traffic "
                f"...`.\n")
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="flint",
                    choices=["flint", "flint8", "lfm25", "lfm25_q8", "ling", "tiny", "prefill", "flint_dense",
                             "lfm25_dense"])
    ap.add_argument("--slots", type=int, default=16, help="distinct input steps cycled")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--swiglu-limit", type=float, default=0.0,
                    help="SwiGLU clamp L for the routed and the shared experts (0: none)")
    ap.add_argument("--stack", default="chained", choices=["chained", "independent"],
                    help="chained (default): every layer has a pre-FFN RMSNorm weight and takes the running "
                         "residual as its input, resid += FFN(rms_norm(resid) * w), a real data-dependent chain; "
                         "independent: every layer takes its own synthetic (already normalised) input")
    ap.add_argument("--no-kernel-timer", action="store_true")
    ap.add_argument("--mode", default="graph", choices=["eager", "graph"],
                    help="graph: each step variant (one native moe_stack_step call) replayed as a captured HIP "
                         "graph; eager: the native call itself, launched step by step")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/<kernel>_<workload>_traffic.{json,md} from rocprofv3 --pmc output folders "
                         "(runs nothing on the GPU)")
    ap.add_argument("--traffic-commands", nargs="*", help="the commands that made the --write-traffic folders")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 8 device-to-device copies of 1 GiB (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()

    if args.write_traffic:
        write_traffic(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              f"the multi-GPU sharding is a design, not a measured path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_synth as S
    import sparse_moe_ffn_topk_amd as moe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    moe.load_library()
    dev = "cuda"
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": src.numel() * 4, "copies": 8}), flush=True)
        return
    wl = S.WORKLOADS[args.workload]
    args.chained = args.stack == "chained" and args.workload != "prefill"
    if args.swiglu_limit > 0:
        import dataclasses
        wl = dataclasses.replace(wl, swiglu_limit=args.swiglu_limit, swiglu_limit_shared=args.swiglu_limit)
    if args.chained:
        import dataclasses
        wl = dataclasses.replace(wl, norm_eps=1e-5)  # every layer carries its pre-FFN RMSNorm weight
        args.slots = 1
    L, T, nS = wl.layers, wl.tokens, args.slots
    if wl.name == "ling":
        L = 28  # 28 generated copies of the one layer shape exceed the 256 MB MALL 4x over
    if wl.name == "prefill":
        L = 4   # 4 generated layers cycled (509 MB each touched per chunk)
    cfg = moe.config_for(wl)
    bs = S.BLOCK_BYTES[wl.qtype]
    per_expert = 3 * wl.expert_ff * (wl.hidden // 32) * bs
    shared_bytes = 3 * wl.shared_ff * (wl.hidden // 32) * bs
    router_bytes = wl.n_experts * wl.hidden * 4 + (wl.n_experts * 4 if wl.has_bias else 0)

    t0 = time.time()
    log(f"workload {wl.name}: H={wl.hidden} E={wl.n_experts} k={wl.top_k} F={wl.expert_ff} SF={wl.shared_ff} "
        f"qtype=Q4_{wl.qtype} T={T} layers={L}; generating weights on the GPU")
    layers, lws = [], []
    for l in range(L):
        w = S.make_layer(wl, layer=l, device=dev)
        layers.append(w)
        lws.append(moe.layer_weights(w))
        if l % 8 == 7:
            log(f"  {l + 1}/{L} layers generated")
    torch.cuda.synchronize()
    resident = sum(sum(t.numel() * t.element_size() for t in w.values() if t is not None) for w in layers)
    log(f"weights resident: {resident / 1e9:.2f} GB in {time.time() - t0:.1f}s")

    if args.chained:
        # the chained stack: each layer's input is the running residual (x aliases resid),
        # resid += FFN(rms_norm(resid) * ffn_norm) layer after layer
        resid = S.make_x(wl, T, layer=0, step=0, device=dev)
        xs = [[resid] * L]
    else:
        xs = [[S.make_x(wl, T, layer=l, step=s, device=dev) for l in range(L)] for s in range(nS)]
        resid = torch.zeros((T, wl.hidden), dtype=torch.float32, device=dev)
    ws = moe.alloc_workspace(cfg, T, dev)
    ids = [torch.empty((L, T, wl.top_k), dtype=torch.int32, device=dev) for _ in range(nS)]
    wts = [torch.empty((L, T, wl.top_k), dtype=torch.float32, device=dev) for _ in range(nS)]
    stacks = [moe.Stack(cfg, layers, xs[s], resid, ids[s], wts[s], ws) for s in range(nS)]

    # one pass over every input variant (loads code objects, fills ids for the byte model)
    for s in range(nS):
        stacks[s].step()
    torch.cuda.synchronize()
    graphs = []
    if args.mode == "graph":
        for s in range(nS):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                stacks[s].step()
            graphs.append(g)
        torch.cuda.synchronize()
        log(f"captured {nS} graphs of {L} layer steps")

    def run(i):
        if graphs:
            graphs[i % nS].replay()
        else:
            stacks[i % nS].step()

    # algorithmic weight bytes per step variant: router + bias + distinct picked experts + shared
    distinct = np.zeros((nS, L))
    for s in range(nS):
        h = ids[s].cpu().numpy()
        for l in range(L):
            distinct[s, l] = len(np.unique(h[l]))
    step_bytes = [float(L * (router_bytes + shared_bytes) + distinct[s].sum() * per_expert) for s in range(nS)]
    log(f"distinct picked experts per layer step: mean {distinct.mean():.1f} (T={T} tokens x {wl.top_k} picks)")

    grouped = T > moe.load_library().moe_decode_max_tokens()
    dominant = (moe.KERNEL_GROUP_GATEUP, "group_gateup") if grouped else (moe.KERNEL_GATEUP, "gateup_swiglu")
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done; timing {args.steps} steps ({args.mode})")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        run(i)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    mean_bytes = sum(step_bytes[i % nS] for i in range(args.steps)) / args.steps
    tok_s = T / (ms_step / 1e3)
    gbps = mean_bytes / (ms_step / 1e3) / 1e9
    log(f"timed: {ms_step * 1e3:.1f} us/step ({ms_step * 1e3 / L:.2f} us/layer), {tok_s:.1f} tok/s, "
        f"{gbps:.1f} GB/s of weights ({100 * gbps / HBM_PEAK_GBPS:.1f}% of 8 TB/s); wall {wall:.3f}s")

    # Kernel durations: a second timed region of eager native steps in which the
    # library attaches HIP start/stop events to every dispatch of one kernel (on
    # the stream it is launched on); events recorded inside a captured graph are
    # not measurable, so graph replays cannot carry them.
    kstats = {}
    if not args.no_kernel_timer:
        nk = min(args.steps, 60)
        others = ((("router", moe.KERNEL_ROUTER), ("select", moe.KERNEL_SELECT), ("sort", moe.KERNEL_SORT),
                   ("group_down", moe.KERNEL_GROUP_DOWN), ("combine", moe.KERNEL_COMBINE)) if grouped else
                  (("router", moe.KERNEL_ROUTER), ("down_accum", moe.KERNEL_DOWN))
                  + ((("prelude", moe.KERNEL_PRELUDE),) if T > 1 else ()))
        for name, kid in ((dominant[1], dominant[0]),) + others:
            with moe.KernelTimer(kid, 2 * nk * L) as kt:  # (room for two launches per layer)
                for i in range(nk):
                    stacks[i % nS].step()
                torch.cuda.synchronize()
            # (mean per launch, and the kernel's time per layer step: the two differ where a
            # kernel runs more than once per layer)
            kstats[name] = {"launches": kt.count, "mean_us": kt.mean_us,
                            "us_per_layer": 1000.0 * kt.total_ms / (nk * L)}
        log("kernel means (us, eager dispatches): " + ", ".join(f"{k}={v['mean_us']:.2f}" for k, v in kstats.items()))
        log("kernel time per layer step (us): " + ", ".join(f"{k}={v['us_per_layer']:.2f}" for k, v in kstats.items()))

    roofline = None
    if "group_gateup" in kstats:
        # grouped gate||up: every distinct expert's gate and up rows once per chunk, the shared expert's,
        # x read, act written; 2*T*k*F*H*2 + 2*T*SF*H*2 useful MFMA flops alongside
        gu_expert = 2 * wl.expert_ff * (wl.hidden // 32) * bs
        gu_shared = 2 * wl.shared_ff * (wl.hidden // 32) * bs
        d_mean = float(np.mean([distinct[i % nS].mean() for i in range(args.steps)]))
        act_bytes = T * (wl.top_k * wl.expert_ff + wl.shared_ff) * 4 + T * wl.hidden * 4
        per_launch = d_mean * gu_expert + gu_shared + act_bytes
        us = kstats["group_gateup"]["mean_us"]
        ach = per_launch / (us * 1e-6) / 1e9
        flops = 2.0 * 2 * T * (wl.top_k * wl.expert_ff + wl.shared_ff) * wl.hidden
        roofline = {"bound": "hbm", "kernel": "k_group_gateup_rows", "achieved": round(ach, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                    "traffic": load_traffic("group_gateup", wl.name), "algorithmic_bytes_per_launch": int(per_launch),
                    "mean_launch_us": round(us, 3),
                    "mfma_tflops": round(flops / (us * 1e-6) / 1e12, 2), "mfma_peak_tflops_f16": 2500.0}
    if "gateup_swiglu" in kstats:
        # algorithmic bytes of one gate||up launch: distinct picked experts' gate and up rows, the shared
        # expert's gate and up rows, x read once per token, act written once
        gu_expert = 2 * wl.expert_ff * (wl.hidden // 32) * bs
        gu_shared = 2 * wl.shared_ff * (wl.hidden // 32) * bs
        d_mean = float(np.mean([distinct[i % nS].mean() for i in range(args.steps)]))
        act_bytes = T * (wl.top_k * wl.expert_ff + wl.shared_ff) * 4 + T * wl.hidden * 4
        per_launch = d_mean * gu_expert + gu_shared + act_bytes
        ach = per_launch / (kstats["gateup_swiglu"]["mean_us"] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": "k_gateup_swiglu", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": load_traffic("gateup_swiglu", wl.name),
                    "algorithmic_bytes_per_launch": int(per_launch),
                    "mean_launch_us": round(kstats["gateup_swiglu"]["mean_us"], 3)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        nl = min(3, L)
        host = [S.to_numpy(layers[l]) for l in range(nl)]
        xh = [xs[0][l].cpu().numpy() for l in range(nl)]
        ocfg = O.make_cfg(wl.hidden, wl.n_experts, wl.top_k, wl.expert_ff, wl.shared_ff, wl.qtype, wl.n_groups,
                          wl.groups_used, wl.weights_scale)
        log(f"cpu baseline: f64 oracle, 1 thread, ~{args.cpu_seconds:.0f}s")
        n, c0 = 0, time.perf_counter()
        while n < nl or time.perf_counter() - c0 < args.cpu_seconds:
            O.layer(ocfg, host[n % nl], xh[n % nl])
            n += 1
        per_layer = (time.perf_counter() - c0) / n
        cpu = {"value": round(T / (per_layer * L), 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} oracle layer-steps (T={T}) cycling {nl} of the {L} generated layers, "
                         f"{per_layer * 1e3:.1f} ms each, scaled to the {L}-layer stack"}
        log(f"cpu baseline: {per_layer * 1e3:.1f} ms per layer-step -> {cpu['value']} tok/s")

    out = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{wl.name}_T{T}_{L}layers" + ("_chained" if args.chained else "")
                               + (f"_clamp{args.swiglu_limit:g}" if args.swiglu_limit > 0 else ""),
                   "hidden": wl.hidden, "n_experts": wl.n_experts,
                   "top_k": wl.top_k, "expert_ff": wl.expert_ff, "shared_ff": wl.shared_ff,
                   "qtype": {0: "Q4_0", 1: "Q4_1", 2: "Q8_0"}[wl.qtype], "tokens": T, "layers": L, "global_batch": T,
                   "parallelism": "single-gpu"},
        "weight_stream_GBps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "us_per_layer": round(ms_step * 1e3 / L, 3), "tok_s_per_layer": round(tok_s * L, 1),
        "weight_bytes_per_step": int(mean_bytes), "kernels_us": {k: round(v["mean_us"], 3) for k, v in kstats.items()},
        "kernels_us_per_layer": {k: round(v["us_per_layer"], 3) for k, v in kstats.items()},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
