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
uniform nibbles; in the chained stack the Q4_1 offsets are centred on the
block (m = -c d, c ~ U(7, 8)), else m ~ U(0.001, 0.02).  Weights are generated directly on the GPU.

Timing: each step variant (one native moe_stack_step call) is captured once as
a HIP graph; W warm-up replays, then K timed replays between two
synchronisations give the headline.  A second timed region of eager native
steps measures kernel durations: the library attaches HIP start/stop events to
every dispatch of the kernel under test, on its stream; the dominant kernel
(gate||up + SwiGLU) gives the roofline line.  The CPU baseline times the f64
oracle over one whole step on one thread and on N threads at once (median of
3 each; a token sample, scaled, where a whole step would exceed the time
budget), and recomputes every layer from the GPU's own input for the parity
figures.

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
    """Hash of the code (comments and blank space removed) of the sources a kernel is built from."""
    import re
    h = hashlib.sha256()
    for fn in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sparse_moe_ffn_topk_amd", "csrc", fn)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
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
        f.write(f"Kernel source hash {rec['kernel_source_sha']} (of the code with comments removed; the bench reports "
                f"this traffic only while that code is unchanged).  Written by `python bench.py --workload "
                f"{args.workload} --write-traffic ...`.\n")
    print(json.dumps(rec))


def stream_peak(moe, torch, reps=5, gib=4):
    """Achievable streaming-read rate: the probe kernel reading `gib` GiB with 16-byte loads, for a few grid
    sizes; returns (best median GB/s, {blocks: median GB/s})."""
    import ctypes as C
    nbytes = gib << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    L = moe.load_library()
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for blocks in (1024, 2048, 4096, 8192):
        L.moe_probe_stream(C.c_void_p(buf.data_ptr()), nbytes, blocks, None, st)  # warm
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rc = L.moe_probe_stream(C.c_void_p(buf.data_ptr()), nbytes, blocks, None, st)
            b.record()
            torch.cuda.synchronize()
            if rc:
                raise RuntimeError(f"moe_probe_stream rc {rc}")
            times.append(a.elapsed_time(b))
        times.sort()
        res[blocks] = nbytes / (times[len(times) // 2] * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return max(res.values()), res


def run_probes(args):
    """Chip probes: the achievable streaming rate, the per-launch floor of a streaming kernel, the kernel
    boundary in a graph, and the cost of an in-kernel all-to-all exchange between blocks."""
    import ctypes as C

    import torch

    import sparse_moe_ffn_topk_amd as moe
    L = moe.load_library()
    out = {"probe": "mi355x"}
    peak, by_blocks = stream_peak(moe, torch)
    out["stream_4GiB_GBps"] = round(peak, 1)
    out["stream_4GiB_by_blocks"] = {str(k): round(v, 1) for k, v in by_blocks.items()}
    log(f"streaming read of 4 GiB: {peak:.1f} GB/s (best grid); by blocks {out['stream_4GiB_by_blocks']}")

    # per-launch floor: N launches over distinct regions of a 4 GiB ring (far beyond the 256 MB MALL, so a
    # launch never finds its bytes cached), captured as one graph and replayed
    ring = torch.zeros(4 << 30, dtype=torch.uint8, device="cuda")
    base = ring.data_ptr()
    floor = {}
    for mb in (2, 5, 10, 17.8, 20):
        nbytes = int(mb * 1e6) // 16 * 16
        stride = (nbytes + 4095) // 4096 * 4096
        per = (4 << 30) // stride
        n = min(per, max(100, -(-(1 << 30) // nbytes)))  # at least 1 GiB of distinct regions per graph
        best = None
        for blocks in (256, 512, 1024, 2048):
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for i in range(3):
                    L.moe_probe_stream(C.c_void_p(base + (i % per) * stride), nbytes, blocks, None,
                                       C.c_void_p(s.cuda_stream))
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=s):
                    for i in range(n):
                        L.moe_probe_stream(C.c_void_p(base + (i % per) * stride), nbytes, blocks, None,
                                           C.c_void_p(s.cuda_stream))
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(5):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / (5 * n)
            if best is None or us < best[0]:
                best = (us, blocks)
            del g
        floor[str(mb)] = {"us_per_launch": round(best[0], 3), "blocks": best[1],
                          "GBps": round(nbytes / (best[0] * 1e-6) / 1e9, 1)}
        log(f"per-launch floor {mb} MB: {best[0]:.2f} us ({best[1]} blocks, {floor[str(mb)]['GBps']} GB/s)")
    out["launch_floor"] = floor
    del ring
    torch.cuda.empty_cache()

    # kernel boundary: empty kernels back to back in a graph
    gaps = {}
    n = 200
    for blocks in (1, 256, 1024):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            L.moe_probe_empty(blocks, C.c_void_p(s.cuda_stream))
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for i in range(n):
                    L.moe_probe_empty(blocks, C.c_void_p(s.cuda_stream))
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        gaps[str(blocks)] = round(a.elapsed_time(b) * 1e3 / (10 * n), 3)
        del g
    out["empty_kernel_us_in_graph"] = gaps
    log(f"empty kernels in a graph, us per launch by blocks: {gaps}")

    # in-kernel all-to-all exchange between co-resident blocks (bounded waits)
    ex = {}
    rounds = 2000
    for blocks in (8, 64, 256, 512):
        slots = torch.zeros(blocks, dtype=torch.int64, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        cyc = torch.zeros(2, dtype=torch.int64, device="cuda")
        rc = L.moe_probe_exchange(blocks, rounds, 20000, C.c_void_p(slots.data_ptr()), C.c_void_p(status.data_ptr()),
                                  C.c_void_p(cyc.data_ptr()), C.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        if rc:
            ex[str(blocks)] = {"error": f"launch rc {rc}"}
            continue
        c = cyc.cpu().tolist()
        ok = int(status.item()) == 0
        ex[str(blocks)] = {"us_per_round": round((c[1] - c[0]) * 0.01 / rounds, 3), "completed": ok}
    out["exchange_all_to_all"] = ex
    log(f"all-to-all exchange, us per round by blocks: {ex}")
    print(json.dumps(out), flush=True)
    if args.probe_out:
        write_probe_md(out, args.probe_out)


def write_probe_md(d, path):
    with open(path, "w") as f:
        f.write("# Chip probes: streaming rate, launch floor, kernel boundary, in-kernel exchange (MI355X)\n\n")
        f.write("Command (repo root on the MI355X host):\n\n    python bench.py --probe --probe-out " + path + "\n\n")
        f.write(f"Streaming read of 4 GiB with 16-byte loads (best grid, median of 5): "
                f"**{d['stream_4GiB_GBps']} GB/s** ({100 * d['stream_4GiB_GBps'] / HBM_PEAK_GBPS:.1f} % of 8 TB/s); "
                f"by blocks of 256 threads: {d['stream_4GiB_by_blocks']}.\n\n")
        f.write("Per-launch floor: launches of the streaming kernel, each over a distinct region of a 4 GiB ring, "
                "at least 100 and at least 1 GiB of regions per graph (so no launch finds its bytes in the 256 MB "
                "MALL), captured in one graph and replayed 5 times; best grid of 256-2048 blocks.\n\n| MB per launch | us per launch | blocks | GB/s |\n|---|---|---|---|\n")
        for mb, v in d["launch_floor"].items():
            f.write(f"| {mb} | {v['us_per_launch']} | {v['blocks']} | {v['GBps']} |\n")
        f.write("\nEmpty kernels back to back in a graph, us per launch (by blocks of 64 threads): "
                f"{d['empty_kernel_us_in_graph']}.\n\n")
        f.write("In-kernel all-to-all exchange (cooperative launch, blocks of 256 threads, 2000 rounds; each round "
                "every block publishes a 64-bit word with a device-scope store and waits until every block's word "
                "of the round is visible through device-scope loads):\n\n| blocks | us per round | completed |\n"
                "|---|---|---|\n")
        for b, v in d["exchange_all_to_all"].items():
            f.write(f"| {b} | {v.get('us_per_round', '-')} | {v.get('completed', v.get('error'))} |\n")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_leg(args, wl, cfg, layers, xs, resid, ws, L, T):
    """The f64 oracle on the host cores, on the same inputs as one GPU step.

    One eager step on the GPU records every layer's input and FFN output (the chained stack: the running
    residual before and after the layer).  The oracle then recomputes each layer from the GPU's own input:
    that gives the parity figures (max row relative error of the FFN delta, ids bit-exact up to certified
    near-ties) and the timing.  Timing: one thread over the whole step (every layer, every token), and
    N threads running the same work concurrently (N sequences, one per thread), median of 3 each.  Where a
    whole step would take longer than the budget, a token sample of every layer is run and scaled."""
    import concurrent.futures as cf

    import numpy as np
    import torch

    import moe_synth as S
    import oracle as O
    import sparse_moe_ffn_topk_amd as moe

    ocfg = O.make_cfg(wl.hidden, wl.n_experts, wl.top_k, wl.expert_ff, wl.shared_ff, wl.qtype, wl.n_groups,
                      wl.groups_used, wl.weights_scale, swiglu_limit=wl.swiglu_limit,
                      swiglu_limit_shared=wl.swiglu_limit_shared, norm_eps=float(np.float32(wl.norm_eps or 1e-5)))
    # one eager step on the GPU, layer by layer, inputs and outputs kept
    k = max(wl.top_k, 1)
    ids_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    h = S.make_x(wl, T, layer=0, step=0, device="cuda") if args.chained else resid.clone()  # (the step's input)
    rec = []
    for l in range(L):
        if args.chained:
            x_in = h.cpu().numpy().copy()
            moe.layer_step(cfg, layers[l], h, h, ids_d, wts_d, workspace=ws)
            torch.cuda.synchronize()
            rec.append((x_in, h.cpu().numpy() - x_in, ids_d.cpu().numpy().copy()))
        else:
            x_l = xs[0][l]
            out = torch.zeros_like(x_l)
            moe.layer_step(cfg, layers[l], x_l, out, ids_d, wts_d, workspace=ws)
            torch.cuda.synchronize()
            rec.append((x_l.cpu().numpy(), out.cpu().numpy(), ids_d.cpu().numpy().copy()))
    t_copy = time.perf_counter()
    host = [S.to_numpy(w) for w in layers]
    log(f"cpu leg: {L} layers copied to the host in {time.perf_counter() - t_copy:.1f}s")

    # tokens per layer: all of them unless one thread would exceed the budget
    t0 = time.perf_counter()
    O.layer(ocfg, host[0], rec[0][0][:1])
    per_tl = time.perf_counter() - t0
    n_tok = max(1, min(T, int(args.cpu_seconds / 4 / (per_tl * L))))
    rows = np.unique(np.linspace(0, T - 1, n_tok).round().astype(int))
    n_tok = len(rows)

    def one_pass():
        res = []
        for l in range(L):
            res.append(O.layer(ocfg, host[l], rec[l][0][rows]))
        return res

    t1s, results = [], None
    for rep in range(3):
        c0 = time.perf_counter()
        results = one_pass()
        t1s.append(time.perf_counter() - c0)
        if t1s[-1] > args.cpu_seconds / 3:
            break
    t1 = sorted(t1s)[len(t1s) // 2]
    N = max(1, min(16, os.cpu_count() or 1))
    tNs = []
    for rep in range(3):
        c0 = time.perf_counter()
        with cf.ThreadPoolExecutor(N) as ex:
            list(ex.map(lambda _: one_pass(), range(N)))
        tNs.append(time.perf_counter() - c0)
        if tNs[-1] > args.cpu_seconds / 3:
            break
    tN = sorted(tNs)[len(tNs) // 2]
    scale = T / n_tok
    oracle_1t_s = t1 * scale                    # one full step (T tokens, L layers) on one thread
    oracle_Nt_s = tN * scale / N                # the same, amortised over N concurrent sequences
    cpu = {"value": round(T / oracle_Nt_s, 4), "unit": "tokens/s", "cores": N, "kind": "oracle",
           "sample": (f"one full step ({L} layers x {T} tokens)" if n_tok == T else
                      f"{n_tok} of the {T} tokens of every layer ({L} layers), scaled x{scale:g}")
                     + f"; 1 thread and {N} threads each running that work concurrently, median of "
                       f"{len(t1s)} / {len(tNs)}",
           "value_1thread": round(T / oracle_1t_s, 4), "oracle_1t_s": round(oracle_1t_s, 4),
           "oracle_Nt_s": round(oracle_Nt_s, 4), "N": N, "cpu": cpu_model()}
    log(f"cpu baseline: 1 thread {oracle_1t_s:.3f} s per step ({cpu['value_1thread']} tok/s), {N} threads "
        f"{cpu['value']} tok/s; {cpu['cpu']}")

    # parity of the GPU step against the oracle, layer by layer on the GPU's own inputs
    worst, mism, ties = 0.0, 0, 0
    for l in range(L):
        ref, ids_ref, _ = results[l]
        x_in, delta, ids_g = rec[l]
        x_in, delta, ids_g = x_in[rows], delta[rows], ids_g[rows]
        ref_delta = ref  # (the oracle ran without a residual: its output is the FFN delta)
        for i in range(len(rows)):
            if wl.top_k > 0 and not np.array_equal(ids_g[i], ids_ref[i]):
                mism += 1
                xn = O.rmsnorm(x_in[i], host[l]["ffn_norm"], ocfg.norm_eps) if args.chained else x_in[i]
                sc = 1.0 / (1.0 + np.exp(-O.router_logits(host[l]["router_w"], xn)))
                if host[l].get("bias") is not None:
                    sc = sc + host[l]["bias"].astype(np.float64)
                dis = sorted(set(ids_g[i].tolist()) ^ set(ids_ref[i].tolist())) or \
                    [int(a) for a, b in zip(ids_g[i], ids_ref[i]) if a != b]
                if max(sc[dis]) - min(sc[dis]) < 1e-6:
                    ties += 1
                continue  # (the output under another routing is not comparable)
            e = np.abs(delta[i] - ref_delta[i]).max() / max(np.abs(ref_delta[i]).max(), 1e-300)
            if l in (0, L - 1) and i == 0:
                log(f"parity layer {l}: |x| {np.abs(x_in[i]).max():.4g}, |gpu delta| {np.abs(delta[i]).max():.4g}, "
                    f"|oracle delta| {np.abs(ref_delta[i]).max():.4g}, row rel err {e:.3g}")
            worst = max(worst, float(e))
    parity = {"max_rel_err": float(f"{worst:.3e}"), "ids_match": mism == 0, "ids_mismatch_tokens": mism,
              "near_ties": ties, "checked": f"{L} layers x {n_tok} tokens, each layer on the GPU's own input"}
    log(f"parity vs oracle: {parity}")
    return cpu, parity


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
    ap.add_argument("--probe", action="store_true",
                    help="only run the chip probes (streaming rate, per-launch floor, kernel boundary, in-kernel "
                         "exchange) and print them as one JSON line")
    ap.add_argument("--probe-out", help="with --probe: also write this markdown summary (e.g. profiles/...)")
    ap.add_argument("--no-stream-peak", action="store_true", help="skip the measured streaming peak")
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
    if args.probe:
        run_probes(args)
        return
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
        # every layer carries its pre-FFN RMSNorm weight; Q4_1 offsets are centred (m = -c d, c ~ U(7, 8)):
        # with all-positive weights (m ~ U(0.001, 0.02)) every layer's output shares one sign across h, the
        # residual turns into a constant vector, and after a few layers each gate pre-activation is about
        # -170 (every FFN output underflows to 0) or +170 (the residual grows without bound)
        wl = dataclasses.replace(wl, norm_eps=1e-5, centred=True)
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
            if name == dominant[1]:
                # the same launches timed with the events in stream order (no drain): the interval then also holds
                # the wait for the previous kernel's end and the dispatch after it
                with moe.KernelTimer(kid, 2 * nk * L, drain=False) as kd:
                    for i in range(nk):
                        stacks[i % nS].step()
                    torch.cuda.synchronize()
                kstats[name]["mean_us_in_stream"] = kd.mean_us
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
                    "mean_launch_source": "HIP events attached to every dispatch of the kernel in eager steps, "
                                          "each from an idle queue (dispatch latency included)",
                    "mean_launch_us_in_stream": round(kstats["group_gateup"]["mean_us_in_stream"], 3),
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
                    "mean_launch_us": round(kstats["gateup_swiglu"]["mean_us"], 3),
                    "mean_launch_source": "HIP events attached to every dispatch of the kernel in eager steps, "
                                          "each from an idle queue (dispatch latency included)",
                    "mean_launch_us_in_stream": round(kstats["gateup_swiglu"]["mean_us_in_stream"], 3)}

    peak = None
    if not args.no_stream_peak:
        peak, _ = stream_peak(moe, torch)
        log(f"measured streaming peak (4 GiB, 16-byte loads): {peak:.1f} GB/s")

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_leg(args, wl, cfg, layers, xs, resid, ws, L, T)

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
        "roofline": roofline, "cpu_baseline": cpu, "parity": parity,
        "measured_peak_GBps": None if peak is None else round(peak, 1),
        "pct_measured_peak": None if peak is None else round(100 * gbps / peak, 2),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
