"""Build the gfx950 HIP library libmoe_q4.so in-tree with hipcc.

Each source is compiled to an object in parallel (objects go to _build/,
which is not committed), then linked into sparse_moe_ffn_topk_amd/libmoe_q4.so.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe_q4.so")
OBJDIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         # packed-FP32 instructions stay off (plain FP32 VALU only)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _clean(stderr):
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def build(verbose=False):
    """Always recompile every kernel for gfx950 into sparse_moe_ffn_topk_amd/libmoe_q4.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    procs = []
    for src in sources():
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    objs, errs = [], []
    for src, obj, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            errs.append(f"{src}:\n{_clean(err)}")
        elif verbose and _clean(err).strip():
            print(_clean(err), file=sys.stderr)
        objs.append(obj)
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{_clean(r.stderr)}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
