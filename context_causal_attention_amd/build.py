"""Builds libcpattn.so (host index builder, C-ABI layer and gfx950 HIP kernels)
in-tree with hipcc.  ``python -m context_causal_attention_amd.build``."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcpattn.so")
# Unit-throughput probes for the measurement harness (bench.py --pass probe);
# not part of the C ABI.
PROBE_LIB = os.path.join(PKG, "libcpattn_probe.so")
PROBE_SOURCES = ["probe.hip"]

ARCH = "gfx950"
SOURCES = ["index.cpp", "api.cpp", "attn_fwd.hip", "attn_bwd.hip", "merge.hip", "a2a.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed fp32 VALU forms stay off in every device compile.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libcpattn.so")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE]
    if src.endswith(".hip"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libcpattn.so failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    pobjs = [_compile(s, verbose) for s in PROBE_SOURCES]
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", PROBE_LIB + ".tmp", *pobjs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libcpattn_probe.so failed:\n{r.stdout}{r.stderr}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
