"""Ahead-of-time build of libwkv6.so for gfx950 with hipcc.

``python -m linear_attention_rnn_amd.build`` compiles the HIP kernels and the
C ABI layer into ``linear_attention_rnn_amd/libwkv6.so`` (in-tree, so it
travels with the source tree).  The build always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libwkv6.so")
SOURCES = ["wkv6_kernels.hip", "wkv6_backward.hip", "wkv6_backward_chunked.hip", "wkv4_kernels.hip", "wkv6_groupnorm.hip", "wkv6_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the WKV-6 library needs ROCm's hipcc to build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def build(verbose: bool = False) -> str:
    """Compile libwkv6.so; returns its path.  Raises on failure.  Each source
    compiles to its own object in parallel, then one link step."""
    tmp = LIB + ".tmp"
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        # packed fp32 VALU instructions stay off: plain scalar fp32 code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]
    noise = "is not a recognized feature for this target"
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        procs.append((src, _run([hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj], verbose)))
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        msgs = "\n".join(l for l in out.splitlines() if noise not in l)
        if pr.returncode != 0:
            failed.append(f"{src} ({pr.returncode}):\n{msgs}")
        elif msgs.strip() and verbose:
            print(msgs, flush=True)
    if failed:
        raise RuntimeError("hipcc failed: " + "\n".join(failed))
    link = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    out, _ = link.communicate()
    if link.returncode != 0:
        raise RuntimeError(f"link failed ({link.returncode}):\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
