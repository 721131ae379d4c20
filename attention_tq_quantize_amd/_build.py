"""Build libtq.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")
SOURCES = ["tq_capi.cpp", "tq_codebook.cpp", "tq_quantize.hip", "tq_aux.hip", "tq_decode.hip", "tq_large.hip", "tq_split_decode.hip"]
OBJDIR = os.path.join(os.path.dirname(HERE), "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, jobs: int = 8, force: bool = True) -> str:
    """Compile every source to an object (in parallel) and link libtq.so next to this file.
    force=False skips sources whose object is newer than every source and header."""
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        raise RuntimeError("hipcc not found; cannot build libtq.so")
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    procs = []
    objs = []
    newest_hdr = max(os.path.getmtime(os.path.join(CSRC, f)) for f in os.listdir(CSRC) if f.endswith(".h"))
    newest_hdr = max(newest_hdr, os.path.getmtime(os.path.join(os.path.dirname(HERE), "include", "tq.h")))
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        objs.append(obj)
        if not force and os.path.exists(obj):
            t = os.path.getmtime(obj)
            if t > os.path.getmtime(os.path.join(CSRC, src)) and t > newest_hdr:
                continue
        cmd = [hipcc] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        while sum(p.poll() is None for _, p in procs) >= jobs:
            procs[0][1].wait()
    failed = False
    for src, p in procs:
        out, _ = p.communicate()
        lines = [l for l in (out or "").splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"--- {src} ---\n" + "\n".join(lines) + "\n")
    if failed:
        raise RuntimeError("hipcc failed building libtq.so")
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libtq.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, force="--force" in sys.argv))
