"""Build libaveris.so (gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed fp32 VALU instructions disabled
and floating-point contraction off (the quantizer's fp32 steps must round once each).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libaveris.so")
SOURCES = ["quant.hip", "gemm.hip", "producers.hip", "api.hip"]
HEADERS = ["common.h", "launch.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def source_digest() -> str:
    """SHA-1 (hex) of every file the library is built from (sources, headers, the public header
    and this build script's flags).  It is compiled into the library, so a loader can tell a
    library built from other sources."""
    import hashlib
    h = hashlib.sha1()
    h.update(" ".join(FLAGS[:-4]).encode())
    for f in [os.path.join(CSRC, s) for s in SOURCES + HEADERS] + [os.path.join(ROOT, "include", "averis.h")]:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    """Compile every source to an object, link libaveris.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]
    digest = [f'-DAVERIS_SOURCE_DIGEST="{source_digest()}"']
    cmds = [[HIPCC, *FLAGS, *(digest if s == "api.hip" else []), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))


def gemm_source_digest():
    """SHA-1 (hex) of the GEMM sources (gemm.hip, common.h) with // comments and blank lines
    removed: it changes when the compiled code can, not when a comment does.  bench.py pairs it
    with the committed HBM-traffic counters of the GEMM."""
    import hashlib
    h = hashlib.sha1()
    for f in ("gemm.hip", "common.h"):
        with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()
