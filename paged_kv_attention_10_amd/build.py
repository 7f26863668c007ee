"""Compile the pkv HIP library (libpkv.so) for gfx950, in place, and the
measurement-only streaming-read probe (libpkv_probe.so) the benchmark uses
for its practical-ceiling line."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["api.hip", "append.hip", "decode.hip", "prefill.hip", "mixed.hip"]
LIB = os.path.join(HERE, "libpkv.so")
PROBE_SOURCES = ["probe.hip"]
PROBE_LIB = os.path.join(HERE, "libpkv_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(sources, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp] + [os.path.join(HERE, "csrc", s) for s in sources]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Build libpkv.so (and libpkv_probe.so) next to this file; returns the
    library's path."""
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
