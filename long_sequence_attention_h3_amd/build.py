"""Build libh3attn.so (gfx950) in-tree with hipcc.

Usage: ``python -m long_sequence_attention_h3_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libh3attn.so")
SOURCES = [os.path.join(CSRC, "h3attn.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("common.hpp", "prologue.hpp", "attention.hpp",
                                                "attention_fp8.hpp", "block.hpp")] + [
    os.path.join(ROOT, "include", "h3attn.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every HIP source into ``out``; always recompiles."""
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, *(extra or []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
