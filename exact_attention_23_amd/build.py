"""Compile libfa.so (the HIP kernels and the C ABI) for gfx950, in-tree, and
libfa_probe.so, the vector-rate probe the benchmark uses.

    python -m exact_attention_23_amd.build

hipcc cross-compiles without a GPU present. Every HIP file is built with
packed-fp32 instructions disabled (-Xclang -target-feature -Xclang
-packed-fp32-ops); hipcc's host pass warns that it does not know that
feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libfa_probe.so")
ARCH = "gfx950"
SOURCES = [os.path.join(CSRC, f) for f in ("fa_lib.hip", "fa_api.hip", "fa_bwd.hip", "fa_fp8.hip",
                                           "fa_std.hip")]
PROBE_SOURCES = [os.path.join(CSRC, "fa_probe.hip")]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(sources, out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-o", tmp] + sources
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in r.stdout.splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libfa.so (and the probe into
    libfa_probe.so) next to this file; return the path of libfa.so."""
    _compile(PROBE_SOURCES, PROBE_LIB_PATH, verbose)
    return _compile(SOURCES, LIB_PATH, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
