"""Compile the HIP library ``libfa92.so`` for gfx950, in-tree.

Run ``python -m exact_attention_92_amd.build`` (or ``__graft_entry__.build()``).
hipcc cross-compiles on a machine without a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f)
        for f in ("fa_fwd.hip", "fa_bwd.hip", "fa_bwd_d64.hip", "fa_fwd_fp8.hip", "fa_decode.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa92.so")
ARCH = "gfx950"

# Packed fp32 VALU ops are switched off for every HIP source.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source additions.  The forward kernels keep their MFMA results in
# ordinary VGPRs: left to its own choice the compiler moves the d = 256
# kernel's accumulators into AGPRs and copies them back on every block
# (425 -> 732 TFLOP/s at d = 256; the d <= 128 kernels never need AGPRs and
# are unchanged).  The backward kernels too: bitwise-identical gradients,
# +4-6% on causal N = 1024 (whose 4-wave dQ kernel otherwise parks values in
# AGPRs), unchanged on the larger shapes.
SRC_FLAGS = {"fa_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
             "fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
             "fa_bwd_d64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


# The d = 128 forward's block loop is an inline-asm program written by a
# generator beside the sources (its output is not kept in version control).
GENERATORS = [os.path.join(PKG, "csrc", "gen_fwd_d128_loop.py")]


def build(verbose: bool = False) -> str:
    """Write the generated kernel bodies, compile libfa92.so (always
    recompiles) and return its path."""
    for gen in GENERATORS:
        if verbose:
            print(f"{sys.executable} {gen}", flush=True)
        res = subprocess.run([sys.executable, gen], capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"{os.path.basename(gen)} failed:\n{res.stdout}{res.stderr}")
    tmp = LIB + ".tmp"
    objs = []
    for src in SRCS:
        obj = os.path.join(PKG, "csrc", os.path.basename(src) + ".o")
        extra = SRC_FLAGS.get(os.path.basename(src), [])
        _run([hipcc(), *HIPCC_FLAGS, *extra, f"-I{INCLUDE}", "-c", src, "-o", obj], verbose)
        objs.append(obj)
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    for obj in objs:
        os.remove(obj)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
