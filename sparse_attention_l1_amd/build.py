"""Builds libhsastep.so (the HIP kernels for gfx950 and the C ABI) in-tree.

    python -m sparse_attention_l1_amd.build        # or build() from Python

Objects go to sparse_attention_l1_amd/_build/, the library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhsastep.so")

SOURCES = ["abi.cpp", "host.cpp", "score.hip", "rank.hip", "active.hip", "rows.hip", "euler.hip",
           "attn.hip", "attn_pipe.hip", "proj.hip", "mfma_probe.hip"]

ARCH = "gfx950"
# files whose fp32 results are specified to the bit: no multiply-add contraction
EXACT = ("score.hip", "euler.hip")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}", f"-I{BUILD}"]
# device code: gfx950 only; no packed-fp32 instructions (v_pk_{add,mul,fma}_f32)
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libhsastep")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON
    if src.endswith(".hip"):
        cmd += ["-x", "hip"] + DEVICE
    if src in EXACT:
        cmd += ["-ffp-contract=off"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    return obj


def generate_sources() -> None:
    """Writes the generated assembly loops into the build folder: the attention key loop
    (attn_loop.inc) and the projection's reduction loop (proj_loop.inc)."""
    sys.path.insert(0, CSRC)
    try:
        import attn_loop_gen
        import proj_loop_gen
    finally:
        sys.path.pop(0)
    attn_loop_gen.write(os.path.join(BUILD, "attn_loop.inc"))
    proj_loop_gen.write(os.path.join(BUILD, "proj_loop.inc"))


def build(verbose: bool = False) -> str:
    """Compiles every source and links the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    generate_sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libhsastep.so failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
