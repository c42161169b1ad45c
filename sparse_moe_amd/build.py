"""Build libhy3moe.so (HIP, gfx950) in-tree with hipcc.

Usage:  python -m sparse_moe_amd.build   (or __graft_entry__.build())
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB_NAME = "libhy3moe.so"
LIB_PATH = os.path.join(LIB_DIR, LIB_NAME)
# Roofline ceiling probes (dense MFMA microkernel, device copy): a separate
# measurement library, not part of the MoE layer's C ABI.
PROBE_SOURCE = "ceiling_probe.hip"
PROBE_PATH = os.path.join(LIB_DIR, "libhy3moe_probe.so")

SOURCES = [
    "hy3moe_api.hip",
    "k_router.hip",
    "k_select.hip",
    "k_permute.hip",
    "k_expert_skinny.hip",
    "k_expert_tiled.hip",
    "k_expert_big.hip",
    "k_combine.hip",
    "k_quant.hip",
    "k_attention.hip",
]

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-result", "-ffp-contract=fast",
    # Keep the compiler from emitting packed-FP32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every kernel source for gfx950 and link libhy3moe.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max(1, min(jobs, len(cmds)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    ptmp = PROBE_PATH + ".tmp"
    _run([hipcc, *CFLAGS, "-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", ptmp], verbose)
    os.replace(ptmp, PROBE_PATH)
    return LIB_PATH


if __name__ == "__main__":
    p = build(verbose="-v" in sys.argv)
    print("built", p)
