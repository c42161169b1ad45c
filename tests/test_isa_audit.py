"""Audit of the gfx950 assembly the kernels compile to (CPU only, needs hipcc).

An MFMA is a whole-wavefront operation: it does not honour a per-lane EXEC
mask, so an MFMA placed under `s_and_saveexec` (a divergent branch the
compiler expects to switch lanes off) still runs and adds its products.  The
kernels keep every MFMA out of such regions by making the guards provably
wave-uniform; this test checks the generated code, and that no kernel spills
to scratch memory.
"""
import os
import re
import shutil
import subprocess

import pytest

from sparse_moe_amd import build as B

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")

KERNEL_SOURCES = ["k_router.hip", "k_expert_skinny.hip", "k_expert_tiled.hip",
                  "k_expert_big.hip", "k_select.hip", "k_permute.hip", "k_combine.hip",
                  "k_quant.hip", "k_attention.hip"]


def assemble(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, *[f for f in B.CFLAGS if f not in ("-fPIC",)], "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return out.read_text()


def masked_mfmas(asm):
    """MFMAs that sit inside an s_and_saveexec ... s_or_b64 exec region."""
    depth, bad, kernel = 0, [], None
    for line in asm.splitlines():
        s = line.strip()
        if re.match(r"^_Z\S*:", s):
            kernel, depth = s.split(":")[0], 0
        elif s.startswith("s_endpgm"):
            depth = 0
        elif s.startswith(("s_or_saveexec", "s_andn2_saveexec")):
            pass        # the else half of an if/else region: same nesting level
        elif "saveexec" in s:
            depth += 1
        elif s.startswith("s_or_b64 exec, exec") and depth:
            depth -= 1
        elif depth and s.startswith("v_mfma"):
            bad.append((kernel, s))
    return bad


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_mfma_under_exec_mask_and_no_scratch(src, tmp_path):
    asm = assemble(src, tmp_path)
    assert not masked_mfmas(asm), masked_mfmas(asm)[:3]
    if src != "k_expert_big.hip":   # its fp32 (test-only) variant may spill
        scratch = [int(v) for v in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)]
        assert all(v == 0 for v in scratch), scratch


def test_large_tile_bf16_kernels_do_not_spill(tmp_path):
    asm = assemble("k_expert_big.hip", tmp_path)
    pairs = re.findall(r"\.name:\s+(\S+)\s+\.private_segment_fixed_size:\s+(\d+)", asm)
    bf16 = [(n, int(v)) for n, v in pairs if "expert_big_kernelINS_6bf16_t" in n]
    # gate-up and down with bf16, FP8 and MXFP4 weights, and FP8 weights with
    # FP8 activations, each for the routed and the shared expert's launches
    # (template <T, GATE_UP, weight format, A8, BRANCH>)
    assert len(bf16) == 16
    tight = [(n, v) for n, v in bf16 if re.search(r"Li[01]ELb0ELi[01]EEEv", n)]
    assert len(tight) == 8
    assert all(v == 0 for _, v in tight), tight
    # the MXFP4 and FP8-MFMA variants keep a few registers of tile bookkeeping
    # in scratch (outside the K loop)
    assert all(v <= 32 for _, v in bf16), bf16
