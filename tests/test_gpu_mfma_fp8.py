"""Accumulation error of the FP8 MFMA (v_mfma_f32_16x16x128_f8f6f4, E4M3 x
E4M3) that the W8A8 large-tile GEMMs use, measured against exact float64
sums of the same products (the measurement library's one-instruction probe).

The instruction does not sum its 128 products to float32 precision (bf16
16x16x32 does, within about one ulp).  The bounds asserted here are the
ones the W8A8 tests use for a GEMM's float32 result: 1024 ulps (2^-23) of
the sum of |products| of one instruction for the layer's operand
distributions, 8192 for operands spread over the whole E4M3 range.

The block-scaled FP4 x FP8 form of the same instruction (the W4A8 GEMMs) is
checked for the operand layout and scale grouping those kernels assume."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import log
from sparse_moe_amd.build import PROBE_PATH
from synth.inputs import _fp8_codes

pytestmark = pytest.mark.gpu

N_INST = 2048


@pytest.fixture(scope="module")
def probe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L = ctypes.CDLL(PROBE_PATH)
    L.hy3moe_probe_mfma_fp8_once.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return L


def run_once(L, a_codes, b_codes):
    dev = torch.device("cuda:0")
    a = torch.from_numpy(a_codes.reshape(-1)).to(dev)
    b = torch.from_numpy(b_codes.reshape(-1)).to(dev)
    d = torch.empty(N_INST * 64 * 4, dtype=torch.float32, device=dev)
    rc = L.hy3moe_probe_mfma_fp8_once(a.data_ptr(), b.data_ptr(), d.data_ptr(), N_INST,
                                      torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    # lane 16 c + r holds rows 4 c + q of column r
    d = d.cpu().numpy().astype(np.float64).reshape(N_INST, 4, 16, 4)   # [n, c, r, q]
    return d.transpose(0, 1, 3, 2).reshape(N_INST, 16, 16)              # [n, row, col]


def exact(a_codes, b_codes):
    va = oracle.fp8_e4m3_value(a_codes).reshape(N_INST, 4, 16, 32)      # [n, g, row, t]
    vb = oracle.fp8_e4m3_value(b_codes).reshape(N_INST, 4, 16, 32)      # [n, g, col, t]
    s = np.einsum("ngit,ngjt->nij", va, vb)
    sa = np.einsum("ngit,ngjt->nij", np.abs(va), np.abs(vb))
    return s, sa


def ulps_of_abs_sum(L, a_codes, b_codes):
    got = run_once(L, a_codes, b_codes)
    s, sa = exact(a_codes, b_codes)
    return np.abs(got - s) / (2.0 ** -23 * np.maximum(sa, 1e-300))


def test_fp8_mfma_error_layer_operands(probe):
    """x ~ N(0, 1) quantised with the layer's static scale against the
    synthetic FP8 weight codes."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal(N_INST * 64 * 32)
    a = oracle.quant_e4m3(x, 4.5 / 448).reshape(N_INST * 64, 32)
    b = _fp8_codes(rng, (N_INST * 64, 32))
    e = ulps_of_abs_sum(probe, a, b)
    log(f"  layer operands: error / (2^-23 sum|p|): median {np.median(e):.3g} "
        f"p99 {np.quantile(e, 0.99):.3g} max {e.max():.3g}")
    assert e.max() <= 1024


def test_fp8_mfma_error_full_range(probe):
    """Codes uniform over all finite E4M3 values (products spanning 2^-18..2^17)."""
    rng = np.random.default_rng(4)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    a = rng.choice(finite, size=(N_INST * 64, 32))
    b = rng.choice(finite, size=(N_INST * 64, 32))
    e = ulps_of_abs_sum(probe, a, b)
    log(f"  full-range operands: error / (2^-23 sum|p|): median {np.median(e):.3g} "
        f"p99 {np.quantile(e, 0.99):.3g} max {e.max():.3g}")
    assert e.max() <= 8192


def _a_position(g, p):
    """Measured K position (in B's byte order, B lane group g' byte q = 32 g'
    + q) of FP4 element p of A lane group g in the block-scaled 16x16x128
    MFMA: two runs of 16."""
    return 32 * (2 * (g & 1) + (p >> 4)) + 16 * (g >> 1) + (p & 15)


def test_fp4_fp8_block_scaled_mfma_layout(probe):
    """The operand layout and scale grouping the W4A8 kernels rely on: A lane
    group g's 32 FP4 values sit at K positions _a_position(g, p) of B's
    order, and the E8M0 scale of lane group c -- on the A and on the B side
    -- applies to exactly A lane group c's positions.  Checked against exact
    sums on random codes with random scales."""
    L = probe
    L.hy3moe_probe_mfma_fp4fp8_once.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int,
                                                                       ctypes.c_void_p]
    n = 256
    rng = np.random.default_rng(9)
    a = np.zeros((n, 64, 32), dtype=np.uint8)
    a[:, :, :16] = rng.integers(0, 256, (n, 64, 16), dtype=np.uint8)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    b = rng.choice(finite, size=(n, 64, 32))
    sa = rng.integers(118, 136, (n, 64)).astype(np.int32)
    sb = rng.integers(118, 136, (n, 64)).astype(np.int32)
    dev = torch.device("cuda:0")
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    tsa, tsb = torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev)
    d = torch.empty(n * 64 * 4, dtype=torch.float32, device=dev)
    assert L.hy3moe_probe_mfma_fp4fp8_once(ta.data_ptr(), tb.data_ptr(), tsa.data_ptr(),
                                           tsb.data_ptr(), d.data_ptr(), n,
                                           torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    got = d.cpu().numpy().astype(np.float64).reshape(n, 4, 16, 4).transpose(0, 1, 3, 2)
    got = got.reshape(n, 16, 16)
    nib = np.empty((n, 64, 32), dtype=np.int64)
    nib[:, :, 0::2] = a[:, :, :16] & 15
    nib[:, :, 1::2] = a[:, :, :16] >> 4
    va = oracle.fp4_e2m1_value(nib).reshape(n, 4, 16, 32)           # [n, g, row, p]
    vb = oracle.fp8_e4m3_value(b).reshape(n, 4, 16, 32)             # [n, g', col, q]
    ea = oracle.e8m0_value(sa.astype(np.uint8)).reshape(n, 4, 16)    # [n, c, row]
    eb = oracle.e8m0_value(sb.astype(np.uint8)).reshape(n, 4, 16)    # [n, c, col]
    ref = np.zeros((n, 16, 16))
    for g in range(4):
        for p in range(32):
            k = _a_position(g, p)
            bk = vb[:, k // 32, :, k % 32]                             # [n, col]
            ref += (ea[:, g, :, None] * va[:, g, :, p][:, :, None]) * (eb[:, g, None, :] * bk[:, None, :])
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    log(f"  block-scaled FP4 x FP8 MFMA vs the measured layout: rel-L2 {rel:.3g}")
    assert rel < 1e-3
