"""Static FP8 activation quantisation on the GPU (hy3moe_quantize_e4m3),
bit-exact against the oracle's quantiser: ties between neighbouring codes
and a float32 ulp either side of them, subnormals, saturation, signed zeros,
random values over 27 binades, bf16 and float32 inputs, and an element count
that leaves a tail for the scalar kernel."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_amd as sm
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sm.load()
    return torch.device("cuda:0")


def crafted(rng) -> np.ndarray:
    """float32 values whose quotient by 1 hits every decision of the quantiser."""
    codes = np.array([c for c in range(0x7F)], dtype=np.uint8)   # +0 .. 448
    v = oracle.fp8_e4m3_value(codes)
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    parts = [v.astype(np.float32), mid,
             np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0)),
             np.array([448.0, 464.0, 464.5, 500.0, 1e6, 3e38, 2.0 ** -10, 2.0 ** -12,
                       1e-30, 0.0], dtype=np.float32)]
    pos = np.concatenate(parts)
    mag = np.exp2(rng.uniform(-16, 11, 50_000)).astype(np.float32)
    allv = np.concatenate([pos, -pos, mag, -mag, np.array([-0.0], np.float32)])
    return allv


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_e4m3_matches_oracle_bit_exact(dev, dtype):
    rng = np.random.default_rng(11)
    v32 = crafted(rng)
    if dtype == "bf16":
        xt = torch.from_numpy(v32).to(torch.bfloat16)
        v_exact = xt.float().numpy()          # the bf16 values the kernel sees
    else:
        xt = torch.from_numpy(v32)
        v_exact = v32
    n = v_exact.size
    assert n % 8 != 0                         # exercises the tail kernel too
    for s in (1.0, 4.5 / 448, 0.37, 3.0e-3):
        scale = torch.tensor([s], dtype=torch.float32, device=dev)
        q = torch.empty(n, dtype=torch.uint8, device=dev)
        sm.hy3moe_quantize_e4m3(xt.to(dev), scale, q)
        torch.cuda.synchronize()
        got = q.cpu().numpy()
        ref = oracle.quant_e4m3(v_exact.astype(np.float64), s)
        bad = np.nonzero(got != ref)[0]
        log(f"  quantize {dtype} scale {s:g}: n={n} mismatches={bad.size}")
        assert bad.size == 0, (f"first mismatches at {bad[:5]}: x={v_exact[bad[:5]]} "
                               f"got={got[bad[:5]]} ref={ref[bad[:5]]}")


def test_quantize_e4m3_empty_and_errors(dev):
    scale = torch.ones(1, dtype=torch.float32, device=dev)
    x = torch.zeros(0, dtype=torch.bfloat16, device=dev)
    q = torch.zeros(0, dtype=torch.uint8, device=dev)
    sm.hy3moe_quantize_e4m3(x, scale, q)      # n == 0: no-op
    lib = sm.load()
    assert lib.hy3moe_quantize_e4m3(None, 1, 8, scale.data_ptr(), None, None) == -1
    assert lib.hy3moe_quantize_e4m3(None, 7, 0, None, None, None) == -1
    assert lib.hy3moe_quantize_e4m3(None, 1, -1, None, None, None) == -1
