"""The router weight's offline split (hy3moe_router_split, the Hy3 Preview
inference case's dual-BF16 router prepared once): the gate and the layer run
on caller-held planes give exactly the results of the per-call split, at the
router-only workload's M = 4096 and on a prefill-sized batch through the
forward, for both router arithmetics."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_amd as sm
from gpu_util import check_route, config_of, log, oracle_route, to_torch, upload_weights
from synth import CONFIGS, MoEInputs, random_small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sm.load()
    return torch.device("cuda:0")


@pytest.mark.parametrize("prec", [sm.HY3MOE_ROUTER_FP32, sm.HY3MOE_ROUTER_SPLIT2_BF16])
def test_route_on_offline_planes_matches_the_per_call_split(dev, prec):
    inp = MoEInputs(CONFIGS["hy3_router_only"].with_T(4096))
    c = inp.cfg
    cfg = config_of(inp, router_prec=prec)
    x = to_torch(inp.x(), c.dtype, dev)
    wr = torch.from_numpy(inp.w_router()).to(dev)
    bias = torch.from_numpy(inp.bias()).to(dev)
    planes = sm.router_split(wr, prec)
    torch.cuda.synchronize()
    L = sm.hy3moe_workspace_layout(cfg)
    assert L.w_planes, "M = 4096 runs the planes kernel"
    ws0, ws1 = sm.alloc_workspace(cfg, False, dev), sm.alloc_workspace(cfg, False, dev)
    i0, w0 = sm.route(cfg, x, wr, bias, workspace=ws0)
    i1, w1 = sm.route(cfg, x, wr, bias, workspace=ws1, w_router_planes=planes)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(i0.cpu().numpy(), i1.cpu().numpy())
    np.testing.assert_array_equal(w0.cpu().numpy(), w1.cpu().numpy())
    # the split the library made per call is the offline one, byte for byte
    n = planes.numel()
    assert torch.equal(ws0[L.w_planes:L.w_planes + n], planes)
    # and the logits: the same partial sums
    n_part = 8 * L.n_ksplit * c.T * c.E
    assert torch.equal(ws0[L.logits_part:L.logits_part + n_part],
                       ws1[L.logits_part:L.logits_part + n_part])
    if prec == sm.HY3MOE_ROUTER_FP32:
        check_route(i1.cpu().numpy(), w1.cpu().numpy(), oracle_route(inp))
    log(f"  prec {prec}: planes {n} bytes, route identical")


def test_forward_on_offline_planes_matches_the_per_call_split(dev):
    inp = random_small(44, T=1500, H=256, E=8, K=3, I=128, I_shared=128, dtype="bf16")
    cfg = config_of(inp)
    w = upload_weights(inp, dev)
    x = to_torch(inp.x(), "bf16", dev)
    ref = sm.forward(cfg, x, w)
    wp = dict(w, w_router_planes=sm.router_split(w["w_router"], sm.HY3MOE_ROUTER_FP32))
    got = sm.forward(cfg, x, wp)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
