"""hy3moe_forward_static (no allocation: the library's static per-GPU
scratch) against hy3moe_forward with a caller workspace, through the C ABI:
two calls in a row, the second with a smaller batch, each checked bit for
bit against the workspace entry point and within the layer's bounds against
the float64 oracle."""
import pytest
import torch

import oracle
import sparse_moe_amd as sm
from gpu_util import (check_output, check_route, config_of, expert_cache, log, oracle_route,
                      out_to_np, route_for_reference, shared_f64, to_torch, upload_weights)
from synth import random_small

pytestmark = pytest.mark.gpu


def test_static_forward_matches_workspace_forward_on_two_calls():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    sm.load()
    base = random_small(41, T=48, H=512, E=32, K=8, I=256, I_shared=256, dtype="bf16")
    w = upload_weights(base, dev)
    for T in (48, 9):              # the second call: a smaller batch on the same array
        inp = random_small(41, T=T, H=512, E=32, K=8, I=256, I_shared=256, dtype="bf16")
        c = inp.cfg
        log(f"static forward T={T}")
        cfg = config_of(inp)
        x = to_torch(inp.x(), "bf16", dev)
        ref = torch.empty_like(x)
        ws = sm.alloc_workspace(cfg, True, dev)
        sm.hy3moe_forward(cfg, x, w, ref, ws)
        out = torch.full_like(x, float("nan"))
        idx = torch.full((T, c.K), -1, dtype=torch.int32, device=dev)
        wt = torch.zeros((T, c.K), dtype=torch.float32, device=dev)
        sm.hy3moe_forward_static(cfg, x, w, out, idx, wt)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"T={T}"
        r = oracle_route(inp)
        gidx, gw = idx.cpu().numpy(), wt.cpu().numpy()
        check_route(gidx, gw, r)
        ridx, rw = route_for_reference(r, gidx)
        want = oracle.forward_given_route(inp.x_f64(), ridx, rw, expert_cache(inp), c.E,
                                          shared_f64(inp))
        check_output(out_to_np(out), want, "bf16", f"static T={T}")
