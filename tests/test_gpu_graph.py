"""The layer captured as a HIP graph: hy3moe_forward enqueues kernels only (no
memset, no host synchronisation, no allocation), so it can be captured once
and replayed.  Every replay, with eager work and synchronisation between the
replays, is checked against the float64 oracle (route indices and outputs,
by the same rules as the eager parity tests), and must also reproduce the
eager output bit for bit (the chain is deterministic)."""
import pytest
import torch

import oracle
import sparse_moe_amd as sm
from gpu_util import (check_output, check_route, config_of, expert_cache, log, oracle_route,
                      out_to_np, route_for_reference, shared_f64, to_torch, upload_weights)
from synth import random_small

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T, H, E, K, I", [
    (16, 512, 32, 4, 128),     # weight-streaming GEMMs, one-workgroup permutation
    (300, 256, 16, 4, 128),    # 128x128 tiles
    (1500, 256, 8, 3, 128),    # 256x256 tiles, three-kernel permutation, router planes
])
def test_graph_replays_match_oracle(T, H, E, K, I):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    inp = random_small(31, T=T, H=H, E=E, K=K, I=I, I_shared=I, dtype="bf16")
    c = inp.cfg
    log(f"graph case T={T} H={H} E={E} K={K} I={I}")
    cfg = config_of(inp)
    w = upload_weights(inp, dev)
    x = to_torch(inp.x(), "bf16", dev)
    ws = sm.alloc_workspace(cfg, True, dev)
    ref = torch.empty_like(x)
    sm.hy3moe_forward(cfg, x, w, ref, ws)
    torch.cuda.synchronize()

    out = torch.zeros_like(x)
    idx = torch.zeros((T, K), dtype=torch.int32, device=dev)
    wt = torch.zeros((T, K), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sm.hy3moe_forward(cfg, x, w, out, ws, idx, wt)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sm.hy3moe_forward(cfg, x, w, out, ws, idx, wt)

    r = oracle_route(inp)
    for rep in range(4):
        out.zero_()
        idx.zero_()
        wt.zero_()
        other = torch.empty_like(x)
        sm.hy3moe_forward(cfg, x, w, other, ws)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gidx, gw = idx.cpu().numpy(), wt.cpu().numpy()
        check_route(gidx, gw, r)
        ridx, rw = route_for_reference(r, gidx)
        want = oracle.forward_given_route(inp.x_f64(), ridx, rw, expert_cache(inp), c.E,
                                          shared_f64(inp))
        check_output(out_to_np(out), want, "bf16", f"replay {rep}")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16))
