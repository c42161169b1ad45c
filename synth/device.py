"""Upload of seeded synthetic inputs to GPU memory (plumbing only).

bf16 tensors travel as their raw 16-bit patterns and are reinterpreted as
torch.bfloat16 on the device; float32 tensors are copied as they are.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .inputs import MoEInputs


def to_torch(a: np.ndarray, dtype: str, device):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def upload_weights(inp: MoEInputs, device) -> Dict[str, object]:
    """Router weight, expert bias (if any), the stacked routed experts and the
    shared expert, each branch in its own weight format, plus the static FP8
    activation scales when a branch uses them."""
    import torch
    c = inp.cfg
    d = {"w_router": torch.from_numpy(inp.w_router()).to(device)}
    if c.w_format == "mxfp4":
        d.update(_routed_mxfp4(inp, device))
    elif c.w_format == "fp8_e4m3":
        d.update(_routed_fp8(inp, device))
    else:
        wg, wu, wd = inp.stacked_experts()
        d.update({"w_gate": to_torch(wg, c.dtype, device), "w_up": to_torch(wu, c.dtype, device),
                  "w_down": to_torch(wd, c.dtype, device)})
        del wg, wu, wd
    b = inp.bias()
    if b is not None:
        d["expert_bias"] = torch.from_numpy(b).to(device)
    if c.I_shared:
        d.update(_shared(inp, device))
    if "fp8_static" in (c.act_format, c.sa_format if c.I_shared else c.act_format):
        d = with_act_scales(inp, d, device)
    return d


def with_act_scales(inp: MoEInputs, weights: Dict[str, object], device) -> Dict[str, object]:
    """The weights plus the static FP8 activation scales (x_scale [1], h_scale [E+1])."""
    import torch
    w = dict(weights)
    a1, a2 = inp.act_scales()
    w["x_scale"] = torch.tensor([a1], dtype=torch.float32).to(device)
    w["h_scale"] = torch.from_numpy(a2).to(device)
    return w


def with_bias_of(inp: MoEInputs, weights: Dict[str, object], device) -> Dict[str, object]:
    """The same model weights with this workload's own expert bias (a data stream)."""
    import torch
    w = dict(weights)
    b = inp.bias()
    w["expert_bias"] = None if b is None else torch.from_numpy(b).to(device)
    return w


def _routed_mxfp4(inp: MoEInputs, device) -> Dict[str, object]:
    """MXFP4 routed experts: packed E2M1 codes (uint8) and E8M0 block scales (uint8)."""
    import torch
    wg, wu, wd, sg, su, sd = inp.stacked_experts_mxfp4()
    d = {}
    for k, a in (("w_gate", wg), ("w_up", wu), ("w_down", wd), ("w_gate_mx", sg),
                 ("w_up_mx", su), ("w_down_mx", sd)):
        d[k] = torch.from_numpy(a).to(device)
    return d


def _routed_fp8(inp: MoEInputs, device) -> Dict[str, object]:
    """FP8 E4M3 routed experts (uint8 codes) with their float32 scales."""
    import torch
    wg, wu, wd, sc = inp.stacked_experts_fp8()
    return {"w_gate": torch.from_numpy(wg).to(device), "w_up": torch.from_numpy(wu).to(device),
            "w_down": torch.from_numpy(wd).to(device),
            "w_gate_scale": torch.from_numpy(np.ascontiguousarray(sc[0])).to(device),
            "w_up_scale": torch.from_numpy(np.ascontiguousarray(sc[1])).to(device),
            "w_down_scale": torch.from_numpy(np.ascontiguousarray(sc[2])).to(device)}


def _shared(inp: MoEInputs, device) -> Dict[str, object]:
    """The shared expert in its weight format."""
    import torch
    c = inp.cfg
    d = {}
    if c.sw_format == "mxfp4":
        codes, scales = inp.shared_mxfp4()
        for k, a in zip(("ws_gate", "ws_up", "ws_down"), codes):
            d[k] = torch.from_numpy(a).to(device)
        for k, a in zip(("ws_gate_mx", "ws_up_mx", "ws_down_mx"), scales):
            d[k] = torch.from_numpy(a).to(device)
    elif c.sw_format == "fp8_e4m3":
        codes, scales = inp.shared_fp8()
        d["ws_gate"], d["ws_up"], d["ws_down"] = (torch.from_numpy(q).to(device) for q in codes)
        d["ws_scale"] = torch.from_numpy(np.array(scales, dtype=np.float32)).to(device)
    else:
        d["ws_gate"], d["ws_up"], d["ws_down"] = (to_torch(a, c.dtype, device)
                                                  for a in inp.shared())
    return d
