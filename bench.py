#!/usr/bin/env python3
"""Throughput of the Hy3-style MoE FFN layer on one MI355X.

One step = one hy3moe_forward (router GEMM, score + top-K select,
permutation, grouped gate-up + SwiGLU, grouped down, weighted combine) over
one batch of seeded synthetic input already resident in HBM.

Default workload: Hy3 decode, T=16 tokens, H=4096, 192 routed experts
(top-8) + 1 shared expert, I=1536, bf16 weights/activations, fp32 router.
`--workload prefill` (T=8192, skewed bias) and `--workload softmax`
(HunyuanImage-3.0 softmax routing, T=32768, E=64) run the other layer shapes;
`--workload decode_fp8` / `prefill_fp8` are the decode and prefill shapes with
FP8 E4M3 expert weights, `decode_w8a8` / `prefill_w8a8` the same with static
FP8 activations as well (FP8 MFMAs on the large-tile path, priced against the
FP8 peak); `_mxfp4` / `_w4a8` use MXFP4 experts (with dynamic MXFP8
activations for W4A8), and `_mixed` runs the routed experts at W4A8 and the
shared expert at W8A8 in one call.

Printed: one JSON line with tokens/s, the dominant kernel's roofline fraction
(its per-launch duration measured live with HIP events on the library's
stream, via hy3moe_forward_timed), the whole-layer fractions, and the CPU
oracle timed on a bounded sample on this host.  The default run (decode)
then times the prefill chunk on the same weights and adds it under
"prefill" with its own roofline (bf16 MFMA) and stage times; the headline
value stays the decode one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

WORKLOADS = {"decode": "hy3_decode_T16", "prefill": "hy3_prefill_T8192_skew", "softmax": "hunyuanimage_softmax_T32768", "decode_fp8": "hy3_decode_T16_fp8", "prefill_fp8": "hy3_prefill_T8192_skew_fp8",
             "decode_w8a8": "hy3_decode_T16_w8a8", "prefill_w8a8": "hy3_prefill_T8192_skew_w8a8", "decode_mxfp4": "hy3_decode_T16_mxfp4", "prefill_mxfp4": "hy3_prefill_T8192_skew_mxfp4",
             "decode_w4a8": "hy3_decode_T16_w4a8", "prefill_w4a8": "hy3_prefill_T8192_skew_w4a8",
             "decode_mixed": "hy3_decode_T16_mixed", "prefill_mixed": "hy3_prefill_T8192_skew_mixed",
             "decode_T32": "hy3_decode_T32", "decode_T32_w8a8": "hy3_decode_T32_w8a8",
             "decode_T64": "hy3_decode_T64"}
ROUTER_WORKLOAD = "hy3_router_only"            # the router-only configuration (gate alone, M tokens)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, published
METRIC = "Hy3 MoE layer tokens/s; % bf16 MFMA peak (prefill) / % HBM BW (decode)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


ATTN_SOURCES = ("k_attention.hip",)   # the split-KV attention path; the rest is the MoE layer's
PROBE_SOURCES = ("ceiling_probe.hip",)  # measurement probes: part of neither path


def kernel_sources_sha(kind: str = "moe"):
    """Hash of the kernel sources a measurement depends on: the MoE layer's
    (every source but the attention path's and the ceiling probes') or the
    attention path's."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name in PROBE_SOURCES or (name in ATTN_SOURCES) != (kind == "attn"):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when the
    kernel sources changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    kind = "attn" if workload.startswith("attn") else "moe"
    if d.get("kernel_sources_sha") != kernel_sources_sha(kind):
        return None
    return d.get("bytes_per_launch")


# Split-KV decode attention workloads (Hy3 GQA: 64 query / 8 KV heads,
# head_dim 128): (description, cached lengths) from seeded generators.
ATTN_WORKLOADS = {"attn_long": "one request, 131072 cached tokens",
                  "attn_mixed": "32 requests, lengths log-uniform in [512, 65536]"}
ATTN_WORKERS = 512


def attention_bench(args, dev):
    """Split + combine kernels of hy3attn_decode over the workload's batch:
    W warm-up and K timed calls between synchronizations; per-kernel times
    from HIP events recorded on the stream the kernels run on."""
    import numpy as np
    import torch
    import sparse_moe_amd as sm
    from synth.attention_inputs import attention_inputs, bits_to_f64, mixed_lengths
    kv_len = [131072] if args.workload == "attn_long" else mixed_lengths(5, 32, 512, 65536)
    hkv, d = 8, 128
    qb, kb, vb = attention_inputs(11, kv_len, hkv)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = bf(qb), bf(kb), bf(vb)
    plan = sm.attn_plan(kv_len, hkv, sm.ATTN_TILE, ATTN_WORKERS)
    out = torch.empty_like(q)
    L = sm.load()
    n_tasks = int(plan.tasks.shape[0])
    ws = torch.empty(int(L.hy3attn_workspace_bytes(n_tasks)) + 256, dtype=torch.uint8, device=dev)
    starts = np.zeros(len(kv_len) + 1, dtype=np.int32)
    starts[1:] = np.cumsum(kv_len)
    kv_start = torch.from_numpy(starts).to(dev)
    tasks = torch.from_numpy(plan.tasks.reshape(-1)).to(dev)
    wb = torch.from_numpy(plan.worker_begin).to(dev)
    rb = torch.from_numpy(plan.row_begin).to(dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        rc = L.hy3attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_start.data_ptr(),
                              len(kv_len), hkv, plan.tile, tasks.data_ptr(), n_tasks,
                              wb.data_ptr(), plan.n_workers, rb.data_ptr(),
                              plan.row_begin.size - 1, ws.data_ptr(), ws.numel(),
                              out.data_ptr(), stream.cuda_stream)
        assert rc == 0, rc

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(args.steps):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ev_ms = ev[0].elapsed_time(ev[1]) / args.steps
    tot = int(sum(kv_len))
    kv_bytes = 2 * hkv * tot * d * 2                       # K and V, bf16
    qo_bytes = 2 * len(kv_len) * 8 * hkv * d * 2            # q and out
    alg = kv_bytes + qo_bytes
    log(f"[bench] {args.workload}: {len(kv_len)} requests, {tot} tokens, {n_tasks} tasks; "
        f"{ms:.4f} ms/call (events {ev_ms:.4f})")
    if args.calib_copy_mib:   # a plain copy of known size for the counter runs
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu_baseline:
        from oracle.attention import attention_decode
        nb = min(len(kv_len), 4)
        qf = bits_to_f64(qb[:nb])
        nt = int(sum(kv_len[:nb]))
        kf, vf = bits_to_f64(kb[:, :nt]), bits_to_f64(vb[:, :nt])
        t1 = time.perf_counter()
        attention_decode(qf, kf, vf, kv_len[:nb], 1.0 / np.sqrt(d))
        dt = time.perf_counter() - t1
        cpu = {"value": nt / dt, "unit": "KV tokens/s", "cores": torch.get_num_threads(),
               "kind": "oracle",
               "sample": f"first {nb} requests ({nt} cached tokens, 64 query heads), float64 numpy, once"}
    return {
        "metric": "Hy3 GQA split-KV decode attention: cached KV tokens/s (% HBM BW)",
        "value": tot / (ms / 1e3), "unit": "KV tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) q, K, V)",
        "config": {"workload": args.workload, "requests": len(kv_len), "kv_tokens": tot,
                   "q_heads": 64, "kv_heads": hkv, "head_dim": d, "tile": plan.tile,
                   "workers": plan.n_workers, "tasks": n_tasks,
                   "lengths": ATTN_WORKLOADS[args.workload]},
        "roofline": {"kernel": "attn_split_mfma_kernel + attn_combine_kernel", "bound": "hbm",
                     "achieved": alg / (ev_ms / 1e3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": alg / (ev_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": measured_traffic(args.workload, "attn"),
                     "per_unit": f"{2 * d * 2} B of K+V per cached token and KV head "
                                 f"x {tot} tokens x {hkv} heads + q and out",
                     "avg_launch_ms": ev_ms},
        "cpu_baseline": cpu,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=sorted(WORKLOADS) + sorted(ATTN_WORKLOADS),
                    default="decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens in the CPU oracle sample (default: 16 decode, 48 otherwise)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time spent timing the oracle sample")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure the achievable MFMA and copy ceilings instead of the layer")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the run, copy this many MiB device-to-device (PMC calibration)")
    ap.add_argument("--router-sweep", action="store_true",
                    help="time the gate alone (hy3moe_route) at M = 2, 64, 512, 4096 tokens, "
                         "fp32-accurate and two-term split router, instead of the layer")
    ap.add_argument("--no-prefill", action="store_true",
                    help="default workload only: skip the prefill chunk timed after decode")
    ap.add_argument("--graph", action="store_true",
                    help="also time the layer as a captured HIP graph replayed K times")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this MoE layer build has no multi-GPU path "
              "(how the path would shard is described with the design).  Run with --gpus 1.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_moe_amd as sm
    from synth import CONFIGS, MoEInputs
    from synth.device import upload_weights, with_bias_of

    dev = torch.device("cuda:0")
    if args.ceilings:
        print(json.dumps(ceilings(dev)), flush=True)
        return
    sm.load()
    if args.router_sweep:
        print(json.dumps(router_sweep(args, dev)), flush=True)
        return
    if args.workload in ATTN_WORKLOADS:
        print(json.dumps(attention_bench(args, dev)), flush=True)
        return
    inp = MoEInputs(CONFIGS[WORKLOADS[args.workload]])
    t0 = time.time()
    weights = upload_weights(inp, dev)
    torch.cuda.synchronize()
    log(f"[bench] {inp.cfg.name}: weights uploaded in {time.time() - t0:.1f}s")
    m = layer_bench(inp, weights, args.workload, args, dev, graph=args.graph)
    c = inp.cfg
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args, m["idx"])

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    res = {
        "metric": METRIC, "value": c.T / (m["ms_per_step"] / 1e3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": m["mma_dtype"],
        "data": "synthetic (seeded, random-init weights of the layer's shapes)",
        "config": m["config"],
        "roofline": m["roofline"], "cpu_baseline": cpu, "layer": m["layer"],
        "graph_ms_per_step": m["graph_ms"],
    }
    # The default run also times the prefill chunk (T=8192, skewed bias) on the
    # same Hy3 weights: the metric's bf16 MFMA half.  Its own roofline and
    # stage times; the headline value stays the decode workload's.
    if args.workload == "decode" and not args.no_prefill:
        pinp = MoEInputs(CONFIGS[WORKLOADS["prefill"]])
        assert pinp.cfg.model_key == c.model_key, "prefill must share the decode weights"
        pw = with_bias_of(pinp, weights, dev)
        pm = layer_bench(pinp, pw, "prefill", args, dev)
        res["prefill"] = {"workload": pinp.cfg.name, "value": pinp.cfg.T / (pm["ms_per_step"] / 1e3),
                          "unit": "tokens/s", "ms_per_step": pm["ms_per_step"],
                          "steps": args.steps, "warmup": args.warmup, "dtype": pm["mma_dtype"],
                          "config": pm["config"], "roofline": pm["roofline"],
                          "layer": pm["layer"]}
    print(json.dumps(res), flush=True)


def layer_bench(inp, weights, key, args, dev, graph=False):
    """Time hy3moe_forward on one workload: K steps between synchronisations
    (wall clock), then K steps through hy3moe_forward_timed for per-stage HIP
    event durations; returns the timings, the roofline of the gate-up kernel
    and the whole-layer figures."""
    import numpy as np
    import torch

    import sparse_moe_amd as sm
    from synth.device import to_torch

    c = inp.cfg
    x = to_torch(inp.x(), c.dtype, dev)
    cfg = sm.make_config(c.T, c.H, c.E, c.K, c.I, c.I_shared, c.dtype, c.route_mode,
                         scale=c.scale, renorm_eps=c.renorm_eps, w_format=c.w_format,
                         act_format=c.act_format, shared_w_format=c.shared_w_format,
                         shared_act_format=c.shared_act_format)
    ws = sm.alloc_workspace(cfg, True, dev)
    out = torch.empty_like(x)
    idx = torch.empty((c.T, c.K), dtype=torch.int32, device=dev)
    wgt = torch.empty((c.T, c.K), dtype=torch.float32, device=dev)

    # The router weight's offline split (Hy3 Preview inference case, section
    # 2: prepared once, like the weights): batches that run the router GEMM
    # on bf16 planes read them instead of splitting per call.
    if sm.hy3moe_workspace_layout(cfg).w_planes:
        weights = dict(weights, w_router_planes=sm.router_split(weights["w_router"],
                                                                cfg.router_prec))
    # Route of this batch (outside the timed region) for the byte/FLOP counts.
    sm.hy3moe_forward(cfg, x, weights, out, ws, idx, wgt)
    torch.cuda.synchronize()
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=c.E)
    U = int((counts > 0).sum())

    for _ in range(args.warmup):
        sm.hy3moe_forward(cfg, x, weights, out, ws)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, synchronised on both sides ----
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        sm.hy3moe_forward(cfg, x, weights, out, ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = wall * 1e3 / args.steps
    log(f"[bench] {c.name}: timed {args.steps} steps: {ms_per_step:.4f} ms/step")

    # ---- optional: the same step captured once as a HIP graph, replayed ----
    graph_ms = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            sm.hy3moe_forward(cfg, x, weights, out, ws)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sm.hy3moe_forward(cfg, x, weights, out, ws)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - w0) * 1e3 / args.steps
        log(f"[bench] graph replay: {graph_ms:.4f} ms/step")

    # ---- per-stage durations: HIP events recorded between the kernels ----
    n_ev = sm.HY3MOE_N_STAGES + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for row in evs:
        sm.hy3moe_forward_timed(cfg, x, weights, out, ws, row)
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([row[i].elapsed_time(row[i + 1]) for row in evs]))
                for i, name in enumerate(sm.STAGE_NAMES)}
    log(f"[bench] {c.name} stage ms: " + ", ".join(f"{k}={v:.4f}" for k, v in stage_ms.items()))

    # ---- algorithmic work ----
    eb = 2 if c.dtype == "bf16" else 4
    lay = sm.hy3moe_workspace_layout(cfg)
    gemm_path, a8_codes = lay.gemm_path, bool(lay.a8_codes)

    def branch(wf, af):
        """(bytes per weight element, bytes per x / h element, FP8-rate MFMAs)
        of one branch.  MXFP4 weights: half a byte + one scale byte per 32.
        Static FP8 activations: E4M3 bytes where the layout reports code rows
        (a8_codes: FP8 MFMAs), their bf16 values elsewhere; dynamic MXFP8:
        codes and a scale byte per 32 on the weight-streaming and large-tile
        paths (FP4 x FP8 MFMAs, which issue at the FP8 rate), bf16 values on
        the 128-row tiled path."""
        web = {"fp8_e4m3": 1, "mxfp4": 0.5 + 1 / 32}.get(wf, eb)
        f8 = ((af == "fp8_static" and a8_codes) or
              (af == "mxfp8" and gemm_path == 2))
        ab = 1 if f8 else eb
        if af == "mxfp8" and gemm_path != 1:
            ab = 1 + 1 / 32
        mma = ("mxfp4_x_mxfp8" if af == "mxfp8" else "fp8_e4m3") if f8 else c.dtype
        return web, ab, f8, mma

    T, H, E, K, I, Is = c.T, c.H, c.E, c.K, c.I, c.I_shared
    web, ab, fp8_mma, mma_dtype = branch(c.w_format, c.act_format)
    mixed = bool(Is) and (c.sw_format, c.sa_format) != (c.w_format, c.act_format)
    web_s, ab_s, f8_s, mma_s = branch(c.sw_format, c.sa_format) if Is else (0, 0, fp8_mma,
                                                                             mma_dtype)
    if mixed and mma_s != mma_dtype:
        mma_dtype += "+" + mma_s
    fp8_mma = fp8_mma and f8_s                 # priced at the FP8 peak only if both are
    peak_mma = PEAK_FP8_TFLOPS if fp8_mma else PEAK_BF16_TFLOPS
    # When hy3moe_forward runs the shared expert's GEMMs on its side stream
    # (large-tile path, or formats of its own: shared_meta in the layout),
    # the gate-up and down stages on the caller's stream (and their kernels'
    # launches) are the routed experts' GEMMs alone; otherwise the shared
    # expert is one more group of those launches.
    side = bool(Is) and sm.hy3moe_workspace_layout(cfg).shared_meta > 0
    Ish = 0 if side else Is
    gu_bytes = (U * 2 * I * H * web + 2 * Ish * H * web_s + T * H * ab + T * K * I * ab
                + T * Ish * ab_s)
    dn_bytes = (U * H * I * web + H * Ish * web_s + T * K * I * ab + T * Ish * ab_s
                + (T * K + (T if Ish else 0)) * H * eb)
    gu_flops = 4.0 * H * (T * K * I + T * Ish)
    dn_flops = 2.0 * H * (T * K * I + T * Ish)
    shared_note = (" (the shared expert runs on the side stream)" if side else
                   f" + {2 * Is * H * web_s:.0f} B of the shared expert's" if Is else "")
    # the whole layer: every weight read once, x in, out written
    layer_bytes = (U * 3 * I * H * web + 3 * Is * H * web_s + E * H * 4 + 2 * T * H * eb)
    layer_flops = 6.0 * H * (T * K * I + T * Is) + 2.0 * T * H * E
    layer_s = ms_per_step / 1e3
    gu_s = stage_ms["gate_up"] / 1e3
    decode = key.startswith("decode")
    names = {"fp8_e4m3": "FP8 E4M3", "mxfp4": "MXFP4"}
    if decode:
        kind = names.get(c.w_format, c.dtype)
        roof = {"kernel": "gate_up (weight-streaming grouped GEMM + SwiGLU)",
                "bound": "hbm", "achieved": gu_bytes / gu_s / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "per_unit": f"{2 * I * H * web:.0f} B of {kind} gate+up weights per touched "
                            f"routed expert x {U} experts{shared_note} + x and h rows"}
    else:
        path = "128x128-tile" if gemm_path == 1 else "256x256-tile"
        if fp8_mma:
            path += " FP4 x FP8 MFMA" if c.act_format == "mxfp8" else " FP8 MFMA"
            if mixed and mma_s != branch(c.w_format, c.act_format)[3]:
                path += " (shared expert: FP8 MFMA)" if c.sa_format == "fp8_static" \
                    else " (shared expert: FP4 x FP8 MFMA)"
        roof = {"kernel": f"gate_up ({path} grouped GEMM + SwiGLU)",
                "bound": "mfma", "achieved": gu_flops / gu_s / 1e12, "peak": peak_mma,
                "unit": "TFLOP/s",
                "per_unit": f"{4 * H * I} FLOP per routed row x {T * K} rows"
                            + (" (the shared expert runs on the side stream)" if side else
                               f" + {4 * H * Is} per shared row x {T}" if Is else "")}
    roof["frac"] = roof["achieved"] / roof["peak"]
    tr = measured_traffic(key, "gate_up")
    roof["traffic"] = tr
    roof["avg_launch_ms"] = stage_ms["gate_up"]

    layer = {
        "unique_experts": U, "max_load": int(counts.max()),
        "stage_ms": stage_ms,
        "bytes": layer_bytes, "GB_s": layer_bytes / layer_s / 1e9,
        "hbm_frac": layer_bytes / layer_s / 1e9 / PEAK_HBM_GBS,
        "flops": layer_flops, "TFLOP_s": layer_flops / layer_s / 1e12,
        "mfma_frac": layer_flops / layer_s / 1e12 / peak_mma,
        "down_achieved": (dn_bytes / (stage_ms["down"] / 1e3) / 1e9 if decode
                          else dn_flops / (stage_ms["down"] / 1e3) / 1e12),
    }

    config = {"workload": c.name, "T": T, "H": H, "E": E, "K": K, "I": I, "I_shared": Is,
              "route": "sigmoid+bias" if c.route_mode == 0 else "softmax",
              "expert_weights": c.w_format if c.w_format != "dtype" else c.dtype,
              "expert_activations": {"fp8_static": "fp8_e4m3_static",
                                     "mxfp8": "mxfp8_dynamic"}.get(c.act_format, c.dtype)}
    if mixed:
        config["shared_expert_weights"] = c.sw_format if c.sw_format != "dtype" else c.dtype
        config["shared_expert_activations"] = {"fp8_static": "fp8_e4m3_static",
                                               "mxfp8": "mxfp8_dynamic"}.get(c.sa_format,
                                                                             c.dtype)
    return {"ms_per_step": ms_per_step, "stage_ms": stage_ms, "roofline": roof, "layer": layer,
            "config": config, "mma_dtype": mma_dtype, "graph_ms": graph_ms,
            "idx": idx.cpu().numpy()}


def router_sweep(args, dev):
    """The gate alone on the router-only workload (H=4096, E=192, top-8):
    hy3moe_route over the first M tokens, both router arithmetics.  Time per
    call from HIP events over `steps` calls; GB/s counts the fp32 router
    weight plus the M activation rows, TFLOP/s the 2*M*H*E of the product."""
    import torch

    import sparse_moe_amd as sm
    from synth import CONFIGS, ROUTER_SWEEP_M, MoEInputs
    from synth.device import to_torch

    inp = MoEInputs(CONFIGS[ROUTER_WORKLOAD])
    c = inp.cfg
    x_all = to_torch(inp.x(), c.dtype, dev)
    wr = torch.from_numpy(inp.w_router()).to(dev)
    bias = torch.from_numpy(inp.bias()).to(dev)
    rows = []
    for M in ROUTER_SWEEP_M:
        x = x_all[:M].contiguous()
        for prec, name in ((sm.HY3MOE_ROUTER_FP32, "fp32-accurate (3-term bf16 split)"),
                           (sm.HY3MOE_ROUTER_SPLIT2_BF16, "two-term bf16 split")):
            cfg = sm.make_config(M, c.H, c.E, c.K, c.I, c.I_shared, c.dtype, c.route_mode,
                                 router_prec=prec, scale=c.scale, renorm_eps=c.renorm_eps)
            ws = sm.alloc_workspace(cfg, False, dev)
            idx = torch.empty((M, c.K), dtype=torch.int32, device=dev)
            wgt = torch.empty((M, c.K), dtype=torch.float32, device=dev)
            for _ in range(args.warmup):
                sm.hy3moe_route(cfg, x, wr, bias, idx, wgt, ws)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                sm.hy3moe_route(cfg, x, wr, bias, idx, wgt, ws)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.steps
            nbytes = c.E * c.H * 4 + M * c.H * 2
            rows.append({"M": M, "router": name, "us_per_call": us,
                         "GB_s": nbytes / us / 1e3, "TFLOP_s": 2.0 * M * c.H * c.E / us / 1e6})
            log(f"[router] M={M:5d} {name:34s} {us:8.2f} us")
            if sm.hy3moe_workspace_layout(cfg).w_planes:
                # the same gate on the weight's offline split (hy3moe_router_split):
                # no per-call split kernel, planes read as they are
                planes = sm.router_split(wr, prec)
                for _ in range(args.warmup):
                    sm.hy3moe_route_planes(cfg, x, wr, planes, bias, idx, wgt, ws)
                e0.record()
                for _ in range(args.steps):
                    sm.hy3moe_route_planes(cfg, x, wr, planes, bias, idx, wgt, ws)
                e1.record()
                torch.cuda.synchronize()
                us2 = e0.elapsed_time(e1) * 1e3 / args.steps
                pb = planes.numel() + M * c.H * 2
                rows.append({"M": M, "router": name + ", offline planes", "us_per_call": us2,
                             "GB_s": pb / us2 / 1e3,
                             "TFLOP_s": 2.0 * M * c.H * c.E / us2 / 1e6})
                log(f"[router] M={M:5d} {name + ', offline planes':34s} {us2:8.2f} us")
    return {"router_sweep": rows, "config": {"workload": c.name, "H": c.H, "E": c.E, "K": c.K},
            "steps": args.steps, "note": "gate only: router GEMM + score/select"}


def ceilings(dev):
    """Achievable ceilings on this GPU: dense bf16 and FP8 MFMA microkernels
    (register operands only, 16 independent chains per wavefront), a 16-byte-per-lane
    device copy of 4 GiB (read + write bytes counted), a streaming read of
    the same 4 GiB, and the weight-streaming GEMMs' reads with the MFMAs
    removed."""
    import ctypes

    import torch

    from sparse_moe_amd.build import PROBE_PATH
    L = ctypes.CDLL(PROBE_PATH)
    L.hy3moe_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.hy3moe_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_int, ctypes.c_void_p]
    s = torch.cuda.current_stream().cuda_stream
    res = {}
    for blocks in (2048, 4096):
        iters = 4000
        out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        assert L.hy3moe_probe_mfma(blocks, 100, out.data_ptr(), s) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        assert L.hy3moe_probe_mfma(blocks, iters, out.data_ptr(), s) == 0
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        flops = blocks * 4 * iters * 16 * 2.0 * 16 * 16 * 32
        res[f"mfma_bf16_tflops_{blocks}blk"] = flops / ms / 1e9
    L.hy3moe_probe_mfma_fp8.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    for blocks in (2048, 4096):
        iters = 2000
        out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        assert L.hy3moe_probe_mfma_fp8(blocks, 100, out.data_ptr(), s) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        assert L.hy3moe_probe_mfma_fp8(blocks, iters, out.data_ptr(), s) == 0
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        flops = blocks * 4 * iters * 16 * 2.0 * 16 * 16 * 128
        res[f"mfma_fp8_tflops_{blocks}blk"] = flops / ms / 1e9
    n = 4 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    best = 0.0
    for blocks in (1024, 2048, 4096, 8192):
        assert L.hy3moe_probe_copy(src.data_ptr(), dst.data_ptr(), n, blocks, s) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            L.hy3moe_probe_copy(src.data_ptr(), dst.data_ptr(), n, blocks, s)
        e1.record()
        torch.cuda.synchronize()
        gbs = 2 * n * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
        res[f"copy_GBs_{blocks}blk"] = gbs
        best = max(best, gbs)
    res["copy_GBs_best"] = best
    L.hy3moe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
    best = 0.0
    for blocks in (1024, 2048, 4096, 8192):
        out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
        assert L.hy3moe_probe_read(src.data_ptr(), n, blocks, out.data_ptr(), s) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            L.hy3moe_probe_read(src.data_ptr(), n, blocks, out.data_ptr(), s)
        e1.record()
        torch.cuda.synchronize()
        gbs = n * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
        res[f"read_GBs_{blocks}blk"] = gbs
        best = max(best, gbs)
    L.hy3moe_probe_read_segments.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    for blocks in (512, 1024, 2048, 4096):
        for depth in (8, 16):
            out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
            assert L.hy3moe_probe_read_segments(src.data_ptr(), n, blocks, depth,
                                                out.data_ptr(), s) == 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                L.hy3moe_probe_read_segments(src.data_ptr(), n, blocks, depth, out.data_ptr(), s)
            e1.record()
            torch.cuda.synchronize()
            gbs = n * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
            res[f"read_seg_GBs_{blocks}blk_d{depth}"] = gbs
            best = max(best, gbs)
    res["read_GBs_best"] = best
    # the weight-streaming GEMMs' reads with the MFMAs removed, at the weight
    # row lengths of the Hy3 decode GEMMs (bf16 gate-up 8 KB, FP8 gate-up
    # 4 KB, bf16 down 3 KB, FP8 down 1.5 KB): 16 rows x 64 B per load (the
    # MFMA operand layout) and 4 rows x 256 B with the non-temporal hint (the
    # four-row loads the kernels transpose through LDS)
    L.hy3moe_probe_read_fragments.argtypes = [
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    blocks = 512
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    for rowbytes in (8192, 4096, 3072, 1536):
        for rows, nt, tag in ((16, 0, "rows16"), (4, 1, "rows4_nt")):
            rb = ctypes.c_size_t(0)
            args = (src.data_ptr(), n, rowbytes, rows, nt, blocks, out.data_ptr(),
                    ctypes.byref(rb), s)
            assert L.hy3moe_probe_read_fragments(*args) == 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                L.hy3moe_probe_read_fragments(*args)
            e1.record()
            torch.cuda.synchronize()
            res[f"read_frag_GBs_{rowbytes}B_{tag}"] = rb.value * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
    res["mfma_bf16_tflops_best"] = max(v for k, v in res.items() if k.startswith("mfma_bf16"))
    res["mfma_fp8_tflops_best"] = max(v for k, v in res.items() if k.startswith("mfma_fp8"))
    res["peak_published"] = {"bf16_tflops": PEAK_BF16_TFLOPS, "fp8_tflops": PEAK_FP8_TFLOPS,
                             "hbm_GBs": PEAK_HBM_GBS}
    return res


def cpu_baseline(inp, args, gpu_idx):
    """The float64 oracle, as it stands, on a bounded sample of the same batch."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [d.get("num_threads") for d in threadpool_info() if d.get("user_api") == "blas"]
        cores = int(blas[0]) if blas else os.cpu_count()
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    c = inp.cfg
    n = args.cpu_sample_tokens or (16 if args.workload.startswith("decode") else 48)
    n = min(n, c.T)
    tokens = np.arange(n)
    x64 = inp.x_f64()[tokens]
    wr = inp.w_router().astype(np.float64)
    b = inp.bias()
    b64 = None if b is None else b.astype(np.float64)
    need = sorted(set(gpu_idx[tokens].reshape(-1).tolist()))
    t0 = time.time()
    # the oracle's own dequantisation of the codes, each branch in its format
    def dequant(fmt, get_codes, plain):
        if fmt == "mxfp4":
            codes, sc = get_codes("mxfp4")
            return tuple(oracle.dequant_mxfp4(q, s) for q, s in zip(codes, sc))
        if fmt == "fp8_e4m3":
            codes, sc = get_codes("fp8")
            return tuple(oracle.dequant_fp8(q, s) for q, s in zip(codes, sc))
        return plain()

    def expert_f64(e):
        return dequant(c.w_format, lambda k: getattr(inp, f"expert_{k}")(e),
                       lambda: inp.expert_f64(e))

    sh = None
    if c.I_shared:
        sh = dequant(c.sw_format, lambda k: getattr(inp, f"shared_{k}")(), inp.shared_f64)

    def a8_of(fmt):
        if fmt != "fp8_static":
            return None
        a1, a2 = inp.act_scales()
        return float(a1), a2.astype(np.float64)
    act = dict(a8=a8_of(c.act_format), amx=c.act_format == "mxfp8",
               shared_a8=a8_of(c.sa_format), shared_amx=c.sa_format == "mxfp8")
    with ThreadPoolExecutor(8) as ex:
        ws = dict(zip(need, ex.map(expert_f64, need)))
    log(f"[bench] oracle sample: {n} tokens, {len(need)} experts in float64 "
        f"(generated in {time.time() - t0:.1f}s)")
    # Experts the oracle picks that the GPU did not (near-ties) are input
    # preparation and are generated before timing.
    r = oracle.route(x64, wr, c.K, c.route_mode, b64, c.scale, c.renorm_eps)
    for e in sorted(set(r.idx.reshape(-1).tolist()) - set(ws)):
        ws[e] = expert_f64(e)
    # Repeat the whole sample (route + experts + combine) until ~target seconds.
    reps, dt = 0, 0.0
    while reps < 3 or (dt < args.cpu_seconds and reps < 10000):
        t1 = time.perf_counter()
        r = oracle.route(x64, wr, c.K, c.route_mode, b64, c.scale, c.renorm_eps)
        oracle.forward_given_route(x64, r.idx, r.weight, ws.__getitem__, c.E, sh, **act)
        dt += time.perf_counter() - t1
        reps += 1
    del ws
    return {"value": n * reps / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} of the {c.T} tokens of the same batch (route over them, "
                      f"{len(need)} experts + shared, float64 numpy), repeated {reps}x "
                      f"in {dt:.1f}s"}


if __name__ == "__main__":
    main()
