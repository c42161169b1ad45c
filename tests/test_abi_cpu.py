"""The C ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments before launching anything (no GPU needed)."""
import ctypes
import os
import re

import numpy as np

import pytest

import sparse_moe_amd as sm
from sparse_moe_amd import binding as b
from synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hy3moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hy3moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(b.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return sm.load()


def test_header_declares_the_documented_entry_points():
    fns = declared_functions()
    for need in ("hy3moe_route", "hy3moe_forward", "hy3moe_workspace_bytes",
                 "hy3moe_workspace_layout", "hy3moe_strerror", "hy3moe_abi_version"):
        assert need in fns
    assert sorted(sm.EXPORTED_SYMBOLS) == fns


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_abi_version_and_strerror(lib):
    assert lib.hy3moe_abi_version() == b.ABI_VERSION == 12
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert sm.strerror(code) and sm.strerror(code) != "unknown error code"
    assert sm.strerror(7) == "unknown error code"


def cfg_of(c, **kw):
    d = dict(T=c.T, H=c.H, E=c.E, K=c.K, I=c.I, I_shared=c.I_shared, dtype=c.dtype,
             route_mode=c.route_mode, scale=c.scale, renorm_eps=c.renorm_eps,
             w_format=c.w_format, act_format=c.act_format,
             shared_w_format=c.shared_w_format, shared_act_format=c.shared_act_format)
    d.update(kw)
    return sm.make_config(**d)


def R_of(c):
    return c.T * c.K + (c.T if c.I_shared else 0)


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_workspace_layout_is_consistent(lib, name):
    cfg = cfg_of(CONFIGS[name])
    L = sm.hy3moe_workspace_layout(cfg)
    assert L.total == sm.hy3moe_workspace_bytes(cfg, True) > 0
    assert 0 < sm.hy3moe_workspace_bytes(cfg, False) <= L.total
    names = ["logits_part", "idx", "weight", "hist", "counts", "offsets", "sorted_token",
             "pos_of", "tiles", "h", "y"]
    c = CONFIGS[name]
    planes = c.dtype == "bf16" and c.T >= 1024
    assert (L.w_planes > 0) == planes
    if planes:
        names.append("w_planes")
    mixed = (c.sw_format, c.sa_format) != (c.w_format, c.act_format)
    assert (L.xq > 0) == (c.act_format != "dtype")
    if L.xq:
        names.append("xq")
        assert L.total - L.xq >= c.T * c.H * 2
    assert (L.xs > 0) == (c.act_format == "mxfp8")
    assert (L.xq_shared > 0) == (mixed and c.sa_format != "dtype")
    assert (L.xs_shared > 0) == (mixed and c.sa_format == "mxfp8")
    for n in ("xq_shared", "xs_shared"):
        if getattr(L, n):
            names.append(n)
    assert L.total - max(L.xq_shared, L.xs_shared) >= (c.T * c.H // 32 if L.xs_shared else 0)
    assert (L.hq > 0) == (L.hs > 0) == ("mxfp8" in (c.act_format, c.sa_format))
    assert (L.shared_meta > 0) == (c.I_shared > 0 and (mixed or L.gemm_path == 2))
    if L.shared_meta:
        names.append("shared_meta")
        assert L.total - L.shared_meta >= 4 * (2 * L.max_tiles + 2 + c.E + 2 + R_of(c))
    if L.xs:
        names.append("xs")
    if L.hq:
        names += ["hq", "hs"]
        assert L.hq - L.xs >= c.T * c.H // 32
        assert L.hs - L.hq >= R_of(c) * max(c.I, c.I_shared)
        assert L.total - L.hs >= R_of(c) * max(c.I, c.I_shared) // 32
    offs = sorted(getattr(L, n) for n in names)
    assert all(o % 256 == 0 for o in offs)
    assert len(set(offs)) == len(offs)
    R = c.T * c.K + (c.T if c.I_shared else 0)
    eb = 2 if c.dtype == "bf16" else 4
    assert L.total - L.y >= R * c.H * eb         # y: fp16 (bf16 layers) or float32
    assert L.y - L.h >= R * max(c.I, c.I_shared) * eb
    assert L.max_tiles >= (R + L.tile_rows - 1) // L.tile_rows
    assert L.tile_rows >= min(c.T, 16)
    want = {0: L.tile_rows, 1: 128, 2: 256}[L.gemm_path]
    assert L.tile_rows == want and (L.gemm_path == 0) == (c.T <= 64)
    # token rows as E4M3 codes: the large-tile path, and the weight-streaming
    # path when every K of its FP8 MFMAs is a multiple of 128
    k128 = c.H % 128 == 0 and c.I % 128 == 0 and c.I_shared % 128 == 0
    assert bool(L.a8_codes) == (L.gemm_path == 2 or (L.gemm_path == 0 and k128))


@pytest.mark.parametrize("bad, code", [
    (dict(K=0), -1), (dict(K=17, E=16), -1), (dict(E=257, K=8), -1), (dict(T=-1), -1),
    (dict(H=100), -2), (dict(I=96), -2), (dict(I_shared=32), -2), (dict(K=65, E=100), -1),
    (dict(dtype="f32", router_prec=1), -2), (dict(route_mode=3), -1),
    (dict(T=1 << 19), -2), (dict(H=65536, I=32768, I_shared=0), -2),
    # FP8 expert weights: bf16 activations and weight-streaming batches only
    (dict(w_format="fp8_e4m3", dtype="f32"), -2),
    # static FP8 activations: with FP8 weights only
    (dict(act_format="fp8_static"), -2),
    # MXFP4 weights: bf16 activations, H, I, I_shared % 128, T <= 64, no W8A8
    (dict(w_format="mxfp4", dtype="f32"), -2), (dict(w_format="mxfp4", H=4096 + 64), -2),
    (dict(w_format="mxfp4", I=1536 + 64), -2), (dict(w_format="mxfp4", I_shared=64), -2),
    (dict(w_format="mxfp4", act_format="fp8_static"), -2),
    # dynamic MXFP8 activations: with MXFP4 weights only
    (dict(act_format="mxfp8"), -2), (dict(w_format="fp8_e4m3", act_format="mxfp8"), -2),
])
def test_invalid_configs_rejected(lib, bad, code):
    c = CONFIGS["hy3_decode_T16"]
    kw = dict(T=16, H=c.H, E=c.E, K=c.K, I=c.I, I_shared=c.I_shared, dtype="bf16",
              route_mode=0, scale=2.826)
    kw.update(bad)
    cfg = sm.make_config(**kw)
    assert sm.hy3moe_workspace_bytes(cfg, True) == 0
    L = b.hy3moe_ws_layout()
    assert lib.hy3moe_workspace_layout(ctypes.byref(cfg), ctypes.byref(L)) == code
    w = b.hy3moe_weights(*([256] * 8))
    rc = lib.hy3moe_forward(ctypes.byref(cfg), 256, ctypes.byref(w), 512, None, None, 1024,
                            1 << 40, None)
    assert rc == code


def test_argument_errors_before_launch(lib):
    cfg = cfg_of(CONFIGS["hy3_decode_T16"])
    need = sm.hy3moe_workspace_bytes(cfg, True)
    good = b.hy3moe_weights(*([4096] * 8))
    fw = lib.hy3moe_forward
    # null pointers
    assert fw(ctypes.byref(cfg), None, ctypes.byref(good), 8192, None, None, 4096, need, None) == -1
    nul = b.hy3moe_weights(4096, 0, 4096, None, 4096, 4096, 4096, 4096)
    assert fw(ctypes.byref(cfg), 4096, ctypes.byref(nul), 8192, None, None, 4096, need, None) == -1
    nsh = b.hy3moe_weights(4096, 0, 4096, 4096, 4096, None, 4096, 4096)
    assert fw(ctypes.byref(cfg), 4096, ctypes.byref(nsh), 8192, None, None, 4096, need, None) == -1
    # aliasing out == x
    assert fw(ctypes.byref(cfg), 4096, ctypes.byref(good), 4096, None, None, 8192, need, None) == -1
    # misaligned tensors
    assert fw(ctypes.byref(cfg), 4104, ctypes.byref(good), 8192, None, None, 4096, need, None) == -4
    assert fw(ctypes.byref(cfg), 4096, ctypes.byref(good), 8192, 4097, None, 4096, need, None) == -4
    # workspace too small
    assert fw(ctypes.byref(cfg), 4096, ctypes.byref(good), 8192, None, None, 4096, need - 1,
              None) == -3
    # route entry point
    rw = lib.hy3moe_route
    rneed = sm.hy3moe_workspace_bytes(cfg, False)
    assert rw(ctypes.byref(cfg), 4096, None, None, 4096, 4096, 4096, rneed, None) == -1
    assert rw(ctypes.byref(cfg), 4096, 4096, None, 4096, 4096, 4096, rneed - 1, None) == -3
    assert rw(ctypes.byref(cfg), 4096, 4104 + 4, None, 4096, 4096, 4096, rneed, None) == -4


def test_zero_tokens_is_a_no_op(lib):
    cfg = cfg_of(CONFIGS["hy3_decode_T16"], T=0)
    w = b.hy3moe_weights(*([4096] * 8))
    assert lib.hy3moe_forward(ctypes.byref(cfg), 4096, ctypes.byref(w), 8192, None, None,
                              4096, 0, None) == 0
    assert lib.hy3moe_route(ctypes.byref(cfg), 4096, 4096, None, 4096, 4096, 4096, 0, None) == 0


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setenv("HY3MOE_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(b, "_LIB", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        b.load()


def test_weight_format_enum_is_checked(lib):
    cfg = cfg_of(CONFIGS["hy3_decode_T16_fp8"])
    assert sm.hy3moe_workspace_bytes(cfg, True) > 0
    cfg.w_format = 3
    assert sm.hy3moe_workspace_bytes(cfg, True) == 0
    L = b.hy3moe_ws_layout()
    assert lib.hy3moe_workspace_layout(ctypes.byref(cfg), ctypes.byref(L)) == -1


def test_activation_format_enum_is_checked(lib):
    cfg = cfg_of(CONFIGS["hy3_decode_T16_w8a8"])
    assert sm.hy3moe_workspace_bytes(cfg, True) > 0
    cfg.act_format = 3
    assert sm.hy3moe_workspace_bytes(cfg, True) == 0
    L = b.hy3moe_ws_layout()
    assert lib.hy3moe_workspace_layout(ctypes.byref(cfg), ctypes.byref(L)) == -1


def test_w8a8_path_choice(lib):
    """W8A8 batches take the large-tile FP8-MFMA path only when H, I and
    I_shared are multiples of 128 (its K stages hold 128 values)."""
    big = sm.hy3moe_workspace_layout(cfg_of(CONFIGS["hy3_prefill_T8192_skew_w8a8"]))
    assert big.gemm_path == 2 and big.tile_rows == 256
    for kw in (dict(H=4096 + 64), dict(I=1536 + 64), dict(I_shared=64)):
        L = sm.hy3moe_workspace_layout(cfg_of(CONFIGS["hy3_prefill_T8192_skew_w8a8"], **kw))
        assert L.gemm_path == 1 and L.tile_rows == 128, kw
        # ... while the same shapes with W8A16 stay on the large-tile path
        L16 = sm.hy3moe_workspace_layout(cfg_of(CONFIGS["hy3_prefill_T8192_skew_w8a8"],
                                                act_format="dtype", **kw))
        assert L16.gemm_path == 2 and L16.tile_rows == 256, kw


def test_mxfp4_weights_need_their_block_scales(lib):
    cfg = cfg_of(CONFIGS["hy3_decode_T16_mxfp4"])
    need = sm.hy3moe_workspace_bytes(cfg, True)
    assert need > 0
    fw = lib.hy3moe_forward
    full = [4096] * 20
    for missing in range(14, 20):                     # each of the six E8M0 arrays
        w = list(full)
        w[missing] = None
        assert fw(ctypes.byref(cfg), 4096, ctypes.byref(b.hy3moe_weights(*w)), 8192, None,
                  None, 4096, need, None) == -1, missing
    for bad in (4098, 4100):                          # down scales not 16-byte aligned
        w = list(full)
        w[16] = bad
        assert fw(ctypes.byref(cfg), 4096, ctypes.byref(b.hy3moe_weights(*w)), 8192, None,
                  None, 4096, need, None) == -4
    # without a shared expert its scale arrays may be NULL
    cfg_ns = cfg_of(CONFIGS["hy3_decode_T16_mxfp4"], I_shared=0)
    w = full[:17] + [None, None, None]
    rc = fw(ctypes.byref(cfg_ns), 4096, ctypes.byref(b.hy3moe_weights(*w)), 8192, None, None,
            4096, sm.hy3moe_workspace_bytes(cfg_ns, True), None)
    assert rc not in (-1, -4)


def test_w8a8_needs_its_activation_scales(lib):
    cfg = cfg_of(CONFIGS["hy3_decode_T16_w8a8"])
    need = sm.hy3moe_workspace_bytes(cfg, True)
    fw = lib.hy3moe_forward
    no_h = b.hy3moe_weights(*([4096] * 13 + [None]))
    no_x = b.hy3moe_weights(*([4096] * 12 + [None, 4096]))
    mis = b.hy3moe_weights(*([4096] * 13 + [4098]))
    for w, code in ((no_h, -1), (no_x, -1), (mis, -4)):
        assert fw(ctypes.byref(cfg), 4096, ctypes.byref(w), 8192, None, None, 4096, need,
                  None) == code


def test_quantize_entry_validation(lib):
    q = lib.hy3moe_quantize_e4m3
    assert q(None, 1, 0, None, None, None) == 0          # n == 0: no-op
    assert q(None, 1, -1, None, None, None) == -1
    assert q(4096, 3, 8, 4096, 4096, None) == -1         # bad dtype
    assert q(4096, 1, 8, None, 4096, None) == -1         # no scale
    assert q(4104, 1, 8, 4096, 4096, None) == -4         # x not 16-byte aligned
    assert q(4096, 0, 8, 4098, 4096, None) == -4         # scale not 4-byte aligned


def test_fp8_weights_need_their_scales(lib):
    cfg = cfg_of(CONFIGS["hy3_decode_T16_fp8"])
    need = sm.hy3moe_workspace_bytes(cfg, True)
    fw = lib.hy3moe_forward
    ok = b.hy3moe_weights(*([4096] * 12))
    missing = b.hy3moe_weights(*([4096] * 11 + [None]))        # no shared scales
    assert fw(ctypes.byref(cfg), 4096, ctypes.byref(missing), 8192, None, None, 4096, need,
              None) == -1
    nosc = b.hy3moe_weights(*([4096] * 8))                      # no scales at all
    assert fw(ctypes.byref(cfg), 4096, ctypes.byref(nosc), 8192, None, None, 4096, need,
              None) == -1
    mis = b.hy3moe_weights(*([4096] * 9 + [4098, 4096, 4096]))  # scale not 4-byte aligned
    assert fw(ctypes.byref(cfg), 4096, ctypes.byref(mis), 8192, None, None, 4096, need,
              None) == -4
    # the same weights without shared expert do not need the shared scales
    cfg_ns = cfg_of(CONFIGS["hy3_decode_T16_fp8"], I_shared=0)
    need_ns = sm.hy3moe_workspace_bytes(cfg_ns, True)
    assert fw(ctypes.byref(cfg_ns), 4096, ctypes.byref(missing), 8192, None, None, 4096,
              need_ns - 1, None) == -3
    del ok


def attn_declared_functions():
    text = open(os.path.join(ROOT, "include", "hy3attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hy3attn_[a-z0-9_]+)\s*\(", text)))


def test_attention_header_symbols_are_exported(lib):
    fns = attn_declared_functions()
    assert sorted(sm.ATTN_EXPORTED_SYMBOLS) == fns
    for name in fns:
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value, name


@pytest.mark.parametrize("kv_len, hkv, tile, workers", [
    ([300, 700], 2, 256, 3), ([131072], 8, 256, 512), ([0, 1, 255, 256, 257, 5000], 8, 256, 7),
    ([7] * 40, 8, 256, 512), ([100000, 3, 40000, 0, 9999], 8, 128, 300), ([], 8, 256, 4),
    ([0, 0], 8, 256, 4)])
def test_attention_plan_matches_the_oracle(lib, kv_len, hkv, tile, workers):
    """The library's task map (host C++) equals the oracle's greedy fill."""
    from oracle.attention import plan_split_kv
    p = sm.attn_plan(kv_len, hkv, tile, workers)
    ref = plan_split_kv(kv_len, hkv, tile, workers)
    np.testing.assert_array_equal(p.tasks.reshape(-1, 4), ref.tasks)
    np.testing.assert_array_equal(p.worker_begin, ref.worker_begin)
    np.testing.assert_array_equal(p.row_begin, ref.row_begin)


def test_attention_plan_rejects_bad_arguments(lib):
    L = lib
    nt = ctypes.c_int64(0)
    buf = np.zeros(64, dtype=np.int32)
    kv = np.array([5], dtype=np.int32)
    assert L.hy3attn_plan(kv.ctypes.data, 1, 0, 256, 4, buf.ctypes.data, 8, buf.ctypes.data,
                          buf.ctypes.data, ctypes.byref(nt)) == -1
    kv_neg = np.array([-1], dtype=np.int32)
    assert L.hy3attn_plan(kv_neg.ctypes.data, 1, 8, 256, 4, buf.ctypes.data, 8, buf.ctypes.data,
                          buf.ctypes.data, ctypes.byref(nt)) == -1
    big = np.array([100000], dtype=np.int32)
    assert L.hy3attn_plan(big.ctypes.data, 1, 8, 256, 4, buf.ctypes.data, 2, buf.ctypes.data,
                          buf.ctypes.data, ctypes.byref(nt)) == -2


def test_attention_decode_rejects_misaligned_or_missing_pointers(lib):
    """Validation happens on the host before any launch (no GPU touched)."""
    L = lib
    ok = 1 << 20   # aligned stand-in addresses: rejected before use
    args = dict(q=ok, k=ok, v=ok, kv=ok, B=1, hkv=8, tile=256, tasks=ok, nt=1, wb=ok, nw=4,
                rb=ok, nrows=8, ws=ok, wsb=1 << 20, out=ok)

    def call(**kw):
        a = dict(args, **kw)
        return L.hy3attn_decode(a["q"], a["k"], a["v"], a["kv"], a["B"], a["hkv"], a["tile"],
                                a["tasks"], a["nt"], a["wb"], a["nw"], a["rb"], a["nrows"],
                                a["ws"], a["wsb"], a["out"], None)
    assert call(q=ok + 8) == -1          # q not 16-byte aligned
    assert call(k=ok + 4) == -1
    assert call(out=ok + 2) == -1        # out not 8-byte aligned
    assert call(ws=ok + 128) == -1       # workspace not 256-byte aligned
    assert call(wsb=16) == -1            # workspace too small
    assert call(q=None) == -1
    assert call(hkv=0) == -1
    assert call(B=0, nrows=0) == 0       # nothing to do
    # a plan made for another batch or KV head count is rejected
    assert call(nrows=7) == -1
    assert call(nrows=16) == -1
    assert call(B=2) == -1               # plan rows 8, call rows 16
    assert call(hkv=4) == -1
    assert call(nt=-1) == -1


def test_attention_binding_rejects_a_plan_for_another_batch(lib):
    """attn_decode checks the plan against the call's shapes on the host,
    before anything is copied to a device (CPU tensors stand in here)."""
    import torch
    import sparse_moe_amd as sm
    plan = sm.attn_plan([300, 500], 2, 256, 4)
    q = torch.zeros((2, 16, 128), dtype=torch.bfloat16)
    k = torch.zeros((2, 800, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):      # three requests, plan for two
        sm.attn_decode(torch.zeros((3, 16, 128), dtype=torch.bfloat16), k, k, [300, 500, 1], plan)
    with pytest.raises(ValueError):      # four KV heads, plan for two
        sm.attn_decode(torch.zeros((2, 32, 128), dtype=torch.bfloat16),
                       torch.zeros((4, 800, 128), dtype=torch.bfloat16),
                       torch.zeros((4, 800, 128), dtype=torch.bfloat16), [300, 500], plan)
    with pytest.raises(ValueError):      # query heads not 8 per KV head
        sm.attn_decode(torch.zeros((2, 8, 128), dtype=torch.bfloat16), k, k, [300, 500], plan)
    bad = sm.AttnPlan(plan.tasks.copy(), plan.worker_begin, plan.row_begin, plan.n_workers,
                      plan.tile)
    bad.tasks[0, 0] = 5                  # a task naming request 5
    with pytest.raises(ValueError):
        sm.attn_decode(q, k, k, [300, 500], bad)


def test_static_forward_rejects_batches_beyond_its_scratch(lib):
    """hy3moe_forward_static validates on the host before touching a device:
    a batch whose workspace exceeds the static array is rejected, and so is a
    bad configuration; T = 0 is a no-op."""
    assert lib.hy3moe_static_scratch_bytes() == 64 << 20
    w = sm.hy3moe_weights()
    big = sm.make_config(4096, 4096, 192, 8, 1536, 1536, "bf16")
    assert sm.hy3moe_workspace_bytes(big) > lib.hy3moe_static_scratch_bytes()
    assert lib.hy3moe_forward_static(ctypes.byref(big), None, ctypes.byref(w), None, None, None,
                                     None) == sm.HY3MOE_ERR_SCRATCH
    bad = sm.make_config(16, 4096, 192, 8, 1536, 1536, "bf16")
    bad.K = 0
    assert lib.hy3moe_forward_static(ctypes.byref(bad), None, ctypes.byref(w), None, None, None,
                                     None) == -1
    empty = sm.make_config(0, 4096, 192, 8, 1536, 1536, "bf16")
    assert lib.hy3moe_forward_static(ctypes.byref(empty), None, ctypes.byref(w), None, None, None,
                                     None) == 0
    # the Hy3 decode batch fits
    dec = sm.make_config(16, 4096, 192, 8, 1536, 1536, "bf16")
    assert sm.hy3moe_workspace_bytes(dec) <= lib.hy3moe_static_scratch_bytes()


def test_router_split_validates_on_the_host(lib):
    """hy3moe_router_split and hy3moe_router_planes_bytes reject bad shapes,
    precisions, sizes and alignment before launching anything."""
    assert lib.hy3moe_router_planes_bytes(192, 4096, 0) == 3 * 192 * 4096 * 2
    assert lib.hy3moe_router_planes_bytes(192, 4096, 1) == 2 * 192 * 4096 * 2
    assert lib.hy3moe_router_planes_bytes(10, 256, 0) == 3 * 16 * 256 * 2   # E padded to 16
    assert lib.hy3moe_router_planes_bytes(0, 4096, 0) == 0
    assert lib.hy3moe_router_planes_bytes(192, 4000, 0) == 0
    assert lib.hy3moe_router_planes_bytes(192, 4096, 7) == 0
    ok = 1 << 20
    n = 3 * 192 * 4096 * 2
    assert lib.hy3moe_router_split(ok, 192, 4096, 0, ok, n - 1, None) == -3
    assert lib.hy3moe_router_split(ok, 192, 4096, 0, None, n, None) == -1
    assert lib.hy3moe_router_split(ok, 192, 4096, 5, ok, n, None) == -1
    assert lib.hy3moe_router_split(ok, 0, 4096, 0, ok, n, None) == -1
    assert lib.hy3moe_router_split(ok, 192, 4000, 0, ok, n, None) == -2
    assert lib.hy3moe_router_split(ok + 8, 192, 4096, 0, ok, n, None) == -4
    assert lib.hy3moe_router_split(ok, 192, 4096, 0, ok + 4, n, None) == -4


@pytest.mark.parametrize("bad, code", [
    (dict(shared_w_format=3), -1), (dict(shared_act_format=3), -1),
    (dict(shared_w_format=-2), -1),
    # a branch's formats follow the same rules: MXFP8 activations need MXFP4
    # weights, static FP8 needs FP8 weights, MXFP4 needs I_shared % 128 == 0
    (dict(shared_act_format="mxfp8"), -2),
    (dict(shared_w_format="mxfp4", shared_act_format="fp8_static"), -2),
    (dict(shared_w_format="mxfp4", I_shared=1536 + 64), -2),
    (dict(w_format="dtype", act_format="dtype", shared_w_format=None,
          shared_act_format="fp8_static"), -2),
])
def test_shared_formats_are_validated(lib, bad, code):
    raw = {k: v for k, v in bad.items() if isinstance(v, int) and k.startswith("shared_")}
    cfg = cfg_of(CONFIGS["hy3_decode_T16_mixed"],
                 **{k: v for k, v in bad.items() if k not in raw})
    for k, v in raw.items():         # enum values the binding has no name for
        setattr(cfg, k, v)
    assert sm.hy3moe_workspace_bytes(cfg, True) == 0
    L = b.hy3moe_ws_layout()
    assert lib.hy3moe_workspace_layout(ctypes.byref(cfg), ctypes.byref(L)) == code


def test_shared_formats_ignored_without_a_shared_expert(lib):
    cfg = cfg_of(CONFIGS["hy3_decode_T16_mixed"], I_shared=0, shared_act_format="mxfp8")
    L = sm.hy3moe_workspace_layout(cfg)
    assert L.xq_shared == L.xs_shared == 0 and L.total > 0


def test_mixed_layer_needs_each_branch_weights(lib):
    """Routed W4A8 + shared W8A8: the routed E8M0 scales, the shared FP8
    scales and the static activation scales are required; the shared E8M0
    scales and the routed FP8 scales are not."""
    cfg = cfg_of(CONFIGS["hy3_decode_T16_mixed"])
    need = sm.hy3moe_workspace_bytes(cfg, True)
    fw = lib.hy3moe_forward
    names = b.WEIGHT_NAMES
    full = {n: 4096 for n in names}
    full["expert_bias"] = 4096
    for n in ("w_router_planes", "w_gate_scale", "w_up_scale", "w_down_scale", "ws_gate_mx",
              "ws_up_mx", "ws_down_mx"):
        full[n] = None

    def call(d):
        w = b.hy3moe_weights(*[d[n] for n in names])
        return fw(ctypes.byref(cfg), 4096, ctypes.byref(w), 8192, None, None, 4096, need - 1,
                  None)

    assert call(full) == -3                     # every check passed, then the workspace size
    for n in ("ws_scale", "x_scale", "h_scale", "w_gate_mx", "w_up_mx", "w_down_mx"):
        d = dict(full)
        d[n] = None
        assert call(d) == -1, n
    d = dict(full)
    d["ws_scale"] = 4098
    assert call(d) == -4
