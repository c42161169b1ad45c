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
from gpu_util import grid_step, h_error_bound, log

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


@pytest.mark.parametrize("T, E, H, path_rows", [(400, 8, 512, 256), (300, 24, 512, 128),
                                                (16, 16, 256, None)])
def test_w8a8_codes_in_the_workspace(dev, T, E, H, path_rows):
    """The quantised activations the forward leaves in its workspace: x codes
    bit-exact against the oracle's quantiser.  h is quantised as the layer's
    bf16 tensor, with a correctly rounded division by a2 on both sides, and
    the GPU's float32 h lies within an accumulation error bound dh of the
    float64 h: its code must lie between the codes of h - dh and h + dh
    (both steps are monotone), and equal the oracle's where those agree.  Where the
    layout reports code rows (a8_codes: the large-tile path, and the
    weight-streaming path when H, I and I_shared are multiples of 128): E4M3
    bytes; otherwise their bf16 values."""
    from gpu_util import a8_of, config_of, expert_cache, shared_f64, to_torch, upload_weights
    from synth import random_small
    inp = random_small(50 + T, T=T, H=H, E=E, K=4, I=256, I_shared=128, dtype="bf16",
                       w_format="fp8_e4m3", act_format="fp8_static")
    c = inp.cfg
    cfg = config_of(inp)
    L = sm.hy3moe_workspace_layout(cfg)
    if path_rows is not None:
        assert L.tile_rows == path_rows
    codes_path = bool(L.a8_codes)
    ws = sm.alloc_workspace(cfg, True, dev)
    weights = upload_weights(inp, dev)
    x = to_torch(inp.x(), c.dtype, dev)
    sm.forward(cfg, x, weights, workspace=ws)
    torch.cuda.synchronize()
    wsh = ws.cpu().numpy()
    a1, a2 = a8_of(inp)

    def values(off, n):   # the stored activations as E4M3 values
        if codes_path:
            return oracle.fp8_e4m3_value(wsh[off:off + n])
        bits = wsh[off:off + 2 * n].view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)

    # x: bit-exact
    x64 = inp.x_f64()
    qx = oracle.quant_e4m3(x64, a1)
    gx = values(L.xq, c.T * c.H).reshape(c.T, c.H)
    np.testing.assert_array_equal(gx, oracle.fp8_e4m3_value(qx))

    # h: per group, in expert-major row order
    def i32(off, n):
        return wsh[off:off + 4 * n].view(np.int32)
    offsets = i32(L.offsets, c.E + 2)
    R = c.T * c.K + c.T
    sorted_token = i32(L.sorted_token, R)
    ldh = max(c.I, c.I_shared)
    xh = oracle.quant_dequant_e4m3(x64, a1)
    experts = expert_cache(inp)
    shared = shared_f64(inp)
    n_all = n_near = 0
    for g in range(c.E + 1):
        r0, r1 = offsets[g], offsets[g + 1]
        if r1 == r0:
            continue
        wg, wu, _ = experts(g) if g < c.E else shared
        Ig = wg.shape[0]
        a = xh[sorted_token[r0:r1]]
        gg, uu = a @ wg.T, a @ wu.T
        got = np.stack([values(L.h + (r * ldh) * (1 if codes_path else 2), Ig)
                        for r in range(r0, r1)])
        u32 = 2.0 ** -24
        h64, dh = h_error_bound(a, wg, wu, (1024 * 2.0 ** -23) if codes_path else 64 * u32)
        ref = oracle.fp8_e4m3_value(oracle.quant_e4m3(oracle.round_bf16(h64), a2[g]))
        # the GPU's float32 h lies in [h - dh, h + dh]; bf16 rounding and the
        # quantisation are monotone, so its code lies between those of the
        # interval's ends and equals the oracle's where the two ends agree
        lo = oracle.fp8_e4m3_value(oracle.quant_e4m3(oracle.round_bf16(h64 - dh), a2[g]))
        hi = oracle.fp8_e4m3_value(oracle.quant_e4m3(oracle.round_bf16(h64 + dh), a2[g]))
        near = lo != hi
        diff = got != ref
        assert ((got >= np.minimum(lo, hi)) & (got <= np.maximum(lo, hi))).all()
        bad = np.argwhere(diff & ~near)
        for i, j in bad[:4]:
            log(f"  group {g} row {i} col {j}: g={gg[i, j]:.9g} u={uu[i, j]:.9g} "
                f"h={h64[i, j]:.9g} bf16(h)={oracle.round_bf16(h64[i, j]):.9g} "
                f"got={got[i, j]} ref={ref[i, j]} dh={dh[i, j]:.3g}")
        assert bad.size == 0, f"{bad.shape[0]} codes off beyond the bound in group {g}"
        big_step = grid_step(np.maximum(np.abs(got), np.abs(ref)))
        assert (np.abs(got - ref) <= big_step * (1 + 1e-12)).all()
        n_all += got.size
        n_near += int(near.sum())
    log(f"  T={T}: x codes exact ({c.T * c.H}); h codes {n_all}, "
        f"{n_near} with an ambiguous code (the interval's ends quantise differently)")
    assert n_near < (0.3 if codes_path else 0.03) * n_all


@pytest.mark.parametrize("T, E", [(1, 16), (16, 16), (400, 8)])
def test_w4a8_codes_in_the_workspace(dev, T, E):
    """Dynamic MXFP8 activations of a W4A8 forward on the paths that multiply
    codes (weight-streaming at T <= 64, large tiles at T = 400 over 8 experts):
    x codes and block scales bit-exact against the oracle.  h: each block
    scale equal to the oracle's unless the block's amax lies within the
    accumulation error bound of a power of two (then one apart); each value
    (code x scale) within the bound (plus bf16 rounding and one grid step) of
    the float64 h; and fewer than 1% of the values different from the
    oracle's."""
    from gpu_util import config_of, expert_cache, shared_f64, to_torch, upload_weights
    from synth import random_small
    inp = random_small(90 + T, T=T, H=256, E=E, K=4, I=128, I_shared=128, dtype="bf16",
                       w_format="mxfp4", act_format="mxfp8")
    c = inp.cfg
    cfg = config_of(inp)
    L = sm.hy3moe_workspace_layout(cfg)
    assert L.tile_rows != 128, "this case must take a path that multiplies codes"
    ws = sm.alloc_workspace(cfg, True, dev)
    weights = upload_weights(inp, dev)
    x = to_torch(inp.x(), c.dtype, dev)
    sm.forward(cfg, x, weights, workspace=ws)
    torch.cuda.synchronize()
    wsh = ws.cpu().numpy()
    x64 = inp.x_f64()
    qx, sx = oracle.quant_mxfp8(x64)
    np.testing.assert_array_equal(wsh[L.xs:L.xs + c.T * c.H // 32].reshape(c.T, -1), sx)
    np.testing.assert_array_equal(wsh[L.xq:L.xq + c.T * c.H].reshape(c.T, c.H), qx)
    offsets = wsh[L.offsets:L.offsets + 4 * (c.E + 2)].view(np.int32)
    R = c.T * c.K + c.T
    sorted_token = wsh[L.sorted_token:L.sorted_token + 4 * R].view(np.int32)
    ldh = max(c.I, c.I_shared)
    hq = wsh[L.hq:L.hq + R * ldh].reshape(R, ldh)
    hs = wsh[L.hs:L.hs + R * ldh // 32].reshape(R, ldh // 32)
    xh = oracle.dequant_mxfp8(qx, sx)
    experts = expert_cache(inp)
    shared = shared_f64(inp)
    n_diff = n_all = n_scale = 0
    for g in range(c.E + 1):
        r0, r1 = offsets[g], offsets[g + 1]
        if r1 == r0:
            continue
        wg, wu, _ = experts(g) if g < c.E else shared
        Ig = wg.shape[0]
        a = xh[sorted_token[r0:r1]]
        h64, dh = h_error_bound(a, wg, wu, 1024 * 2.0 ** -23)
        hb = oracle.round_bf16(h64)
        _, ref_sc = oracle.quant_mxfp8(hb)
        ref = oracle.quant_dequant_mxfp8(hb)
        got_sc = hs[r0:r1, :Ig // 32]
        got = oracle.dequant_mxfp8(hq[r0:r1, :Ig], got_sc)
        # block scales: the exponent of the block's amax, less 8
        blk = lambda v: v.reshape(v.shape[0], -1, 32)
        amax = np.abs(blk(hb)).max(axis=2)
        slack = blk(dh).max(axis=2) + 2.0 ** -8 * amax
        sdiff = got_sc.astype(np.int64) - ref_sc.astype(np.int64)
        edge = np.exp2(np.maximum(got_sc, ref_sc).astype(np.float64) - 127 + 8)
        ok_sc = (sdiff == 0) | ((np.abs(sdiff) == 1) & (np.abs(amax - edge) <= slack))
        if not ok_sc.all():
            i, b = np.argwhere(~ok_sc)[0]
            log(f"  group {g} row {i} block {b}: amax={amax[i, b]:.9g} "
                f"scale code got={got_sc[i, b]} ref={ref_sc[i, b]}")
        assert ok_sc.all()
        n_scale += int((sdiff != 0).sum())
        # values: |got - h| within the GEMM bound, bf16 rounding of h, and a
        # grid step of the stored code (rounding, or saturation at 448)
        sc = np.repeat(oracle.e8m0_value(got_sc), 32, axis=1)
        step = grid_step(np.abs(got) / sc) * sc
        sat = np.maximum(np.abs(h64) + dh - 448.0 * sc, 0.0)
        allowed = dh + 2.0 ** -8 * np.abs(h64) + step + sat
        bad = np.abs(got - h64) > allowed * (1 + 1e-12)
        if bad.any():
            i, j = np.argwhere(bad)[0]
            log(f"  group {g} row {i} col {j}: h={h64[i, j]:.9g} dh={dh[i, j]:.3g} "
                f"got={got[i, j]} ref={ref[i, j]}")
        assert not bad.any()
        n_diff += int((got != ref).sum())
        n_all += got.size
    log(f"  T={T}: x codes exact; h values {n_all}, {n_diff} differ from the oracle's, "
        f"{n_scale} block scales one apart")
    assert n_diff < 0.01 * n_all


def crafted_mx_rows(rng, H: int) -> np.ndarray:
    """Rows of bf16-exact float32 values whose 32-value blocks hit every
    decision of the MXFP8 quantiser: all-zero and negative-zero blocks;
    blocks whose amax scales to exactly 448 with the other values on E4M3
    codes or on the midpoints between neighbouring codes (ties to even);
    amax mantissas up to 1 + 127/128 (scaled values in (448, 512)
    saturate); block exponents from -100 to 100; bf16 subnormal blocks (E8M0
    code 0); and random signed blocks spanning 2^20 in magnitude."""
    vals = oracle.fp8_e4m3_value(np.arange(0x7F, dtype=np.uint8))   # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    blocks = [np.zeros(32), -np.zeros(32)]
    for m in (-100, -3, 0, 5, 100):
        sc = 2.0 ** (m - 8)
        for pool in (vals, mids):
            for b0 in range(0, len(pool), 31):
                part = pool[b0:b0 + 31]
                blk = np.concatenate([[1.75 * 2.0 ** m], part * sc,
                                      np.zeros(31 - len(part))])
                sign = np.where(rng.random(32) < 0.5, -1.0, 1.0)
                blocks.append(blk * sign)
        for mant in (1.0, 1.5, 1.75, 1.78125, 1.8125, 1.875, 1.9921875):
            blk = np.concatenate([[mant * 2.0 ** m], rng.choice(vals, 31) * sc])
            blocks.append(blk)
    for k in range(4):   # bf16 subnormals: multiples of 2^-133 below 2^-126
        blocks.append(rng.integers(0, 128, 32) * 2.0 ** -133 * (-1) ** k)
    for _ in range(16):   # rounded to bf16 below
        mag = np.exp2(rng.uniform(-20, 0, 32) + rng.integers(-60, 60))
        blocks.append(mag * np.where(rng.random(32) < 0.5, -1.0, 1.0))
    flat = np.concatenate(blocks)
    per_row = H // 32
    n_rows = -(-len(blocks) // per_row)
    flat = np.concatenate([flat, np.zeros(n_rows * H - flat.size)])
    x = flat.reshape(n_rows, H).astype(np.float32)
    # to bf16, nearest even (exact for all but the random blocks)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def test_mxfp8_quantiser_crafted_blocks(dev):
    """The W4A8 forward's x quantisation on crafted blocks: codes and E8M0
    scales bit-exact against the oracle's MXFP8 quantiser, in the layout the
    weight-streaming kernels read, and the same from the large-tile path."""
    from gpu_util import config_of, to_torch, upload_weights
    from synth import random_small
    rng = np.random.default_rng(7)
    H = 256
    x32 = crafted_mx_rows(rng, H)
    qx, sx = oracle.quant_mxfp8(x32.astype(np.float64))
    for T in (x32.shape[0], 400):
        xx = np.resize(x32, (T, H))   # the large-tile case repeats the rows
        inp = random_small(7, T=T, H=H, E=8, K=4, I=128, I_shared=128, dtype="bf16",
                           w_format="mxfp4", act_format="mxfp8")
        cfg = config_of(inp)
        L = sm.hy3moe_workspace_layout(cfg)
        assert L.tile_rows != 128
        ws = sm.alloc_workspace(cfg, True, dev)
        xb = (xx.view(np.uint32) >> 16).astype(np.uint16)   # bf16 bits
        sm.forward(cfg, to_torch(xb, "bf16", dev), upload_weights(inp, dev), workspace=ws)
        torch.cuda.synchronize()
        wsh = ws.cpu().numpy()
        got_s = wsh[L.xs:L.xs + T * H // 32].reshape(T, -1)
        got_q = wsh[L.xq:L.xq + T * H].reshape(T, H)
        ref_q, ref_s = np.resize(qx, (T, H)), np.resize(sx, (T, H // 32))
        bad = np.argwhere(got_s != ref_s)
        for i, b in bad[:4]:
            log(f"  row {i} block {b}: scale got {got_s[i, b]} ref {ref_s[i, b]}")
        np.testing.assert_array_equal(got_s, ref_s)
        bad = np.argwhere(got_q != ref_q)
        for i, j in bad[:4]:
            log(f"  row {i} col {j}: x={xx[i, j]!r} code got {got_q[i, j]:#04x} "
                f"ref {ref_q[i, j]:#04x} (scale code {ref_s[i, j // 32]})")
        np.testing.assert_array_equal(got_q, ref_q)
        log(f"  T={T}: {T * H // 32} blocks bit-exact (path rows {L.tile_rows})")
