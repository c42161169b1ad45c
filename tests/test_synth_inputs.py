"""The seeded input generator: determinism, distributions, bf16 rounding."""
import numpy as np
import pytest
import torch

from synth import (CONFIGS, MoEInputs, bf16_bits_to_f32, f32_to_bf16_bits,
                   make_inputs, random_small)


def test_bf16_rne_matches_torch():
    """torch's float32 -> bfloat16 cast is an independent round-to-nearest-even."""
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.normal(size=100000).astype(np.float32),
                        np.array([1.0, -2.5, 3.0039062, 1.00390625, 1.01171875,
                                  65504.0, 1e-30, -0.0], dtype=np.float32)])
    mine = f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    back = bf16_bits_to_f32(mine)
    np.testing.assert_array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_ties_round_to_even():
    # 1 + 2^-8 is exactly halfway between bf16 neighbours 1 and 1 + 2^-7.
    a = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    np.testing.assert_array_equal(bf16_bits_to_f32(f32_to_bf16_bits(a)),
                                  np.array([1.0, 1.0 + 2.0 ** -6], dtype=np.float32))


def test_determinism_and_independence():
    a, b = make_inputs("tiny_fp32"), make_inputs("tiny_fp32")
    np.testing.assert_array_equal(a.x(), b.x())
    np.testing.assert_array_equal(a.expert(3)[0], b.expert(3)[0])
    assert not np.array_equal(a.expert(3)[0], a.expert(4)[0])
    assert not np.array_equal(make_inputs("tiny_fp32", seed=1).x(), a.x())


def test_decode_and_prefill_share_weights_not_data():
    d = MoEInputs(CONFIGS["hy3_decode_T16"].with_(T=4, H=64, I=32, I_shared=32))
    p = MoEInputs(CONFIGS["hy3_prefill_T8192_skew"].with_(T=4, H=64, I=32, I_shared=32))
    np.testing.assert_array_equal(d.w_router(), p.w_router())
    np.testing.assert_array_equal(d.expert(5)[2], p.expert(5)[2])
    assert not np.array_equal(d.x(), p.x())


def test_distributions_cfg0():
    inp = make_inputs("tiny_fp32")
    c = inp.cfg
    x = inp.x()
    assert x.dtype == np.float32 and x.shape == (c.T, c.H)
    assert abs(x.std() - 1.0) < 0.05
    wr = inp.w_router()
    assert wr.shape == (c.E, c.H) and abs(wr.std() - 0.02) < 0.002
    b = inp.bias()
    assert b.shape == (c.E,) and b.min() >= -0.1 and b.max() <= 0.1
    g, u, d = inp.expert(0)
    assert g.shape == (c.I, c.H) and d.shape == (c.H, c.I)
    assert abs(g.std() - 1 / np.sqrt(c.H)) < 0.1 / np.sqrt(c.H)
    assert abs(d.std() - 1 / np.sqrt(c.I)) < 0.1 / np.sqrt(c.I)


def test_skew_bias_and_softmax_have_expected_kinds():
    p = MoEInputs(CONFIGS["hy3_prefill_T8192_skew"].with_(T=2, H=64, I=32, I_shared=32))
    b = p.bias()
    assert abs(b.std() - 0.3) < 0.1
    s = MoEInputs(CONFIGS["hunyuanimage_softmax_T32768"].with_(T=2, H=64, I=32, I_shared=32))
    assert s.bias() is None and s.cfg.route_mode == 1


def test_bf16_storage_and_stack():
    inp = random_small(1, T=3, H=16, E=3, K=2, I=8, I_shared=8, dtype="bf16")
    assert inp.x().dtype == np.uint16
    wg, wu, wd = inp.stacked_experts(threads=2)
    assert wg.shape == (3, 8, 16) and wd.shape == (3, 16, 8)
    np.testing.assert_array_equal(wg[2], inp.expert(2)[0])


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_config_shapes(name):
    c = CONFIGS[name]
    assert 1 <= c.K <= c.E and c.H % 8 == 0 and c.I % 8 == 0


def test_fp8_codes_and_scales():
    from synth import CONFIGS, MoEInputs
    inp = MoEInputs(CONFIGS["hy3_decode_T16_fp8"].with_T(2).with_(H=256, E=3, I=128, I_shared=64))
    (g, u, d), sc = inp.expert_fp8(1)
    assert g.dtype == np.uint8 and g.shape == (128, 256) and d.shape == (256, 128)
    for q in (g, u, d):
        assert not ((q & 0x7F) == 0x7F).any()          # never the NaN pattern
    assert all(isinstance(s, np.float32) and s > 0 for s in sc)
    (g2, _, _), sc2 = inp.expert_fp8(1)
    assert (g2 == g).all() and sc2 == sc                # reproducible
    (g3, _, _), _ = inp.expert_fp8(2)
    assert (g3 != g).mean() > 0.5                       # independent per expert
    wg, wu, wd, s = inp.stacked_experts_fp8()
    assert (wg[1] == g).all() and s.shape == (3, 3) and s[0, 1] == sc[0]
    sh_codes, sh_sc = inp.shared_fp8()
    assert sh_codes[2].shape == (256, 64) and len(sh_sc) == 3


def test_static_activation_scales():
    inp = MoEInputs(CONFIGS["hy3_prefill_T8192_skew_w8a8"])
    a1, a2 = inp.act_scales()
    assert a1.dtype == np.float32 and a2.dtype == np.float32
    assert a2.shape == (inp.cfg.E + 1,)
    assert a1 == np.float32(4.5 / 448)
    assert (a2 >= np.float32(12 / 448)).all() and (a2 <= np.float32(1.25 * 12 / 448)).all()
    # one model: the decode and prefill W8A8 workloads share the scales
    np.testing.assert_array_equal(MoEInputs(CONFIGS["hy3_decode_T16_w8a8"]).act_scales()[1], a2)
    assert CONFIGS["hy3_decode_T16_w8a8"].act_format == CONFIGS["hy3_prefill_T8192_skew_w8a8"].act_format == "fp8_static"


def test_mxfp4_codes_and_scales():
    inp = MoEInputs(CONFIGS["hy3_decode_T16_mxfp4"].with_(H=256, I=128, I_shared=128, E=4))
    (g, u, d), (sg, su, sd) = inp.expert_mxfp4(1)
    assert g.shape == (128, 128) and d.shape == (256, 64) and g.dtype == np.uint8
    assert sg.shape == (128, 8) and sd.shape == (256, 4)
    import oracle
    wg = oracle.dequant_mxfp4(g, sg)
    # about the spread of the bf16 weights (std 1/sqrt(fan_in)), no NaN
    assert 0.5 / np.sqrt(256) < wg.std() < 1.5 / np.sqrt(256)
    assert np.isfinite(wg).all()
    # deterministic, and the stacked form holds the same bytes
    np.testing.assert_array_equal(inp.expert_mxfp4(1)[0][0], g)
    st = inp.stacked_experts_mxfp4(threads=2)
    np.testing.assert_array_equal(st[0][1], g)
    np.testing.assert_array_equal(st[5][1], sd)
