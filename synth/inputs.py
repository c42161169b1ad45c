"""Seeded synthetic inputs for the Hy3-style MoE FFN layer.

This module is shared by the tests, the benchmark and the CPU oracle's
callers.  It holds no arithmetic of the method itself: it only draws random
tensors with the shapes and distributions of the layer's workloads, rounds
them to bfloat16 where the workload stores bfloat16, and decodes bfloat16 bit
patterns back to exact float64 values.

Shapes follow the Hy3 model facts (hy3 README, "Model facts" table: hidden
4096, 192 routed experts with top-8 plus one shared expert, expert
intermediate 1536) and the HunyuanImage-3.0 MoE reading (64 routed experts,
softmax routing).

Random streams
--------------
Every tensor has its own numpy PCG64 stream,
``default_rng(SeedSequence([seed, key, tensor_id, expert_id]))``, so that any
tensor (and any single expert of a stacked weight) can be regenerated on its
own, in any order, on any number of threads.

* ``key`` is a *model key* for weights (so that the decode and the prefill
  workloads of the same model share one set of weights) and ``1000 + data_id``
  for per-workload data (activations and the expert bias).
* tensor ids: 0 x, 1 router weight, 2 expert bias, 3 gate, 4 up, 5 down,
  6/7/8 shared gate/up/down.

Distributions: x ~ N(0, 1); router weight ~ N(0, 0.02); bias ~ U(-0.1, 0.1)
(or 0.3 * N(0, 1) for the skewed prefill chunk, and none for softmax
routing); gate/up ~ N(0, 1/sqrt(H)); down ~ N(0, 1/sqrt(I)).  The second
parameter of N is the standard deviation.

bfloat16 values are produced from float32 draws by round-to-nearest-even on
the bit pattern and are stored as ``uint16`` arrays of the raw bits.

FP8 expert weights (``w_format == "fp8_e4m3"``) are drawn directly as byte
codes of the OCP FP8 E4M3 layout (sign, 4 exponent bits, 3 mantissa bits),
not by quantising float draws: sign uniform, exponent field
round(N(11.5, 1.3)) clipped to 0..15, mantissa field uniform, and the NaN
pattern (exponent 15, mantissa 7) replaced by mantissa 6.  The encoded
values then have a standard deviation of about 74, and 1 % of them lie in
the top binade (up to 448).  Each matrix gets its own float32 scale
(1 + U(0, 0.25)) / (74 sqrt(fan_in)), so that scale times value has about
the spread of the bf16 weights.  Nothing here decodes the codes: that is
the layer's own (de-quantisation) step.

MXFP4 expert weights (``w_format == "mxfp4"``) are drawn as E2M1 codes
(sign uniform; magnitude 0, 0.5, 1, 1.5, 2, 3, 4, 6 with probabilities
.08, .17, .20, .17, .14, .12, .08, .04, standard deviation about 2.2),
packed two per byte (even element in the low nibble), with one E8M0 scale
per 32 consecutive weights of a row: 2^(round(log2(1 / (2.2 sqrt(fan_in))))
- j), j uniform in {0, 1}, so scale times value has about the spread of the
bf16 weights.

The shared expert may take formats of its own (``shared_w_format``,
``shared_act_format``); its tensors are then drawn in those formats, from
the same streams as above.

Static FP8 activation scales (``act_format == "fp8_static"``, W8A8) stand
in for calibrated ones: a1 = 4.5 / 448 for the layer input (x ~ N(0, 1):
about 7 in a million values saturate) and a2[e] = (1 + U(0, 0.25)) * 12 / 448
for each expert's h (a2[E] for the shared expert), float32.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import numpy as np

T_X, T_WR, T_BIAS, T_GATE, T_UP, T_DOWN, T_SGATE, T_SUP, T_SDOWN = range(9)
T_CODES, T_SCALES = 100, 200     # offsets of the FP8 code and scale streams
T_ASCALES = 300                  # static FP8 activation scales
T_FP4, T_MX = 400, 500           # MXFP4 code and E8M0 scale streams

ROUTE_SIGMOID_BIAS = 0
ROUTE_SOFTMAX = 1


# --------------------------------------------------------------------------
# bfloat16 bit handling (input plumbing, not part of the method)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Works on the IEEE-754 bit pattern: add 0x7FFF plus the lowest kept bit,
    then drop the 16 low bits.  Inputs are finite by construction.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact decode of bfloat16 bits to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact decode of bfloat16 bits to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    data_id: int               # seed id of the workload's activations and expert bias
    model_key: int
    T: int
    H: int
    E: int
    K: int
    I: int
    I_shared: int
    dtype: str                 # "f32" or "bf16": activations and expert weights
    route_mode: int            # ROUTE_SIGMOID_BIAS or ROUTE_SOFTMAX
    scale: float               # router scaling factor applied to routed weights
    renorm_eps: float          # clamp of the renormalisation denominator
    bias_kind: str             # "uniform", "skew" or "none"
    w_format: str = "dtype"    # expert weights: "dtype" (as `dtype`), "fp8_e4m3" or "mxfp4"
    act_format: str = "dtype"  # expert activations: "dtype", "fp8_static" (W8A8) or
                               # "mxfp8" (dynamic, with MXFP4 weights: W4A8)
    shared_w_format: Optional[str] = None    # the shared expert's, None: as the routed ones
    shared_act_format: Optional[str] = None

    @property
    def sw_format(self) -> str:
        """Weight format of the shared expert."""
        return self.w_format if self.shared_w_format is None else self.shared_w_format

    @property
    def sa_format(self) -> str:
        """Activation format of the shared expert."""
        return self.act_format if self.shared_act_format is None else self.shared_act_format

    def with_T(self, T: int) -> "MoEConfig":
        return dataclasses.replace(self, T=int(T))

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# Hy3 router scaling factor (hy3 README "Model facts", MoE routing row; the
# CANN deployment article section 一 lists router_scaling_factor=2.826).
HY3_SCALE = 2.826

CONFIGS: Dict[str, MoEConfig] = {
    "tiny_fp32": MoEConfig("tiny_fp32", 0, 0, T=8, H=256, E=16, K=4, I=128, I_shared=128,
                 dtype="f32", route_mode=ROUTE_SIGMOID_BIAS, scale=HY3_SCALE,
                 renorm_eps=0.0, bias_kind="uniform"),
    "hy3_decode_T16": MoEConfig("hy3_decode_T16", 1, 1, T=16, H=4096, E=192, K=8, I=1536,
                 I_shared=1536, dtype="bf16", route_mode=ROUTE_SIGMOID_BIAS,
                 scale=HY3_SCALE, renorm_eps=0.0, bias_kind="uniform"),
    "hy3_prefill_T8192_skew": MoEConfig("hy3_prefill_T8192_skew", 2, 1, T=8192, H=4096, E=192, K=8,
                 I=1536, I_shared=1536, dtype="bf16",
                 route_mode=ROUTE_SIGMOID_BIAS, scale=HY3_SCALE, renorm_eps=0.0,
                 bias_kind="skew"),
    # Router-only sweep: M in {2, 64, 512, 4096}; the expert weights are not used.
    "hy3_router_only": MoEConfig("hy3_router_only", 3, 1, T=4096, H=4096, E=192, K=8, I=1536,
                 I_shared=1536, dtype="bf16", route_mode=ROUTE_SIGMOID_BIAS,
                 scale=HY3_SCALE, renorm_eps=0.0, bias_kind="uniform"),
    "hunyuanimage_softmax_T32768": MoEConfig("hunyuanimage_softmax_T32768", 4, 4, T=32768, H=4096, E=64,
                 K=8, I=1536, I_shared=1536, dtype="bf16",
                 route_mode=ROUTE_SOFTMAX, scale=1.0, renorm_eps=1e-8,
                 bias_kind="none"),
    # Hy3 decode with FP8 E4M3 expert weights (one scale per matrix).
    "hy3_decode_T16_fp8": MoEConfig("hy3_decode_T16_fp8", 5, 5, T=16, H=4096, E=192, K=8, I=1536,
                 I_shared=1536, dtype="bf16", route_mode=ROUTE_SIGMOID_BIAS,
                 scale=HY3_SCALE, renorm_eps=0.0, bias_kind="uniform",
                 w_format="fp8_e4m3"),
    # Hy3 prefill chunk with the same FP8 experts and a skewed bias.
    "hy3_prefill_T8192_skew_fp8": MoEConfig("hy3_prefill_T8192_skew_fp8", 6, 5, T=8192, H=4096, E=192, K=8,
                 I=1536, I_shared=1536, dtype="bf16",
                 route_mode=ROUTE_SIGMOID_BIAS, scale=HY3_SCALE, renorm_eps=0.0,
                 bias_kind="skew", w_format="fp8_e4m3"),
    # The same two shapes and FP8 experts with static FP8 activations (W8A8).
    "hy3_decode_T16_w8a8": MoEConfig("hy3_decode_T16_w8a8", 7, 5, T=16, H=4096, E=192, K=8, I=1536,
                 I_shared=1536, dtype="bf16", route_mode=ROUTE_SIGMOID_BIAS,
                 scale=HY3_SCALE, renorm_eps=0.0, bias_kind="uniform",
                 w_format="fp8_e4m3", act_format="fp8_static"),
    "hy3_prefill_T8192_skew_w8a8": MoEConfig("hy3_prefill_T8192_skew_w8a8", 8, 5, T=8192, H=4096, E=192, K=8,
                 I=1536, I_shared=1536, dtype="bf16",
                 route_mode=ROUTE_SIGMOID_BIAS, scale=HY3_SCALE, renorm_eps=0.0,
                 bias_kind="skew", w_format="fp8_e4m3", act_format="fp8_static"),
    # Hy3 decode and prefill with MXFP4 experts (bf16 activations).
    "hy3_decode_T16_mxfp4": MoEConfig("hy3_decode_T16_mxfp4", 9, 9, T=16, H=4096, E=192, K=8, I=1536,
                 I_shared=1536, dtype="bf16", route_mode=ROUTE_SIGMOID_BIAS,
                 scale=HY3_SCALE, renorm_eps=0.0, bias_kind="uniform", w_format="mxfp4"),
    "hy3_prefill_T8192_skew_mxfp4": MoEConfig("hy3_prefill_T8192_skew_mxfp4", 10, 9, T=8192, H=4096, E=192, K=8,
                  I=1536, I_shared=1536, dtype="bf16",
                  route_mode=ROUTE_SIGMOID_BIAS, scale=HY3_SCALE, renorm_eps=0.0,
                  bias_kind="skew", w_format="mxfp4"),
    # The same MXFP4 experts with dynamic MXFP8 activations (W4A8).
    "hy3_decode_T16_w4a8": MoEConfig("hy3_decode_T16_w4a8", 11, 9, T=16, H=4096, E=192, K=8, I=1536,
                  I_shared=1536, dtype="bf16", route_mode=ROUTE_SIGMOID_BIAS,
                  scale=HY3_SCALE, renorm_eps=0.0, bias_kind="uniform", w_format="mxfp4",
                  act_format="mxfp8"),
    "hy3_prefill_T8192_skew_w4a8": MoEConfig("hy3_prefill_T8192_skew_w4a8", 12, 9, T=8192, H=4096, E=192, K=8,
                  I=1536, I_shared=1536, dtype="bf16",
                  route_mode=ROUTE_SIGMOID_BIAS, scale=HY3_SCALE, renorm_eps=0.0,
                  bias_kind="skew", w_format="mxfp4", act_format="mxfp8"),
    # Hy3 decode with 32 tokens (the shared expert in two 16-row tiles), on the
    # bf16 and on the FP8 weights, the latter with static FP8 activations.
    "hy3_decode_T32": MoEConfig("hy3_decode_T32", 15, 1, T=32, H=4096, E=192, K=8, I=1536,
                 I_shared=1536, dtype="bf16", route_mode=ROUTE_SIGMOID_BIAS,
                 scale=HY3_SCALE, renorm_eps=0.0, bias_kind="uniform"),
    "hy3_decode_T32_w8a8": MoEConfig("hy3_decode_T32_w8a8", 16, 5, T=32, H=4096, E=192, K=8,
                 I=1536, I_shared=1536, dtype="bf16", route_mode=ROUTE_SIGMOID_BIAS,
                 scale=HY3_SCALE, renorm_eps=0.0, bias_kind="uniform",
                 w_format="fp8_e4m3", act_format="fp8_static"),
    # ... and with 64 tokens (the shared expert in four 16-row tiles), bf16.
    "hy3_decode_T64": MoEConfig("hy3_decode_T64", 17, 1, T=64, H=4096, E=192, K=8, I=1536,
                 I_shared=1536, dtype="bf16", route_mode=ROUTE_SIGMOID_BIAS,
                 scale=HY3_SCALE, renorm_eps=0.0, bias_kind="uniform"),
    # Mixed precision in one layer: the routed experts at W4A8 (the MXFP4
    # experts above, MXFP8 activations) and the shared expert at W8A8 (FP8
    # E4M3 weights, static FP8 activations).
    "hy3_decode_T16_mixed": MoEConfig("hy3_decode_T16_mixed", 13, 9, T=16, H=4096, E=192, K=8,
                  I=1536, I_shared=1536, dtype="bf16", route_mode=ROUTE_SIGMOID_BIAS,
                  scale=HY3_SCALE, renorm_eps=0.0, bias_kind="uniform", w_format="mxfp4",
                  act_format="mxfp8", shared_w_format="fp8_e4m3",
                  shared_act_format="fp8_static"),
    "hy3_prefill_T8192_skew_mixed": MoEConfig("hy3_prefill_T8192_skew_mixed", 14, 9, T=8192,
                  H=4096, E=192, K=8, I=1536, I_shared=1536, dtype="bf16",
                  route_mode=ROUTE_SIGMOID_BIAS, scale=HY3_SCALE, renorm_eps=0.0,
                  bias_kind="skew", w_format="mxfp4", act_format="mxfp8",
                  shared_w_format="fp8_e4m3", shared_act_format="fp8_static"),
}

ROUTER_SWEEP_M = (2, 64, 512, 4096)


def _rng(seed: int, key: int, tensor_id: int, expert_id: int = 0):
    return np.random.default_rng(
        np.random.SeedSequence([int(seed), int(key), int(tensor_id), int(expert_id)]))


def _normal_f32(rng, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    a *= np.float32(std)
    return a.reshape(shape)


def _fp8_codes(rng, shape) -> np.ndarray:
    """E4M3 byte codes with the distribution described in the module notes."""
    n = int(np.prod(shape))
    sign = rng.integers(0, 2, n, dtype=np.int64)
    ex = np.clip(np.rint(rng.normal(11.5, 1.3, n)), 0, 15).astype(np.int64)
    man = rng.integers(0, 8, n, dtype=np.int64)
    man = np.where((ex == 15) & (man == 7), 6, man)
    return ((sign << 7) | (ex << 3) | man).astype(np.uint8).reshape(shape)


def _fp8_scale(rng, fan_in: int) -> np.float32:
    return np.float32((1.0 + 0.25 * rng.random()) / (74.0 * np.sqrt(fan_in)))


_FP4_P = np.array([.08, .17, .20, .17, .14, .12, .08, .04])


def _fp4_packed(rng, rows: int, k: int) -> np.ndarray:
    """[rows, k/2] bytes of E2M1 codes (even element in the low nibble)."""
    n = rows * k
    mag = rng.choice(8, size=n, p=_FP4_P).astype(np.uint8)
    sign = rng.integers(0, 2, n, dtype=np.uint8) << 3
    c = (mag | sign).reshape(rows, k // 2, 2)
    return (c[:, :, 0] | (c[:, :, 1] << 4)).astype(np.uint8)


def _mx_scales(rng, rows: int, k: int, fan_in: int) -> np.ndarray:
    """[rows, k/32] E8M0 codes."""
    base = 127 + int(np.rint(np.log2(1.0 / (2.2 * np.sqrt(fan_in)))))
    return (base - rng.integers(0, 2, (rows, k // 32))).astype(np.uint8)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored tensor (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def _default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class MoEInputs:
    """Lazily generated, seeded inputs of one workload.

    Storage dtypes: x and expert weights are float32 or bf16 bits (uint16)
    per ``cfg.dtype``; the router weight and the bias are always float32.
    """

    def __init__(self, cfg: MoEConfig, seed: int = 0):
        self.cfg = cfg
        self.seed = int(seed)
        self._cache: Dict[Tuple, np.ndarray] = {}

    # ---- data streams (per workload) ----
    def _data_key(self) -> int:
        return 1000 + self.cfg.data_id

    def x(self) -> np.ndarray:
        k = ("x",)
        if k not in self._cache:
            c = self.cfg
            a = _normal_f32(_rng(self.seed, self._data_key(), T_X), (c.T, c.H), 1.0)
            self._cache[k] = _store(a, c.dtype)
        return self._cache[k]

    def bias(self) -> Optional[np.ndarray]:
        c = self.cfg
        if c.bias_kind == "none":
            return None
        k = ("bias",)
        if k not in self._cache:
            rng = _rng(self.seed, self._data_key(), T_BIAS)
            if c.bias_kind == "uniform":
                b = rng.uniform(-0.1, 0.1, size=c.E).astype(np.float32)
            elif c.bias_kind == "skew":
                b = (np.float32(0.3) * rng.standard_normal(c.E, dtype=np.float32))
            else:
                raise ValueError(c.bias_kind)
            self._cache[k] = np.ascontiguousarray(b, dtype=np.float32)
        return self._cache[k]

    # ---- model streams (shared between workloads of one model) ----
    def w_router(self) -> np.ndarray:
        k = ("wr",)
        if k not in self._cache:
            c = self.cfg
            self._cache[k] = _normal_f32(_rng(self.seed, c.model_key, T_WR), (c.E, c.H), 0.02)
        return self._cache[k]

    def expert(self, e: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """(gate [I,H], up [I,H], down [H,I]) of routed expert ``e``, stored dtype."""
        c = self.cfg
        if c.w_format != "dtype":
            raise ValueError("quantised expert weights: use expert_fp8() or expert_mxfp4()")
        mk = c.model_key
        g = _normal_f32(_rng(self.seed, mk, T_GATE, e), (c.I, c.H), 1.0 / np.sqrt(c.H))
        u = _normal_f32(_rng(self.seed, mk, T_UP, e), (c.I, c.H), 1.0 / np.sqrt(c.H))
        d = _normal_f32(_rng(self.seed, mk, T_DOWN, e), (c.H, c.I), 1.0 / np.sqrt(c.I))
        return _store(g, c.dtype), _store(u, c.dtype), _store(d, c.dtype)

    def shared(self) -> Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
        c = self.cfg
        if c.I_shared == 0:
            return None
        if c.sw_format != "dtype":
            raise ValueError("quantised expert weights: use shared_fp8() or shared_mxfp4()")
        k = ("shared",)
        if k not in self._cache:
            mk, Is = c.model_key, c.I_shared
            g = _normal_f32(_rng(self.seed, mk, T_SGATE), (Is, c.H), 1.0 / np.sqrt(c.H))
            u = _normal_f32(_rng(self.seed, mk, T_SUP), (Is, c.H), 1.0 / np.sqrt(c.H))
            d = _normal_f32(_rng(self.seed, mk, T_SDOWN), (c.H, Is), 1.0 / np.sqrt(Is))
            self._cache[k] = (_store(g, c.dtype), _store(u, c.dtype), _store(d, c.dtype))
        return self._cache[k]

    def stacked_experts(self, threads: Optional[int] = None):
        """All routed experts stacked: gate/up [E,I,H], down [E,H,I] (stored dtype)."""
        c = self.cfg
        st = np.uint16 if c.dtype == "bf16" else np.float32
        wg = np.empty((c.E, c.I, c.H), dtype=st)
        wu = np.empty((c.E, c.I, c.H), dtype=st)
        wd = np.empty((c.E, c.H, c.I), dtype=st)

        def job(e):
            g, u, d = self.expert(e)
            wg[e], wu[e], wd[e] = g, u, d

        with ThreadPoolExecutor(threads or _default_threads()) as ex:
            list(ex.map(job, range(c.E)))
        return wg, wu, wd

    # ---- FP8 expert weights (w_format == "fp8_e4m3") ----
    def expert_fp8(self, e: int):
        """((gate, up, down) uint8 E4M3 codes, (s_gate, s_up, s_down) float32) of expert e."""
        c = self.cfg
        mk = c.model_key
        codes = (_fp8_codes(_rng(self.seed, mk, T_CODES + T_GATE, e), (c.I, c.H)),
                 _fp8_codes(_rng(self.seed, mk, T_CODES + T_UP, e), (c.I, c.H)),
                 _fp8_codes(_rng(self.seed, mk, T_CODES + T_DOWN, e), (c.H, c.I)))
        rs = _rng(self.seed, mk, T_SCALES, e)
        scales = (_fp8_scale(rs, c.H), _fp8_scale(rs, c.H), _fp8_scale(rs, c.I))
        return codes, scales

    def shared_fp8(self):
        c = self.cfg
        if c.I_shared == 0:
            return None
        k = ("shared_fp8",)
        if k not in self._cache:
            mk, Is = c.model_key, c.I_shared
            codes = (_fp8_codes(_rng(self.seed, mk, T_CODES + T_SGATE), (Is, c.H)),
                     _fp8_codes(_rng(self.seed, mk, T_CODES + T_SUP), (Is, c.H)),
                     _fp8_codes(_rng(self.seed, mk, T_CODES + T_SDOWN), (c.H, Is)))
            rs = _rng(self.seed, mk, T_SCALES + T_SGATE)
            scales = (_fp8_scale(rs, c.H), _fp8_scale(rs, c.H), _fp8_scale(rs, Is))
            self._cache[k] = (codes, scales)
        return self._cache[k]

    def stacked_experts_fp8(self, threads: Optional[int] = None):
        """Codes gate/up [E,I,H], down [E,H,I] (uint8) and scales [3, E] (float32)."""
        c = self.cfg
        wg = np.empty((c.E, c.I, c.H), dtype=np.uint8)
        wu = np.empty((c.E, c.I, c.H), dtype=np.uint8)
        wd = np.empty((c.E, c.H, c.I), dtype=np.uint8)
        sc = np.empty((3, c.E), dtype=np.float32)

        def job(e):
            (g, u, d), s = self.expert_fp8(e)
            wg[e], wu[e], wd[e] = g, u, d
            sc[:, e] = s

        with ThreadPoolExecutor(threads or _default_threads()) as ex:
            list(ex.map(job, range(c.E)))
        return wg, wu, wd, sc

    # ---- MXFP4 expert weights (w_format == "mxfp4") ----
    def expert_mxfp4(self, e: int):
        """((gate, up, down) packed codes, (gate, up, down) E8M0 scales) of expert e."""
        c = self.cfg
        mk = c.model_key
        shapes = ((c.I, c.H), (c.I, c.H), (c.H, c.I))
        ids = (T_GATE, T_UP, T_DOWN)
        codes = tuple(_fp4_packed(_rng(self.seed, mk, T_FP4 + t, e), *sh)
                      for t, sh in zip(ids, shapes))
        scales = tuple(_mx_scales(_rng(self.seed, mk, T_MX + t, e), sh[0], sh[1], sh[1])
                       for t, sh in zip(ids, shapes))
        return codes, scales

    def shared_mxfp4(self):
        c = self.cfg
        if c.I_shared == 0:
            return None
        k = ("shared_mxfp4",)
        if k not in self._cache:
            mk, Is = c.model_key, c.I_shared
            shapes = ((Is, c.H), (Is, c.H), (c.H, Is))
            ids = (T_SGATE, T_SUP, T_SDOWN)
            codes = tuple(_fp4_packed(_rng(self.seed, mk, T_FP4 + t), *sh)
                          for t, sh in zip(ids, shapes))
            scales = tuple(_mx_scales(_rng(self.seed, mk, T_MX + t), sh[0], sh[1], sh[1])
                           for t, sh in zip(ids, shapes))
            self._cache[k] = (codes, scales)
        return self._cache[k]

    def stacked_experts_mxfp4(self, threads: Optional[int] = None):
        """Packed codes gate/up [E,I,H/2], down [E,H,I/2] and E8M0 scales
        gate/up [E,I,H/32], down [E,H,I/32] (uint8)."""
        c = self.cfg
        wg = np.empty((c.E, c.I, c.H // 2), dtype=np.uint8)
        wu = np.empty_like(wg)
        wd = np.empty((c.E, c.H, c.I // 2), dtype=np.uint8)
        sg = np.empty((c.E, c.I, c.H // 32), dtype=np.uint8)
        su = np.empty_like(sg)
        sd = np.empty((c.E, c.H, c.I // 32), dtype=np.uint8)

        def job(e):
            (g, u, d), (a, b2, dd) = self.expert_mxfp4(e)
            wg[e], wu[e], wd[e], sg[e], su[e], sd[e] = g, u, d, a, b2, dd

        with ThreadPoolExecutor(threads or _default_threads()) as ex:
            list(ex.map(job, range(c.E)))
        return wg, wu, wd, sg, su, sd

    def act_scales(self):
        """Static FP8 activation scales: (a1 float32, a2 float32 [E + 1])."""
        c = self.cfg
        rs = _rng(self.seed, c.model_key, T_ASCALES)
        a2 = ((1.0 + 0.25 * rs.random(c.E + 1)) * (12.0 / 448.0)).astype(np.float32)
        return np.float32(4.5 / 448.0), a2

    # ---- float64 views for the oracle ----
    def x_f64(self) -> np.ndarray:
        return to_f64(self.x(), self.cfg.dtype)

    def expert_f64(self, e: int):
        return tuple(to_f64(a, self.cfg.dtype) for a in self.expert(e))

    def shared_f64(self):
        s = self.shared()
        return None if s is None else tuple(to_f64(a, self.cfg.dtype) for a in s)


def make_inputs(name: str, seed: int = 0, T: Optional[int] = None) -> MoEInputs:
    cfg = CONFIGS[name]
    if T is not None:
        cfg = cfg.with_T(T)
    return MoEInputs(cfg, seed)


def random_small(seed: int, T: int, H: int, E: int, K: int, I: int, I_shared: int,
                 dtype: str = "f32", route_mode: int = ROUTE_SIGMOID_BIAS,
                 scale: float = HY3_SCALE, renorm_eps: float = 0.0,
                 bias_kind: str = "uniform", w_format: str = "dtype",
                 act_format: str = "dtype", shared_w_format: Optional[str] = None,
                 shared_act_format: Optional[str] = None) -> MoEInputs:
    """A small ad-hoc workload with the same distributions (for property tests)."""
    cfg = MoEConfig(f"small_{seed}", 900 + (seed % 97), 900 + seed, T=T, H=H, E=E, K=K,
                    I=I, I_shared=I_shared, dtype=dtype, route_mode=route_mode,
                    scale=scale, renorm_eps=renorm_eps, bias_kind=bias_kind,
                    w_format=w_format, act_format=act_format,
                    shared_w_format=shared_w_format, shared_act_format=shared_act_format)
    return MoEInputs(cfg, seed)
