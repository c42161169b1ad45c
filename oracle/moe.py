"""CPU oracle of the Hy3-style MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only the tests, the smoke check and the benchmark's CPU
baseline leg do.  It shares no code with the HIP library.

It is a plain, slow, float64 statement of what the layer computes.  Inputs
arrive as exact float64 values (bfloat16 and float32 widen to float64 without
error), and nothing is rounded on the way.

Sources (the pages this follows):

* hy3 README ("hy3 — tencent/Hy3 GGUF Converter and Inference Engine"),
  "Model facts" table: 192 routed experts, top-8, plus one shared expert that
  is always active.  MoE routing row: sigmoid of the router logits; the top-8
  are chosen on sigmoid + expert_bias; the combine weights are the unbiased
  sigmoid scores, renormalised to sum 1 and then scaled by 2.826.
* CANN deployment article on Hy3, section 一: HYV3Config defaults
  router_scaling_factor=2.826, num_experts_per_tok=8, route_norm=True,
  moe_router_use_sigmoid=True.
* HunyuanImage 3.0 MoE reading, "HunyuanTopKGate easy_topk" path: router
  Linear H->E without bias, float32 weight with activations cast to float32;
  softmax over the expert axis, top-K, sum of the K picked probabilities
  clamped at 1e-8, division.  "Routed Experts" eager path: tokens repeated K
  times, one mask per expert, each expert run on its selected rows, outputs
  written back, reshaped to [T, K, H], multiplied by the routing weights and
  summed over K.  "Shared MLP": one expert that every token goes through,
  added to the routed output.  The experts use SiLU/SwiGLU
  (down(silu(gate(a)) * up(a))).

Readings where the pages are silent (each is listed with the other readings
in the design notes):

* ties in the selection score go to the lower expert index, and the K picked
  indices are returned in descending selection score;
* the bias is added to the sigmoid score, not to the logit;
* the shared expert has weight 1 (the 2.826 factor is for routed experts);
* sigmoid mode has no renormalisation epsilon (a sum of sigmoids is > 0);
* selection is flat over all E experts (no expert groups).

FP8 expert weights (the CANN deployment article, section 8.2 "量化策略":
FP8 W8A8 weights with tensor-wise scales, routed experts quantised further
to MXFP4 there; Hy3 Preview inference case, section 12: W8A8 among the
deployed precisions).  A weight matrix is stored as one byte per element in
the OCP FP8 E4M3 encoding (1 sign, 4 exponent bits with bias 7, 3 mantissa
bits; subnormals at exponent field 0; no infinities; S.1111.111 is NaN) and
one float32 scale per matrix; its value is scale * decode(code).  The pages
fix neither the encoding variant nor the scale granularity beyond "tensor":
E4M3 as above and one scale per expert matrix is the reading taken here.
The oracle dequantises exactly (every E4M3 value times a float32 scale is
exact in float64) and then runs the same float64 layer.

MXFP4 expert weights (the CANN deployment article, section 8.2: routed
experts W4A8 with W4 = MXFP4; section 五: MXFP4 weights derived from the
MXFP8 conversion).  OCP microscaling: each block of 32 consecutive weights
of a row (along the reduction axis) shares one E8M0 scale 2^(s-127), and
each weight is an FP4 E2M1 code (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 with a
sign); two codes per byte, the even element in the low nibble (the packing
order is a reading: the pages do not give one).  Built weight-only
(W4A16): activations stay bf16, and the oracle runs the float64 layer on
the exactly dequantised weights.

Dynamic MXFP8 activations (W4A8 with MXFP4 weights; the CANN article,
section 8.2: W4A8, and section 六: the MXFP4 path produces dynamic MXFP8
values).  Each block of 32 consecutive values of an activation row (x
along H, h along I) shares an E8M0 scale set from the block's maximum as
the OCP microscaling conversion does (floor(log2 amax) - 8), and the
values are E4M3 codes of v / scale (saturating, nearest even), decided in
float32.  The dynamic quantisation is an operator on the layer's bfloat16
activation tensors: x is bfloat16 already, and h is the SwiGLU output
rounded to bfloat16 (round_bf16) before it is quantised.

Static FP8 activations (W8A8; the CANN article, section 8.2 and the FP8
path of section 六, where an FP8 Linear quantises its input with a static
per-tensor input scale).  The expert input x is quantised with one float32
scale a1 of the layer, and each expert's h (the down projection's input)
with that expert's float32 scale a2[e] (a2[E]: shared expert): code =
E4M3(v / a), saturating, round to nearest even, decided in float32; the
GEMMs then run on scale times value.  What the FP8 Linear receives is the
layer's activation tensor in the model's dtype: x is bfloat16 already, and
h is the SwiGLU output rounded to bfloat16 (round_bf16) before it is
quantised, exactly as for the dynamic MXFP8 quantiser below, so both
activation quantisers see the same tensor.  Granularity, saturation,
rounding and the precision of the decision are readings: the pages name
only "static per-tensor".

Parity pins: every public function is pinned by a test in
``tests/test_oracle_pins.py`` (hand-derived golden values, brute force over
all K-subsets, a loop-only dense evaluation, closed forms and invariants).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional, Sequence, Tuple

import numpy as np

ROUTE_SIGMOID_BIAS = 0
ROUTE_SOFTMAX = 1

ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


# --------------------------------------------------------------------------
# Router
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * w_router[e, h]   (bias-free linear H->E).

    HunyuanImage 3.0 MoE reading, HunyuanTopKGate: ``wg`` is a bias-free
    float32 Linear of weight shape [E, H]; the hy3 README keeps the router
    gate in F32.  Evaluated in float64, where every product of a bf16 or fp32
    activation with an fp32 weight is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    return x @ w.T


def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + exp(-z)), evaluated without overflow."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Softmax over the expert axis (dim=1), with the row maximum subtracted."""
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=1, keepdims=True)


def topk_desc(score: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of each row, in descending score.

    Equal scores are ordered by ascending expert index (a stable sort of the
    negated scores), so the lower index wins a tie at the k-th place.
    """
    order = np.argsort(-np.asarray(score, dtype=np.float64), axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


@dataclasses.dataclass
class Route:
    idx: np.ndarray        # [T, K] int64, descending selection score
    weight: np.ndarray     # [T, K] float64 combine weights
    margin: np.ndarray     # [T] selection score of the K-th minus the (K+1)-th pick
    select_score: np.ndarray  # [T, E] the score the selection is taken on
    prob: np.ndarray       # [T, E] sigmoid scores / softmax probabilities


def route_from_logits(logits: np.ndarray, K: int, mode: int = ROUTE_SIGMOID_BIAS,
                      bias: Optional[np.ndarray] = None, scale: float = 2.826,
                      renorm_eps: float = 1e-8) -> Route:
    """Scores, top-K selection and combine weights from router logits.

    Sigmoid mode (hy3 README, Model facts / MoE routing; HYV3Config
    moe_router_use_sigmoid, route_norm, router_scaling_factor):
        s = sigmoid(L);  pick top-K of s + bias;
        w_j = scale * s[pick_j] / sum_j' s[pick_j'].
    The bias only steers the choice; the weights use the unbiased s.

    Softmax mode (HunyuanImage 3.0 MoE reading, easy_topk):
        p = softmax(L);  pick top-K of p;
        w_j = p[pick_j] / max(sum_j' p[pick_j'], renorm_eps).
    No bias, no scale.
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    if not (1 <= K <= E):
        raise ValueError("need 1 <= K <= E")
    if mode == ROUTE_SIGMOID_BIAS:
        prob = sigmoid(L)
        b = np.zeros(E) if bias is None else np.asarray(bias, dtype=np.float64)
        sel = prob + b[None, :]
    elif mode == ROUTE_SOFTMAX:
        prob = softmax_rows(L)
        sel = prob
    else:
        raise ValueError("unknown route mode")
    idx = topk_desc(sel, K)
    weight = combine_weights(prob, idx, mode, scale, renorm_eps)
    if K < E:
        ssorted = -np.sort(-sel, axis=1)
        margin = ssorted[:, K - 1] - ssorted[:, K]
    else:
        margin = np.full(T, np.inf)
    return Route(idx=idx, weight=weight, margin=margin, select_score=sel, prob=prob)


def combine_weights(prob: np.ndarray, idx: np.ndarray, mode: int = ROUTE_SIGMOID_BIAS,
                    scale: float = 2.826, renorm_eps: float = 1e-8) -> np.ndarray:
    """Combine weights of the picks ``idx`` [T, K] from the unbiased scores.

    Sigmoid mode (hy3 README, MoE routing row; HYV3Config route_norm and
    router_scaling_factor): the picked sigmoid scores renormalised to sum 1,
    times ``scale``.  Softmax mode (HunyuanImage 3.0 MoE reading, easy_topk):
    the picked probabilities divided by their sum clamped below at
    ``renorm_eps``.  The selection bias never enters: ``prob`` holds the
    unbiased scores.
    """
    prob = np.asarray(prob, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    picked = np.take_along_axis(prob, idx, axis=1)
    tot = picked.sum(axis=1, keepdims=True)
    if mode == ROUTE_SIGMOID_BIAS:
        return scale * (picked / tot)
    return picked / np.maximum(tot, renorm_eps)


def route(x, w_router, K: int, mode: int = ROUTE_SIGMOID_BIAS, bias=None,
          scale: float = 2.826, renorm_eps: float = 1e-8) -> Route:
    """The gate of the layer: router logits, then scores/selection/weights."""
    return route_from_logits(router_logits(x, w_router), K, mode, bias, scale, renorm_eps)


# --------------------------------------------------------------------------
# FP8 expert weights
# --------------------------------------------------------------------------
def fp8_e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Value of OCP FP8 E4M3 codes (uint8) in float64; NaN for S.1111.111.

    Normal codes (exponent field e in 1..15): (-1)^s * (1 + m/8) * 2^(e-7).
    Subnormal codes (e = 0): (-1)^s * (m/8) * 2^-6.  E4M3 has no infinities:
    exponent field 15 is an ordinary binade except for mantissa 7 (NaN), so
    the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, out)


def dequant_fp8(codes: np.ndarray, scale) -> np.ndarray:
    """scale * E4M3 value of every code, in float64 (one scale per matrix)."""
    return np.float64(np.float32(scale)) * fp8_e4m3_value(codes)


def fp4_e2m1_value(nibbles: np.ndarray) -> np.ndarray:
    """Value of OCP FP4 E2M1 codes (4-bit, given as integers 0..15), float64.

    1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; no infinities or
    NaN.  Exponent field 0 is subnormal: (m/2) * 2^0; otherwise
    (1 + m/2) * 2^(e-1).  Magnitudes: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    """
    c = np.asarray(nibbles).astype(np.int64) & 15
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m / 2.0, (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0))
    return np.where(c >> 3, -mag, mag)


def e8m0_value(codes: np.ndarray) -> np.ndarray:
    """Value of OCP E8M0 scale codes: 2^(c - 127), float64; 255 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c.astype(np.float64) - 127.0))


MX_BLOCK = 32


def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 matrix [rows, K] in float64 from packed E2M1 codes and E8M0 scales.

    packed [rows, K/2] uint8 holds element 2j in the low nibble of byte j and
    element 2j+1 in the high nibble; scales [rows, K/32] uint8 holds one
    E8M0 scale per block of 32 consecutive elements of a row (along K).
    value[r, k] = e8m0(scales[r, k // 32]) * e2m1(element k of row r).
    """
    p = np.asarray(packed, dtype=np.uint8)
    rows, half = p.shape
    nib = np.empty((rows, 2 * half), dtype=np.int64)
    nib[:, 0::2] = p & 15
    nib[:, 1::2] = p >> 4
    sc = np.repeat(e8m0_value(scales), MX_BLOCK, axis=1)
    assert sc.shape == nib.shape, (sc.shape, nib.shape)
    return sc * fp4_e2m1_value(nib)


E4M3_MAX = 448.0


def quant_e4m3(v: np.ndarray, scale) -> np.ndarray:
    """E4M3 codes of v / scale: static per-tensor activation quantisation.

    The decision is taken in float32: v is rounded to float32, divided by the
    float32 scale (one correctly rounded float32 division), clamped to
    [-448, 448] (saturating: an overflow becomes the largest finite code) and
    rounded to the nearest E4M3 value, ties to the even mantissa.  The E4M3
    grid has spacing 2^(e-3) in the binade [2^e, 2^(e+1)) for e >= -6 and
    spacing 2^-9 below 2^-6 (subnormals).  A value that rounds to zero keeps
    its sign (0x80 for negative).  NaN inputs are not handled.
    """
    q = (np.asarray(v, dtype=np.float32) / np.float32(scale)).astype(np.float64)
    neg = np.signbit(q)
    a = np.minimum(np.abs(q), E4M3_MAX)
    # exponent of the binade of a (a = f * 2^ex with f in [0.5, 1))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, -6)     # binade [2^e, 2^(e+1)), subnormals at -6
    step = np.exp2((e - 3).astype(np.float64))      # grid spacing (2^-9 for subnormals)
    r = np.rint(a / step) * step                    # exact: step is a power of two
    # encode r
    _, ex_r = np.frexp(np.where(r > 0, r, 1.0))
    er = ex_r.astype(np.int64) - 1
    normal = r >= 2.0 ** -6
    field = np.where(normal, er + 7, 0)
    man = np.where(normal, np.rint((r / np.exp2(er.astype(np.float64)) - 1.0) * 8.0),
                   np.rint(r / 2.0 ** -9)).astype(np.int64)
    code = np.where(r == 0, 0, (field << 3) | man)
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def quant_dequant_e4m3(v: np.ndarray, scale) -> np.ndarray:
    """scale * value(quant_e4m3(v, scale)) in float64."""
    return dequant_fp8(quant_e4m3(v, scale), scale)


E4M3_EMAX = 8          # exponent of the largest E4M3 binade (448 = 1.75 * 2^8)


def quant_mxfp8(v: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Dynamic MXFP8 (E4M3) quantisation of rows v [..., K] (K % 32 == 0).

    OCP microscaling conversion, per block of 32 consecutive values of a row:
    the shared exponent is floor(log2(max |v|)) - 8 (8: the largest E4M3
    exponent), floored at -127 (and -127 for an all-zero block); the block's
    scale is that power of two (E8M0 code = exponent + 127) and each element
    is quant_e4m3(v, scale): v / scale (exact: a power of two), clamped to
    +-448 (so magnitudes in (448, 512) * scale saturate) and rounded to the
    nearest E4M3 value, ties to even.  v is rounded to float32 first (the
    decision is taken in float32).  Returns (codes [..., K] uint8, scale
    codes [..., K/32] uint8).
    """
    v32 = np.asarray(v, dtype=np.float32)
    shp = v32.shape
    blk = v32.reshape(shp[:-1] + (shp[-1] // MX_BLOCK, MX_BLOCK)).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))         # amax = f 2^ex, f in [0.5, 1)
    shared = np.where(amax > 0, np.maximum(ex.astype(np.int64) - 1 - E4M3_EMAX, -127), -127)
    scale = np.exp2(shared.astype(np.float64))
    codes = quant_e4m3(blk / scale[..., None], 1.0)           # exact division
    return codes.reshape(shp), (shared + 127).astype(np.uint8)


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """e8m0(scale of the block) * E4M3 value, float64 (blocks of 32 along the last axis)."""
    return np.repeat(e8m0_value(scales), MX_BLOCK, axis=-1) * fp8_e4m3_value(codes)


def quant_dequant_mxfp8(v: np.ndarray) -> np.ndarray:
    return dequant_mxfp8(*quant_mxfp8(v))


def round_bf16(v: np.ndarray) -> np.ndarray:
    """v rounded to float32 and then to bfloat16 (8 significant bits, round
    to nearest even), as float64."""
    v64 = np.asarray(v, dtype=np.float32).astype(np.float64)
    m, e = np.frexp(v64)                                    # v = m 2^e, |m| in [0.5, 1)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


# --------------------------------------------------------------------------
# Experts
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z)."""
    return np.asarray(z, dtype=np.float64) * sigmoid(z)


def expert_h(a: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
             a2: Optional[float] = None, amx: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """The SwiGLU activation of one expert on rows ``a`` [n, H].

    Returns (h, h_in): h = silu(a W_gate^T) * (a W_up^T) in float64, and
    h_in, what the down projection reads.  Without activation quantisation
    h_in is h.  With ``a2`` (static FP8 activations, W8A8) h, as the layer's
    bfloat16 activation tensor (``round_bf16``), is quantised to E4M3 with
    the static scale a2 and dequantised (``quant_dequant_e4m3``), as an FP8
    Linear quantises its input.  With ``amx`` (dynamic MXFP8 activations,
    W4A8) the same bfloat16 h is quantised per block of 32 along I instead
    (``quant_dequant_mxfp8``).
    """
    a = np.asarray(a, dtype=np.float64)
    g = a @ np.asarray(w_gate, dtype=np.float64).T
    u = a @ np.asarray(w_up, dtype=np.float64).T
    h = silu(g) * u
    h_in = h
    if a2 is not None:
        h_in = quant_dequant_e4m3(round_bf16(h), a2)
    if amx:
        h_in = quant_dequant_mxfp8(round_bf16(h))
    return h, h_in


def swiglu_expert(a: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                  w_down: np.ndarray, a2: Optional[float] = None,
                  amx: bool = False) -> np.ndarray:
    """One SwiGLU expert on rows ``a`` [n, H]:  down( silu(a W_gate^T) * (a W_up^T) ).

    Weights are in nn.Linear layout [out, in]: gate/up [I, H], down [H, I]
    (HunyuanImage 3.0 MoE reading, stacked gate/up and down weights).  The
    down projection reads ``expert_h``'s h_in (quantised with ``a2`` or
    ``amx``, see there).
    """
    _, h_in = expert_h(a, w_gate, w_up, a2, amx)
    return h_in @ np.asarray(w_down, dtype=np.float64).T


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
# The shared expert's activation format when it is the routed experts' one.
AS_ROUTED = "as_routed"


def _branch_inputs(x: np.ndarray, E: int, a8, amx: bool, shared_a8, shared_amx):
    """Expert inputs and h formats of the two branches of the layer.

    Returns ((x_r, a2_r, amx_r), (x_s, a2_s, amx_s)): the routed experts'
    input rows, their static h scales (a2_r[e], None without static FP8
    activations) and MXFP8 flag, then the same for the shared expert.  A
    branch quantises x once with its own activation format: static FP8 with
    the layer's scale a1 (``quant_dequant_e4m3``), or dynamic MXFP8 per 32
    along H (``quant_dequant_mxfp8``).  The shared expert takes the routed
    formats unless ``shared_a8`` / ``shared_amx`` say otherwise (the CANN
    deployment article, section 8.2, runs the routed experts at W4A8 and the
    shared expert at W8A8); its static h scale is a2[E].
    """
    if isinstance(shared_a8, str):
        shared_a8 = a8
    if isinstance(shared_amx, str):
        shared_amx = amx

    def quant_x(f8, mx):
        v = x
        if f8 is not None:
            v = quant_dequant_e4m3(v, f8[0])
        if mx:
            v = quant_dequant_mxfp8(v)
        return v

    x_r = quant_x(a8, amx)
    a2_r = [None] * E if a8 is None else [float(a8[1][e]) for e in range(E)]
    same = (shared_a8 is a8) and (bool(shared_amx) == bool(amx))
    x_s = x_r if same else quant_x(shared_a8, shared_amx)
    a2_s = None if shared_a8 is None else float(shared_a8[1][E])
    return (x_r, a2_r, bool(amx)), (x_s, a2_s, bool(shared_amx))


def forward_given_route(x: np.ndarray, idx: np.ndarray, weight: np.ndarray,
                        experts: ExpertFn, E: int,
                        shared: Optional[Sequence[np.ndarray]] = None,
                        a8: Optional[Tuple[float, Sequence[float]]] = None,
                        amx: bool = False, shared_a8=AS_ROUTED,
                        shared_amx=AS_ROUTED) -> np.ndarray:
    """Routed experts + shared expert for a given route (the eager path).

    Follows the eager path of the HunyuanImage 3.0 MoE reading: every token
    row is repeated K times so that copy j of token t pairs with expert
    idx[t, j]; for each expert, the copies routed to it are selected by a mask
    and run through that expert; the outputs are written back in copy order,
    viewed as [T, K, H], multiplied by the routing weights and summed over K.
    The shared expert (a parallel branch every token passes through) is
    computed first and added, as that reading's "Shared MLP" section states.

    ``experts(e)`` returns (gate, up, down) of routed expert e in float64;
    experts no copy is routed to are never requested.

    ``a8 = (a1, a2)`` selects static FP8 activations (W8A8): the expert input
    x is quantised once with the layer's scale a1 (``quant_dequant_e4m3``)
    and every expert's h with its own scale a2[e] (a2[E] for the shared
    expert).  ``amx`` selects dynamic MXFP8 activations (W4A8): x and every
    expert's h are quantised per block of 32 along the reduction axis
    (``quant_dequant_mxfp8``).  The router is not affected: it reads the
    unquantised x.  ``shared_a8`` / ``shared_amx`` give the shared expert
    formats of its own (``_branch_inputs``).
    """
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx)
    weight = np.asarray(weight, dtype=np.float64)
    T, H = x.shape
    K = idx.shape[1] if idx.ndim == 2 else 0
    (x_r, a2_r, amx_r), (x_s, a2_s, amx_s) = _branch_inputs(x, E, a8, amx, shared_a8,
                                                             shared_amx)
    out_shared = np.zeros((T, H))
    if shared is not None:
        out_shared = swiglu_expert(x_s, *shared, a2=a2_s, amx=amx_s)
    if T == 0 or K == 0:
        return out_shared
    flat_idx = idx.reshape(-1)
    x_rep = np.repeat(x_r, K, axis=0)               # [T*K, H], copy j of token t at t*K+j
    expert_out = np.zeros_like(x_rep)
    for e in range(E):
        mask = flat_idx == e
        if not mask.any():
            continue
        wg, wu, wd = experts(e)
        expert_out[mask] = swiglu_expert(x_rep[mask], wg, wu, wd, a2=a2_r[e], amx=amx_r)
    routed = (expert_out.reshape(T, K, H) * weight[:, :, None]).sum(axis=1)
    return out_shared + routed


def forward_by_expert(x: np.ndarray, idx: np.ndarray, weight: np.ndarray,
                      experts: ExpertFn, E: int,
                      shared: Optional[Sequence[np.ndarray]] = None,
                      a8: Optional[Tuple[float, Sequence[float]]] = None,
                      amx: bool = False, h_hook=None, shared_a8=AS_ROUTED,
                      shared_amx=AS_ROUTED) -> np.ndarray:
    """The same sum as ``forward_given_route``, gathered expert by expert.

    out[t] = shared(x_t) + sum_e sum_{j: idx[t, j] = e} weight[t, j] f_e(x_t).
    Each routed expert is requested once, evaluated on the tokens routed to
    it and its weighted rows added into the output, so no [T*K, H] copy of x
    is built and only one expert's weights need to be held at a time: the
    form used to check layers with tens of thousands of tokens.  Only the
    order of the float64 additions differs from the eager path.

    ``h_hook(e, tok, a, w_gate, w_up, h, h_in) -> h_in`` (optional, e = E
    for the shared expert, tok its tokens in ascending order, a their input
    rows) sees each expert's activation before the down projection and
    returns what the down projection reads: the tests use it where a
    quantised activation code has two valid answers (a value within
    rounding of a decision boundary), to continue with the one the GPU took
    after checking it, as they do with the picks of near-tie tokens.
    """
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx)
    weight = np.asarray(weight, dtype=np.float64)
    T, H = x.shape
    (x_r, a2_r, amx_r), (x_s, a2_s, amx_s) = _branch_inputs(x, E, a8, amx, shared_a8,
                                                             shared_amx)

    def expert_out(e, tok, wg, wu, wd):
        a, a2, mx = (x_s[tok], a2_s, amx_s) if e == E else (x_r[tok], a2_r[e], amx_r)
        h, h_in = expert_h(a, wg, wu, a2=a2, amx=mx)
        if h_hook is not None:
            h_in = h_hook(e, tok, a, wg, wu, h, h_in)
        return h_in @ np.asarray(wd, dtype=np.float64).T

    out = np.zeros((T, H))
    if shared is not None:
        out += expert_out(E, np.arange(T), *shared)
    if T == 0 or idx.size == 0:
        return out
    for e in np.unique(idx):
        tok, slot = np.nonzero(idx == e)
        y = expert_out(int(e), tok, *experts(int(e)))
        np.add.at(out, tok, weight[tok, slot][:, None] * y)
    return out


def forward(x, w_router, experts: ExpertFn, E: int, K: int,
            shared: Optional[Sequence[np.ndarray]] = None,
            mode: int = ROUTE_SIGMOID_BIAS, bias=None, scale: float = 2.826,
            renorm_eps: float = 1e-8) -> Tuple[np.ndarray, Route]:
    """The full MoE FFN layer: gate, then routed + shared experts."""
    r = route(x, w_router, K, mode, bias, scale, renorm_eps)
    return forward_given_route(x, r.idx, r.weight, experts, E, shared), r


def dense_masked(x, idx, weight, experts: ExpertFn, E: int,
                 shared: Optional[Sequence[np.ndarray]] = None,
                 a8: Optional[Tuple[float, Sequence[float]]] = None,
                 amx: bool = False, shared_a8=AS_ROUTED,
                 shared_amx=AS_ROUTED) -> np.ndarray:
    """Brute force: evaluate every expert on every token and mask.

    out[t] = shared(x_t) + sum_e M[t, e] * f_e(x_t), where M is zero except
    M[t, idx[t, j]] = weight[t, j].  Used on tiny inputs only, as a check of
    the sparse dispatch above (activation formats as there).
    """
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    M = np.zeros((T, E))
    idx = np.asarray(idx)
    for t in range(T):
        for j in range(idx.shape[1]):
            M[t, idx[t, j]] += weight[t, j]
    (x_r, a2_r, amx_r), (x_s, a2_s, amx_s) = _branch_inputs(x, E, a8, amx, shared_a8,
                                                             shared_amx)
    out = (np.zeros((T, H)) if shared is None
           else swiglu_expert(x_s, *shared, a2=a2_s, amx=amx_s))
    for e in range(E):
        out = out + M[:, e:e + 1] * swiglu_expert(x_r, *experts(e), a2=a2_r[e], amx=amx_r)
    return out


def layer_flops(T: int, H: int, E: int, K: int, I: int, I_shared: int) -> dict:
    """Algorithmic FLOP counts of the layer (real rows only, no padding)."""
    routed = 6.0 * H * I * T * K
    shared = 6.0 * H * I_shared * T
    router = 2.0 * T * H * E
    return {"routed": routed, "shared": shared, "router": router,
            "experts": routed + shared, "total": routed + shared + router}
