"""Writes the hand-worked fixtures in this folder.

The pages print no numeric worked example of the MoE layer, so these cases are
worked by hand from closed forms: sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4,
sigmoid(ln 9) = 9/10, softmax of logs is the normalised arguments, and
silu(ln 3) = (3/4) ln 3.  Each expected value is written as that closed form,
evaluated with Python float arithmetic.  This script calls neither the oracle
nor the HIP library.  Run:  python tests/golden/make_hand_fixtures.py
"""
import json
import math
import os

ln3 = math.log(3.0)
HERE = os.path.dirname(os.path.abspath(__file__))

CASES = {
    "route_sigmoid_bias_hand.json": {
        "cite": "hy3 README, 'Model facts' table, MoE routing row: top-8 chosen on "
                "sigmoid + expert_bias, combined with the unbiased sigmoid weights "
                "renormalised to sum 1 and scaled by 2.826",
        "derivation": "Identity router weight (H=E), so logits = x. Token 0: logits "
                      "[0, ln3, -ln3, ln9] give s = [1/2, 3/4, 1/4, 9/10]; with bias "
                      "[0.5, 0, 0.6, -0.5], s+b = [1.0, 0.75, 0.85, 0.4]; top-2 = [0, 2] "
                      "(the unbiased top-2 would be [3, 1]); margin 0.85-0.75; weights "
                      "2.826*[1/2, 1/4]/(3/4). Token 1: logits [0, 0, ln3, ln3] give "
                      "s = [1/2, 1/2, 3/4, 3/4]; s+b = [1.0, 0.5, 1.35, 0.25]; top-2 = "
                      "[2, 0]; margin 1.0-0.5; weights 2.826*[3/4, 1/2]/(5/4).",
        "K": 2, "scale": 2.826,
        "logits": [[0.0, ln3, -ln3, math.log(9.0)], [0.0, 0.0, ln3, ln3]],
        "bias": [0.5, 0.0, 0.6, -0.5],
        "idx": [[0, 2], [2, 0]],
        "weight": [[2.826 * 0.5 / 0.75, 2.826 * 0.25 / 0.75],
                   [2.826 * 0.75 / 1.25, 2.826 * 0.5 / 1.25]],
        "margin": [0.85 - 0.75, 1.0 - 0.5],
    },
    "route_sigmoid_ties_hand.json": {
        "cite": "hy3 README, 'Model facts' table, MoE routing row. The tie order "
                "(lower expert index first) is a reading: the pages do not fix it",
        "derivation": "logits [0, 0, ln3, ln3, -ln3], zero bias: s = [1/2, 1/2, 3/4, "
                      "3/4, 1/4]. K=2: picks [2, 3] (tie at 3/4, lower index first), "
                      "margin 3/4-1/2, weights 2.826*[1/2, 1/2]. K=3: picks [2, 3, 0] "
                      "(tie 0/1 at 1/2, lower index wins), margin 0, weights "
                      "2.826*[3/8, 3/8, 1/4].",
        "logits": [[0.0, 0.0, ln3, ln3, -ln3]],
        "bias": [0.0, 0.0, 0.0, 0.0, 0.0],
        "scale": 2.826,
        "by_K": {
            "2": {"idx": [[2, 3]], "weight": [[2.826 / 2, 2.826 / 2]], "margin": [0.25]},
            "3": {"idx": [[2, 3, 0]], "weight": [[2.826 * 3 / 8, 2.826 * 3 / 8, 2.826 / 4]],
                  "margin": [0.0]},
        },
    },
    "route_softmax_hand.json": {
        "cite": "HunyuanImage 3.0 MoE reading, HunyuanTopKGate easy_topk path: softmax "
                "over experts, top-K, sum clamped at 1e-8, divide",
        "derivation": "logits [ln4, ln2, 0, 0]: softmax = [4, 2, 1, 1]/8. K=2: picks "
                      "[0, 1], weights [1/2, 1/4]/(3/4) = [2/3, 1/3], margin 1/4-1/8. "
                      "K=3: picks [0, 1, 2] (tie between 2 and 3 goes to the lower "
                      "index), weights [4, 2, 1]/7, margin 0.",
        "logits": [[math.log(4.0), math.log(2.0), 0.0, 0.0]],
        "by_K": {
            "2": {"idx": [[0, 1]], "weight": [[2 / 3, 1 / 3]], "margin": [0.125]},
            "3": {"idx": [[0, 1, 2]], "weight": [[4 / 7, 2 / 7, 1 / 7]], "margin": [0.0]},
        },
    },
    "swiglu_hand.json": {
        "cite": "HunyuanImage 3.0 MoE reading: experts use SiLU/SwiGLU, gate/up weights "
                "[I, H] and down [H, I] in Linear [out, in] layout",
        "derivation": "a = [1, 0]; W_gate = [[ln3, 5], [0, 7]] -> g = [ln3, 0]; W_up = "
                      "[[2, 11], [3, 13]] -> u = [2, 3]; silu(g) = [(3/4) ln3, 0]; h = "
                      "[(3/2) ln3, 0]; W_down = [[1, 17], [4, 19]] -> out = [(3/2) ln3, "
                      "6 ln3]. A transposed gate would give g = [ln3, 5], a transposed "
                      "down [(3/2) ln3, (51/2) ln3], swapped gate/up h = [silu(2) ln3, 0].",
        "a": [[1.0, 0.0]],
        "w_gate": [[ln3, 5.0], [0.0, 7.0]],
        "w_up": [[2.0, 11.0], [3.0, 13.0]],
        "w_down": [[1.0, 17.0], [4.0, 19.0]],
        "out": [[1.5 * ln3, 6.0 * ln3]],
    },
    "layer_hand.json": {
        "cite": "hy3 README 'Model facts' (routing rule; one shared expert, always "
                "active); HunyuanImage 3.0 MoE reading 'Shared MLP' (shared branch "
                "added to the routed output)",
        "derivation": "T=1, H=I=I_shared=1, E=3, K=2. x=1, router weight [0, ln3, -ln3] "
                      "-> s = [1/2, 3/4, 1/4]; bias [0, 0, 0.6] -> s+b = [1/2, 3/4, 0.85]; "
                      "picks [2, 1]; weights 2.826*[1/4, 3/4]/1. Every expert has gate "
                      "ln3, so silu = (3/4) ln3; (up, down) = e0 (8, 1), e1 (2, 1), "
                      "e2 (4, -1): f1 = (3/2) ln3, f2 = -3 ln3; shared (gate ln3, up 1, "
                      "down 2) = (3/2) ln3. out = ln3*(3/2 + 0.7065*(-3) + 2.1195*(3/2)).",
        "x": [[1.0]],
        "w_router": [[0.0], [ln3], [-ln3]],
        "bias": [0.0, 0.0, 0.6],
        "K": 2, "scale": 2.826,
        "experts": [{"gate": [[ln3]], "up": [[8.0]], "down": [[1.0]]},
                    {"gate": [[ln3]], "up": [[2.0]], "down": [[1.0]]},
                    {"gate": [[ln3]], "up": [[4.0]], "down": [[-1.0]]}],
        "shared": {"gate": [[ln3]], "up": [[1.0]], "down": [[2.0]]},
        "idx": [[2, 1]],
        "weight": [[2.826 * 0.25, 2.826 * 0.75]],
        "out": [[ln3 * (1.5 + 2.826 * 0.25 * (-3.0) + 2.826 * 0.75 * 1.5)]],
    },
}

if __name__ == "__main__":
    for name, case in CASES.items():
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(case, f, indent=1)
            f.write("\n")
    print("wrote", len(CASES), "fixtures")
