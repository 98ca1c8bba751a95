"""Writes the closed-form fixtures in this folder. It evaluates hand-derived
closed forms with Python's math module only: it calls neither the oracle nor the
GPU library. Run: python tests/golden/derive_closed_forms.py
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ln2 = math.log(2.0)


def hand_two_tokens():
    # The recurrence: state and output equations of the aidatadrop page ("State-Space
    # Models (SSMs): A Resurgent Paradigm for Sequence Modeling"), discretized with
    # exp(Delta*A) and Delta*B*x; per-token B, C, Delta from the promptingindex page
    # ("The selective mechanism: input-dependent SSM parameters"); gating by
    # SiLU of the second branch from the sivaro page ("The Architecture in Practice").
    inputs = {
        "A": [-1.0, -2.0], "D": 0.5, "delta_bias": -0.75, "h0": [1.0, -1.0],
        "x": [2.0, 0.0], "delta_raw": [0.75, 0.75], "z": [1.0, 2.0],
        "B": [[1.0, 2.0], [5.0, 7.0]], "C": [[3.0, -1.0], [-1.0, 2.0]],
    }
    h1 = [0.5 + 2 * ln2, -0.25 + 4 * ln2]
    y1_pre = 2.75 + 2 * ln2
    y1 = y1_pre / (1 + math.exp(-1.0))
    h2 = [h1[0] / 2, h1[1] / 4]
    y2 = (ln2 - 0.375) * 2.0 / (1 + math.exp(-2.0))
    return {
        "what": "two tokens of one channel, N = 2, worked by hand",
        "derivation": [
            "v = delta_raw + delta_bias = 0.75 - 0.75 = 0 for both tokens, so Delta = softplus(0) = ln 2",
            "exp(Delta*A) = (exp(-ln2), exp(-2 ln2)) = (1/2, 1/4)",
            "token 1: Delta*x = 2 ln2; h1 = (1/2*1 + 2ln2*1, 1/4*(-1) + 2ln2*2) = (0.5 + 2 ln2, -0.25 + 4 ln2)",
            "token 1: C.h1 = 3(0.5 + 2ln2) - (-0.25 + 4ln2) = 1.75 + 2 ln2; + D*x = 1 -> 2.75 + 2 ln2",
            "token 1: y1 = (2.75 + 2 ln2) * silu(1), silu(1) = 1/(1 + e^-1)",
            "token 2: x = 0 so h2 = (h1[0]/2, h1[1]/4) = (0.25 + ln2, -0.0625 + ln2)",
            "token 2: C.h2 = -(0.25 + ln2) + 2(-0.0625 + ln2) = ln2 - 0.375; D*x = 0",
            "token 2: y2 = (ln2 - 0.375) * silu(2), silu(2) = 2/(1 + e^-2)",
        ],
        "inputs": inputs,
        "expected_closed_form": {
            "h1": ["0.5 + 2 ln2", "-0.25 + 4 ln2"], "y1": "(2.75 + 2 ln2)/(1 + e^-1)",
            "h2": ["0.25 + ln2", "-0.0625 + ln2"], "y2": "(ln2 - 0.375) * 2/(1 + e^-2)",
        },
        "expected_decimal": {"h1": h1, "y1_pre_gate": y1_pre, "y1": y1, "h2": h2, "y2": y2},
    }


def lti_step_response():
    # With Delta, B, C fixed the SSM is a convolution with K_k = C Delta B r^k (the
    # S4 view: promptingindex page, "State space models before Mamba: HiPPO and S4";
    # sivaro page, "How State Space Models Work"). N = 1, A = -1, Delta =
    # softplus(0) = ln 2 -> r = 1/2, B = C = 1, D = 0, x_t = 1 (a unit step):
    # y_t = ln2 * sum_{k<=t} 2^-k = 2 ln2 (1 - 2^-(t+1)).
    ys = [2 * ln2 * (1 - 2.0 ** -(t + 1)) for t in range(8)]
    return {
        "what": "unit-step response of a one-state LTI SSM",
        "derivation": "y_t = sum_{k=0..t} C*Delta*B*r^k with r = exp(Delta*A) = 1/2, Delta = ln 2",
        "inputs": {"N": 1, "A": -1.0, "delta_raw": 0.0, "delta_bias": 0.0, "softplus": True,
                   "B": 1.0, "C": 1.0, "D": 0.0, "x": 1.0},
        "y": ys,
    }


if __name__ == "__main__":
    for name, fn in [("hand_two_tokens.json", hand_two_tokens),
                     ("lti_step_response.json", lti_step_response)]:
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(fn(), f, indent=1)
            f.write("\n")
        print("wrote", name)
