"""Writes worked_example_s3_d2.json: a hand-worked instance of attention with
three keys and head dim 2, whose values follow in closed form from the
definition the pages state (scores s_ij = scale * q_i . k_j; under causal
masking keys j <= i only; P = softmax over the kept keys; O = P V;
lse_i = log sum_j exp(s_ij)). The pages print no worked numbers, so the
expected values here are those closed forms, evaluated with Python's math
module; nothing from the oracle or the GPU path goes into them.

    python tests/golden/make_worked_example.py
"""
import json
import math
import os

E = math.e
Q = [[2, 0], [0, 2], [2, 2]]
K = [[1, 0], [0, 1], [1, -1]]
V = [[1, 2], [3, 4], [5, -6]]
SCALE = 0.5


def combo(weights):
    """(sum_j w_j v_j) / (sum_j w_j) for the first len(weights) keys."""
    den = math.fsum(weights)
    return [math.fsum(w * V[j][d] for j, w in enumerate(weights)) / den for d in range(2)]


def build():
    # scores by hand: row 0 = (1, 0, 1), row 1 = (0, 1, -1), row 2 = (1, 1, 0)
    scores = [[1, 0, 1], [0, 1, -1], [1, 1, 0]]
    noncausal = {
        "o_exact": ["(e v0 + v1 + e v2) / (2e + 1)", "(v0 + e v1 + v2 / e) / (1 + e + 1/e)",
                    "(e v0 + e v1 + v2) / (2e + 1)"],
        "lse_exact": ["log(2e + 1)", "log(1 + e + 1/e)", "log(2e + 1)"],
        "o": [combo([E, 1.0, E]), combo([1.0, E, 1 / E]), combo([E, E, 1.0])],
        "lse": [math.log(2 * E + 1), math.log(1 + E + 1 / E), math.log(2 * E + 1)],
    }
    causal = {
        "o_exact": ["v0", "(v0 + e v1) / (1 + e)", "(e v0 + e v1 + v2) / (2e + 1)"],
        "lse_exact": ["1", "log(1 + e)", "log(2e + 1)"],
        "o": [combo([1.0]), combo([1.0, E]), combo([E, E, 1.0])],
        "lse": [1.0, math.log(1 + E), math.log(2 * E + 1)],
    }
    return {
        "note": "Hand-worked attention instance: scores s_ij = scale q_i.k_j, causal keeps j <= i, "
                "P = softmax over kept keys, O = P V, lse_i = log sum_j exp(s_ij) (natural log). "
                "The definition the online-softmax recurrences of the infra.bea.ai FlashAttention V2 "
                "guide (Optimization 2: Delay Rescaling) and the cookbook's Triton kernel end in; "
                "jared-hpc Lecture 6 names lse as the forward pass's second output. Values are the "
                "closed forms in o_exact / lse_exact evaluated in double precision.",
        "scale": SCALE, "q": Q, "k": K, "v": V, "scores": scores,
        "noncausal": noncausal, "causal": causal,
    }


PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_example_s3_d2.json")

if __name__ == "__main__":
    with open(PATH, "w") as f:
        json.dump(build(), f, indent=1)
        f.write("\n")
    print(PATH)
