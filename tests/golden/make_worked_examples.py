"""Writes worked_examples.json: tiny cases whose answers follow by hand from the
definitions (closed forms with exact fractions; no code under test is called).

Definitions used: "Efficient and portable mixture-of-experts communication"
(Perplexity, 2025-04-02) -- Introduction (router distribution, top-K choice,
weighted sum of expert outputs), Dispatch section (expert-contiguous rows plus
source-index records), Combine section (weighted sum into a caller-owned
tensor).  Slot order and tie rule: descending score, equal scores to the lower
expert id; rows ordered by expert then token.
"""
import json
import math
import os

ln = math.log


def cases():
    return {
        "source": "Efficient and portable mixture-of-experts communication (Perplexity, "
                  "2025-04-02): Introduction, Dispatch and Combine sections. Values derived by "
                  "hand from the definitions (exact fractions, written in decimal).",
        "route_cases": [
            {"name": "softmax_renorm", "score": "softmax", "renorm": True, "K": 2,
             "logits": [0.0, ln(2), ln(3), ln(6)],
             "derivation": "exp(logits) = 1,2,3,6; p = 1/12,2/12,3/12,6/12; top-2 = experts 3,2; "
                           "renormalised 6/9, 3/9",
             "ids": [3, 2], "weights": [2 / 3, 1 / 3]},
            {"name": "softmax_plain", "score": "softmax", "renorm": False, "K": 2,
             "logits": [0.0, ln(2), ln(3), ln(6)],
             "derivation": "same probabilities, not renormalised: 6/12, 3/12",
             "ids": [3, 2], "weights": [0.5, 0.25]},
            {"name": "softmax_all_experts", "score": "softmax", "renorm": False, "K": 4,
             "logits": [0.0, ln(2), ln(3), ln(6)],
             "derivation": "K = E: every probability, descending",
             "ids": [3, 2, 1, 0], "weights": [0.5, 0.25, 1 / 6, 1 / 12]},
            {"name": "sigmoid_renorm", "score": "sigmoid", "renorm": True, "K": 2,
             "logits": [0.0, ln(3), -ln(3), ln(7)],
             "derivation": "sigmoid = 1/2, 3/4, 1/4, 7/8; top-2 = experts 3,1; renormalised "
                           "(7/8)/(13/8), (6/8)/(13/8)",
             "ids": [3, 1], "weights": [7 / 13, 6 / 13]},
            {"name": "tie_lower_id_first", "score": "softmax", "renorm": True, "K": 2,
             "logits": [1.0, 2.0, 2.0, 0.0],
             "derivation": "experts 1 and 2 tie; the lower id takes the first slot; equal scores "
                           "renormalise to 1/2 each",
             "ids": [1, 2], "weights": [0.5, 0.5]},
            {"name": "shift_invariance", "score": "softmax", "renorm": False, "K": 1,
             "logits": [1000.0, 1000.0 + ln(3), 1000.0],
             "derivation": "softmax is shift invariant: exp ratios 1,3,1 -> top-1 expert 1 with 3/5",
             "ids": [1], "weights": [0.6]},
        ],
        "dispatch_case": {
            "T": 4, "K": 2, "E": 4, "expert_begin": 1, "expert_end": 3,
            "ids": [[1, 2], [3, 1], [2, 0], [1, 3]],
            "derivation": "counts over all experts: e0 {t2}, e1 {t0,t1,t3}, e2 {t0,t2}, e3 {t1,t3}; "
                          "local experts 1,2 in order, tokens ascending: rows = (t0,k0),(t1,k1),"
                          "(t3,k0) then (t0,k1),(t2,k0)",
            "counts": [1, 3, 2, 2], "offsets": [0, 3, 5],
            "src_index": [0, 3, 6, 1, 4],
            "row_of": [0, 3, -1, 1, 4, -1, 2, -1]},
        "mlp_case": {
            "d": 1, "I": 1, "x": [1.0], "w_gate": [ln(3)], "w_up": [2.0], "w_down": [0.5],
            "derivation": "gate = ln 3, SiLU(ln 3) = ln 3 * sigmoid(ln 3) = (3/4) ln 3; up = 2; "
                          "h = (3/2) ln 3; y = 0.5 h = (3/4) ln 3",
            "y": [0.75 * ln(3)]},
        "combine_case": {
            "T": 2, "K": 2, "d": 2,
            "y_sorted": [[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]],
            "row_of": [2, 0, -1, 1], "weights": [[0.25, 0.75], [0.5, 0.5]],
            "derivation": "token 0: 0.25*row2 + 0.75*row0 = (25.75, 51.5); token 1: slot 0 is "
                          "remote (-1), 0.5*row1 = (5, 10)",
            "out": [[25.75, 51.5], [5.0, 10.0]]},
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_examples.json")
    with open(path, "w") as f:
        json.dump(cases(), f, indent=1)
    print(path)
