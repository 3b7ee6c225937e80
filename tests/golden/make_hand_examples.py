"""Writes the hand-derived fixtures of this folder from their closed forms.

Every expected value below is the arithmetic of the derivation written next to
it (logarithms of small integers as scores, so softmax weights are integer
ratios). Nothing here imports the oracle or the HIP path. Run from the repo
root: ``python tests/golden/make_hand_examples.py``.
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ln2, ln3, ln4 = math.log(2), math.log(3), math.log(4)
ZD = math.sqrt(3) + math.sqrt(2) + 2          # drift normaliser of pooled query 0 (x e^-M)

hand = {
    "citation": [
        "VASC summary (paperlayer.ai 2610.01013v1), section 3: retained attention weights are "
        "renormalised after connections are dropped",
        "ReSS (thelatestinai.com 2609.35593), Table S5 SpargeAttn row: selection on pooled "
        "query/key inner products",
        "ReSS abstract and Fig. 3(a)-(b): per-block contribution to what attention writes into "
        "the residual stream",
    ],
    "layout": {"batch": 1, "heads": 1, "head_dim": 2, "frames": 1, "frame_len": 4,
               "frame_valid": 3, "block": 2, "scale": 1.0},
    "q": [[1, 0], [0, 1], [1, 1], [0, 0]],
    "k": [[0, ln3], [ln2, 0], [ln4, 0], [0, 0]],
    "v": [[1, 0], [0, 1], [1, 1], [0, 0]],
    "derivation": [
        "token 3 is padding (frame_valid = 3); blocks are {0,1} and {2,3}",
        "query 0 = (1,0): scores 0, ln2, ln4 -> weights 1:2:4 over 7 -> o = (5/7, 6/7), lse = ln 7",
        "query 1 = (0,1): scores ln3, 0, 0 -> weights 3:1:1 over 5 -> o = (4/5, 2/5), lse = ln 5",
        "query 2 = (1,1): scores ln3, ln2, ln4 -> weights 3:2:4 over 9 -> o = (7/9, 2/3), lse = ln 9",
        "keep block 0 only: weights 1:2 -> (1/3, 2/3), lse ln3; 3:1 -> (3/4, 1/4), lse ln4; "
        "3:2 -> (3/5, 2/5), lse ln5",
        "keep block 1 only: one key (token 2) -> o = v2 = (1,1); lse = its score: ln4, 0, ln4",
        "pooled q: block 0 mean(q0,q1) = (1/2,1/2); block 1 mean over real tokens only = q2 = (1,1)",
        "pooled k: block 0 mean(k0,k1) = (ln2/2, ln3/2); block 1 = k2 = (ln4, 0)",
        "S[i][j] = <qbar_i, kbar_j>: S00 = ln6/4, S01 = ln2, S10 = ln6/2, S11 = ln4; "
        "top-1 keeps block 1 in both rows",
        "drift of pooled query 0: logits ln3/2, ln2/2, ln2 -> e^(l - max) = (sqrt3, sqrt2, 2)/2; "
        "Z e^max = sqrt3 + sqrt2 + 2",
        "c0/Z = (sqrt3*v0 + sqrt2*v1)/(sqrt3+sqrt2+2); c1/Z = 2*v2/(sqrt3+sqrt2+2)",
    ],
    "dense_o": [[5 / 7, 6 / 7], [4 / 5, 2 / 5], [7 / 9, 2 / 3], [0, 0]],
    "dense_lse": [math.log(7), math.log(5), math.log(9), None],
    "keep0_o": [[1 / 3, 2 / 3], [3 / 4, 1 / 4], [3 / 5, 2 / 5], [0, 0]],
    "keep0_lse": [math.log(3), math.log(4), math.log(5), None],
    "keep1_o": [[1, 1], [1, 1], [1, 1], [0, 0]],
    "keep1_lse": [ln4, 0.0, ln4, None],
    "qbar": [[0.5, 0.5], [1, 1]],
    "kbar": [[ln2 / 2, ln3 / 2], [ln4, 0]],
    "scores": [[math.log(6) / 4, ln2], [math.log(6) / 2, ln4]],
    "top1": [[1], [1]],
    "drift_q0_chat": [[math.sqrt(3) / ZD, math.sqrt(2) / ZD], [2 / ZD, 2 / ZD]],
    "drift_q0_z_over_Z": [(math.sqrt(3) + math.sqrt(2)) / ZD, 2 / ZD],
}

restoration = {
    "citation": [
        "ReSS (thelatestinai.com 2609.35593) abstract and Fig. 3(b)-(c): initial set by drift "
        "score, then swaps at a fixed budget that reduce the drop set's drift, which depends on "
        "the directions of the contribution vectors, not on their magnitudes alone",
    ],
    "chat": [[3, 0], [-2.5, 0], [2, 0], [0, 1]],
    "keep": 2,
    "derivation": [
        "norms 3, 2.5, 2, 1 -> initial kept {0,1}, drop {2,3}, r = (2,1), J^2 = 5",
        "round 1 (restore a, drop b): (2,0): (3,1) -> 10; (2,1): (-2.5,1) -> 7.25; "
        "(3,0): (5,0) -> 25; (3,1): (-0.5,0) -> 0.25",
        "best (3,1) < 5: kept {0,3}, drop {1,2}, r = (-0.5,0), J = 0.5",
        "round 2: (1,0): (5,0) -> 25; (1,3): (2,1) -> 5; (2,0): (0.5,0) -> 0.25; "
        "(2,3): (-2.5,1) -> 7.25; min 0.25 is not < 0.25 -> stop",
        "exhaustive over the six kept pairs: J = sqrt5, sqrt7.25, 5, sqrt10, 0.5 ({0,3}), "
        "0.5 ({2,3}); optimum 0.5",
    ],
    "initial_kept": [0, 1],
    "initial_J": math.sqrt(5),
    "swaps": [[3, 1]],
    "final_kept_3_rounds": [0, 3],
    "final_J": 0.5,
    "exhaustive_best_J": 0.5,
}

if __name__ == "__main__":
    for name, obj in (("hand_example.json", hand), ("restoration_example.json", restoration)):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(obj, f, indent=1)
            f.write("\n")
