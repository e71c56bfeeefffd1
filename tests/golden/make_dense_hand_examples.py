"""Writes dense_hand_examples.json: tiny attention cases whose results are derived by hand.

The values come from the definition O = softmax(Q K^T * scale) V (page "SparseFlashMla",
Description: formula), the bottom-right causal mask ("RightDownCausal", same page, Parameters
table) and the sink read as an extra logit with a zero value vector. Each case states its
derivation; nothing here calls the oracle or the HIP path.
"""
import json
import math
import os

E05, E1 = math.exp(0.5), math.exp(1.0)
CASES = [
    {"name": "two_keys_weights_1_to_3",
     "derivation": "scale=1, q=[1,0]; k0=[0,0] gives logit 0, k1=[ln 3, 0] gives logit ln 3, so the "
                   "softmax weights are 1/4 and 3/4. v0=[1,-2], v1=[5,2]: O = [1/4+15/4, -2/4+6/4] = [4, 1]; "
                   "LSE = ln(1+3) = ln 4.",
     "scale": 1.0, "causal": False, "q": [[1.0, 0.0]], "k": [[0.0, 0.0], [math.log(3.0), 0.0]],
     "v": [[1.0, -2.0], [5.0, 2.0]], "sink": None, "O": [[4.0, 1.0]], "LSE": [math.log(4.0)]},
    {"name": "causal_first_row_sees_one_key",
     "derivation": "Sq=Sk=2, causal: row 0 sees only k0, so O_0 = v0 and LSE_0 = scale*q0.k0 = 0.5*2 = 1. "
                   "Row 1 sees both keys with logits 0.5*(1*1)=0.5 and 0.5*(1*1+1*1)=1.0, weights "
                   "e^0.5/(e^0.5+e^1) and e^1/(e^0.5+e^1).",
     "scale": 0.5, "causal": True, "q": [[2.0, 0.0], [1.0, 1.0]], "k": [[1.0, 0.0], [1.0, 1.0]],
     "v": [[3.0, 0.0], [0.0, 3.0]], "sink": None,
     "O": [[3.0, 0.0], [3 * E05 / (E05 + E1), 3 * E1 / (E05 + E1)]],
     "LSE": [1.0, math.log(E05 + E1)]},
    {"name": "sink_takes_half_the_mass",
     "derivation": "One key with logit 0 (q.k=0) and a sink logit 0: the sink is an extra logit with a zero "
                   "value vector, so the key weight is 1/2. O = v/2 = [1, -1]; LSE = ln(e^0 + e^0) = ln 2.",
     "scale": 1.0, "causal": False, "q": [[1.0, 0.0]], "k": [[0.0, 1.0]], "v": [[2.0, -2.0]],
     "sink": [0.0], "O": [[1.0, -1.0]], "LSE": [math.log(2.0)]},
    {"name": "bottom_right_causal_sq1_sk3",
     "derivation": "One query against three keys with the bottom-right causal mask: j <= i + Sk - Sq = 0 + 2, "
                   "so all three keys are visible. All logits are 0, so O is the mean of v = [2, 4, 6] -> 4, "
                   "LSE = ln 3.",
     "scale": 1.0, "causal": True, "q": [[0.0]], "k": [[1.0], [2.0], [3.0]], "v": [[2.0], [4.0], [6.0]],
     "sink": None, "O": [[4.0]], "LSE": [math.log(3.0)]},
    {"name": "bottom_right_causal_sq3_sk1_empty_rows",
     "derivation": "Three queries against one key, bottom-right causal: j <= i + 1 - 3 = i - 2. Rows 0 and 1 "
                   "see no key: O = 0, LSE = -inf. Row 2 sees k0 only: O = v0 = [7], LSE = q2.k0 = 1*2 = 2.",
     "scale": 1.0, "causal": True, "q": [[5.0], [5.0], [1.0]], "k": [[2.0]], "v": [[7.0]],
     "sink": None, "O": [[0.0], [0.0], [7.0]], "LSE": ["-inf", "-inf", 2.0]},
]

if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dense_hand_examples.json")
    with open(path, "w") as f:
        json.dump({"source": "Hand-derived from the attention definition (page 'SparseFlashMla', "
                             "Description: formula) with the masking and sink readings stated per case. "
                             "The pages print no worked numeric example.",
                   "cases": CASES}, f, indent=1)
