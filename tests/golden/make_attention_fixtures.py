"""Writes the hand-worked attention fixtures in this folder.

The expected outputs are closed forms of scaled dot-product attention
evaluated with ``math`` (no oracle, no GPU): the inputs are chosen so that
the scores ``scale * (q . k)`` are small exact numbers and the softmax
weights have a known expression.  Run from the repository root:
``python tests/golden/make_attention_fixtures.py``.
"""

import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def two_tokens():
    e = math.e
    v0 = [1.0, -2.0, 0.5, 4.0]
    v1 = [3.0, 0.25, -1.0, 2.0]
    return {
        "derivation": "q=[2,0,0,0], k0=[0,5,0,0], k1=[0.5,0,0,0], scale=1 -> z=[0,1]; "
                      "weights 1/(1+e), e/(1+e); out=(v0+e*v1)/(1+e)",
        "section": "closed form of scaled dot-product attention (the pages give no formula)",
        "dtype": "fp32", "block_size": 2, "scale": 1.0,
        "q": [2.0, 0.0, 0.0, 0.0],
        "k": [[0.0, 5.0, 0.0, 0.0], [0.5, 0.0, 0.0, 0.0]],
        "v": [v0, v1],
        "physical_blocks": [1], "num_blocks": 3,
        "expected": [(a + e * b) / (1 + e) for a, b in zip(v0, v1)],
    }


def three_tokens():
    t = math.exp(-31.0)
    return {
        "derivation": "q=[1,1], keys [1,1],[2,0],[-30,-30], scale=0.5 -> z=[1,1,-30]; "
                      "weights [1,1,e^-31]/(2+e^-31)",
        "section": "closed form of scaled dot-product attention (the pages give no formula)",
        "dtype": "fp32", "block_size": 2, "scale": 0.5,
        "q": [1.0, 1.0],
        "k": [[1.0, 1.0], [2.0, 0.0], [-30.0, -30.0]],
        "v": [[4.0, 0.0], [0.0, 8.0], [100.0, 100.0]],
        "physical_blocks": [2, 0], "num_blocks": 3,
        "expected": [(4.0 + 100.0 * t) / (2 + t), (8.0 + 100.0 * t) / (2 + t)],
    }


if __name__ == "__main__":
    for name, fix in (("attention_two_tokens.json", two_tokens()),
                      ("attention_three_tokens.json", three_tokens())):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(fix, f, indent=1)
            f.write("\n")
