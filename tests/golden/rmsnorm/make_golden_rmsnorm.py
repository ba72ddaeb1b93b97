"""Writes the hand-derived fixtures of the gated grouped RMSNorm.

The operator (page "ops-transformer MambaV2 算子套件", section 4.6,
mamba2_rmsnormgated): g = x * SiLU(z), normalised per group of the last
dimension by sqrt(mean(g^2) + eps), times the weight w.  Each expected value
below is worked out by hand (closed forms in sqrt 2 and ln 3, with
sigma(ln 3) = 3/4); nothing here calls the oracle or the HIP library.
"""
import json
import math
import os

r2 = math.sqrt(2.0)
ln3 = math.log(3.0)

CASES = [
    {
        "name": "two_groups_weight",
        "derivation": "D=4, G=2, no gate, eps=0. Group 0 = [3,4]: mean of squares 12.5, RMS "
                      "5/sqrt2, normalised [3sqrt2/5, 4sqrt2/5], times w=[1,2]. Group 1 = [1,1]: "
                      "RMS 1, times w=[3,4]. Interleaved groups (0,2),(1,3) would give other "
                      "numbers; a sum instead of a mean would divide by 5 instead of 5/sqrt2.",
        "ngroups": 2, "eps": 0.0,
        "x": [[3.0, 4.0, 1.0, 1.0]], "z": None, "w": [1.0, 2.0, 3.0, 4.0],
        "out": [[3 * r2 / 5, 8 * r2 / 5, 3.0, 4.0]],
    },
    {
        "name": "eps_inside_root",
        "derivation": "D=2, G=1, x=[1,1], eps=3: sqrt(1+3)=2, out=[0.5,0.5]. eps added after "
                      "the root would give 1/(1+3)=0.25.",
        "ngroups": 1, "eps": 3.0,
        "x": [[1.0, 1.0]], "z": None, "w": [1.0, 1.0],
        "out": [[0.5, 0.5]],
    },
    {
        "name": "silu_gate",
        "derivation": "z=ln3 everywhere: SiLU(ln3) = ln3*sigma(ln3) = 0.75 ln3, so g = 1.5 ln3 for "
                      "x=2. eps = 3*(1.5 ln3)^2 makes the RMS sqrt(4*(1.5 ln3)^2) = 3 ln3, so out = "
                      "0.5. A sigmoid gate (g=1.5) would give 1.5/sqrt(2.25+eps) instead.",
        "ngroups": 1, "eps": 3.0 * (1.5 * ln3) ** 2,
        "x": [[2.0, 2.0]], "z": [[ln3, ln3]], "w": [1.0, 1.0],
        "out": [[0.5, 0.5]],
    },
    {
        "name": "negative_gate_flips_sign",
        "derivation": "z=-ln3: SiLU(-ln3) = -ln3*sigma(-ln3) = -ln3/4 < 0, eps=0, so g is x times "
                      "a negative constant and out = -x/RMS(x) = -[3,4]/(5/sqrt2).",
        "ngroups": 1, "eps": 0.0,
        "x": [[3.0, 4.0]], "z": [[-ln3, -ln3]], "w": [1.0, 1.0],
        "out": [[-3 * r2 / 5, -4 * r2 / 5]],
    },
]
CITATION = ("Gated grouped RMSNorm: page 'ops-transformer MambaV2 算子套件', section 4.6 "
            "(mamba2_rmsnormgated: SiLU(z) gate, grouped RMSNorm, weight w).")

if __name__ == "__main__":
    here = os.path.dirname(os.path.abspath(__file__))
    for c in CASES:
        c = dict(c, citation=CITATION)
        with open(os.path.join(here, c["name"] + ".json"), "w") as f:
            json.dump(c, f, indent=1, ensure_ascii=False)
    print("wrote", len(CASES), "fixtures")
