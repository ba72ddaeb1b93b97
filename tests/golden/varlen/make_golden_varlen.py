"""Writes the hand-derived fixtures of the packed variable-length forward.

Packed sequences (page "Mamba-2 SSD for Ascend NPU", "Limitations and
roadmap": varlen / cu_seqlens; page "ops-transformer MambaV2 算子套件" §1.4:
sequences concatenated on one token axis, delimited by cumulative offsets).
The recurrence is page "ops-transformer MambaV2 算子套件" §1.1 with the state
reset at every sequence start.  H = P = N = G = 1 throughout; each expected
value is worked out by hand below; nothing here calls the oracle or the HIP
library.
"""
import json
import math
import os

LN2 = math.log(2.0)

CASES = [
    {
        "name": "reset_at_boundary",
        "derivation": "cu=[0,1,3], dt=1 (no softplus) so delta=1, A=-ln2 so each step halves "
                      "the state, B=C=1, x=[1,2,3], h0=[0.5, 4]. Sequence 0: h=0.5/2+1=1.25, "
                      "y=1.25. Sequence 1 starts from its own h0=4: h=4/2+2=4, y=4; h=4/2+3=5, "
                      "y=5. Final states [1.25, 5]. Carrying 1.25 across the boundary instead "
                      "would give y=1.25/2+2=2.625 at token 1.",
        "cu_seqlens": [0, 1, 3], "dt_softplus": False,
        "x": [1.0, 2.0, 3.0], "dt": [1.0, 1.0, 1.0], "A": -LN2,
        "B": [1.0, 1.0, 1.0], "C": [1.0, 1.0, 1.0], "D": None, "h0": [0.5, 4.0],
        "out": [1.25, 4.0, 5.0], "final": [1.25, 5.0],
    },
    {
        "name": "empty_sequence_and_skip",
        "derivation": "cu=[0,2,2,3] (sequence 1 is empty), A=0 (no decay), delta=dt=[1,0.5,2], "
                      "x=[1,2,3], B=[1,2,1], C=[3,1,2], D=0.5, no h0. Sequence 0: h=1*1*1=1, "
                      "y=3*1+0.5*1=3.5; h=1+0.5*2*2=3, y=1*3+0.5*2=4. Sequence 1 has no tokens: "
                      "its final state is the (zero) initial state. Sequence 2: h=2*3*1=6, "
                      "y=2*6+0.5*3=13.5. Final states [3, 0, 6].",
        "cu_seqlens": [0, 2, 2, 3], "dt_softplus": False,
        "x": [1.0, 2.0, 3.0], "dt": [1.0, 0.5, 2.0], "A": 0.0,
        "B": [1.0, 2.0, 1.0], "C": [3.0, 1.0, 2.0], "D": 0.5, "h0": None,
        "out": [3.5, 4.0, 13.5], "final": [3.0, 0.0, 6.0],
    },
]
CITATION = ("Packed sequences: page 'Mamba-2 SSD for Ascend NPU', 'Limitations and roadmap' "
            "(varlen, cu_seqlens); page 'ops-transformer MambaV2 算子套件' §1.1 (recurrence) "
            "and §1.4 (packed batches delimited by cumulative offsets).")

if __name__ == "__main__":
    here = os.path.dirname(os.path.abspath(__file__))
    for c in CASES:
        c = dict(c, citation=CITATION)
        with open(os.path.join(here, c["name"] + ".json"), "w") as f:
            json.dump(c, f, indent=1, ensure_ascii=False)
            f.write("\n")
