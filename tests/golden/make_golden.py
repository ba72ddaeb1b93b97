"""Writes the hand-derived golden fixtures in this folder.

Every expected value below is worked out by hand from the recurrence
h(t) = exp(delta*A) h(t-1) + delta x(t) (outer) B(t), y(t) = C(t).h(t) + D x(t),
then y *= silu(z); the derivation is stored next to the numbers.  Nothing
here calls the oracle or the HIP library: the values are closed forms in
ln 2, ln 3 and sqrt 2.
"""
import json
import math
import os

l2 = math.log(2.0)
ln3 = math.log(3.0)
silu_ln3 = ln3 * 0.75   # sigma(ln 3) = 3/4

CASES = [
    {
        "name": "scalar_half_decay",
        "citation": "Recurrence h(t) = A_bar h(t-1) + B_bar x(t), y(t) = C h(t): page "
                    "'ops-transformer MambaV2 算子套件', section 1.1; A_bar = exp(delta*A), "
                    "B_bar = delta*B (plain reading of 'discretised from the step size').",
        "derivation": "delta=1, A=-ln2 so A_bar=1/2. h1 = 1*1 = 1 -> y1 = 1; h2 = 1/2*1 + 2 = 2.5 "
                      "-> y2 = 2.5; h3 = 1/2*2.5 + 3 = 4.25 -> y3 = 4.25. Reading C against "
                      "h(t-1) would give 0, 1, 2.5; decaying after the input would give 1, 1.5, 2.25.",
        "shape": {"B": 1, "L": 3, "H": 1, "P": 1, "N": 1, "G": 1},
        "dt_softplus": False, "dt_limit": [0.0, None],
        "x": [[[[1.0]], [[2.0]], [[3.0]]]],
        "dt": [[[1.0], [1.0], [1.0]]],
        "A": [-l2],
        "B": [[[[1.0]], [[1.0]], [[1.0]]]],
        "C": [[[[1.0]], [[1.0]], [[1.0]]]],
        "out": [[[[1.0]], [[2.5]], [[4.25]]]],
        "final_state": [[[[4.25]]]],
    },
    {
        "name": "two_heads_one_group_D_bias",
        "citation": "Tensor semantics x[B,L,H,P], B/C[B,L,G,N], state[B,H,P,N], D skip and "
                    "dt_bias: page 'Mamba-2 SSD for Ascend NPU', section 'Implementation'; "
                    "recurrence: page 'ops-transformer MambaV2 算子套件', section 1.1.",
        "derivation": "Both heads share group 0. Head 0: delta=1, A_bar=1/2. t0: S=[1,0]x[1,2]="
                      "[[1,2],[0,0]], y=S.C0+0.5x=[1,0]+[0.5,0]=[1.5,0]. t1: S=0.5S+[2,1]x[0,1]="
                      "[[0.5,3],[0,1]], y=[3.5,1]+0.5*[2,1]=[4.5,1.5]. Head 1: dt+bias=[1,2], "
                      "A_bar=[1/2,1/4]. t0: S=[0,1]x[1,2]=[[0,0],[1,2]], y=[0,1]-[0,1]=[0,0]. "
                      "t1: S=0.25S+2*[1,-1]x[0,1]=[[0,2],[0.25,-1.5]], y=[2,-1.25]-[1,-1]=[1,-0.25].",
        "shape": {"B": 1, "L": 2, "H": 2, "P": 2, "N": 2, "G": 1},
        "dt_softplus": False, "dt_limit": [0.0, None],
        "x": [[[[1.0, 0.0], [0.0, 1.0]], [[2.0, 1.0], [1.0, -1.0]]]],
        "dt": [[[1.0, 0.5], [1.0, 1.5]]],
        "dt_bias": [0.0, 0.5],
        "A": [-l2, -l2],
        "B": [[[[1.0, 2.0]], [[0.0, 1.0]]]],
        "C": [[[[1.0, 0.0]], [[1.0, 1.0]]]],
        "D": [0.5, -1.0],
        "out": [[[[1.5, 0.0], [0.0, 0.0]], [[4.5, 1.5], [1.0, -0.25]]]],
        "final_state": [[[[0.5, 3.0], [0.0, 1.0]], [[0.0, 2.0], [0.25, -1.5]]]],
    },
    {
        "name": "softplus_initial_state_gate",
        "citation": "softplus discretisation, initial_states and the z gate y*silu(z): page "
                    "'Mamba-2 SSD for Ascend NPU', section 'Implementation' (Preprocess softplus; "
                    "StateEpilogue D/z; initial_states); recurrence: page 'ops-transformer "
                    "MambaV2 算子套件', section 1.1.",
        "derivation": "dt=0 so delta=softplus(0)=ln2; A=-1 so A_bar=1/2. h0=[2,-2]. t0: "
                      "S=0.5*[2,-2]+ln2*[1,0]=[1+ln2,-1], C0.S=ln2, silu(ln3)=0.75 ln3 -> "
                      "y0=0.75 ln2 ln3. t1: S=0.5*S+ln2*[0,1]=[(1+ln2)/2, ln2-0.5], "
                      "C1.S=(1+ln2)/2 -> y1=0.75 ln3 (1+ln2)/2.",
        "shape": {"B": 1, "L": 2, "H": 1, "P": 1, "N": 2, "G": 1},
        "dt_softplus": True, "dt_limit": [0.0, None],
        "x": [[[[1.0]], [[1.0]]]],
        "dt": [[[0.0], [0.0]]],
        "A": [-1.0],
        "B": [[[[1.0, 0.0]], [[0.0, 1.0]]]],
        "C": [[[[1.0, 1.0]], [[1.0, 0.0]]]],
        "z": [[[[ln3]], [[ln3]]]],
        "initial_states": [[[[2.0, -2.0]]]],
        "out": [[[[l2 * silu_ln3]], [[(1 + l2) / 2 * silu_ln3]]]],
        "final_state": [[[[(1 + l2) / 2, l2 - 0.5]]]],
    },
    {
        "name": "dt_limit_clamp",
        "citation": "clamp of the step to dt_limit: page 'Mamba-2 SSD for Ascend NPU', section "
                    "'Implementation' (Preprocess: softplus / clamp / decay; dt_limit listed "
                    "among supported features).",
        "derivation": "dt=[3,0.1] clamped to [0.5,2] gives delta=[2,0.5]; A=-ln2. t0: S=2*1*1=2, "
                      "y0=2. t1: S=2*2^-0.5+0.5=sqrt(2)+0.5, y1=sqrt(2)+0.5.",
        "shape": {"B": 1, "L": 2, "H": 1, "P": 1, "N": 1, "G": 1},
        "dt_softplus": False, "dt_limit": [0.5, 2.0],
        "x": [[[[1.0]], [[1.0]]]],
        "dt": [[[3.0], [0.1]]],
        "A": [-l2],
        "B": [[[[1.0]], [[1.0]]]],
        "C": [[[[1.0]], [[1.0]]]],
        "out": [[[[2.0]], [[math.sqrt(2.0) + 0.5]]]],
        "final_state": [[[[math.sqrt(2.0) + 0.5]]]],
    },
]

if __name__ == "__main__":
    here = os.path.dirname(os.path.abspath(__file__))
    for c in CASES:
        with open(os.path.join(here, c["name"] + ".json"), "w") as f:
            json.dump(c, f, indent=1, ensure_ascii=False)
    print("wrote", len(CASES), "fixtures")
