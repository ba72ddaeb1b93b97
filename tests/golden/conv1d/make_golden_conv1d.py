"""Writes the hand-derived fixtures of the depthwise causal conv1d.

Page "ops-transformer MambaV2 算子套件", §1.4 and §4.1 (mamba2_causal_conv1d:
width-4 depthwise causal conv over time, bias, SiLU; reference = grouped
conv1d padded by W-1 and cut to the first S steps).  Each expected value is
worked out by hand below; nothing here calls the oracle or the HIP library.
"""
import json
import math
import os

LN3 = math.log(3.0)

CASES = [
    {
        "name": "tap_order_digits",
        "derivation": "One channel, W=4, taps w=[1,10,100,1000], x=[1,2,3,4,5], no bias, no "
                      "activation. Tap k weighs x[t-3+k], so w[3]=1000 weighs the current step: "
                      "out[0]=1000*1, out[1]=100*1+1000*2=2100, out[2]=10+200+3000=3210, "
                      "out[3]=1+20+300+4000=4321, out[4]=2+30+400+5000=5432. Reversed taps "
                      "would give out[0]=1. The final conv state is the last three inputs [3,4,5].",
        "x": [[[1.0, 2.0, 3.0, 4.0, 5.0]]], "w": [[1.0, 10.0, 100.0, 1000.0]], "bias": None,
        "x_prev": None, "activation": False,
        "out": [[[1000.0, 2100.0, 3210.0, 4321.0, 5432.0]]], "final": [[[3.0, 4.0, 5.0]]],
    },
    {
        "name": "conv_state_and_bias_silu",
        "derivation": "One channel, W=3, taps w=[1,1,1], bias b=ln3-3, x=[1,2], previous "
                      "state x_prev=[1,1]. Pre-activation: out[0]=1+1+1+b=ln3, "
                      "out[1]=1+1+2+b=ln3+1. SiLU(ln3)=ln3*sigma(ln3)=0.75*ln3; "
                      "SiLU(ln3+1)=(ln3+1)/(1+e^-(ln3+1))=(ln3+1)/(1+1/(3e)). The final state "
                      "is the last two inputs [1,2]; with a zero state out[0] would be ln3-2.",
        "x": [[[1.0, 2.0]]], "w": [[1.0, 1.0, 1.0]], "bias": [LN3 - 3.0],
        "x_prev": [[[1.0, 1.0]]], "activation": True,
        "out": [[[0.75 * LN3, (LN3 + 1.0) / (1.0 + 1.0 / (3.0 * math.e))]]],
        "final": [[[1.0, 2.0]]],
    },
    {
        "name": "short_sequence_state_carry",
        "derivation": "Two channels, W=4, S=2 < W-1: the final state mixes the previous state "
                      "and the input. Channel 0: x_prev=[7,8,9], x=[1,2], w=[0,0,0,1] (identity): "
                      "out=[1,2], final=[9,1,2]. Channel 1: x_prev=[1,2,3], x=[4,5], "
                      "w=[1,0,0,0] (delay 3): out=[x[-3], x[-2]]=[1,2], final=[3,4,5].",
        "x": [[[1.0, 2.0], [4.0, 5.0]]], "w": [[0.0, 0.0, 0.0, 1.0], [1.0, 0.0, 0.0, 0.0]],
        "bias": None, "x_prev": [[[7.0, 8.0, 9.0], [1.0, 2.0, 3.0]]], "activation": False,
        "out": [[[1.0, 2.0], [1.0, 2.0]]], "final": [[[9.0, 1.0, 2.0], [3.0, 4.0, 5.0]]],
    },
]
CITATION = ("Causal conv1d: page 'ops-transformer MambaV2 算子套件', §1.4 (width-4 depthwise "
            "causal conv then SiLU, cached conv states) and §4.1 (mamba2_causal_conv1d: x [B,D,S], "
            "per-channel weight and bias, reference = conv1d with groups=D, padding W-1, cut to "
            "S steps, then SiLU).")

if __name__ == "__main__":
    here = os.path.dirname(os.path.abspath(__file__))
    for c in CASES:
        c = dict(c, citation=CITATION)
        with open(os.path.join(here, c["name"] + ".json"), "w") as f:
            json.dump(c, f, indent=1, ensure_ascii=False)
            f.write("\n")
