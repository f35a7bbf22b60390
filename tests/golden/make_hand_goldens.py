"""Writes rope_hand.json and attn_hand.json from closed-form expressions.

Every number is a hand derivation (cosines and sines of stated angles, simple
fractions, logarithms); this script only evaluates those expressions.  It calls
neither the oracle nor the GPU library.
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    r2 = math.sqrt(2.0)
    rope = {
        "cite": "zhao9797 page, 模型架构 (standard RoPE, base theta); RoFormer rotation of pairs (x[2i],x[2i+1]) by pos*theta^(-2i/D)",
        "cases": [
            {"D": 4, "theta": 100.0, "pos": 2, "x": [1.0, 0.0, 0.0, 1.0],
             "derivation": "w = (100^0, 100^(-1/2)) = (1, 0.1); angles (2, 0.2); (1,0)->(cos2, sin2); (0,1)->(-sin0.2, cos0.2)",
             "y": [math.cos(2.0), math.sin(2.0), -math.sin(0.2), math.cos(0.2)]},
            {"D": 128, "theta": 10000.0, "pos": 1, "pair": 1,
             "derivation": "unit vector on pair 1 at pos 1 turns by w_1 = 10000^(-2/128) rad",
             "angle": 10000.0 ** (-2.0 / 128.0)},
            {"D": 2, "theta": 5e7, "pos": 0, "x": [0.3, -1.7],
             "derivation": "pos 0: angle 0, identity", "y": [0.3, -1.7]},
        ],
    }
    l2, l3 = math.log(2.0), math.log(3.0)
    attn = {
        "cite": "exact softmax attention (elamur.ai summary: no approximation); causal mask (zhao9797 page, 模型架构); packing mask (zhao9797 page, 训练方法)",
        "D": 2, "scale": 1.0 / r2,
        "q": [[r2, 0.0], [r2, 0.0], [r2, 0.0]],
        "k": [[0.0, 0.0], [l3, 0.0], [l2, 0.0]],
        "v": [[1.0, 0.0], [0.0, 1.0], [2.0, -2.0]],
        "derivation": "s_ij = (1/sqrt2)*<q_i,k_j> = (0, ln3, ln2)[j]; exp(s) = (1,3,2). Causal row 1: P=(1/4,3/4), LSE=ln4; row 2: P=(1/6,1/2,1/3), LSE=ln6, O=(1/6+2/3, 1/2-2/3). Non-causal: every row equals causal row 2. Segments [0,0,1], causal: row 2 sees only itself, O=v_2, LSE=s_22=ln2.",
        "causal": {"o": [[1.0, 0.0], [0.25, 0.75], [5.0 / 6.0, -1.0 / 6.0]], "lse": [0.0, math.log(4.0), math.log(6.0)]},
        "noncausal": {"o": [[5.0 / 6.0, -1.0 / 6.0]] * 3, "lse": [math.log(6.0)] * 3},
        "causal_segments": {"segment_ids": [0, 0, 1], "o": [[1.0, 0.0], [0.25, 0.75], [2.0, -2.0]],
                            "lse": [0.0, math.log(4.0), l2]},
        "bwd": {
            "dout": [[0.0, 0.0], [0.0, 0.0], [1.0, 0.0]],
            "derivation": "only row 2 has dO. Delta=<dO_2,O_2>=5/6. dP_2j=<dO_2,v_j>=(1,0,2). dS_2j=P_2j(dP_2j-Delta)=(1/36,-5/12,7/18). dq_2=scale*sum_j dS_2j k_j=((-5/12 ln3+7/18 ln2)/sqrt2, 0). dk_j=scale*dS_2j*q_2=dS_2j*(1,0). dv_j=P_2j*dO_2=((1/6,0),(1/2,0),(1/3,0)).",
            "dq": [[0.0, 0.0], [0.0, 0.0], [(-5.0 / 12.0 * l3 + 7.0 / 18.0 * l2) / r2, 0.0]],
            "dk": [[1.0 / 36.0, 0.0], [-5.0 / 12.0, 0.0], [7.0 / 18.0, 0.0]],
            "dv": [[1.0 / 6.0, 0.0], [0.5, 0.0], [1.0 / 3.0, 0.0]],
        },
    }
    with open(os.path.join(HERE, "rope_hand.json"), "w") as f:
        json.dump(rope, f, indent=1, ensure_ascii=False)
    with open(os.path.join(HERE, "attn_hand.json"), "w") as f:
        json.dump(attn, f, indent=1, ensure_ascii=False)


if __name__ == "__main__":
    main()
