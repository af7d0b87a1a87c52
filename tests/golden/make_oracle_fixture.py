"""Write oracle_regression_small.json: the fp64 oracle's output on a small
seeded problem (block = window = 8, D = 16, H = 2, T = 40).  Calls only the
oracle and the seeded input generator."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

SEED, T, H, D, BLOCK = 77, 40, 2, 16, 8


def inputs():
    return (synth.normal_bf16(SEED, synth.Q, (T, H, D)), synth.normal_bf16(SEED, synth.G, (T, H, D)),
            synth.normal_bf16(SEED, synth.K, (T, D)), synth.normal_bf16(SEED, synth.V, (T, D)))


def compute():
    q, g, k, v = inputs()
    ck, cv = oracle.compress(k, BLOCK), oracle.compress(v, BLOCK)
    return oracle.attn(q, g, np.arange(T), k, v, 0, ck, cv, block=BLOCK, window=BLOCK,
                       scale=1.0 / np.sqrt(D))


if __name__ == "__main__":
    out = compute()
    rec = {"seed": SEED, "T": T, "H": H, "D": D, "block": BLOCK, "window": BLOCK,
           "scale": "1/sqrt(D)", "out": [float(x).hex() for x in out.ravel()]}
    with open(os.path.join(HERE, "oracle_regression_small.json"), "w") as f:
        json.dump(rec, f)
    print("wrote", out.size, "values")
