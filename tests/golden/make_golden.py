"""Writes tests/golden/tiny_layer.json from the oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
The fixture freezes the oracle's result on the tiny workload (T=32,
hidden 128, intermediate 128, 4 experts, top-2, gate/up split, seed 0) so
that any later change to the oracle's arithmetic shows up as a diff.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from oracle import moe  # noqa: E402
from workloads import gen  # noqa: E402


def main():
    s = gen.preset("tiny")
    li = gen.layer_inputs(s)
    x = moe.activations(x_bf16=li.x_bf16.view(__import__("torch").int16).numpy())
    wts = lambda e: [t.numpy() for t in gen.expert_weights(s, e)]
    out, it = moe.moe_layer(x, li.logits, s.k, wts, s.layout, return_intermediates=True)
    doc = {
        "workload": "tiny: T=32 H=128 I=128 E=4 k=2 split seed=0",
        "ids": it["ids"].tolist(),
        "w": [[float(v) for v in r] for r in it["w"]],
        "offsets": it["offsets"].tolist(),
        "perm_src": it["perm_src"].tolist(),
        "out_rows_0_1": [[float(v) for v in r] for r in out[:2]],
        "out_row_sums": [float(v) for v in out.sum(axis=1)],
        "out_abs_max": float(np.abs(out).max()),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_layer.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
