"""Writes tests/golden/oracle_tiny_layer.json from the fp64 oracle alone.

The pages print no worked numeric example, so this fixture is a regression
guard for the oracle itself: a later change to the oracle's arithmetic that
moves these numbers must name, in its commit message, the passage that
justifies it.  Inputs are drawn with numpy's PCG64 from a fixed seed and stored
in the file, so the fixture does not depend on any generator's future behaviour.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle.tpa_oracle as O  # noqa: E402

CASES = [
    # name, dims, B, T, split, causal
    ("factored_causal_chunked", O.Dims(8, 2, 4, 3, 2, 2, 10000.0), 2, 6, 2, True),
    ("kvonly_noncausal", O.Dims(6, 3, 4, 0, 2, 1, 100.0), 1, 5, 0, False),
]


def main():
    out = {"source": "fp64 oracle (oracle/tpa_oracle.py), seed 20250111", "cases": []}
    rng = np.random.default_rng(20250111)
    for name, dims, B, T, split, causal in CASES:
        x = rng.normal(0, 1, (B, T, dims.d_model))
        w = {}
        h, d = dims.n_heads, dims.head_dim
        if dims.kv_only:
            w["w_q"] = rng.normal(0, 0.5, (h * d, dims.d_model))
        else:
            w["w_a_q"] = rng.normal(0, 0.5, (h * dims.rank_q, dims.d_model))
            w["w_b_q"] = rng.normal(0, 0.5, (dims.rank_q * d, dims.d_model))
        w["w_a_k"] = rng.normal(0, 0.5, (h * dims.rank_k, dims.d_model))
        w["w_b_k"] = rng.normal(0, 0.5, (dims.rank_k * d, dims.d_model))
        w["w_a_v"] = rng.normal(0, 0.5, (h * dims.rank_v, dims.d_model))
        w["w_b_v"] = rng.normal(0, 0.5, (dims.rank_v * d, dims.d_model))
        cache = O.cache_new(dims, B, T)
        outs = []
        if split:
            outs.append(O.layer_forward(x[:, :split], w, dims, cache, 0, causal))
        outs.append(O.layer_forward(x[:, split:], w, dims, cache, split, causal))
        y = np.concatenate(outs, axis=1)
        out["cases"].append({
            "name": name, "dims": dims.__dict__, "batch": B, "tokens": T, "split": split, "causal": causal,
            "x": x.tolist(), "w": {k: v.tolist() for k, v in w.items()}, "out": y.tolist(),
        })
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_layer.json")
    with open(path, "w") as f:
        json.dump(out, f)
    print("wrote", path)


if __name__ == "__main__":
    main()
