"""CPU test: the oracle reproduces its stored regression fixture."""
import json
import os

import numpy as np

import oracle.tpa_oracle as O

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_tiny_layer.json")


def test_oracle_matches_golden():
    with open(_PATH) as f:
        data = json.load(f)
    for case in data["cases"]:
        dims = O.Dims(**case["dims"])
        x = np.array(case["x"])
        w = {k: np.array(v) for k, v in case["w"].items()}
        B, T, split, causal = case["batch"], case["tokens"], case["split"], case["causal"]
        cache = O.cache_new(dims, B, T)
        outs = []
        if split:
            outs.append(O.layer_forward(x[:, :split], w, dims, cache, 0, causal))
        outs.append(O.layer_forward(x[:, split:], w, dims, cache, split, causal))
        got = np.concatenate(outs, axis=1)
        np.testing.assert_allclose(got, np.array(case["out"]), rtol=0, atol=1e-13, err_msg=case["name"])
