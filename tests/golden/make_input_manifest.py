"""Writes input_manifest.json: SHA-256 of the seeded generator's output for the
small workloads, so a change in the generator (or in numpy's RNG stream) is
caught. Calls only the input generator; no GPU code and no expected results.

    python tests/golden/make_input_manifest.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from gemm_mamba_ssm_amd import inputs  # noqa: E402


def manifest():
    out = {}
    (p,) = inputs.WORKLOADS["tiny_gemv"]
    A, W, S = inputs.make(p)
    out["tiny_gemv"] = {"A": inputs.sha256(A), "W": inputs.sha256(W), "S": inputs.sha256(S)}
    A = inputs.activations(3, 512, 77)
    W, S = inputs.weights(300, 384, 0.02, 78)
    out["m3_n300_k384_seed77"] = {"A": inputs.sha256(A), "W": inputs.sha256(W), "S": inputs.sha256(S)}
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "input_manifest.json"), "w") as f:
        json.dump(manifest(), f, indent=1, sort_keys=True)
        f.write("\n")
