"""Writes the stored hashes under tests/golden/.

  inputs_sha256.json          sha256 of every named workload's A and B bytes
                              (from the seeded generator only)
  oracle_outputs_sha256.json  sha256 of the oracle's C for the small 512^3
                              workload (calls only the oracle)

Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads as wl  # noqa: E402


def main():
    hashes = {}
    for name, w in wl.WORKLOADS.items():
        a, b = wl.generate(w)
        hashes[name] = {"A": wl.sha256_of(a), "B": wl.sha256_of(b)}
    with open(os.path.join(HERE, "inputs_sha256.json"), "w") as f:
        json.dump(hashes, f, indent=1, sort_keys=True)
    w = wl.WORKLOADS["small_512"]
    a, b = wl.generate(w)
    c = oracle.gemm_relu(a, b, w.M, w.N, w.K)
    with open(os.path.join(HERE, "oracle_outputs_sha256.json"), "w") as f:
        json.dump({"small_512": wl.sha256_of(c)}, f, indent=1)


if __name__ == "__main__":
    main()
