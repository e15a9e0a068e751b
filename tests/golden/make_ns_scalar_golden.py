"""Write ns_scalar.json: the scalar Newton-Schulz map composed k times.

Calls only ``oracle`` (its exact-rational scalar map).  The values are the
singular-value map that k Newton-Schulz iterations apply, for the quintic
coefficients (3.4445, -4.7750, 2.0315) and for the cubic Newton-Schulz
iteration (1.5, -0.5, 0) [textbook: Bjorck & Bowie 1971; Higham, Functions of
Matrices, ch. 8].  Run from the repository root:

    python tests/golden/make_ns_scalar_golden.py
"""

import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(
    os.path.abspath(__file__)))))

from oracle import quintic_scalar_exact  # noqa: E402

SIGMAS = ["1", "0.5", "0.1", "0.01", "0.001", "0.0001", "0.9", "0.3"]
COEFFS = {"quintic": ["3.4445", "-4.7750", "2.0315"],
          "cubic": ["1.5", "-0.5", "0"]}


def main():
    out = {"note": "p composed k times at sigma, p(s) = a s + b s^3 + c s^5; "
                   "exact rational arithmetic rounded to binary64",
           "values": {}}
    for name, abc in COEFFS.items():
        from fractions import Fraction
        q = [Fraction(x) for x in abc]
        table = {}
        for s in SIGMAS:
            table[s] = [float(quintic_scalar_exact(Fraction(s), k, q))
                        for k in range(0, 6)]
        out["values"][name] = {"abc": abc, "by_sigma": table}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "ns_scalar.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
