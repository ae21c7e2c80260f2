"""Writes gelu_examples.json: GELU(x) = x * Phi(x) at textbook points.

Phi values are standard normal table entries (15 significant digits), typed
in below; the expected bf16 bits are x * Phi(x) rounded to nearest even by
the oracle's fp64 -> bf16 conversion (itself pinned by bf16_rounding.json).
The script checks that every case lies well away from a rounding midpoint,
so the table's last digits cannot decide the rounding.  Run from the
repository root: python tests/golden/make_gelu_examples.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "..", ".."))
import oracle  # noqa: E402

PHI = [(0.5, "0.691462461274963"), (1.0, "0.841344746068543"), (2.0, "0.977249868051821"),
       (3.0, "0.998650101968370"), (-0.5, "0.308537538725037"), (-1.0, "0.158655253931457"),
       (-2.0, "0.022750131948179"), (-3.0, "0.001349898031630"), (-4.0, "3.16712418331200e-05"),
       (-6.0, "9.86587645037698e-10"), (-10.0, "7.61985302416047e-24")]


def main():
    cases = []
    for x, phi in PHI:
        g = x * float(phi)
        e = np.frexp(abs(g))[1]
        frac = (abs(g) / 2.0 ** (e - 8)) % 1.0
        assert abs(frac - 0.5) > 0.03, (x, frac)  # at least 0.03 ulp from a midpoint
        cases.append({"x": x, "phi": phi, "expected_bits": f"0x{oracle.f64_to_bf16(g):04x}"})
    out = {"source": "GELU(x) = x * Phi(x) with Phi the standard normal CDF (the exact, erf-based GELU of "
                     "Hendrycks and Gimpel, 'Gaussian Error Linear Units'); Phi values from standard normal "
                     "tables (15 significant digits). expected_bits = bf16 round-to-nearest-even of x*Phi(x); "
                     "every case lies at least 0.037 bf16 ulp away from a rounding midpoint, so the table "
                     "digits decide the rounding. Written by make_gelu_examples.py.",
           "cases": cases}
    with open(os.path.join(HERE, "gelu_examples.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
