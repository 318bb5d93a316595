"""Writes erf_phi_table.txt: erf(x) and Phi(x) = (1 + erf(x / sqrt(2))) / 2 at a
few points, computed with mpmath in 50-digit arithmetic and rounded to 16
significant digits. Run from anywhere: python tests/golden/make_erf_phi_table.py
"""
import os

import mpmath

HERE = os.path.dirname(os.path.abspath(__file__))
ERF_X = ["0.1", "0.25", "0.5", "0.75", "1.0", "1.5", "2.0", "2.5", "3.0"]
PHI_X = ["0.5", "1.0", "1.5", "2.0", "3.0", "4.0"]

HEADER = """\
# Values of the error function and of the standard normal distribution
# function Phi(x) = (1 + erf(x / sqrt(2))) / 2, computed by make_erf_phi_table.py
# (mpmath, 50 decimal digits of working precision, rounded to 16 significant
# digits). The abscissae are points that printed tables of these functions list
# (e.g. Abramowitz and Stegun, Handbook of Mathematical Functions, Tables 7.1
# and 26.1); the printed tables carry fewer digits than these values.
# These pin the oracle's erf-form GELU, GELU(z) = z * Phi(z), the activation of
# the fused epilogue ("TileLang: Write, Autotune, and Ship Fused Tensor-Core
# Kernels from Python", section "Why tile-level control matters").
# kind  x     value
"""


def main():
    mpmath.mp.dps = 50
    rows = [("erf", x, mpmath.erf(mpmath.mpf(x))) for x in ERF_X]
    rows += [("phi", x, mpmath.ncdf(mpmath.mpf(x))) for x in PHI_X]
    with open(os.path.join(HERE, "erf_phi_table.txt"), "w") as f:
        f.write(HEADER)
        for kind, x, v in rows:
            f.write("%-7s %-5s %s\n" % (kind, x, mpmath.nstr(v, 16, min_fixed=-10, max_fixed=10,
                                                              strip_zeros=False)))


if __name__ == "__main__":
    main()
