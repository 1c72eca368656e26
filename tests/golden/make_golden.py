"""Writes the closed-form fixtures of this folder (plain `math`, no oracle or library
code):  python tests/golden/make_golden.py"""
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def bessel_envelope(rc=5.0):
    rows = ["# Radial basis and cutoff envelope at fixed distances, from their closed forms:",
            "#   B_n(r) = sqrt(2/r_c) sin(n pi r / r_c) / r, n = 1..8 (Bessel basis: 'Exascale Multi-Task Graph",
            "#   Foundation Models ...', Table IV, radial basis type Bessel; Table V, Bessel radial basis functions)",
            "#   u(r) = 1 - 28 d^6 + 48 d^7 - 21 d^8, d = r / r_c (polynomial envelope of exponent 6, within the",
            "#   4-6 range of Table IV; expanded form), u = 0 for r >= r_c",
            "# written by make_golden.py.  r_c = 5.  Columns: r u B_1 .. B_8"]
    for r in (0.5, 1.0, 2.5, 4.0, 4.99, 5.0, 6.0):
        d = r / rc
        u = 1 - 28 * d ** 6 + 48 * d ** 7 - 21 * d ** 8 if r < rc else 0.0
        b = [math.sqrt(2 / rc) * math.sin(n * math.pi * r / rc) / r for n in range(1, 9)]
        rows.append(f"{r:.17g} {u:.17g} " + " ".join(f"{x:.17g}" for x in b))
    return rows


def hilbert_one_bit():
    rows = ["# Hilbert keys of the 8 cells for one bit per axis.  In J. Skilling's transpose formulation",
            "# ('Programming the Hilbert curve', AIP Conf. Proc. 707, 2004) the one-bit case has no undo sweep,",
            "# so the transposed index is the Gray code of the corner (x, y, z) -> (x, x^y, x^y^z), read with",
            "# x most significant.  The curve orders the atoms as the space-filling-curve sort of the Tessera",
            "# abstract ('Ab Initio Accuracy Beyond the Cutoff', Abstract).  written by make_golden.py.",
            "# Columns: gx gy gz key"]
    for x in (0, 1):
        for y in (0, 1):
            for z in (0, 1):
                key = (x << 2) | ((x ^ y) << 1) | (x ^ y ^ z)
                rows.append(f"{x} {y} {z} {key}")
    return rows


if __name__ == "__main__":
    for name, rows in (("bessel_envelope_closed_form.txt", bessel_envelope()),
                       ("hilbert_one_bit.txt", hilbert_one_bit())):
        with open(os.path.join(HERE, name), "w") as f:
            f.write("\n".join(rows) + "\n")
