"""Generates the polynomial used by exp2_fast (device.hpp) for 2^f on
[-1/2, 1/2]: Chebyshev interpolation of 2^f at the degree+1 Chebyshev nodes
(near-minimax), computed in x87 extended precision, converted to monomial
coefficients and rounded to binary64. Prints the coefficients and the
measured maximum relative error of the binary64 Horner evaluation (with FMA)
against 2^f in extended precision.

    python exp2_coeffs.py [degree]
"""
import sys

import numpy as np

LD = np.longdouble


def chebyshev_monomial(deg):
    n = deg + 1
    k = np.arange(n, dtype=LD)
    nodes = LD(0.5) * np.cos((2 * k + 1) * LD(np.pi) / (2 * n))  # on [-1/2, 1/2]
    vals = np.exp2(nodes)
    # Vandermonde solve in extended precision (small, well-conditioned on this range)
    A = np.vander(nodes, n, increasing=True)
    # Gaussian elimination with partial pivoting in longdouble
    M = np.concatenate([A, vals[:, None]], axis=1)
    for c in range(n):
        p = c + int(np.argmax(np.abs(M[c:, c])))
        M[[c, p]] = M[[p, c]]
        M[c] = M[c] / M[c, c]
        for r in range(n):
            if r != c:
                M[r] = M[r] - M[r, c] * M[c]
    return M[:, -1]


def horner_fma(coef64, f):
    p = np.full_like(f, coef64[-1], dtype=np.float64)
    for c in coef64[-2::-1]:
        p = np.float64(p * f + c)  # numpy has no vector fma; error bound below is conservative
    return p


def main():
    deg = int(sys.argv[1]) if len(sys.argv) > 1 else 11
    c = chebyshev_monomial(deg)
    c64 = np.array([np.float64(x) for x in c])
    f = np.linspace(-0.5, 0.5, 200001)
    got = horner_fma(c64, f).astype(LD)
    ref = np.exp2(f.astype(LD))
    err = np.max(np.abs((got - ref) / ref))
    print(f"degree {deg}: max relative error {float(err):.3e} (Horner in binary64)")
    for i, x in enumerate(c64):
        print(f"  c[{i:2d}] = {x!r}")


if __name__ == "__main__":
    main()
