"""The polynomial behind the forward kernel's software 2^x (the opt-in
fa_fwd_soft_exp2 entry point): p(f) ~ 2^f on [0, 1], degree 3, minimising the
maximum RELATIVE error |p(f) / 2^f - 1| ("FlashAttention 1～4 全解汇总",
FlashAttention-4, software-emulated exponential: 2^x = 2^floor(x) * 2^frac(x),
the integer part applied to the exponent bits, the fraction by a polynomial on
the FMA units).

The coefficients come from the Remez exchange algorithm (minimax
approximation: the best polynomial of degree n equioscillates at n + 2
points), run here in float64 and rounded to float32; the kernel holds the
float32 values as hex literals (KERNEL_COEFFS below, checked against this fit
by the CPU tests).  Run as a script to print them:

    python -m exact_attention_20_amd.exp2_poly
"""

from __future__ import annotations

import numpy as np

DEGREE = 3

# float32 coefficients c0..c3 of p(f) = c0 + f (c1 + f (c2 + f c3)) as the
# kernel writes them (hex floats of fa_device.h's exp2_poly)
KERNEL_COEFFS = ("0x1.fff632p-1", "0x1.64444cp-1", "0x1.cefc4cp-3", "0x1.3f96a4p-4")


def _rel_err(c, f):
    return np.polynomial.polynomial.polyval(f, c) / np.exp2(f) - 1.0


def remez(degree: int = DEGREE, iters: int = 50, grid: int = 200001):
    """Minimax (relative error) coefficients of degree `degree` for 2^f on
    [0, 1] by the Remez exchange, and the levelled error |E|."""
    n = degree
    k = np.arange(n + 2)
    x = 0.5 - 0.5 * np.cos(np.pi * k / (n + 1))          # Chebyshev extrema as the first reference
    fine = np.linspace(0.0, 1.0, grid)
    E = 0.0
    for _ in range(iters):
        # p(x_i) - 2^x_i = (-1)^i E 2^x_i  for the n + 2 reference points
        A = np.zeros((n + 2, n + 2))
        for i, xi in enumerate(x):
            A[i, : n + 1] = xi ** np.arange(n + 1)
            A[i, n + 1] = -((-1) ** i) * np.exp2(xi)
        sol = np.linalg.solve(A, np.exp2(x))
        c, E = sol[: n + 1], sol[n + 1]
        # new reference: the extremum of the error on each run of constant sign
        e = _rel_err(c, fine)
        sign = np.sign(e)
        cuts = np.flatnonzero(np.diff(sign) != 0) + 1
        runs = np.split(np.arange(grid), cuts)
        ext = np.array([r[np.argmax(np.abs(e[r]))] for r in runs if len(r)])
        if len(ext) != n + 2:   # keep the n + 2 largest, preserving order
            keep = np.sort(np.argsort(-np.abs(e[ext]))[: n + 2])
            ext = ext[keep]
        x_new = fine[ext]
        if np.allclose(x_new, x, atol=1e-12):
            break
        x = x_new
    return c, abs(E)


def fit_float32() -> np.ndarray:
    """The fit rounded to float32 (as float64 values)."""
    c, _ = remez()
    return c.astype(np.float32).astype(np.float64)


def coeffs_from_hex(hexes=KERNEL_COEFFS) -> np.ndarray:
    return np.array([float.fromhex(h) for h in hexes])


def max_rel_error(coeffs, grid: int = 1_000_001) -> float:
    f = np.linspace(0.0, 1.0, grid)
    return float(np.max(np.abs(_rel_err(np.asarray(coeffs, dtype=np.float64), f))))


if __name__ == "__main__":
    c, E = remez()
    print("float64:", [repr(v) for v in c], "levelled |E| =", E)
    c32 = [np.float32(v) for v in c]
    print("float32:", [float(v).hex() for v in c32], "max rel err", max_rel_error(np.array(c32, dtype=np.float64)))
