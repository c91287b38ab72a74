"""The polynomial of the opt-in software exponential (fa_fwd_soft_exp2):
p(f) ~ 2^f on [0, 1], degree 3, minimax in relative error by the Remez
exchange ("FlashAttention 1～4 全解汇总", FlashAttention-4, software-emulated
exponential).  Pinned against float64 2^f, the alternation theorem that
characterises the minimax polynomial, simpler approximations it must beat,
an emulation of the kernel's float32 evaluation, and the literals the kernel
source holds."""

import math
import os
import re

import numpy as np

from exact_attention_20_amd import exp2_poly as ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BOUND = 7.5e-5   # the relative error the kernel's header comment states


def rel_err(c, f):
    return np.polynomial.polynomial.polyval(f, np.asarray(c, dtype=np.float64)) / np.exp2(f) - 1.0


def test_kernel_coefficients_are_the_fit_rounded_to_float32():
    assert np.array_equal(ep.fit_float32(), ep.coeffs_from_hex())


def test_kernel_source_holds_the_same_literals():
    src = open(os.path.join(ROOT, "exact_attention_20_amd", "csrc", "fa_device.h")).read()
    body = src[src.index("float exp2_poly(float x)"):]
    body = body[: body.index("}")]
    lits = re.findall(r"(0x1\.[0-9a-f]+p[-+]?\d+)f", body)
    # Horner order in the source: c3, c2, then c1, then c0
    assert [float.fromhex(x) for x in lits] == [float.fromhex(h) for h in
                                                 (ep.KERNEL_COEFFS[3], ep.KERNEL_COEFFS[2],
                                                  ep.KERNEL_COEFFS[1], ep.KERNEL_COEFFS[0])]


def test_relative_error_bound_against_float64():
    f = np.linspace(0.0, 1.0, 2_000_001)
    err = np.abs(rel_err(ep.coeffs_from_hex(), f))
    assert err.max() <= BOUND
    assert err.max() > 5e-5   # a degree-3 polynomial cannot do much better (the levelled error)


def test_error_equioscillates_at_five_points():
    # the minimax polynomial of degree 3 attains its maximum error, with
    # alternating signs, at 3 + 2 points (Chebyshev alternation theorem)
    c, E = ep.remez()
    f = np.linspace(0.0, 1.0, 400_001)
    e = rel_err(c, f)
    sign = np.sign(e)
    runs = np.split(np.arange(f.size), np.flatnonzero(np.diff(sign) != 0) + 1)
    peaks = [e[r][np.argmax(np.abs(e[r]))] for r in runs]
    assert len(peaks) == 5
    assert all(np.sign(peaks[i]) == -np.sign(peaks[i + 1]) for i in range(4))
    assert np.allclose(np.abs(peaks), E, rtol=1e-6)
    assert f[0] == 0.0 and abs(e[0]) >= 0.999 * E and abs(e[-1]) >= 0.999 * E   # both ends are extrema


def test_beats_taylor_and_chebyshev_interpolation():
    f = np.linspace(0.0, 1.0, 200_001)
    ours = np.abs(rel_err(ep.coeffs_from_hex(), f)).max()
    ln2 = np.log(2.0)
    # Taylor about 1/2: 2^f = sqrt(2) * sum (ln2 (f - 1/2))^k / k!
    t = np.sqrt(2.0) * sum((ln2 * (f - 0.5)) ** k / math.factorial(k) for k in range(4))
    taylor = np.abs(t / np.exp2(f) - 1.0).max()
    # interpolation at the Chebyshev nodes of [0, 1]
    nodes = 0.5 - 0.5 * np.cos((2 * np.arange(4) + 1) * np.pi / 8)
    cheb = np.polynomial.polynomial.polyfit(nodes, np.exp2(nodes), 3)
    interp = np.abs(rel_err(cheb, f)).max()
    assert ours < interp < taylor


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def soft_exp2_f32(x):
    """The kernel's sequence in float32: clamp at -200 (NaN kept), n = floor,
    f = x - n, three fused multiply-adds (each rounded once to float32), and
    the exponent shifted by n (ldexp; results below the float32 range are 0
    here as they are in the kernel, which runs with denormals flushed or
    rounds them to 0 below 2^-150)."""
    x = np.where(x < -200.0, -200.0, np.asarray(x, dtype=np.float64))
    n = np.floor(x)
    f = _f32(x - n)
    c0, c1, c2, c3 = ep.coeffs_from_hex()
    p = _f32(c3 * f + c2)
    p = _f32(p * f + c1)
    p = _f32(p * f + c0)
    out = np.ldexp(p, np.where(np.isnan(n), 0.0, n).astype(np.int64))
    return np.where(out < 2.0 ** -149, 0.0, _f32(out))


def test_full_software_exp2_in_float32():
    x = _f32(np.linspace(-126.0, 64.0, 1_900_001))
    rel = np.abs(soft_exp2_f32(x) / np.exp2(x) - 1.0)
    assert rel.max() <= BOUND + 2.0 ** -22   # the fit plus float32 rounding of f and of three FMAs
    # masked scores (-inf) and far-negative arguments give exactly 0; NaN stays NaN
    assert soft_exp2_f32(np.array([-np.inf, -1000.0, -200.0, -151.0]))[0:4].tolist() == [0.0, 0.0, 0.0, 0.0]
    assert np.isnan(soft_exp2_f32(np.array([np.nan])))[0]
    # integers: p(0) * 2^n, within the bound of the exact power
    ints = np.arange(-120, 60, dtype=np.float64)
    assert np.all(np.abs(soft_exp2_f32(ints) / np.exp2(ints) - 1.0) <= BOUND)
