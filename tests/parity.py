"""Tolerances and comparison helpers for the GPU parity tests.

Forward (the stated bar):
  fp32 inputs : ||O - O_ref||_inf <= 1e-5 * ||O_ref||_inf  and
                max |LSE - LSE_ref| <= 1e-5 * max(1, ||LSE_ref||_inf)
  bf16 inputs : max |O - O_ref| <= 2e-2  and  max |LSE - LSE_ref| <= 1e-3
Backward (no bar is stated; derived from the arithmetic -- bf16 operands,
fp32 accumulation, bf16 outputs -- with >= 3x margin over a bf16 emulation):
  per tensor  : max |G - G_ref| <= 2e-2 * max(1, ||G_ref||_inf)  and
                ||G - G_ref||_F <= 1e-2 * ||G_ref||_F
fp32 backward (no bar is stated either): every product and sum in float32
(unit roundoff u = 2^-24).  A float32 CPU emulation of the same algorithm
(fp32 forward for O and LSE, P = 2^(S c - LSE2), D = rowsum(dO O), then
the five products) stays within 1.7e-6 of ||G_ref||_inf and 7e-7 in
relative Frobenius norm up to N = 2000, d = 128; the bar takes the
forward's fp32 form with >= 5x margin over that, floored at 1 like the
other bars: a gradient that is exactly 0 (one key: dS = P (dP - D) = 0)
keeps the rounding of the cancelling dP - D, of order u |dP| with
|dP| = O(1) for unit-variance inputs:
  per tensor  : max |G - G_ref| <= 1e-5 * max(1, ||G_ref||_inf)  and
                ||G - G_ref||_F <= 5e-6 * max(1, ||G_ref||_F)
Rows the oracle marks empty (LSE = -inf) must be exactly O = 0, LSE = -inf.
"""

import numpy as np

FWD_TOL = {"fp32": {"o_rel": 1e-5, "lse_rel": 1e-5}, "bf16": {"o_abs": 2e-2, "lse_abs": 1e-3}}
BWD_TOL = {"max_rel": 2e-2, "fro_rel": 1e-2}
BWD_TOL_F32 = {"max_rel": 1e-5, "fro_rel": 5e-6}


def to64(t):
    return t.detach().to("cpu").double().numpy()


def check_forward(o, lse, o_ref, lse_ref, dtype, what=""):
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty-row pattern differs"
    if empty.any():
        assert np.all(o[empty] == 0.0), f"{what}: empty rows must be zero"
    live = ~empty
    if not live.any():
        return {}
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    err_l = float(np.max(np.abs(lse[live] - lse_ref[live])))
    if dtype == "fp32":
        ref_o = float(np.max(np.abs(o_ref))) if o.size else 0.0
        ref_l = max(1.0, float(np.max(np.abs(lse_ref[live]))))
        assert err_o <= FWD_TOL["fp32"]["o_rel"] * ref_o, f"{what}: O err {err_o:.3e} vs {ref_o:.3e}"
        assert err_l <= FWD_TOL["fp32"]["lse_rel"] * ref_l, f"{what}: LSE err {err_l:.3e}"
    else:
        assert err_o <= FWD_TOL["bf16"]["o_abs"], f"{what}: O max-abs err {err_o:.3e}"
        assert err_l <= FWD_TOL["bf16"]["lse_abs"], f"{what}: LSE max-abs err {err_l:.3e}"
    return {"o_err": err_o, "lse_err": err_l}


def check_grad(g, g_ref, what=""):
    g = np.asarray(g, dtype=np.float64)
    ref_inf = float(np.max(np.abs(g_ref))) if g_ref.size else 0.0
    err = float(np.max(np.abs(g - g_ref))) if g.size else 0.0
    assert err <= BWD_TOL["max_rel"] * max(1.0, ref_inf), f"{what}: max-abs err {err:.3e} (ref {ref_inf:.3e})"
    nref = float(np.linalg.norm(g_ref))
    if nref > 0:
        fro = float(np.linalg.norm(g - g_ref)) / nref
        assert fro <= BWD_TOL["fro_rel"], f"{what}: rel-Frobenius err {fro:.3e}"
    return err


def check_grad_f32(g, g_ref, what=""):
    """The fp32 backward bar: errors relative to the reference's own size,
    or to 1 when that is smaller."""
    g = np.asarray(g, dtype=np.float64)
    ref_inf = float(np.max(np.abs(g_ref))) if g_ref.size else 0.0
    err = float(np.max(np.abs(g - g_ref))) if g.size else 0.0
    assert err <= BWD_TOL_F32["max_rel"] * max(1.0, ref_inf), f"{what}: max-abs err {err:.3e} (ref {ref_inf:.3e})"
    nref = float(np.linalg.norm(g_ref))
    fro = float(np.linalg.norm(g - g_ref)) / max(1.0, nref)
    assert fro <= BWD_TOL_F32["fro_rel"], f"{what}: rel-Frobenius err {fro:.3e} (ref {nref:.3e})"
    return err
