"""Error bound of the kernels' GELU (CPU only).

The HIP kernels evaluate GELU(z) = z * Phi(z) with Phi taken from the
complementary error function in the form of Abramowitz & Stegun, Handbook of
Mathematical Functions, formula 7.1.26 (a degree-5 polynomial in
t = 1 / (1 + p x) times exp(-x^2), absolute error <= 1.5e-7 for x >= 0).  This
test evaluates the same float32 operation sequence in NumPy and checks it
against the exact erf form from SciPy over |z| <= 12:

* the handbook formula itself stays within its published 1.5e-7 of erfc;
* the float32 GELU stays within 4.3e-7 (absolute) of the exact GELU, also
  when the reciprocal and the exp2 are each off by one unit in the last place
  (the device's v_rcp_f32 and v_exp_f32 are approximations of about that size).
"""
import numpy as np
from scipy.special import erf, erfc

F = np.float32
P = F(0.3275911)
A = [F(0.254829592), F(-0.284496736), F(1.421413741), F(-1.453152027), F(1.061405429)]


def _ulp_step(v, direction):
    if direction == 0:
        return v
    return np.nextafter(v, F(np.inf) if direction > 0 else F(-np.inf)).astype(F)


def gelu_f32(z, t_ulp=0, e_ulp=0):
    """The kernels' float32 GELU, operation by operation."""
    z = z.astype(F)
    x = np.abs(z) * F(0.70710678118654752)
    t = _ulp_step((F(1) / (P * x + F(1))).astype(F), t_ulp)
    poly = A[4] * t + A[3]
    poly = poly * t + A[2]
    poly = poly * t + A[1]
    poly = poly * t + A[0]
    e = _ulp_step(np.exp2((z * z) * F(-0.72134752044448170)).astype(F), e_ulp)   # e^(-z^2/2)
    h = F(0.5) * poly * t * e
    return z * np.where(z >= 0, F(1) - h, h)


def test_handbook_formula_bound():
    x = np.linspace(0.0, 10.0, 400_001)
    t = 1.0 / (1.0 + float(P) * x)
    poly = sum(float(a) * t ** (i + 1) for i, a in enumerate(A))
    assert np.abs(poly * np.exp(-x * x) - erfc(x)).max() <= 1.5e-7


def test_float32_gelu_bound():
    z = np.linspace(-12.0, 12.0, 800_001).astype(F)
    zd = z.astype(np.float64)
    exact = zd * 0.5 * (1.0 + erf(zd / np.sqrt(2.0)))
    worst = 0.0
    for t_ulp in (-1, 0, 1):
        for e_ulp in (-1, 0, 1):
            err = np.abs(gelu_f32(z, t_ulp, e_ulp).astype(np.float64) - exact)
            worst = max(worst, float(err.max()))
    assert worst <= 4.3e-7, worst
    # the tails: GELU(z) -> 0 for z -> -inf (no cancellation) and -> z for z -> +inf
    assert -1e-30 < gelu_f32(np.array([-12.0]))[0] <= 0.0
    assert gelu_f32(np.array([12.0]))[0] == F(12.0)
