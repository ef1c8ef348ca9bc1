"""Fits of the float polynomials in ssb_math.hpp (run by hand; prints C constants).

Lawson's iteratively reweighted least squares (C. L. Lawson, "Contributions to the
theory of linear least maximum approximation", thesis, UCLA 1961): repeated weighted
least-squares fits on a dense grid, each weight multiplied by its point's current
error, which drives the fit towards the minimax (equal-ripple) one.

* atan(t) = t (1 + sum_k c_k t^(2k)), k = 1 .. 7, on t in (0, 1], relative error.
* sin(pi f / 2) = f (s_0 + s_1 f^2 + s_2 f^4 + s_3 f^6) and
  cos(pi f / 2) = 1 + sum_k d_k f^(2k), k = 1 .. 4, on f in [-1/2, 1/2], absolute error.

The coefficients are rounded to float32 and the fits' errors are reported for
float32 evaluation (each fused multiply-add rounded once).

Usage: python aberration_phase_variance_amd/csrc/fit_math_polys.py
"""
import numpy as np


def lawson(a, b, iters=200):
    w = np.ones(a.shape[0])
    for _ in range(iters):
        sw = np.sqrt(w)
        c, *_ = np.linalg.lstsq(a * sw[:, None], b * sw, rcond=None)
        e = np.abs(a @ c - b)
        w = w * (e + 1e-300)
        w /= w.sum()
    return c


def f32(x):
    return np.float32(x).astype(np.float64) if np.isscalar(x) else x.astype(np.float32).astype(np.float64)


def fma32(a, b, c):
    """a * b + c rounded once to float32 (the product of two floats is exact in float64)."""
    return f32(a * b + c)


def horner32(coefs_hi_to_lo, s, last):
    p = np.full_like(s, coefs_hi_to_lo[0])
    for c in coefs_hi_to_lo[1:]:
        p = fma32(p, s, c)
    return fma32(p, s, last)


def fit_atan():
    t = np.concatenate([np.linspace(1e-4, 1.0, 20001), np.geomspace(1e-8, 1e-4, 200)])
    s = t * t
    r = np.arctan(t)
    a = np.stack([t * s ** k / r for k in range(1, 8)], axis=1)
    b = (r - t) / r
    c = f32(lawson(a, b))
    tt = f32(np.linspace(0.0, 1.0, 2_000_001)[1:])
    ss = f32(tt * tt)
    p = horner32(c[::-1], ss, 1.0)
    got = f32(tt * p)
    err = np.abs(got - np.arctan(tt))
    return c, err.max(), np.max(err / np.arctan(tt))


def fit_sincos():
    f = np.linspace(-0.5, 0.5, 20001)
    s = f * f
    sa = np.stack([f * s ** k for k in range(4)], axis=1)
    cs = lawson(sa, np.sin(np.pi * f / 2))
    ca = np.stack([s ** k for k in range(1, 5)], axis=1)
    cc = lawson(ca, np.cos(np.pi * f / 2) - 1.0)
    cs, cc = f32(cs), f32(cc)
    ff = f32(np.linspace(-0.5, 0.5, 2_000_001))
    s2 = f32(ff * ff)
    sn = f32(ff * horner32(cs[:0:-1], s2, cs[0]))
    cn = horner32(cc[::-1], s2, 1.0)
    return cs, cc, np.max(np.abs(sn - np.sin(np.pi * ff / 2))), np.max(np.abs(cn - np.cos(np.pi * ff / 2)))


def main():
    c, emax, rmax = fit_atan()
    print("atan: P(s) = 1 + c1 s + ... + c7 s^7, Horner from c7:")
    print("  " + ", ".join(f"{v:.9e}f" for v in c[::-1]))
    print(f"  float evaluation on (0, 1]: max abs error {emax:.2e}, max rel error {rmax:.2e}")
    cs, cc, es, ec = fit_sincos()
    print("sin(pi f/2) / f: S(s) from s3 down to s0:")
    print("  " + ", ".join(f"{v:.9e}f" for v in cs[::-1]))
    print("cos(pi f/2): C(s) = 1 + d1 s + ... + d4 s^4, Horner from d4:")
    print("  " + ", ".join(f"{v:.9e}f" for v in cc[::-1]))
    print(f"  float evaluation on [-1/2, 1/2]: max abs error sin {es:.2e}, cos {ec:.2e}")


if __name__ == "__main__":
    main()
