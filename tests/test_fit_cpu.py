"""Host-side checks of the fit driver's Nelder-Mead refinement (ssb_nelder_mead in
libssb.so, called through the binding with Python objectives; no GPU).

The simplex is compared with scipy.optimize's Nelder-Mead started from the same
initial simplex with the same tolerances on the same float32-input objective: the
two implementations of the standard method must request the same number of points
and end at the same vertex (up to the rounding order of the reflection formula).
"""
import numpy as np
import pytest
import scipy.optimize as so

import aberration_phase_variance_amd as ssb


def _quad(p):
    p = np.asarray(p, dtype=np.float32).astype(np.float64)
    return ((p[0] - 41.3) ** 2 / 50 + (p[1] - 4.2) ** 2 / 3 + 20 * (p[2] - 0.35) ** 2
            + 0.02 * (p[0] - 41.3) * (p[1] - 4.2))


def _rosen(p):
    p = np.asarray(p, dtype=np.float32).astype(np.float64)
    return (1 - p[0] / 50) ** 2 + 100 * (p[1] / 5 - (p[0] / 50) ** 2) ** 2 + (p[2] - 0.3) ** 2


def _steps(x0):
    """The pages' initial axis steps: 5% of the start value, floors 0.01 / 2 nm / 0.04 rad, two decimals."""
    floors = (0.01, 2.0, 0.04)
    out = []
    for x, fl in zip(x0, floors):
        m = round(max(abs(x) * 0.05, fl), 2) or 0.01
        out.append(-m if x < 0 else m)
    return out


@pytest.mark.parametrize("fn,x0,tol", [(_quad, [30.0, 9.0, 0.1], (1e-4, 1e-10)),
                                       (_quad, [-20.0, 60.0, 2.0], (1e-3, 1e-9)),
                                       (_rosen, [10.0, 1.0, 0.0], (1e-4, 1e-10))])
def test_matches_scipy_nelder_mead(fn, x0, tol):
    xatol, fatol = tol
    r = ssb.ssb_nelder_mead(x0, fn, {"xatol": xatol, "fatol": fatol, "max_iter": 2000})
    sim = np.array([x0] + [np.array(x0) + np.eye(3)[k] * s for k, s in enumerate(_steps(x0))])
    s = so.minimize(fn, x0, method="Nelder-Mead",
                    options={"initial_simplex": sim, "xatol": xatol, "fatol": fatol, "maxiter": 2000,
                             "maxfev": 10 ** 7})
    assert r["converged"] == 1
    assert r["requests"] == s.nfev
    assert np.max(np.abs(np.array(r["best"]) - s.x)) <= 1e-9 * max(1.0, np.max(np.abs(s.x)))
    assert abs(r["loss"] - s.fun) <= 1e-12 * max(1.0, abs(s.fun))


def test_initial_simplex_follows_the_policy():
    """First four evaluations: the start and one step per axis (5% of C10; C12 and phi12
    floored at 2 nm and 0.04 rad; two decimals)."""
    x0 = [73.64, 10.2, 0.387]
    r = ssb.ssb_nelder_mead(x0, _quad, {"max_evals": 4})
    t = r["trace"]
    assert r["evals"] == 4 and r["converged"] == 0
    np.testing.assert_array_equal(t[0, :3], np.float32(x0))
    expect = [3.68, 2.0, 0.04]
    for k in range(3):
        want = np.array(x0, dtype=np.float64)
        want[k] += expect[k]
        np.testing.assert_array_equal(t[k + 1, :3], np.float32(want))


def test_float32_repeats_are_memoized():
    """Near 1e6 a float32 step is 0.0625, so a collapsing simplex requests float32
    triples it has already evaluated: those reuse the stored loss."""
    calls = []

    def f(p):
        calls.append(tuple(np.asarray(p, dtype=np.float32)))
        q = np.asarray(p, dtype=np.float32).astype(np.float64)
        return (q[0] - 1e6 - 0.3) ** 2 + (q[1] - 2.0) ** 2 + (q[2] - 0.5) ** 2

    r = ssb.ssb_nelder_mead([1e6 + 7.0, 3.0, 0.4], f, {"xatol": 1e-9, "fatol": 0.0, "max_iter": 300})
    assert len(calls) == r["evals"] == len(set(calls))       # one call per distinct float32 triple
    assert r["requests"] > r["evals"]
    assert r["loss"] == min(t[3] for t in r["trace"])


def test_evaluation_cap_and_errors():
    r = ssb.ssb_nelder_mead([30.0, 9.0, 0.1], _quad, {"max_evals": 10})
    assert r["evals"] == 10 and r["converged"] == 0
    assert r["loss"] == r["trace"][:, 3].min()
    with pytest.raises(ssb.SSBError) as e:
        ssb.ssb_nelder_mead([float("nan"), 1.0, 0.0], _quad)
    assert e.value.code == ssb._ssb.SSB_EINVAL
    with pytest.raises(ssb.SSBError) as e:
        ssb.ssb_nelder_mead([1.0, 1.0, 0.0], lambda p: float("nan"))
    assert e.value.code == ssb._ssb.SSB_EINVAL
