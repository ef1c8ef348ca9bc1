"""Pins of the float64 oracle against things other than itself.

Each test fixes part of the oracle with a brute-force computation, a closed form,
an invariant of the mathematics, or a value printed on the pages.  None of them
re-calls the oracle's own formula to check it.
"""
import dataclasses
import math
import os

import numpy as np
import pytest

from oracle import ssb_oracle as O
from synth import WORKLOADS, bf_pixels, cached_counts

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _geom(name, **kw):
    g = O.OGeom.from_any(WORKLOADS[name].geometry)
    return dataclasses.replace(g, **kw) if kw else g


def _read_golden(fname):
    out = {}
    with open(os.path.join(GOLDEN, fname)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = int(v)
    return out


# ------------------------------------------------------------------ BF set (P14)
@pytest.mark.parametrize("name,expected", [("tiny", 49), ("small", 317), ("medium", 2121), ("full", 8937)])
def test_bf_count(name, expected):
    g = _geom(name)
    i, j = O.bf_indices(g)
    assert i.size == expected
    # independent lattice count of the disk, column by column
    r2 = int(g.bf_r2)
    c = int(g.det_cy)
    count = sum(2 * math.isqrt(r2 - dy * dy) + 1 for dy in range(-math.isqrt(r2), math.isqrt(r2) + 1))
    assert count == expected
    # the generator's independent selection gives the same pixels in the same order
    gi, gj = bf_pixels(WORKLOADS[name].geometry)
    assert np.array_equal(gi, i) and np.array_equal(gj, j)
    assert c == g.det_n // 2


def test_full_counts_match_pages():
    gold = _read_golden("full_bf_count.txt")
    g = _geom("full")
    i, _ = O.bf_indices(g)
    assert g.scan_n == gold["scan_n"] and g.det_n == gold["det_n"]
    assert i.size == gold["n_bf"]
    assert i.size * g.scan_n ** 2 == gold["samples_per_eval"]


# ------------------------------------------------------------------ transforms (P1-P4)
def _direct_dft2(x, sign):
    n = x.shape[0]
    k = np.arange(n)
    w = np.exp(sign * 2j * np.pi * np.outer(k, k) / n)
    out = np.zeros((n, n), dtype=np.complex128)
    for a in range(n):           # explicit double sum, row by row
        for b in range(n):
            out[a, b] = np.sum(x * np.outer(w[a], w[b]))
    return out


@pytest.fixture(scope="module")
def tiny_counts():
    return cached_counts(WORKLOADS["tiny"])


def test_scan_spectrum_brute_force(tiny_counts):
    for b in (0, 24, 48):
        x = tiny_counts[b].astype(np.float64)
        ref = _direct_dft2(x, -1.0)[:, :17]
        got = O.scan_spectrum(tiny_counts[b])
        assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


def test_object_brute_force(tiny_counts):
    g = _geom("tiny")
    kx, ky = O.bf_kvectors(g)
    dc = O.dc_value(tiny_counts)
    n = g.scan_n
    for b in (3, 24, 40):
        t = O.transfer(g, (40.0, 5.0, 0.3), kx[b], ky[b])
        c = O.corrected_spectrum(O.scan_spectrum(tiny_counts[b]), t, dc)
        full = O.full_plane(c)
        ref = _direct_dft2(full, +1.0) / n ** 2
        got = O.bf_object(full)
        assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)
        assert np.max(np.abs(O.bf_phase(got) - np.angle(ref))) < 1e-12


def test_hermitian_half_plane(tiny_counts):
    x = tiny_counts[7].astype(np.float64)
    g = O.scan_spectrum(x)
    n = x.shape[0]
    u = np.arange(n)
    for v in (0, n // 2):
        assert np.allclose(g[(n - u) % n, v], np.conj(g[u, v]), rtol=0, atol=1e-9 * np.abs(g).max())
    # rebuild the full plane by Hermitian symmetry and compare with a complex 2-D FFT
    full = np.empty((n, n), dtype=np.complex128)
    full[:, : n // 2 + 1] = g
    for v in range(n // 2 + 1, n):
        full[:, v] = np.conj(g[(n - u) % n, n - v])
    ref = _direct_dft2(x, -1.0)
    assert np.linalg.norm(full - ref) <= 1e-12 * np.linalg.norm(ref)


def test_parseval(tiny_counts):
    n = 32
    for b in range(0, 49, 6):
        x = tiny_counts[b].astype(np.float64)
        g = O.scan_spectrum(x)
        w = np.full(g.shape[1], 2.0)
        w[0] = w[-1] = 1.0
        assert abs(np.sum(w * np.abs(g) ** 2) / n ** 2 - np.sum(x * x)) <= 1e-12 * np.sum(x * x)


def test_dc_is_exact_integer_mean(tiny_counts):
    sums = [int(v) for v in tiny_counts.reshape(49, -1).sum(axis=1, dtype=np.uint64)]
    for b in (0, 10, 48):
        assert O.scan_spectrum(tiny_counts[b])[0, 0].real == float(sums[b])
    assert O.dc_value(tiny_counts) == sum(sums) / 49


# ------------------------------------------------------------------ aperture closed form
def test_aperture_closed_form():
    g = _geom("small")                     # R_a = 10 px, w = 1 px
    assert abs(g.aperture_px - 10.0) < 1e-12
    r = np.array([0.0, 5.0, 9.5, 9.75, 10.0, 10.25, 10.5, 11.0, 30.0])
    a = O.aperture(g, r, 0.0 * r)
    assert np.allclose(a, [1, 1, 1, 0.75, 0.5, 0.25, 0, 0, 0], atol=1e-15)
    # radial: direction does not matter
    assert np.allclose(O.aperture(g, 0.6 * r, 0.8 * r), a, atol=1e-14)


def test_single_sideband_transfer_ignores_edge_weight(monkeypatch):
    """T = conj(Gamma)/|Gamma| with one shifted aperture nonzero is a unit phasor whatever
    that aperture's weight: an edge-ring weight matters only where both sidebands are in."""
    g = _geom("small")
    kx, ky = O.bf_kvectors(g)
    qx, qy = O.q_vectors(g)
    soft = O.aperture
    params = (37.0, 8.0, 1.1)
    ts = {b: O.transfer(g, params, kx[b], ky[b], qx, qy) for b in (0, 70, 200, 316)}
    monkeypatch.setattr(O, "aperture", lambda gg, x, y: (soft(gg, x, y) > 0).astype(np.float64))
    n_one = n_two = 0
    for b, t in ts.items():
        am = soft(g, kx[b] - qx, ky[b] - qy)
        ap = soft(g, kx[b] + qx, ky[b] + qy)
        hard = O.transfer(g, params, kx[b], ky[b], qx, qy)
        one = ((am > 0) != (ap > 0)) & (((am > 0) & (am < 1)) | ((ap > 0) & (ap < 1)))
        two = (am > 0) & (ap > 0) & (((am < 1) | (ap < 1)) & (np.abs(am - ap) > 0.05))
        n_one += int(one.sum())
        n_two += int(two.sum())
        assert np.max(np.abs(t[one] - hard[one])) < 1e-12
        # where both are in and the weights differ, the weights do change T
        if two.any():
            assert np.max(np.abs(t[two] - hard[two])) > 1e-3
    assert n_one > 100 and n_two > 10


# ------------------------------------------------------------------ zero aberration (P5)
def test_zero_aberration_transfer_is_sign_of_sidebands():
    g = _geom("small")
    kx, ky = O.bf_kvectors(g)
    qx, qy = O.q_vectors(g)
    ra = g.aperture_px
    for b in (0, 50, 158, 316):
        t = O.transfer(g, (0.0, 0.0, 0.0), kx[b], ky[b], qx, qy)
        assert np.all(t.imag == 0.0)
        assert set(np.unique(t.real)).issubset({-1.0, 0.0, 1.0})
        # closed form: both probe factors are exactly 1, so T = sign(a(k - q) - a(k + q))
        rm = np.hypot(kx[b] - qx, ky[b] - qy)
        rp = np.hypot(kx[b] + qx, ky[b] + qy)
        am = np.clip(ra + 0.5 - rm, 0.0, 1.0)
        ap = np.clip(ra + 0.5 - rp, 0.0, 1.0)
        assert np.array_equal(t.real, np.sign(am - ap))


def test_closed_form_single_sideband_cosine():
    """One BF, counts A0 + A1 cos(2 pi u0 y / N), zero aberration: phi(y) = -atan(A1 sin / A0)."""
    g = _geom("tiny")                      # N = 32, R_a = 4, s = 0.5
    i, j = O.bf_indices(g)
    b = int(np.flatnonzero((i == 5) & (j == 8))[0])   # kappa = (0, -3) px
    n, u0, a0, a1 = 32, 4, 100.0, 30.0             # q0 = (0, 2) px: k - q0 outside, k + q0 inside
    y = np.arange(n)
    counts = np.repeat((a0 + a1 * np.cos(2 * np.pi * u0 * y / n))[:, None], n, axis=1)
    dc = a0 * n * n
    s1, s2 = O.bf_moments(g, counts[None], (0.0, 0.0, 0.0), dc, [b])
    expect = -np.arctan(a1 * np.sin(2 * np.pi * u0 * y / n) / a0)
    assert np.max(np.abs(s1 - expect[:, None])) < 1e-13
    assert abs(s2 - n * np.sum(expect ** 2)) < 1e-11


def test_closed_form_sideband_with_aberration():
    """Same single-sideband case with defocus: C(q0) = -G(q0) exp(i(chi(k) - chi(k+q0)))."""
    g = _geom("tiny")
    i, j = O.bf_indices(g)
    b = int(np.flatnonzero((i == 5) & (j == 8))[0])
    n, u0, a0, a1 = 32, 4, 100.0, 30.0
    y = np.arange(n)
    counts = np.repeat((a0 + a1 * np.cos(2 * np.pi * u0 * y / n))[:, None], n, axis=1)
    params = (25.0, 0.0, 0.0)
    # chi written out for k = (0, -3) px, k + q0 = (0, -1), k - q0 = (0, -5)
    lam, dk = g.wavelength_A, g.dk
    c10 = float(np.float32(25.0)) * 10.0
    chi = lambda r2: math.pi * lam * dk * dk * c10 * r2
    ph = chi(9.0) - chi(1.0)
    s1, _ = O.bf_moments(g, counts[None], params, a0 * n * n, [b])
    # C(u0) = -(A1 N^2/2) e^{i ph}; C(-u0) = -conj(C(u0)) -> O = A0 + (A1/2)(-e^{i(ph+th)} + e^{-i(ph+th)})
    th = 2 * np.pi * u0 * y / n
    o = a0 + 0.5 * a1 * (-np.exp(1j * (ph + th)) + np.exp(-1j * (ph + th)))
    assert np.max(np.abs(s1 - np.angle(o)[:, None])) < 1e-12


# ------------------------------------------------------------------ inactive BF (P6), vacuum (P7)
def test_inactive_bf_phase_is_zero():
    w = WORKLOADS["tiny"]
    counts = cached_counts(w)
    # shrink the probe aperture to 2.5 px: BF pixels beyond 3 px have a(k_b) = 0
    g = _geom("tiny")
    g = dataclasses.replace(g, alpha_rad=g.alpha_rad * 2.5 / g.aperture_px)
    kx, ky = O.bf_kvectors(g)
    inactive = np.flatnonzero(kx ** 2 + ky ** 2 >= 9.0)
    assert inactive.size > 10
    dc = O.dc_value(counts)
    for b in inactive[:5]:
        s1, s2 = O.bf_moments(g, counts[b][None], (40.0, 5.0, 0.3), dc, [b])
        assert np.all(s1 == 0.0) and s2 == 0.0
    # they still count in n_bf: loss over all == moments over the active ones, normalized by 49
    s1a, s2a = O.bf_moments(g, counts, (40.0, 5.0, 0.3), dc)
    assert O.loss(g, counts, (40.0, 5.0, 0.3), dc) == O.loss_from_moments(s1a, s2a, 49)


@pytest.mark.parametrize("params", [(0.0, 0.0, 0.0), (40.0, 5.0, 0.3), (-150.0, 18.0, 2.0)])
def test_vacuum_loss_is_zero(params):
    g = _geom("tiny")
    counts = np.full((49, 32, 32), 200, dtype=np.uint32)
    assert abs(O.loss(g, counts, params)) < 1e-24


# ------------------------------------------------------------------ symmetry (P8, P9)
def test_transfer_antihermitian():
    g = _geom("small")
    kx, ky = O.bf_kvectors(g)
    qx, qy = O.q_vectors(g)
    for b in (5, 120, 300):
        t = O.transfer(g, (33.0, -7.0, 1.1), kx[b], ky[b], qx, qy)
        tm = O.transfer(g, (33.0, -7.0, 1.1), kx[b], ky[b], -qx, -qy)
        assert np.max(np.abs(tm + np.conj(t))) < 1e-12


def test_conjugate_branch_small():
    """Negating q (rotation by pi) and the aberrations negates every BF phase exactly.

    At the small workload every Nyquist-line entry has zero transfer, so the
    identity holds to rounding (the Notes page reports agreement within 1.13e-7
    on real data, where Nyquist terms break it slightly).
    """
    w = WORKLOADS["small"]
    counts = cached_counts(w)
    g = _geom("small")
    kx, ky = O.bf_kvectors(g)
    qx, qy = O.q_vectors(g)
    dc = O.dc_value(counts)
    s1p = np.zeros((128, 128))
    s1m = np.zeros((128, 128))
    for b in range(0, 317, 3):
        gb = O.scan_spectrum(counts[b])
        tp = O.transfer(g, (40.0, 5.0, 0.3), kx[b], ky[b], qx, qy)
        tm = O.transfer(g, (-40.0, -5.0, 0.3), kx[b], ky[b], -qx, -qy)
        pp = O.bf_phase(O.bf_object(O.full_plane(O.corrected_spectrum(gb, tp, dc))))
        pm = O.bf_phase(O.bf_object(O.full_plane(O.corrected_spectrum(gb, tm, dc))))
        assert np.max(np.abs(pp + pm)) < 1e-12
        s1p += pp
        s1m += pm
    assert np.max(np.abs(s1p + s1m)) < 1e-10


# ------------------------------------------------------------------ object linearity (P10)
def test_phase_of_mean_linearity(tiny_counts):
    g = _geom("tiny")
    kx, ky = O.bf_kvectors(g)
    dc = O.dc_value(tiny_counts)
    acc = np.zeros((32, 32), dtype=np.complex128)
    for b in range(49):
        t = O.transfer(g, (40.0, 5.0, 0.3), kx[b], ky[b])
        acc += O.bf_object(O.full_plane(O.corrected_spectrum(O.scan_spectrum(tiny_counts[b]), t, dc)))
    phase, psi = O.object_wave(g, tiny_counts, (40.0, 5.0, 0.3), dc)
    assert np.max(np.abs(psi - acc / 49)) < 1e-12 * np.abs(psi).max()
    assert np.max(np.abs(phase - np.angle(acc))) < 1e-12


def test_real_part_of_bf_object_depends_on_row_and_column_parity(tiny_counts):
    """Away from its v = 0 and v = N/2 columns the extended plane is anti-Hermitian, so those
    entries transform to a purely imaginary object; the v = 0 column (with the DC term) adds
    a term constant along each row and the Nyquist column one that alternates in sign with x.
    So Re O_b(y, x) depends on x only through its parity: the fact that lets a row pass carry
    the object's real part as two sums per row."""
    g = _geom("tiny")
    kx, ky = O.bf_kvectors(g)
    dc = O.dc_value(tiny_counts)
    for b in (0, 17, 48):
        t = O.transfer(g, (40.0, 5.0, 0.3), kx[b], ky[b])
        c = O.corrected_spectrum(O.scan_spectrum(tiny_counts[b]), t, dc)
        obj = O.bf_object(O.full_plane(c))
        re = obj.real
        scale = np.abs(obj).max()
        assert np.max(np.abs(re - np.tile(re[:, :2], (1, 16)))) < 1e-12 * scale
        # the two parity terms are the v = 0 and v = N/2 columns' transforms along the rows
        col0 = np.fft.ifft(c[:, 0]) / 32
        nyq = np.fft.ifft(c[:, 16]) / 32
        assert np.max(np.abs(re[:, 0] - (col0.real + nyq.real))) < 1e-12 * scale
        assert np.max(np.abs(re[:, 1] - (col0.real - nyq.real))) < 1e-12 * scale
        # and with those columns removed the object is purely imaginary
        c2 = c.copy()
        c2[:, 0] = 0.0
        c2[:, 16] = 0.0
        assert np.max(np.abs(O.bf_object(O.full_plane(c2)).real)) < 1e-12 * scale


# ------------------------------------------------------------------ physics (P13)
@pytest.fixture(scope="module")
def small_setup():
    w = WORKLOADS["small"]
    counts = cached_counts(w)
    return _geom("small"), counts, O.dc_value(counts)


def test_defocus_minimum_at_truth(small_setup):
    g, counts, dc = small_setup
    grid = [20.0, 30.0, 35.0, 40.0, 45.0, 50.0, 60.0]
    losses = [O.loss(g, counts, (c10, 5.0, 0.3), dc) for c10 in grid]
    assert grid[int(np.argmin(losses))] == 40.0
    assert max(losses) > 1.3 * min(losses)


def test_astigmatism_minimum_at_truth(small_setup):
    g, counts, dc = small_setup
    ref = O.loss(g, counts, (40.0, 5.0, 0.3), dc)
    for other in [(40.0, 0.0, 0.3), (40.0, 10.0, 0.3), (40.0, -5.0, 0.3),
                  (40.0, 5.0, -0.3), (40.0, 5.0, 0.3 + math.pi / 4)]:
        assert O.loss(g, counts, other, dc) > ref * 1.1


# ------------------------------------------------------------------ two-pass half-plane form
def test_two_pass_half_plane_equals_definition(tiny_counts):
    """Column IFFT over the half plane, then the anti-Hermitian row extension and a row
    IFFT, reproduces ifft2 of the full plane; and its imaginary part is the real inverse
    transform (C2R) of -i times the column result, its real part set by columns 0 and N/2.
    """
    g = _geom("tiny")
    n, h = 32, 16
    kx, ky = O.bf_kvectors(g)
    dc = O.dc_value(tiny_counts)
    for b in (2, 30):
        t = O.transfer(g, (-60.0, 12.0, 2.2), kx[b], ky[b])
        c = O.corrected_spectrum(O.scan_spectrum(tiny_counts[b]), t, dc)
        ref = O.bf_object(O.full_plane(c))
        a = np.fft.ifft(c, axis=0)                     # (N, N/2+1) column transforms
        row = np.empty((n, n), dtype=np.complex128)
        row[:, : h + 1] = a
        for v in range(h + 1, n):
            row[:, v] = -np.conj(a[:, n - v])
        two_pass = np.fft.ifft(row, axis=1)
        assert np.linalg.norm(two_pass - ref) <= 1e-13 * np.linalg.norm(ref)
        im = np.fft.irfft(-1j * a, n=n, axis=1)        # C2R: imag parts of bins 0 and N/2 ignored
        x = np.arange(n)
        re = (a[:, 0].real[:, None] + ((-1.0) ** x)[None, :] * a[:, h].real[:, None]) / n
        assert np.max(np.abs(im - ref.imag)) < 1e-12 * np.abs(ref).max()
        assert np.max(np.abs(re - ref.real)) < 1e-12 * np.abs(ref).max()


# ------------------------------------------------------------------ loss formula (O12)
def _variance_pin(loss_fn):
    """loss_fn(s1, s2, n_bf) against the population variance over BF of a phase stack,
    averaged over pixels (numpy's var with ddof = 0), and against a two-BF, 2 x 2 example
    worked by hand: per-pixel variances ((a - b)/2)^2 = 0.01, 0.01, 0, 0.16, mean 0.045."""
    rng = np.random.Generator(np.random.PCG64(7))
    ok = True
    for n_bf, n in ((2, 2), (5, 8), (37, 16)):
        phi = rng.uniform(-math.pi, math.pi, (n_bf, n, n))
        ref = float(np.var(phi, axis=0).mean())
        got = loss_fn(phi.sum(axis=0), float((phi * phi).sum()), n_bf)
        ok = ok and abs(got - ref) <= 1e-14 * max(1.0, abs(ref))
    phi = np.array([[[0.1, 0.2], [0.3, 0.4]], [[0.3, 0.0], [0.3, -0.4]]])
    got = loss_fn(phi.sum(axis=0), float((phi * phi).sum()), 2)
    return ok and abs(got - 0.045) <= 1e-15


def test_loss_from_moments_is_population_variance():
    assert _variance_pin(O.loss_from_moments)


def test_loss_is_variance_of_per_bf_phases(tiny_counts):
    """The whole loss equals numpy's population variance over the stack of per-BF phase
    images, each built by its own 2-D inverse DFT (written out as a direct sum here)."""
    g = _geom("tiny")
    kx, ky = O.bf_kvectors(g)
    dc = O.dc_value(tiny_counts)
    params = (-55.0, 11.0, 1.9)
    stack = []
    for b in range(49):
        t = O.transfer(g, params, kx[b], ky[b])
        full = O.full_plane(O.corrected_spectrum(O.scan_spectrum(tiny_counts[b]), t, dc))
        stack.append(np.angle(_direct_dft2(full, +1.0)))
    ref = float(np.var(np.array(stack), axis=0).mean())
    assert abs(O.loss(g, tiny_counts, params, dc) - ref) <= 1e-12 * ref


def test_variance_pin_catches_planted_mistakes():
    """Plausible slips in the loss formula each fail the variance pin."""
    def sample_var(s1, s2, n_bf):              # divides by n_bf - 1
        n2 = s1.size
        return (s2 - float(np.sum(s1 * s1)) / n_bf) / ((n_bf - 1) * n2)

    def var_of_mean(s1, s2, n_bf):             # variance of the mean phase image instead
        m = s1 / n_bf
        return float(np.var(m))

    def no_pixel_norm(s1, s2, n_bf):           # drops the 1/N^2 of the second term
        return s2 / (n_bf * s1.size) - float(np.sum((s1 / n_bf) ** 2))

    for bad in (sample_var, var_of_mean, no_pixel_norm):
        assert not _variance_pin(bad), bad.__name__


# ------------------------------------------------------------------ rotation branch of q (O5)
def _rotation_pin(qfun):
    """qfun(g) -> (qx, qy) against the scan frequencies rotated counterclockwise by rho
    written as a complex product: (qx + i qy) = e^{i rho} s (v + i u'), u' signed
    (fftfreq), v = 0 .. N/2."""
    ok = True
    for name, rho in (("tiny", 0.3), ("tiny", -2.1), ("small", 0.3 + math.pi)):
        g = _geom(name, rotation_rad=rho)
        n = g.scan_n
        u = np.arange(n)
        up = np.where(u < n // 2, u, u - n).astype(np.float64)
        v = np.arange(n // 2 + 1, dtype=np.float64)
        z = np.exp(1j * rho) * g.q_step_px * (v[None, :] + 1j * up[:, None])
        qx, qy = qfun(g)
        ok = ok and np.max(np.abs(qx - z.real)) < 1e-12 and np.max(np.abs(qy - z.imag)) < 1e-12
    return ok


def test_q_rotation_is_counterclockwise():
    assert _rotation_pin(O.q_vectors)


def test_rotation_pin_catches_planted_mistake():
    def flipped(g):                            # the sine term of one component with the wrong sign
        qx, qy = O.q_vectors(dataclasses.replace(g, rotation_rad=0.0))
        c, s = math.cos(g.rotation_rad), math.sin(g.rotation_rad)
        return c * qx + s * qy, s * qx + c * qy

    def transposed(g):                         # u and v swapped before rotating
        qx, qy = O.q_vectors(dataclasses.replace(g, rotation_rad=0.0))
        c, s = math.cos(g.rotation_rad), math.sin(g.rotation_rad)
        return c * qy - s * qx, s * qy + c * qx

    assert not _rotation_pin(flipped)
    assert not _rotation_pin(transposed)


def test_transfer_rotation_covariance():
    """With pure defocus and a round aperture the probe is rotation invariant, so
    rotating the scan frequencies by rho equals rotating the BF offset by -rho:
    T_rho(q; k) = T_0(q; Rot(-rho) k) (both shifted apertures move together)."""
    g0 = _geom("small")
    rho = 0.7
    g = dataclasses.replace(g0, rotation_rad=rho)
    kx, ky = O.bf_kvectors(g0)
    c, s = math.cos(rho), math.sin(rho)
    for b in (3, 150, 301):
        kxr, kyr = c * kx[b] + s * ky[b], -s * kx[b] + c * ky[b]
        t_rot = O.transfer(g, (-37.0, 0.0, 0.0), kx[b], ky[b])
        t_ref = O.transfer(g0, (-37.0, 0.0, 0.0), kxr, kyr)
        assert np.max(np.abs(t_rot - t_ref)) < 1e-12, b
    # the opposite sense of rotation fails the same check
    t_bad = O.transfer(dataclasses.replace(g0, rotation_rad=-rho), (-37.0, 0.0, 0.0), kx[150], ky[150])
    kxr, kyr = c * kx[150] + s * ky[150], -s * kx[150] + c * ky[150]
    assert np.count_nonzero(np.abs(t_bad - O.transfer(g0, (-37.0, 0.0, 0.0), kxr, kyr)) > 1e-9) > 100


def test_conjugate_branch_through_rotation():
    """L(rho + pi, -theta) = L(rho, theta) with the conjugate branch reached through the
    geometry's rotation (q -> -q) and negated aberrations (Notes, "Conditional joint
    rotation check": the 180-degree branch reverses the aberration signs).  At the small
    workload no Nyquist-line entry has nonzero transfer, so the identity is exact to
    rounding; per-BF phases are exact negatives."""
    w = WORKLOADS["small"]
    counts = cached_counts(w)
    dc = O.dc_value(counts)
    ga = _geom("small", rotation_rad=0.3)
    gb = _geom("small", rotation_rad=0.3 + math.pi)
    la = O.loss(ga, counts, (40.0, 5.0, 0.3), dc)
    lb = O.loss(gb, counts, (-40.0, -5.0, 0.3), dc)
    assert abs(la - lb) <= 1e-12 * la
    s1a, _ = O.bf_moments(ga, counts[:40], (40.0, 5.0, 0.3), dc, list(range(40)))
    s1b, _ = O.bf_moments(gb, counts[:40], (-40.0, -5.0, 0.3), dc, list(range(40)))
    assert np.max(np.abs(s1a + s1b)) < 1e-10
    # and it is not a tautology: the same aberrations on the rotated branch differ
    assert abs(O.loss(gb, counts, (40.0, 5.0, 0.3), dc) - la) > 1e-3 * la
