"""Pins of the oracle's full-plane variant (every entry of the N x N plane corrected on
its own) against brute force, the lattice symmetry of the transfer, and the
half-plane form where the two must agree.
"""
import dataclasses

import numpy as np
import pytest

from oracle import ssb_oracle as O
from synth import WORKLOADS, cached_counts


def _geom(name, **kw):
    g = O.OGeom.from_any(WORKLOADS[name].geometry)
    return dataclasses.replace(g, **kw) if kw else g


@pytest.fixture(scope="module")
def tiny_counts():
    return cached_counts(WORKLOADS["tiny"])


def _direct_dft2(x, sign):
    n = x.shape[0]
    k = np.arange(n)
    w = np.exp(sign * 2j * np.pi * np.outer(k, k) / n)
    out = np.zeros((n, n), dtype=np.complex128)
    for a in range(n):
        for b in range(n):
            out[a, b] = np.sum(x * np.outer(w[a], w[b]))
    return out


def test_full_spectrum_brute_force(tiny_counts):
    for b in (0, 31):
        ref = _direct_dft2(tiny_counts[b].astype(np.float64), -1.0)
        got = O.scan_spectrum_full(tiny_counts[b])
        assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


def test_full_plane_q_grid_by_entry():
    """Each entry's q from its signed indices, written out per entry: index N/2 is -N/2 on
    both axes (columns too, unlike the half plane's +N/2)."""
    g = _geom("tiny", rotation_rad=0.4)
    n, s = g.scan_n, g.q_step_px
    qx, qy = O.q_vectors_full(g)
    c, sn = np.cos(0.4), np.sin(0.4)
    for u in (0, 1, 15, 16, 17, 31):
        for v in (0, 3, 16, 20, 31):
            fu = u - n if u >= n // 2 else u
            fv = v - n if v >= n // 2 else v
            ex, ey = s * fv, s * fu
            assert abs(qx[u, v] - (c * ex - sn * ey)) < 1e-15 and abs(qy[u, v] - (sn * ex + c * ey)) < 1e-15
    hx, _ = O.q_vectors(_geom("tiny"))
    assert hx[0, 16] == +16 * s and O.q_vectors_full(_geom("tiny"))[0][0, 16] == -16 * s


def test_full_plane_object_brute_force(tiny_counts):
    g = _geom("tiny")
    kx, ky = O.bf_kvectors(g)
    dc = O.dc_value(tiny_counts)
    for b in (5, 40):
        c = O.corrected_full_plane(g, tiny_counts[b], (40.0, 5.0, 0.3), kx[b], ky[b], dc)
        assert c[0, 0] == dc
        ref = _direct_dft2(c, +1.0) / 32 ** 2
        got = O.bf_object(c)
        assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


def _nyquist_lines(n):
    m = np.zeros((n, n), dtype=bool)
    m[n // 2, :] = True
    m[:, n // 2] = True
    return m


@pytest.mark.parametrize("params", [(40.0, 5.0, 0.3), (-120.0, 15.0, 2.4)])
def test_full_plane_is_extension_off_nyquist(tiny_counts, params):
    """Off the Nyquist row and column, -q of a lattice q is on the lattice, G(-q) = conj G(q)
    and T(-q) = -conj T(q), so the independently corrected plane equals the half plane's
    anti-Hermitian extension there; on those lines it does not (tiny's apertures reach them)."""
    g = _geom("tiny")
    kx, ky = O.bf_kvectors(g)
    dc = O.dc_value(tiny_counts)
    ny = _nyquist_lines(32)
    differs = 0
    for b in (0, 12, 24, 36, 48):
        full = O.corrected_full_plane(g, tiny_counts[b], params, kx[b], ky[b], dc)
        t = O.transfer(g, params, kx[b], ky[b])
        ext = O.full_plane(O.corrected_spectrum(O.scan_spectrum(tiny_counts[b]), t, dc))
        scale = np.abs(full).max()
        assert np.max(np.abs(full - ext)[~ny]) <= 1e-12 * scale
        differs += int(np.max(np.abs(full - ext)[ny]) > 1e-6 * scale)
    assert differs > 0


def test_full_plane_difference_is_two_nyquist_lines(tiny_counts):
    """ifft2 is linear: O_full - O_half = (1/N^2) [(-1)^x A(y) + (-1)^y B(x)] with A the
    inverse transform over u of the Nyquist-column differences and B that over v of the
    Nyquist-row differences (v > N/2).  Checked with the differences formed from the
    transfer at the two signs of the Nyquist frequency."""
    g = _geom("tiny")
    n, h = 32, 16
    kx, ky = O.bf_kvectors(g)
    dc = O.dc_value(tiny_counts)
    params = (40.0, 5.0, 0.3)
    s = g.q_step_px
    fu = np.fft.fftfreq(n) * n
    y = np.arange(n)
    for b in (3, 24):
        gb = O.scan_spectrum(tiny_counts[b])
        o_full = O.bf_object(O.corrected_full_plane(g, tiny_counts[b], params, kx[b], ky[b], dc))
        t = O.transfer(g, params, kx[b], ky[b])
        o_half = O.bf_object(O.full_plane(O.corrected_spectrum(gb, t, dc)))
        # column v = N/2: q_x = -N/2 s (full) versus +N/2 s (half), every u
        tcol_m = O.transfer(g, params, kx[b], ky[b], np.full(n, -h * s), s * fu)
        tcol_p = O.transfer(g, params, kx[b], ky[b], np.full(n, +h * s), s * fu)
        d_col = gb[:, h] * (tcol_m - tcol_p)
        # row u = N/2 at v = N - v' (v' = 1 .. N/2-1): conj(G(N/2, v') [T(-N/2, v') - T(+N/2, v')])
        vp = np.arange(1, h)
        trow_m = O.transfer(g, params, kx[b], ky[b], s * vp, np.full(vp.size, -h * s))
        trow_p = O.transfer(g, params, kx[b], ky[b], s * vp, np.full(vp.size, +h * s))
        d_row = np.zeros(n, dtype=np.complex128)
        d_row[n - vp] = np.conj(gb[h, vp] * (trow_m - trow_p))
        a = np.fft.ifft(d_col) * n
        bb = np.fft.ifft(d_row) * n
        pred = o_half + (((-1.0) ** y)[None, :] * a[:, None] + ((-1.0) ** y)[:, None] * bb[None, :]) / n ** 2
        assert np.max(np.abs(pred - o_full)) <= 1e-12 * np.abs(o_full).max()


def test_full_plane_equals_half_plane_without_nyquist_transfer():
    """At the small workload the transfer vanishes on both Nyquist lines for every BF, so
    the two variants give the same loss (to rounding) and the same object."""
    w = WORKLOADS["small"]
    counts = cached_counts(w)
    g = _geom("small")
    kx, ky = O.bf_kvectors(g)
    qx, qy = O.q_vectors_full(g)
    ny = _nyquist_lines(128)
    for b in range(0, 317, 29):
        t = O.transfer(g, (40.0, 5.0, 0.3), kx[b], ky[b], qx, qy)
        assert np.all(t[ny] == 0)
    dc = O.dc_value(counts)
    sub = counts[::8]
    idx = list(range(0, 317, 8))
    s1h, s2h = O.bf_moments(g, sub, (40.0, 5.0, 0.3), dc, idx)
    s1f, s2f = O.bf_moments_full_plane(g, sub, (40.0, 5.0, 0.3), dc, idx)
    assert abs(s2f - s2h) <= 1e-12 * s2h
    assert np.max(np.abs(s1f - s1h)) <= 1e-10


def test_full_plane_vacuum_and_single_sideband():
    g = _geom("tiny")
    counts = np.full((49, 32, 32), 200, dtype=np.uint32)
    assert abs(O.loss_full_plane(g, counts, (40.0, 5.0, 0.3))) < 1e-24
    # one BF, a cosine along the scan rows, zero aberration: the closed form of the half
    # plane (no Nyquist content) holds for the full plane too
    i, j = O.bf_indices(g)
    b = int(np.flatnonzero((i == 5) & (j == 8))[0])
    n, u0, a0, a1 = 32, 4, 100.0, 30.0
    y = np.arange(n)
    c1 = np.repeat((a0 + a1 * np.cos(2 * np.pi * u0 * y / n))[:, None], n, axis=1)
    s1, _ = O.bf_moments_full_plane(g, c1[None], (0.0, 0.0, 0.0), a0 * n * n, [b])
    expect = -np.arctan(a1 * np.sin(2 * np.pi * u0 * y / n) / a0)
    assert np.max(np.abs(s1 - expect[:, None])) < 1e-13


def test_full_plane_object_linearity(tiny_counts):
    g = _geom("tiny")
    kx, ky = O.bf_kvectors(g)
    dc = O.dc_value(tiny_counts)
    acc = np.zeros((32, 32), dtype=np.complex128)
    for b in range(49):
        acc += O.bf_object(O.corrected_full_plane(g, tiny_counts[b], (40.0, 5.0, 0.3), kx[b], ky[b], dc))
    phase, psi = O.object_wave_full_plane(g, tiny_counts, (40.0, 5.0, 0.3), dc)
    assert np.max(np.abs(psi - acc / 49)) < 1e-12 * np.abs(psi).max()
    assert np.max(np.abs(phase - np.angle(acc))) < 1e-12
