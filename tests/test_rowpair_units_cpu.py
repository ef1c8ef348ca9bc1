"""Host check of the row-pair units that pass 1 stores and the row pass reads back
(ssb_kernels.hip: pass1_tile's store phase, RowPairUnits): the index algebra, written out
here in NumPy from the kernel's description, must give the row pass exactly the packed
transform input it defines.

For a row pair (y0, y0 + 1) with column results C0(v), C1(v), v = 0..N/2, the row pass
transforms Z(v) = B0(v) + i B1(v), where B_k(v) = -i C_k(v) extended Hermitian
(B_k(N - v) = conj B_k(v)) with only the real parts kept at v = 0 and v = N/2.  Pass 1 stores
per column v < N/2 the unit [Z(v), Z(N - v)] (at v = 0: [(C0.y, C1.y), (C0.x, C1.x)]) and per
row pair the Nyquist unit [(C0.y, C1.y), (C0.x, C1.x)] of column N/2.  Lane j of a transform
with R values per lane and L lanes holds input index j + r L: for r < R/2 the Z half of unit
j + r L, for r >= R/2 the Z(N - w) half of unit w = N/2 - j - (r - R/2) L, and for j = 0 the
Nyquist unit's first half at r = R/2.  The transform's input built that way must equal Z,
and the inverse transform of Z must carry the two rows' imaginary object parts in its real
and imaginary halves; the second halves of the DC and Nyquist units are the real parts the
row pass adds back."""
import numpy as np
import pytest

# (N, R): the wave transform's radix per scan size (L = N / R lanes per transform)
SHAPES = [(32, 2), (64, 4), (128, 2), (256, 4), (512, 8), (1024, 16)]


def units_from_columns(c0, c1):
    """Pass 1's units for one row pair: main [N/2][2] (Z half, Z(N - v) half) and Nyquist [2]."""
    h = c0.size - 1
    zs = (c0[:h].imag + c1[:h].real) + 1j * (c1[:h].imag - c0[:h].real)
    zm = (c0[:h].imag - c1[:h].real) + 1j * (c0[:h].real + c1[:h].imag)
    zs[0] = c0[0].imag + 1j * c1[0].imag
    zm[0] = c0[0].real + 1j * c1[0].real
    main = np.stack([zs, zm], axis=1)
    nyq = np.array([c0[h].imag + 1j * c1[h].imag, c0[h].real + 1j * c1[h].real])
    return main, nyq


def row_pass_input(main, nyq, n, r_per_lane):
    """The row pass's transform input assembled lane by lane from the units."""
    h = n // 2
    lanes = n // r_per_lane
    x = np.zeros(n, dtype=complex)
    for j in range(lanes):
        for r in range(r_per_lane // 2):
            v = j + r * lanes
            x[v] = main[v, 0]
            w = h - j - r * lanes
            x[v + h] = nyq[0] if w == h else main[w, 1]
    return x


def packed_rows(c0, c1, n):
    """Z = B0 + i B1 from the definition (anti-Hermitian extension of the column results)."""
    h = n // 2
    out = []
    for c in (c0, c1):
        b = np.zeros(n, dtype=complex)
        b[1:h] = -1j * c[1:h]
        b[h + 1:] = np.conj(b[1:h][::-1])
        b[0] = (-1j * c[0]).real
        b[h] = (-1j * c[h]).real
        out.append(b)
    return out[0] + 1j * out[1], out


@pytest.mark.parametrize("n,r_per_lane", SHAPES)
def test_units_give_the_packed_transform_input(n, r_per_lane):
    rng = np.random.default_rng(n)
    h = n // 2
    c0 = rng.standard_normal(h + 1) + 1j * rng.standard_normal(h + 1)
    c1 = rng.standard_normal(h + 1) + 1j * rng.standard_normal(h + 1)
    main, nyq = units_from_columns(c0, c1)
    x = row_pass_input(main, nyq, n, r_per_lane)
    z, (b0, b1) = packed_rows(c0, c1, n)
    np.testing.assert_allclose(x, z, rtol=0, atol=1e-12)
    # the transform separates the two rows: real part row y0, imaginary part row y0 + 1
    o = np.fft.ifft(x) * n
    np.testing.assert_allclose(o.real, (np.fft.ifft(b0) * n).real, rtol=0, atol=1e-9)
    np.testing.assert_allclose(o.imag, (np.fft.ifft(b1) * n).real, rtol=0, atol=1e-9)
    # B_k is Hermitian, so each row's transform is real
    assert np.abs((np.fft.ifft(b0) * n).imag).max() < 1e-9
    # the real parts the row pass adds back: DC unit's and Nyquist unit's second halves
    assert main[0, 1] == c0[0].real + 1j * c1[0].real
    assert nyq[1] == c0[h].real + 1j * c1[h].real


def test_mirrored_columns_cover_the_upper_half_once():
    # every input index v + N/2 (v < N/2) is filled from exactly one unit half, and
    # the mirrored column w stays inside (0, N/2] for every lane and register
    for n, r_per_lane in SHAPES:
        h = n // 2
        lanes = n // r_per_lane
        ws = sorted(h - j - r * lanes for j in range(lanes) for r in range(r_per_lane // 2))
        assert ws == list(range(1, h + 1))


def test_planted_index_mistake_is_caught():
    # the mirrored column taken as N/2 - j - r L + 1 (one off) must break the equality
    n, r_per_lane = 512, 8
    rng = np.random.default_rng(7)
    h = n // 2
    c0 = rng.standard_normal(h + 1) + 1j * rng.standard_normal(h + 1)
    c1 = rng.standard_normal(h + 1) + 1j * rng.standard_normal(h + 1)
    main, nyq = units_from_columns(c0, c1)
    lanes = n // r_per_lane
    x = np.zeros(n, dtype=complex)
    for j in range(lanes):
        for r in range(r_per_lane // 2):
            v = j + r * lanes
            x[v] = main[v, 0]
            w = (h - j - r * lanes + 1) % h
            x[v + h] = main[w, 1]
    z, _ = packed_rows(c0, c1, n)
    assert np.abs(x - z).max() > 1e-3
