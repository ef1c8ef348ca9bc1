"""Pins of the detector-side oracle (oracle/ssb_detector.py) against facts that do not
come from its own arithmetic: brute-force integer sums, symmetric disks whose centroid is
exact, lattice counts, and index-encoded frames."""
import math

import numpy as np

from oracle import ssb_detector as OD


def test_detector_sum_brute_force_and_no_overflow():
    rng = np.random.default_rng(5)
    frames = rng.integers(0, 2 ** 32, size=(37, 12), dtype=np.uint64).astype(np.uint32)
    frames[:, 3] = 2 ** 32 - 1                       # the sum exceeds 32 bits
    got = OD.detector_sum(frames)
    for p in range(12):
        assert int(got[p]) == sum(int(v) for v in frames[:, p])
    assert got.dtype == np.uint64 and int(got[3]) == 37 * (2 ** 32 - 1)


def _disk_image(d, cy, cx, r2, inside=100, outside=0):
    i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    return np.where((i - cy) ** 2 + (j - cx) ** 2 <= r2, inside, outside).astype(np.uint64)


def test_fit_symmetric_disk_is_exact():
    """A uniform disk about a lattice point covering < 1/2 of the detector: the
    threshold lies between the two levels, the mask is the disk, the centroid is the
    center exactly, and the area radius reproduces the lattice count."""
    d, n = 40, 8
    img = _disk_image(d, 20, 20, 81)                 # radius 9
    count = sum(1 for i in range(d) for j in range(d) if (i - 20) ** 2 + (j - 20) ** 2 <= 81)
    f = OD.fit_probe(img * n * n, n, d)              # sums of n^2 identical frames
    assert 0 < f["threshold"] < 100
    assert f["n_disk"] == count
    assert f["cy"] == 20.0 and f["cx"] == 20.0
    assert f["bf_r2"] == count / math.pi
    # mean + population std of a two-level image, by hand
    p = count / d ** 2
    assert abs(f["threshold"] - 100 * (p + math.sqrt(p * (1 - p)))) < 1e-9
    # the BF disk of the fitted area radius, counted directly
    want = sum(1 for i in range(d) for j in range(d) if (i - 20) ** 2 + (j - 20) ** 2 <= count / math.pi)
    assert f["n_bf"] == want and f["n_zero"] == 0


def test_fit_off_lattice_center():
    d = 48
    img = _disk_image(d, 20.3, 18.7, 11.0 ** 2, inside=50, outside=1)
    f = OD.fit_probe(img, 1, d)
    # lattice sampling of an off-lattice disk moves the centroid by a fraction of a pixel
    assert abs(f["cy"] - 20.3) < 0.1 and abs(f["cx"] - 18.7) < 0.1
    assert abs(f["radius"] - 11.0) < 0.1


def test_bf_requires_positive_sum():
    d = 30
    img = _disk_image(d, 15, 15, 36)
    img[15, 15] = 0                                   # a dead pixel at the center
    f = OD.fit_probe(img, 1, d)
    assert f["n_zero"] == 1
    bi, bj = OD.bf_pixels(img, f["cy"], f["cx"], f["bf_r2"])
    assert bi.size == f["n_bf"] and not np.any((bi == 15) & (bj == 15))


def test_gather_index_encoded():
    n, d = 8, 6
    s = np.arange(n * n)[:, None]
    p = np.arange(d * d)[None, :]
    frames = (s * d * d + p).astype(np.uint32)
    bi = np.array([0, 2, 5, 3])
    bj = np.array([1, 4, 0, 3])
    got = OD.gather_bf(frames, n, d, bi, bj)
    for b in range(4):
        for y in range(n):
            for x in range(n):
                assert got[b, y, x] == (y * n + x) * d * d + bi[b] * d + bj[b]
