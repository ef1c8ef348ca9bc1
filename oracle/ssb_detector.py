"""Float64/integer CPU oracle of the detector-side steps before the SSB objective.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the test suite and the benchmark's CPU legs use it.  It shares
no code with the GPU library.

Source: the quantem.gpu maintainer page "SSB performance notes" (cited as *Notes*),
sections "Cross-backend and native-size validation notes" (the automatic-probe path:
mean diffraction pattern, mean-plus-standard-deviation probe fit, disk crop),
"Automatic full-probe MPS optimizer" (the fitted center and radius select the
positive-count pixels of the disk) and "Automatic-probe detector-sum reduction"
(the mean diffraction pattern comes from an exact integer detector sum).  The fit
itself is not printed; the reading taken here:

D1  S(p) = sum over all N^2 scan frames of the counts at detector pixel p (exact
    integers); m(p) = S(p) / N^2 is the mean diffraction pattern.
D2  threshold = mean(m) + std(m) over all D^2 detector pixels (population std);
    mask = {p : m(p) > threshold}.
D3  disk center (cy, cx) = unweighted centroid of the mask; disk radius^2 =
    |mask| / pi (the radius of a disk with the mask's area).
D4  BF pixels = row-major detector pixels (i, j) with (i - cy)^2 + (j - cx)^2 <=
    radius^2 and S > 0.
D5  BF-major counts: counts[b][y][x] = frame (y N + x) at BF pixel b.
"""
from __future__ import annotations

import math

import numpy as np


def detector_sum(frames: np.ndarray) -> np.ndarray:
    """D1: exact per-pixel sums over all frames; frames [N^2][D^2] unsigned -> uint64 [D^2]."""
    return np.asarray(frames).astype(np.uint64).sum(axis=0, dtype=np.uint64)


def fit_probe(sums: np.ndarray, scan_n: int, det_n: int) -> dict:
    """D2-D4 on the exact sums: threshold, mask centroid, area radius and the BF count."""
    s = np.asarray(sums, dtype=np.uint64).reshape(det_n, det_n)
    m = s.astype(np.float64) / float(scan_n * scan_n)
    mu = float(m.mean())
    sd = float(np.sqrt(np.mean((m - mu) ** 2)))
    thr = mu + sd
    ii, jj = np.nonzero(m > thr)
    n_disk = int(ii.size)
    if n_disk == 0:
        raise ValueError("empty probe mask")
    cy = float(ii.sum()) / n_disk
    cx = float(jj.sum()) / n_disk
    r2 = n_disk / math.pi
    bi, bj = bf_pixels(s, cy, cx, r2, positive=False)
    pos = s[bi, bj] > 0
    return {"cy": cy, "cx": cx, "bf_r2": r2, "radius": math.sqrt(r2), "threshold": thr,
            "n_disk": n_disk, "n_bf": int(np.count_nonzero(pos)), "n_zero": int(np.count_nonzero(~pos))}


def bf_pixels(sums2d: np.ndarray, cy: float, cx: float, r2: float, positive: bool = True):
    """D4: row-major (i, j) inside the disk (and with a positive sum when asked)."""
    d = sums2d.shape[0]
    out_i, out_j = [], []
    for i in range(d):
        for j in range(d):
            if (i - cy) ** 2 + (j - cx) ** 2 <= r2 and (not positive or sums2d[i, j] > 0):
                out_i.append(i)
                out_j.append(j)
    return np.array(out_i, dtype=np.int64), np.array(out_j, dtype=np.int64)


def gather_bf(frames: np.ndarray, scan_n: int, det_n: int, bi: np.ndarray, bj: np.ndarray) -> np.ndarray:
    """D5: BF-major counts [n_bf][N][N] from frames [N^2][D^2]."""
    cols = np.asarray(bi) * det_n + np.asarray(bj)
    return np.ascontiguousarray(np.asarray(frames)[:, cols].T.reshape(cols.size, scan_n, scan_n))
