"""Host-side probe fit of the library (ssb_fit_probe) against the detector oracle,
on exact integer sums (no GPU)."""
import math

import numpy as np
import pytest

import aberration_phase_variance_amd as ssb
from oracle import ssb_detector as OD
from synth import WORKLOADS, make_frames_numpy


def _same_fit(got, ref):
    assert got["n_disk"] == ref["n_disk"] and got["n_bf"] == ref["n_bf"] and got["n_zero"] == ref["n_zero"]
    assert got["det_cy"] == ref["cy"] and got["det_cx"] == ref["cx"]   # exact integer index sums / count
    assert got["bf_r2"] == ref["bf_r2"]
    assert abs(got["threshold"] - ref["threshold"]) <= 1e-12 * ref["threshold"]


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_fit_matches_oracle_on_synthetic_frames(name):
    w = WORKLOADS[name]
    g = w.geometry
    sums = OD.detector_sum(make_frames_numpy(w))
    _same_fit(ssb.ssb_fit_probe(sums, g.scan_n, g.det_n), OD.fit_probe(sums, g.scan_n, g.det_n))


def test_fit_symmetric_disk_and_dead_pixel():
    d = 40
    i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    img = np.where((i - 20) ** 2 + (j - 17) ** 2 <= 64, 300, 2).astype(np.uint64)
    img[20, 17] = 0
    got = ssb.ssb_fit_probe(img * 16, 4, d)
    _same_fit(got, OD.fit_probe(img * 16, 4, d))
    assert got["n_zero"] == 1


def test_fit_errors():
    with pytest.raises(ssb.SSBError):
        ssb.ssb_fit_probe(np.zeros(16, np.uint64), 4, 4)        # nothing above the threshold
    with pytest.raises(ssb.SSBError):
        ssb.ssb_fit_probe(np.zeros(16, np.uint64), 4, 0)
