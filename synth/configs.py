"""Workload definitions for the SSB phase-variance objective.

Four scan/detector sizes follow the workloads the SSB performance notes
(quantem.gpu "SSB performance notes" and "Later SSB performance
checkpoints") measure on: the full one is a 512 x 512 scan with a
192 x 192 detector and 8,937 bright-field (BF) pixels (checkpoints page,
section "2026-09-11 full-aperture Apple M5 floor checkpoint").  The smaller
ones keep the same optics and scale the scan and detector down so a float64
CPU oracle finishes in seconds.  A fifth, ``full1024``, is the 1024 x 1024
scan of the size-scaling runs (notes page, "128 GB Apple M5 Max size-scaling
follow-up"): same optics, detector and BF set as the full one, the scan field
twice as wide at the same step.  Those runs zero-pad the 512 spectra instead,
which integer counts cannot express; the transform length, the BF count and
the 4.2 MB spectrum per BF pixel are the same.

Everything here is plain numbers: the beam energy, the probe semi-angle,
the BF disk, and the derived sampling.  Nothing in this module evaluates the
objective.

Geometry conventions (the pages do not print them; these are the readings
used on both sides of every parity check):

* Detector pixel (i, j) is row i, column j; the detector center is
  (cy, cx) = (D/2, D/2) and the BF set is every pixel with
  (i - cy)^2 + (j - cx)^2 <= bf_r2, in row-major order.
* The probe aperture edge (a(k) = 1/2) sits on the BF disk radius, which fixes
  the detector sampling dk = k_alpha / sqrt(bf_r2) in 1/Angstrom per pixel.
* The scan step equals one pixel of the D x D probe window, 1 / (D dk), so
  one scan-frequency index is D/N detector pixels (``q_step_px``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, asdict

# CODATA 2018 exact / recommended constants (SI).
_H = 6.62607015e-34
_M0 = 9.1093837015e-31
_E = 1.602176634e-19
_C = 299792458.0


def electron_wavelength_A(kv: float) -> float:
    """Relativistic electron wavelength in Angstrom for an accelerating voltage in kV."""
    ev = _E * kv * 1e3
    lam_m = _H / math.sqrt(2.0 * _M0 * ev * (1.0 + ev / (2.0 * _M0 * _C * _C)))
    return lam_m * 1e10


@dataclass(frozen=True)
class Geometry:
    """Sampling and optics of one workload, in detector-pixel units where possible."""

    scan_n: int          # N: scan side (power of two)
    det_n: int           # D: detector side
    bf_r2: float         # BF disk radius squared, detector pixels^2
    det_cy: float        # detector center row (pixels)
    det_cx: float        # detector center column (pixels)
    q_step_px: float     # detector pixels per scan-frequency index, 1/(N * scan_step * dk)
    dk: float            # detector sampling, 1/Angstrom per pixel
    wavelength_A: float  # electron wavelength, Angstrom
    alpha_rad: float     # probe-forming semi-angle, rad
    rotation_rad: float  # scan-to-detector rotation, rad
    edge_px: float       # width of the soft aperture edge, detector pixels

    @property
    def scan_step_A(self) -> float:
        return 1.0 / (self.scan_n * self.q_step_px * self.dk)

    @property
    def aperture_px(self) -> float:
        """Aperture radius k_alpha / dk in detector pixels."""
        return self.alpha_rad / self.wavelength_A / self.dk

    def as_dict(self) -> dict:
        return asdict(self)


@dataclass(frozen=True)
class Workload:
    name: str
    geometry: Geometry
    n_bf: int                 # expected BF count for the disk rule
    true_params: tuple        # (C10 nm, C12 nm, phi12 rad) used to simulate the probe
    object_sigma_px: float    # Gaussian smoothing of the random phase field
    object_strength: float    # phase amplitude of the specimen (rad per unit std)
    dose: float               # mean counts per BF pixel (I0)
    object_seed: int
    poisson_seed: int
    trial_seed: int
    n_trials: int
    c10_range_nm: tuple
    c12_range_nm: tuple | None
    phi12_range: tuple | None


KV = 300.0
ALPHA = 0.020
TRUE_PARAMS = (40.0, 5.0, 0.3)


def make_geometry(scan_n: int, det_n: int, bf_r2: int, *, kv: float = KV, alpha: float = ALPHA,
                  rotation: float = 0.0, edge_px: float = 1.0) -> Geometry:
    lam = electron_wavelength_A(kv)
    k_alpha = alpha / lam
    dk = k_alpha / math.sqrt(bf_r2)
    return Geometry(scan_n=scan_n, det_n=det_n, bf_r2=float(bf_r2),
                    det_cy=det_n / 2.0, det_cx=det_n / 2.0,
                    q_step_px=det_n / scan_n, dk=dk, wavelength_A=lam,
                    alpha_rad=alpha, rotation_rad=rotation, edge_px=edge_px)


def _workload(name, n, d, r2, n_bf, n_trials, c10, c12=None, phi=None):
    return Workload(name=name, geometry=make_geometry(n, d, r2), n_bf=n_bf,
                    true_params=TRUE_PARAMS, object_sigma_px=2.0, object_strength=0.2,
                    dose=200.0, object_seed=42, poisson_seed=43, trial_seed=42,
                    n_trials=n_trials, c10_range_nm=c10, c12_range_nm=c12, phi12_range=phi)


WORKLOADS = {
    # one evaluation at the true parameters
    "tiny": _workload("tiny", 32, 16, 16, 49, 1, (40.0, 40.0)),
    # 200 random defocus trials, C12 / phi12 fixed at their true values
    "small": _workload("small", 128, 48, 100, 317, 200, (-100.0, 100.0)),
    "medium": _workload("medium", 256, 96, 676, 2121, 200, (-100.0, 100.0)),
    # the full field: 512^2 scan x 8,937 BF
    "full": _workload("full", 512, 192, 2837, 8937, 200, (-200.0, 200.0), (-20.0, 20.0), (0.0, math.pi)),
    # the 1024^2 scan of the size-scaling runs: the full workload's optics, detector and
    # 8,937 BF, scanned over a field twice as wide at the same step (1024-point
    # transforms, 4.2 MB of spectrum per BF pixel)
    "full1024": _workload("full1024", 1024, 192, 2837, 8937, 200, (-200.0, 200.0), (-20.0, 20.0),
                          (0.0, math.pi)),
}


def trial_params(w: Workload, n: int | None = None):
    """Seeded trial parameters, float32 [n][3] = (C10 nm, C12 nm, phi12 rad)."""
    import numpy as np

    n = w.n_trials if n is None else n
    rng = np.random.Generator(np.random.PCG64(w.trial_seed))
    out = np.empty((n, 3), dtype=np.float64)
    out[:, 0] = rng.uniform(w.c10_range_nm[0], w.c10_range_nm[1], n)
    if w.c12_range_nm is None:
        out[:, 1] = w.true_params[1]
        out[:, 2] = w.true_params[2]
    else:
        out[:, 1] = rng.uniform(w.c12_range_nm[0], w.c12_range_nm[1], n)
        out[:, 2] = rng.uniform(w.phi12_range[0], w.phi12_range[1], n)
    if w.name == "tiny":
        out[:] = w.true_params
    return out.astype(np.float32)
