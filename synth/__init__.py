"""Seeded synthetic inputs for the SSB phase-variance objective (workloads, counts, trials).

Inputs only: neither the CPU oracle nor the GPU library imports this package, and it
contains none of the objective's arithmetic.
"""
from .configs import WORKLOADS, Geometry, Workload, make_geometry, trial_params, electron_wavelength_A
from .generate import (bf_pixels, cached_counts, make_counts_numpy, make_counts_torch, make_frames_numpy,
                       make_frames_torch)

__all__ = ["WORKLOADS", "Geometry", "Workload", "make_geometry", "trial_params",
           "electron_wavelength_A", "bf_pixels", "cached_counts", "make_counts_numpy",
           "make_counts_torch", "make_frames_numpy", "make_frames_torch"]
