"""The device code's own float atan2 and sincos (csrc/ssb_math.hpp), compiled for the host
with g++ and swept against float64 libm (NumPy) over dense grids.

On the host the division inside atan2 is exact; the device uses the hardware reciprocal
(about 1 ulp), which moves t = min/max by at most ~1.2e-7 relative and atan(t) by at
most ~6e-8 rad more.  The bounds below are the host ones the fits were made for."""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "aberration_phase_variance_amd", "csrc")

ATAN2_MAX_REL = 2.9e-7      # relative, every angle
ATAN2_MAX_ERR = 3.9e-7      # rad, every angle (one float ulp near pi is 2.4e-7)
ATAN2_OCTANT_ERR = 1.9e-7   # rad, |phase| <= pi/4 (the row pass's usual range)
COSSIN_MAX_ERR = 1.2e-7

SRC = r'''
#include "ssb_math.hpp"
extern "C" void sweep_atan2(const float* y, const float* x, float* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = ssb::atan2_f(y[i], x[i]);
}
extern "C" void sweep_cossin(const float* r, float* c, float* s, long n) {
    for (long i = 0; i < n; ++i) ssb::cossin_rev_cs(r[i], c[i], s[i]);
}
'''


@pytest.fixture(scope="module")
def mathlib(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("ssbmath")
    src = d / "sweep.cpp"
    src.write_text(SRC)
    so = d / "libsweep.so"
    subprocess.run([cxx, "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-I", CSRC, str(src), "-o", str(so)],
                   check=True)
    lib = ctypes.CDLL(str(so))
    fp = ctypes.POINTER(ctypes.c_float)
    lib.sweep_atan2.argtypes = [fp, fp, fp, ctypes.c_long]
    lib.sweep_cossin.argtypes = [fp, fp, fp, ctypes.c_long]
    return lib


def _p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _atan2(lib, y, x):
    y = np.ascontiguousarray(y, np.float32)
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty_like(y)
    lib.sweep_atan2(_p(y), _p(x), _p(out), y.size)
    return out


def test_atan2_accuracy(mathlib):
    rng = np.random.Generator(np.random.PCG64(11))
    th = np.concatenate([rng.uniform(-np.pi, np.pi, 2_000_000),
                         np.arange(-8, 9) * (np.pi / 8)])              # octant edges
    mag = np.exp(rng.uniform(np.log(1e-6), np.log(1e6), th.size))
    y = (mag * np.sin(th)).astype(np.float32)
    x = (mag * np.cos(th)).astype(np.float32)
    got = _atan2(mathlib, y, x).astype(np.float64)
    ref = np.arctan2(y.astype(np.float64), x.astype(np.float64))
    err = np.abs(np.angle(np.exp(1j * (got - ref))))
    assert err.max() <= ATAN2_MAX_ERR, err.max()
    nz = np.abs(ref) > 0
    assert np.max(err[nz] / np.abs(ref[nz])) <= ATAN2_MAX_REL
    # the range the row pass meets most: Re > 0, |Im| <= Re (t = Im / Re in [-1, 1])
    t = np.linspace(-1.0, 1.0, 400_001).astype(np.float32)
    got = _atan2(mathlib, t, np.ones_like(t)).astype(np.float64)
    assert np.max(np.abs(got - np.arctan(t.astype(np.float64)))) <= ATAN2_OCTANT_ERR


def test_atan2_special_values(mathlib):
    y = np.array([0.0, -0.0, 0.0, -0.0, 1.0, -1.0, 1.0, np.nan, 0.0, np.inf], np.float32)
    x = np.array([0.0, 0.0, -1.0, -1.0, 0.0, 0.0, -1.0, 1.0, np.nan, 1.0], np.float32)
    got = _atan2(mathlib, y, x)
    assert got[0] == 0.0 and got[1] == 0.0
    assert abs(got[2] - np.pi) < 1e-6 and abs(got[3] + np.pi) < 1e-6       # the branch cut's two sides
    assert abs(got[4] - np.pi / 2) < 1e-6 and abs(got[5] + np.pi / 2) < 1e-6
    assert abs(got[6] - 3 * np.pi / 4) < 1e-6
    assert np.isnan(got[7]) and np.isnan(got[8])
    assert np.all(np.abs(got[:7]) <= np.float32(np.pi))


def test_cossin_accuracy(mathlib):
    r = np.concatenate([np.linspace(-0.5, 0.5, 2_000_001), np.arange(-4, 5) / 8.0]).astype(np.float32)
    c = np.empty_like(r)
    s = np.empty_like(r)
    mathlib.sweep_cossin(_p(r), _p(c), _p(s), r.size)
    a = 2 * np.pi * r.astype(np.float64)
    assert np.max(np.abs(c - np.cos(a))) <= COSSIN_MAX_ERR
    assert np.max(np.abs(s - np.sin(a))) <= COSSIN_MAX_ERR
    # quarter turns land on exact axes
    q = np.arange(-4, 5) / 8.0
    idx = r.size - 9 + np.arange(9)
    assert np.all(np.abs(c[idx[::2]] - np.cos(2 * np.pi * q[::2])) <= 1e-7)
