"""Seeded synthetic 4D-STEM bright-field counts.

This module only makes inputs.  It simulates a weak phase specimen scanned by
an aberrated probe and draws Poisson counts; it holds none of the objective's
arithmetic and neither the oracle nor the GPU library imports it.  Both sides
receive the same count bytes.

Forward model (the workload description of the SSB notes names its pieces:
a probe made of an aperture times exp(-i chi), a Gaussian-smoothed random phase
field, and Poisson counts of |FFT2(probe * transmission)|^2):

1. phi: N x N standard-normal field from PCG64(object_seed), smoothed with a
   periodic Gaussian of sigma px (multiplication by exp(-2 pi^2 sigma^2 |f|^2)
   in Fourier space), then shifted and scaled to zero mean and unit standard
   deviation.  Transmission t = exp(i * strength * phi).
2. Probe in the detector plane, centered at (D/2, D/2):
   A(k) = a(k) exp(-i chi(k)), soft aperture a(k) = clip((R_a - |k|)/w + 1/2, 0, 1)
   with R_a = alpha / (lambda dk) pixels; chi(k) = pi lambda dk^2 [C10 |k|^2 +
   C12 ((kx^2 - ky^2) cos 2 phi12 + 2 kx ky sin 2 phi12)], k in pixels, C in
   Angstrom.  Real-space probe P = ifft2(ifftshift(A)) on a D x D window whose
   pixel equals the scan step.
3. For scan position (y0, x0) the exit wave is P(m) t((y0, x0) + r(m)) where the
   window offset r(m) = m for m < D/2 and m - D otherwise (the probe is centered
   on the window origin, wrapping).  I = |fftshift(fft2(exit wave))|^2 and the
   counts at BF pixel b are Poisson(dose * I[b]).

Poisson draws are taken scan row by scan row (y0), then x0, then BF index,
from PCG64(poisson_seed) (NumPy back end).  The torch back end, used for the
full 512^2 x 8,937 workload whose 2.3e9 draws are too slow on host cores, runs
the same model on the device in complex64 with a seeded torch generator; its
bytes differ from the NumPy back end's but both sides of a parity check always
receive the same bytes.
"""
from __future__ import annotations

import hashlib
import os

import numpy as np

from .configs import Workload, Geometry


def bf_pixels(g: Geometry):
    """Detector (row, col) of every BF pixel in row-major order (integer disk rule)."""
    ii, jj = np.meshgrid(np.arange(g.det_n), np.arange(g.det_n), indexing="ij")
    inside = (ii - g.det_cy) ** 2 + (jj - g.det_cx) ** 2 <= g.bf_r2
    return ii[inside].astype(np.int64), jj[inside].astype(np.int64)


def object_phase(w: Workload) -> np.ndarray:
    n = w.geometry.scan_n
    rng = np.random.Generator(np.random.PCG64(w.object_seed))
    white = rng.standard_normal((n, n))
    f = np.fft.fftfreq(n)
    f2 = f[:, None] ** 2 + f[None, :] ** 2
    smooth = np.real(np.fft.ifft2(np.fft.fft2(white) * np.exp(-2.0 * np.pi ** 2 * w.object_sigma_px ** 2 * f2)))
    return (smooth - smooth.mean()) / smooth.std()


def probe_window(w: Workload) -> np.ndarray:
    g = w.geometry
    d = g.det_n
    ky, kx = np.meshgrid(np.arange(d) - g.det_cy, np.arange(d) - g.det_cx, indexing="ij")
    kr = np.sqrt(kx ** 2 + ky ** 2)
    amp = np.clip((g.aperture_px - kr) / g.edge_px + 0.5, 0.0, 1.0)
    c10 = float(w.true_params[0]) * 10.0
    c12 = float(w.true_params[1]) * 10.0
    phi12 = float(w.true_params[2])
    chi = np.pi * g.wavelength_A * g.dk ** 2 * (
        c10 * (kx ** 2 + ky ** 2)
        + c12 * ((kx ** 2 - ky ** 2) * np.cos(2 * phi12) + 2 * kx * ky * np.sin(2 * phi12)))
    a_det = amp * np.exp(-1j * chi)
    return np.fft.ifft2(np.fft.ifftshift(a_det))


def _window_offsets(d: int) -> np.ndarray:
    m = np.arange(d)
    return np.where(m < d // 2, m, m - d)


def make_counts_numpy(w: Workload) -> np.ndarray:
    """uint32 counts [n_bf][N][N] (BF-major, BF order of ``bf_pixels``)."""
    g = w.geometry
    n, d = g.scan_n, g.det_n
    t = np.exp(1j * w.object_strength * object_phase(w))
    probe = probe_window(w)
    bi, bj = bf_pixels(g)
    # detector pixels after fftshift: shifted index s -> unshifted (s - d//2) % d
    ui = (bi - d // 2) % d
    uj = (bj - d // 2) % d
    r = _window_offsets(d)
    rng = np.random.Generator(np.random.PCG64(w.poisson_seed))
    counts = np.empty((bi.size, n, n), dtype=np.uint32)
    x0 = np.arange(n)
    cols = (x0[:, None] + r[None, :]) % n                      # (N, D)
    for y0 in range(n):
        rows = (y0 + r) % n                                    # (D,)
        patch = t[rows][:, cols]                               # (D, N, D)
        exit_wave = probe[:, None, :] * patch                  # (D, N, D)
        det = np.fft.fft2(exit_wave, axes=(0, 2))              # unshifted detector
        inten = np.abs(det[ui, :, uj]) ** 2                    # (n_bf, N)
        draws = rng.poisson(w.dose * inten.T)                  # (N, n_bf), order x0 then BF
        counts[:, y0, :] = draws.T.astype(np.uint32)
    return counts


def make_counts_torch(w: Workload, device, rows_per_chunk: int = 16):
    """Same model on a torch device (complex64); returns an int32 tensor [n_bf][N][N].

    Counts are non-negative and far below 2^31, so the int32 tensor's bytes are the
    uint32 counts the library takes.
    """
    import torch

    g = w.geometry
    n, d = g.scan_n, g.det_n
    t = torch.from_numpy(np.exp(1j * w.object_strength * object_phase(w)).astype(np.complex64)).to(device)
    probe = torch.from_numpy(probe_window(w).astype(np.complex64)).to(device)
    bi, bj = bf_pixels(g)
    flat = torch.from_numpy(((bi - d // 2) % d) * d + ((bj - d // 2) % d)).to(device)
    r = torch.from_numpy(_window_offsets(d)).to(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.poisson_seed)
    counts = torch.empty((bi.size, n, n), dtype=torch.int32, device=device)
    x0 = torch.arange(n, device=device)
    cols = (x0[:, None] + r[None, :]) % n                      # (N, D)
    for y_start in range(0, n, rows_per_chunk):
        ys = torch.arange(y_start, min(n, y_start + rows_per_chunk), device=device)
        rows = (ys[:, None] + r[None, :]) % n                  # (Y, D)
        patch = t[rows[:, None, :, None], cols[None, :, None, :]]   # (Y, N, D, D)
        exit_wave = probe[None, None] * patch
        det = torch.fft.fft2(exit_wave)                        # (Y, N, D, D)
        inten = det.reshape(ys.numel(), n, d * d).abs().square().index_select(2, flat)  # (Y, N, n_bf)
        draws = torch.poisson(w.dose * inten.double(), generator=gen)
        counts[:, y_start:y_start + ys.numel(), :] = draws.permute(2, 0, 1).to(torch.int32)
        del patch, exit_wave, det, inten, draws
    return counts


def make_frames_numpy(w: Workload) -> np.ndarray:
    """uint32 detector frames [N^2][D^2]: frame y0 N + x0 is the whole D x D detector
    (fftshifted, row-major) at scan position (y0, x0); same forward model as the BF
    counts, Poisson draws over every detector pixel (rows y0, then x0, then pixel)."""
    g = w.geometry
    n, d = g.scan_n, g.det_n
    t = np.exp(1j * w.object_strength * object_phase(w))
    probe = probe_window(w)
    r = _window_offsets(d)
    rng = np.random.Generator(np.random.PCG64(w.poisson_seed))
    frames = np.empty((n * n, d * d), dtype=np.uint32)
    x0 = np.arange(n)
    cols = (x0[:, None] + r[None, :]) % n
    for y0 in range(n):
        rows = (y0 + r) % n
        patch = t[rows][:, cols]                               # (D, N, D)
        det = np.fft.fft2(probe[:, None, :] * patch, axes=(0, 2))
        inten = np.fft.fftshift(np.abs(det) ** 2, axes=(0, 2))  # detector order
        draws = rng.poisson(w.dose * inten.transpose(1, 0, 2).reshape(n, d * d))
        frames[y0 * n:(y0 + 1) * n] = draws.astype(np.uint32)
    return frames


def make_frames_torch(w: Workload, device, rows_per_chunk: int = 8):
    """The frames on a torch device (complex64 model, seeded torch generator); int32
    tensor [N^2][D^2] holding the uint32 counts."""
    import torch

    g = w.geometry
    n, d = g.scan_n, g.det_n
    t = torch.from_numpy(np.exp(1j * w.object_strength * object_phase(w)).astype(np.complex64)).to(device)
    probe = torch.from_numpy(probe_window(w).astype(np.complex64)).to(device)
    r = torch.from_numpy(_window_offsets(d)).to(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.poisson_seed)
    frames = torch.empty((n * n, d * d), dtype=torch.int32, device=device)
    x0 = torch.arange(n, device=device)
    cols = (x0[:, None] + r[None, :]) % n
    for y_start in range(0, n, rows_per_chunk):
        ys = torch.arange(y_start, min(n, y_start + rows_per_chunk), device=device)
        rows = (ys[:, None] + r[None, :]) % n
        patch = t[rows[:, None, :, None], cols[None, :, None, :]]   # (Y, N, D, D)
        det = torch.fft.fft2(probe[None, None] * patch)
        inten = torch.fft.fftshift(det.abs().square(), dim=(2, 3)).reshape(ys.numel() * n, d * d)
        draws = torch.poisson(w.dose * inten.double(), generator=gen)
        frames[y_start * n:(y_start + ys.numel()) * n] = draws.to(torch.int32)
        del patch, det, inten, draws
    return frames


def _cache_dir() -> str:
    return os.environ.get("SSB_SYNTH_CACHE", os.path.join("/tmp", "ssb_synth_cache"))


_GEN_VERSION = "v1"


def cached_counts(w: Workload) -> np.ndarray:
    """NumPy-back-end counts, cached on local disk keyed by workload and generator version."""
    key = hashlib.sha256(repr((w, _GEN_VERSION)).encode()).hexdigest()[:16]
    path = os.path.join(_cache_dir(), f"{w.name}_{key}.npy")
    if os.path.exists(path):
        try:
            arr = np.load(path, allow_pickle=False)
            if arr.shape == (w.n_bf, w.geometry.scan_n, w.geometry.scan_n) and arr.dtype == np.uint32:
                return arr
        except (OSError, ValueError):
            pass
    arr = make_counts_numpy(w)
    os.makedirs(_cache_dir(), exist_ok=True)
    tmp = f"{path}.{os.getpid()}.tmp.npy"
    np.save(tmp, arr)
    os.replace(tmp, path)
    return arr
