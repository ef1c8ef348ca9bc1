"""Float64 CPU oracle of the SSB phase-variance objective.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the test suite, the smoke check and the CPU-baseline leg of the
benchmark use it.  It shares no code with the GPU library.

It computes the objective by its plain definition, one bright-field (BF) pixel
at a time, with ordinary NumPy 2-D FFTs in float64 (no blocking, no fusion, no
half-plane tricks).  Sources are the quantem.gpu maintainer pages
"SSB performance notes" (cited below as *Notes*) and "Later SSB performance
checkpoints" (*Checkpoints*).  The pages describe the objective by its pieces
and properties but never print its formula; each step names the passage it
follows and, where the pages are silent, the reading taken.

Steps (theta = (C10 nm, C12 nm, phi12 rad) rounded to float32 at the boundary,
then promoted to float64; Notes, "MPS wider exact-simplex checkpoint": the
evaluator's inputs are float32 C10, C12, cos 2phi12, sin 2phi12):

O2  BF set: detector pixels with (i-cy)^2 + (j-cx)^2 <= R^2, row-major.
O3  G_b = rfft2 of the BF pixel's scan counts (forward sign, unnormalized,
    Hermitian half plane N x (N/2+1)); Notes, "Automatic whole-probe
    sparse-storage checkpoint" and the BF-major G_qk layout passage.
O4  DC = mean over BF of Re G_b(0,0) (a single scalar; Notes, the exact
    BF-companion "DC value" passage and the sparse-storage checkpoint).
O5  q(u, v) = s * (v, u_signed) detector pixels, u_signed = fftfreq index
    (u = N/2 maps to -N/2), v = rfftfreq index (v = N/2 is +N/2), rotated by rho.
O6  A(k) = a(k) exp(-i chi(k)), soft aperture a = clip((R_a - |k|)/w + 1/2, 0, 1),
    chi = pi lambda dk^2 [C10 |k|^2 + C12((kx^2 - ky^2) cos 2phi12 + 2 kx ky sin 2phi12)].
O7  Gamma(q) = conj(A(k)) A(k - q) - A(k) conj(A(k + q)) ("both shifted
    apertures", "two shifted-phase sincos", "gamma normalization": Notes, "MPS
    zero-transfer q-space checkpoint" and the v8 follow-ups); T = conj(Gamma)/|Gamma|,
    T = 0 where Gamma = 0 (zero transfer: exact complex zero).
O8  C_b = G_b T for q != 0; C_b(0, 0) = DC.
O9  Full plane by the anti-Hermitian relation C(-q) = -conj(C(q)) (Notes,
    sparse-storage checkpoint): columns v > N/2 are -conj(C(N-u, N-v)); columns
    v = 0 and v = N/2 are used as computed.
O10 O_b = ifft2(C_full) (two 512-point inverse transforms per BF: Checkpoints,
    "fftA intermediate and M5 hardware floor").
O11 phi_b = atan2(Im O_b, Re O_b).
O12 S1 = sum_b phi_b (per scan pixel), S2 = sum_b sum_px phi_b^2;
    L = S2/(n_bf N^2) - (1/N^2) sum_px (S1/n_bf)^2  (phase-sum image and
    squared-phase partials: Notes, "Pack-aware column dispatch" passage).
O13 Object: psi = ifft2(full plane of mean_b C_b), phase = angle(psi)
    ("phase-of-mean" output: Notes, "Standard-only CUDA native 512 calibration").

Full-plane variant (functions with ``full_plane`` in their names).  Notes,
"Automatic whole-probe sparse-storage checkpoint": the accepted evaluator
corrects every entry of the N x N plane on its own; building the columns past
N/2 from the anti-Hermitian relation (O9) moved the loss in the fourth digit,
mostly through the Nyquist column, which has no positive-frequency partner.
F5  q(u, v) = s * (v_signed, u_signed), fftfreq on both axes (v = N/2 -> -N/2).
F3  G_b = fft2 of the counts (the whole complex plane).
F8  C_b = G_b T on every entry, C_b(0, 0) = DC.
F10 O_b = ifft2(C_b); phase, moments, loss and object as in O11-O13.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class OGeom:
    """Geometry as plain numbers (same fields as the library's geometry struct)."""
    scan_n: int
    det_n: int
    bf_r2: float
    det_cy: float
    det_cx: float
    q_step_px: float
    dk: float
    wavelength_A: float
    alpha_rad: float
    rotation_rad: float
    edge_px: float

    @classmethod
    def from_any(cls, g) -> "OGeom":
        if isinstance(g, OGeom):
            return g
        if isinstance(g, dict):
            return cls(**{k: g[k] for k in cls.__dataclass_fields__})
        return cls(**{k: getattr(g, k) for k in cls.__dataclass_fields__})

    @property
    def aperture_px(self) -> float:
        return self.alpha_rad / self.wavelength_A / self.dk


def boundary_params(params3):
    """Float32 rounding at the boundary, then float64: (C10 A, C12 A, cos 2phi12, sin 2phi12).

    Notes, "MPS wider exact-simplex checkpoint": two distinct float64 simplex points
    with identical float32 C10, C12, cos 2phi12, sin 2phi12 are the same evaluation.
    """
    p = np.asarray(params3, dtype=np.float32).astype(np.float64)
    c10 = p[0] * 10.0
    c12 = p[1] * 10.0
    return c10, c12, math.cos(2.0 * p[2]), math.sin(2.0 * p[2])


# ---------------------------------------------------------------- O2: BF set
def bf_indices(g: OGeom):
    """Row-major detector (i, j) of the BF pixels: integer disk rule about (cy, cx)."""
    d = g.det_n
    out_i, out_j = [], []
    for i in range(d):
        for j in range(d):
            if (i - g.det_cy) ** 2 + (j - g.det_cx) ** 2 <= g.bf_r2:
                out_i.append(i)
                out_j.append(j)
    return np.array(out_i, dtype=np.int64), np.array(out_j, dtype=np.int64)


def bf_kvectors(g: OGeom):
    """BF detector offsets kappa_b in pixels as (kx, ky) = (j - cx, i - cy)."""
    i, j = bf_indices(g)
    return j - g.det_cx, i - g.det_cy


# ---------------------------------------------------------------- O3 / O4
def scan_spectrum(counts_b: np.ndarray) -> np.ndarray:
    """G_b: forward real 2-D DFT of one BF pixel's N x N scan counts, half plane (N, N/2+1)."""
    return np.fft.rfft2(np.asarray(counts_b, dtype=np.float64))


def dc_value(counts: np.ndarray) -> float:
    """Mean over BF of the scan sum Re G_b(0,0), from exact integer sums."""
    sums = np.asarray(counts).reshape(counts.shape[0], -1).astype(np.int64).sum(axis=1)
    return float(sums.sum()) / counts.shape[0]


# ---------------------------------------------------------------- O5
def q_vectors(g: OGeom):
    """Scan frequencies of the half plane in detector pixels, rotated: (qx, qy), each (N, N/2+1)."""
    n = g.scan_n
    fy = np.fft.fftfreq(n) * n          # signed row index, u = N/2 -> -N/2
    fx = np.fft.rfftfreq(n) * n         # column index 0..N/2, v = N/2 -> +N/2
    sx = g.q_step_px * fx[None, :] + 0.0 * fy[:, None]
    sy = g.q_step_px * fy[:, None] + 0.0 * fx[None, :]
    if g.rotation_rad == 0.0:
        return sx, sy
    c, s = math.cos(g.rotation_rad), math.sin(g.rotation_rad)
    return c * sx - s * sy, s * sx + c * sy


# ---------------------------------------------------------------- O6
def aperture(g: OGeom, kx, ky):
    """Soft aperture a(k) = clip((R_a - |k|)/w + 1/2, 0, 1) with k in detector pixels.

    The clip's flat regions are decided on the squared radius (a = 0 for
    |k|^2 >= (R_a + w/2)^2, a = 1 for |k|^2 <= (R_a - w/2)^2), which is the same
    function and keeps the support decision exact on dyadic pixel lattices.
    """
    ra, w = g.aperture_px, g.edge_px
    r2 = kx * kx + ky * ky
    a = np.clip((ra - np.sqrt(r2)) / w + 0.5, 0.0, 1.0)
    a = np.where(r2 >= (ra + 0.5 * w) ** 2, 0.0, a)
    if ra >= 0.5 * w:
        a = np.where(r2 <= (ra - 0.5 * w) ** 2, 1.0, a)
    return a


def chi(g: OGeom, params3, kx, ky):
    """Aberration phase chi(k) in radians for k in detector pixels (C10 defocus, C12 astigmatism)."""
    c10, c12, c2, s2 = boundary_params(params3)
    scale = math.pi * g.wavelength_A * g.dk * g.dk
    return scale * (c10 * (kx * kx + ky * ky) + c12 * ((kx * kx - ky * ky) * c2 + 2.0 * kx * ky * s2))


def probe(g: OGeom, params3, kx, ky):
    """A(k) = a(k) exp(-i chi(k))."""
    return aperture(g, kx, ky) * np.exp(-1j * chi(g, params3, kx, ky))


# ---------------------------------------------------------------- O7 / O8
def transfer(g: OGeom, params3, kbx: float, kby: float, qx=None, qy=None):
    """T(q) = conj(Gamma)/|Gamma|, 0 where Gamma = 0, for BF offset (kbx, kby)."""
    if qx is None:
        qx, qy = q_vectors(g)
    a0 = probe(g, params3, kbx, kby)
    am = probe(g, params3, kbx - qx, kby - qy)
    ap = probe(g, params3, kbx + qx, kby + qy)
    gamma = np.conj(a0) * am - a0 * np.conj(ap)
    mag = np.abs(gamma)
    t = np.zeros_like(gamma)
    nz = mag > 0.0
    # conj(Gamma)/|Gamma| as two real divisions (exact +-1 when Gamma is real)
    t.real[nz] = gamma.real[nz] / mag[nz]
    t.imag[nz] = -gamma.imag[nz] / mag[nz]
    return t


def corrected_spectrum(g_b: np.ndarray, t: np.ndarray, dc: float) -> np.ndarray:
    c = g_b * t
    c[0, 0] = dc
    return c


# ---------------------------------------------------------------- O9 - O11
def full_plane(c_half: np.ndarray) -> np.ndarray:
    """Extend the half plane (N, N/2+1) to (N, N) with C(u, v) = -conj(C(N-u, N-v)) for v > N/2."""
    n = c_half.shape[0]
    h = n // 2
    full = np.empty((n, n), dtype=np.complex128)
    full[:, : h + 1] = c_half
    u = np.arange(n)
    v = np.arange(h + 1, n)
    full[:, h + 1:] = -np.conj(c_half[((n - u) % n)[:, None], (n - v)[None, :]])
    return full


def bf_object(c_full: np.ndarray) -> np.ndarray:
    return np.fft.ifft2(c_full)


def bf_phase(obj: np.ndarray) -> np.ndarray:
    return np.arctan2(obj.imag, obj.real)


# ---------------------------------------------------------------- O12
def bf_moments(g, counts: np.ndarray, params3, dc: float, bf_list=None):
    """Phase-sum image S1 (N, N) and total squared phase S2 over the listed BF pixels.

    counts[k] must hold the scan counts of BF index bf_list[k] (or of every BF in
    order when bf_list is None).  Each BF is corrected, extended, inverse-transformed
    and reduced on its own, in increasing BF order.
    """
    g = OGeom.from_any(g)
    kx_all, ky_all = bf_kvectors(g)
    if bf_list is None:
        bf_list = np.arange(kx_all.size)
    qx, qy = q_vectors(g)
    n = g.scan_n
    s1 = np.zeros((n, n), dtype=np.float64)
    s2 = 0.0
    for k, b in enumerate(bf_list):
        t = transfer(g, params3, kx_all[b], ky_all[b], qx, qy)
        c = corrected_spectrum(scan_spectrum(counts[k]), t, dc)
        phi = bf_phase(bf_object(full_plane(c)))
        s1 += phi
        s2 += float(np.sum(phi * phi))
    return s1, s2


def loss_from_moments(s1: np.ndarray, s2: float, n_bf: int) -> float:
    n2 = s1.size
    mean = s1 / n_bf
    return s2 / (n_bf * n2) - float(np.sum(mean * mean)) / n2


def loss(g, counts: np.ndarray, params3, dc: float | None = None) -> float:
    """Phase-variance loss over all BF pixels (population variance, averaged over scan pixels)."""
    if dc is None:
        dc = dc_value(counts)
    s1, s2 = bf_moments(g, counts, params3, dc)
    return loss_from_moments(s1, s2, counts.shape[0])


def mean_phase(g, counts, params3, dc=None):
    if dc is None:
        dc = dc_value(counts)
    s1, _ = bf_moments(g, counts, params3, dc)
    return s1 / counts.shape[0]


# ---------------------------------------------------------------- O13
def corrected_sum(g, counts: np.ndarray, params3, dc: float, bf_list=None) -> np.ndarray:
    """Sum of the corrected half planes C_b over the listed BF pixels, in increasing BF
    order (counts[k] holds BF bf_list[k], or every BF in order when bf_list is None)."""
    g = OGeom.from_any(g)
    kx_all, ky_all = bf_kvectors(g)
    if bf_list is None:
        bf_list = np.arange(kx_all.size)
    qx, qy = q_vectors(g)
    acc = np.zeros((g.scan_n, g.scan_n // 2 + 1), dtype=np.complex128)
    for k, b in enumerate(bf_list):
        t = transfer(g, params3, kx_all[b], ky_all[b], qx, qy)
        acc += corrected_spectrum(scan_spectrum(counts[k]), t, dc)
    return acc


def object_from_sum(acc: np.ndarray, n_bf: int):
    """Phase-of-mean object from the BF sum of corrected half planes: (phase, psi)."""
    psi = bf_object(full_plane(acc / n_bf))
    return bf_phase(psi), psi


def object_wave(g, counts: np.ndarray, params3, dc: float | None = None):
    """Phase-of-mean object: psi = ifft2(extension of mean_b C_b); returns (phase, psi)."""
    if dc is None:
        dc = dc_value(counts)
    return object_from_sum(corrected_sum(g, counts, params3, dc), counts.shape[0])


# ---------------------------------------------------------------- full-plane variant
def q_vectors_full(g: OGeom):
    """Scan frequencies of the full plane in detector pixels, rotated: (qx, qy), each (N, N).
    Both axes signed as fftfreq, so u = N/2 and v = N/2 both map to -N/2."""
    n = g.scan_n
    f = np.fft.fftfreq(n) * n
    sx = g.q_step_px * f[None, :] + 0.0 * f[:, None]
    sy = g.q_step_px * f[:, None] + 0.0 * f[None, :]
    if g.rotation_rad == 0.0:
        return sx, sy
    c, s = math.cos(g.rotation_rad), math.sin(g.rotation_rad)
    return c * sx - s * sy, s * sx + c * sy


def scan_spectrum_full(counts_b: np.ndarray) -> np.ndarray:
    """Forward complex 2-D DFT of one BF pixel's scan counts, the whole (N, N) plane."""
    return np.fft.fft2(np.asarray(counts_b, dtype=np.float64))


def corrected_full_plane(g: OGeom, counts_b, params3, kbx, kby, dc, qx=None, qy=None):
    """C_b on every entry of the full plane (each corrected on its own), DC at q = 0."""
    if qx is None:
        qx, qy = q_vectors_full(g)
    c = scan_spectrum_full(counts_b) * transfer(g, params3, kbx, kby, qx, qy)
    c[0, 0] = dc
    return c


def bf_moments_full_plane(g, counts: np.ndarray, params3, dc: float, bf_list=None):
    """S1 (N, N) and S2 of the full-plane variant over the listed BF pixels (as bf_moments)."""
    g = OGeom.from_any(g)
    kx_all, ky_all = bf_kvectors(g)
    if bf_list is None:
        bf_list = np.arange(kx_all.size)
    qx, qy = q_vectors_full(g)
    n = g.scan_n
    s1 = np.zeros((n, n), dtype=np.float64)
    s2 = 0.0
    for k, b in enumerate(bf_list):
        c = corrected_full_plane(g, counts[k], params3, kx_all[b], ky_all[b], dc, qx, qy)
        phi = bf_phase(bf_object(c))
        s1 += phi
        s2 += float(np.sum(phi * phi))
    return s1, s2


def loss_full_plane(g, counts: np.ndarray, params3, dc: float | None = None) -> float:
    if dc is None:
        dc = dc_value(counts)
    s1, s2 = bf_moments_full_plane(g, counts, params3, dc)
    return loss_from_moments(s1, s2, counts.shape[0])


def object_wave_full_plane(g, counts: np.ndarray, params3, dc: float | None = None):
    """Phase-of-mean object of the full-plane variant: psi = ifft2(mean_b C_b); (phase, psi)."""
    g = OGeom.from_any(g)
    if dc is None:
        dc = dc_value(counts)
    kx_all, ky_all = bf_kvectors(g)
    qx, qy = q_vectors_full(g)
    acc = np.zeros((g.scan_n, g.scan_n), dtype=np.complex128)
    for b in range(counts.shape[0]):
        acc += corrected_full_plane(g, counts[b], params3, kx_all[b], ky_all[b], dc, qx, qy)
    psi = bf_object(acc / counts.shape[0])
    return bf_phase(psi), psi
