"""GPU parity: the HIP library through its C ABI against the float64 oracle.

Tolerances: loss within 1e-5 relative, object phase within 1e-4 rad RMS, BF
selection and spectrum indexing bit-exact (the targets stated for this path);
cached spectra within 2e-6 relative L2 per BF (float32 FFT of a 2-D plane).
"""
import dataclasses
import math
import os
import sys

import numpy as np
import pytest

import aberration_phase_variance_amd as ssb
from oracle import ssb_oracle as O
from synth import WORKLOADS, Workload, cached_counts, make_geometry, trial_params

pytestmark = pytest.mark.gpu

LOSS_RTOL = 1e-5
PHASE_RMS = 1e-4
SPEC_RTOL = 2e-6


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return torch


def _say(msg):
    print(msg, file=sys.stderr, flush=True)

def _check_range(s1, s2, r1, r2, n, what):
    """Moments of a BF range against the oracle's: S2 and the range's own loss (the formula
    applied to each side's moments) within LOSS_RTOL, and no pixel of S1 off by more than
    1e-4 sqrt(n) rad (a phase that crosses the branch cut at +-pi, an error of 2 pi, fails)."""
    d = s1 - r1
    lg, lr = O.loss_from_moments(s1, s2, n), O.loss_from_moments(r1, r2, n)
    rms, mx = float(np.sqrt(np.mean(d * d))), float(np.max(np.abs(d)))
    _say(f"{what}: S1 error rms {rms:.2e} max {mx:.2e}; loss rel error {abs(lg - lr) / abs(lr):.2e}")
    assert abs(s2 - r2) <= LOSS_RTOL * abs(r2), what
    assert abs(lg - lr) <= LOSS_RTOL * abs(lr), what
    assert mx <= 1e-4 * n ** 0.5, what



class Prepared:
    def __init__(self, geometry, counts_np=None, counts_dev=None):
        torch = _torch()
        self.torch = torch
        self.g = geometry
        if counts_dev is None:
            counts_dev = torch.from_numpy(np.ascontiguousarray(counts_np).view(np.int32)).cuda()
        self.n_bf = counts_dev.shape[0]
        self.h = ssb.ssb_prepare(geometry, counts_dev, self.n_bf)
        torch.cuda.synchronize()
        self.n = geometry.scan_n

    def loss(self, params, mean_phase=None):
        return ssb.ssb_loss(self.h, params, mean_phase)

    def obj(self, params, with_psi=True):
        t = self.torch
        phase = t.full((self.n, self.n), float("nan"), dtype=t.float32, device="cuda")
        psi = t.full((self.n, self.n, 2), float("nan"), dtype=t.float32, device="cuda") if with_psi else None
        ssb.ssb_object(self.h, params, phase, psi)
        t.cuda.synchronize()
        out_psi = None
        if psi is not None:
            p = psi.cpu().numpy()
            out_psi = p[..., 0] + 1j * p[..., 1]
        return phase.cpu().numpy(), out_psi

    def loss_obj(self, params, with_psi=True):
        """ssb_loss_object on NaN-filled outputs: (loss, phase, psi or None)."""
        t = self.torch
        phase = t.full((self.n, self.n), float("nan"), dtype=t.float32, device="cuda")
        psi = t.full((self.n, self.n, 2), float("nan"), dtype=t.float32, device="cuda") if with_psi else None
        loss = ssb.ssb_loss_object(self.h, params, phase, psi)
        out_psi = None
        if psi is not None:
            q = psi.cpu().numpy()
            out_psi = q[..., 0] + 1j * q[..., 1]
        return loss, phase.cpu().numpy(), out_psi

    def moments(self, params, b0, b1):
        t = self.torch
        s1 = t.full((self.n, self.n), float("nan"), dtype=t.float64, device="cuda")
        s2 = ssb.ssb_moments(self.h, params, b0, b1, s1)
        return s1.cpu().numpy(), s2

    def spectrum(self, b):
        t = self.torch
        out = t.full((self.n, self.n // 2 + 1, 2), float("nan"), dtype=t.float32, device="cuda")
        ssb.ssb_spectrum(self.h, b, out)
        t.cuda.synchronize()
        o = out.cpu().numpy()
        return o[..., 0] + 1j * o[..., 1]

    def release(self):
        ssb.ssb_release(self.h)
        self.h = None


@pytest.fixture(scope="module")
def tiny():
    w = WORKLOADS["tiny"]
    counts = cached_counts(w)
    p = Prepared(w.geometry, counts)
    yield w, counts, p
    p.release()


@pytest.fixture(scope="module")
def small():
    w = WORKLOADS["small"]
    counts = cached_counts(w)
    p = Prepared(w.geometry, counts)
    yield w, counts, p
    p.release()


def _rel(a, b):
    return abs(a - b) / abs(b)


# ---------------------------------------------------------------- prepare / spectra
@pytest.mark.parametrize("fx", ["tiny", "small"])
def test_prepare_info_exact(fx, request):
    w, counts, p = request.getfixturevalue(fx)
    info = ssb.ssb_query(p.h)
    g = O.OGeom.from_any(w.geometry)
    kx, ky = O.bf_kvectors(g)
    assert info["n_bf"] == w.n_bf == kx.size
    assert info["n_active_bf"] == int(np.count_nonzero(O.aperture(g, kx, ky) > 0))
    assert info["dc"] == O.dc_value(counts)          # exact integer mean
    assert info["spectrum_bytes"] == w.n_bf * g.scan_n * (g.scan_n // 2 + 1) * 8


def _oracle_support_counts(g, kx, ky):
    """Nonzero-transfer entries (q = 0 aside) and 1 + last nonzero column, per BF, from
    the oracle's aperture: the transfer is zero exactly where both shifted apertures are."""
    qx, qy = O.q_vectors(g)
    nsup, vend = [], []
    for b in range(kx.size):
        on = (O.aperture(g, kx[b] - qx, ky[b] - qy) > 0) | (O.aperture(g, kx[b] + qx, ky[b] + qy) > 0)
        on[0, 0] = False
        cols = np.flatnonzero(on.any(axis=0))
        nsup.append(int(np.count_nonzero(on)))
        vend.append(int(cols[-1]) + 1 if cols.size else 1)
    return np.array(nsup), np.array(vend)


@pytest.mark.parametrize("fx", ["tiny", "small"])
def test_support_tables_exact(fx, request):
    """The library's per-column support intervals select exactly the oracle's
    nonzero-transfer entries (counted) and its nonzero columns (rho = 0: exact lattice)."""
    w, counts, p = request.getfixturevalue(fx)
    g = O.OGeom.from_any(w.geometry)
    kx, ky = O.bf_kvectors(g)
    nsup, vend = _oracle_support_counts(g, kx, ky)
    info = ssb.ssb_query(p.h)
    h = g.scan_n // 2
    assert info["support_entries"] == int(nsup.sum())
    assert info["columns_read"] == int(np.minimum(vend, h).sum() + np.count_nonzero(vend > h))


@pytest.mark.parametrize("fx", ["tiny", "small"])
def test_spectrum_vs_oracle(fx, request):
    w, counts, p = request.getfixturevalue(fx)
    for b in sorted({0, 1, w.n_bf // 2, w.n_bf - 1}):
        ref = O.scan_spectrum(counts[b])
        got = p.spectrum(b)
        assert np.linalg.norm(got - ref) <= SPEC_RTOL * np.linalg.norm(ref), b


def test_spectrum_indexing_bit_exact():
    """Constant planes c_b = 1 + 3b: every cached spectrum is exactly (c_b N^2 at DC, 0 elsewhere)."""
    w = WORKLOADS["small"]
    n = w.geometry.scan_n
    c = (1 + 3 * np.arange(w.n_bf, dtype=np.uint32))[:, None, None] * np.ones((1, n, n), np.uint32)
    p = Prepared(w.geometry, c)
    try:
        for b in (0, 5, 160, w.n_bf - 1):
            got = p.spectrum(b)
            exp = np.zeros_like(got)
            exp[0, 0] = float((1 + 3 * b) * n * n)
            assert np.array_equal(got, exp), b
        assert ssb.ssb_query(p.h)["dc"] == float(np.mean((1 + 3 * np.arange(w.n_bf)) * n * n))
        # vacuum-like planes: every BF phase is 0, so every loss is exactly 0
        assert np.all(p.loss([[40.0, 5.0, 0.3], [-90.0, 12.0, 2.0]]) == 0.0)
    finally:
        p.release()


# ---------------------------------------------------------------- loss
def test_loss_tiny(tiny):
    w, counts, p = tiny
    g = O.OGeom.from_any(w.geometry)
    params = np.array([[40.0, 5.0, 0.3], [0.0, 0.0, 0.0], [-73.5, 14.0, 0.47], [120.0, -8.0, 2.9]], np.float32)
    got = p.loss(params)
    for k in range(len(params)):
        ref = O.loss(g, counts, params[k])
        assert _rel(got[k], ref) <= LOSS_RTOL, (k, got[k], ref)


def test_loss_small_batch(small):
    w, counts, p = small
    g = O.OGeom.from_any(w.geometry)
    dc = O.dc_value(counts)
    params = trial_params(w, 12)
    got = p.loss(params)
    for k in range(len(params)):
        ref = O.loss(g, counts, params[k], dc)
        assert _rel(got[k], ref) <= LOSS_RTOL, (k, got[k], ref)


def test_loss_small_200_trial_batch(small):
    """The small workload's whole 200-trial batch in one call, every trial against the
    oracle (run over BF ranges in a process pool), and two of them again as single-trial
    calls."""
    from oracle.pool import OraclePool
    w, counts, p = small
    g = O.OGeom.from_any(w.geometry)
    dc = O.dc_value(counts)
    params = trial_params(w)
    assert params.shape == (200, 3)
    got = p.loss(params)
    worst = 0.0
    with OraclePool(counts) as pool:
        for k in range(200):
            ref = pool.loss(g, params[k], dc)
            worst = max(worst, _rel(got[k], ref))
            assert _rel(got[k], ref) <= LOSS_RTOL, (k, got[k], ref)
    _say(f"[small] 200 trials: largest relative loss difference {worst:.2e}")
    for k in (3, 199):
        assert p.loss(params[k:k + 1])[0] == got[k]


def test_mean_phase_small(small):
    w, counts, p = small
    t = _torch()
    g = O.OGeom.from_any(w.geometry)
    mp = t.full((128, 128), float("nan"), dtype=t.float32, device="cuda")
    p.loss([[40.0, 5.0, 0.3]], mp)
    ref = O.mean_phase(g, counts, (40.0, 5.0, 0.3))
    d = mp.cpu().numpy() - ref
    assert np.sqrt(np.mean(d * d)) < 1e-5 and np.max(np.abs(d)) < 1e-4


def test_batch_chunk_and_repeat_invariance(small):
    """Per-trial losses are bitwise independent of batch size, batch position, chunking and repetition."""
    w, counts, p = small
    a = np.array([[37.0, 4.0, 0.25]], np.float32)
    others = trial_params(w, 6)
    single = p.loss(a)[0]
    batch = p.loss(np.concatenate([a, others[:2], a, others[2:]]))
    assert batch[0] == single and batch[3] == single
    assert np.array_equal(p.loss(others), batch[[1, 2, 4, 5, 6, 7]])
    ssb.ssb_set_chunk(p.h, 32)
    try:
        assert p.loss(a)[0] == single
        assert np.array_equal(p.loss(others), batch[[1, 2, 4, 5, 6, 7]])
    finally:
        ssb.ssb_set_chunk(p.h, 0)
    assert p.loss(a)[0] == single


def test_reserved_batch_allocates_nothing(small):
    """After ssb_reserve(64), loss calls of up to 64 trials, moments and the object leave the
    handle's workspace as it was (no allocation in the call), and reserve only grows."""
    w, counts, p = small
    assert ssb.ssb_query(p.h)["reserved_trials"] >= 1
    ssb.ssb_reserve(p.h, 64)
    before = ssb.ssb_query(p.h)
    assert before["reserved_trials"] == 64 and before["workspace_bytes"] > 0
    full = p.loss(trial_params(w, 64))
    part = p.loss(trial_params(w, 17))
    assert np.array_equal(part, full[:17])
    p.moments([40.0, 5.0, 0.3], 3, 100)
    p.obj([40.0, 5.0, 0.3])
    ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_FULL_PLANE)
    try:
        p.loss(trial_params(w, 64))
        p.obj([40.0, 5.0, 0.3])
    finally:
        ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_HALF_PLANE)
    ssb.ssb_set_chunk(p.h, 32)
    try:
        p.loss(trial_params(w, 64))
    finally:
        ssb.ssb_set_chunk(p.h, 0)
    ssb.ssb_reserve(p.h, 8)                          # a smaller request keeps the larger reservation
    after = ssb.ssb_query(p.h)
    assert after["workspace_bytes"] == before["workspace_bytes"]
    assert after["reserved_trials"] == 64
    with pytest.raises(ssb.SSBError):
        ssb.ssb_reserve(p.h, 0)


def test_moments_range_small(small):
    w, counts, p = small
    g = O.OGeom.from_any(w.geometry)
    dc = O.dc_value(counts)
    b0, b1 = 37, 131                                  # not aligned to the 32-BF groups
    s1, s2 = p.moments([40.0, 5.0, 0.3], b0, b1)
    r1, r2 = O.bf_moments(g, counts[b0:b1], (40.0, 5.0, 0.3), dc, list(range(b0, b1)))
    assert _rel(s2, r2) <= LOSS_RTOL
    assert np.max(np.abs(s1 - r1)) <= 1e-4 * (b1 - b0) ** 0.5


# ---------------------------------------------------------------- object
@pytest.mark.parametrize("fx", ["tiny", "small"])
def test_object_vs_oracle(fx, request):
    w, counts, p = request.getfixturevalue(fx)
    g = O.OGeom.from_any(w.geometry)
    for params in ([40.0, 5.0, 0.3], [-55.0, 9.0, 1.9]):
        phase, psi = p.obj(params)
        ref_phase, ref_psi = O.object_wave(g, counts, params)
        d = np.angle(np.exp(1j * (phase - ref_phase)))
        assert np.sqrt(np.mean(d * d)) <= PHASE_RMS
        assert np.linalg.norm(psi - ref_psi) <= 1e-5 * np.linalg.norm(ref_psi)


def _wrapped(a, b):
    return np.angle(np.exp(1j * (a - b)))


def check_loss_object(p, params, ref_phase=None, ref_psi=None, what=""):
    """ssb_loss_object against ssb_loss (bitwise), ssb_object (float rounding: at most
    1e-5 rad, psi within 1e-6 relative L2) and, when given, the oracle's object."""
    loss, phase, psi = p.loss_obj(params)
    assert loss == p.loss([params])[0], what
    ph2, psi2 = p.obj(params)
    d = _wrapped(phase, ph2)
    _say(f"[loss+object] {what} {params}: phase vs ssb_object max {np.max(np.abs(d)):.2e} rad")
    assert np.max(np.abs(d)) <= 1e-5, what
    assert np.linalg.norm(psi - psi2) <= 1e-6 * np.linalg.norm(psi2), what
    if ref_phase is not None:
        assert np.sqrt(np.mean(_wrapped(phase, ref_phase) ** 2)) <= PHASE_RMS, what
    if ref_psi is not None:
        assert np.linalg.norm(psi - ref_psi) <= 1e-5 * np.linalg.norm(ref_psi), what


@pytest.mark.parametrize("fx", ["tiny", "small"])
def test_loss_object_vs_oracle(fx, request):
    """The fused call: the loss of ssb_loss and the object of ssb_object from one pass."""
    w, counts, p = request.getfixturevalue(fx)
    g = O.OGeom.from_any(w.geometry)
    for params in ([40.0, 5.0, 0.3], [-55.0, 9.0, 1.9], [0.0, 0.0, 0.0]):
        ref_phase, ref_psi = O.object_wave(g, counts, params)
        check_loss_object(p, params, ref_phase, ref_psi, fx)
        assert _rel(p.loss_obj(params, with_psi=False)[0], O.loss(g, counts, params)) <= LOSS_RTOL


def test_loss_object_allocates_nothing_after_prepare():
    """ssb_prepare reserves what ssb_loss_object needs, in both variants: the call leaves the
    handle's workspace as it was."""
    w = WORKLOADS["tiny"]
    counts = cached_counts(w)
    p = Prepared(w.geometry, counts)
    try:
        before = ssb.ssb_query(p.h)["workspace_bytes"]
        p.loss_obj([40.0, 5.0, 0.3])
        ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_FULL_PLANE)
        p.loss_obj([40.0, 5.0, 0.3])
        assert ssb.ssb_query(p.h)["workspace_bytes"] == before
    finally:
        p.release()


def test_loss_object_chunked(small):
    """Chunks smaller than the BF set: the object sums carry over from chunk to chunk."""
    w, counts, p = small
    g = O.OGeom.from_any(w.geometry)
    params = [-30.0, 6.0, 0.7]
    ref_phase, ref_psi = O.object_wave(g, counts, params)
    ssb.ssb_set_chunk(p.h, 64)
    try:
        check_loss_object(p, params, ref_phase, ref_psi, "small, 64-BF chunks")
    finally:
        ssb.ssb_set_chunk(p.h, 0)


# ---------------------------------------------------------------- edge cases
@pytest.mark.parametrize("fx", ["tiny", "small"])
def test_zero_aberration(fx, request):
    """theta = 0: chi vanishes, so sin chi_q is exactly 0 and every entry with both
    sidebands on their flat tops has zero transfer; one-sideband entries keep T = +-1."""
    w, counts, p = request.getfixturevalue(fx)
    g = O.OGeom.from_any(w.geometry)
    zero = [0.0, 0.0, 0.0]
    assert _rel(p.loss([zero])[0], O.loss(g, counts, zero)) <= LOSS_RTOL
    r1, r2 = O.bf_moments(g, counts, zero, O.dc_value(counts))
    s1, s2 = p.moments(zero, 0, w.n_bf)
    assert _rel(s2, r2) <= LOSS_RTOL
    _check_range(s1, s2, r1, r2, w.n_bf, f"[parity] {fx} zero aberration")
    phase, _ = p.obj(zero, with_psi=False)
    ref, _ = O.object_wave(g, counts, zero)
    assert np.sqrt(np.mean(np.angle(np.exp(1j * (phase - ref))) ** 2)) <= PHASE_RMS


@pytest.mark.parametrize("params", [[40.0, 5.0, 0.3], [-75.0, 12.0, 2.2]])
def test_vacuum_counts(params):
    """Constant counts: every scan spectrum is zero away from q = 0, so every phase and
    the loss are zero for any aberrations (the oracle gives exactly 0)."""
    w = WORKLOADS["small"]
    counts = np.full((w.n_bf, 128, 128), 200, dtype=np.uint32)
    p = Prepared(w.geometry, counts)
    try:
        # float transforms of a constant plane cancel to zero up to roundoff
        assert abs(p.loss([params])[0]) <= 1e-18
        s1, s2 = p.moments(params, 0, w.n_bf)
        assert s2 <= 1e-12 and np.max(np.abs(s1)) <= 1e-6
        phase, _ = p.obj(params, with_psi=False)
        assert np.max(np.abs(phase)) <= 1e-6
    finally:
        p.release()


def test_fit_small(small):
    """Batch + refinement through ssb_fit: the batch's best trial is the oracle's, the
    refinement's first evaluation repeats it bitwise, sampled refinement points match
    the oracle, and the returned loss is the lowest evaluated."""
    w, counts, p = small
    g = O.OGeom.from_any(w.geometry)
    dc = O.dc_value(counts)
    trials = trial_params(w, 16)
    _say("[fit] ssb_fit small, 16 trials + refinement capped at 24 evaluations")
    r = ssb.ssb_fit(p.h, trials, {"max_evals": 24})
    ref = np.array([O.loss(g, counts, t, dc) for t in trials])
    assert r["batch_best"] == int(np.argmin(ref))
    assert _rel(r["batch_loss"], ref.min()) <= LOSS_RTOL
    t = r["trace"]
    assert r["evals"] == t.shape[0] and 4 < r["evals"] <= 24 and r["requests"] >= r["evals"]
    np.testing.assert_array_equal(t[0, :3], trials[r["batch_best"]])
    assert t[0, 3] == r["batch_loss"]                  # single-trial call = batch call, bitwise
    assert r["loss"] == t[:, 3].min()
    for i in sorted({1, int(np.argmin(t[:, 3])), t.shape[0] - 1}):
        assert _rel(t[i, 3], O.loss(g, counts, t[i, :3].astype(np.float32), dc)) <= LOSS_RTOL, i


def test_inactive_bf_pixels():
    """Probe aperture smaller than the BF disk: zero-aperture BF keep phase 0 but count in n_bf."""
    w = WORKLOADS["tiny"]
    counts = cached_counts(w)
    g0 = w.geometry
    geom = dataclasses.replace(g0, alpha_rad=g0.alpha_rad * 2.5 / g0.aperture_px)
    p = Prepared(geom, counts)
    try:
        og = O.OGeom.from_any(geom)
        kx, ky = O.bf_kvectors(og)
        n_act = int(np.count_nonzero(O.aperture(og, kx, ky) > 0))
        assert 0 < n_act < w.n_bf
        assert ssb.ssb_query(p.h)["n_active_bf"] == n_act
        for params in ([40.0, 5.0, 0.3], [10.0, -3.0, 1.0]):
            assert _rel(p.loss([params])[0], O.loss(og, counts, params)) <= LOSS_RTOL
            phase, _ = p.obj(params, with_psi=False)
            ref, ref_psi = O.object_wave(og, counts, params)
            assert np.sqrt(np.mean(np.angle(np.exp(1j * (phase - ref))) ** 2)) <= PHASE_RMS
            # the fused call adds the inactive pixels' DC terms itself
            check_loss_object(p, params, ref, ref_psi, "inactive BF pixels")
    finally:
        p.release()


def test_rotation():
    """Rotated scan.  The edge width is 0.9 px: with 1 px the center BF pixel's |k -+ q| = |q|
    (rotation-invariant) lands exactly on the aperture edge 10.5 px for some lattice q, a tie
    that rounding of the rotation breaks either way."""
    w = WORKLOADS["small"]
    counts = cached_counts(w)
    geom = dataclasses.replace(w.geometry, rotation_rad=0.3, edge_px=0.9)
    og = O.OGeom.from_any(geom)
    # no half-plane entry may sit within rounding of an aperture edge for this rotation
    kx, ky = O.bf_kvectors(og)
    qx, qy = O.q_vectors(og)
    hi2 = (og.aperture_px + 0.5 * og.edge_px) ** 2
    for s in (-1.0, 1.0):
        r2 = (kx[:, None, None] + s * qx[None]) ** 2 + (ky[:, None, None] + s * qy[None]) ** 2
        assert np.min(np.abs(r2 - hi2)) > 1e-9 * hi2
    p = Prepared(geom, counts)
    try:
        for params in ([40.0, 5.0, 0.3], [-20.0, 15.0, 0.8]):
            assert _rel(p.loss([params])[0], O.loss(og, counts, params)) <= LOSS_RTOL
    finally:
        p.release()


def _custom_workload(n, d, r2):
    base = WORKLOADS["tiny"]
    g = make_geometry(n, d, r2)
    i = np.arange(d)[:, None] - d / 2
    j = np.arange(d)[None, :] - d / 2
    nbf = int(np.count_nonzero(i * i + j * j <= r2))
    return dataclasses.replace(base, name=f"n{n}", geometry=g, n_bf=nbf)


@pytest.mark.parametrize("n,d,r2", [(64, 24, 20), (256, 40, 36)])
def test_other_scan_sizes(n, d, r2):
    w = _custom_workload(n, d, r2)
    counts = cached_counts(w)
    og = O.OGeom.from_any(w.geometry)
    p = Prepared(w.geometry, counts)
    try:
        for params in ([40.0, 5.0, 0.3], [-25.0, 7.0, 2.4]):
            assert _rel(p.loss([params])[0], O.loss(og, counts, params)) <= LOSS_RTOL
        phase, _ = p.obj([40.0, 5.0, 0.3], with_psi=False)
        ref, ref_psi = O.object_wave(og, counts, [40.0, 5.0, 0.3])
        assert np.sqrt(np.mean(np.angle(np.exp(1j * (phase - ref))) ** 2)) <= PHASE_RMS
        check_loss_object(p, [40.0, 5.0, 0.3], ref, ref_psi, f"N = {n}")
    finally:
        p.release()


def test_error_paths_on_device(small):
    w, counts, p = small
    t = _torch()
    with pytest.raises(ssb.SSBError) as ei:
        p.loss([[float("nan"), 1.0, 0.0]])
    assert ei.value.code == ssb._ssb.SSB_EINVAL
    with pytest.raises(ssb.SSBError) as ei:          # an empty batch
        p.loss(np.zeros((0, 3), np.float32))
    assert ei.value.code == ssb._ssb.SSB_EINVAL
    # the handle still works after the errors
    assert _rel(p.loss([[40.0, 5.0, 0.3]])[0], O.loss(O.OGeom.from_any(w.geometry), counts, (40.0, 5.0, 0.3))) <= LOSS_RTOL
    s1 = t.full((128, 128), float("nan"), dtype=t.float64, device="cuda")
    for b0, b1 in ((-1, 5), (10, 10), (0, w.n_bf + 1)):
        with pytest.raises(ssb.SSBError) as ei:
            ssb.ssb_moments(p.h, [40.0, 5.0, 0.3], b0, b1, s1)
        assert ei.value.code == ssb._ssb.SSB_ESHAPE
    spec = t.full((128, 65, 2), float("nan"), dtype=t.float32, device="cuda")
    with pytest.raises(ssb.SSBError) as ei:
        ssb.ssb_spectrum(p.h, w.n_bf, spec)
    assert ei.value.code == ssb._ssb.SSB_ESHAPE
    # the binding checks tensors before the call: dtype, size, contiguity
    with pytest.raises(ValueError):
        ssb.ssb_moments(p.h, [40.0, 5.0, 0.3], 0, 5, spec)
    with pytest.raises(ValueError):
        ssb.ssb_moments(p.h, [40.0, 5.0, 0.3], 0, 5, s1[:64])
    with pytest.raises(ValueError):
        ssb.ssb_object(p.h, [40.0, 5.0, 0.3], t.full((128, 128), 0.0, dtype=t.float32, device="cuda").t())
    ph = t.full((128, 128), float("nan"), dtype=t.float32, device="cuda")
    with pytest.raises(ssb.SSBError) as ei:
        ssb.ssb_loss_object(p.h, [float("inf"), 5.0, 0.3], ph)
    assert ei.value.code == ssb._ssb.SSB_EINVAL
    assert bool(t.isnan(ph).all())                    # nothing written on the error
    with pytest.raises(ValueError):
        ssb.ssb_loss_object(p.h, [40.0, 5.0, 0.3], ph[:64])
    dev = t.zeros((w.n_bf - 1, 128, 128), dtype=t.int32, device="cuda")
    with pytest.raises(ssb.SSBError) as ei:
        ssb.ssb_prepare(w.geometry, dev, w.n_bf - 1)
    assert ei.value.code == ssb._ssb.SSB_ESHAPE


# ---------------------------------------------------------------- full-plane variant
@pytest.fixture
def full_plane_tiny(tiny):
    w, counts, p = tiny
    ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_FULL_PLANE)
    yield w, counts, p
    ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_HALF_PLANE)


def test_full_plane_loss_tiny(full_plane_tiny):
    w, counts, p = full_plane_tiny
    g = O.OGeom.from_any(w.geometry)
    assert ssb.ssb_query(p.h)["variant"] == 1
    params = np.array([[40.0, 5.0, 0.3], [0.0, 0.0, 0.0], [-73.5, 14.0, 0.47], [120.0, -8.0, 2.9]], np.float32)
    got = p.loss(params)
    for k in range(len(params)):
        ref = O.loss_full_plane(g, counts, params[k])
        half = O.loss(g, counts, params[k])
        assert _rel(got[k], ref) <= LOSS_RTOL, (k, got[k], ref)
        # the two variants differ here by more than the tolerance for some trial
        if k == 0:
            assert abs(ref - half) > 0.0
    # single-trial calls repeat the batch bitwise
    assert p.loss(params[2:3])[0] == got[2]


def test_full_plane_differs_where_pages_say(full_plane_tiny):
    """Switching the variant changes only the Nyquist-line terms: with the half plane
    restored, the library returns its half-plane losses again, bitwise."""
    w, counts, p = full_plane_tiny
    params = [[-73.5, 14.0, 0.47]]
    fp = p.loss(params)[0]
    ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_HALF_PLANE)
    hp1 = p.loss(params)[0]
    ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_FULL_PLANE)
    assert p.loss(params)[0] == fp
    ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_HALF_PLANE)
    assert p.loss(params)[0] == hp1
    g = O.OGeom.from_any(w.geometry)
    assert _rel(hp1, O.loss(g, counts, params[0])) <= LOSS_RTOL
    ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_FULL_PLANE)


def test_full_plane_moments_and_object_tiny(full_plane_tiny):
    w, counts, p = full_plane_tiny
    g = O.OGeom.from_any(w.geometry)
    dc = O.dc_value(counts)
    for params in ([40.0, 5.0, 0.3], [-55.0, 9.0, 1.9]):
        s1, s2 = p.moments(params, 7, 45)
        r1, r2 = O.bf_moments_full_plane(g, counts[7:45], params, dc, list(range(7, 45)))
        assert _rel(s2, r2) <= LOSS_RTOL
        assert np.max(np.abs(s1 - r1)) <= 1e-4 * 38 ** 0.5
        phase, psi = p.obj(params)
        ref_phase, ref_psi = O.object_wave_full_plane(g, counts, params)
        d = np.angle(np.exp(1j * (phase - ref_phase)))
        assert np.sqrt(np.mean(d * d)) <= PHASE_RMS
        assert np.linalg.norm(psi - ref_psi) <= 1e-5 * np.linalg.norm(ref_psi)
        # the fused call in this variant: the full-plane row pass sums Re and Im of O_b per pixel
        check_loss_object(p, params, ref_phase, ref_psi, "full plane, tiny")


def test_full_plane_small_equals_half_plane(small):
    """Hardly any transfer reaches the Nyquist lines at the small workload, where the
    smooth specimen's spectrum is ~1e-9 of its peak: the variant's loss is the oracle's
    and equals the half-plane loss to float rounding."""
    w, counts, p = small
    g = O.OGeom.from_any(w.geometry)
    dc = O.dc_value(counts)
    params = trial_params(w, 3)
    half = p.loss(params)
    ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_FULL_PLANE)
    try:
        full = p.loss(params)
        phase, _ = p.obj(params[0], with_psi=False)
    finally:
        ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_HALF_PLANE)
    for k in range(3):
        assert _rel(full[k], O.loss_full_plane(g, counts, params[k], dc)) <= LOSS_RTOL
        assert abs(full[k] - half[k]) <= 1e-9 * abs(half[k])
    ref, ref_psi = O.object_wave_full_plane(g, counts, params[0], dc)
    assert np.sqrt(np.mean(np.angle(np.exp(1j * (phase - ref))) ** 2)) <= PHASE_RMS
    ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_FULL_PLANE)
    try:
        check_loss_object(p, params[0].tolist(), ref, ref_psi, "full plane, small")
    finally:
        ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_HALF_PLANE)


@pytest.mark.parametrize("n,d,r2", [(64, 16, 20), (256, 24, 36)])   # transfer reaches the Nyquist lines
def test_full_plane_other_scan_sizes(n, d, r2):
    w = _custom_workload(n, d, r2)
    counts = cached_counts(w)
    og = O.OGeom.from_any(w.geometry)
    p = Prepared(w.geometry, counts)
    try:
        ssb.ssb_set_variant(p.h, ssb.SSB_VARIANT_FULL_PLANE)
        for params in ([40.0, 5.0, 0.3], [-25.0, 7.0, 2.4]):
            assert _rel(p.loss([params])[0], O.loss_full_plane(og, counts, params)) <= LOSS_RTOL
        phase, _ = p.obj([40.0, 5.0, 0.3], with_psi=False)
        ref, ref_psi = O.object_wave_full_plane(og, counts, [40.0, 5.0, 0.3])
        assert np.sqrt(np.mean(np.angle(np.exp(1j * (phase - ref))) ** 2)) <= PHASE_RMS
        check_loss_object(p, [40.0, 5.0, 0.3], ref, ref_psi, f"full plane, N = {n}")
    finally:
        p.release()


def test_variant_errors(tiny):
    w, counts, p = tiny
    for bad in (-1, 2, 7):
        with pytest.raises(ssb.SSBError) as ei:
            ssb.ssb_set_variant(p.h, bad)
        assert ei.value.code == ssb._ssb.SSB_EINVAL
    assert ssb.ssb_query(p.h)["variant"] == 0
