"""GPU parity at the full and medium workload sizes, in the launch configuration the
benchmark times (N = 512, 8,937 BF, default chunking).

The complete loss over all 8,937 BF pixels of the 512^2 scan, the mean phase and
the phase-of-mean object are compared with the float64 oracle run over BF ranges
in a process pool on the host's cores (the measurement the Checkpoints page's
"2026-09-11 full-aperture Apple M5 floor checkpoint" insists on: no crop and no BF
reduction).  Sampled outputs are also checked one by one (cached spectra of single
BF pixels, phase moments of BF ranges including the ragged last group), with
properties that hold at any size (the loss equals the formula applied to the
moments of the whole range; moments are additive over a split of the range).
Counts come from the seeded device generator; the oracle gets the same bytes.
Every device output starts as NaN, so a region the library leaves unwritten fails.
"""
import dataclasses
import sys

import numpy as np
import pytest

import aberration_phase_variance_amd as ssb
from oracle import ssb_oracle as O
from oracle.pool import OraclePool
from synth import WORKLOADS, make_counts_torch, trial_params

pytestmark = pytest.mark.gpu

LOSS_RTOL = 1e-5
PHASE_RMS = 1e-4
TRUE = [40.0, 5.0, 0.3]


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


@pytest.fixture(scope="module")
def full():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    w = WORKLOADS["full"]
    _say("[full] generating counts on the device")
    counts = make_counts_torch(w, torch.device("cuda:0"))
    h = ssb.ssb_prepare(w.geometry, counts, w.n_bf)
    torch.cuda.synchronize()
    yield w, counts, h
    ssb.ssb_release(h)
    del counts
    torch.cuda.empty_cache()


def _host(counts, b0, b1):
    return counts[b0:b1].cpu().numpy().view(np.uint32)


@pytest.fixture(scope="module")
def full_pool(full):
    """The pooled float64 oracle over the full workload's counts (same bytes as the device's)."""
    w, counts, h = full
    _say("[full] staging counts for the pooled oracle")
    with OraclePool(lambda b0, b1: _host(counts, b0, b1), shape=(w.n_bf, 512, 512)) as pool:
        _say(f"[full] oracle pool of {pool.workers} workers")
        yield pool


def test_full_loss_all_bf(full, full_pool):
    """The complete exact loss at full size (all 8,937 BF) for the true aberrations and two
    seeded trials of the full fit's batch, in one batched call, within 1e-5 relative of the
    oracle; the mean phase of trial 0 within float rounding of the oracle's S1 / n_bf."""
    import torch
    w, counts, h = full
    og = O.OGeom.from_any(w.geometry)
    dc = ssb.ssb_query(h)["dc"]
    trials = np.concatenate([np.array([TRUE], np.float32), trial_params(w, 2)])
    mp = torch.full((512, 512), float("nan"), dtype=torch.float32, device="cuda")
    got = ssb.ssb_loss(h, trials, mp)
    mean_phase = mp.cpu().numpy()
    for k in range(len(trials)):
        _say(f"[full] oracle over all {w.n_bf} BF, trial {k} {trials[k].tolist()}")
        s1, s2 = full_pool.moments(og, trials[k], dc)
        ref = O.loss_from_moments(s1, s2, w.n_bf)
        _say(f"[full]   gpu {got[k]!r} oracle {ref!r} rel {abs(got[k] - ref) / abs(ref):.2e}")
        assert abs(got[k] - ref) <= LOSS_RTOL * abs(ref), (k, got[k], ref)
        if k == 0:
            d = mean_phase - s1 / w.n_bf
            assert np.all(np.isfinite(mean_phase))
            assert np.sqrt(np.mean(d * d)) <= 1e-6 and np.max(np.abs(d)) <= 1e-5


def test_full_object_all_bf(full, full_pool):
    """The phase-of-mean object over all 8,937 BF pixels within 1e-4 rad RMS of the oracle,
    from ssb_object and from the fused ssb_loss_object."""
    import torch
    w, counts, h = full
    og = O.OGeom.from_any(w.geometry)
    dc = ssb.ssb_query(h)["dc"]
    for params in (TRUE, trial_params(w, 1)[0].tolist()):
        phase = torch.full((512, 512), float("nan"), dtype=torch.float32, device="cuda")
        psi = torch.full((512, 512, 2), float("nan"), dtype=torch.float32, device="cuda")
        ssb.ssb_object(h, params, phase, psi)
        torch.cuda.synchronize()
        _say(f"[full] oracle object over all {w.n_bf} BF at {params}")
        ref_phase, ref_psi = full_pool.object_wave(og, params, dc)
        d = np.angle(np.exp(1j * (phase.cpu().numpy() - ref_phase)))
        rms = float(np.sqrt(np.mean(d * d)))
        p = psi.cpu().numpy()
        rel = np.linalg.norm(p[..., 0] + 1j * p[..., 1] - ref_psi) / np.linalg.norm(ref_psi)
        _say(f"[full]   object rms {rms:.2e} rad, psi rel L2 {rel:.2e}")
        assert rms <= PHASE_RMS and rel <= 1e-5
        # the fused loss and object: the loss bitwise ssb_loss's, the object the oracle's
        phase.fill_(float("nan"))
        psi.fill_(float("nan"))
        loss = ssb.ssb_loss_object(h, params, phase, psi)
        assert loss == ssb.ssb_loss(h, [params])[0]
        d2 = np.angle(np.exp(1j * (phase.cpu().numpy() - ref_phase)))
        rms2 = float(np.sqrt(np.mean(d2 * d2)))
        p2 = psi.cpu().numpy()
        rel2 = np.linalg.norm(p2[..., 0] + 1j * p2[..., 1] - ref_psi) / np.linalg.norm(ref_psi)
        _say(f"[full]   fused loss and object: object rms {rms2:.2e} rad, psi rel L2 {rel2:.2e}")
        assert rms2 <= PHASE_RMS and rel2 <= 1e-5


def _moments(h, n, params, b0, b1):
    import torch
    s1 = torch.full((n, n), float("nan"), dtype=torch.float64, device="cuda")
    s2 = ssb.ssb_moments(h, params, b0, b1, s1)
    return s1.cpu().numpy(), s2


def test_full_prepare_exact(full):
    w, counts, h = full
    info = ssb.ssb_query(h)
    assert info["n_bf"] == 8937 and info["n_active_bf"] == 8937
    assert info["scan_n"] == 512 and info["det_n"] == 192
    total = 0
    for b0 in range(0, w.n_bf, 1024):       # exact integer scan sums on the host
        total += int(_host(counts, b0, min(w.n_bf, b0 + 1024)).astype(np.int64).sum())
    assert info["dc"] == total / w.n_bf


def test_full_spectra_sampled(full):
    import torch
    w, counts, h = full
    for b in (0, 4468, 8936):
        ref = O.scan_spectrum(_host(counts, b, b + 1)[0])
        out = torch.full((512, 257, 2), float("nan"), dtype=torch.float32, device="cuda")
        ssb.ssb_spectrum(h, b, out)
        o = out.cpu().numpy()
        got = o[..., 0] + 1j * o[..., 1]
        assert np.linalg.norm(got - ref) <= 2e-6 * np.linalg.norm(ref), b


@pytest.mark.parametrize("b0,b1", [(0, 32), (4450, 4493), (8896, 8937)])
def test_full_moments_sampled(full, b0, b1):
    w, counts, h = full
    og = O.OGeom.from_any(w.geometry)
    dc = ssb.ssb_query(h)["dc"]
    for params in (TRUE, [-137.0, 16.5, 2.7]):
        s1, s2 = _moments(h, 512, params, b0, b1)
        r1, r2 = O.bf_moments(og, _host(counts, b0, b1), params, dc, list(range(b0, b1)))
        _check_range(s1, s2, r1, r2, b1 - b0, f"BF {b0}..{b1} at {params}")


def test_full_loss_is_formula_of_moments(full):
    w, counts, h = full
    for params in (TRUE, [88.0, -12.0, 1.1]):
        loss = ssb.ssb_loss(h, [params])[0]
        s1, s2 = _moments(h, 512, params, 0, w.n_bf)
        assert abs(loss - O.loss_from_moments(s1, s2, w.n_bf)) <= 1e-12 * abs(loss)
        # additivity over a split at a 32-BF group boundary
        a1, a2 = _moments(h, 512, params, 0, 4480)
        b1, b2 = _moments(h, 512, params, 4480, w.n_bf)
        assert abs((a2 + b2) - s2) <= 1e-12 * s2
        assert np.max(np.abs((a1 + b1) - s1)) <= 1e-9 * np.max(np.abs(s1))


def test_full_batch_invariance(full):
    w, counts, h = full
    p = np.array([TRUE, [-150.0, 3.0, 0.9], [20.0, 19.0, 2.2]], np.float32)
    batch = ssb.ssb_loss(h, p)
    for k in range(3):
        assert ssb.ssb_loss(h, p[k:k + 1])[0] == batch[k]


@pytest.fixture(scope="module")
def subdisk(full):
    """The full counts restricted to the 317 BF pixels of radius <= 10 px, same 512^2 scan."""
    import torch
    w, counts, h = full
    g = dataclasses.replace(w.geometry, bf_r2=100.0)
    og_full = O.OGeom.from_any(w.geometry)
    i, j = O.bf_indices(og_full)
    sel = np.flatnonzero((i - 96) ** 2 + (j - 96) ** 2 <= 100)
    sub = counts[torch.from_numpy(sel).cuda()].contiguous()
    hs = ssb.ssb_prepare(g, sub, sel.size)
    torch.cuda.synchronize()
    yield g, sub.cpu().numpy().view(np.uint32), hs
    ssb.ssb_release(hs)


def test_n512_subdisk_loss_and_object(subdisk):
    import torch
    g, counts, hs = subdisk
    og = O.OGeom.from_any(g)
    assert counts.shape[0] == 317
    dc = O.dc_value(counts)
    assert ssb.ssb_query(hs)["dc"] == dc
    for params in (TRUE, [-60.0, 9.0, 2.0]):
        got = ssb.ssb_loss(hs, [params])[0]
        ref = O.loss(og, counts, params, dc)
        assert abs(got - ref) <= LOSS_RTOL * abs(ref), (params, got, ref)
    phase = torch.full((512, 512), float("nan"), dtype=torch.float32, device="cuda")
    ssb.ssb_object(hs, TRUE, phase)
    torch.cuda.synchronize()
    ref_phase, _ = O.object_wave(og, counts, TRUE, dc)
    d = np.angle(np.exp(1j * (phase.cpu().numpy() - ref_phase)))
    assert np.sqrt(np.mean(d * d)) <= PHASE_RMS


def test_medium_loss_and_object():
    """Medium workload: its whole 200-trial batch and the true parameters in one call, every
    trial against the pooled oracle, single-trial calls equal to the batch bitwise, and the
    object."""
    import torch
    w = WORKLOADS["medium"]
    counts = make_counts_torch(w, torch.device("cuda:0"))
    h = ssb.ssb_prepare(w.geometry, counts, w.n_bf)
    try:
        host = counts.cpu().numpy().view(np.uint32)
        og = O.OGeom.from_any(w.geometry)
        dc = O.dc_value(host)
        trials = np.concatenate([np.array([TRUE], np.float32), trial_params(w)])
        assert trials.shape == (201, 3)
        got = ssb.ssb_loss(h, trials)
        _say("[medium] pooled oracle, 201 trials")
        worst = 0.0
        with OraclePool(host) as pool:
            for k in range(len(trials)):
                ref = pool.loss(og, trials[k], dc)
                worst = max(worst, abs(got[k] - ref) / abs(ref))
                assert abs(got[k] - ref) <= LOSS_RTOL * abs(ref), (k, got[k], ref)
                if k % 50 == 0:
                    _say(f"[medium]   trial {k}: largest relative difference so far {worst:.2e}")
        _say(f"[medium] 201 trials: largest relative loss difference {worst:.2e}")
        for k in (0, 5, 200):
            assert ssb.ssb_loss(h, trials[k:k + 1])[0] == got[k]
        phase = torch.full((256, 256), float("nan"), dtype=torch.float32, device="cuda")
        ssb.ssb_object(h, TRUE, phase)
        torch.cuda.synchronize()
        ref_phase, _ = O.object_wave(og, host, TRUE, dc)
        d = np.angle(np.exp(1j * (phase.cpu().numpy() - ref_phase)))
        assert np.sqrt(np.mean(d * d)) <= PHASE_RMS
    finally:
        ssb.ssb_release(h)


@pytest.mark.parametrize("b0,b1", [(0, 32), (8896, 8937)])
def test_full_plane_variant_moments_sampled(full, b0, b1):
    """The full-plane variant at full size: BF-range moments against the oracle's
    full-plane definition (Nyquist transfer is nonzero for BF pixels near the disk edge)."""
    w, counts, h = full
    og = O.OGeom.from_any(w.geometry)
    dc = ssb.ssb_query(h)["dc"]
    params = [-137.0, 16.5, 2.7]
    ssb.ssb_set_variant(h, ssb.SSB_VARIANT_FULL_PLANE)
    try:
        s1, s2 = _moments(h, 512, params, b0, b1)
    finally:
        ssb.ssb_set_variant(h, ssb.SSB_VARIANT_HALF_PLANE)
    r1, r2 = O.bf_moments_full_plane(og, _host(counts, b0, b1), params, dc, list(range(b0, b1)))
    _check_range(s1, s2, r1, r2, b1 - b0, f"full plane BF {b0}..{b1}")


def test_full_fit_trials_sampled(full):
    """Eight seeded trials of the full fit's batch (C10 +-200 nm, C12 +-20 nm, phi12 in
    [0, pi)): moments of a mid-disk BF range against the oracle, and their losses in one
    batched call equal to single-trial calls."""
    from synth import trial_params
    w, counts, h = full
    og = O.OGeom.from_any(w.geometry)
    dc = ssb.ssb_query(h)["dc"]
    trials = trial_params(w, 8)
    host = _host(counts, 4450, 4493)
    for k in range(8):
        s1, s2 = _moments(h, 512, trials[k], 4450, 4493)
        r1, r2 = O.bf_moments(og, host, trials[k], dc, list(range(4450, 4493)))
        _check_range(s1, s2, r1, r2, 43, f"trial {k}")
    batch = ssb.ssb_loss(h, trials)
    assert ssb.ssb_loss(h, trials[5:6])[0] == batch[5]
