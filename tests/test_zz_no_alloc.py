"""The no-allocation loss entry point (ssb_loss_noalloc) through the C ABI against
ssb_loss on the same handles: two calls in a row, the second on a smaller input, then
the scan size the benchmark runs (N = 512), a request too large for the scratch, and
the handle's own workspace and the device's free memory left as they were."""
import sys

import numpy as np
import pytest

import aberration_phase_variance_amd as ssb
from synth import WORKLOADS, cached_counts, make_counts_torch, make_geometry, trial_params

pytestmark = pytest.mark.gpu

LOSS_RTOL = 1e-5


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return torch


def _compare(t, h, n, params):
    """ssb_loss_noalloc against ssb_loss (losses and trial 0's mean phase): the same
    kernels on the same data, only the chunking differs, so the results are bitwise the
    same; the tolerance of the loss is checked as well.  Nothing is allocated: the
    handle's workspace and the device's free memory are unchanged across the call."""
    mp_ref = t.full((n, n), float("nan"), dtype=t.float32, device="cuda")
    ref = ssb.ssb_loss(h, params, mp_ref)
    mp = t.full((n, n), float("nan"), dtype=t.float32, device="cuda")
    ws = ssb.ssb_query(h)["workspace_bytes"]
    t.cuda.synchronize()
    free0 = t.cuda.mem_get_info()[0]
    got = ssb.ssb_loss_noalloc(h, params, mp)
    free1 = t.cuda.mem_get_info()[0]
    assert free1 == free0
    assert ssb.ssb_query(h)["workspace_bytes"] == ws
    assert np.all(np.abs(got - ref) <= LOSS_RTOL * np.abs(ref)), (got, ref)
    assert np.array_equal(got, ref), (got, ref)
    a, b = mp.cpu().numpy(), mp_ref.cpu().numpy()
    assert np.all(np.isfinite(a)) and np.array_equal(a, b)
    return got


def test_noalloc_two_calls_then_smaller():
    t = _torch()
    wm, ws = WORKLOADS["medium"], WORKLOADS["small"]
    _say("[noalloc] medium handle, 3 trials")
    cm = make_counts_torch(wm, t.device("cuda:0"))
    hm = ssb.ssb_prepare(wm.geometry, cm, wm.n_bf)
    cs = t.from_numpy(cached_counts(ws).view(np.int32)).cuda()
    hs = ssb.ssb_prepare(ws.geometry, cs, ws.n_bf)
    try:
        first = _compare(t, hm, 256, trial_params(wm, 3))
        _say("[noalloc] small handle, 1 trial (a smaller input into the same scratch)")
        _compare(t, hs, 128, trial_params(ws, 1))
        _say("[noalloc] the medium handle again")
        assert np.array_equal(ssb.ssb_loss_noalloc(hm, trial_params(wm, 3)), first)
        # a batch too large for the scratch is rejected with a clear error, and the handle
        # still works afterwards
        with pytest.raises(ssb.SSBError) as ei:
            ssb.ssb_loss_noalloc(hs, trial_params(ws, 200))
        assert ei.value.code == ssb._ssb.SSB_EINVAL and "scratch" in str(ei.value)
        _compare(t, hs, 128, trial_params(ws, 5))
    finally:
        ssb.ssb_release(hm)
        ssb.ssb_release(hs)


def test_noalloc_scan512():
    """The benchmark's scan size (N = 512): 317 BF on a 48-pixel detector, both variants."""
    t = _torch()
    w = WORKLOADS["full"]
    import dataclasses
    g = make_geometry(512, 48, 100)
    wl = dataclasses.replace(w, name="n512_d48", geometry=g, n_bf=317)
    _say("[noalloc] N = 512 handle, 317 BF")
    c = make_counts_torch(wl, t.device("cuda:0"))
    h = ssb.ssb_prepare(g, c, 317)
    try:
        params = trial_params(w, 4)
        _compare(t, h, 512, params)
        ssb.ssb_set_variant(h, ssb.SSB_VARIANT_FULL_PLANE)
        _compare(t, h, 512, params[:2])
    finally:
        ssb.ssb_release(h)
