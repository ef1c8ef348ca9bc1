"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A copy of libssb.so is built with the sanitizers on the host side only (each
-fsanitize= behind -Xarch_host; the device code is built as usual) and loaded in a
fresh Python process with the sanitizer runtime preloaded.  The process runs every
host-only path: geometry validation and its errors, the BF rule, null-handle calls,
the thread-local error text, the Nelder-Mead refinement on a Python objective, and the
probe-disk fit.  Any sanitizer report aborts that process, which fails the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import ctypes, dataclasses, math, sys
import numpy as np
sys.path.insert(0, ROOT)
from aberration_phase_variance_amd import _ssb as S
from synth import WORKLOADS
lib = S.load_library(LIB)
g = WORKLOADS["tiny"].geometry
for bad in (dict(scan_n=48), dict(scan_n=2048), dict(det_n=0), dict(dk=0.0), dict(dk=float("nan")),
            dict(edge_px=-1.0), dict(alpha_rad=float("inf")), dict(bf_r2=-1.0), dict(rotation_rad=float("nan"))):
    try:
        S.ssb_prepare(dataclasses.replace(g, **bad), 0x1000, 49)
        raise SystemExit("accepted a bad geometry")
    except S.SSBError as e:
        assert e.code == S.SSB_EINVAL and S.ssb_last_error()
for gname in ("small", "medium", "full"):
    w = WORKLOADS[gname]
    try:
        S.ssb_prepare(w.geometry, 0x1000, w.n_bf + 1)
        raise SystemExit("accepted a wrong BF count")
    except S.SSBError as e:
        assert e.code == S.SSB_ESHAPE
counts = np.zeros((49, 32, 32), np.uint32)
try:
    S.ssb_prepare(g, counts.ctypes.data, 49)
    raise SystemExit("accepted host counts")
except S.SSBError as e:
    assert e.code == S.SSB_EINVAL
p = (ctypes.c_float * 3)(40.0, 5.0, 0.3)
out = (ctypes.c_double * 2)()
for rc in (lib.ssb_loss(None, p, 1, out, None, None), lib.ssb_loss_noalloc(None, p, 1, out, None, None),
           lib.ssb_object(None, p, None, None, None), lib.ssb_query(None, None), lib.ssb_set_chunk(None, 64),
           lib.ssb_set_variant(None, 1), lib.ssb_reserve(None, 4), lib.ssb_moments(None, p, 0, 1, None, out, None),
           lib.ssb_prepare(None, None, 1, None, None), lib.ssb_profile(None, 1, None)):
    assert rc == S.SSB_EINVAL
lib.ssb_release(None)
# Nelder-Mead on a smooth objective with a float32-identical memo
f = lambda q: (q[0] - 40.0) ** 2 / 100.0 + (q[1] - 5.0) ** 2 + 10.0 * (q[2] - 0.3) ** 2 + 1.0
r = S.ssb_nelder_mead([30.0, 9.0, 0.8], f, {"fatol": 1e-12, "xatol": 1e-6, "max_iter": 400})
assert abs(r["best"][0] - 40.0) < 1e-2 and r["evals"] > 10
r = S.ssb_nelder_mead([0.0, 0.0, 0.0], f, {"max_evals": 7}, trace_cap=3)
assert r["evals"] <= 7 and r["trace"].shape[0] == 3
# probe-disk fit on a synthetic mean pattern
d = 48
yy, xx = np.mgrid[0:d, 0:d]
sums = np.where((yy - 23.5) ** 2 + (xx - 24.25) ** 2 <= 100.0, 1000, 1).astype(np.uint64)
fit = S.ssb_fit_probe(sums, 16, d)
assert abs(fit["det_cy"] - 23.5) < 0.6 and fit["n_bf"] > 250
try:
    S.ssb_fit_probe(np.zeros(d * d, np.uint64), 16, d)
    raise SystemExit("fitted an empty pattern")
except S.SSBError as e:
    assert e.code == S.SSB_EINVAL
print("SANITIZED_HOST_OK", flush=True)
'''


def _runtime():
    libs = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return libs[0] if libs else None


@pytest.mark.skipif(_runtime() is None, reason="no clang AddressSanitizer runtime")
def test_host_code_under_asan_ubsan(tmp_path):
    from aberration_phase_variance_amd import build as B
    lib = str(tmp_path / "libssb_sanitized.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    cmd = [B.hipcc()] + B.flags() + san + [os.path.join(B.CSRC, s) for s in B.SOURCES] + ["-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    # the copy is instrumented: it imports the sanitizers' reporting entry points
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    env = dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    code = f"ROOT = {ROOT!r}\nLIB = {lib!r}\n" + SCRIPT
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=300)
    assert p.returncode == 0 and "SANITIZED_HOST_OK" in p.stdout, (p.stdout[-2000:], p.stderr[-4000:])
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr, p.stderr[-4000:]
