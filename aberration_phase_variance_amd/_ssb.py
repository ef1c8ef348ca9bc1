"""ctypes binding of libssb.so (declared in include/ssb.h): argument marshalling only.

Every step of the computation runs in the HIP library.  Device buffers and
streams may be passed as torch tensors / torch streams (used for their device
pointers only) or as raw integer addresses.  There is no fallback: if the built
library is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssb.so")

SSB_OK, SSB_EINVAL, SSB_ESHAPE, SSB_ENOMEM, SSB_EDEVICE = 0, -1, -2, -3, -4


class SSBError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"ssb error {code}: {msg}")
        self.code = code


class ssb_geometry(ctypes.Structure):
    _fields_ = [
        ("scan_n", ctypes.c_int32),
        ("det_n", ctypes.c_int32),
        ("bf_r2", ctypes.c_double),
        ("det_cy", ctypes.c_double),
        ("det_cx", ctypes.c_double),
        ("q_step_px", ctypes.c_double),
        ("dk", ctypes.c_double),
        ("wavelength_A", ctypes.c_double),
        ("alpha_rad", ctypes.c_double),
        ("rotation_rad", ctypes.c_double),
        ("edge_px", ctypes.c_double),
    ]


class ssb_info(ctypes.Structure):
    _fields_ = [
        ("n_bf", ctypes.c_int64),
        ("n_active_bf", ctypes.c_int64),
        ("scan_n", ctypes.c_int32),
        ("det_n", ctypes.c_int32),
        ("spectrum_bytes", ctypes.c_int64),
        ("dc", ctypes.c_double),
        ("chunk_bf", ctypes.c_int64),
        ("support_entries", ctypes.c_int64),
        ("columns_written", ctypes.c_int64),
        ("columns_read", ctypes.c_int64),
        ("variant", ctypes.c_int32),
        ("pad", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64),
        ("reserved_trials", ctypes.c_int32),
        ("pad2", ctypes.c_int32),
    ]


SSB_STAGES = ("pass1", "pass2", "reduce", "obj_sum", "obj_fft")


class ssb_profile_data(ctypes.Structure):
    _fields_ = [
        ("ms", ctypes.c_double * len(SSB_STAGES)),
        ("launches", ctypes.c_int64 * len(SSB_STAGES)),
        ("units", ctypes.c_int64 * len(SSB_STAGES)),
    ]


class ssb_fit_options(ctypes.Structure):
    _fields_ = [
        ("fatol", ctypes.c_double),
        ("xatol", ctypes.c_double),
        ("step_frac", ctypes.c_double),
        ("step_floor", ctypes.c_double * 3),
        ("max_evals", ctypes.c_int32),
        ("max_iter", ctypes.c_int32),
    ]


class ssb_fit_result(ctypes.Structure):
    _fields_ = [
        ("best", ctypes.c_double * 3),
        ("loss", ctypes.c_double),
        ("batch_best", ctypes.c_int32),
        ("requests", ctypes.c_int32),
        ("evals", ctypes.c_int32),
        ("iterations", ctypes.c_int32),
        ("converged", ctypes.c_int32),
        ("pad", ctypes.c_int32),
        ("batch_loss", ctypes.c_double),
    ]


SSB_OBJECTIVE = ctypes.CFUNCTYPE(ctypes.c_double, ctypes.POINTER(ctypes.c_float), ctypes.c_void_p)

FIT_DEFAULTS = {"fatol": 3e-6, "xatol": 0.1, "step_frac": 0.05, "step_floor": (0.01, 2.0, 0.04),
                "max_evals": 0, "max_iter": 0}

class ssb_probe_fit(ctypes.Structure):
    _fields_ = [
        ("det_cy", ctypes.c_double),
        ("det_cx", ctypes.c_double),
        ("bf_r2", ctypes.c_double),
        ("threshold", ctypes.c_double),
        ("n_disk", ctypes.c_int64),
        ("n_bf", ctypes.c_int64),
        ("n_zero", ctypes.c_int64),
    ]


EXPORTS = ("ssb_prepare", "ssb_reserve", "ssb_loss", "ssb_loss_noalloc", "ssb_moments", "ssb_object",
           "ssb_loss_object", "ssb_spectrum", "ssb_set_chunk",
           "ssb_profile", "ssb_query", "ssb_release", "ssb_last_error", "ssb_nelder_mead", "ssb_fit",
           "ssb_detector_sum", "ssb_fit_probe", "ssb_fit_probe_device", "ssb_gather_bf", "ssb_set_variant")

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libssb.so (once) and declare its signatures.  Raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m aberration_phase_variance_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    dp, fp = ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_float)
    lib.ssb_prepare.argtypes = [ctypes.POINTER(ssb_geometry), vp, i64, vp, ctypes.POINTER(vp)]
    lib.ssb_reserve.argtypes = [vp, i32]
    lib.ssb_loss.argtypes = [vp, fp, i32, dp, vp, vp]
    lib.ssb_loss_noalloc.argtypes = [vp, fp, i32, dp, vp, vp]
    lib.ssb_moments.argtypes = [vp, fp, i64, i64, vp, dp, vp]
    lib.ssb_object.argtypes = [vp, fp, vp, vp, vp]
    lib.ssb_loss_object.argtypes = [vp, fp, dp, vp, vp, vp]
    lib.ssb_spectrum.argtypes = [vp, i64, vp, vp]
    lib.ssb_set_chunk.argtypes = [vp, i64]
    lib.ssb_set_variant.argtypes = [vp, i32]
    lib.ssb_profile.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ssb_profile_data)]
    lib.ssb_query.argtypes = [vp, ctypes.POINTER(ssb_info)]
    lib.ssb_release.argtypes = [vp]
    lib.ssb_release.restype = None
    lib.ssb_last_error.argtypes = []
    lib.ssb_last_error.restype = ctypes.c_char_p
    lib.ssb_nelder_mead.argtypes = [dp, ctypes.POINTER(ssb_fit_options), SSB_OBJECTIVE, vp,
                                    ctypes.POINTER(ssb_fit_result), dp, i32]
    lib.ssb_fit.argtypes = [vp, fp, i32, ctypes.POINTER(ssb_fit_options), ctypes.POINTER(ssb_fit_result), dp, i32,
                            vp]
    lib.ssb_detector_sum.argtypes = [vp, i32, i32, vp, vp]
    lib.ssb_fit_probe.argtypes = [ctypes.POINTER(ctypes.c_uint64), i32, i32, ctypes.POINTER(ssb_probe_fit)]
    lib.ssb_gather_bf.argtypes = [vp, ctypes.POINTER(ssb_geometry), vp, i64, vp]
    lib.ssb_fit_probe_device.argtypes = [vp, i32, i32, ctypes.POINTER(ssb_probe_fit), vp]
    for name in EXPORTS:
        if name not in ("ssb_release", "ssb_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int):
    if rc != SSB_OK:
        raise SSBError(rc, load_library().ssb_last_error().decode())


def _ptr(x) -> int | None:
    """Device address of a torch tensor, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _dev(x, name: str, dtypes: tuple, numel: int, optional: bool = False) -> int | None:
    """Device address of x after checking it, when it is a tensor: one of the dtypes
    (names such as "float32"), exactly numel elements, contiguous, on a GPU.  Raw
    integer addresses are passed through unchecked (the caller vouches for them)."""
    if x is None:
        if optional:
            return None
        raise ValueError(f"{name}: a device buffer is required")
    if isinstance(x, int):
        return x
    dt = str(x.dtype).replace("torch.", "")
    if dt not in dtypes:
        raise ValueError(f"{name}: dtype {dt}, expected one of {', '.join(dtypes)}")
    if x.numel() != numel:
        raise ValueError(f"{name}: {x.numel()} elements, expected {numel}")
    if not x.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if not x.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    return int(x.data_ptr())


def _scan_n(handle: int) -> int:
    info = ssb_info()
    _check(load_library().ssb_query(handle, ctypes.byref(info)))
    return info.scan_n


_U32 = ("int32", "uint32")
_C64 = ("float32", "complex64")   # complex64 values as interleaved float32 pairs, or complex64


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def make_geometry(g) -> ssb_geometry:
    get = (lambda k: g[k]) if isinstance(g, dict) else (lambda k: getattr(g, k))
    return ssb_geometry(*[get(name) if typ is not ctypes.c_int32 else int(get(name))
                          for name, typ in ssb_geometry._fields_])


def _params(params, n_expected=None):
    p = np.ascontiguousarray(np.asarray(params, dtype=np.float32).reshape(-1, 3))
    if n_expected is not None and p.shape[0] != n_expected:
        raise ValueError("expected a single (C10, C12, phi12) triple")
    return p


# ----------------------------------------------------------------- C ABI, same names
def ssb_prepare(geometry, counts, n_bf: int, stream=None) -> int:
    """Returns an opaque handle (int).  counts: device uint32 [n_bf][N][N] (tensor or address)."""
    lib = load_library()
    g = make_geometry(geometry)
    ptr = _dev(counts, "counts", _U32, int(n_bf) * g.scan_n * g.scan_n)
    h = ctypes.c_void_p()
    _check(lib.ssb_prepare(ctypes.byref(g), ptr, int(n_bf), _stream(stream), ctypes.byref(h)))
    return h.value


def ssb_reserve(handle: int, max_trials: int) -> None:
    """Size the workspace so that loss calls of up to max_trials trials allocate nothing."""
    _check(load_library().ssb_reserve(handle, int(max_trials)))


def ssb_loss(handle: int, params, mean_phase=None, stream=None) -> np.ndarray:
    """Losses (float64 [n_trials]) for host params [n_trials][3]; optional device float [N][N] mean phase."""
    lib = load_library()
    p = _params(params)
    out = np.empty(p.shape[0], dtype=np.float64)
    mp = None
    if mean_phase is not None:
        n = _scan_n(handle)
        mp = _dev(mean_phase, "mean_phase", ("float32",), n * n)
    _check(lib.ssb_loss(handle, p.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), p.shape[0],
                        out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), mp, _stream(stream)))
    return out


def ssb_loss_noalloc(handle: int, params, mean_phase=None, stream=None) -> np.ndarray:
    """ssb_loss with every per-call buffer in the library's fixed device scratch (no allocation)."""
    lib = load_library()
    p = _params(params)
    out = np.empty(p.shape[0], dtype=np.float64)
    mp = None
    if mean_phase is not None:
        n = _scan_n(handle)
        mp = _dev(mean_phase, "mean_phase", ("float32",), n * n)
    _check(lib.ssb_loss_noalloc(handle, p.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), p.shape[0],
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), mp, _stream(stream)))
    return out


def ssb_moments(handle: int, params3, bf_begin: int, bf_end: int, s1, stream=None) -> float:
    """S1 into device double [N][N] s1; returns S2."""
    lib = load_library()
    p = _params(params3, 1)
    n = _scan_n(handle)
    ptr = _dev(s1, "s1", ("float64",), n * n)
    s2 = ctypes.c_double()
    _check(lib.ssb_moments(handle, p.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), int(bf_begin), int(bf_end),
                           ptr, ctypes.byref(s2), _stream(stream)))
    return s2.value


def ssb_object(handle: int, params3, phase, psi=None, stream=None) -> None:
    lib = load_library()
    p = _params(params3, 1)
    n = _scan_n(handle)
    ph = _dev(phase, "phase", ("float32",), n * n)
    ps = None
    if psi is not None:
        ps = _dev(psi, "psi", _C64, n * n * (2 if str(getattr(psi, "dtype", "")).endswith("float32") else 1))
    _check(lib.ssb_object(handle, p.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), ph, ps, _stream(stream)))


def ssb_loss_object(handle: int, params3, phase, psi=None, stream=None) -> float:
    """One trial's loss (returned) and its phase-of-mean object into device float [N][N] phase
    (and complex64 [N][N] psi when given), from one pass over the spectra."""
    lib = load_library()
    p = _params(params3, 1)
    n = _scan_n(handle)
    ph = _dev(phase, "phase", ("float32",), n * n)
    ps = None
    if psi is not None:
        ps = _dev(psi, "psi", _C64, n * n * (2 if str(getattr(psi, "dtype", "")).endswith("float32") else 1))
    loss = ctypes.c_double()
    _check(lib.ssb_loss_object(handle, p.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), ctypes.byref(loss), ph, ps,
                               _stream(stream)))
    return loss.value


def ssb_spectrum(handle: int, bf: int, out, stream=None) -> None:
    """Cached spectrum of BF pixel bf into out: complex64 [N][N/2+1] (or float32 pairs)."""
    n = _scan_n(handle)
    ne = n * (n // 2 + 1) * (2 if str(getattr(out, "dtype", "")).endswith("float32") else 1)
    _check(load_library().ssb_spectrum(handle, int(bf), _dev(out, "out", _C64, ne), _stream(stream)))


def ssb_set_chunk(handle: int, chunk_bf: int) -> None:
    _check(load_library().ssb_set_chunk(handle, int(chunk_bf)))


SSB_VARIANT_HALF_PLANE = 0
SSB_VARIANT_FULL_PLANE = 1


def ssb_set_variant(handle: int, variant: int) -> None:
    """0: corrected half plane with the anti-Hermitian extension (default); 1: every entry
    of the full plane corrected on its own."""
    _check(load_library().ssb_set_variant(handle, int(variant)))


def ssb_profile(handle: int, mode: int = 2) -> dict:
    """mode 1: enable and clear, 0: disable, 2: keep.  Returns the per-stage totals."""
    data = ssb_profile_data()
    _check(load_library().ssb_profile(handle, int(mode), ctypes.byref(data)))
    return {name: {"ms": data.ms[i], "launches": data.launches[i], "units": data.units[i]}
            for i, name in enumerate(SSB_STAGES)}


def ssb_query(handle: int) -> dict:
    info = ssb_info()
    _check(load_library().ssb_query(handle, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in ssb_info._fields_}


def ssb_release(handle: int) -> None:
    load_library().ssb_release(handle)


def ssb_last_error() -> str:
    return load_library().ssb_last_error().decode()


def _fit_options(opts) -> ssb_fit_options:
    o = dict(FIT_DEFAULTS)
    o.update(opts or {})
    return ssb_fit_options(o["fatol"], o["xatol"], o["step_frac"], (ctypes.c_double * 3)(*o["step_floor"]),
                           int(o["max_evals"]), int(o["max_iter"]))


def _fit_dict(res: ssb_fit_result, trace: np.ndarray) -> dict:
    out = {name: getattr(res, name) for name, _ in ssb_fit_result._fields_ if name != "pad"}
    out["best"] = list(res.best)
    out["trace"] = trace[:min(res.evals, trace.shape[0])].copy()
    return out


def ssb_nelder_mead(x0, objective, options=None, trace_cap: int = 4096) -> dict:
    """Refinement on a Python objective f(params3 float32 ndarray) -> float (host only).
    Returns the result fields plus 'trace' (evals x 4: float32 params, loss)."""
    lib = load_library()
    x = (ctypes.c_double * 3)(*[float(v) for v in x0])

    def cb(p, _ctx):
        return float(objective(np.array([p[0], p[1], p[2]], dtype=np.float32)))

    fn = SSB_OBJECTIVE(cb)
    res = ssb_fit_result()
    trace = np.zeros((trace_cap, 4), dtype=np.float64)
    opt = _fit_options(options)
    _check(lib.ssb_nelder_mead(x, ctypes.byref(opt), fn, None, ctypes.byref(res),
                               trace.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), trace_cap))
    return _fit_dict(res, trace)


def ssb_fit(handle: int, trials, options=None, trace_cap: int = 4096, stream=None) -> dict:
    """Batch of host trials [n][3], then refinement from the best one (see ssb.h)."""
    lib = load_library()
    p = _params(trials)
    res = ssb_fit_result()
    trace = np.zeros((trace_cap, 4), dtype=np.float64)
    opt = _fit_options(options)
    _check(lib.ssb_fit(handle, p.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), p.shape[0], ctypes.byref(opt),
                       ctypes.byref(res), trace.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), trace_cap,
                       _stream(stream)))
    return _fit_dict(res, trace)


def ssb_detector_sum(frames, scan_n: int, det_n: int, sums, stream=None) -> None:
    """sums (device uint64 [det_n^2]) = exact sum of the device uint32 frames [scan_n^2][det_n^2]."""
    f = _dev(frames, "frames", _U32, int(scan_n) ** 2 * int(det_n) ** 2)
    sp = _dev(sums, "sums", ("int64", "uint64"), int(det_n) ** 2)
    _check(load_library().ssb_detector_sum(f, int(scan_n), int(det_n), sp, _stream(stream)))


def ssb_fit_probe(sums, scan_n: int, det_n: int) -> dict:
    """Probe-disk fit from host sums (array-like of uint64, det_n^2 values)."""
    s = np.ascontiguousarray(np.asarray(sums, dtype=np.uint64).reshape(-1))
    out = ssb_probe_fit()
    _check(load_library().ssb_fit_probe(s.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), int(scan_n), int(det_n),
                                        ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in ssb_probe_fit._fields_}


def ssb_fit_probe_device(sums, scan_n: int, det_n: int, stream=None) -> dict:
    """The same probe-disk fit on the device from the device sums (uint64 [det_n^2])."""
    sp = _dev(sums, "sums", ("int64", "uint64"), int(det_n) ** 2)
    out = ssb_probe_fit()
    _check(load_library().ssb_fit_probe_device(sp, int(scan_n), int(det_n), ctypes.byref(out), _stream(stream)))
    return {name: getattr(out, name) for name, _ in ssb_probe_fit._fields_}


def ssb_gather_bf(frames, geometry, counts, n_bf: int, stream=None) -> None:
    """counts (device uint32 [n_bf][N][N]) = the BF pixels of the device frames, BF-major."""
    g = make_geometry(geometry)
    f = _dev(frames, "frames", _U32, g.scan_n ** 2 * g.det_n ** 2)
    c = _dev(counts, "counts", _U32, int(n_bf) * g.scan_n ** 2)
    _check(load_library().ssb_gather_bf(f, ctypes.byref(g), c, int(n_bf), _stream(stream)))
