"""MI355X (gfx950) SSB phase-variance objective: HIP kernels behind a C ABI (include/ssb.h).

The Python layer is a thin ctypes binding with the C ABI's names; all computation runs
in libssb.so.  Build it with ``python -m aberration_phase_variance_amd.build``.
"""
from ._ssb import (EXPORTS, FIT_DEFAULTS, LIB_PATH, SSBError, load_library, make_geometry, ssb_detector_sum,
                   ssb_fit, ssb_fit_probe, ssb_fit_probe_device, ssb_gather_bf,
                   ssb_geometry, ssb_info, ssb_last_error, ssb_loss, ssb_loss_noalloc, ssb_loss_object, ssb_moments, ssb_nelder_mead,
                   ssb_object,
                   ssb_prepare, ssb_query, ssb_reserve, ssb_release, ssb_set_chunk, ssb_set_variant, ssb_spectrum, ssb_profile,
                   SSB_STAGES, SSB_VARIANT_FULL_PLANE, SSB_VARIANT_HALF_PLANE)

__all__ = ["EXPORTS", "FIT_DEFAULTS", "LIB_PATH", "SSBError", "load_library", "make_geometry", "ssb_detector_sum",
           "ssb_fit", "ssb_fit_probe", "ssb_fit_probe_device", "ssb_gather_bf",
           "ssb_geometry", "ssb_info", "ssb_last_error", "ssb_loss", "ssb_loss_noalloc", "ssb_loss_object", "ssb_moments",
           "ssb_nelder_mead",
           "ssb_object", "ssb_prepare", "ssb_reserve", "ssb_query", "ssb_release", "ssb_set_chunk", "ssb_spectrum",
           "ssb_profile", "SSB_STAGES", "ssb_set_variant", "SSB_VARIANT_FULL_PLANE", "SSB_VARIANT_HALF_PLANE"]
