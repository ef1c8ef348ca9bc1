"""Host-only checks of the C ABI library: it loads, exports what include/ssb.h declares,
and rejects bad arguments before touching a device (no compute calls, no GPU needed)."""
import ctypes
import dataclasses
import os
import re
import subprocess

import numpy as np
import pytest

import aberration_phase_variance_amd as ssb
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssb.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssb_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert "ssb_prepare" in declared and "ssb_loss" in declared and "ssb_object" in declared
    lib = ssb.load_library()
    for name in declared:
        assert hasattr(lib, name), name
    # dynamic symbol table, C linkage (unmangled)
    out = subprocess.run(["nm", "-D", "--defined-only", ssb.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ssb_[a-z_]+)\b", out))
    assert set(declared) <= exported
    assert set(declared) == set(ssb.EXPORTS)


def test_struct_layout_matches_header(tmp_path):
    """Size and every field offset of the binding's structs equal what a C compiler
    makes of include/ssb.h."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"ssb_geometry": ssb._ssb.ssb_geometry, "ssb_info": ssb._ssb.ssb_info,
               "ssb_profile_data": ssb._ssb.ssb_profile_data, "ssb_fit_options": ssb._ssb.ssb_fit_options,
               "ssb_fit_result": ssb._ssb.ssb_fit_result}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ssb.h"', 'int main(void) {']
    for name, cls in structs.items():
        lines.append(f'printf("{name} size %zu\\n", sizeof({name}));')
        for field, _ in cls._fields_:
            lines.append(f'printf("{name} {field} %zu\\n", offsetof({name}, {field}));')
    lines += ['return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    include = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-I", include, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(ln.split()[:2]): int(ln.split()[2]) for ln in out if ln.strip()}
    for name, cls in structs.items():
        assert got[(name, "size")] == ctypes.sizeof(cls), name
        for field, _ in cls._fields_:
            assert got[(name, field)] == getattr(cls, field).offset, (name, field)


def _geom(name="tiny", **kw):
    g = WORKLOADS[name].geometry
    return dataclasses.replace(g, **kw) if kw else g


def _code(fn, *a):
    with pytest.raises(ssb.SSBError) as ei:
        fn(*a)
    return ei.value.code


@pytest.mark.parametrize("bad", [dict(scan_n=48), dict(scan_n=2048), dict(scan_n=16), dict(det_n=0), dict(dk=0.0),
                                 dict(dk=float("nan")), dict(edge_px=-1.0), dict(alpha_rad=float("inf")),
                                 dict(bf_r2=-1.0), dict(rotation_rad=float("nan"))])
def test_prepare_rejects_bad_geometry(bad):
    assert _code(ssb.ssb_prepare, _geom(**bad), 0x1000, 49) == ssb._ssb.SSB_EINVAL
    assert ssb.ssb_last_error()


def test_prepare_rejects_wrong_bf_count():
    assert _code(ssb.ssb_prepare, _geom(), 0x1000, 48) == ssb._ssb.SSB_ESHAPE
    assert "49" in ssb.ssb_last_error()


def test_prepare_rejects_host_counts():
    counts = np.zeros((49, 32, 32), np.uint32)
    assert _code(ssb.ssb_prepare, _geom(), counts.ctypes.data, 49) == ssb._ssb.SSB_EINVAL


def test_null_handle_calls():
    lib = ssb.load_library()
    p = (ctypes.c_float * 3)(40.0, 5.0, 0.3)
    out = (ctypes.c_double * 1)()
    assert lib.ssb_loss(None, p, 1, out, None, None) == ssb._ssb.SSB_EINVAL
    assert lib.ssb_object(None, p, None, None, None) == ssb._ssb.SSB_EINVAL
    assert lib.ssb_loss_object(None, p, out, None, None, None) == ssb._ssb.SSB_EINVAL
    assert lib.ssb_query(None, None) == ssb._ssb.SSB_EINVAL
    assert lib.ssb_set_chunk(None, 64) == ssb._ssb.SSB_EINVAL
    assert lib.ssb_set_variant(None, 1) == ssb._ssb.SSB_EINVAL
    assert lib.ssb_moments(None, p, 0, 1, None, out, None) == ssb._ssb.SSB_EINVAL
    assert lib.ssb_prepare(None, None, 1, None, None) == ssb._ssb.SSB_EINVAL
    lib.ssb_release(None)          # no-op
    assert lib.ssb_last_error() is not None


def test_binding_checks_tensors_before_the_call():
    """Wrong dtype, element count, layout or device is a ValueError raised by the binding
    before any library call (no GPU needed: CPU tensors fail the device check last)."""
    import torch
    g = _geom()
    with pytest.raises(ValueError, match="dtype"):
        ssb.ssb_prepare(g, torch.zeros((49, 32, 32), dtype=torch.float32), 49)
    with pytest.raises(ValueError, match="elements"):
        ssb.ssb_prepare(g, torch.zeros((48, 32, 32), dtype=torch.int32), 49)
    with pytest.raises(ValueError, match="contiguous"):
        ssb.ssb_prepare(g, torch.zeros((49, 32, 32), dtype=torch.int32).transpose(1, 2), 49)
    with pytest.raises(ValueError, match="GPU"):
        ssb.ssb_prepare(g, torch.zeros((49, 32, 32), dtype=torch.int32), 49)
    with pytest.raises(ValueError, match="dtype"):
        ssb.ssb_detector_sum(0x1000, 2, 2, torch.zeros(4, dtype=torch.float64))
    with pytest.raises(ValueError, match="elements"):
        ssb.ssb_gather_bf(0x1000, g, torch.zeros((49, 32, 31), dtype=torch.int32),
                          49)
