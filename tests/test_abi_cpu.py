"""The C-ABI library loads and behaves at its boundary, without a GPU.

No computation is launched here: only symbol presence, static strings and the
argument checks that run before any device call.
"""
import ctypes
import os
import re

import pytest

import deterministic_invariant_gemm_det_amd as dg

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "det_gemm.h")
PEAK_HEADER = os.path.join(os.path.dirname(HEADER), "det_peak.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(det_gemm_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(dg.LIB_PATH)
    names = declared_functions()
    assert {"det_gemm_fwd", "det_gemm_dx", "det_gemm_dw"} <= set(names)
    for name in names:
        assert hasattr(L, name), name


def test_static_strings_and_version():
    assert dg.det_gemm_version() >= 100
    assert dg.det_gemm_strerror(0) == "success"
    for st in (-1, -2, -3, -4, -5):
        assert dg.det_gemm_strerror(st) != "unknown status"
    assert dg.det_gemm_strerror(-99) == "unknown status"


def test_force_family_validation():
    for bad in (-2, 2, 9, 17):
        with pytest.raises(dg.DetGemmError):
            dg.det_gemm_debug_force_family(bad)
    for good in (-1, 0, 1, 10, 15, 16):
        dg.det_gemm_debug_force_family(good)
    dg.det_gemm_debug_force_family(-1)


def _status(fn, *args):
    return fn(*args)


@pytest.mark.parametrize("op", ["fwd", "dx", "dw"])
def test_argument_checks_before_any_device_call(op):
    L = dg.lib()
    p = 0x1000  # never dereferenced: every call below is rejected before launch

    def call(out, a, b, m, k, n, dt, tier):
        if op == "fwd":
            return L.det_gemm_fwd(out, a, b, None, m, k, n, dt, tier, None)
        return getattr(L, "det_gemm_" + op)(out, a, b, m, k, n, dt, tier, None)

    assert call(None, p, p, 4, 4, 4, 0, 0) == -1
    assert call(p, None, p, 4, 4, 4, 0, 0) == -1
    assert call(p, p, None, 4, 4, 4, 0, 0) == -1
    assert call(p, p, p, 0, 4, 4, 0, 0) == -1
    assert call(p, p, p, 4, -1, 4, 0, 0) == -1
    assert call(p, p, p, 4, 4, 0, 0, 0) == -1
    assert call(p, p, p, 1 << 40, 1 << 40, 4, 0, 0) == -1
    assert call(p, p, p, 4, 4, 4, 7, 0) == -2
    assert call(p, p, p, 4, 4, 4, 0, 5) == -3
    assert "m, k and n" in dg.det_gemm_last_error() or dg.det_gemm_last_error()


def test_no_device_is_refused_cleanly():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; this checks the no-device path only")
    L = dg.lib()
    p = 0x1000
    assert L.det_gemm_fwd(p, p, p, None, 4, 4, 4, 0, 0, None) == -4
    assert dg.det_gemm_last_error()


def test_dw_out_and_db_argument_checks():
    L = dg.lib()
    p = 0x1000  # never dereferenced: every call below is rejected before launch
    F32, BF16, F16 = 0, 1, 2
    # the output dtype is the input dtype or f32; nothing else
    assert L.det_gemm_dw_out(p, F16, p, p, 4, 4, 4, BF16, 0, None) == -2
    assert L.det_gemm_dw_out(p, BF16, p, p, 4, 4, 4, F32, 0, None) == -2
    assert L.det_gemm_dw_out(p, 7, p, p, 4, 4, 4, BF16, 0, None) == -2
    assert L.det_gemm_dw_out(None, F32, p, p, 4, 4, 4, BF16, 0, None) == -1
    assert L.det_gemm_dw_out(p, F32, p, p, 0, 4, 4, BF16, 0, None) == -1
    assert L.det_gemm_dw_out(p, F32, p, p, 4, 4, 4, BF16, 5, None) == -3
    assert L.det_gemm_db(p, F16, p, 4, 4, BF16, 0, None) == -2
    assert L.det_gemm_db(p, BF16, p, 4, 4, F16, 0, None) == -2
    assert L.det_gemm_db(p, F32, p, 4, 4, 9, 0, None) == -2
    assert L.det_gemm_db(p, F32, p, 4, 4, BF16, 7, None) == -3
    assert L.det_gemm_db(None, F32, p, 4, 4, BF16, 0, None) == -1
    assert L.det_gemm_db(p, F32, None, 4, 4, BF16, 0, None) == -1
    assert L.det_gemm_db(p, F32, p, 0, 4, BF16, 0, None) == -1
    assert L.det_gemm_db(p, F32, p, 4, -3, BF16, 0, None) == -1
    assert L.det_gemm_db(p, F32, p, 1 << 40, 1 << 40, BF16, 0, None) == -1
    assert "dtype" in dg.det_gemm_last_error() or dg.det_gemm_last_error()


def test_cr_tier_checks():
    L = dg.lib()
    p = 0x1000  # never dereferenced: every call below is rejected before launch
    BF16, CR = 1, 2
    assert L.det_gemm_fwd(p, p, p, None, 4, 1 << 27, 4, BF16, CR, None) == -1   # reduction too long
    assert L.det_gemm_dw(p, p, p, 1 << 27, 4, 4, BF16, CR, None) == -1
    assert L.det_gemm_db(p, BF16, p, 1 << 27, 4, BF16, CR, None) == -1
    assert L.det_gemm_fwd(p, p, p, None, 4, 4, 4, BF16, 3, None) == -3
    assert dg.lib().det_gemm_debug_force_cr_fallback(3) == -1
    assert dg.lib().det_gemm_debug_force_cr_fallback(-1) == -1
    assert dg.lib().det_gemm_debug_force_cr_fallback(0) == 0


def test_peak_library_is_separate_and_checks_arguments():
    """The peak-rate microkernels live in libdetpeak.so (include/det_peak.h), not in the GEMM library."""
    from deterministic_invariant_gemm_det_amd import peak
    L = peak.lib()
    text = re.sub(r"/\*.*?\*/", "", open(PEAK_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(det_peak_\w+)\s*\(", text)))
    assert names == ["det_peak_run"]
    for name in names:
        assert hasattr(L, name)
    assert not hasattr(ctypes.CDLL(dg.LIB_PATH), "det_gemm_measure_peak")
    fl = ctypes.c_double(0.0)
    p = 0x1000  # never dereferenced: rejected before any device call
    assert L.det_peak_run(3, 10, p, 1 << 20, ctypes.byref(fl), None) == -1
    assert L.det_peak_run(-1, 10, p, 1 << 20, ctypes.byref(fl), None) == -1
    assert L.det_peak_run(0, 0, p, 1 << 20, ctypes.byref(fl), None) == -1
    assert L.det_peak_run(0, 10, None, 1 << 20, ctypes.byref(fl), None) == -1
    assert L.det_peak_run(0, 10, p, 1 << 20, None, None) == -1


def test_force_arch_validation():
    assert dg.lib().det_gemm_debug_force_arch(b"x" * 64) == -1
    dg.det_gemm_debug_force_arch("gfx942")
    dg.det_gemm_debug_force_arch(None)
    dg.det_gemm_debug_force_arch("")


def test_out_tensor_checks_before_launch():
    """A caller-supplied out of the wrong shape, dtype, layout or device is refused before any
    launch (the kernels would write shape x dtype bytes into it)."""
    import torch
    cpu = torch.device("cpu")
    good = torch.empty((4, 6), dtype=torch.bfloat16)
    assert dg._out(good, (4, 6), torch.bfloat16, cpu) is good
    assert dg._out(None, (4, 6), torch.float32, cpu).shape == (4, 6)
    for bad in (torch.empty((4, 5), dtype=torch.bfloat16),            # too small
                torch.empty((6, 4), dtype=torch.bfloat16),            # transposed shape
                torch.empty((4, 6), dtype=torch.float16),             # narrower or other dtype
                torch.empty((4, 6), dtype=torch.float32),             # wider dtype
                torch.empty((6, 4), dtype=torch.bfloat16).t(),        # non-contiguous view
                torch.empty((4, 6), dtype=torch.bfloat16, device="meta")):   # another device
        with pytest.raises(ValueError):
            dg._out(bad, (4, 6), torch.bfloat16, cpu)
