"""The C-ABI library loads, exports every symbol include/wvd.h declares, and
validates arguments on the host (no GPU work is enqueued by these calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wvd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wvd_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def wvd():
    from video_diffusion_vae_amd import wvd as m
    return m


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("wvd_prepared_bytes", "wvd_prepare", "wvd_workspace_bytes", "wvd_decode", "wvd_destroy",
              "wvd_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(wvd):
    lib = ctypes.CDLL(wvd.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(wvd):
    assert wvd.status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert wvd.status_string(s) not in ("ok", "unknown status")
    assert wvd.status_string(7) == "unknown status"


def test_prepared_bytes_validation(wvd):
    n16 = wvd.wvd_prepared_bytes(16, 4, 6)
    n64 = wvd.wvd_prepared_bytes(64, 22, 39)
    assert 0 < n16 < n64
    # 424M parameters as fp16 (0.85 GB), the phase-form up-convs at 16/9 of
    # their 3x3 size, and the ResBlock convs (383M parameters) held in
    # Winograd form: F(6,3) along x keeps 8 planes x 9 (t, y) taps = 8/3 of
    # their 27 taps (2.16 GB in all).
    n256 = wvd.wvd_prepared_bytes(256, 44, 78)
    assert 2.0e9 < n256 < 2.4e9
    for bad in ((0, 4, 6), (24, 4, 6), (512, 4, 6), (16, 0, 6), (16, 4, 5000)):
        with pytest.raises(wvd.WvdError) as e:
            wvd.wvd_prepared_bytes(*bad)
        assert e.value.status == wvd.WVD_EUNSUPPORTED
    assert wvd.lib().wvd_prepared_bytes(16, 4, 6, None) == wvd.WVD_EINVAL


def test_prepare_rejects_bad_arguments_before_any_launch(wvd):
    lib = wvd.lib()
    plan = ctypes.c_void_p(0)
    ptrs = (ctypes.c_void_p * 84)(*([16] * 84))
    # null weights / prepared / plan_out
    assert lib.wvd_prepare(16, 4, 6, None, 84, 0, 16, 1 << 30, None, ctypes.byref(plan)) == wvd.WVD_EINVAL
    assert lib.wvd_prepare(16, 4, 6, ptrs, 84, 0, None, 1 << 30, None, ctypes.byref(plan)) == wvd.WVD_EINVAL
    assert lib.wvd_prepare(16, 4, 6, ptrs, 84, 0, 16, 1 << 30, None, None) == wvd.WVD_EINVAL
    # wrong count, unsupported width, too small a buffer, a null weight
    assert lib.wvd_prepare(16, 4, 6, ptrs, 83, 0, 16, 1 << 30, None, ctypes.byref(plan)) == wvd.WVD_EINVAL
    assert lib.wvd_prepare(20, 4, 6, ptrs, 84, 0, 16, 1 << 30, None, ctypes.byref(plan)) == wvd.WVD_EUNSUPPORTED
    assert lib.wvd_prepare(16, 4, 6, ptrs, 84, 0, 16, 10, None, ctypes.byref(plan)) == wvd.WVD_ENOSPACE
    ptrs2 = (ctypes.c_void_p * 84)(*([16] * 83 + [None]))
    assert lib.wvd_prepare(16, 4, 6, ptrs2, 84, 0, 16, 1 << 30, None, ctypes.byref(plan)) == wvd.WVD_EINVAL
    # unknown weight dtype
    assert lib.wvd_prepare(16, 4, 6, ptrs, 84, 7, 16, 1 << 30, None, ctypes.byref(plan)) == wvd.WVD_EINVAL
    assert plan.value is None


def test_decode_and_workspace_reject_bad_plans(wvd):
    lib = wvd.lib()
    n = ctypes.c_size_t(0)
    assert lib.wvd_workspace_bytes(None, 3, 1, ctypes.byref(n)) == wvd.WVD_EINVAL
    assert lib.wvd_decode(None, 16, 0, 3, 1, 16, 16, 1 << 30, None) == wvd.WVD_EINVAL
    lib.wvd_destroy(None)  # ignored
    assert lib.wvd_profile_enable(None, 1) == wvd.WVD_EINVAL
