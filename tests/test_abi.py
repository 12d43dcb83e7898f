"""The C-ABI library loads and exports what include/mla_verify.h declares (no GPU calls)."""
import ctypes
import os
import re
import subprocess

import pytest

from speculative_decode_mla_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_verify.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(mla_verify_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    return _lib.load()


def test_header_declares_the_boundary():
    assert _declared() == ["mla_verify_build_metadata", "mla_verify_compact", "mla_verify_create",
                           "mla_verify_debug_flags", "mla_verify_destroy", "mla_verify_error_string",
                           "mla_verify_merge", "mla_verify_partials", "mla_verify_run", "mla_verify_run_noalloc",
                           "mla_verify_workspace"]


@pytest.mark.parametrize("debug", [False, True], ids=["release", "debug build"])
def test_every_declared_symbol_is_exported(lib, debug):
    path = _lib.DEBUG_LIB_PATH if debug else _lib.LIB_PATH
    if not os.path.exists(path):
        pytest.skip("library not built")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (mla_verify_\w+)$", out, re.M))
    assert set(_declared()) == exported  # and nothing else under the library's prefix
    assert set(_declared()) == set(_lib.SIGNATURES)
    dl = _lib.load(debug)
    for name in _declared():
        assert hasattr(dl, name)


def test_debug_flags_host_checks(lib):
    flags = ctypes.c_int32(7)
    assert lib.mla_verify_debug_flags(None, ctypes.byref(flags), 0) == _lib.MLA_ERR_INVALID_ARGUMENT
    if os.path.exists(_lib.DEBUG_LIB_PATH):
        assert _lib.load(True).mla_verify_debug_flags(None, ctypes.byref(flags), 0) == _lib.MLA_ERR_INVALID_ARGUMENT


def test_config_struct_layout_matches_header():
    assert ctypes.sizeof(_lib.MlaVerifyConfig) == 48
    assert _lib.MlaVerifyConfig.num_slots.offset == 24 and _lib.MlaVerifyConfig.sm_scale.offset == 32
    assert _lib.MlaVerifyConfig.form.offset == 36 and _lib.MlaVerifyConfig.flags.offset == 40


def test_error_strings(lib):
    assert _lib.error_string(0) == "MLA_OK"
    assert _lib.error_string(-1) == "MLA_ERR_INVALID_ARGUMENT"
    assert _lib.error_string(-4) == "MLA_ERR_HIP"
    assert _lib.error_string(12345) == "MLA_ERR_UNKNOWN"


def test_host_validation_before_any_hip_call(lib):
    P = ctypes.c_void_p
    assert lib.mla_verify_run(None, None, None, None, None, None, None, None, 1, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_verify_merge(None, None, None, 1, 1, 1, 1, None, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_verify_partials(None, None, None, None, None, None, 1, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_verify_destroy(None) == _lib.MLA_OK
    # compaction: checks come before any HIP call; an empty copy enqueues nothing
    assert lib.mla_verify_compact(None, None, 0, None, 0, 0, None, None) == _lib.MLA_OK
    assert lib.mla_verify_compact(None, None, 1, None, 1, 0, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_verify_compact(None, None, -1, None, 0, 0, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    fake = P(1 << 20)  # never dereferenced: every call below fails its host checks
    assert lib.mla_verify_compact(fake, fake, 10, fake, 9, 0, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_verify_compact(fake, fake, 10, fake, 20, 11, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_verify_compact(fake, fake, 10, fake, 20, -1, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_verify_compact(P((1 << 20) + 8), fake, 10, fake, 20, 0, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_verify_compact(fake, fake, 10, fake, 1 << 40, (1 << 31) - 5, fake, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    # step metadata: host checks (never launched here)
    bm = lib.mla_verify_build_metadata
    assert bm(None, 1, 1, 1, fake, fake, fake, 1, fake, 1, fake, fake, fake, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert bm(fake, 1, 1, 1, fake, fake, fake, 1, fake, 1, fake, fake, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert bm(fake, 1, 1, 1, fake, fake, fake, 1, None, 1, fake, fake, fake, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert bm(fake, 0, 1, 1, fake, fake, fake, 1, fake, 1, fake, fake, fake, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert bm(fake, 1, 8, 4, fake, fake, fake, 1, fake, 1, fake, fake, fake, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert bm(fake, 1, 1, 1, fake, fake, fake, 1025, fake, 1, fake, fake, fake, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert bm(fake, 1, 1, 1, fake, fake, fake, 1, fake, 1 << 31, fake, fake, fake, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert bm(fake, 1, 1, 1, fake, fake, fake, 1, P((1 << 20) + 2), 1, fake, fake, fake, None) == \
        _lib.MLA_ERR_INVALID_ARGUMENT
    h = P()
    assert lib.mla_verify_create(None, ctypes.byref(h)) == _lib.MLA_ERR_INVALID_ARGUMENT
    bad = _lib.MlaVerifyConfig(16, 512, 512, 1, 4, 1, 4096, 0.07)
    assert lib.mla_verify_create(ctypes.byref(bad), ctypes.byref(h)) == _lib.MLA_ERR_UNSUPPORTED
    bad = _lib.MlaVerifyConfig(0, 576, 512, 1, 4, 1, 4096, 0.07)
    assert lib.mla_verify_create(ctypes.byref(bad), ctypes.byref(h)) == _lib.MLA_ERR_INVALID_ARGUMENT
    bad = _lib.MlaVerifyConfig(16, 576, 512, 1, 4, 1, 4096, float("nan"))
    assert lib.mla_verify_create(ctypes.byref(bad), ctypes.byref(h)) == _lib.MLA_ERR_INVALID_ARGUMENT
    bad = _lib.MlaVerifyConfig(16, 576, 512, 1, 4, 1, 4096, 0.07, 4)  # no kernel form 4
    assert lib.mla_verify_create(ctypes.byref(bad), ctypes.byref(h)) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert h.value is None


def test_create_without_a_gpu_reports_hip_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    cfg = _lib.MlaVerifyConfig(16, 576, 512, 1, 4, 1, 4096, 0.07)
    assert lib.mla_verify_create(ctypes.byref(cfg), ctypes.byref(h)) == _lib.MLA_ERR_HIP
    assert h.value is None


def test_torch_wrapper_rejects_bad_tensors():
    import torch
    from speculative_decode_mla_amd import api
    with pytest.raises(ValueError):
        api._need(torch.zeros(3, dtype=torch.float32), "x", torch.bfloat16, 1)
    with pytest.raises(ValueError):
        api._need(torch.zeros(3, 4, dtype=torch.bfloat16).t(), "x", torch.bfloat16, 2)
    with pytest.raises(ValueError):
        api._need(torch.zeros(3, dtype=torch.bfloat16), "x", torch.bfloat16, 1)  # not on a GPU


def test_noalloc_rejects_what_its_scratch_cannot_hold(lib):
    """mla_verify_run_noalloc checks the call's partials against its fixed scratch before any HIP call."""
    P = ctypes.c_void_p
    dummy = P(1 << 20)  # never dereferenced: every call below is rejected on the host
    cfg = _lib.MlaVerifyConfig(64, 576, 512, 16, 16, 32, 1 << 22, 0.072, 0, 0)  # batch16: 16 x 32 x 1024 rows
    assert lib.mla_verify_run_noalloc(ctypes.byref(cfg), dummy, dummy, dummy, dummy, dummy, dummy, dummy, 32,
                                      None) == _lib.MLA_ERR_SCRATCH_TOO_SMALL
    cfg = _lib.MlaVerifyConfig(64, 576, 512, 1, 16, 64, 1 << 21, 0.072, 0, 0)    # 1,024 rows at nsplit 40
    assert lib.mla_verify_run_noalloc(ctypes.byref(cfg), dummy, dummy, dummy, dummy, dummy, dummy, dummy, 40,
                                      None) == _lib.MLA_ERR_SCRATCH_TOO_SMALL
    assert lib.mla_verify_run_noalloc(ctypes.byref(cfg), dummy, dummy, dummy, dummy, dummy, dummy, dummy, 65,
                                      None) == _lib.MLA_ERR_INVALID_ARGUMENT       # nsplit > max_nsplit
    assert lib.mla_verify_run_noalloc(None, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 1,
                                      None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert _lib.error_string(_lib.MLA_ERR_SCRATCH_TOO_SMALL) == "MLA_ERR_SCRATCH_TOO_SMALL"
