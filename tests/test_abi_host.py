"""Host-only checks of the C ABI library: it builds, loads and exports every
function that include/specverify.h declares; host-side argument checks that
return before touching the device."""
import ctypes
import os
import re

import pytest

from rejection_sampling_verifier_specverify_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "specverify.h")).read()
    return sorted(set(re.findall(r"\b(specverify_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = binding.load_library()
    declared = _declared()
    assert set(declared) >= set(binding.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_struct_layouts_match_header():
    # sizes of the C structs on x86-64 (int32 fields, 8-byte pointers/int64)
    assert ctypes.sizeof(binding.Config) == 24
    assert ctypes.sizeof(binding.Inputs) == 8 + 8 + 8 + 8 + 8 + 8 + 8 + 8 + 8 + 8
    assert ctypes.sizeof(binding.Outputs) == 48
    assert ctypes.sizeof(binding.CommitArgs) == 88


def test_null_arguments_rejected_without_device():
    lib = binding.load_library()
    assert lib.specverify_run(None, None, None, None) == binding.ERR_INVALID_ARGUMENT
    assert lib.specverify_commit(None, None, None) == binding.ERR_INVALID_ARGUMENT
    assert lib.specverify_destroy(None) == binding.OK
    assert lib.specverify_chunks_per_row(None) == 0
    h = ctypes.c_void_p()
    assert lib.specverify_create(None, ctypes.byref(h)) == binding.ERR_INVALID_ARGUMENT
    bad = binding.Config(0, 4, 1000, binding.BF16, 0, 0)          # max_batch 0
    assert lib.specverify_create(ctypes.byref(bad), ctypes.byref(h)) == binding.ERR_INVALID_ARGUMENT
    assert not h.value
    bad = binding.Config(1, 4, 1000, 7, 0, 0)                      # unknown dtype
    assert lib.specverify_create(ctypes.byref(bad), ctypes.byref(h)) == binding.ERR_INVALID_ARGUMENT
    # more than 256 fp32 or 128 bf16 chunks of 4 KB
    for V, dt in ((262144 + 1, binding.F32), (262144 + 1, binding.BF16)):
        bad = binding.Config(1, 4, V, dt, 0, 0)
        assert lib.specverify_create(ctypes.byref(bad), ctypes.byref(h)) == binding.ERR_UNSUPPORTED


def test_static_run_checks_its_config_without_device():
    """specverify_run_static checks its configuration as create does, before
    touching a device."""
    lib = binding.load_library()
    assert lib.specverify_run_static(None, None, None, None) == binding.ERR_INVALID_ARGUMENT
    bad = binding.Config(0, 4, 1000, binding.BF16, 0, 0)          # max_batch 0
    assert lib.specverify_run_static(ctypes.byref(bad), None, None, None) == binding.ERR_INVALID_ARGUMENT
    bad = binding.Config(1, 4, 262144 + 1, binding.BF16, 0, 0)     # more than 128 bf16 chunks
    assert lib.specverify_run_static(ctypes.byref(bad), None, None, None) == binding.ERR_UNSUPPORTED


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        binding.load_library(str(tmp_path / "nope.so"))


def test_create_without_a_device_fails_cleanly():
    """On a host with no GPU, create returns SPECVERIFY_ERR_DEVICE, leaves the
    handle NULL and does not crash (a failure the caller can handle)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    lib = binding.load_library()
    h = ctypes.c_void_p(12345)
    cfg = binding.Config(4, 4, 32000, binding.F32, 0, 0)
    assert lib.specverify_create(ctypes.byref(cfg), ctypes.byref(h)) == binding.ERR_DEVICE
    assert not h.value
    with pytest.raises(binding.SpecVerifyError) as e:
        binding.SpecVerify(max_batch=4, max_gamma=4, vocab=32000, dtype="f32")
    assert e.value.status == binding.ERR_DEVICE
    # the allocation-free run fails the same way, before reading its inputs
    assert lib.specverify_run_static(ctypes.byref(cfg), None, None, None) == binding.ERR_DEVICE
