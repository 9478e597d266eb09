"""The C-ABI library loads on a host without a GPU, exports every function
declared in include/*.h, and rejects bad arguments on the host before
touching a device (no compute calls here)."""
import ctypes
import os
import re

import pytest

from streaming_sinkhorn_solver_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE, h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(fs_[a-z_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.lib_path()):
        pytest.fail("libfs_sinkhorn.so is not built (run __graft_entry__.build())")
    return binding.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"fs_potentials_init", "fs_lse_update_f", "fs_lse_update_g", "fs_sinkhorn_solve",
            "fs_apply_transport", "fs_workspace_bytes", "fs_destroy",
            "fs_probe_peak"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_workspace_is_linear_in_points(lib):
    # O((n + m) d) working memory: doubling n and m roughly doubles the bytes.
    b1 = binding.fs_workspace_bytes(20_000, 20_000, 512, 512, "bf16")
    b2 = binding.fs_workspace_bytes(40_000, 40_000, 512, 512, "bf16")
    assert 1.8 < b2 / b1 < 2.2
    # never anywhere near an n x m buffer
    assert b2 < 40_000 * 40_000
    assert binding.fs_workspace_bytes(250_000, 250_000, 3, 0, "auto") < 64 << 20


def test_host_argument_validation(lib):
    assert binding.fs_workspace_bytes(0, 10, 3) == 0
    assert binding.fs_workspace_bytes(10, 10, 0) == 0
    assert binding.fs_workspace_bytes(10, 10, 2000, 0, "bf16") == 0
    assert binding.fs_workspace_bytes(10, 10, 600, 0, "fp32") == 0
    assert "fp32 scores support d <= 512" in binding.fs_last_error()
    h = ctypes.c_void_p()
    st = lib.fs_potentials_init(None, None, None, None, 10, 10, 3, 0, 0, None, 0, None, None,
                                None, ctypes.byref(h))
    assert st == binding.FS_ERR_INVALID_ARG
    st = lib.fs_potentials_init(1, 1, 1, 1, 10, 10, 3, 0, 9, None, 0, None, None, None,
                                ctypes.byref(h))
    assert st == binding.FS_ERR_INVALID_ARG
    # misaligned / short workspace is reported before any device work
    st = lib.fs_potentials_init(256, 256, 256, 256, 10, 10, 3, 0, 0, 257, 1 << 20, None, None,
                                None, ctypes.byref(h))
    assert st == binding.FS_ERR_WORKSPACE
    st = lib.fs_potentials_init(256, 256, 256, 256, 10, 10, 3, 0, 0, 512, 16, None, None, None,
                                ctypes.byref(h))
    assert st == binding.FS_ERR_WORKSPACE
    assert lib.fs_sinkhorn_solve(None, None, None, None, None, None) == binding.FS_ERR_INVALID_ARG
    assert binding.fs_status_string(4) == "FS_ERR_NONFINITE"


def test_no_device_is_reported_not_crashed(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    need = binding.fs_workspace_bytes(10, 10, 3)
    h = ctypes.c_void_p()
    st = lib.fs_potentials_init(256, 256, 256, 256, 10, 10, 3, 0, 0, 4096, need, None, None,
                                None, ctypes.byref(h))
    assert st == binding.FS_ERR_DEVICE


def test_probe_argument_validation(lib):
    rate = ctypes.c_double()
    # bad kind, bad repetition count, NULL sink: rejected before any device call
    assert lib.fs_probe_peak(0, 16, 3, None, ctypes.byref(rate)) == binding.FS_ERR_INVALID_ARG
    assert lib.fs_probe_peak(5, 16, 3, None, ctypes.byref(rate)) == binding.FS_ERR_INVALID_ARG
    assert lib.fs_probe_peak(1, 16, 0, None, ctypes.byref(rate)) == binding.FS_ERR_INVALID_ARG
    assert lib.fs_probe_peak(1, 16, 65, None, ctypes.byref(rate)) == binding.FS_ERR_INVALID_ARG
    assert lib.fs_probe_peak(1, None, 3, None, ctypes.byref(rate)) == binding.FS_ERR_INVALID_ARG
    assert lib.fs_probe_peak(1, 16, 3, None, None) == binding.FS_ERR_INVALID_ARG
