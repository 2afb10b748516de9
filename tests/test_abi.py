"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashsampling.h")
LIB = os.path.join(ROOT, "lm_head_matmul_amd", "libflashsampling.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fs_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        # the build script by path: importing the package would load the library
        import importlib.util

        spec = importlib.util.spec_from_file_location("_fs_lib_build", os.path.join(ROOT, "lm_head_matmul_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ["fs_create", "fs_destroy", "fs_last_error", "fs_fmms_tiling", "fs_fmms_sample",
                     "fs_fmms_sample_multi", "fs_unfused_sample", "fs_softmax_sample", "fs_group_summaries", "fs_group_summary", "fs_group_combine", "fs_debug_philox",
                     "fs_debug_gumbel_bits", "fs_debug_gumbel_scan"]:
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_signatures_cover_the_header():
    from lm_head_matmul_amd import binding

    assert sorted(binding.SIGNATURES) == declared_functions()


def test_null_context_is_rejected(lib):
    from lm_head_matmul_amd import binding

    L = binding.load_library()
    rc = L.fs_fmms_sample(None, None, None, 0, None, 0, 1, 8, 16, 1.0, 0, 0, None, 0, 0, None, None, None, 0)
    assert rc == binding.FS_ERR_INVALID_ARG
    assert b"ctx" in L.fs_last_error()
    assert L.fs_fmms_sample_multi(None, None, None, 0, None, 0, 1, 8, 16, 1.0, 0, 0, None, 0, 2, None, 0) == \
        binding.FS_ERR_INVALID_ARG
    assert L.fs_group_combine(None, None, None, 1, 1, 0, 0, 0, None) == binding.FS_ERR_INVALID_ARG
    assert L.fs_debug_gumbel_scan(None, None, None) == binding.FS_ERR_INVALID_ARG


def test_create_validates_before_touching_the_device(lib):
    from lm_head_matmul_amd import binding

    L = binding.load_library()
    h = ctypes.c_void_p()
    assert L.fs_create(ctypes.byref(h), 0, 0, 100, 0) == binding.FS_ERR_INVALID_ARG
    assert L.fs_create(ctypes.byref(h), 0, 4, 2**31, 0) == binding.FS_ERR_INVALID_ARG
    assert L.fs_create(ctypes.byref(h), 0, 4, 100, -1) == binding.FS_ERR_INVALID_ARG
    assert h.value is None
    L.fs_destroy(None)  # NULL is ignored
