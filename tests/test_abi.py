"""The C-ABI library loads and exports every symbol include/hgb.h declares.

CPU only: nothing here launches a kernel.  (hgb_available may be called: it
only counts devices.)
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hgb.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(hgb_[a-z_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_five_verbs():
    names = declared_symbols()
    for verb in ("upload_bins", "begin_tree", "build_level", "subtract_siblings", "find_splits"):
        assert f"hgb_{verb}" in names


def test_library_exports_every_declared_symbol():
    from histogram_gradient_boosted_amd import binding
    path = binding.lib_path()
    if not os.path.exists(path):
        pytest.fail(f"{path} not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    missing = [s for s in declared_symbols() if not hasattr(lib, s)]
    assert not missing, missing
    assert set(binding.EXPORTED) == set(declared_symbols())


def test_split_record_layout_matches_header():
    from histogram_gradient_boosted_amd import binding
    assert binding.SPLIT_DTYPE.itemsize == binding.SPLIT_BYTES == 56
    text = open(HEADER).read()
    assert "56 bytes" in text


def test_binding_raises_without_device_instead_of_falling_back():
    """On a host without a device the binding must fail loudly, not compute."""
    from histogram_gradient_boosted_amd import binding
    binding.load()
    if binding.available():
        pytest.skip("a device is present")
    with pytest.raises(Exception):
        binding.Context(0)


def test_lds_rate_microbenchmark_exports_its_entry():
    """bench.py reports the LDS atomic ceiling from this library."""
    path = os.path.join(ROOT, "histogram_gradient_boosted_amd", "liblds_rate.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "lds_rate_measure")
    fn = lib.lds_rate_measure
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                   ctypes.POINTER(ctypes.c_int)]
    r, n = ctypes.c_double(0), ctypes.c_int(0)
    # argument checks return before any device call
    assert fn(0, 7, 1, ctypes.byref(r), ctypes.byref(n)) == 1
    assert fn(0, 0, 3, ctypes.byref(r), ctypes.byref(n)) == 1
