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
