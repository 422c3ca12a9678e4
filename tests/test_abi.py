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


def declared_prototypes():
    """{name: (return type, [parameter types])} of every function the header
    declares, with comments removed, parameter names dropped and whitespace
    normalised ("const int64_t*", "hgb_ctx**", ...)."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)   # preprocessor lines
    protos = {}
    for m in re.finditer(r"([A-Za-z_][\w\s\*]*?)\b(hgb_[a-z_]+)\s*\(([^)]*)\)\s*;", text):
        ret = norm_type(m.group(1))
        params = []
        for p in m.group(3).split(","):
            p = p.strip()
            if p == "void" or not p:
                continue
            # drop the parameter's name: the last identifier
            p = re.sub(r"\b[A-Za-z_]\w*\s*$", "", p)
            params.append(norm_type(p))
        protos[m.group(2)] = (ret, params)
    return protos


def norm_type(t):
    t = re.sub(r"\s+", " ", t.strip())
    t = re.sub(r"\s*\*\s*", "*", t)
    return t.strip()


# The boundary's calls with their argument types, as the contract states them:
# the context calls, then the five verbs (upload the bins, start a tree from
# its gradients, build a level, derive siblings by subtraction, find splits).
CONTRACT = {
    "hgb_available": ("int", []),
    "hgb_create": ("hgb_status", ["int", "void*", "hgb_ctx**"]),
    "hgb_destroy": ("void", ["hgb_ctx*"]),
    "hgb_last_error": ("const char*", ["const hgb_ctx*"]),
    "hgb_upload_bins": ("hgb_status", ["hgb_ctx*", "const void*", "int", "int", "int32_t", "int32_t",
                                       "int32_t", "int32_t"]),
    "hgb_begin_tree": ("hgb_status", ["hgb_ctx*", "const float*", "const float*"]),
    "hgb_get_scales": ("hgb_status", ["const hgb_ctx*", "int32_t*", "int32_t*"]),
    "hgb_build_level": ("hgb_status", ["hgb_ctx*", "const int32_t*", "const int32_t*", "int32_t",
                                       "int64_t*", "const int32_t*"]),
    "hgb_subtract_siblings": ("hgb_status", ["hgb_ctx*", "const int64_t*", "int64_t*", "const uint8_t*",
                                             "int32_t"]),
    "hgb_find_splits": ("hgb_status", ["hgb_ctx*", "const int64_t*", "int32_t", "double", "double",
                                       "hgb_split*"]),
}


def test_header_declares_the_five_verbs():
    names = declared_symbols()
    for verb in ("upload_bins", "begin_tree", "build_level", "subtract_siblings", "find_splits"):
        assert f"hgb_{verb}" in names


@pytest.mark.parametrize("name", sorted(CONTRACT))
def test_header_prototype_matches_the_contract(name):
    """A caller written to the contract's prototypes links and passes its
    arguments in the declared slots: return and parameter types match."""
    protos = declared_prototypes()
    assert name in protos, f"{name} is not declared"
    assert protos[name] == CONTRACT[name], f"{name}: header {protos[name]} vs contract {CONTRACT[name]}"


def test_prototype_parser_sees_every_declaration():
    """The prototype parser and the symbol scan agree (no declaration missed)."""
    assert sorted(declared_prototypes()) == declared_symbols()


def test_status_codes_and_split_fields_match_the_contract():
    text = open(HEADER).read()
    codes = dict((k, int(v)) for k, v in re.findall(r"\b(HGB_(?:OK|E_[A-Z]+))\s*=\s*(\d+)", text))
    assert codes == {"HGB_OK": 0, "HGB_E_INVALID": 1, "HGB_E_STATE": 2, "HGB_E_UNSUPPORTED": 3,
                     "HGB_E_NONFINITE": 4, "HGB_E_DEVICE": 5}
    body = re.search(r"typedef struct \{(.*?)\} hgb_split;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(\w+)\s+(\w+);", body)
    assert fields[:4] == [("int32_t", "feature"), ("int32_t", "bin"), ("int32_t", "default_left"),
                          ("int32_t", "pad")]
    assert fields[4] == ("double", "gain")
    assert [f for _, f in fields[5:]] == ["g_left", "h_left", "g_total", "h_total"]
    assert all(t == "int64_t" for t, _ in fields[5:])


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
