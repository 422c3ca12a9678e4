"""Serial CPU oracle for the level histogram build (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke entry
point and the benchmark's CPU-baseline leg may import this package.  It shares
no code with the HIP library (histogram_gradient_boosted_amd); the product
path never imports it.

Functions mirror the steps of the method (see oracle.c for the passages each
one restates): quantize, check_bins, build_hist, subtract, find_splits,
find_level_split, partition, objective (with its exp).  All arrays are numpy arrays on the host.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")
# ORACLE_SANITIZE=1: build and load a copy instrumented with the address and
# undefined-behaviour sanitizers (the process must preload the ASan runtime;
# tests/test_sanitizers.py runs the oracle's tests that way).
_SANITIZE = os.environ.get("ORACLE_SANITIZE", "") == "1"
if _SANITIZE:
    _LIB = os.path.join(_HERE, "liboracle_san.so")

OK = 0
E_INVALID = 1
E_NONFINITE = 4

OBJ_SQUARED = 0
OBJ_LOGISTIC = 1
OBJ_POISSON = 2
OBJECTIVES = {"squared": OBJ_SQUARED, "logistic": OBJ_LOGISTIC, "poisson": OBJ_POISSON}

SPLIT_DTYPE = np.dtype([
    ("feature", "<i4"), ("bin", "<i4"), ("default_left", "<i4"), ("pad", "<i4"),
    ("gain", "<f8"),
    ("g_left", "<i8"), ("h_left", "<i8"), ("g_total", "<i8"), ("h_total", "<i8"),
])
assert SPLIT_DTYPE.itemsize == 56


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: oracle status {status}")
        self.status = status


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (serial, no FMA contraction)."""
    stale = (not os.path.exists(_LIB)
             or os.path.getmtime(_LIB) < max(os.path.getmtime(_SRC), os.path.getmtime(_HDR)))
    if force or stale:
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        if _SANITIZE:
            cmd[1:1] = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.oracle_quantize.argtypes = [vp, i64, ctypes.c_int, i32, vp, vp]
        lib.oracle_quantize.restype = ctypes.c_int
        lib.oracle_check_bins.argtypes = [vp, ctypes.c_int, i64, i32, i32, i32]
        lib.oracle_check_bins.restype = ctypes.c_int
        lib.oracle_build_hist.argtypes = [vp, ctypes.c_int, i64, i32, i32, i32,
                                          vp, vp, vp, vp, i32, vp]
        lib.oracle_build_hist.restype = None
        lib.oracle_subtract.argtypes = [vp, vp, vp, i32, i64]
        lib.oracle_subtract.restype = None
        lib.oracle_find_splits.argtypes = [vp, i32, i32, i32, i32, i32, i32,
                                           ctypes.c_double, ctypes.c_double, vp]
        lib.oracle_find_splits.restype = None
        lib.oracle_partition.argtypes = [vp, ctypes.c_int, i64, i32, vp, vp, i32,
                                         vp, vp, vp]
        lib.oracle_partition.restype = i32
        lib.oracle_find_level_split.argtypes = [vp, i32, i32, i32, i32, i32, i32,
                                                ctypes.c_double, ctypes.c_double, vp]
        lib.oracle_find_level_split.restype = None
        lib.oracle_exp_array.argtypes = [vp, i64, vp]
        lib.oracle_exp_array.restype = None
        lib.oracle_objective.argtypes = [i32, vp, vp, vp, i64, vp, vp]
        lib.oracle_objective.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bins_arg(bins):
    bins = np.ascontiguousarray(bins)
    if bins.dtype == np.uint8:
        return bins, 1
    if bins.dtype == np.uint16:
        return bins, 2
    raise TypeError("bins must be uint8 or uint16")


def quantize(c, require_nonneg: bool, bits: int = 30):
    """Fixed-point encode one component at `bits` of precision.  Returns (q int32 [n], k)."""
    c = np.ascontiguousarray(c, dtype=np.float32)
    q = np.empty(c.shape[0], dtype=np.int32)
    k = ctypes.c_int32(0)
    st = _load().oracle_quantize(_ptr(c), c.shape[0], int(bool(require_nonneg)), int(bits),
                                 _ptr(q), ctypes.byref(k))
    if st != OK:
        raise OracleError(st, "quantize")
    return q, int(k.value)


def check_bins(bins, n_bins: int, has_missing: bool) -> int:
    bins, w = _bins_arg(bins)
    F, n = bins.shape
    return int(_load().oracle_check_bins(_ptr(bins), w, n, F, n_bins, int(has_missing)))


def n_slots(n_bins: int, has_missing: bool) -> int:
    return n_bins + (1 if has_missing else 0)


def build_hist(bins, n_bins: int, has_missing: bool, qg, qh,
               row_index=None, node_offsets=None):
    """Histograms [n_nodes][F][S][2] int64 of the given nodes (root if row_index is None)."""
    bins, w = _bins_arg(bins)
    F, n = bins.shape
    qg = np.ascontiguousarray(qg, dtype=np.int32)
    qh = np.ascontiguousarray(qh, dtype=np.int32)
    if row_index is None:
        n_nodes = 1
        ri = None
        no = None
    else:
        ri = np.ascontiguousarray(row_index, dtype=np.int32)
        no = np.ascontiguousarray(node_offsets, dtype=np.int64)
        n_nodes = no.shape[0] - 1
    S = n_slots(n_bins, has_missing)
    hist = np.empty((n_nodes, F, S, 2), dtype=np.int64)
    _load().oracle_build_hist(_ptr(bins), w, n, F, n_bins, int(has_missing),
                              _ptr(qg), _ptr(qh), _ptr(ri), _ptr(no), n_nodes, _ptr(hist))
    return hist


def subtract(parent, child, built_is_right):
    """In place: child[2i + 1 - r] = parent[i] - child[2i + r], r = built_is_right[i]."""
    parent = np.ascontiguousarray(parent, dtype=np.int64)
    assert child.dtype == np.int64 and child.flags.c_contiguous
    bir = np.ascontiguousarray(built_is_right, dtype=np.uint8)
    P = parent.shape[0]
    assert child.shape[0] == 2 * P and bir.shape[0] == P
    node_elems = int(np.prod(parent.shape[1:]))
    _load().oracle_subtract(_ptr(parent), _ptr(child), _ptr(bir), P, node_elems)
    return child


def find_splits(hist, n_bins: int, has_missing: bool, k_g: int, k_h: int,
                lam: float = 1.0, gamma: float = 0.0):
    hist = np.ascontiguousarray(hist, dtype=np.int64)
    N, F, S, two = hist.shape
    assert two == 2 and S == n_slots(n_bins, has_missing)
    out = np.zeros(N, dtype=SPLIT_DTYPE)
    _load().oracle_find_splits(_ptr(hist), N, F, n_bins, int(has_missing),
                               int(k_g), int(k_h), float(lam), float(gamma), _ptr(out))
    return out


def find_level_split(hist, n_bins: int, has_missing: bool, k_g: int, k_h: int,
                     lam: float = 1.0, gamma: float = 0.0):
    """Oblivious level split: n_nodes + 1 records (per node, then the level)."""
    hist = np.ascontiguousarray(hist, dtype=np.int64)
    N, F, S, two = hist.shape
    assert two == 2 and S == n_slots(n_bins, has_missing)
    out = np.zeros(N + 1, dtype=SPLIT_DTYPE)
    _load().oracle_find_level_split(_ptr(hist), N, F, n_bins, int(has_missing),
                                    int(k_g), int(k_h), float(lam), float(gamma), _ptr(out))
    return out


def partition(bins, n_bins: int, row_index, node_offsets, splits):
    """Children row lists of the split nodes.  Returns (row_index, node_offsets)."""
    bins, w = _bins_arg(bins)
    F, n = bins.shape
    if row_index is None:
        ri, no, n_nodes, total = None, None, 1, n
    else:
        ri = np.ascontiguousarray(row_index, dtype=np.int32)
        no = np.ascontiguousarray(node_offsets, dtype=np.int64)
        n_nodes = no.shape[0] - 1
        total = int(no[-1])
    splits = np.ascontiguousarray(splits, dtype=SPLIT_DTYPE)
    assert splits.shape[0] == n_nodes
    out_ri = np.empty(total, dtype=np.int32)
    out_no = np.zeros(2 * n_nodes + 1, dtype=np.int64)
    nc = _load().oracle_partition(_ptr(bins), w, n, n_bins, _ptr(ri), _ptr(no), n_nodes,
                                  _ptr(splits), _ptr(out_ri), _ptr(out_no))
    out_no = out_no[: nc + 1].copy()
    return out_ri[: int(out_no[-1])].copy(), out_no


def exp(x):
    """The oracle's own exp (Cody-Waite reduction, degree-13 Taylor), elementwise, f64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    _load().oracle_exp_array(_ptr(x), x.size, _ptr(out))
    return out


def objective(kind, margin, label, weight=None):
    """(grad, hess) fp32 [n] of loss `kind` ("squared", "logistic", "poisson" or
    its code) at scores `margin` for labels `label`, optionally weighted."""
    code = OBJECTIVES[kind] if isinstance(kind, str) else int(kind)
    m = np.ascontiguousarray(margin, dtype=np.float32)
    y = np.ascontiguousarray(label, dtype=np.float32)
    w = None if weight is None else np.ascontiguousarray(weight, dtype=np.float32)
    assert y.shape == m.shape and (w is None or w.shape == m.shape)
    g = np.empty(m.shape[0], dtype=np.float32)
    h = np.empty(m.shape[0], dtype=np.float32)
    st = _load().oracle_objective(code, _ptr(m), _ptr(y), _ptr(w), m.shape[0], _ptr(g), _ptr(h))
    if st != OK:
        raise OracleError(st, "objective")
    return g, h
