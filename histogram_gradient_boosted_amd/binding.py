"""Thin ctypes binding over libhgb.so (include/hgb.h).

Argument marshalling only: torch tensors carry device memory and the stream;
every step of the computation runs in the library's HIP kernels.  The binding
checks what the C ABI cannot see -- tensor devices, dtypes, contiguity and
buffer sizes -- so that no kernel is ever handed a buffer too small for it.
There is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhgb.so")

HGB_OK, HGB_E_INVALID, HGB_E_STATE, HGB_E_UNSUPPORTED, HGB_E_NONFINITE, HGB_E_DEVICE = range(6)
_STATUS_NAMES = {0: "HGB_OK", 1: "HGB_E_INVALID", 2: "HGB_E_STATE", 3: "HGB_E_UNSUPPORTED",
                 4: "HGB_E_NONFINITE", 5: "HGB_E_DEVICE"}
MAX_SLOTS = 4096

# hgb_split, 56 bytes
SPLIT_DTYPE = np.dtype([
    ("feature", "<i4"), ("bin", "<i4"), ("default_left", "<i4"), ("pad", "<i4"),
    ("gain", "<f8"),
    ("g_left", "<i8"), ("h_left", "<i8"), ("g_total", "<i8"), ("h_total", "<i8"),
])
SPLIT_BYTES = 56

EXPORTED = ("hgb_available", "hgb_create", "hgb_destroy", "hgb_last_error", "hgb_sync",
            "hgb_upload_bins", "hgb_begin_tree", "hgb_get_scales", "hgb_build_level",
            "hgb_subtract_siblings", "hgb_subtract_siblings_slots", "hgb_find_splits",
            "hgb_profile_enable",
            "hgb_profile_query", "hgb_set_precision", "hgb_partition_level",
            "hgb_subtract_find_splits", "hgb_begin_tree_objective", "hgb_copy_quantized",
            "hgb_find_level_split", "hgb_find_splits_noalloc", "hgb_set_async_begin",
            "hgb_grow_level")

# hgb_objective
OBJECTIVES = {"squared": 0, "logistic": 1, "poisson": 2}

KERNELS = {"quantize": 0, "gather": 1, "zero": 2, "fill": 3, "subtract": 4, "split": 5,
           "partition": 6, "fill_root": 7, "fill_level": 8, "merge": 9}


class HGBError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libhgb.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: run __graft_entry__.build() "
                          "(or python -m histogram_gradient_boosted_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, c_int = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    lib.hgb_available.argtypes = []
    lib.hgb_available.restype = c_int
    lib.hgb_create.argtypes = [c_int, vp, ctypes.POINTER(vp)]
    lib.hgb_create.restype = c_int
    lib.hgb_destroy.argtypes = [vp]
    lib.hgb_destroy.restype = None
    lib.hgb_last_error.argtypes = [vp]
    lib.hgb_last_error.restype = ctypes.c_char_p
    lib.hgb_sync.argtypes = [vp]
    lib.hgb_sync.restype = c_int
    lib.hgb_upload_bins.argtypes = [vp, vp, c_int, c_int, i32, i32, i32, i32]
    lib.hgb_upload_bins.restype = c_int
    lib.hgb_begin_tree.argtypes = [vp, vp, vp]
    lib.hgb_begin_tree.restype = c_int
    lib.hgb_begin_tree_objective.argtypes = [vp, i32, vp, vp, vp]
    lib.hgb_begin_tree_objective.restype = c_int
    lib.hgb_copy_quantized.argtypes = [vp, vp]
    lib.hgb_copy_quantized.restype = c_int
    lib.hgb_set_async_begin.argtypes = [vp, c_int]
    lib.hgb_set_async_begin.restype = c_int
    lib.hgb_set_precision.argtypes = [vp, i32]
    lib.hgb_set_precision.restype = c_int
    lib.hgb_get_scales.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.hgb_get_scales.restype = c_int
    lib.hgb_build_level.argtypes = [vp, vp, vp, i32, vp, vp]
    lib.hgb_build_level.restype = c_int
    lib.hgb_subtract_siblings.argtypes = [vp, vp, vp, vp, i32]
    lib.hgb_subtract_siblings.restype = c_int
    lib.hgb_subtract_siblings_slots.argtypes = [vp, vp, vp, vp, vp, i32]
    lib.hgb_subtract_siblings_slots.restype = c_int
    lib.hgb_find_splits.argtypes = [vp, vp, i32, ctypes.c_double, ctypes.c_double, vp]
    lib.hgb_find_splits.restype = c_int
    lib.hgb_find_splits_noalloc.argtypes = [vp, vp, i32, ctypes.c_double, ctypes.c_double, vp]
    lib.hgb_find_splits_noalloc.restype = c_int
    lib.hgb_find_level_split.argtypes = [vp, vp, i32, ctypes.c_double, ctypes.c_double, vp]
    lib.hgb_find_level_split.restype = c_int
    lib.hgb_partition_level.argtypes = [vp, vp, vp, i32, vp, vp, vp, ctypes.POINTER(i32), vp]
    lib.hgb_partition_level.restype = c_int
    lib.hgb_subtract_find_splits.argtypes = [vp, vp, vp, vp, vp, i32, ctypes.c_double,
                                             ctypes.c_double, vp]
    lib.hgb_subtract_find_splits.restype = c_int
    lib.hgb_grow_level.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, ctypes.POINTER(i32), vp, vp,
                                   ctypes.POINTER(ctypes.c_int64), ctypes.c_double, ctypes.c_double, i32]
    lib.hgb_grow_level.restype = c_int
    lib.hgb_profile_enable.argtypes = [vp, c_int]
    lib.hgb_profile_enable.restype = c_int
    lib.hgb_profile_query.argtypes = [vp, c_int, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64)]
    lib.hgb_profile_query.restype = c_int
    _lib = lib
    return lib


def available() -> bool:
    """hgb_available(): a usable HIP device is present."""
    return bool(load().hgb_available())


def _i32_host(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def splits_to_numpy(t) -> np.ndarray:
    """View a uint8 tensor/array of N*56 bytes (hgb_split records) as a record array."""
    import torch
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().numpy()
    return np.frombuffer(np.ascontiguousarray(t).tobytes(), dtype=SPLIT_DTYPE)


class Context:
    """One hgb_ctx: resident bins, the current tree's fixed-point (g, h), scratch.

    stream: a torch.cuda.Stream (default: the current stream of `device`)."""

    def __init__(self, device: int = 0, stream=None):
        import torch
        self._torch = torch
        self._lib = load()
        self.device = int(device)
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        self.stream = stream
        h = ctypes.c_void_p()
        st = self._lib.hgb_create(self.device, ctypes.c_void_p(stream.cuda_stream), ctypes.byref(h))
        if st != HGB_OK:
            raise HGBError(st, "hgb_create failed")
        self._h = h
        self.n_rows = self.n_features = self.n_bins = self.n_slots = 0
        self.has_missing = False

    # -- plumbing ---------------------------------------------------------
    def _check(self, st: int, what: str):
        if st != HGB_OK:
            msg = self._lib.hgb_last_error(self._h)
            raise HGBError(st, f"{what}: {msg.decode() if msg else ''}")

    def _dev(self, t, name, dtype=None, numel=None):
        torch = self._torch
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.device.index != self.device:
            raise ValueError(f"{name} must be a CUDA tensor on device {self.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if numel is not None and t.numel() < numel:
            raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
        return ctypes.c_void_p(t.data_ptr())

    @property
    def node_elems(self) -> int:
        return self.n_features * self.n_slots * 2

    def close(self):
        if getattr(self, "_h", None):
            self._lib.hgb_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def sync(self):
        self._check(self._lib.hgb_sync(self._h), "sync")

    def profile_enable(self, on: bool = True):
        self._check(self._lib.hgb_profile_enable(self._h, int(bool(on))), "profile_enable")

    def profile_query(self, kernel: str):
        """(total device ms, launches) of a kernel class since the last reset."""
        ms, n = ctypes.c_double(), ctypes.c_int64()
        self._check(self._lib.hgb_profile_query(self._h, KERNELS[kernel], ctypes.byref(ms),
                                                ctypes.byref(n)), "profile_query")
        return float(ms.value), int(n.value)

    # -- the five verbs ---------------------------------------------------
    def upload_bins(self, bins, n_bins: int, has_missing: bool):
        """bins: [F][n] uint8/uint16 numpy array (host) or 1-/2-byte CUDA tensor."""
        torch = self._torch
        if isinstance(bins, torch.Tensor):
            if bins.element_size() not in (1, 2) or bins.dim() != 2:
                raise ValueError("bins tensor must be 2-D with 1- or 2-byte elements")
            ptr = self._dev(bins, "bins")
            w, on_dev = bins.element_size(), 1
            F, n = bins.shape
            keep = bins
        else:
            keep = np.ascontiguousarray(bins)
            if keep.dtype not in (np.uint8, np.uint16) or keep.ndim != 2:
                raise ValueError("bins array must be 2-D uint8 or uint16")
            ptr = ctypes.c_void_p(keep.ctypes.data)
            w, on_dev = keep.dtype.itemsize, 0
            F, n = keep.shape
        self._check(self._lib.hgb_upload_bins(self._h, ptr, w, on_dev, int(n), int(F),
                                              int(n_bins), int(bool(has_missing))), "upload_bins")
        del keep
        self.n_rows, self.n_features, self.n_bins = int(n), int(F), int(n_bins)
        self.has_missing = bool(has_missing)
        self.n_slots = self.n_bins + (1 if self.has_missing else 0)

    def begin_tree(self, grad, hess):
        torch = self._torch
        g = self._dev(grad, "grad", torch.float32, self.n_rows)
        h = self._dev(hess, "hess", torch.float32, self.n_rows)
        self._check(self._lib.hgb_begin_tree(self._h, g, h), "begin_tree")

    def begin_tree_objective(self, objective, margin, label, weight=None):
        """Start a tree from (g, h) that the library derives on the device from
        scores `margin` and labels `label` (and optional weights), for loss
        `objective` ("squared", "logistic", "poisson" or its hgb_objective code)."""
        torch = self._torch
        code = OBJECTIVES[objective] if isinstance(objective, str) else int(objective)
        m = self._dev(margin, "margin", torch.float32, self.n_rows)
        y = self._dev(label, "label", torch.float32, self.n_rows)
        w = None if weight is None else self._dev(weight, "weight", torch.float32, self.n_rows)
        self._check(self._lib.hgb_begin_tree_objective(self._h, code, m, y, w),
                    "begin_tree_objective")

    def copy_quantized(self, out=None):
        """The current tree's (qg, qh) pairs as an int32 [n_rows, 2] CUDA tensor."""
        torch = self._torch
        if out is None:
            out = torch.empty((self.n_rows, 2), dtype=torch.int32, device=f"cuda:{self.device}")
        q = self._dev(out, "out", torch.int32, 2 * self.n_rows)
        self._check(self._lib.hgb_copy_quantized(self._h, q), "copy_quantized")
        return out

    def set_async_begin(self, on: bool = True):
        """begin_tree without waiting for the maxima; a non-finite value is
        then reported by the next sync()."""
        self._check(self._lib.hgb_set_async_begin(self._h, int(bool(on))), "set_async_begin")

    def set_precision(self, bits: int):
        """Fixed-point precision (bits below the largest |value|) of the next begin_tree."""
        self._check(self._lib.hgb_set_precision(self._h, int(bits)), "set_precision")

    def get_scales(self):
        kg, kh = ctypes.c_int32(), ctypes.c_int32()
        self._check(self._lib.hgb_get_scales(self._h, ctypes.byref(kg), ctypes.byref(kh)),
                    "get_scales")
        return int(kg.value), int(kh.value)

    def build_level(self, hist, row_index=None, node_offsets=None, out_slot=None):
        """Histograms of a level's nodes into `hist` ([slots][F][S][2] int64 CUDA tensor)."""
        torch = self._torch
        if row_index is None:
            n_nodes = 1
            offs = None
            ri = None
        else:
            offs = _i32_host(node_offsets)
            n_nodes = int(offs.shape[0]) - 1
            ri = self._dev(row_index, "row_index", torch.int32, int(offs[-1]) if n_nodes >= 0 else 0)
        slots = None if out_slot is None else _i32_host(out_slot)
        top = (int(slots.max()) + 1) if slots is not None and slots.size else n_nodes
        hp = self._dev(hist, "hist", torch.int64, top * self.node_elems)
        self._check(self._lib.hgb_build_level(
            self._h, ri,
            None if offs is None else offs.ctypes.data_as(ctypes.c_void_p), n_nodes, hp,
            None if slots is None else slots.ctypes.data_as(ctypes.c_void_p)), "build_level")

    def subtract_siblings(self, parent, child, built_is_right, parent_slot=None):
        """child[2i + 1 - r] = parent[parent_slot[i]] - child[2i + r], r = built_is_right[i]
        (parent_slot None: parent[i], through the five-argument hgb_subtract_siblings)."""
        torch = self._torch
        bir = np.ascontiguousarray(np.asarray(built_is_right), dtype=np.uint8)
        P = int(bir.shape[0])
        ps = None if parent_slot is None else _i32_host(parent_slot)
        if ps is not None and ps.shape[0] != P:
            raise ValueError("parent_slot must have one entry per pair")
        ptop = (int(ps.max()) + 1) if ps is not None and P else P
        pp = self._dev(parent, "parent", torch.int64, ptop * self.node_elems)
        cp = self._dev(child, "child", torch.int64, 2 * P * self.node_elems)
        if ps is None:   # the five-argument verb: pair i's parent at slot i
            self._check(self._lib.hgb_subtract_siblings(
                self._h, pp, cp, bir.ctypes.data_as(ctypes.c_void_p), P), "subtract_siblings")
        else:
            self._check(self._lib.hgb_subtract_siblings_slots(
                self._h, pp, cp, bir.ctypes.data_as(ctypes.c_void_p),
                ps.ctypes.data_as(ctypes.c_void_p), P), "subtract_siblings_slots")

    def subtract_find_splits(self, parent, child, built_is_right, lam: float, gamma: float, out,
                             parent_slot=None):
        """subtract_siblings then find_splits over the 2P children, in one pass."""
        torch = self._torch
        bir = np.ascontiguousarray(np.asarray(built_is_right), dtype=np.uint8)
        P = int(bir.shape[0])
        ps = None if parent_slot is None else _i32_host(parent_slot)
        if ps is not None and ps.shape[0] != P:
            raise ValueError("parent_slot must have one entry per pair")
        ptop = (int(ps.max()) + 1) if ps is not None and P else P
        pp = self._dev(parent, "parent", torch.int64, ptop * self.node_elems)
        cp = self._dev(child, "child", torch.int64, 2 * P * self.node_elems)
        op = self._dev(out, "out", torch.uint8, 2 * P * SPLIT_BYTES)
        self._check(self._lib.hgb_subtract_find_splits(
            self._h, pp, cp, bir.ctypes.data_as(ctypes.c_void_p),
            None if ps is None else ps.ctypes.data_as(ctypes.c_void_p), P, float(lam), float(gamma),
            op), "subtract_find_splits")

    def partition_level(self, splits, out_rows, row_index=None, node_offsets=None):
        """Children's rows of every split node into `out_rows` (int32 CUDA tensor).

        `splits`: the level's hgb_split records (uint8 CUDA tensor, as
        find_splits writes them).  Returns (children's offsets, parents): int32
        numpy arrays of 2c + 1 and c entries for c nodes with a split, parent j
        being the node whose children are 2j and 2j + 1."""
        torch = self._torch
        if row_index is None:
            n_nodes, offs, ri, total = 1, None, None, self.n_rows
        else:
            offs = _i32_host(node_offsets)
            n_nodes = int(offs.shape[0]) - 1
            total = int(offs[-1])
            ri = self._dev(row_index, "row_index", torch.int32, total)
        sp = self._dev(splits, "splits", torch.uint8, n_nodes * SPLIT_BYTES)
        op = self._dev(out_rows, "out_rows", torch.int32, total) if total else None
        child = np.zeros(2 * n_nodes + 1, dtype=np.int32)
        parent = np.zeros(n_nodes, dtype=np.int32)
        nc = ctypes.c_int32(0)
        self._check(self._lib.hgb_partition_level(
            self._h, ri, None if offs is None else offs.ctypes.data_as(ctypes.c_void_p), n_nodes,
            sp, op, child.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nc),
            parent.ctypes.data_as(ctypes.c_void_p)), "partition_level")
        return child[: nc.value + 1].copy(), parent[: nc.value // 2].copy()

    def grow_level(self, parent_hist, parent_splits, parent_rows, parent_offsets, child_rows, child_hist,
                   child_splits, lam: float, gamma: float, oblivious: bool = False):
        """One level in one call (hgb_grow_level): partition the parents' rows
        into `child_rows`, build the smaller child of each pair into
        `child_hist` (room for 2 * n_parents slots), derive the other and
        score every child into `child_splits` (depthwise splits, or with
        oblivious the level split: room for 2 * n_parents + 1 records).
        parent_rows / parent_offsets None: the root.  Returns (child offsets,
        built_is_right, parents, built rows) as numpy arrays and an int; no
        children (offsets [0]) ends the tree."""
        torch = self._torch
        if parent_rows is None:
            n_par, offs, pr, total = 1, None, None, self.n_rows
        else:
            offs = _i32_host(parent_offsets)
            n_par = int(offs.shape[0]) - 1
            total = int(offs[-1])
            pr = self._dev(parent_rows, "parent_rows", torch.int32, total)
        ph = self._dev(parent_hist, "parent_hist", torch.int64, n_par * self.node_elems)
        ps = self._dev(parent_splits, "parent_splits", torch.uint8, n_par * SPLIT_BYTES)
        cr = self._dev(child_rows, "child_rows", torch.int32, total) if total else None
        ch = self._dev(child_hist, "child_hist", torch.int64, 2 * n_par * self.node_elems)
        cs = self._dev(child_splits, "child_splits", torch.uint8, (2 * n_par + (1 if oblivious else 0)) * SPLIT_BYTES)
        child = np.zeros(2 * n_par + 1, dtype=np.int32)
        bir = np.zeros(n_par, dtype=np.uint8)
        parent = np.zeros(n_par, dtype=np.int32)
        nc = ctypes.c_int32(0)
        built = ctypes.c_int64(0)
        self._check(self._lib.hgb_grow_level(
            self._h, ph, ps, pr, None if offs is None else offs.ctypes.data_as(ctypes.c_void_p), n_par,
            cr, ch, cs, child.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nc),
            bir.ctypes.data_as(ctypes.c_void_p), parent.ctypes.data_as(ctypes.c_void_p), ctypes.byref(built),
            ctypes.c_double(lam), ctypes.c_double(gamma), 1 if oblivious else 0), "grow_level")
        P = nc.value // 2
        return child[: nc.value + 1].copy(), bir[:P].copy(), parent[:P].copy(), int(built.value)

    def find_level_split(self, hist, n_nodes: int, lam: float, gamma: float, out):
        """Oblivious level split.  out: uint8 CUDA tensor of at least
        (n_nodes + 1) * 56 bytes: the n_nodes node records, then the level's."""
        torch = self._torch
        hp = self._dev(hist, "hist", torch.int64, int(n_nodes) * self.node_elems)
        op = self._dev(out, "out", torch.uint8, (int(n_nodes) + 1) * SPLIT_BYTES)
        self._check(self._lib.hgb_find_level_split(self._h, hp, int(n_nodes), float(lam),
                                                   float(gamma), op), "find_level_split")

    def find_splits_noalloc(self, hist, n_nodes: int, lam: float, gamma: float, out):
        """find_splits with its scratch in the library's fixed per-device array
        (no allocation in the call); out as for find_splits."""
        torch = self._torch
        hp = self._dev(hist, "hist", torch.int64, int(n_nodes) * self.node_elems)
        op = self._dev(out, "out", torch.uint8, int(n_nodes) * SPLIT_BYTES)
        self._check(self._lib.hgb_find_splits_noalloc(self._h, hp, int(n_nodes), float(lam),
                                                      float(gamma), op), "find_splits_noalloc")

    def find_splits(self, hist, n_nodes: int, lam: float, gamma: float, out):
        """out: uint8 CUDA tensor of at least n_nodes * 56 bytes (hgb_split records)."""
        torch = self._torch
        hp = self._dev(hist, "hist", torch.int64, int(n_nodes) * self.node_elems)
        op = self._dev(out, "out", torch.uint8, int(n_nodes) * SPLIT_BYTES)
        self._check(self._lib.hgb_find_splits(self._h, hp, int(n_nodes), float(lam),
                                              float(gamma), op), "find_splits")
