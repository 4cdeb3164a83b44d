"""CPU oracle of the dynamic-embedding hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it.  The arithmetic lives in ``oracle.cpp`` (plain
sequential C++17, double-precision sums); this file only compiles it with g++
and marshals numpy arrays through ctypes.

Every function of ``oracle.cpp`` states the page passage it follows and the
reading taken where the pages are silent.  Pins (tests that tie the oracle to
something other than itself) live in ``tests/test_oracle_*.py``.  Parts with
no external pin: none of the table logic; the hash constant set is pinned
through MurmurHash3_x64_128, Philox through rocRAND's host-callable engine.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

DT = {"f32": 0, "bf16": 1}
OPT = {"none": 0, "adagrad": 1, "adam": 2}
POOL = {"sum": 0, "mean": 1, "none": 2}
FIND_ONLY = 1


def build(force: bool = True) -> str:
    """Compile oracle.cpp into liboracle.so with g++ (no GPU toolchain)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-shared", "-fPIC",
                               _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = C.CDLL(_LIB)
        p = C.c_void_p
        L.orc_fmix64.restype = C.c_uint64
        L.orc_fmix64.argtypes = [C.c_uint64]
        L.orc_philox4x32_10.argtypes = [p, p, p]
        L.orc_init_row.argtypes = [C.c_uint64, C.c_int64, C.c_int, C.c_float, p]
        L.orc_round_bf16.argtypes = [p, C.c_int64, p]
        L.orc_transform.restype = C.c_int
        L.orc_transform.argtypes = [p, C.c_int64, C.c_uint32, C.c_uint64, p, C.c_int64, C.c_uint32, p]
        L.orc_create.restype = p
        L.orc_create.argtypes = [C.c_int, C.c_int, C.c_int, C.c_uint64, C.c_float, C.c_int64,
                                 C.c_int64, C.c_uint32]
        L.orc_destroy.argtypes = [p]
        L.orc_insert_find.restype = C.c_int
        L.orc_insert_find.argtypes = [p, C.c_int32, C.c_int32] + [p] * 8 + [C.c_uint32] + [p] * 6
        L.orc_forward.restype = C.c_int
        L.orc_forward.argtypes = [p, p, p, p, C.c_int32, C.c_int32, C.c_int32, p, p]
        L.orc_reduce_grads.restype = C.c_int
        L.orc_reduce_grads.argtypes = [p, p, p, C.c_int64, C.c_int32, C.c_int32, C.c_int32, p,
                                       C.c_int32, p, p]
        L.orc_apply_update.restype = C.c_int
        L.orc_apply_update.argtypes = [p, p, C.c_int64, p, C.c_double, C.c_double, C.c_double,
                                       C.c_double, p]
        L.orc_backward_update.restype = C.c_int
        L.orc_backward_update.argtypes = [p, p, p, p, C.c_int64, C.c_int32, C.c_int32, C.c_int32,
                                          p, C.c_int32, C.c_double, C.c_double, C.c_double,
                                          C.c_double]
        L.orc_evict.restype = C.c_int64
        L.orc_evict.argtypes = [p, C.c_uint32]
        L.orc_evict_decay.restype = C.c_int64
        L.orc_evict_decay.argtypes = [p, C.c_uint32, C.c_double]
        L.orc_evict_lru.restype = C.c_int64
        L.orc_evict_lru.argtypes = [p, C.c_int64]
        L.orc_set_sketch.restype = C.c_int
        L.orc_set_sketch.argtypes = [p, C.c_int]
        L.orc_writeback.restype = C.c_int
        L.orc_writeback.argtypes = [p, p, C.c_int64, p]
        L.orc_current_rows.restype = C.c_int
        L.orc_current_rows.argtypes = [p, p, C.c_int64, p]
        L.orc_size.restype = C.c_int64
        L.orc_size.argtypes = [p]
        L.orc_rows_in_use.restype = C.c_int64
        L.orc_rows_in_use.argtypes = [p]
        L.orc_export.restype = C.c_int64
        L.orc_export.argtypes = [p, C.c_int64, p, p, p, p, p]
        L.orc_adam_step.restype = C.c_int64
        L.orc_adam_step.argtypes = [p]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- primitives
def fmix64(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint64)
    L = lib()
    return np.array([L.orc_fmix64(int(v)) for v in x.ravel()], dtype=np.uint64).reshape(x.shape)


def philox4x32_10(ctr, key) -> np.ndarray:
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def init_row(seed: int, key: int, dim: int, bound: float = 0.05) -> np.ndarray:
    out = np.zeros(dim, dtype=np.float32)
    lib().orc_init_row(seed, key, dim, bound, _ptr(out))
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Bit patterns of x (float64) rounded once to bfloat16."""
    x = _c(x, np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    lib().orc_round_bf16(_ptr(x), x.size, _ptr(out))
    return out


def transform(values, ops: int = 0, mod: int = 0, boundaries=None, slot: int = 0):
    """Returns (status, keys)."""
    v = _c(values, np.int64)
    b = _c(boundaries if boundaries is not None else np.zeros(0), np.int64)
    keys = np.zeros(v.shape[0], dtype=np.int64)
    st = lib().orc_transform(_ptr(v), v.shape[0], ops, mod, _ptr(b), b.shape[0], slot, _ptr(keys))
    return st, keys


# ---------------------------------------------------------------- the table
class LookupResult:
    def __init__(self, n: int, nbags: int):
        self.unique_keys = np.zeros(max(n, 1), dtype=np.int64)
        self.unique_rows = np.zeros(max(n, 1), dtype=np.int64)
        self.inverse = np.zeros(max(n, 1), dtype=np.int32)
        self.counts = np.zeros(max(n, 1), dtype=np.int32)
        self.merged_offsets = np.zeros(nbags + 1, dtype=np.int32)
        self.num_unique = np.zeros(1, dtype=np.int64)
        self.n = n
        self.status = 0

    @property
    def U(self) -> int:
        return int(self.num_unique[0])


class OracleTable:
    """Plain CPU table; mirrors the C ABI's calls one for one."""

    def __init__(self, spec, max_rows: int = 1 << 62, max_keys: int = 1 << 62):
        self.spec = spec
        self.dim = spec.dim
        self.h = lib().orc_create(spec.dim, DT[spec.dtype], OPT[spec.optim], spec.seed,
                                  spec.init_bound, max_rows, max_keys, spec.admit_threshold)
        if not self.h:
            raise ValueError("bad oracle table spec")

    def close(self):
        if self.h:
            lib().orc_destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()

    # features: list of workloads.FeatureInput
    def insert_find(self, features: List, batch: int, flags: int = 0) -> LookupResult:
        F = len(features)
        vals = _c(np.concatenate([f.values for f in features]) if F else np.zeros(0), np.int64)
        feat_n = _c([f.n for f in features], np.int64)
        offs = _c(np.concatenate([f.bag_offsets for f in features]) if F else np.zeros(0), np.int32)
        slots = _c([f.slot for f in features], np.uint32)
        ops = _c([f.ops for f in features], np.uint32)
        mods = _c([f.mod for f in features], np.uint64)
        bl = [f.boundaries if f.boundaries is not None else np.zeros(0, np.int64) for f in features]
        bounds = _c(np.concatenate(bl) if bl else np.zeros(0), np.int64)
        nb = _c([b.shape[0] for b in bl], np.int64)
        n = int(vals.shape[0])
        r = LookupResult(n, F * batch)
        r.status = lib().orc_insert_find(self.h, F, batch, _ptr(vals), _ptr(feat_n), _ptr(offs),
                                         _ptr(slots), _ptr(ops), _ptr(mods), _ptr(bounds), _ptr(nb),
                                         flags, _ptr(r.unique_keys), _ptr(r.unique_rows),
                                         _ptr(r.inverse), _ptr(r.counts), _ptr(r.merged_offsets),
                                         _ptr(r.num_unique))
        r.num_feats, r.batch = F, batch
        return r

    def current_rows(self, r: LookupResult) -> np.ndarray:
        """The rows the map holds now for r's distinct keys (-1: none): what
        the lookup's forward and backward act on."""
        rows = np.zeros(max(r.U, 1), dtype=np.int64)
        keys = _c(r.unique_keys[:max(r.U, 1)], np.int64)
        assert lib().orc_current_rows(self.h, _ptr(keys), r.U, _ptr(rows)) == 0
        return rows

    def forward(self, r: LookupResult, pool: str, with_abs: bool = False):
        D = self.dim
        if pool == "none":
            shape = (r.n, D)
            out = np.zeros(shape, dtype=np.uint16 if self.spec.dtype == "bf16" else np.float32)
            ab = None
        else:
            shape = (r.batch, r.num_feats * D)
            out = np.zeros(shape, dtype=np.float32)
            ab = np.zeros(shape, dtype=np.float64) if with_abs else None
        rows = self.current_rows(r)
        st = lib().orc_forward(self.h, _ptr(rows), _ptr(r.inverse), _ptr(r.merged_offsets),
                               r.num_feats, r.batch, POOL[pool], _ptr(out), _ptr(ab))
        assert st == 0, st
        return (out, ab) if with_abs else out

    def reduce_grads(self, r: LookupResult, pool: str, grad: np.ndarray, grad_dtype: str = "f32",
                     with_abs: bool = False):
        g = _c(grad, np.uint16 if grad_dtype == "bf16" else np.float32)
        G = np.zeros((max(r.U, 1), self.dim), dtype=np.float64)
        ab = np.zeros_like(G) if with_abs else None
        st = lib().orc_reduce_grads(self.h, _ptr(r.inverse), _ptr(r.merged_offsets), r.U,
                                    r.num_feats, r.batch, POOL[pool], _ptr(g), DT[grad_dtype],
                                    _ptr(G), _ptr(ab))
        assert st == 0, st
        G = G[:r.U]
        return (G, ab[:r.U]) if with_abs else G

    def apply_update(self, r: LookupResult, G: np.ndarray, only: Optional[np.ndarray] = None) -> int:
        s = self.spec
        G = _c(G, np.float64)
        o = None if only is None else _c(only, np.uint8)
        rows = self.current_rows(r)
        return lib().orc_apply_update(self.h, _ptr(rows), r.U, _ptr(G), s.lr, s.beta1,
                                      s.beta2, s.eps, _ptr(o))

    def backward_update(self, r: LookupResult, pool: str, grad: np.ndarray, grad_dtype: str = "f32") -> int:
        s = self.spec
        g = _c(grad, np.uint16 if grad_dtype == "bf16" else np.float32)
        rows = self.current_rows(r)
        return lib().orc_backward_update(self.h, _ptr(rows), _ptr(r.inverse),
                                         _ptr(r.merged_offsets), r.U, r.num_feats, r.batch,
                                         POOL[pool], _ptr(g), DT[grad_dtype], s.lr, s.beta1,
                                         s.beta2, s.eps)

    def evict(self, min_count: int, decay: float = 0.0) -> int:
        if decay == 0.0:
            return int(lib().orc_evict(self.h, min_count))
        return int(lib().orc_evict_decay(self.h, min_count, decay))

    def set_sketch(self, bits: int) -> None:
        """Count-min sketch admission with 4 x 2**bits counters (0: off)."""
        assert lib().orc_set_sketch(self.h, bits) == 0

    def evict_lru(self, max_keys: int) -> int:
        return int(lib().orc_evict_lru(self.h, max_keys))

    def writeback(self, keys: np.ndarray, rows: np.ndarray) -> int:
        k = _c(keys, np.int64)
        e = _c(rows, np.float32)
        assert e.shape == (k.shape[0], self.dim)
        return lib().orc_writeback(self.h, _ptr(k), k.shape[0], _ptr(e))

    def size(self) -> int:
        return int(lib().orc_size(self.h))

    def rows_in_use(self) -> int:
        return int(lib().orc_rows_in_use(self.h))

    @property
    def adam_step(self) -> int:
        return int(lib().orc_adam_step(self.h))

    def export(self):
        """dict of arrays sorted by key: keys, rows (-1 = none), counts, params (float32
        values, exact in the storage dtype), state (float32 [n, slots*dim])."""
        n = self.size()
        S = {"none": 0, "adagrad": 1, "adam": 2}[self.spec.optim] * self.dim
        out = {
            "keys": np.zeros(n, np.int64), "rows": np.zeros(n, np.int64),
            "counts": np.zeros(n, np.uint32), "params": np.zeros((n, self.dim), np.float32),
            "state": np.zeros((n, S), np.float32),
        }
        got = lib().orc_export(self.h, n, _ptr(out["keys"]), _ptr(out["rows"]), _ptr(out["counts"]),
                               _ptr(out["params"]), _ptr(out["state"]))
        assert got == n
        return out
