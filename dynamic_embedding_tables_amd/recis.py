"""Thin Python binding of librecis.so (ctypes): argument marshalling only.

Every step of the hot path runs in the library's HIP kernels; PyTorch only
provides device memory (tensors) and the stream handle.  The functions carry
the names of the C ABI in ``include/recis.h``; ``Table`` and ``LookupResult``
are conveniences that allocate the buffers a call needs.

The binding refuses to work without the built library: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Iterable, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librecis.so")

# ------------------------------------------------------------ ABI constants
RECIS_OK = 0
RECIS_ERR_INVALID_ARG = 1
RECIS_ERR_OUT_OF_MEMORY = 2
RECIS_ERR_CAPACITY = 3
RECIS_ERR_KEY_RANGE = 4
RECIS_ERR_HIP = 5
RECIS_ERR_UNSUPPORTED = 6
RECIS_DTYPE_F32 = 0
RECIS_DTYPE_BF16 = 1
RECIS_OPTIM_NONE = 0
RECIS_OPTIM_ADAGRAD = 1
RECIS_OPTIM_ADAM = 2
RECIS_MEM_DEVICE = 0
RECIS_MEM_HOST = 1
RECIS_POOL_SUM = 0
RECIS_POOL_MEAN = 1
RECIS_POOL_NONE = 2
RECIS_OP_HASH = 1
RECIS_OP_MOD = 2
RECIS_OP_BUCKETIZE = 4
RECIS_FIND_ONLY = 1
RECIS_GROUP_BY_OCCURRENCE = 2

DTYPES = {"f32": RECIS_DTYPE_F32, "bf16": RECIS_DTYPE_BF16}
OPTIMS = {"none": RECIS_OPTIM_NONE, "adagrad": RECIS_OPTIM_ADAGRAD, "adam": RECIS_OPTIM_ADAM}
POOLS = {"sum": RECIS_POOL_SUM, "mean": RECIS_POOL_MEAN, "none": RECIS_POOL_NONE}

EXPORTED_SYMBOLS = (
    "recis_table_config_default", "recis_plan_words", "recis_idmap_create", "recis_idmap_destroy",
    "recis_idmap_insert_find", "recis_idmap_evict", "recis_idmap_evict_decay", "recis_idmap_evict_lru",
    "recis_idmap_retier",
    "recis_lookup_pool_fwd",
    "recis_pool_bwd_update", "recis_pool_bwd_update_noalloc", "recis_noalloc_scratch_bytes",
    "recis_writeback", "recis_idmap_export", "recis_idmap_import", "recis_idmap_key_ages", "recis_idmap_sketch",
    "recis_idmap_stats", "recis_get_error",
    "recis_status_string", "recis_profile_kernel",
)


class recis_table_config(C.Structure):
    _fields_ = [("dim", C.c_int32), ("dtype", C.c_int32), ("optim", C.c_int32),
                ("admit_threshold", C.c_uint32), ("seed", C.c_uint64), ("init_bound", C.c_float),
                ("max_load", C.c_float), ("slot_capacity", C.c_int64), ("block_rows", C.c_int64),
                ("max_rows", C.c_int64), ("reserve_rows", C.c_int64), ("block_memory", C.c_int32),
                ("track_last_use", C.c_int32), ("admit_sketch_bits", C.c_int32), ("device_rows", C.c_int64),
                ("hot_grad_bytes", C.c_int64)]


class recis_allocator(C.Structure):
    _fields_ = [("ctx", C.c_void_p), ("alloc", C.c_void_p), ("free", C.c_void_p)]


class recis_feature_desc(C.Structure):
    _fields_ = [("values", C.c_void_p), ("bag_offsets", C.c_void_p), ("n", C.c_int64),
                ("slot", C.c_uint32), ("ops", C.c_uint32), ("mod", C.c_uint64),
                ("boundaries", C.c_void_p), ("nb", C.c_int64)]


class recis_lookup_result(C.Structure):
    _fields_ = [("unique_keys", C.c_void_p), ("unique_rows", C.c_void_p), ("inverse", C.c_void_p),
                ("counts", C.c_void_p), ("bag_offsets", C.c_void_p), ("num_unique", C.c_void_p),
                ("unique_offsets", C.c_void_p), ("grouped", C.c_void_p), ("plan", C.c_void_p),
                ("capacity", C.c_int64), ("bag_capacity", C.c_int64), ("n", C.c_int64), ("num_feats", C.c_int32),
                ("batch", C.c_int32), ("flags", C.c_uint32), ("epoch", C.c_uint64),
                ("map_version", C.c_uint64)]


class recis_optim_params(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double), ("eps", C.c_double)]


class recis_table_stats(C.Structure):
    _fields_ = [("keys", C.c_int64), ("rows_in_use", C.c_int64), ("rows_allocated", C.c_int64),
                ("blocks", C.c_int64), ("slot_capacity", C.c_int64), ("adam_step", C.c_int64),
                ("bytes", C.c_int64), ("probationary_keys", C.c_int64), ("claim_attempts", C.c_int64),
                ("claim_failures", C.c_int64), ("hbm_rows", C.c_int64),
                ("lookup_pairs", C.c_int64), ("hot_keys", C.c_int64)]


class RecisError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = int(status)
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def load_library() -> C.CDLL:
    """Loads librecis.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with dynamic_embedding_tables_amd.build.build()")
    L = C.CDLL(LIB_PATH)
    p, i32, i64, u32 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32
    L.recis_table_config_default.argtypes = [C.POINTER(recis_table_config)]
    L.recis_table_config_default.restype = None
    L.recis_plan_words.argtypes = [i64]
    L.recis_plan_words.restype = i64
    L.recis_idmap_create.argtypes = [C.POINTER(recis_table_config), C.POINTER(recis_allocator), p, C.POINTER(p)]
    L.recis_idmap_destroy.argtypes = [p]
    L.recis_idmap_insert_find.argtypes = [p, C.POINTER(recis_feature_desc), i32, i32, u32,
                                          C.POINTER(recis_lookup_result), p]
    L.recis_idmap_evict.argtypes = [p, u32, p, p]
    L.recis_idmap_evict_decay.argtypes = [p, u32, C.c_double, p, p]
    L.recis_idmap_evict_lru.argtypes = [p, i64, p, p]
    L.recis_idmap_retier.argtypes = [p, p, p]
    L.recis_lookup_pool_fwd.argtypes = [p, C.POINTER(recis_lookup_result), i32, p, p]
    L.recis_pool_bwd_update.argtypes = [p, C.POINTER(recis_lookup_result), i32, p, i32,
                                        C.POINTER(recis_optim_params), p]
    L.recis_pool_bwd_update_noalloc.argtypes = [p, C.POINTER(recis_lookup_result), i32, p, i32,
                                                C.POINTER(recis_optim_params), p]
    L.recis_noalloc_scratch_bytes.argtypes = []
    L.recis_noalloc_scratch_bytes.restype = i64
    L.recis_writeback.argtypes = [p, p, i64, p, p]
    L.recis_idmap_export.argtypes = [p, i64, p, p, p, p, p, C.POINTER(i64), p]
    L.recis_idmap_import.argtypes = [p, i64, p, p, p, p, p, i64, p]
    L.recis_idmap_key_ages.argtypes = [p, p, i64, p, i32, p]
    L.recis_idmap_sketch.argtypes = [p, p, i32, p]
    L.recis_idmap_stats.argtypes = [p, C.POINTER(recis_table_stats), p]
    L.recis_get_error.argtypes = [p, p]
    L.recis_profile_kernel.argtypes = [p, C.c_char_p, p, p]
    L.recis_status_string.argtypes = [i32]
    L.recis_status_string.restype = C.c_char_p
    for name in ("recis_idmap_create", "recis_idmap_destroy", "recis_idmap_insert_find",
                 "recis_idmap_evict", "recis_idmap_evict_decay", "recis_idmap_evict_lru", "recis_idmap_retier",
                 "recis_lookup_pool_fwd",
                 "recis_pool_bwd_update", "recis_pool_bwd_update_noalloc",
                 "recis_writeback", "recis_idmap_export", "recis_idmap_import", "recis_idmap_key_ages",
                 "recis_idmap_sketch", "recis_idmap_stats", "recis_get_error"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def status_string(st: int) -> str:
    return load_library().recis_status_string(int(st)).decode()


def _check(st: int, where: str):
    if st != RECIS_OK:
        raise RecisError(st, where)


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# ------------------------------------------------------------ C ABI, by name
def recis_table_config_default() -> recis_table_config:
    c = recis_table_config()
    load_library().recis_table_config_default(C.byref(c))
    return c


def recis_plan_words(capacity: int) -> int:
    return int(load_library().recis_plan_words(capacity))


# ------------------------------------------------ allocator bridge to torch
# The table's device memory (IDMap, EmbeddingBlocks, scratch) comes from
# torch's caching allocator through these two callbacks, so the library never
# calls hipMalloc when torch drives it and torch's memory statistics include
# the table.  A block is tied to the stream of the call that asked for it;
# the library frees memory only after that stream's work on it has finished.
_ALLOC_FN = C.CFUNCTYPE(C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p)
_FREE_FN = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p, C.c_void_p)
_allocator_calls = {"alloc": 0, "free": 0}


def _torch_alloc(ctx, nbytes, stream):
    try:
        import torch
        p = torch.cuda.caching_allocator_alloc(int(nbytes), stream=int(stream or 0))
        _allocator_calls["alloc"] += 1
        return p
    except Exception:  # out of memory (or torch unusable): the library sees NULL
        return None


def _torch_free(ctx, p, stream):
    try:
        import torch
        torch.cuda.caching_allocator_delete(int(p))
        _allocator_calls["free"] += 1
    except Exception:  # interpreter shutdown: the process is ending anyway
        pass


_torch_alloc_c = _ALLOC_FN(_torch_alloc)
_torch_free_c = _FREE_FN(_torch_free)
TORCH_ALLOCATOR = recis_allocator(None, C.cast(_torch_alloc_c, C.c_void_p), C.cast(_torch_free_c, C.c_void_p))


def allocator_calls() -> dict:
    """Calls made through the torch allocator bridge so far (alloc, free)."""
    return dict(_allocator_calls)


def recis_idmap_create(cfg: recis_table_config, stream=None, allocator: Optional[recis_allocator] = None
                       ) -> C.c_void_p:
    """allocator: a recis_allocator (e.g. TORCH_ALLOCATOR), or None for the
    library's own hipMalloc / hipFree."""
    h = C.c_void_p()
    a = C.byref(allocator) if allocator is not None else None
    _check(load_library().recis_idmap_create(C.byref(cfg), a, _stream(stream), C.byref(h)),
           "recis_idmap_create")
    return h


def recis_idmap_destroy(h):
    _check(load_library().recis_idmap_destroy(h), "recis_idmap_destroy")


def recis_idmap_insert_find(h, descs, num_feats: int, batch: int, flags: int,
                            res: recis_lookup_result, stream=None):
    _check(load_library().recis_idmap_insert_find(h, descs, num_feats, batch, flags, C.byref(res),
                                                  _stream(stream)), "recis_idmap_insert_find")


def recis_idmap_evict(h, min_count: int, num_evicted=None, stream=None):
    _check(load_library().recis_idmap_evict(h, min_count, _ptr(num_evicted), _stream(stream)),
           "recis_idmap_evict")


def recis_idmap_evict_lru(h, max_keys: int, num_evicted=None, stream=None):
    _check(load_library().recis_idmap_evict_lru(h, max_keys, _ptr(num_evicted), _stream(stream)),
           "recis_idmap_evict_lru")


def recis_idmap_retier(h, num_moved=None, stream=None):
    _check(load_library().recis_idmap_retier(h, _ptr(num_moved), _stream(stream)), "recis_idmap_retier")


def recis_idmap_evict_decay(h, min_count: int, decay: float, num_evicted=None, stream=None):
    _check(load_library().recis_idmap_evict_decay(h, min_count, decay, _ptr(num_evicted), _stream(stream)),
           "recis_idmap_evict_decay")


def recis_lookup_pool_fwd(h, res: recis_lookup_result, pool: int, out, stream=None):
    _check(load_library().recis_lookup_pool_fwd(h, C.byref(res), pool, _ptr(out), _stream(stream)),
           "recis_lookup_pool_fwd")


def recis_pool_bwd_update(h, res: recis_lookup_result, pool: int, grad, grad_dtype: int,
                          opt: recis_optim_params, stream=None):
    _check(load_library().recis_pool_bwd_update(h, C.byref(res), pool, _ptr(grad), grad_dtype,
                                                C.byref(opt), _stream(stream)), "recis_pool_bwd_update")


def recis_pool_bwd_update_noalloc(h, res: recis_lookup_result, pool: int, grad, grad_dtype: int,
                                  opt: recis_optim_params, stream=None):
    _check(load_library().recis_pool_bwd_update_noalloc(h, C.byref(res), pool, _ptr(grad), grad_dtype,
                                                        C.byref(opt), _stream(stream)),
           "recis_pool_bwd_update_noalloc")


def recis_noalloc_scratch_bytes() -> int:
    return int(load_library().recis_noalloc_scratch_bytes())


def recis_profile_kernel(h, kernel: Optional[str], start=None, stop=None):
    """Bracket launches of library kernel `kernel` with two torch.cuda.Event
    objects (already recorded once, so their HIP events exist); None clears."""
    name = None if kernel is None else kernel.encode()
    a = None if start is None else C.c_void_p(start.cuda_event)
    b = None if stop is None else C.c_void_p(stop.cuda_event)
    _check(load_library().recis_profile_kernel(h, name, a, b), "recis_profile_kernel")


def recis_writeback(h, keys, n: int, rows, stream=None):
    _check(load_library().recis_writeback(h, _ptr(keys), n, _ptr(rows), _stream(stream)), "recis_writeback")


def recis_idmap_export(h, cap: int, keys, rows, counts, params, state, stream=None) -> int:
    n = C.c_int64()
    _check(load_library().recis_idmap_export(h, cap, _ptr(keys), _ptr(rows), _ptr(counts), _ptr(params),
                                             _ptr(state), C.byref(n), _stream(stream)), "recis_idmap_export")
    return int(n.value)


def recis_idmap_import(h, n: int, keys, rows, counts, params, state, adam_step: int, stream=None):
    _check(load_library().recis_idmap_import(h, n, _ptr(keys), _ptr(rows), _ptr(counts), _ptr(params),
                                             _ptr(state), adam_step, _stream(stream)), "recis_idmap_import")


def recis_idmap_key_ages(h, keys, n: int, ages, set_: bool, stream=None):
    _check(load_library().recis_idmap_key_ages(h, _ptr(keys), n, _ptr(ages), 1 if set_ else 0, _stream(stream)),
           "recis_idmap_key_ages")


def recis_idmap_sketch(h, counters, set_: bool, stream=None):
    _check(load_library().recis_idmap_sketch(h, _ptr(counters), 1 if set_ else 0, _stream(stream)),
           "recis_idmap_sketch")


def recis_idmap_stats(h, stream=None) -> recis_table_stats:
    st = recis_table_stats()
    _check(load_library().recis_idmap_stats(h, C.byref(st), _stream(stream)), "recis_idmap_stats")
    return st


def recis_get_error(h, stream=None) -> int:
    return int(load_library().recis_get_error(h, _stream(stream)))


# --------------------------------------------------------- conveniences
class LookupResult:
    """Device buffers of one insert_find, sized for `capacity` occurrences and
    `nbags` merged bags."""

    def __init__(self, capacity: int, nbags: int, device="cuda"):
        import torch
        cap = max(int(capacity), 1)
        i32, i64 = torch.int32, torch.int64
        self.unique_keys = torch.empty(cap, dtype=i64, device=device)
        self.unique_rows = torch.empty(cap, dtype=i64, device=device)
        self.inverse = torch.empty(cap, dtype=i32, device=device)
        self.counts = torch.empty(cap, dtype=i32, device=device)
        self.bag_offsets = torch.empty(max(nbags, 0) + 1, dtype=i32, device=device)
        self.num_unique = torch.zeros(1, dtype=i64, device=device)
        self.unique_offsets = torch.empty(cap + 1, dtype=i32, device=device)
        self.grouped = torch.empty(cap, dtype=i32, device=device)
        self.plan = torch.zeros(recis_plan_words(cap), dtype=i32, device=device)
        self.c = recis_lookup_result(
            self.unique_keys.data_ptr(), self.unique_rows.data_ptr(), self.inverse.data_ptr(),
            self.counts.data_ptr(), self.bag_offsets.data_ptr(), self.num_unique.data_ptr(),
            self.unique_offsets.data_ptr(), self.grouped.data_ptr(), self.plan.data_ptr(),
            cap, max(int(nbags), 0), 0, 0, 0, 0, 0, 0)
        self.capacity = cap
        self.nbags = nbags

    @property
    def n(self) -> int:
        return int(self.c.n)

    def U(self) -> int:
        return int(self.num_unique.item())


class DeviceFeature:
    """A feature whose values / bag offsets already live on the GPU."""

    def __init__(self, values, bag_offsets, slot: int, ops: int = 0, mod: int = 0, boundaries=None):
        self.values = values
        self.bag_offsets = bag_offsets
        self.slot, self.ops, self.mod = int(slot), int(ops), int(mod)
        self.boundaries = None if boundaries is None else np.ascontiguousarray(boundaries, dtype=np.int64)

    @property
    def n(self) -> int:
        return int(self.values.numel())


def make_descs(feats: Sequence[DeviceFeature]):
    arr = (recis_feature_desc * max(len(feats), 1))()
    for i, f in enumerate(feats):
        b = f.boundaries
        arr[i] = recis_feature_desc(f.values.data_ptr() if f.n else 0, f.bag_offsets.data_ptr(), f.n,
                                    f.slot, f.ops, f.mod,
                                    b.ctypes.data if b is not None and b.size else None,
                                    0 if b is None else int(b.size))
    return arr


def _as_u32_bits(x):
    """int32 tensor holding the bits of uint32 values given as int64."""
    import torch
    v = x.to(torch.int64) & 0xFFFFFFFF
    return torch.where(v >= 2**31, v - 2**32, v).to(torch.int32).contiguous()


class Table:
    """Owns one recis table handle."""

    def __init__(self, dim: int, dtype: str = "f32", optim: str = "adagrad", seed: int = 20250925,
                 init_bound: float = 0.05, admit_threshold: int = 1, slot_capacity: int = 1 << 20,
                 block_rows: int = 1 << 20, max_rows: int = (1 << 30) - 1, reserve_rows: int = 0,
                 max_load: float = 0.5, block_memory: str = "device", track_last_use: bool = False,
                 admit_sketch_bits: int = 0, stream=None, allocator: str = "torch", device_rows: int = 0,
                 hot_grad_bytes: int = 0):
        cfg = recis_table_config_default()
        cfg.dim, cfg.dtype, cfg.optim = dim, DTYPES[dtype], OPTIMS[optim]
        cfg.seed, cfg.init_bound, cfg.admit_threshold = seed, init_bound, admit_threshold
        cfg.slot_capacity, cfg.block_rows, cfg.max_rows = slot_capacity, block_rows, max_rows
        cfg.reserve_rows, cfg.max_load = reserve_rows, max_load
        cfg.block_memory = {"device": RECIS_MEM_DEVICE, "host": RECIS_MEM_HOST}[block_memory]
        cfg.track_last_use = 1 if track_last_use else 0
        cfg.admit_sketch_bits = admit_sketch_bits
        cfg.device_rows = device_rows
        cfg.hot_grad_bytes = hot_grad_bytes
        self.dim, self.dtype, self.optim = dim, dtype, optim
        self.config = {"seed": seed, "init_bound": init_bound, "admit_threshold": admit_threshold,
                       "block_memory": block_memory, "track_last_use": bool(track_last_use),
                       "admit_sketch_bits": int(admit_sketch_bits), "device_rows": int(device_rows),
                       "hot_grad_bytes": int(hot_grad_bytes)}
        if allocator not in ("torch", "hip"):
            raise ValueError("allocator is 'torch' (torch's caching allocator) or 'hip' (hipMalloc)")
        self.allocator = allocator
        self.h = recis_idmap_create(cfg, stream, TORCH_ALLOCATOR if allocator == "torch" else None)

    def close(self):
        if getattr(self, "h", None):
            recis_idmap_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def insert_find(self, feats: Sequence[DeviceFeature], batch: int, res: LookupResult,
                    flags: int = 0, stream=None, descs=None):
        d = descs if descs is not None else make_descs(feats)
        recis_idmap_insert_find(self.h, d, len(feats), batch, flags, res.c, stream)
        return res

    def forward(self, res: LookupResult, pool: str, out, stream=None):
        recis_lookup_pool_fwd(self.h, res.c, POOLS[pool], out, stream)
        return out

    def backward_update(self, res: LookupResult, pool: str, grad, grad_dtype: str = "f32",
                        lr: float = 0.01, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-10,
                        stream=None, noalloc: bool = False):
        """noalloc: the allocation-free entry point (fixed scratch; see
        recis_pool_bwd_update_noalloc)."""
        opt = recis_optim_params(lr, beta1, beta2, eps)
        fn = recis_pool_bwd_update_noalloc if noalloc else recis_pool_bwd_update
        fn(self.h, res.c, POOLS[pool], grad, DTYPES[grad_dtype], opt, stream)

    def evict(self, min_count: int, num_evicted=None, stream=None, decay: float = 0.0):
        """Eviction pass; survivors keep floor(count * decay) (0: restart)."""
        if decay == 0.0:
            recis_idmap_evict(self.h, min_count, num_evicted, stream)
        else:
            recis_idmap_evict_decay(self.h, min_count, decay, num_evicted, stream)

    def evict_lru(self, max_keys: int, num_evicted=None, stream=None):
        """Keeps at most max_keys keys, the most recently used (needs
        track_last_use)."""
        recis_idmap_evict_lru(self.h, max_keys, num_evicted, stream)

    def retier(self, num_moved=None, stream=None):
        """Host-memory blocks with an HBM tier: the most frequent keys move
        into the HBM rows (see recis_idmap_retier)."""
        recis_idmap_retier(self.h, num_moved, stream)

    def key_ages(self, keys, stream=None):
        """uint32 ages of the given keys (device int64 tensor) as an int64 tensor
        (0xFFFFFFFF: not in the table); needs track_last_use."""
        import torch
        ages = torch.empty(keys.shape[0], dtype=torch.int32, device="cuda")
        recis_idmap_key_ages(self.h, keys.contiguous(), int(keys.shape[0]), ages, False, stream)
        return ages.to(torch.int64) & 0xFFFFFFFF

    def set_key_ages(self, keys, ages, stream=None):
        a = _as_u32_bits(ages)
        recis_idmap_key_ages(self.h, keys.contiguous(), int(keys.shape[0]), a, True, stream)

    def sketch_counters(self, stream=None):
        """The count-min sketch's counters (int64 tensor of the uint32 values)."""
        import torch
        c = torch.empty(4 << self.config["admit_sketch_bits"], dtype=torch.int32, device="cuda")
        recis_idmap_sketch(self.h, c, False, stream)
        return c.to(torch.int64) & 0xFFFFFFFF

    def set_sketch_counters(self, counters, stream=None):
        recis_idmap_sketch(self.h, _as_u32_bits(counters), True, stream)

    def writeback(self, keys, rows, stream=None):
        recis_writeback(self.h, keys, int(keys.numel()), rows, stream)

    def stats(self, stream=None) -> recis_table_stats:
        return recis_idmap_stats(self.h, stream)

    def profile_kernel(self, kernel, start=None, stop=None):
        recis_profile_kernel(self.h, kernel, start, stop)

    def get_error(self, stream=None) -> int:
        return recis_get_error(self.h, stream)

    def check(self, stream=None):
        _check(self.get_error(stream), "device error")

    def export(self, stream=None) -> dict:
        """All keys with row, count, params and state (device tensors, unsorted)."""
        import torch
        st = self.stats(stream)
        cap = max(int(st.keys), 1) + 1024
        sw = {"none": 0, "adagrad": 1, "adam": 2}[self.optim] * self.dim
        pdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        keys = torch.empty(cap, dtype=torch.int64, device="cuda")
        rows = torch.empty(cap, dtype=torch.int64, device="cuda")
        counts = torch.empty(cap, dtype=torch.int32, device="cuda")
        params = torch.empty(cap, self.dim, dtype=pdt, device="cuda")
        state = torch.empty(cap, max(sw, 1), dtype=torch.float32, device="cuda")
        n = recis_idmap_export(self.h, cap, keys, rows, counts, params, state if sw else None, stream)
        assert n <= cap
        return {"keys": keys[:n], "rows": rows[:n], "counts": counts[:n], "params": params[:n],
                "state": state[:n, :sw]}

    def import_(self, keys, rows, counts, params, state, adam_step: int = 0, stream=None):
        """Loads exported arrays (device tensors) into this never-used table."""
        import torch
        n = int(keys.shape[0])
        sw = {"none": 0, "adagrad": 1, "adam": 2}[self.optim] * self.dim
        pdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        if params.dtype != pdt or tuple(params.shape) != (n, self.dim):
            raise ValueError(f"params must be {pdt} [{n}, {self.dim}]")
        if sw and (state is None or state.dtype != torch.float32 or tuple(state.shape) != (n, sw)):
            raise ValueError(f"state must be float32 [{n}, {sw}]")
        keys = keys.to(torch.int64).contiguous()
        rows = rows.to(torch.int64).contiguous()
        counts = counts.to(torch.int32).contiguous()
        params = params.contiguous()
        state = state.contiguous() if sw else None
        recis_idmap_import(self.h, n, keys, rows, counts, params, state, adam_step, stream)
