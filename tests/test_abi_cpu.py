"""The C ABI without a GPU: the library loads, exports every function the
header declares, the ctypes structures match the C layouts, and argument
errors come back synchronously before any device work."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "recis.h")


@pytest.fixture(scope="module")
def lib():
    from dynamic_embedding_tables_amd import recis
    if not os.path.exists(recis.LIB_PATH):
        pytest.fail("librecis.so is not built (run __graft_entry__.build())")
    return recis


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(recis_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 13
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(names) == set(lib.EXPORTED_SYMBOLS)
    L = lib.load_library()
    for n in names:
        assert hasattr(L, n)


def test_struct_layouts_match_header(lib, tmp_path):
    src = tmp_path / "layout.c"
    structs = {
        "recis_table_config": lib.recis_table_config,
        "recis_allocator": lib.recis_allocator,
        "recis_feature_desc": lib.recis_feature_desc,
        "recis_lookup_result": lib.recis_lookup_result,
        "recis_optim_params": lib.recis_optim_params,
        "recis_table_stats": lib.recis_table_stats,
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "recis.h"', "int main(void){"]
    for name, cls in structs.items():
        lines.append(f'printf("{name} %zu\\n", sizeof({name}));')
        for fname, _ in cls._fields_:
            lines.append(f'printf("{name}.{fname} %zu\\n", offsetof({name}, {fname}));')
    lines.append("return 0;}")
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                           "-I", "/opt/rocm/include", str(src), "-o", str(exe)])
    got = dict(l.rsplit(" ", 1) for l in subprocess.check_output([str(exe)], text=True).splitlines())
    for name, cls in structs.items():
        assert int(got[name]) == C.sizeof(cls), name
        for fname, _ in cls._fields_:
            assert int(got[f"{name}.{fname}"]) == getattr(cls, fname).offset, (name, fname)


def test_config_defaults_and_plan_words(lib):
    c = lib.recis_table_config_default()
    assert c.dim == 64 and c.dtype == lib.RECIS_DTYPE_F32 and c.optim == lib.RECIS_OPTIM_ADAGRAD
    assert abs(c.init_bound - 0.05) < 1e-9 and c.max_load == 0.5 and c.max_rows == 2**30 - 1
    assert c.block_memory == lib.RECIS_MEM_DEVICE
    assert lib.recis_plan_words(0) > 0
    assert lib.recis_plan_words(1 << 20) > lib.recis_plan_words(1 << 10)
    assert lib.recis_plan_words(-1) == -1


def test_status_strings(lib):
    for st in range(7):
        assert lib.status_string(st)
    assert lib.status_string(99) == "unknown status"


def test_invalid_arguments_return_synchronously(lib):
    L = lib.load_library()
    h = C.c_void_p()
    assert L.recis_idmap_create(None, None, None, C.byref(h)) == lib.RECIS_ERR_INVALID_ARG
    c = lib.recis_table_config_default()
    assert L.recis_idmap_create(C.byref(c), None, None, None) == lib.RECIS_ERR_INVALID_ARG
    for field, bad in [("dtype", 7), ("optim", 9), ("max_load", 0.0), ("max_load", 0.8),
                       ("slot_capacity", 0), ("block_rows", 0), ("max_rows", 0), ("max_rows", 2**30),
                       ("reserve_rows", -1), ("init_bound", -1.0), ("block_memory", 2), ("track_last_use", 2),
                       ("admit_sketch_bits", -1), ("admit_sketch_bits", 31)]:
        c = lib.recis_table_config_default()
        setattr(c, field, bad)
        assert L.recis_idmap_create(C.byref(c), None, None, C.byref(h)) == lib.RECIS_ERR_INVALID_ARG, field
    c = lib.recis_table_config_default()
    c.dim = 48
    assert L.recis_idmap_create(C.byref(c), None, None, C.byref(h)) == lib.RECIS_ERR_UNSUPPORTED
    alloc = lib.recis_allocator(None, None, None)
    c = lib.recis_table_config_default()
    assert L.recis_idmap_create(C.byref(c), C.byref(alloc), None, C.byref(h)) == lib.RECIS_ERR_INVALID_ARG
    # NULL table handles
    res = lib.recis_lookup_result()
    assert L.recis_idmap_insert_find(None, None, 0, 0, 0, C.byref(res), None) == lib.RECIS_ERR_INVALID_ARG
    assert L.recis_idmap_evict(None, 1, None, None) == lib.RECIS_ERR_INVALID_ARG
    assert L.recis_idmap_evict_decay(None, 1, 0.5, None, None) == lib.RECIS_ERR_INVALID_ARG
    assert L.recis_idmap_evict_lru(None, 1, None, None) == lib.RECIS_ERR_INVALID_ARG
    assert L.recis_idmap_import(None, 0, None, None, None, None, None, 0, None) == lib.RECIS_ERR_INVALID_ARG
    assert L.recis_lookup_pool_fwd(None, C.byref(res), 0, None, None) == lib.RECIS_ERR_INVALID_ARG
    opt = lib.recis_optim_params(0.01, 0.9, 0.999, 1e-8)
    assert L.recis_pool_bwd_update(None, C.byref(res), 0, None, 0, C.byref(opt), None) == lib.RECIS_ERR_INVALID_ARG
    assert L.recis_writeback(None, None, 0, None, None) == lib.RECIS_ERR_INVALID_ARG
    n = C.c_int64()
    assert L.recis_idmap_export(None, 0, None, None, None, None, None, C.byref(n), None) == lib.RECIS_ERR_INVALID_ARG
    st = lib.recis_table_stats()
    assert L.recis_idmap_stats(None, C.byref(st), None) == lib.RECIS_ERR_INVALID_ARG
    assert L.recis_get_error(None, None) == lib.RECIS_ERR_INVALID_ARG
    assert L.recis_idmap_destroy(None) == lib.RECIS_ERR_INVALID_ARG


def _failing_allocator(lib, calls):
    ALLOC = C.CFUNCTYPE(C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p)
    FREE = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p, C.c_void_p)

    def a(ctx, n, s):
        calls.append(n)
        return None

    def f(ctx, p, s):
        pass
    fa, ff = ALLOC(a), FREE(f)
    return lib.recis_allocator(None, C.cast(fa, C.c_void_p), C.cast(ff, C.c_void_p)), (fa, ff)


def test_allocator_failure_is_out_of_memory(lib):
    L = lib.load_library()
    calls = []
    alloc, keep = _failing_allocator(lib, calls)
    c = lib.recis_table_config_default()
    h = C.c_void_p()
    assert L.recis_idmap_create(C.byref(c), C.byref(alloc), None, C.byref(h)) == lib.RECIS_ERR_OUT_OF_MEMORY
    assert calls and not h.value


def test_binding_fails_loudly_without_library(lib, monkeypatch, tmp_path):
    import importlib
    import dynamic_embedding_tables_amd.recis as r
    monkeypatch.setattr(r, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(r, "_lib", None)
    with pytest.raises(ImportError):
        r.load_library()
    importlib.reload(r)


def test_binding_constants_match_the_header(lib):
    """Every integer #define of include/recis.h has the same value in the binding."""
    import re
    text = open(os.path.join(ROOT, "include", "recis.h")).read()
    found = re.findall(r"^#define (RECIS_[A-Z0-9_]+) (\d+)u?\b", text, flags=re.M)
    assert len(found) > 20
    for name, value in found:
        assert getattr(lib, name) == int(value), name
