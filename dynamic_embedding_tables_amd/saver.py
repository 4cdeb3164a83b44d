"""Save and restore a sparse table as one SafeTensors file.

The pages store and deliver sparse parameters in the standard SafeTensors
format (page "RecIS (Recommendation Intelligence System)" README, section
"Core architecture > Saver").  This module writes the file from
recis_idmap_export's arrays and reads it back through recis_idmap_import;
every step on the device is the library's.

File layout (tensor names, shapes, dtypes; n keys, unsorted):
    keys     int64   [n]         the table keys ((slot << 48) | id)
    has_row  uint8   [n]         1: the key has a row; 0: admission has not
                                 given it one yet
    counts   int64   [n]         the key's occurrence count (admission state)
    params   f32|bf16 [n, dim]   the row's parameters (the initializer's
                                 values for a row never updated); zeros
                                 where has_row is 0
    state    f32     [n, s*dim]  optimizer state (s = 2 for Adam: m then v;
                                 1 for Adagrad); absent when there is none
    last_use_age int64 [n]      (tables with last-use stamps) each key's age in
                                 counting lookups
    sketch   int64   [4 << bits] (tables with count-min admission) the
                                 sketch's counters, row after row
and the string metadata
    format, dim, dtype, optim, seed, init_bound, admit_threshold, adam_step,
    track_last_use, admit_sketch_bits.
"""
from __future__ import annotations

from typing import Optional

from . import recis

FORMAT = "recis-sparse-table/1"


def write(path: str, tensors: dict, meta: dict) -> None:
    """Writes the named CPU tensors and the string metadata (host only)."""
    from safetensors.torch import save_file
    meta = dict(meta, format=FORMAT)
    save_file({k: v.contiguous() for k, v in tensors.items()}, path, metadata={k: str(v) for k, v in meta.items()})


def read(path: str):
    """(tensors, metadata) of a file written by `write` (host only)."""
    from safetensors import safe_open
    from safetensors.torch import load_file
    with safe_open(path, framework="pt") as f:
        meta = dict(f.metadata() or {})
    if meta.get("format") != FORMAT:
        raise ValueError(f"{path}: not a {FORMAT} file")
    return load_file(path), meta


def save(table: "recis.Table", path: str, stream=None) -> int:
    """Writes `table` to `path`; returns the number of keys."""
    import torch
    ex = table.export(stream)
    st = table.stats(stream)
    cfg = table.config
    tensors = {
        "keys": ex["keys"].cpu(),
        "has_row": (ex["rows"] >= 0).to(torch.uint8).cpu(),
        "counts": ex["counts"].to(torch.int64).cpu(),
        "params": ex["params"].cpu(),
    }
    if ex["state"].shape[1] > 0:
        tensors["state"] = ex["state"].cpu()
    if cfg["track_last_use"]:
        tensors["last_use_age"] = table.key_ages(ex["keys"], stream).cpu()
    if cfg["admit_sketch_bits"]:
        tensors["sketch"] = table.sketch_counters(stream).cpu()
    write(path, tensors, {"dim": table.dim, "dtype": table.dtype, "optim": table.optim, "seed": cfg["seed"],
                          "init_bound": repr(float(cfg["init_bound"])),
                          "admit_threshold": cfg["admit_threshold"], "adam_step": int(st.adam_step),
                          "track_last_use": int(cfg["track_last_use"]),
                          "admit_sketch_bits": int(cfg["admit_sketch_bits"])})
    return int(ex["keys"].shape[0])


def load(path: str, stream=None, **table_kw) -> "recis.Table":
    """A new table holding what `path` holds.  table_kw sets the layout
    (slot_capacity, block_rows, block_memory, ...); the table's attributes
    (dim, dtype, optimizer, initializer, admission) come from the file."""
    import torch
    t, meta = read(path)
    table = recis.Table(int(meta["dim"]), meta["dtype"], meta["optim"], seed=int(meta["seed"]),
                        init_bound=float(meta["init_bound"]), admit_threshold=int(meta["admit_threshold"]),
                        track_last_use=bool(int(meta.get("track_last_use", "0"))),
                        admit_sketch_bits=int(meta.get("admit_sketch_bits", "0")), **table_kw)
    keys = t["keys"].cuda()
    rows = torch.where(t["has_row"].to(torch.bool), 0, -1).to(torch.int64)
    state: Optional[torch.Tensor] = t["state"].cuda() if "state" in t else None
    table.import_(keys, rows.cuda(), t["counts"].cuda(), t["params"].cuda(), state,
                  adam_step=int(meta["adam_step"]), stream=stream)
    if "last_use_age" in t:
        table.set_key_ages(keys, t["last_use_age"].cuda(), stream)
    if "sketch" in t:
        table.set_sketch_counters(t["sketch"].cuda(), stream)
    return table
