#!/usr/bin/env python3
"""Throughput of the dynamic-embedding hot path on one MI355X.

Default workload (--workload ctr): the CTR ranking batch -- 26 sparse
features merged into one logical table (dim 64, fp32 parameters, sparse Adam
with two fp32 moments per row), batch 8192, bag lengths Zipf(1.05) truncated
to 1..50, raw IDs Zipf(1.05) over 2^40 through the fused Hash + Mod(1e8)
transform, mean pooling, with about 20M resident rows.  The table is filled
by running full steps from empty until 20M rows are resident; then W warm-up
steps; then K timed steps.

--workload seq: the lifelong behaviour sequence (1 feature, length 1000,
batch 2048, dim 128 bf16 storage, gather only, bf16 gradients, Adagrad),
10 full steps from empty before the warm-up.  --workload capacity: the
capacity stress (200M pre-populated rows of dim 64 fp32 + Adam, 100 features,
batch 65536, Poisson(8) bags, 2% novel IDs, sum pooling).

--block-memory host puts the EmbeddingBlocks in pinned host memory (the
IDMap and scratch stay in HBM); the roofline is then taken against the host
link, and the line also gives a pinned copy's rate in each direction.

A step is one pass of the whole path through the C ABI: insert_find
(transform, dedup, IDMap insert / find) -> lookup_pool_fwd -> pool_bwd_update
(duplicate-gradient reduce + optimizer).  Inputs (IDs, bag offsets, upstream
gradients) are resident in HBM before the timed region starts.

Prints one JSON line: IDs/s over the timed steps, the roofline of the
dominant kernel (algorithmic bytes per launch / its mean duration from HIP
events on the launch stream), and (CTR) the CPU oracle timed on a bounded
sample.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import subprocess
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
# the host link of an MI355X: PCIe 5.0 x16, 64 GB/s in each direction
LINK_PEAK_GBS = 64.0
RESIDENT_TARGET = 20_000_000


# The workloads: table spec, shape, how the table is filled before the
# warm-up, default step counts, and the kernels the warm-up times to find the
# dominant one.
WORKLOADS = {
    "ctr": {
        "title": "CTR ranking batch: 26 features merged, dim 64 fp32, batch 8192, Zipf(1.05) bag lengths "
                 "1..50 and IDs over 2^40, Hash+Mod(1e8), mean pooling, sparse Adam, ~20M resident rows",
        "spec": W.spec_ctr, "F": 26, "B": 8192, "fill": "resident", "steps": 20, "warmup": 5,
        "new_per_step": 1_000_000,
        "table": {"slot_capacity": 1 << 27, "block_rows": 1 << 20},
        "candidates": ("k_bwd_short", "k_fwd_pool", "k_bucket_emit", "k_occ_tile", "k_tile"),
    },
    "seq": {
        "title": "Lifelong behaviour sequence: 1 feature of length 1000, batch 2048, dim 128 bf16 storage "
                 "(fp32 accumulate), Zipf(1.2) IDs over 1e8 items, gather only (output [2048,1000,128] "
                 "bf16), bf16 gradients, Adagrad; 10 steps from empty before the warm-up",
        "spec": W.spec_seq, "F": 1, "B": 2048, "fill": "steps", "fill_steps": 10, "steps": 20, "warmup": 5,
        "new_per_step": 250_000,
        "table": {"slot_capacity": 1 << 23, "block_rows": 1 << 20},
        "candidates": ("k_fwd_gather", "k_bwd_short", "k_bwd_long_partial", "k_bucket_emit", "k_occ_tile"),
    },
    "capacity": {
        "title": "Capacity stress: 200M pre-populated rows x dim 64 fp32 + Adam m/v, 100 features, batch 65536, "
                 "bag length Poisson(8), Zipf(1.2) IDs with 2% novel per step, sum pooling",
        "spec": W.spec_capacity, "F": 100, "B": 65536, "fill": "keys", "steps": 5, "warmup": 10,
        # max_load 0.6: before a call the IDMap's growth check counts each of its
        # 52.4M occurrences as a possible new key, so at 0.5 the 2^29-slot map
        # would double (a rehash inside the timed steps) once it held 216M keys,
        # although the keys fill only about 0.42 of it
        "table": {"slot_capacity": 1 << 29, "block_rows": 1 << 20, "max_load": 0.6},
        "candidates": ("k_bwd_short", "k_fwd_pool", "k_bwd_long_partial", "k_occ_tile", "k_bucket_emit"),
        # the oracle baseline: these features of the first timed step (21M IDs)
        "cpu_features": 40,
    },
    # config 1: ten steps from an empty table; launch-bound, so its figure is
    # the step latency
    "tiny": {
        "title": "Tiny single table: dim 16 fp32, 1 feature, batch 256, bag length max(1, Poisson(4)), IDs "
                 "uniform over [0, 1e5), sum pooling, Adagrad lr 0.01; 10 steps from an empty table",
        "spec": W.spec_tiny, "F": 1, "B": 256, "fill": "none", "steps": 10, "warmup": 0,
        "table": {"slot_capacity": 1 << 16, "block_rows": 1 << 14},
        "candidates": (),
    },
    # the five tables of one model, each with its own handle (see run_multi)
    "multi": {
        "title": "Multi-table with admission: 5 tables (dims 8/16/32/64/128) x 60 features, batch 32768, "
                 "bag length max(1, Poisson(4)), Zipf(1.1) IDs over 2^40, mean pooling, Adagrad, a row at "
                 "the 2nd occurrence, 4 steps from empty before the warm-up, then one eviction pass "
                 "(count < 2) per table",
        "special": "multi", "F": 60, "B": 32768, "fill_steps": 4, "steps": 4, "warmup": 2,
        "kernel_filter": "<128,",  # the roofline's kernel is the dim-128 table's
        "reserve_rows": 24_000_000,
        "table": {"slot_capacity": 1 << 26, "block_rows": 1 << 20},
    },
    # exact-assignment writeback into an item cache (see run_cache)
    "cache": {
        "title": "Item-cache writeback: 10M keys pre-inserted, dim 256 bf16, 16,384 writes per step drawn "
                 "with replacement, rows N(0,1) fp32, the last write of a key wins",
        "special": "cache", "keys": 10_000_000, "writes": 16384, "steps": 100, "warmup": 10,
        "table": {"slot_capacity": 1 << 25, "block_rows": 1 << 20},
    },
}


def _gen(arg):
    name, step = arg
    if name == "multi":  # step = (step, table)
        b = W.multi_batch(step[0], step[1], grad=False)
        return [(f.values, f.bag_offsets, f.slot, f.ops, f.mod) for f in b.features], b.batch
    if name == "tiny":
        b = W.tiny_batch(step)
        return [(f.values, f.bag_offsets, f.slot, f.ops, f.mod) for f in b.features], b.batch
    fn = {"ctr": W.ctr_batch, "seq": W.seq_batch, "capacity": W.capacity_batch}[name]
    b = fn(step, grad=False)
    return [(f.values, f.bag_offsets, f.slot, f.ops, f.mod) for f in b.features], b.batch


def gen_batches(name, steps, workers):
    with ProcessPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(_gen, [(name, s) for s in steps]))




def host_info():
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return os.cpu_count(), model


def cpu_baseline(spec, timed, grads, nfeat=None, seconds_budget=20.0, what=""):
    """The oracle, single-threaded, on the timed steps' own inputs: the first
    timed step (only its first `nfeat` features when given), then further
    timed steps while the time stays within the budget.  The oracle's table
    starts empty and holds only the keys these steps touch: a row the GPU
    table holds but the step has not touched is, by the initializer's
    definition, the same as a row made on first touch, so the oracle does the
    same work per distinct key (one row made or read, one update).  The
    gradients are the timed steps' own (the first nfeat features' columns)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    oracle.build(force=False)
    tab = oracle.OracleTable(spec)
    ids, steps, t_total = 0, 0, 0.0
    for (feats, bsz), grad in zip(timed, grads):
        fs = feats if nfeat is None else feats[:nfeat]
        fin = [W.FeatureInput(values=v, bag_offsets=o, slot=sl, ops=ops, mod=mod) for (v, o, sl, ops, mod) in fs]
        g = grad(len(fs))
        t0 = time.perf_counter()
        r = tab.insert_find(fin, bsz)
        tab.forward(r, spec.pool)
        tab.backward_update(r, spec.pool, g, spec.grad_dtype)
        t_total += time.perf_counter() - t0
        ids += sum(f.n for f in fin)
        steps += 1
        if t_total >= seconds_budget or nfeat is not None:
            break
    part = f"features 0..{nfeat - 1} of " if nfeat is not None else ""
    return {"value": ids / t_total, "unit": "IDs/s", "cores": 1, "kind": "oracle",
            "sample": f"{part}{steps} timed step(s) of the {what} workload, the GPU's own inputs and "
                      f"upstream gradients ({ids} IDs; insert_find + forward + backward/update), oracle "
                      f"table holding only the touched keys, single-threaded g++ -O2 oracle, {t_total:.1f} s"}


COPY_BYTES = 1 << 30


def copy_calibration(torch, dev):
    """Three plain device-to-device copies of COPY_BYTES (reads COPY_BYTES,
    writes COPY_BYTES each): the reference for scaling FETCH_SIZE/WRITE_SIZE."""
    x = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()


def hot_mask(keys, counts, batch, dim):
    """The long keys the pooled backward sums bag-major (the rule the
    library's stats field hot_keys documents): per feature bin (key slot
    modulo 4096), of the keys with more than SHORT_MAX occurrences and at
    least 8 per block of 2048 bags, whole count classes floor(log2(count))
    from the top while at most 8192 / dim keys fit."""
    hot = np.zeros(keys.size, bool)
    if dim not in (64, 128):
        return hot
    blocks = -(-batch // 2048)
    kmax = 8192 // dim
    elig = (counts > SHORT_MAX) & (counts >= 8 * blocks) & (keys >= 0)
    bins = (keys >> 48) & 4095
    cls = np.floor(np.log2(np.maximum(counts, 1))).astype(np.int64)
    for b in np.unique(bins[elig]):
        m = elig & (bins == b)
        taken, thr = 0, 32
        for k in range(31, -1, -1):
            x = int((cls[m] == k).sum())
            if taken + x > kmax:
                break
            taken += x
            if x:
                thr = k
        hot |= m & (cls >= thr)
    return hot


def step_shapes(results, U, resident0, hot=None):
    """Per timed step: distinct keys with a row and count <= SHORT_MAX (short)
    or more (long), how many short ones got their row in that step, and the
    occurrences of short keys; of the long keys, those summed bag-major (hot,
    when hot = (batch, dim) says the pass runs) and the chunks of the others;
    averaged over the steps."""
    per = []
    for r, u in zip(results, U):
        counts = r.counts[:u].cpu().numpy().astype(np.int64)
        raw = r.unique_rows[:u].cpu().numpy()
        keys = r.unique_keys[:u].cpu().numpy()
        hm = hot_mask(keys, counts, *hot) if hot else np.zeros(u, bool)
        per.append((counts, raw >= 0, raw & ((1 << 62) - 1), hm))
    # a row allocated in the timed steps is new in the first step that uses it
    cand = [np.nonzero(h & (rw >= resident0))[0] for (_, h, rw, _) in per]
    allrows = np.concatenate([per[k][2][c] for k, c in enumerate(cand)]) if cand else np.zeros(0, np.int64)
    _, first = np.unique(allrows, return_index=True)
    is_first = np.zeros(allrows.size, bool)
    is_first[first] = True
    out, pos = [], 0
    for (counts, has, _, hm), c in zip(per, cand):
        new = np.zeros(counts.size, bool)
        new[c[is_first[pos:pos + c.size]]] = True
        pos += c.size
        short = counts <= SHORT_MAX
        lc = counts[~short & has]
        cold = counts[~short & ~hm]  # the chunked plan takes every long key that is not hot
        out.append({"U_s": int((short & has).sum()), "U_s_new": int((short & new).sum()),
                    "E_s": int(counts[short & has].sum()), "U_l": int((~short & has).sum()),
                    "E_l": int(lc.sum()), "U_hot": int(hm.sum()), "E_hot": int(counts[hm].sum()),
                    "E_l_cold": int(cold.sum()), "chunks_l": int(long_chunks(cold).sum())})
    return {k: float(np.mean([o[k] for o in out])) for k in out[0]}


SHORT_MAX = 64   # occurrences up to which the backward treats a key as short
GRAD_POOL = 8    # distinct upstream gradients staged for the warm-up and timed steps
KEEP_RESULTS = 5  # timed steps whose lookup results are kept for the step shapes
MAX_KEY_CHUNKS = 1024  # a long key is summed in at most this many chunks


def long_chunks(c):
    """Chunks of a long key with c entries: chunks of a multiple of 64 entries,
    at most MAX_KEY_CHUNKS of them."""
    c = np.asarray(c, np.int64)
    per = np.maximum((c + SHORT_MAX * MAX_KEY_CHUNKS - 1) // (SHORT_MAX * MAX_KEY_CHUNKS), 1)
    z = SHORT_MAX * per
    return (c + z - 1) // z


def algorithmic_bytes(shape, N, Um, Unew, Uhit, Bg, D, s=4, S=2, gs=4, pooled=True):
    """Bytes the method must move, per launch / per step (s = parameter bytes,
    S = fp32 state words per element, gs = gradient bytes; P = D s + S D 4
    bytes per row: 768 for the CTR and capacity tables).
      k_bwd_short: per short key 16 (count, group offset, row) + its grouped
        entries 4 each; resident rows read and written 2P, new rows written P;
        the upstream gradient, Bg D gs once when pooled, else one row per entry.
      k_fwd_pool: per occurrence its row reference 8; offsets 4 (Bg + 1);
        resident rows' params D s; the output Bg D 4.
      k_fwd_gather: per occurrence its row reference 8 and its output row D s;
        resident rows' params D s.
      Lookup kernels, with Pp the (key, tile) pairs of the call: the
      distinct keys of each tile of 4096 consecutive occurrences, summed.
      k_tile: per occurrence its raw ID 8 read and its index among its
        tile's pairs 2 written; per pair its key and count 12 written.
      k_pair_scatter: per pair its key and count 12 read, and its partition
        record (key, pair, count) 16 written.
      k_bucket_count: per pair its record's key and count 12.
      k_bucket_emit: per pair its record 16 read and its resolved record
        (forward reference, distinct-key index, group position) 16 written
        at the pair's slot;
        per distinct key its key and count 12, group offset 4, IDMap slot read
        16 and slot index 8; per new key its IDMap slot written 16.
      k_occ_tile: per occurrence its pair index 2 read, and its inverse index
        4, grouped entry 4 and forward reference 8 written; per pair its
        resolved record 16 read; offsets 4 (Bg + 1).
      k_bwd_long_partial: per entry of a long key that is not hot 4; per
        chunk a partial of D fp64 written; the gradient rows of the bags its
        entries touch, at most min(E_l_cold, Bg) pooled (one row per entry
        when not pooled).
      k_hot_sort: per occurrence its distinct-key index 4 and that key's hot
        index 1 read; per hot entry 4 written.
      k_bwd_hot: every bag's gradient row once, Bg D gs; per hot entry 4; per
        hot key a partial of D fp64 per block of 2048 bags written.
      step: insert_find 12 N + 4 (Bg + 1) + 32 U + 16 U_new, forward
        4 N + 8 U + U_hit D s + output, backward 4 N + 8 U + U_hit 2P
        + U_new P + gradient; output and gradient Bg D 4 each when pooled,
        N D s and N D gs when not."""
    P = D * s + S * D * 4
    Us, Usn = shape["U_s"], shape["U_s_new"]
    g_short = Bg * D * gs if pooled else shape["E_s"] * D * gs
    bwd_short = 16 * Us + 4 * shape["E_s"] + (Us - Usn) * 2 * P + Usn * P + g_short
    fwd = 8 * N + 4 * (Bg + 1) + Uhit * D * s + Bg * D * 4
    gather = 8 * N + Uhit * D * s + N * D * s
    Pp = shape.get("pairs", 0)
    tile = 10 * N + 12 * Pp
    scatter = 28 * Pp
    count = 12 * Pp
    emit = 32 * Pp + 40 * Um + 16 * Unew
    occ = 18 * N + 16 * Pp + 4 * (Bg + 1)
    El = shape.get("E_l_cold", shape["E_l"])
    g_long = min(El, Bg) * D * gs if pooled else El * D * gs
    long_partial = 4 * El + shape["chunks_l"] * D * 8 + g_long
    Eh, Uh = shape.get("E_hot", 0), shape.get("U_hot", 0)
    hot_sort = 5 * N + 4 * Eh if Uh else 0
    hot_pass = Bg * D * gs + 4 * Eh + Uh * shape.get("hot_nc", 1) * D * 8 if Uh else 0
    out_b, grad_b = (Bg * D * 4, Bg * D * 4) if pooled else (N * D * s, N * D * gs)
    ins = 12 * N + 4 * (Bg + 1) + 32 * Um + 16 * Unew
    fwd_call = 4 * N + 8 * Um + Uhit * D * s + out_b
    bwd_call = 4 * N + 8 * Um + Uhit * 2 * P + Unew * P + grad_b
    return {"k_bwd_short": bwd_short, "k_fwd_pool": fwd, "k_fwd_gather": gather,
            "k_tile": tile, "k_pair_scatter": scatter, "k_bucket_count": count, "k_bucket_emit": emit,
            "k_occ_tile": occ, "k_hot_sort": hot_sort, "k_bwd_hot": hot_pass,
            "k_bwd_long_partial": long_partial, "step": ins + fwd_call + bwd_call}


def link_bytes(kernel, shape, Uhit, D, s=4, S=2):
    """(read, written) bytes of EmbeddingBlock rows that `kernel` moves across
    the host link per launch when the blocks are in host memory (the IDMap,
    inputs, outputs and scratch stay in HBM): the rows the method must read
    and write, as in algorithmic_bytes."""
    P = D * s + S * D * 4
    Us, Usn = shape["U_s"], shape["U_s_new"]
    return {"k_bwd_short": ((Us - Usn) * P, Us * P),
            "k_fwd_pool": (Uhit * D * s, 0), "k_fwd_gather": (Uhit * D * s, 0),
            "k_bwd_long_final": (shape["U_l"] * P, shape["U_l"] * P)}.get(kernel, (0, 0))


def host_link_copy(torch, dev, nbytes=1 << 30):
    """GB/s of one pinned host-to-device and one device-to-host copy."""
    h = torch.empty(nbytes // 4, dtype=torch.float32, pin_memory=True)
    d = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    out = {}
    for name, (dst, src) in (("h2d", (d, h)), ("d2h", (h, d))):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dst.copy_(src, non_blocking=True)  # once untimed
        a.record()
        dst.copy_(src, non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        out[name] = nbytes / (a.elapsed_time(b) * 1e-3) / 1e9
    return out


def export_import(torch, recis, table, spec, wl, D, s, S, block_memory):
    """The device side of a save and restore: the whole table exported to
    device arrays, then imported into a new table with room for it.  The
    import kernel moves per key its key, row flag and count (20 B) and its
    IDMap slot (16 B), and per key with a row the row's P bytes read and P
    written."""
    P = D * s + S * D * 4
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ex = table.export()
    torch.cuda.synchronize()
    t_export = time.perf_counter() - t0
    n = int(ex["keys"].shape[0])
    nrow = int((ex["rows"] >= 0).sum().item())
    fresh = recis.Table(D, spec.dtype, spec.optim, seed=spec.seed, init_bound=spec.init_bound,
                        admit_threshold=spec.admit_threshold, reserve_rows=nrow + 1,
                        slot_capacity=wl["table"]["slot_capacity"], block_rows=wl["table"]["block_rows"],
                        block_memory=block_memory)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    counts = ex["counts"]
    a.record()
    fresh.import_(ex["keys"], ex["rows"], counts, ex["params"], ex["state"] if S else None)
    b.record()
    torch.cuda.synchronize()
    fresh.check()
    st = fresh.stats()
    assert st.keys == n and st.rows_in_use == nrow, (st.keys, n, st.rows_in_use, nrow)
    t_import = a.elapsed_time(b) * 1e-3
    alg = 36 * n + 2 * P * nrow
    fresh.close()
    return {"keys": n, "rows": nrow, "export_s": t_export, "import_ms": t_import * 1e3,
            "import_algorithmic_bytes": alg, "import_GBps": alg / t_import / 1e9,
            "import_frac": alg / t_import / 1e9 / HBM_PEAK_GBS}


def evict_lru_pass(torch, table):
    """One LRU-bounded pass to half the table's keys, wall-clock (it
    synchronises).  It moves per IDMap slot 16 B read and 4 B of stamp read
    by the age histogram, the same again by the marking, and 32 B by the
    rebuild; per surviving key 16 B written."""
    st0 = table.stats()
    slots = int(st0.slot_capacity)
    ne = torch.zeros(1, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    table.evict_lru(int(st0.keys) // 2, ne)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    table.check()
    st1 = table.stats()
    alg = 72 * slots + 16 * int(st1.keys)
    return {"max_keys": int(st0.keys) // 2, "keys_before": int(st0.keys), "evicted": int(ne.item()),
            "keys_after": int(st1.keys), "slots": slots, "ms": dt * 1e3, "algorithmic_bytes": alg,
            "GBps": alg / dt / 1e9, "frac": alg / dt / 1e9 / HBM_PEAK_GBS}


def evict_pass(torch, table, min_count=2, decay=0.5):
    """One eviction pass over the whole table, wall-clock (the call reads the
    device counters back, so it synchronises).  It moves per IDMap slot 16 B
    read by the marking pass, and for the rebuild 16 B filled and 16 B read;
    per surviving key 16 B written."""
    st0 = table.stats()
    slots = int(st0.slot_capacity)
    ne = torch.zeros(1, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    table.evict(min_count, ne, decay=decay)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    table.check()
    st1 = table.stats()
    alg = 48 * slots + 16 * int(st1.keys)
    return {"min_count": min_count, "decay": decay, "keys_before": int(st0.keys), "evicted": int(ne.item()),
            "keys_after": int(st1.keys), "slots": slots, "ms": dt * 1e3, "algorithmic_bytes": alg,
            "GBps": alg / dt / 1e9, "frac": alg / dt / 1e9 / HBM_PEAK_GBS}


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dynamic_embedding_tables_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload="ctr"):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/<kernel>_<workload>_counters.txt: FETCH_SIZE / WRITE_SIZE in KiB
    per dispatch, scaled by the copy-kernel factors), or None when there is
    none or the kernel sources changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _kernel_label(name):
    import re
    m = re.search(r"(k_[a-z_]+)", name)
    if m:
        if m.group(1) == "k_bucket":  # the two launches of the bucket kernel: k_bucket<TAB, EMIT, ...>
            return "k_bucket_emit" if re.search(r"k_bucket<\d+, true", name) else "k_bucket_count"
        return m.group(1)
    if "copy" in name:
        return "copy"
    return name[:60]


def summarize(prof_dir, kernel, command, out_path, workload="ctr", block_memory="device"):
    """Writes the committed summary of a profiled bench run: per-kernel mean
    durations (rocprofv3 --kernel-trace --stats, csv) from prof_dir/trace, and
    for `kernel` the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch, from
    prof_dir/fetch and prof_dir/write, when those runs exist) scaled by the
    same counters of the plain copies of COPY_BYTES that --copy-calibration
    runs."""
    import csv
    stats = list(csv.DictReader(open(os.path.join(prof_dir, "trace", "p_kernel_stats.csv"))))
    where = "" if block_memory == "device" else " (EmbeddingBlocks in pinned host memory)"
    lines = [f"# rocprofv3 summary: {kernel} on the workload: {WORKLOADS[workload]['title']}{where}",
             f"# command: {command}", f"kernel={kernel}", f"source_hash={kernel_source_hash()}"]
    dur = {}
    for r in stats:
        lab = _kernel_label(r["Name"])
        dur.setdefault(lab, []).append((float(r["AverageNs"]), int(r["Calls"]), float(r["Percentage"])))
    for lab, v in sorted(dur.items(), key=lambda kv: -sum(x[2] for x in kv[1])):
        avg = sum(a * c for a, c, _ in v) / sum(c for _, c, _ in v)
        lines.append(f"kernel_avg_us[{lab}]={avg / 1e3:.2f}  calls={sum(c for _, c, _ in v)}  "
                     f"pct={sum(p for *_, p in v):.2f}")
    # (a workload with several tables names the instance the bench times)
    flt = WORKLOADS[workload].get("kernel_filter", "")
    mine = [(float(r["AverageNs"]), int(r["Calls"])) for r in stats
            if _kernel_label(r["Name"]) == kernel and flt in r["Name"]]
    lines.append(f"avg_duration_us={sum(a * c for a, c in mine) / sum(c for _, c in mine) / 1e3:.2f}"
                 + (f"  (instances named *{flt}*)" if flt else ""))
    # the timed steps are the last dispatches of the run (the table fill
    # before the warm-up can call the same kernel on other sizes)
    trace = [r for r in csv.DictReader(open(os.path.join(prof_dir, "trace", "p_kernel_trace.csv")))
             if _kernel_label(r["Kernel_Name"]) == kernel and flt in r["Kernel_Name"]]
    last = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace[-5:]]
    if last:
        lines.append(f"timed_steps_avg_duration_us={np.mean(last) / 1e3:.2f}  (last {len(last)} dispatches)")

    def counter(sub, cname):
        rows = list(csv.DictReader(open(os.path.join(prof_dir, sub, "p_counter_collection.csv"))))
        per = {}
        for r in rows:
            if r["Counter_Name"] != cname:
                continue
            lab = _kernel_label(r["Kernel_Name"])
            if lab == kernel and flt not in r["Kernel_Name"]:
                continue
            v = float(r["Counter_Value"])
            # the calibration copies are the copy dispatches that move COPY_BYTES
            # (a counter that reads 1/4 or more of it); other copies are small
            if lab == "copy" and v * 1024 < COPY_BYTES / 4:
                continue
            per.setdefault(lab, []).append(v)
        return per
    if not os.path.isdir(os.path.join(prof_dir, "fetch")):  # a kernel-trace run only
        open(out_path, "w").write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    fetch, write = counter("fetch", "FETCH_SIZE"), counter("write", "WRITE_SIZE")
    cf, cw = fetch.get("copy", [])[-3:], write.get("copy", [])[-3:]
    kf, kw = fetch.get(kernel, []), write.get(kernel, [])
    if cf and cw and kf and kw:
        fs = COPY_BYTES / (np.mean(cf) * 1024.0)
        ws = COPY_BYTES / (np.mean(cw) * 1024.0)
        # the timed steps are the last dispatches of the run
        f_kib, w_kib = float(np.mean(kf[-5:])), float(np.mean(kw[-5:]))
        lines += [f"copy_bytes={COPY_BYTES}", f"copy_fetch_kib={np.mean(cf):.1f}", f"copy_write_kib={np.mean(cw):.1f}",
                  f"fetch_scale={fs:.4f}", f"write_scale={ws:.4f}",
                  f"fetch_kib_per_dispatch={f_kib:.1f}", f"write_kib_per_dispatch={w_kib:.1f}",
                  f"traffic_bytes_per_launch={f_kib * 1024 * fs + w_kib * 1024 * ws:.0f}"]
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_atomics(prof_dir, command, out_path, workload="ctr", last=5):
    """Writes the committed summary of a TCC_ATOMIC / TCC_EA0_ATOMIC run
    (rocprofv3 --pmc, csv, in prof_dir/atomics): device-scope atomics per
    dispatch of every kernel over its last `last` dispatches (the timed
    steps) -- the IDMap's insert / find and the rest of the step."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(prof_dir, "atomics", "p_counter_collection.csv"))))
    per = {}
    for r in rows:
        lab = _kernel_label(r["Kernel_Name"])
        per.setdefault((lab, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    lines = [f"# rocprofv3 summary: device atomics per dispatch on the workload: {WORKLOADS[workload]['title']}",
             f"# command: {command}", f"source_hash={kernel_source_hash()}"]
    for (lab, cname), v in sorted(per.items()):
        if lab == "copy" or lab.startswith("void at::"):
            continue
        lines.append(f"{cname}[{lab}]={np.mean(v[-last:]):.0f}  (last {min(last, len(v))} dispatches)")
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _upload(torch, recis, dev, batch):
    feats, _ = batch
    dfs = [recis.DeviceFeature(torch.from_numpy(v).to(dev), torch.from_numpy(o).to(dev), sl, ops, mod)
           for (v, o, sl, ops, mod) in feats]
    return dfs, recis.make_descs(dfs), sum(f.n for f in dfs)


def run_multi(args, wl):
    """The five tables of one model through full steps (per table: insert_find
    with admission at the 2nd occurrence, mean-pooled forward, backward with
    Adagrad), then one eviction pass per table.  value = IDs/s over all five
    tables; the roofline is k_bwd_short of the dim-128 table, timed by HIP
    events in every timed step."""
    import torch
    from dynamic_embedding_tables_amd import recis
    K = args.steps if args.steps is not None else wl["steps"]
    Wm = args.warmup if args.warmup is not None else wl["warmup"]
    nfill, F, B = wl["fill_steps"], wl["F"], wl["B"]
    T = len(W.MULTI_DIMS)
    t_gen = time.perf_counter()
    with ProcessPoolExecutor(max_workers=args.workers) as ex:
        batches = list(ex.map(_gen, [("multi", (s, t)) for s in range(nfill + Wm + K) for t in range(T)]))
    print(f"[bench] multi: generated {len(batches)} batches in {time.perf_counter() - t_gen:.1f}s",
          file=sys.stderr, flush=True)
    recis.load_library()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    specs = [W.spec_multi(t) for t in range(T)]
    cap = max(sum(v.shape[0] for (v, *_r) in b[0]) for b in batches)
    tables = [recis.Table(sp.dim, sp.dtype, sp.optim, seed=sp.seed, init_bound=sp.init_bound,
                          admit_threshold=sp.admit_threshold, reserve_rows=wl["reserve_rows"], **wl["table"])
              for sp in specs]
    gen = torch.Generator(device=dev)
    gen.manual_seed(20250925)

    def fresh_grad(t):
        """A new N(0,1) upstream gradient for one step of table t."""
        return torch.randn(B, F * specs[t].dim, device=dev, generator=gen, dtype=torch.float32)

    outs = [torch.empty(B, F * sp.dim, device=dev, dtype=torch.float32) for sp in specs]
    res = [recis.LookupResult(cap, F * B) for _ in range(T)]
    big = T - 1

    def step_table(t, dfs, descs, r, grad):
        sp = specs[t]
        tables[t].insert_find(dfs, B, r, descs=descs)
        tables[t].forward(r, sp.pool, outs[t])
        tables[t].backward_update(r, sp.pool, grad, sp.grad_dtype, lr=sp.lr, beta1=sp.beta1,
                                  beta2=sp.beta2, eps=sp.eps)

    for s in range(nfill):
        for t in range(T):
            dfs, descs, _ = _upload(torch, recis, dev, batches[s * T + t])
            step_table(t, dfs, descs, res[t], fresh_grad(t))
        torch.cuda.synchronize()
    # warm-up and timed inputs in HBM, each step with its own gradient
    staged = [_upload(torch, recis, dev, batches[j]) + (fresh_grad(j % T),)
              for j in range(nfill * T, (nfill + Wm + K) * T)]
    for w in range(Wm):
        for t in range(T):
            dfs, descs, _, g = staged[w * T + t]
            step_table(t, dfs, descs, res[t], g)
    for tb in tables:
        tb.check()
    st0 = [tb.stats() for tb in tables]
    stream = torch.cuda.current_stream()
    timed_res = [recis.LookupResult(cap, F * B) for _ in range(K)]
    kev = []
    for _ in range(K):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        b.record(stream)
        kev.append((a, b))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(T + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record(stream)
        for t in range(T):
            dfs, descs, _, g = staged[(Wm + k) * T + t]
            if t == big:
                tables[t].profile_kernel("k_bwd_short", *kev[k])
            step_table(t, dfs, descs, timed_res[k] if t == big else res[t], g)
            if t == big:
                tables[t].profile_kernel(None)
            ev[k][t + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for tb in tables:
        tb.check()
    st1 = [tb.stats() for tb in tables]
    ids = sum(staged[(Wm + k) * T + t][2] for k in range(K) for t in range(T))
    per_table = [float(np.mean([ev[k][t].elapsed_time(ev[k][t + 1]) for k in range(K)])) for t in range(T)]
    t_dom = float(np.mean([a.elapsed_time(b) for a, b in kev])) * 1e-3
    U = [int(r.num_unique.item()) for r in timed_res]
    shape = step_shapes(timed_res, U, int(st0[big].rows_in_use))
    D = specs[big].dim
    a_bytes = algorithmic_bytes(shape, 0, 0, 0, 0, F * B, D, 4, 1, 4, True)["k_bwd_short"]
    achieved = a_bytes / t_dom / 1e9
    if args.copy_calibration:
        copy_calibration(torch, dev)
    evict = [evict_pass(torch, tb, min_count=2, decay=0.0) for tb in tables]
    result = {
        "metric": "lookup+pool+update IDs/sec and achieved HBM GB/s vs peak, 1xMI355X",
        "value": ids / elapsed, "unit": "IDs/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": elapsed / K * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl["title"], "global_batch": B, "num_features": F, "tables": T,
                   "dims": list(W.MULTI_DIMS), "ids_per_step": ids / K,
                   "keys_end": [int(s.keys) for s in st1], "rows_end": [int(s.rows_in_use) for s in st1],
                   "parallelism": "single GPU"},
        "table_step_ms": per_table,
        "roofline": {"bound": "hbm", "kernel": "k_bwd_short", "table_dim": D, "kernel_ms": t_dom * 1e3,
                     "algorithmic_bytes": a_bytes, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": read_traffic("k_bwd_short", "multi")},
        "backward_key_split": shape,
        "evict_pass": evict,
    }
    print(json.dumps(result))


def run_cache(args, wl):
    """Exact-assignment writeback into an item cache: K calls of
    recis_writeback, each with 16,384 (key, row) pairs drawn with replacement
    from 10M resident keys.  Per call the method moves 8 B per written key,
    and per distinct key its last row read in fp32 (4 D), the stored row
    written (2 D, bf16) and its IDMap slot read (16 B); the dedup table and
    the distinct list add 16 B per write and 24 B per distinct key.  The
    whole call (three launches) is timed by HIP events on its stream."""
    import torch
    from dynamic_embedding_tables_amd import recis
    K = args.steps if args.steps is not None else wl["steps"]
    Wm = args.warmup if args.warmup is not None else wl["warmup"]
    spec = W.spec_cache()
    D, n = spec.dim, wl["writes"]
    keys = W.cache_keys(wl["keys"])
    writes = [W.cache_writes(s, keys, n=n, dim=D) for s in range(Wm + K)]
    distinct = [int(np.unique(k).size) for k, _ in writes[Wm:]]
    recis.load_library()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    table = recis.Table(D, spec.dtype, spec.optim, seed=spec.seed, init_bound=spec.init_bound,
                        reserve_rows=wl["keys"] + (1 << 20), **wl["table"])
    chunk = 1 << 20
    zero = torch.zeros(chunk, D, device=dev, dtype=torch.float32)
    for c0 in range(0, keys.size, chunk):
        kd = torch.from_numpy(keys[c0:c0 + chunk]).to(dev)
        table.writeback(kd, zero[:kd.numel()])
    torch.cuda.synchronize()
    table.check()
    staged = [(torch.from_numpy(k).to(dev), torch.from_numpy(e).to(dev)) for k, e in writes]
    for w in range(Wm):
        table.writeback(*staged[w])
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record(stream)
        table.writeback(*staged[Wm + k])
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    table.check()
    st = table.stats()
    t_call = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    Ud = float(np.mean(distinct))
    a_bytes = 8 * n + 16 * n + Ud * (4 * D + 2 * D + 16 + 24)
    achieved = a_bytes / t_call / 1e9
    result = {
        "metric": "writeback rows/sec (exact assignment) and achieved HBM GB/s vs peak, 1xMI355X",
        "value": n * K / elapsed, "unit": "rows/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": elapsed / K * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl["title"], "writes_per_step": n, "distinct_per_step": Ud, "dim": D,
                   "keys_end": int(st.keys), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "recis_writeback (k_set_scratch, k_wb_dedup, k_wb_apply)",
                     "kernel_ms": t_call * 1e3, "algorithmic_bytes": a_bytes, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None},
    }
    table.close()
    print(json.dumps(result))


def parse_args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=None,
                    help="one workload alone (default: the capacity line, with the tiny, CTR and sequence "
                         "workloads as extra keys)")
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: the workload's)")
    ap.add_argument("--warmup", type=int, default=None, help="warm-up steps (default: the workload's)")
    ap.add_argument("--no-extras", action="store_true", help="default line: skip the extra workloads")
    ap.add_argument("--resident", type=int, default=RESIDENT_TARGET, help="CTR: rows resident before warm-up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--export-import", action="store_true",
                    help="after the timed steps, export the whole table and import it into a new one (the "
                         "device side of saving and restoring), timed against the HBM roofline")
    ap.add_argument("--evict-pass", action="store_true",
                    help="after the timed steps, one eviction pass with decayed counts (min count 2, decay "
                         "0.5) over the whole table, timed against the HBM roofline (with --track-last-use, "
                         "first an LRU-bounded pass to half the keys)")
    ap.add_argument("--track-last-use", action="store_true",
                    help="the table stamps every key a lookup counts (for LRU-bounded eviction)")
    ap.add_argument("--admit-sketch-bits", type=int, default=0,
                    help="count-min sketch admission with 4 x 2^bits counters (the workload's admission "
                         "threshold; timing only: the default line keeps exact admission)")
    ap.add_argument("--block-memory", choices=["device", "host"], default="device",
                    help="where the EmbeddingBlocks live: HBM, or pinned host memory across the host link")
    ap.add_argument("--device-rows", type=int, default=0,
                    help="with --block-memory host: rows of the HBM tier in front of the host blocks")
    ap.add_argument("--retier-every", type=int, default=0,
                    help="with an HBM tier: a hot-tier pass (recis_idmap_retier) after every K-th step, "
                         "warm-up and timed steps alike (its time is part of the step time)")
    ap.add_argument("--workers", type=int, default=8)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run plain device copies of known size (for HBM counter scaling)")
    ap.add_argument("--summarize", metavar="PROF_DIR",
                    help="write the profiles/ summary of a profiled run (see summarize()) and exit")
    ap.add_argument("--kernel", default="k_bwd_short")
    ap.add_argument("--summarize-atomics", metavar="PROF_DIR")
    ap.add_argument("--command", default="")
    ap.add_argument("--out", default=None)
    return ap.parse_args(argv)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def run_standard(name, args, K=None, Wm=None, cpu=True, extra=False):
    """One of the single-table workloads (tiny, ctr, seq, capacity) through K
    timed steps; returns the result dict.  extra: a shorter run for the extra
    keys of the default line (no export, eviction or host-memory options)."""
    import torch
    from dynamic_embedding_tables_amd import recis
    wl = WORKLOADS[name]
    K = K if K is not None else (args.steps if args.steps is not None and not extra else wl["steps"])
    Wm = Wm if Wm is not None else (args.warmup if args.warmup is not None and not extra else wl["warmup"])
    block_memory = "device" if extra else args.block_memory
    spec = wl["spec"]()
    F, B, D = wl["F"], wl["B"], spec.dim
    pooled = spec.pool != "none"
    s_bytes = 2 if spec.dtype == "bf16" else 4
    S = {"adam": 2, "adagrad": 1}[spec.optim]
    gs = 2 if spec.grad_dtype == "bf16" else 4
    # ---- inputs: generated in a process pool (the first call before the GPU is touched)
    t_gen = time.perf_counter()
    if wl["fill"] == "resident":
        fill_steps = int(np.ceil(args.resident / 850_000)) + 4
    elif wl["fill"] == "steps":
        fill_steps = wl["fill_steps"]
    else:
        fill_steps = 0
    batches = gen_batches(name, list(range(fill_steps + Wm + K)), args.workers)
    resident_keys = list(W.capacity_resident_keys()) if wl["fill"] == "keys" else []
    log(f"{name}: generated {len(batches)} batches in {time.perf_counter() - t_gen:.1f}s")

    recis.load_library()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    cap = max(sum(v.shape[0] for (v, *_r) in b[0]) for b in batches)
    pre_rows = sum(k.shape[0] for _, k in resident_keys)
    if wl["fill"] == "keys":  # a call may add up to its N rows; 2% of N are new per step (2.2% reserved)
        reserve = pre_rows + cap + (Wm + K + 1) * (cap // 45)
    elif wl["fill"] == "resident":  # the fill stops within one step of the target
        reserve = args.resident + (Wm + K + 3) * wl["new_per_step"]
    elif wl["fill"] == "steps":
        reserve = (fill_steps + Wm + K + 2) * wl["new_per_step"]
    else:
        reserve = (Wm + K) * cap
    table = recis.Table(D, spec.dtype, spec.optim, seed=spec.seed, init_bound=spec.init_bound,
                        admit_threshold=spec.admit_threshold, reserve_rows=reserve,
                        block_memory=block_memory, track_last_use=args.track_last_use and not extra,
                        admit_sketch_bits=0 if extra else args.admit_sketch_bits,
                        device_rows=args.device_rows if block_memory == "host" else 0, **wl["table"])
    retier_every = args.retier_every if block_memory == "host" and args.device_rows > 0 else 0
    gen = torch.Generator(device=dev)
    gen.manual_seed(20250925)
    pdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    gdt = torch.bfloat16 if spec.grad_dtype == "bf16" else torch.float32
    flags = 0 if pooled else recis.RECIS_GROUP_BY_OCCURRENCE

    grad_pool = []

    def upload(batch, j=None):
        """The batch's IDs and offsets in HBM, and its N(0,1) upstream
        gradient: a fresh one for a fill step (j None), else gradient j of the
        staged pool (one per timed step while they number at most GRAD_POOL,
        then reused in turn; the warm-up steps reuse them too)."""
        feats, bsz = batch
        dfs = [recis.DeviceFeature(torch.from_numpy(v).to(dev), torch.from_numpy(o).to(dev), sl, ops, mod)
               for (v, o, sl, ops, mod) in feats]
        n = sum(f.n for f in dfs)
        if j is None:
            shape = (bsz, F * D) if pooled else (n, D)
            grad = torch.randn(*shape, device=dev, generator=gen, dtype=torch.float32).to(gdt)
        else:
            grad = grad_pool[j % len(grad_pool)]
            grad = grad if pooled else grad[:n]
        return dfs, recis.make_descs(dfs), n, grad

    out = torch.empty(B, F * D, device=dev, dtype=torch.float32) if pooled else \
        torch.empty(cap, D, device=dev, dtype=pdt)
    res_pool = [recis.LookupResult(cap, F * B) for _ in range(2)]

    def fwd(res):
        table.forward(res, spec.pool, out)

    def bwd(res, grad):
        table.backward_update(res, spec.pool, grad, spec.grad_dtype, lr=spec.lr, beta1=spec.beta1,
                              beta2=spec.beta2, eps=spec.eps)

    def step(dfs, descs, grad, res):
        table.insert_find(dfs, B, res, flags=flags, descs=descs)
        fwd(res)
        bwd(res, grad)

    retier_ms = []

    def maybe_retier(k):
        """The hot-tier pass after every retier_every-th step (it synchronises)."""
        if retier_every and (k + 1) % retier_every == 0:
            moved = torch.zeros(1, dtype=torch.int64, device=dev)
            t0 = time.perf_counter()
            table.retier(moved)
            retier_ms.append(((time.perf_counter() - t0) * 1e3, int(moved.item())))

    # ---- fill the table (untimed)
    i = 0
    if wl["fill"] == "keys":  # pre-populate: each feature's resident IDs, one per bag
        for j, (f, keys) in enumerate(resident_keys):
            kd = torch.from_numpy(keys).to(dev)
            od = torch.arange(keys.shape[0] + 1, dtype=torch.int32, device=dev)
            r = recis.LookupResult(keys.shape[0], keys.shape[0])
            table.insert_find([recis.DeviceFeature(kd, od, f)], keys.shape[0], r)
            del r, kd, od
            if j % 25 == 24:
                log(f"{name} fill: {j + 1} features' resident keys inserted")
        torch.cuda.synchronize()
        table.check()
    else:
        while i < fill_steps:
            dfs, descs, n, grad = upload(batches[i])
            step(dfs, descs, grad, res_pool[i % 2])
            i += 1
            if wl["fill"] == "resident" and table.stats().rows_in_use >= args.resident:
                break
    resident0 = table.stats().rows_in_use
    log(f"{name} fill: {i} steps, {resident0} resident rows")

    # ---- stage warm-up + timed inputs in HBM.  Device memory stays within
    # bounds for any K: at most GRAD_POOL upstream gradients (1.7 GB each on the
    # capacity workload), and full lookup results (2.3 GB each there) for the
    # first KEEP_RESULTS timed steps only -- the measured step shapes come from
    # those; later timed steps reuse the two fill buffers in turn.
    first_timed = i + Wm
    for _ in range(min(GRAD_POOL, max(K, 1))):
        shape = (B, F * D) if pooled else (cap, D)
        grad_pool.append(torch.randn(*shape, device=dev, generator=gen, dtype=torch.float32).to(gdt))
    staged = [upload(batches[i + w], w) for w in range(Wm)] + [upload(batches[i + Wm + k], k) for k in range(K)]
    timed_res = [recis.LookupResult(cap, F * B) for _ in range(min(K, KEEP_RESULTS))]
    stream = torch.cuda.current_stream()

    def event_pair():
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)  # creates the HIP events, so the library can record them
        b.record(stream)
        return a, b

    # warm-up; each warm-up step also times one candidate kernel, to find the
    # dominant one (the kernel with the longest launch)
    cands = wl["candidates"]
    probe_ms = {}
    for w in range(Wm):
        dfs, descs, n, grad = staged[w]
        name_k = cands[w % len(cands)] if cands else None
        if name_k:
            a, b = event_pair()
            table.profile_kernel(name_k, a, b)
        step(dfs, descs, grad, res_pool[w % 2])
        torch.cuda.synchronize()
        if name_k:
            probe_ms.setdefault(name_k, []).append(a.elapsed_time(b))
        maybe_retier(w)
    table.profile_kernel(None)
    # the longest; a candidate within 5% of it that comes earlier in the list
    # wins, so that two kernels of about the same length (the sequence
    # workload's backward and gather) do not trade places from run to run
    dom = None
    if probe_ms:
        top = max(np.mean(v) for v in probe_ms.values())
        dom = next(k for k in cands if k in probe_ms and np.mean(probe_ms[k]) >= 0.95 * top)
    table.check()
    st0 = table.stats()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    kev = [event_pair() for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        dfs, descs, n, grad = staged[Wm + k]
        res = timed_res[k] if k < len(timed_res) else res_pool[k % 2]
        e = ev[k]
        if dom:
            table.profile_kernel(dom, *kev[k])
        e[0].record(stream)
        table.insert_find(dfs, B, res, flags=flags, descs=descs)
        e[1].record(stream)
        fwd(res)
        e[2].record(stream)
        bwd(res, grad)
        e[3].record(stream)
        maybe_retier(Wm + k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    free_b, total_b = torch.cuda.mem_get_info()
    log(f"{name}: {K} timed steps in {elapsed * 1e3:.1f} ms; device memory free {free_b / 1e9:.1f} of "
        f"{total_b / 1e9:.1f} GB")
    table.profile_kernel(None)
    table.check()
    st1 = table.stats()
    t_dom = float(np.mean([a.elapsed_time(b) for a, b in kev])) * 1e-3 if dom else None
    if args.copy_calibration and not extra:
        copy_calibration(torch, dev)

    ids = sum(staged[Wm + k][2] for k in range(K))
    U = [int(r.num_unique.item()) for r in timed_res]
    new_rows = st1.rows_in_use - st0.rows_in_use
    t_ins = np.mean([e[0].elapsed_time(e[1]) for e in ev]) * 1e-3
    t_fwd = np.mean([e[1].elapsed_time(e[2]) for e in ev]) * 1e-3
    t_bwd = np.mean([e[2].elapsed_time(e[3]) for e in ev]) * 1e-3
    t_steps = [e[0].elapsed_time(e[3]) for e in ev]

    # Measured shape of each timed step: N, U, and per distinct key its count and
    # whether its row is new (allocated in this step: no eviction runs here, so a
    # row >= the resident count before the timed steps that no earlier timed
    # step used).
    N = ids / K
    Um = float(np.mean(U))
    Unew = new_rows / K
    Uhit = Um - Unew
    Bg = F * B
    # the hot keys by the documented rule, checked against the library's count
    hot_lib = (st1.hot_keys - st0.hot_keys) / K
    shape = step_shapes(timed_res, U, int(st0.rows_in_use), hot=(B, D) if pooled and hot_lib > 0 else None)
    shape["hot_keys_counted_by_library"] = hot_lib
    shape["hot_nc"] = -(-B // 2048)
    shape["pairs"] = (st1.lookup_pairs - st0.lookup_pairs) / K
    alg = algorithmic_bytes(shape, N, Um, Unew, Uhit, Bg, D, s_bytes, S, gs, pooled)
    a_bytes = alg[dom] if dom in alg else None
    achieved = a_bytes / t_dom / 1e9 if a_bytes else None
    step_bytes = alg["step"]
    traffic = read_traffic(dom, name) if dom else None
    claims = (st1.claim_attempts - st0.claim_attempts) / K
    lost = (st1.claim_failures - st0.claim_failures) / K
    # rows in host blocks: the share of the timed lookups' rows past the HBM
    # tier (all of them without one) scales the rows that cross the host link
    host_keys, host_share = [], 1.0
    if block_memory == "host":
        H = int(st1.hbm_rows)
        with_rows = []
        for r, u in zip(timed_res, U):
            rw = r.unique_rows[:u].cpu().numpy()
            rw = rw[rw >= 0] & ((1 << 62) - 1)
            host_keys.append(int(np.count_nonzero(rw >= H)))
            with_rows.append(int(rw.size))
        host_share = sum(host_keys) / max(sum(with_rows), 1)

    def link(kernel):
        rd, wr = link_bytes(kernel, shape, Uhit, D, s_bytes, S)
        return rd * host_share, wr * host_share

    result = {
        "metric": "lookup+pool+update IDs/sec and achieved HBM GB/s vs peak, 1xMI355X",
        "value": ids / elapsed,
        "unit": "IDs/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl["title"],
            "global_batch": B, "num_features": F, "dim": D, "storage": spec.dtype,
            "ids_per_step": N, "unique_per_step": Um, "new_rows_per_step": Unew,
            "resident_rows_start": int(st0.rows_in_use), "resident_rows_end": int(st1.rows_in_use),
            # timed steps with a gradient of their own (reused in turn past it), and the
            # first timed steps whose lookup results give the measured step shape
            "distinct_timed_gradients": len(grad_pool), "shape_from_first_steps": len(timed_res),
            "parallelism": "single GPU",
        },
        "step_breakdown_ms": {"insert_find": t_ins * 1e3, "lookup_pool_fwd": t_fwd * 1e3,
                              "pool_bwd_update": t_bwd * 1e3},
        "step_ms_median_p90": [float(np.median(t_steps)), float(np.percentile(t_steps, 90))],
        # the whole step against the HBM roofline: the step's algorithmic bytes
        # over the wall-clock time per step
        "step_roofline": {"bound": "hbm", "algorithmic_bytes": step_bytes,
                          "achieved": step_bytes / (elapsed / K) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": step_bytes / (elapsed / K) / 1e9 / HBM_PEAK_GBS},
        "idmap_claims_per_step": {"attempts": claims, "lost": lost,
                                  "attempts_per_s": claims / (elapsed / K)},
        "roofline": ({"bound": "hbm", "kernel": dom, "kernel_ms": t_dom * 1e3,
                      "algorithmic_bytes": a_bytes, "achieved": achieved, "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS if achieved else None,
                      "traffic": traffic} if block_memory == "device" else
                     # rows in host memory: the dominant kernel against the host link, in
                     # the direction that carries more of its row bytes
                     {"bound": "host-link", "kernel": dom, "kernel_ms": t_dom * 1e3,
                      "link_bytes_read_written": list(link(dom)), "host_row_share": host_share,
                      "achieved": max(link(dom)) / t_dom / 1e9,
                      "peak": LINK_PEAK_GBS, "unit": "GB/s",
                      "frac": max(link(dom)) / t_dom / 1e9 / LINK_PEAK_GBS,
                      "traffic": None}) if dom else None,
        "warmup_kernel_ms": {k: float(np.mean(v)) for k, v in probe_ms.items()},
        # every kernel timed in the warm-up, against the same algorithmic
        # bytes as the roofline above
        "kernel_rooflines": {k: {"ms": float(np.mean(v)), "algorithmic_bytes": alg.get(k),
                                 "GBps": alg[k] / (np.mean(v) * 1e-3) / 1e9 if alg.get(k) else None,
                                 "frac": alg[k] / (np.mean(v) * 1e-3) / 1e9 / HBM_PEAK_GBS
                                 if alg.get(k) else None}
                             for k, v in probe_ms.items()},
        "backward_key_split": shape,
    }
    if not extra:
        if args.export_import:
            result["export_import"] = export_import(torch, recis, table, spec, wl, D, s_bytes, S, block_memory)
        if args.track_last_use:
            result["config"]["track_last_use"] = True
        if args.admit_sketch_bits:
            result["config"]["admit_sketch_bits"] = args.admit_sketch_bits
        if args.evict_pass:
            if args.track_last_use:
                result["evict_lru_pass"] = evict_lru_pass(torch, table)
            result["evict_pass"] = evict_pass(torch, table)
        if block_memory == "host":
            result["config"]["block_memory"] = "host (pinned, mapped; IDMap and scratch in HBM)"
            result["host_link_copy_GBps"] = host_link_copy(torch, dev)
            H = int(st1.hbm_rows)
            result["config"]["hbm_tier_rows"] = H
            result["config"]["retier_every"] = retier_every
            if retier_ms:
                result["retier_passes"] = [{"ms": m, "rows_moved": n} for m, n in retier_ms]
            # row traffic across the host link per timed step, from the rows the
            # timed lookups handed out: keys on host rows read their row in the
            # forward and read + write it with its state in the update
            P = D * s_bytes + S * D * 4
            result["host_tier_keys_per_step"] = float(np.mean(host_keys))
            result["host_link_row_bytes_per_step"] = float(np.mean(host_keys)) * (D * s_bytes + 2 * P)
    cpu_src = None
    if cpu and block_memory == "device" and not args.no_cpu_baseline:
        # the timed steps' inputs and gradients, kept for the oracle
        nf = wl.get("cpu_features")
        cpu_src = ([batches[j] for j in range(first_timed, first_timed + K)],
                   [staged[Wm + k][3] for k in range(K)], nf)
    table.close()
    del staged, timed_res, res_pool, out
    torch.cuda.synchronize()
    if cpu_src is not None:
        timed, grads, nf = cpu_src

        def host_grad(g):
            def cols(nfe):
                x = g[:, :nfe * D] if pooled and nf is not None else g
                if spec.grad_dtype == "bf16":
                    return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                return x.contiguous().cpu().numpy()
            return cols
        result["cpu_baseline"] = cpu_baseline(spec, timed, [host_grad(g) for g in grads], nf,
                                              what=name)
        ncpu, model = host_info()
        result["cpu_baseline"]["host"] = f"{ncpu} logical CPUs, {model}"
    return result


def run_tiny(args):
    """Config 1: ten steps from an empty table, each timed alone (HIP events
    around the step); the figure is the step latency (launch-bound)."""
    r = run_standard("tiny", args, K=10, Wm=0, cpu=False, extra=True)
    return {"ms_per_step_median": r["step_ms_median_p90"][0], "ms_per_step_p90": r["step_ms_median_p90"][1],
            "ids_per_step": r["config"]["ids_per_step"], "value": r["value"], "unit": "IDs/s",
            "step_breakdown_ms": r["step_breakdown_ms"], "workload": r["config"]["workload"]}


def brief(r):
    """The extra-key form of a workload's result line."""
    return {"workload": r["config"]["workload"], "value": r["value"], "unit": r["unit"],
            "ms_per_step": r["ms_per_step"], "steps": r["steps"], "ids_per_step": r["config"]["ids_per_step"],
            "step_breakdown_ms": r["step_breakdown_ms"], "step_roofline": r["step_roofline"],
            "roofline": r["roofline"], "kernel_rooflines": r["kernel_rooflines"]}


def main():
    args = parse_args()
    if args.summarize_atomics:
        w = args.workload or "capacity"
        summarize_atomics(args.summarize_atomics, args.command,
                          args.out or os.path.join(ROOT, "profiles", f"atomics_{w}.txt"), w)
        return
    if args.summarize:
        w = args.workload or "capacity"
        summarize(args.summarize, args.kernel, args.command,
                  args.out or os.path.join(ROOT, "profiles", f"{args.kernel}_{w}_counters.txt"),
                  w, args.block_memory)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    if args.workload is not None:
        wl = WORKLOADS[args.workload]
        if wl.get("special") == "multi":
            return run_multi(args, wl)
        if wl.get("special") == "cache":
            return run_cache(args, wl)
        if args.workload == "tiny":
            print(json.dumps(run_tiny(args)))
            return
        print(json.dumps(run_standard(args.workload, args)))
        return
    # the default line: the capacity configuration (the largest that fits one
    # GPU); then the tiny, CTR and sequence configurations as extra keys
    result = run_standard("capacity", args)
    result["config"]["workload_id"] = "capacity (config 4 of 5)"
    if not args.no_extras:
        extras = {}
        extras["tiny"] = run_tiny(args)
        log("tiny done")
        extras["ctr"] = brief(run_standard("ctr", args, K=10, Wm=5, cpu=False, extra=True))
        log("ctr done")
        extras["seq"] = brief(run_standard("seq", args, K=10, Wm=5, cpu=False, extra=True))
        log("seq done")
        result["other_configs"] = extras
    print(json.dumps(result))


if __name__ == "__main__":
    main()
