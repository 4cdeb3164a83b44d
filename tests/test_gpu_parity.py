"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element, on seeded inputs shaped like the five workloads (scaled so the
oracle finishes in seconds while still spanning many tiles, ragged tails,
long duplicate runs and the backward's multi-chunk path).

Bar: bit-exact for keys, inverse, counts, bag segments, row presence, the
initial rows and bf16 gather / writeback values; pooled outputs within
1e-5 of the sum of |terms| (1e-2 for bf16 storage once rows have been
updated); updated fp32 parameters within 1e-5 and bf16
parameters within 1e-2 of max(|w|, lr); optimizer state within 1e-5
relative."""
import numpy as np
import pytest

import oracle
import workloads as W
from harness import (canon_export, canon_lookup, check_export, check_forward, check_gather_is_copy, check_lookup,
                     device_features, forward_out, gpu_step, lookup_flags, make_table, oracle_step)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dynamic_embedding_tables_amd import recis
    recis.load_library()  # raises when the HIP library is missing
    print(f"\n[gpu] {torch.cuda.get_device_name(0)}", flush=True)


def check_tiers(table):
    """After a hot-tier pass: with H HBM rows and keys ranked in classes
    floor(log2(count)) + 1, the top classes that fit H rows are hot; either no
    hot key is left on a host row or no cooler key on an HBM row (the pass
    swaps as many pairs as both lists allow).  Brute force over the export."""
    ex = table.export()
    rows = ex["rows"].cpu().numpy()
    counts = ex["counts"].cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    has = rows >= 0
    H = table.stats().hbm_rows
    cls = np.zeros(counts.size, np.int64)
    nz = counts > 0
    cls[nz] = np.floor(np.log2(counts[nz])).astype(np.int64) + 1
    hist = np.bincount(cls[has], minlength=33)
    acc, cut = 0, 0
    for j in range(32, -1, -1):
        acc += hist[j]
        if acc > H:
            cut = j + 1
            break
    hot = cls >= cut
    a = np.count_nonzero(has & hot & (rows >= H))
    b = np.count_nonzero(has & ~hot & (rows < H))
    assert a == 0 or b == 0, (a, b, H, cut)
    return np.count_nonzero(has & (rows < H)), np.count_nonzero(has & hot)


def run_parity(spec, batches, table_kw=None, evict_every=0, evict_min=2, prepopulate=None,
               export_every=1, evict_decay=0.0, lru_max=None, find_only_steps=(), retier_every=0,
               stats_out=None):
    import torch
    from dynamic_embedding_tables_amd import recis
    table = make_table(spec, **(table_kw or {}))
    otab = oracle.OracleTable(spec)
    if (table_kw or {}).get("admit_sketch_bits"):
        otab.set_sketch(table_kw["admit_sketch_bits"])
    passes = []  # LRU passes: (keys before, keys evicted)
    if prepopulate is not None:
        cap = max(prepopulate.n, 1)
        res = recis.LookupResult(cap, prepopulate.num_feats * prepopulate.batch)
        table.insert_find(device_features(prepopulate), prepopulate.batch, res,
                          flags=lookup_flags(spec))
        r = otab.insert_find(prepopulate.features, prepopulate.batch)
        assert r.status == 0
    for step, b in enumerate(batches):
        print(f"[parity] step {step} N={b.n}", flush=True)
        res = recis.LookupResult(max(b.n, 1), b.num_feats * b.batch)
        fo = step in find_only_steps
        # a gather is a copy: its rows are the table's own, bit for bit
        copy_check = (lambda out: check_gather_is_copy(out, table, res, spec)) if spec.pool == "none" else None
        out, _ = gpu_step(table, spec, b, res, find_only=fo, with_backward=not fo, after_forward=copy_check)
        r, oout, oab = oracle_step(otab, spec, b, find_only=fo, with_backward=not fo)
        torch.cuda.synchronize()
        assert table.get_error() == 0
        check_lookup(canon_lookup(res), r)
        check_forward(out, spec, oout, oab, r.merged_offsets, r.num_feats, exact=step == 0 and prepopulate is None)
        if retier_every and (step + 1) % retier_every == 0:
            moved = torch.zeros(1, dtype=torch.int64, device="cuda")
            table.retier(moved)
            in_hbm, n_hot = check_tiers(table)
            print(f"[parity] retier: moved {int(moved.item())}, rows in HBM {in_hbm}, hot keys {n_hot}", flush=True)
        if evict_every and (step + 1) % evict_every == 0:
            ne = torch.zeros(1, dtype=torch.int64, device="cuda")
            if lru_max is not None:
                before = otab.size()
                table.evict_lru(lru_max, ne)
                assert int(ne.item()) == otab.evict_lru(lru_max)
                passes.append((before, int(ne.item())))
            else:
                table.evict(evict_min, ne, decay=evict_decay)
                assert int(ne.item()) == otab.evict(evict_min, evict_decay)
        if (step + 1) % export_every == 0 or step == len(batches) - 1:
            check_export(canon_export(table), otab.export(), spec)
    st = table.stats()
    assert st.keys == otab.size()
    assert st.rows_in_use == otab.rows_in_use()
    if stats_out is not None:
        stats_out.append(st)
    table.close()
    return passes


def test_tiny_config_all_ten_steps():
    run_parity(W.spec_tiny(), [W.tiny_batch(s) for s in range(10)])


def test_ctr_config_scaled():
    run_parity(W.spec_ctr(), [W.ctr_batch(s, batch=256) for s in range(3)])


def test_sequence_config_scaled_bf16_long_keys():
    run_parity(W.spec_seq(), [W.seq_batch(s, batch=12, seq_len=1000) for s in range(3)])


def test_capacity_config_scaled_prepopulated():
    spec = W.spec_capacity()
    feats = []
    for f, ids in W.capacity_resident_keys(num_feats=5, per_feature=20000):
        feats.append(W.FeatureInput(values=ids, bag_offsets=np.array([0, ids.size], np.int32), slot=f))
    pre = W.Batch(feats, 1, np.zeros((1, 5 * spec.dim), np.float32))
    batches = [W.capacity_batch(s, batch=1024, num_feats=5, resident_per_feature=20000) for s in range(3)]
    run_parity(spec, batches, prepopulate=pre)


@pytest.mark.parametrize("table", range(5))
def test_multi_table_config_scaled_with_eviction(table):
    spec = W.spec_multi(table)
    batches = [W.multi_batch(s, table, batch=128, num_feats=6) for s in range(6)]
    run_parity(spec, batches, evict_every=2)


@pytest.mark.parametrize("decay", [0.5, 0.3, 1.0])
def test_eviction_with_decayed_counts(decay):
    """Eviction passes whose survivors keep floor(count * decay), on the
    multi-table config with admission at 2: evicted counts, key sets, counts,
    rows and their reuse step by step."""
    spec = W.spec_multi(3)
    batches = [W.multi_batch(s, 3, batch=128, num_feats=6) for s in range(8)]
    run_parity(spec, batches, evict_every=2, evict_min=3, evict_decay=decay)


@pytest.mark.parametrize("lru_max", [0, 2500, 4000])
def test_eviction_lru_bounded(lru_max):
    """LRU-bounded passes every other step (at most lru_max keys kept, whole
    lookups youngest first) on the multi-table config with admission at 2
    and a FIND_ONLY lookup between (which must not refresh ages): the
    evicted counts, key sets, counts and rows step by step."""
    spec = W.spec_multi(4)
    batches = [W.multi_batch(s, 4, batch=64, num_feats=4) for s in range(9)]
    passes = run_parity(spec, batches, table_kw=dict(track_last_use=True), evict_every=2, lru_max=lru_max,
                        find_only_steps=(4,))
    if lru_max > 0:  # some pass kept part of the table and removed the rest
        assert any(0 < ev < before for before, ev in passes), passes


def test_eviction_lru_after_growth():
    """The stamps move with their keys when the IDMap grows (64 slots to
    start) and when a pass rebuilds it."""
    spec = W.spec_ctr()
    run_parity(spec, [W.ctr_batch(s, batch=64, num_feats=8) for s in range(6)],
               table_kw=dict(slot_capacity=64, block_rows=64, track_last_use=True), evict_every=2, lru_max=2000)


@pytest.mark.parametrize("bits", [6, 18])
def test_count_min_sketch_admission(bits):
    """Count-min sketch admission (admission at 2, keys outside the IDMap
    counted in 4 x 2^bits counters) on the multi-table config with eviction
    passes that clear the sketch, and a FIND_ONLY lookup; a 6-bit sketch
    collides heavily, an 18-bit one hardly."""
    spec = W.spec_multi(1)
    batches = [W.multi_batch(s, 1, batch=128, num_feats=6) for s in range(8)]
    run_parity(spec, batches, table_kw=dict(admit_sketch_bits=bits), evict_every=3, find_only_steps=(4,))


def test_count_min_sketch_admission_hot_keys():
    """Sketch admission at 3 through the heavy-bucket path (one key with 20k
    occurrences per step, sliced across blocks) and a cold tail."""
    spec = W.TableSpec(dim=32, dtype="f32", optim="adagrad", pool="sum", lr=0.01, eps=1e-10, admit_threshold=3)
    batches = []
    for step in range(3):
        rng = W.rng_for(78, step)
        B = 2000
        lens = rng.poisson(12, B)
        off = W.offsets_from_lengths(lens)
        n = int(off[-1])
        vals = np.where(rng.random(n) < 0.8, 123456789, rng.integers(0, 4000, n))
        batches.append(W.Batch([W.FeatureInput(values=vals.astype(np.int64), bag_offsets=off, slot=1)], B,
                               rng.standard_normal((B, 32), dtype=np.float32)))
    run_parity(spec, batches, table_kw=dict(admit_sketch_bits=10))


def test_all_table_options_together():
    """Host-memory blocks, last-use stamps and sketch admission on one table,
    with a decayed-count pass and an LRU pass between lookups (one of them
    FIND_ONLY), a writeback of some keys, and the bf16 storage of Adam rows."""
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.TableSpec(dim=32, dtype="bf16", optim="adam", pool="mean", lr=1e-3, eps=1e-8, admit_threshold=2)
    table = make_table(spec, block_memory="host", track_last_use=True, admit_sketch_bits=9, block_rows=512)
    otab = oracle.OracleTable(spec)
    otab.set_sketch(9)
    ne = torch.zeros(1, dtype=torch.int64, device="cuda")
    for step in range(8):
        b = W.multi_batch(step, 2, batch=96, num_feats=5)
        b.grad = W.rng_for(79, step).standard_normal((b.batch, b.num_feats * 32), dtype=np.float32)
        fo = step == 5
        res = recis.LookupResult(max(b.n, 1), b.num_feats * b.batch)
        out, _ = gpu_step(table, spec, b, res, find_only=fo, with_backward=not fo)
        r, oout, oab = oracle_step(otab, spec, b, find_only=fo, with_backward=not fo)
        torch.cuda.synchronize()
        assert table.get_error() == 0
        check_lookup(canon_lookup(res), r)
        check_forward(out, spec, oout, oab, r.merged_offsets, r.num_feats, exact=step == 0)
        if step == 2:
            table.evict(2, ne, decay=0.5)
            assert int(ne.item()) == otab.evict(2, 0.5)
        if step == 4:
            table.evict_lru(600, ne)
            assert int(ne.item()) == otab.evict_lru(600)
        if step == 6:
            keys = np.unique(np.concatenate([(np.int64(f.slot) << np.int64(48)) | f.values for f in b.features]))[:50]
            rows = W.rng_for(80).standard_normal((keys.size, 32), dtype=np.float32)
            table.writeback(torch.from_numpy(keys).cuda(), torch.from_numpy(rows).cuda())
            assert otab.writeback(keys, rows) == 0
        check_export(canon_export(table), otab.export(), spec)
    st = table.stats()
    assert st.keys == otab.size() and st.rows_in_use == otab.rows_in_use()
    table.close()


# ---- full sizes: the bench's workload and table configuration, and the
# largest per-table shape of the multi-table config (which takes the lookup's
# large-bucket path)
@pytest.mark.timeout(900)
def test_ctr_full_size_bench_configuration():
    """Two full CTR steps (8192 x 26 features, 2.2M IDs each) on a table laid
    out as the benchmark's (2^27 IDMap slots, 2^20-row blocks)."""
    run_parity(W.spec_ctr(), [W.ctr_batch(s) for s in range(2)],
               table_kw=dict(slot_capacity=1 << 27, block_rows=1 << 20, reserve_rows=1 << 22))


@pytest.mark.timeout(900)
def test_sequence_full_size():
    """Two full sequence steps (2048 x 1000 positions, bf16 gather + Adagrad)."""
    run_parity(W.spec_seq(), [W.seq_batch(s) for s in range(2)])


@pytest.mark.timeout(900)
def test_multi_table_full_size_with_eviction():
    """One merged table of the multi-table config at full size (32768 x 60
    features, 7.9M IDs per step, admission threshold 2), with an eviction
    pass after the second step."""
    spec = W.spec_multi(0)
    run_parity(spec, [W.multi_batch(s, 0) for s in range(3)], evict_every=2, export_every=2)


def lookup_by_feature(res):
    """Host copies of a full-size lookup's distinct keys, counts, inverse and
    merged offsets, for per-feature checks."""
    U = res.U()
    return {"keys": res.unique_keys[:U].cpu().numpy(), "counts": res.counts[:U].cpu().numpy(),
            "rows": res.unique_rows[:U].cpu().numpy(), "inverse": res.inverse[:res.n].cpu().numpy(),
            "offsets": res.bag_offsets.cpu().numpy()}


def check_feature_lookup(look, batch, f, r, sub=None):
    """Feature f of a merged lookup against the oracle's lookup of a sub-batch
    of features (`sub`: their indices in `batch`, default [f]); keys carry the
    feature's slot, so they are the same keys: each of f's occurrences' key,
    its distinct keys with their counts and row presence, and its bags'
    merged offsets -- all bit-exact."""
    sub = [f] if sub is None else list(sub)
    k = sub.index(f)
    base = sum(batch.features[x].n for x in range(f))
    sbase = sum(batch.features[x].n for x in sub[:k])
    n_f = batch.features[f].n
    B = batch.batch
    np.testing.assert_array_equal(look["keys"][look["inverse"][base:base + n_f]],
                                  r.unique_keys[r.inverse[sbase:sbase + n_f]])
    slot = batch.features[f].slot
    sel = (look["keys"] >> 48) == slot
    kg, cg, rg = look["keys"][sel], look["counts"][sel], look["rows"][sel]
    order = np.argsort(kg, kind="stable")
    osel = (r.unique_keys[:r.U] >> 48) == slot
    np.testing.assert_array_equal(kg[order], r.unique_keys[:r.U][osel])
    np.testing.assert_array_equal(cg[order], r.counts[:r.U][osel])
    np.testing.assert_array_equal(rg[order] >= 0, r.unique_rows[:r.U][osel] >= 0)
    np.testing.assert_array_equal(look["offsets"][f * B:(f + 1) * B + 1] - base,
                                  r.merged_offsets[k * B:(k + 1) * B + 1] - sbase)


def canon_export_slots(table, slots):
    """canon_export restricted on the device to the keys of the given feature
    slots (a full-size table is too large to copy whole)."""
    import torch
    ex = table.export()
    sl = torch.bitwise_right_shift(ex["keys"], 48)
    m = torch.zeros_like(sl, dtype=torch.bool)
    for x in slots:
        m |= sl == x
    keys = ex["keys"][m].cpu().numpy()
    order = np.argsort(keys, kind="stable")
    params = ex["params"][m]
    params = params.float() if params.dtype == torch.bfloat16 else params
    return {"keys": keys[order], "rows": ex["rows"][m].cpu().numpy()[order],
            "counts": ex["counts"][m].cpu().numpy().astype(np.uint32)[order],
            "params": params.cpu().numpy()[order], "state": ex["state"][m].cpu().numpy()[order]}


@pytest.mark.timeout(900)
def test_multi_table_dim128_full_size_with_eviction():
    """The dim-128 table of the multi-table config at full size (32768 x 60
    features, 7.9M IDs per step, mean pooling, Adagrad, a row at the 2nd
    occurrence), three steps with an eviction pass (count < 2) after the
    second.  Keys carry their feature's slot, so the oracle recomputes two
    whole features: their lookups, pooled outputs, and after every step the
    keys, counts, row presence, parameters and state of every key of theirs
    the table holds."""
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.spec_multi(4)
    D = spec.dim
    checked = (0, 41)
    table = make_table(spec, slot_capacity=1 << 24, block_rows=1 << 20, reserve_rows=1 << 23)
    otab = oracle.OracleTable(spec)
    try:
        for step in range(3):
            b = W.multi_batch(step, 4)
            print(f"[multi128] step {step} N={b.n}", flush=True)
            res = recis.LookupResult(b.n, b.num_feats * b.batch)
            out, _ = gpu_step(table, spec, b, res)
            sub = W.Batch([b.features[f] for f in checked], b.batch,
                          np.ascontiguousarray(np.concatenate([b.grad[:, f * D:(f + 1) * D] for f in checked], 1)))
            r, o_out, o_abs = oracle_step(otab, spec, sub)
            torch.cuda.synchronize()
            assert table.get_error() == 0
            look = lookup_by_feature(res)
            for k, f in enumerate(checked):
                check_feature_lookup(look, b, f, r, sub=checked)
                cols, ocols = slice(f * D, (f + 1) * D), slice(k * D, (k + 1) * D)
                check_forward(out[:, cols].contiguous(), spec, np.ascontiguousarray(o_out[:, ocols]),
                              np.ascontiguousarray(o_abs[:, ocols]),
                              r.merged_offsets[k * b.batch:(k + 1) * b.batch + 1], 1, exact=step == 0)
            if step == 1:
                ne = torch.zeros(1, dtype=torch.int64, device="cuda")
                table.evict(2, ne)
                assert int(ne.item()) >= otab.evict(2) > 0
            check_export(canon_export_slots(table, checked), otab.export(), spec)
    finally:
        table.close()


@pytest.mark.timeout(900)
def test_capacity_full_size_two_features_checked():
    """The capacity configuration at full size, laid out as the benchmark's
    table: 100 features x 2M resident IDs (200M rows of dim 64 fp32 + Adam),
    then one full step (65536 bags per feature, Poisson(8), 52.4M IDs).  Keys
    carry their feature's slot, so one feature's bags, keys and gradient
    columns do not depend on the other features: the oracle recomputes two
    whole features, their pooled outputs and, after the Adam update, the
    parameters of every key they touched (read back by a FIND_ONLY gather)."""
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.spec_capacity()
    D = spec.dim
    b = W.capacity_batch(0)
    # the benchmark's reservation: resident rows, one step's IDs, and 2% new
    # rows for each of its eleven other steps
    table = make_table(spec, slot_capacity=1 << 29, block_rows=1 << 20,
                       reserve_rows=200_000_000 + b.n + 11 * (b.n // 30))
    try:
        for f, ids in W.capacity_resident_keys():
            kd = torch.from_numpy(ids).cuda()
            od = torch.arange(ids.size + 1, dtype=torch.int32, device="cuda")
            r = recis.LookupResult(ids.size, ids.size)
            table.insert_find([recis.DeviceFeature(kd, od, f)], ids.size, r)
            del r, kd, od
        torch.cuda.synchronize()
        assert table.get_error() == 0
        assert table.stats().rows_in_use == 200_000_000
        res = recis.LookupResult(b.n, b.num_feats * b.batch)
        out, _ = gpu_step(table, spec, b, res)
        torch.cuda.synchronize()
        assert table.get_error() == 0
        look = lookup_by_feature(res)
        for f in (0, 77):
            cols = slice(f * D, (f + 1) * D)
            sub = W.Batch([b.features[f]], b.batch, np.ascontiguousarray(b.grad[:, cols]))
            otab = oracle.OracleTable(spec)
            r, o_out, o_abs = oracle_step(otab, spec, sub)
            check_feature_lookup(look, b, f, r)
            check_forward(out[:, cols].contiguous(), spec, o_out, o_abs, r.merged_offsets, 1, exact=True)
            ex = otab.export()
            ids = ex["keys"] & ((1 << 48) - 1)
            nk = int(ids.size)
            fd = [recis.DeviceFeature(torch.from_numpy(ids).cuda(),
                                      torch.arange(nk + 1, dtype=torch.int32, device="cuda"), f)]
            rr = recis.LookupResult(nk, nk)
            table.insert_find(fd, nk, rr, flags=recis.RECIS_GROUP_BY_OCCURRENCE | recis.RECIS_FIND_ONLY)
            g = torch.empty(nk, D, dtype=torch.float32, device="cuda")
            table.forward(rr, "none", g)
            gv = g.cpu().numpy().astype(np.float64)
            ov = ex["params"].astype(np.float64)
            bad = np.abs(gv - ov) > 1e-5 * np.maximum(np.abs(ov), spec.lr)
            assert not bad.any(), f"feature {f}: {bad.sum()} updated parameters off"
    finally:
        table.close()


@pytest.mark.timeout(900)
def test_cache_writeback_full_size():
    """The item cache at full size, laid out as the benchmark's table: 10M
    keys inserted with zero rows, then two calls of 16,384 writes drawn with
    replacement.  Read back by a FIND_ONLY gather, every written key holds
    the RNE of its last write (the oracle's writeback of the same pairs) and
    a sample of the other keys still holds zeros."""
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.spec_cache()
    keys = W.cache_keys()
    table = make_table(spec, slot_capacity=1 << 25, block_rows=1 << 20, reserve_rows=keys.size + (1 << 20))
    chunk = 1 << 20
    zero = torch.zeros(chunk, spec.dim, device="cuda")
    for c0 in range(0, keys.size, chunk):
        kd = torch.from_numpy(keys[c0:c0 + chunk]).cuda()
        table.writeback(kd, zero[:kd.numel()])
    otab = oracle.OracleTable(spec)
    for step in range(2):
        k, e = W.cache_writes(step, keys)
        table.writeback(torch.from_numpy(k).cuda(), torch.from_numpy(e).cuda())
        assert otab.writeback(k, e) == 0
    torch.cuda.synchronize()
    assert table.get_error() == 0
    assert table.stats().keys == keys.size
    o = otab.export()
    rng = np.random.default_rng(7)
    others = np.setdiff1d(keys[rng.integers(0, keys.size, 4000)], o["keys"])[:2000]
    probe = np.concatenate([o["keys"], others])
    b = W.Batch([W.FeatureInput(values=probe, bag_offsets=np.arange(probe.size + 1, dtype=np.int32), slot=0)],
                int(probe.size), None)
    res = recis.LookupResult(int(probe.size), int(probe.size))
    out, _ = gpu_step(table, spec, b, res, find_only=True, with_backward=False)
    got = out.float().cpu().numpy()
    nw = o["keys"].size
    np.testing.assert_array_equal(got[:nw], o["params"])
    assert not got[nw:].any()
    table.close()


def test_lookup_rejects_a_small_bag_buffer():
    """A result whose bag_offsets buffer holds fewer than num_feats * batch
    bags is refused before any work (INVALID_ARG), and the table stays
    usable; the same lookup with room for every bag then matches the oracle."""
    from dynamic_embedding_tables_amd import recis
    spec = W.spec_ctr()
    b = W.ctr_batch(0, batch=64, num_feats=3)
    table = make_table(spec)
    small = recis.LookupResult(b.n, b.batch)   # room for one feature's bags only
    with pytest.raises(recis.RecisError) as e:
        table.insert_find(device_features(b), b.batch, small)
    assert e.value.status == recis.RECIS_ERR_INVALID_ARG
    table.close()
    run_parity(spec, [b])


def test_growth_of_idmap_and_blocks():
    spec = W.spec_ctr()
    run_parity(spec, [W.ctr_batch(s, batch=64, num_feats=8) for s in range(3)],
               table_kw=dict(slot_capacity=64, block_rows=64))


# ---- EmbeddingBlocks in pinned host memory (the IDMap and scratch in HBM)
@pytest.mark.parametrize("optim,pool", [("adam", "mean"), ("adagrad", "sum")])
def test_hbm_tier_in_front_of_host_blocks(optim, pool):
    """EmbeddingBlocks in host memory with a two-block HBM tier (128 rows of
    64): new rows fill the HBM tier first, then host blocks; after every step
    the hot-tier pass moves the most frequent keys into HBM.  Content is
    checked against the oracle at every step (the tiers change where rows
    live, not what they hold), and the placement by brute force."""
    spec = W.TableSpec(dim=32, dtype="f32", optim=optim, pool=pool, lr=1e-3 if optim == "adam" else 0.01,
                       eps=1e-8 if optim == "adam" else 1e-10)
    run_parity(spec, [W.ctr_batch(s, batch=96, num_feats=3, dim=32) for s in range(6)],
               table_kw=dict(block_memory="host", block_rows=64, device_rows=100), retier_every=1)


def test_hbm_tier_with_eviction_and_admission():
    """The hot tier with admission at 2 and eviction passes: probationary keys
    hold no row and take no part; freed rows of either tier are reused."""
    spec = W.spec_multi(2)
    run_parity(spec, [W.multi_batch(s, 2, batch=128, num_feats=6) for s in range(6)],
               table_kw=dict(block_memory="host", block_rows=256, device_rows=512), retier_every=1, evict_every=2)


def test_hbm_tier_between_a_lookup_and_its_backward():
    """A hot-tier pass between a lookup and its forward / backward: rows have
    moved, so the stale lookup re-probes its keys."""
    import torch
    spec = W.TableSpec(dim=32, dtype="f32", optim="adam", pool="mean", lr=1e-3, eps=1e-8)
    table = make_table(spec, block_memory="host", block_rows=64, device_rows=64)
    otab = oracle.OracleTable(spec)
    from dynamic_embedding_tables_amd import recis
    warm = W.ctr_batch(5, batch=200, num_feats=2, dim=32)
    res = recis.LookupResult(warm.n, warm.num_feats * warm.batch)
    gpu_step(table, spec, warm, res)
    oracle_step(otab, spec, warm)

    def retier():
        moved = torch.zeros(1, dtype=torch.int64, device="cuda")
        table.retier(moved)
        assert int(moved.item()) > 0
        check_tiers(table)

    _stale_pair(spec, table, otab, W.ctr_batch(6, batch=200, num_feats=2, dim=32),
                W.ctr_batch(7, batch=100, num_feats=2, dim=32), retier)
    table.close()


def test_host_memory_blocks_ctr():
    """The CTR step with small blocks, so rows spread over many host blocks
    that are added as the table grows."""
    run_parity(W.spec_ctr(), [W.ctr_batch(s, batch=256) for s in range(3)],
               table_kw=dict(block_rows=4096, block_memory="host"))


def test_host_memory_blocks_sequence_and_eviction():
    """The bf16 gather with hot keys, and a table with admission and an
    eviction pass, both on host blocks."""
    run_parity(W.spec_seq(), [W.seq_batch(s, batch=12, seq_len=1000) for s in range(2)],
               table_kw=dict(block_memory="host"))
    spec = W.spec_multi(1)
    run_parity(spec, [W.multi_batch(s, 1, batch=128, num_feats=6) for s in range(4)], evict_every=2,
               table_kw=dict(block_memory="host"))


def test_initial_rows_bit_exact():
    import torch
    from dynamic_embedding_tables_amd import recis
    for spec in (W.spec_tiny(), W.spec_seq(), W.spec_multi(0)):
        spec.admit_threshold = 1
        b = W.tiny_batch(3, id_space=5000)
        table = make_table(spec)
        otab = oracle.OracleTable(spec)
        res = recis.LookupResult(b.n, b.batch)
        table.insert_find(device_features(b), b.batch, res, flags=lookup_flags(spec))
        otab.insert_find(b.features, b.batch)
        torch.cuda.synchronize()
        g, o = canon_export(table), otab.export()
        np.testing.assert_array_equal(g["keys"], o["keys"])
        np.testing.assert_array_equal(g["params"], o["params"])   # exact, including bf16 rounding
        assert not g["state"].any()
        table.close()


def test_transforms_hash_mod_bucketize_and_find_only():
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.TableSpec(dim=32, dtype="f32", optim="adagrad", pool="sum", lr=0.01, eps=1e-10)
    rng = W.rng_for(42)
    B = 300
    f0 = W.FeatureInput(values=rng.integers(-2**62, 2**62, 900, dtype=np.int64),
                        bag_offsets=W.offsets_from_lengths(rng.poisson(3, B)[:B] * 0 + 3), slot=0,
                        ops=W.OP_HASH | W.OP_MOD, mod=1000)
    lens = rng.poisson(2.0, B)
    off = W.offsets_from_lengths(lens)
    f1 = W.FeatureInput(values=rng.integers(-5000, 5000, int(off[-1]), dtype=np.int64), bag_offsets=off,
                        slot=7, ops=W.OP_MOD, mod=97)
    f2 = W.bucketize_feature(rng, B, 50, slot=9)
    f3 = W.FeatureInput(values=rng.integers(0, 1 << 47, 500, dtype=np.int64),
                        bag_offsets=W.offsets_from_lengths(np.full(B, 0, np.int64) + np.r_[np.full(250, 2), np.zeros(50, np.int64)]),
                        slot=(1 << 15) - 1)
    batches = []
    for step in range(2):
        g = W.rng_for(43, step).standard_normal((B, 4 * 32), dtype=np.float32)
        batches.append(W.Batch([f0, f1, f2, f3], B, g))
    run_parity(spec, batches)
    # FIND_ONLY: absent keys report no row and nothing is inserted or counted
    table = make_table(spec)
    otab = oracle.OracleTable(spec)
    b = batches[0]
    half = W.Batch([f1], B, b.grad[:, :32].copy())
    res = recis.LookupResult(b.n, b.num_feats * B)
    gpu_step(table, spec, half, recis.LookupResult(half.n, B))
    oracle_step(otab, spec, half)
    out, _ = gpu_step(table, spec, b, res, find_only=True, with_backward=False)
    r, oout, oab = oracle_step(otab, spec, b, find_only=True, with_backward=False)
    torch.cuda.synchronize()
    check_lookup(canon_lookup(res), r)
    check_forward(out, spec, oout, oab, r.merged_offsets, r.num_feats)
    check_export(canon_export(table), otab.export(), spec)


def test_mod_transform_edges():
    """The remainder by multiplication at the edges: the extreme int64 values,
    moduli 1, 3, 2^47 + 12345 and 2^48 (the largest that keeps every key in
    range), on raw signed values (floor remainder) and after Hash."""
    spec = W.TableSpec(dim=16, dtype="f32", optim="adagrad", pool="sum", lr=0.01, eps=1e-10)
    rng = W.rng_for(44)
    edges = np.array([-2**63, -2**63 + 1, -2**48 - 1, -2**48, -2**47, -1, 0, 1, 2**47, 2**48 - 1, 2**48,
                      2**63 - 1, 2**63 - 2], dtype=np.int64)
    vals = np.concatenate([edges, rng.integers(-2**63, 2**63 - 1, 400, dtype=np.int64, endpoint=True)])
    B = vals.size
    off = W.offsets_from_lengths(np.ones(B, np.int64))
    feats = [W.FeatureInput(values=vals, bag_offsets=off, slot=1, ops=W.OP_MOD, mod=2**48),
             W.FeatureInput(values=vals, bag_offsets=off, slot=2, ops=W.OP_MOD, mod=1),
             W.FeatureInput(values=vals, bag_offsets=off, slot=3, ops=W.OP_MOD, mod=2**47 + 12345),
             W.FeatureInput(values=vals, bag_offsets=off, slot=4, ops=W.OP_HASH | W.OP_MOD, mod=2**48),
             W.FeatureInput(values=vals, bag_offsets=off, slot=5, ops=W.OP_HASH | W.OP_MOD, mod=3)]
    g = W.rng_for(45).standard_normal((B, len(feats) * 16), dtype=np.float32)
    run_parity(spec, [W.Batch(feats, B, g)])


def test_empty_batches_and_empty_bags():
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.TableSpec(dim=16, dtype="f32", optim="adam", pool="mean", lr=1e-3, eps=1e-8)
    table = make_table(spec)
    otab = oracle.OracleTable(spec)
    # all bags empty
    B = 37
    f = W.FeatureInput(values=np.zeros(0, np.int64), bag_offsets=np.zeros(B + 1, np.int32), slot=0)
    b = W.Batch([f, f], B, np.ones((B, 32), np.float32))
    res = recis.LookupResult(1, 2 * B)
    out, _ = gpu_step(table, spec, b, res)
    r, oout, oab = oracle_step(otab, spec, b)
    torch.cuda.synchronize()
    assert res.U() == 0 and not out.cpu().numpy().any()
    check_forward(out, spec, oout, oab, r.merged_offsets, r.num_feats)
    # mostly-empty bags with a few long ones
    lens = np.zeros(B, np.int64)
    lens[[3, 17, 36]] = [40, 1, 300]
    off = W.offsets_from_lengths(lens)
    vals = W.rng_for(5).integers(0, 50, int(off[-1]), dtype=np.int64)
    b = W.Batch([W.FeatureInput(values=vals, bag_offsets=off, slot=2)], B,
                W.rng_for(6).standard_normal((B, 16), dtype=np.float32))
    res = recis.LookupResult(b.n, B)
    out, _ = gpu_step(table, spec, b, res)
    r, oout, oab = oracle_step(otab, spec, b)
    torch.cuda.synchronize()
    check_lookup(canon_lookup(res), r)
    check_forward(out, spec, oout, oab, r.merged_offsets, r.num_feats)
    check_export(canon_export(table), otab.export(), spec)
    # zero features
    res = recis.LookupResult(1, 0)
    table.insert_find([], 5, res)
    torch.cuda.synchronize()
    assert res.U() == 0 and table.get_error() == 0


def _ragged_pool_batch(seed, B, dim, key_space, num_feats=2):
    """Bag lengths that stress the pooled forward's occurrence runs: many
    empty bags (a run of 100 of them, more than one 64-bag window), short
    bags, bags longer than a run, and one bag spanning several runs."""
    rng = W.rng_for(seed)
    feats = []
    for f in range(num_feats):
        lens = rng.choice([0, 1, 2, 3, 5, 8, 13, 40], B, p=[0.2, 0.2, 0.15, 0.15, 0.1, 0.1, 0.06, 0.04])
        lens[100:200] = 0
        lens[300] = 400
        lens[301:305] = 70
        lens[-1] = 0
        off = W.offsets_from_lengths(lens)
        vals = rng.integers(0, key_space, int(off[-1]), dtype=np.int64)
        feats.append(W.FeatureInput(values=vals, bag_offsets=off, slot=f + 1))
    return W.Batch(feats, B, rng.standard_normal((B, num_feats * dim), dtype=np.float32))


@pytest.mark.parametrize("dtype,dim,pool", [("f32", d, "mean") for d in (8, 16, 32, 64, 128, 256)]
                         + [("f32", 64, "sum")]
                         + [("bf16", d, p) for d in (8, 64, 256) for p in ("sum", "mean")])
def test_pooled_forward_bag_shapes(dtype, dim, pool):
    """Pooled forward over ragged bags, first with every row pending (the
    initializer's values), then with stored and pending rows mixed."""
    spec = W.TableSpec(dim=dim, dtype=dtype, optim="adagrad", pool=pool, lr=0.01)
    a = _ragged_pool_batch(31, 700, dim, 3000)
    b = _ragged_pool_batch(32, 700, dim, 6000)
    run_parity(spec, [a, b])


@pytest.mark.parametrize("dtype,optim,pool,grad_dtype,dim", [
    ("bf16", "adam", "mean", "f32", 64), ("bf16", "adam", "sum", "bf16", 128),
    ("f32", "adam", "none", "f32", 32), ("bf16", "adam", "none", "bf16", 256),
    ("f32", "adagrad", "none", "bf16", 16)])
def test_storage_optimizer_pooling_combinations(dtype, optim, pool, grad_dtype, dim):
    """Storage dtype x optimizer x pooling x gradient dtype combinations the
    workload configs leave out, over three steps with hot and cold keys."""
    spec = W.TableSpec(dim=dim, dtype=dtype, optim=optim, pool=pool, lr=1e-3 if optim == "adam" else 0.01,
                       eps=1e-8 if optim == "adam" else 1e-10, grad_dtype=grad_dtype)
    batches = []
    for step in range(3):
        b = _ragged_pool_batch(60 + step, 700, dim, 2000)
        if pool == "none":
            b.grad = W.rng_for(61, step).standard_normal((b.n, dim), dtype=np.float32)
        else:
            b.grad = W.rng_for(61, step).standard_normal((b.batch, b.num_feats * dim), dtype=np.float32)
        batches.append(b)
    run_parity(spec, batches)


@pytest.mark.parametrize("optim", ["adam", "adagrad"])
def test_interleaved_lookups(optim):
    """Lookup A, lookup B (sharing keys that are new in A), update A, then
    forward and update B: B's rows must be the ones A's update wrote, not
    their initial values."""
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.TableSpec(dim=32, dtype="f32", optim=optim, pool="mean", lr=1e-3 if optim == "adam" else 0.01,
                       eps=1e-8 if optim == "adam" else 1e-10)
    table = make_table(spec)
    otab = oracle.OracleTable(spec)
    a = W.ctr_batch(0, batch=200, num_feats=3, dim=32)
    b = W.ctr_batch(1, batch=200, num_feats=3, dim=32)
    b.features = [W.FeatureInput(values=np.concatenate([fa.values[:100], fb.values]),
                                 bag_offsets=np.concatenate([fb.bag_offsets[:1], fb.bag_offsets[1:] + 100]).astype(np.int32),
                                 slot=fb.slot, ops=fb.ops, mod=fb.mod)
                  for fa, fb in zip(a.features, b.features)]   # B's first bag repeats 100 of A's IDs
    ra, rb = recis.LookupResult(a.n, 600), recis.LookupResult(b.n, 600)
    table.insert_find(device_features(a), 200, ra)
    table.insert_find(device_features(b), 200, rb)
    oa = otab.insert_find(a.features, 200)
    ob = otab.insert_find(b.features, 200)
    for batch, res, r in ((a, ra, oa), (b, rb, ob)):
        out = forward_out(spec, batch, res)
        table.forward(res, spec.pool, out)
        g = torch.from_numpy(batch.grad).cuda()
        table.backward_update(res, spec.pool, g, "f32", lr=spec.lr, beta1=spec.beta1, beta2=spec.beta2,
                              eps=spec.eps)
        oout, oab = otab.forward(r, spec.pool, with_abs=True)
        assert otab.backward_update(r, spec.pool, batch.grad) == 0
        torch.cuda.synchronize()
        check_forward(out, spec, oout, oab, r.merged_offsets, r.num_feats)
    check_export(canon_export(table), otab.export(), spec)
    table.close()


def _stale_pair(spec, table, otab, a, b, between):
    """Lookup A; `between` (GPU, oracle) runs; lookup B; then A's forward and
    backward, then B's -- each checked against the oracle, whose forward and
    backward act on the rows the keys hold when they run."""
    import torch
    from dynamic_embedding_tables_amd import recis
    ra = recis.LookupResult(a.n, a.num_feats * a.batch)
    rb = recis.LookupResult(b.n, b.num_feats * b.batch)
    table.insert_find(device_features(a), a.batch, ra)
    oa = otab.insert_find(a.features, a.batch)
    between()
    table.insert_find(device_features(b), b.batch, rb)
    ob = otab.insert_find(b.features, b.batch)
    torch.cuda.synchronize()
    assert table.get_error() == 0
    check_lookup(canon_lookup(rb), ob)
    for batch, res, r in ((a, ra, oa), (b, rb, ob)):
        out = forward_out(spec, batch, res)
        table.forward(res, spec.pool, out)
        g = torch.from_numpy(batch.grad).cuda()
        table.backward_update(res, spec.pool, g, "f32", lr=spec.lr, beta1=spec.beta1, beta2=spec.beta2,
                              eps=spec.eps)
        oout, oab = otab.forward(r, spec.pool, with_abs=True)
        assert otab.backward_update(r, spec.pool, batch.grad) == 0
        torch.cuda.synchronize()
        assert table.get_error() == 0
        check_forward(out, spec, oout, oab, r.merged_offsets, r.num_feats)
        check_export(canon_export(table), otab.export(), spec)
    st = table.stats()
    assert st.keys == otab.size() and st.rows_in_use == otab.rows_in_use()


@pytest.mark.parametrize("optim", ["adagrad", "adam"])
def test_interleaved_lookups_across_idmap_growth(optim):
    """Lookup A on a 64-slot IDMap, then lookup B, which grows it (every key
    moves to a new slot): A's forward and backward must find A's keys at their
    new slots, not write through the old slot indices."""
    spec = W.TableSpec(dim=32, dtype="f32", optim=optim, pool="mean", lr=1e-3 if optim == "adam" else 0.01,
                       eps=1e-8 if optim == "adam" else 1e-10)
    table = make_table(spec, slot_capacity=64, block_rows=64)
    otab = oracle.OracleTable(spec)
    a = W.ctr_batch(0, batch=40, num_feats=2, dim=32)
    b = W.ctr_batch(1, batch=300, num_feats=3, dim=32)
    slots0 = table.stats().slot_capacity
    _stale_pair(spec, table, otab, a, b, lambda: None)
    assert table.stats().slot_capacity > slots0
    table.close()


@pytest.mark.parametrize("admit", [1, 2])
def test_eviction_between_a_lookup_and_its_backward(admit):
    """Lookup A; an eviction pass (A's once-seen keys leave and free their
    rows); lookup B (new keys take the freed rows); then A's forward and
    backward: the evicted keys get zeros and no update, and the rows now held
    by B's keys are not touched by A's gradient."""
    import torch
    spec = W.TableSpec(dim=16, dtype="f32", optim="adagrad", pool="sum", lr=0.01, eps=1e-10, admit_threshold=admit)
    table = make_table(spec, slot_capacity=1 << 12, block_rows=256)
    otab = oracle.OracleTable(spec)
    a = W.tiny_batch(0, id_space=3000)
    b = W.tiny_batch(1, id_space=3000)

    def evict():
        ne = torch.zeros(1, dtype=torch.int64, device="cuda")
        table.evict(2, ne)
        assert int(ne.item()) == otab.evict(2) > 0

    _stale_pair(spec, table, otab, a, b, evict)
    table.close()


def test_capacity_error_is_sticky_until_an_eviction_pass():
    """A row limit reached on the device: CAPACITY stays reported (while
    KEY_RANGE, read and cleared, still comes through first) until an eviction
    pass makes room."""
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.spec_tiny()
    table = make_table(spec, max_rows=100, block_rows=64)
    b = W.tiny_batch(0, id_space=100000)
    res = recis.LookupResult(b.n, b.batch)
    table.insert_find(device_features(b), b.batch, res)
    torch.cuda.synchronize()
    assert table.get_error() == recis.RECIS_ERR_CAPACITY
    assert table.get_error() == recis.RECIS_ERR_CAPACITY
    bad = W.Batch([W.FeatureInput(values=np.array([-4], np.int64), bag_offsets=np.array([0, 1], np.int32),
                                  slot=0)], 1, np.ones((1, 16), np.float32))
    r2 = recis.LookupResult(1, 1)
    table.insert_find(device_features(bad), 1, r2)
    assert table.get_error() == recis.RECIS_ERR_KEY_RANGE
    assert table.get_error() == recis.RECIS_ERR_CAPACITY
    st = table.stats()
    assert st.rows_in_use == 100 and st.probationary_keys == st.keys - 100 > 0
    ne = torch.zeros(1, dtype=torch.int64, device="cuda")
    table.evict(2, ne)
    assert int(ne.item()) > 0
    assert table.get_error() == 0
    table.close()


def test_stats_count_idmap_claims():
    """Every key a counting lookup inserts claims one empty IDMap slot: the
    claim attempts are at least the inserted keys, and a FIND_ONLY lookup
    adds none."""
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.spec_ctr()
    table = make_table(spec)
    b = W.ctr_batch(0, batch=512, num_feats=4)
    res = recis.LookupResult(b.n, b.num_feats * b.batch)
    table.insert_find(device_features(b), b.batch, res)
    torch.cuda.synchronize()
    st = table.stats()
    assert st.keys == res.U() and st.probationary_keys == 0
    assert st.claim_attempts >= st.keys and 0 <= st.claim_failures <= st.claim_attempts - st.keys
    table.insert_find(device_features(b), b.batch, res, flags=recis.RECIS_FIND_ONLY)
    st2 = table.stats()
    assert st2.claim_attempts == st.claim_attempts and st2.claim_failures == st.claim_failures
    table.close()


@pytest.mark.parametrize("batch,num_feats", [(64, 2), (4096, 8)])
def test_lookup_pairs_are_tile_distinct_keys(batch, num_feats):
    """insert_find first deduplicates each tile of 4096 consecutive
    occurrences (merged order) on its own: the stats' pair count grows, per
    call, by the number of distinct keys in each such tile, summed -- counted
    here from the oracle's per-occurrence keys (one ragged tile, then many
    with a ragged tail)."""
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.spec_ctr()
    table = make_table(spec)
    otab = oracle.OracleTable(spec)
    b = W.ctr_batch(3, batch=batch, num_feats=num_feats)
    r = otab.insert_find(b.features, b.batch)
    assert r.status == 0
    occ = r.unique_keys[r.inverse[:r.n]]
    want = sum(np.unique(occ[i:i + 4096]).size for i in range(0, occ.size, 4096))
    res = recis.LookupResult(b.n, b.num_feats * b.batch)
    table.insert_find(device_features(b), b.batch, res)
    torch.cuda.synchronize()
    assert table.stats().lookup_pairs == want
    table.insert_find(device_features(b), b.batch, res, flags=recis.RECIS_FIND_ONLY)
    assert table.stats().lookup_pairs == 2 * want
    table.close()
    otab.close()


def _hot_batch(seed, B, dim, key_space, num_feats, slots, alpha, long_bags=False):
    """Power-law IDs that give each feature many keys with more than 64
    occurrences (the backward's long keys), ragged bags with empty ones in
    the middle and at the end, or long bags (a stage of the bag-major pass
    then holds more occurrences than one sorted batch)."""
    rng = W.rng_for(seed)
    feats = []
    for f in range(num_feats):
        lens = rng.integers(40, 81, B) if long_bags else rng.poisson(8, B)
        lens[::97] = 0
        lens[-3:] = 0
        off = W.offsets_from_lengths(lens)
        # ranks 1..key_space with P(k) proportional to k**-alpha
        pk = np.arange(1, key_space + 1, dtype=np.float64) ** -alpha
        vals = rng.choice(key_space, int(off[-1]), p=pk / pk.sum()).astype(np.int64) + 1
        feats.append(W.FeatureInput(values=vals, bag_offsets=off, slot=slots[f]))
    return W.Batch(feats, B, rng.standard_normal((B, num_feats * dim), dtype=np.float32))


def _expected_hot_keys(batch, dim):
    """The keys the pooled backward sums bag-major, by the rule the stats
    field documents: per feature (each in its own slot modulo 4096), of the
    keys with more than 64 occurrences and at least 8 per block of 2048 bags,
    whole count classes floor(log2(count)) from the top while at most
    8192 / dim keys fit."""
    bins = [f.slot % 4096 for f in batch.features]
    if len(set(bins)) != len(bins):
        return 0
    blocks = -(-batch.batch // 2048)
    kmax = 8192 // dim
    total = 0
    for f in batch.features:
        _, counts = np.unique(f.values, return_counts=True)
        c = counts[(counts > 64) & (counts >= 8 * blocks)]
        cls = np.floor(np.log2(c)).astype(np.int64)
        taken = 0
        for k in range(31, -1, -1):
            x = int((cls == k).sum())
            if taken + x > kmax:
                break
            taken += x
        total += taken
    return total


@pytest.mark.parametrize("case", ["sum64_threshold_split", "mean128_bf16_grad", "long_bags", "shared_slot",
                                  "slots_alike_mod_4096", "small_gradient_default"])
def test_hot_keys_summed_bag_major(case):
    """The pooled backward's bag-major pass for hot long keys (forced on for
    these small gradients with hot_grad_bytes = 1), at parity with the oracle
    over two steps: several 2048-bag blocks with a partial last one; more
    eligible keys than a feature's limit (the count classes split); mean
    pooling with bf16 gradients at dim 128; stages with more occurrences than
    one sorted batch; features whose slots coincide modulo 4096 (the pass
    stays off); and the default threshold, under which a gradient of a few
    MB keeps the key-by-key sums.  The stats count exactly the keys the
    documented rule selects."""
    spec_kw = dict(dtype="f32", optim="adam", lr=1e-3, eps=1e-8)
    if case == "sum64_threshold_split":
        dim, pool, gdt = 64, "sum", "f32"
        mk = lambda s: _hot_batch(s, 5000, dim, 400, 2, (1, 2), 0.8)
    elif case == "mean128_bf16_grad":
        dim, pool, gdt = 128, "mean", "bf16"
        mk = lambda s: _hot_batch(s, 3000, dim, 300, 3, (4, 5, 6), 0.8)
    elif case == "long_bags":
        dim, pool, gdt = 64, "sum", "f32"
        mk = lambda s: _hot_batch(s, 600, dim, 4000, 1, (7,), 1.2, long_bags=True)
    elif case == "shared_slot":
        dim, pool, gdt = 64, "mean", "f32"
        mk = lambda s: _hot_batch(s, 2500, dim, 1500, 2, (8, 8), 1.1)
    elif case == "slots_alike_mod_4096":
        dim, pool, gdt = 64, "mean", "f32"
        mk = lambda s: _hot_batch(s, 2500, dim, 1500, 2, (3, 4099), 1.1)
    else:
        dim, pool, gdt = 64, "sum", "f32"
        mk = lambda s: _hot_batch(s, 5000, dim, 400, 2, (1, 2), 0.8)
    spec = W.TableSpec(dim=dim, pool=pool, grad_dtype=gdt, **spec_kw)
    batches = [mk(900 + s) for s in range(2)]
    want = sum(_expected_hot_keys(b, dim) for b in batches)
    if case in ("shared_slot", "slots_alike_mod_4096"):
        assert want == 0
    else:
        assert want > 0
    if case == "small_gradient_default":
        want, table_kw = 0, {}
    else:
        table_kw = {"hot_grad_bytes": 1}
    st = []
    run_parity(spec, batches, stats_out=st, table_kw=table_kw)
    assert st[0].hot_keys == want


def test_torch_allocator_bridge():
    """A table created through the torch allocator bridge takes all its device
    memory from torch's caching allocator (and gives it back at close), and
    computes what a table on the library's own hipMalloc computes (to the
    parity bar)."""
    import gc
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.spec_ctr()
    gc.collect()
    torch.cuda.synchronize()
    before = recis.allocator_calls()
    mem0 = torch.cuda.memory_allocated()
    t_torch = make_table(spec, allocator="torch", reserve_rows=5000)
    assert recis.allocator_calls()["alloc"] > before["alloc"]
    assert torch.cuda.memory_allocated() - mem0 >= t_torch.stats().bytes
    t_hip = make_table(spec, allocator="hip", reserve_rows=5000)
    outs = []
    for t in (t_torch, t_hip):
        for s in range(2):
            b = W.ctr_batch(s, batch=128, num_feats=3)
            res = recis.LookupResult(b.n, b.num_feats * b.batch)
            out, _ = gpu_step(t, spec, b, res)
        torch.cuda.synchronize()
        assert t.get_error() == 0
        outs.append((out.cpu(), canon_export(t)))
    # the same keys, counts and rows; values to the parity bar (a key's
    # occurrences are grouped in an order that can differ from run to run, and
    # double sums in another order can round differently)
    np.testing.assert_allclose(outs[0][0].numpy(), outs[1][0].numpy(), rtol=1e-5, atol=1e-7)
    check_export(outs[0][1], outs[1][1], spec)
    t_torch.close()
    t_hip.close()
    after = recis.allocator_calls()
    # everything the table took through the bridge went back through it
    assert after["alloc"] - before["alloc"] == after["free"] - before["free"] > 0


def test_one_key_dominates():
    """A single key with 20k occurrences (80 backward chunks) plus a tail."""
    spec = W.TableSpec(dim=64, dtype="f32", optim="adagrad", pool="sum", lr=0.01, eps=1e-10)
    rng = W.rng_for(77)
    B = 2000
    lens = rng.poisson(12, B)
    off = W.offsets_from_lengths(lens)
    vals = np.where(rng.random(int(off[-1])) < 0.8, 123456789, rng.integers(0, 3000, int(off[-1])))
    b = W.Batch([W.FeatureInput(values=vals.astype(np.int64), bag_offsets=off, slot=1)], B,
                rng.standard_normal((B, 64), dtype=np.float32))
    run_parity(spec, [b, b])


def _long_keys_batch(seed, step, nkeys, per_key, hot, hot_count):
    """nkeys keys (drawn from `seed`) with per_key occurrences each plus `hot`
    keys with hot_count each, shuffled (by `step`) over bags of 8, the last
    one taking the rest."""
    keys = W.rng_for(seed).choice(1 << 40, nkeys + hot, replace=False).astype(np.int64)
    rng = W.rng_for(seed, step)
    vals = np.concatenate([np.repeat(keys[:nkeys], per_key), np.repeat(keys[nkeys:], hot_count)])
    rng.shuffle(vals)
    B = vals.size // 8
    lens = np.full(B, 8, dtype=np.int64)
    lens[-1] += vals.size - 8 * B
    off = W.offsets_from_lengths(lens)
    return W.Batch([W.FeatureInput(values=vals, bag_offsets=off, slot=1)], B,
                   rng.standard_normal((B, 64), dtype=np.float32))


@pytest.mark.parametrize("per_key", [100, 200])
def test_many_long_keys(per_key):
    """Thousands of keys just past the short path's 64 occurrences, so that
    the merge of the chunk partials takes four (100 occurrences each) or two
    (200 each) keys per block, mixed with hot keys whose partials a whole
    block merges; the same keys again in a second step (stored rows)."""
    spec = W.TableSpec(dim=64, dtype="f32", optim="adam", pool="sum", lr=1e-3, eps=1e-8)
    a = _long_keys_batch(90 + per_key, 0, 3000, per_key, 4, 5000)
    b = _long_keys_batch(90 + per_key, 1, 3000, per_key, 4, 5000)
    run_parity(spec, [a, b])


def test_long_keys_by_feature_large_gradient():
    """A pooled gradient larger than the memory-side cache (4 features x 270k
    bags x 64 fp32 = 276 MB), so the long keys' chunks are reordered feature
    by feature; every feature has hot keys and a cold tail; two steps."""
    spec = W.TableSpec(dim=64, dtype="f32", optim="adam", pool="mean", lr=1e-3, eps=1e-8)
    B, F = 270_000, 4
    batches = []
    for step in range(2):
        rng = W.rng_for(97, step)
        feats = []
        for f in range(F):
            lens = rng.integers(1, 4, B)
            off = W.offsets_from_lengths(lens)
            n = int(off[-1])
            hot = rng.integers(0, 300, n)                 # 300 hot keys: ~1.8k occurrences each
            cold = rng.integers(1000, 2_000_000, n)
            vals = np.where(rng.random(n) < 0.5, hot, cold).astype(np.int64)
            feats.append(W.FeatureInput(values=vals, bag_offsets=off, slot=f + 1))
        batches.append(W.Batch(feats, B, rng.standard_normal((B, F * 64), dtype=np.float32)))
    assert B * F * 64 * 4 > 256 * 2**20
    run_parity(spec, batches, export_every=2)


@pytest.mark.parametrize("pool,admit", [("sum", 1), ("mean", 2)])
def test_long_keys_extremes_large_gradient(pool, admit):
    """A pooled gradient larger than the memory-side cache (the long keys'
    plan rebuilt feature by feature) with one key of about 160k occurrences
    (past 64 x 1024 entries, so its chunks grow to 192), hot keys of 700 to
    2800 occurrences, long keys of about 150 and a cold tail, in 4 features
    of 270k bags, with empty bags for sum pooling; two steps."""
    spec = W.TableSpec(dim=64, dtype="f32", optim="adam", pool=pool, lr=1e-3, eps=1e-8, admit_threshold=admit)
    B, F = 270_000, 4
    batches = []
    for step in range(2):
        rng = W.rng_for(98, step)
        feats = []
        for f in range(F):
            lens = rng.integers(0 if pool == "sum" else 1, 5, B)
            off = W.offsets_from_lengths(lens)
            n = int(off[-1])
            r = rng.random(n)
            vals = rng.integers(100_000, 5_000_000, n)                          # cold tail
            vals = np.where(r < 0.35, rng.integers(10_000, 11_000, n), vals)    # ~150 each
            # 20 hot keys, rates 1..2 x 1/400: from about 1300 down to 700
            hot = (20 * rng.random(n) ** 1.4).astype(np.int64)
            vals = np.where(r < 0.05, hot, vals)
            if f == 0:
                vals = np.where(rng.random(n) < 0.30, 7, vals)                  # ~160k of key 7
            feats.append(W.FeatureInput(values=vals.astype(np.int64), bag_offsets=off, slot=f + 1))
        batches.append(W.Batch(feats, B, rng.standard_normal((B, F * 64), dtype=np.float32)))
    assert B * F * 64 * 4 > 256 * 2**20
    v0 = batches[0].features[0].values
    counts = np.bincount(v0[v0 < 64])
    assert (counts[:20] >= 1024).any() and (counts[:20] < 1024).any()
    assert np.count_nonzero(batches[0].features[0].values == 7) > 131072
    run_parity(spec, batches, export_every=2)


@pytest.mark.parametrize("pool,admit", [("mean", 1), ("sum", 2)])
def test_heavy_buckets(pool, admit):
    """Hot keys whose buckets exceed the single-block size (tens of thousands
    of occurrences each, sliced across blocks) next to a tail of ordinary
    keys; a second step mixes new and stored rows, a third looks up only."""
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.TableSpec(dim=32, dtype="f32", optim="adam", pool=pool, lr=1e-3, eps=1e-8, admit_threshold=admit)
    rng = W.rng_for(123, admit)
    B = 6000

    def batch(step):
        r = W.rng_for(124, admit, step)
        lens = r.poisson(16, B)
        off = W.offsets_from_lengths(lens)
        n = int(off[-1])
        hot = np.array([11, 22, 33, 44], np.int64) + step
        p = r.random(n)
        vals = np.where(p < 0.30, hot[0], np.where(p < 0.50, hot[1], np.where(p < 0.62, hot[2],
                        np.where(p < 0.64, hot[3], r.integers(1000, 40000, n)))))
        return W.Batch([W.FeatureInput(values=vals.astype(np.int64), bag_offsets=off, slot=3)], B,
                       r.standard_normal((B, 32), dtype=np.float32))
    run_parity(spec, [batch(0), batch(1)])
    # find-only over the same table (hot keys present and absent)
    table = make_table(spec)
    otab = oracle.OracleTable(spec)
    for st in range(2):
        b = batch(st)
        res = recis.LookupResult(b.n, B)
        gpu_step(table, spec, b, res)
        oracle_step(otab, spec, b)
    b = batch(5)
    res = recis.LookupResult(b.n, B)
    out, _ = gpu_step(table, spec, b, res, find_only=True, with_backward=False)
    r, oout, oab = oracle_step(otab, spec, b, find_only=True, with_backward=False)
    torch.cuda.synchronize()
    assert table.get_error() == 0
    check_lookup(canon_lookup(res), r)
    check_forward(out, spec, oout, oab, r.merged_offsets, r.num_feats)
    table.close()


def _ids_in_first_hash_bucket(count, bits, rng):
    """Ids (slot 0, no transform: key == id) whose Fibonacci hash has `bits`
    leading zero bits, i.e. that all land in the first hash bucket of the
    lookup's partition."""
    out = []
    while sum(len(x) for x in out) < count:
        c = rng.integers(1, 1 << 47, 200000, dtype=np.int64)
        h = c.astype(np.uint64) * np.uint64(0x9E3779B97F4A7C15)   # wraps mod 2^64
        out.append(c[(h >> np.uint64(64 - bits)) == 0])
    return np.unique(np.concatenate(out))[:count]


def test_bucket_overflow_path():
    """2000 distinct keys that collide in the top 8 bits of the partition
    hash: 3000 occurrences make 256 buckets (the floor for small calls, bits
    = 8), so all of them land in one bucket and overflow its LDS table; the
    global-table path must give the same lookup, forward and update as the
    oracle.  In the IDMap (1024 regions of 1024 slots) they share 4 regions."""
    spec = W.TableSpec(dim=16, dtype="f32", optim="adagrad", pool="sum", lr=0.05)
    rng = W.rng_for(91)
    ids = _ids_in_first_hash_bucket(2000, 8, rng)
    vals = np.concatenate([ids, rng.choice(ids, 1000)])
    rng.shuffle(vals)
    B = 300
    off = (np.arange(B + 1) * (vals.size // B)).astype(np.int32)
    b = W.Batch([W.FeatureInput(values=vals.astype(np.int64), bag_offsets=off, slot=0)], B,
                rng.standard_normal((B, 16), dtype=np.float32))
    run_parity(spec, [b, b])


@pytest.mark.parametrize("pool", ["sum", "none"])
def test_heavy_bucket_sliced(pool):
    """20,000 distinct keys that collide in the top 8 bits of the partition
    hash, three occurrences each, shuffled, beside 4000 ordinary occurrences:
    64,000 occurrences make 256 buckets (the floor for small calls, bits =
    8), and the first one gets about 56k (key, tile) pairs, past the 16,384
    at which a bucket is cut into slices that separate blocks deduplicate
    through the global table.  Two steps (inserts, then stored rows) at
    parity with the oracle.  The keys also share their IDMap regions (the
    same top bits pick them), 1/256 of the slots: a 2^24-slot IDMap gives
    them 65,536."""
    spec = W.TableSpec(dim=16, dtype="f32", optim="adagrad", pool=pool, lr=0.05, eps=1e-10)
    rng = W.rng_for(93)
    ids = _ids_in_first_hash_bucket(20000, 8, rng)
    assert ids.size == 20000
    batches = []
    for step in range(2):
        r = W.rng_for(94, step)
        vals = np.concatenate([np.repeat(ids, 3), r.integers(1, 1 << 40, 4000)])
        r.shuffle(vals)
        B = 1000
        off = (np.arange(B + 1) * (vals.size // B)).astype(np.int32)
        rows = vals.size if pool == "none" else B
        batches.append(W.Batch([W.FeatureInput(values=vals.astype(np.int64), bag_offsets=off, slot=0)], B,
                               r.standard_normal((rows, 16), dtype=np.float32)))
    run_parity(spec, batches, table_kw=dict(slot_capacity=1 << 24))


@pytest.mark.parametrize("row_offset", [0, 1])
def test_writeback_cache_last_writer_wins(row_offset):
    """row_offset 1 hands the rows over 4 bytes past a 16-byte boundary (the
    one-wave-per-key path); 0 takes the sixteen-lanes-per-key path."""
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.spec_cache()
    table = make_table(spec)
    otab = oracle.OracleTable(spec)
    keys = W.cache_keys(5000)

    def dev_rows(e):
        buf = torch.empty(e.size + row_offset, dtype=torch.float32, device="cuda")
        rows = buf[row_offset:].view(e.shape)
        rows.copy_(torch.from_numpy(e))
        assert (rows.data_ptr() % 16 == 0) == (row_offset == 0)
        return rows
    # pre-insert the cache keys, then write batches with repeated keys
    table.writeback(torch.from_numpy(keys).cuda(), dev_rows(np.zeros((keys.size, 256), np.float32)))
    otab.writeback(keys, np.zeros((keys.size, 256), np.float32))
    for step in range(3):
        k, e = W.cache_writes(step, keys, n=3000)
        k = np.concatenate([k, np.array([1 << 45, 1 << 45], np.int64)])   # a miss, written twice
        e = np.concatenate([e, W.rng_for(step, 99).standard_normal((2, 256), dtype=np.float32)])
        table.writeback(torch.from_numpy(k).cuda(), dev_rows(e))
        assert otab.writeback(k, e) == 0
        torch.cuda.synchronize()
        assert table.get_error() == 0
        g, o = canon_export(table), otab.export()
        np.testing.assert_array_equal(g["keys"], o["keys"])
        np.testing.assert_array_equal(g["params"], o["params"])   # bit-exact RNE of the last write
    table.close()


def test_device_errors_are_reported():
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.spec_tiny()
    # raw negative id -> KEY_RANGE
    table = make_table(spec)
    b = W.Batch([W.FeatureInput(values=np.array([5, -3, 7], np.int64), bag_offsets=np.array([0, 2, 3], np.int32),
                                slot=0)], 2, np.ones((2, 16), np.float32))
    res = recis.LookupResult(3, 2)
    gpu_step(table, spec, b, res)
    assert table.get_error() == recis.RECIS_ERR_KEY_RANGE
    assert table.get_error() == 0   # read-and-clear
    # malformed bag offsets -> INVALID_ARG, no fault
    bad = W.Batch([W.FeatureInput(values=np.array([1, 2, 3, 4], np.int64),
                                  bag_offsets=np.array([0, 3, 1, 4], np.int32), slot=0)], 3,
                  np.ones((3, 16), np.float32))
    res = recis.LookupResult(4, 3)
    gpu_step(table, spec, bad, res)
    assert table.get_error() == recis.RECIS_ERR_INVALID_ARG
    table.close()
    # row capacity -> CAPACITY, keys past the limit get no row
    table = make_table(spec, max_rows=100, block_rows=64)
    b = W.tiny_batch(0, id_space=100000)
    res = recis.LookupResult(b.n, b.batch)
    table.insert_find(device_features(b), b.batch, res)
    torch.cuda.synchronize()
    assert table.get_error() == recis.RECIS_ERR_CAPACITY
    rows = res.unique_rows[:res.U()].cpu().numpy()
    offsets = rows[rows >= 0] & ((1 << 62) - 1)     # bit 62: not yet written
    assert offsets.size == 100 and offsets.max() < 100 and np.unique(offsets).size == 100
    table.close()
    # argument errors surface as exceptions
    with pytest.raises(recis.RecisError):
        recis.Table(dim=48)


# ---- save / restore through a SafeTensors file (export -> file -> import)
def _save_load_resume(spec, before, after, path, load_kw):
    """Steps `before` on a table and on the oracle; the table saved to `path`
    and restored into a new table laid out by load_kw; its content checked
    against the oracle's; then the steps `after` on the restored table and on
    the oracle (which never stopped), checked step by step."""
    import torch
    from dynamic_embedding_tables_amd import recis, saver
    table = make_table(spec)
    otab = oracle.OracleTable(spec)
    for b in before:
        res = recis.LookupResult(max(b.n, 1), b.num_feats * b.batch)
        gpu_step(table, spec, b, res)
        oracle_step(otab, spec, b)
    torch.cuda.synchronize()
    assert table.get_error() == 0
    n = saver.save(table, path)
    assert n == otab.size()
    adam_step = table.stats().adam_step
    table.close()
    restored = saver.load(path, **load_kw)
    assert restored.get_error() == 0
    st = restored.stats()
    assert st.adam_step == adam_step and st.keys == otab.size() and st.rows_in_use == otab.rows_in_use()
    check_export(canon_export(restored), otab.export(), spec)
    for step, b in enumerate(after):
        print(f"[resume] step {step} N={b.n}", flush=True)
        res = recis.LookupResult(max(b.n, 1), b.num_feats * b.batch)
        out, _ = gpu_step(restored, spec, b, res)
        r, oout, oab = oracle_step(otab, spec, b)
        torch.cuda.synchronize()
        assert restored.get_error() == 0
        check_lookup(canon_lookup(res), r)
        check_forward(out, spec, oout, oab, r.merged_offsets, r.num_feats)
    check_export(canon_export(restored), otab.export(), spec)
    restored.close()


def test_save_load_resume_ctr_adam(tmp_path):
    """Adam (its step counter travels in the file), restored into a small
    table that grows while the keys are imported."""
    spec = W.spec_ctr()
    _save_load_resume(spec, [W.ctr_batch(s, batch=256) for s in range(2)], [W.ctr_batch(2, batch=256)],
                      str(tmp_path / "ctr.safetensors"), dict(slot_capacity=64, block_rows=256))


def test_save_load_resume_admission_and_bf16(tmp_path):
    """Keys still waiting for admission (no row, count kept), restored into
    host-memory blocks; and the bf16 sequence table with its hot keys."""
    spec = W.spec_multi(2)
    _save_load_resume(spec, [W.multi_batch(s, 2, batch=128, num_feats=6) for s in range(2)],
                      [W.multi_batch(s, 2, batch=128, num_feats=6) for s in range(2, 4)],
                      str(tmp_path / "multi.safetensors"), dict(block_memory="host"))
    _save_load_resume(W.spec_seq(), [W.seq_batch(0, batch=12, seq_len=1000)], [W.seq_batch(1, batch=12, seq_len=1000)],
                      str(tmp_path / "seq.safetensors"), {})


def test_save_load_resume_admission_state(tmp_path):
    """A table with last-use stamps and count-min admission saved and
    restored (the ages and the sketch travel in the file), then LRU-bounded
    and sketch-admitted steps against the oracle that never stopped."""
    import torch
    from dynamic_embedding_tables_amd import recis, saver
    spec = W.spec_multi(3)
    table = make_table(spec, track_last_use=True, admit_sketch_bits=8)
    otab = oracle.OracleTable(spec)
    otab.set_sketch(8)
    for s in range(3):
        b = W.multi_batch(s, 3, batch=96, num_feats=5)
        gpu_step(table, spec, b, recis.LookupResult(max(b.n, 1), b.num_feats * b.batch))
        oracle_step(otab, spec, b)
    torch.cuda.synchronize()
    assert table.get_error() == 0
    path = str(tmp_path / "adm.safetensors")
    saver.save(table, path)
    table.close()
    restored = saver.load(path)
    check_export(canon_export(restored), otab.export(), spec)
    ne = torch.zeros(1, dtype=torch.int64, device="cuda")
    for s in range(3, 7):
        b = W.multi_batch(s, 3, batch=96, num_feats=5)
        res = recis.LookupResult(max(b.n, 1), b.num_feats * b.batch)
        out, _ = gpu_step(restored, spec, b, res)
        r, oout, oab = oracle_step(otab, spec, b)
        torch.cuda.synchronize()
        assert restored.get_error() == 0
        check_lookup(canon_lookup(res), r)
        check_forward(out, spec, oout, oab, r.merged_offsets, r.num_feats)
        if s == 4:
            restored.evict_lru(1500, ne)
            assert int(ne.item()) == otab.evict_lru(1500)
        check_export(canon_export(restored), otab.export(), spec)
    restored.close()


def test_import_rejects_used_tables_and_repeated_keys():
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.spec_tiny()
    keys = torch.tensor([5, 9, 5], dtype=torch.int64, device="cuda")
    rows = torch.zeros(3, dtype=torch.int64, device="cuda")
    counts = torch.ones(3, dtype=torch.int32, device="cuda")
    params = torch.zeros(3, spec.dim, dtype=torch.float32, device="cuda")
    state = torch.zeros(3, spec.dim, dtype=torch.float32, device="cuda")
    t = make_table(spec)
    t.import_(keys, rows, counts, params, state)           # 5 twice
    assert t.get_error() == recis.RECIS_ERR_INVALID_ARG
    with pytest.raises(recis.RecisError) as e:              # the table now holds keys
        t.import_(keys[:2], rows[:2], counts[:2], params[:2], state[:2])
    assert e.value.status == recis.RECIS_ERR_INVALID_ARG
    t.close()
    t = make_table(spec)
    b = W.tiny_batch(0)
    res = recis.LookupResult(b.n, b.batch)
    gpu_step(t, spec, b, res)
    with pytest.raises(recis.RecisError):
        t.import_(keys[:2], rows[:2], counts[:2], params[:2], state[:2])
    t.close()
