"""Pins of the oracle's table-level steps against libraries, brute force,
closed forms and invariants (no GPU).

dedup      -> numpy.unique(return_inverse, return_counts)
IDMap      -> a brute-force Python dict with counts, admission and eviction
forward    -> torch.nn.functional.embedding_bag / embedding (float64)
reduce     -> torch autograd through embedding_bag(sparse=True), coalesced
Adagrad    -> torch.optim.Adagrad (sparse gradients)
Adam       -> torch.optim.SparseAdam (lazy, one step counter per table)
writeback  -> torch.optim.SGD(lr=1) on 0.5*||M - e||^2, and last-writer brute force
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import (FeatureInput, TableSpec, bucketize_feature, offsets_from_lengths,
                       rng_for, tiny_batch, to_bf16_bits)


def small_features(seed, nfeat=3, batch=17, id_space=40, mean_len=3.0, empty_ok=True):
    rng = rng_for(99, seed)
    feats = []
    for f in range(nfeat):
        lens = rng.poisson(mean_len, batch)
        if not empty_ok:
            lens = np.maximum(lens, 1)
        off = offsets_from_lengths(lens)
        vals = rng.integers(0, id_space, int(off[-1]), dtype=np.int64)
        feats.append(FeatureInput(values=vals, bag_offsets=off, slot=f))
    return feats


def keys_of(feats):
    return np.concatenate([(np.int64(f.slot) << np.int64(48)) | f.values for f in feats])


def canonical_matrix(tab, keys_needed):
    """Dense [len(keys_needed), D] float64 matrix of the oracle's rows (zeros where
    the key has no row) and the export it came from."""
    ex = tab.export()
    pos = np.searchsorted(ex["keys"], keys_needed)
    found = (pos < ex["keys"].size) & (ex["keys"][np.minimum(pos, ex["keys"].size - 1)] == keys_needed)
    W = np.zeros((keys_needed.size, tab.dim))
    has = found.copy()
    has[found] = ex["rows"][pos[found]] >= 0
    W[has] = ex["params"][pos[has]]
    return W, ex


# --------------------------------------------------------------------- dedup
def test_dedup_and_merge_match_numpy():
    feats = small_features(1, nfeat=4, batch=23)
    tab = oracle.OracleTable(TableSpec(dim=8, dtype="f32", optim="adagrad", pool="sum"))
    r = tab.insert_find(feats, 23)
    assert r.status == 0
    keys = keys_of(feats)
    u, inv, cnt = np.unique(keys, return_inverse=True, return_counts=True)
    assert r.U == u.size
    np.testing.assert_array_equal(r.unique_keys[:r.U], u)
    np.testing.assert_array_equal(r.inverse[:keys.size], inv)
    np.testing.assert_array_equal(r.counts[:r.U], cnt)
    base = np.cumsum([0] + [f.n for f in feats])
    want = np.concatenate([f.bag_offsets[:-1] + base[i] for i, f in enumerate(feats)] + [[base[-1]]])
    np.testing.assert_array_equal(r.merged_offsets, want)


def test_empty_batch():
    feats = [FeatureInput(values=np.zeros(0, np.int64), bag_offsets=np.zeros(6, np.int32), slot=0)]
    tab = oracle.OracleTable(TableSpec(dim=8, dtype="f32", optim="adagrad", pool="mean"))
    r = tab.insert_find(feats, 5)
    assert r.status == 0 and r.U == 0
    out = tab.forward(r, "mean")
    assert out.shape == (5, 8) and not out.any()
    assert tab.backward_update(r, "mean", np.ones((5, 8), np.float32)) == 0


# --------------------------------------------------------------------- IDMap
class DictTable:
    """Brute force: key -> [has_row, count], and per key the number of the
    counting lookup that last saw it."""

    def __init__(self, admit):
        self.m, self.admit = {}, admit
        self.last, self.now = {}, 0

    def step(self, keys, find_only=False):
        out = {}
        if not find_only:
            self.now += 1
            for k in np.unique(keys):
                self.last[k] = self.now
        for k in np.unique(keys):
            c = int((keys == k).sum())
            if find_only:
                out[k] = k in self.m and self.m[k][0]
                continue
            e = self.m.setdefault(k, [False, 0])
            e[1] += c
            if not e[0] and e[1] >= self.admit:
                e[0] = True
            out[k] = e[0]
        return out

    def evict_lru(self, max_keys):
        """Keeps the keys seen most recently, whole lookups at a time (ages
        from 255 on are one), within max_keys; returns how many left."""
        by_age = sorted(self.m, key=lambda k: min(self.now - self.last[k], 255))
        ages = [min(self.now - self.last[k], 255) for k in by_age]
        kept, i = 0, 0
        while i < len(by_age):
            j = i
            while j < len(by_age) and ages[j] == ages[i]:
                j += 1
            if kept + (j - i) > max_keys:
                break
            kept, i = kept + (j - i), j
        gone = by_age[i:]
        for k in gone:
            del self.m[k]
        return len(gone)

    def evict(self, t, decay=0.0):
        """Survivors keep floor(count * decay): written with integer
        arithmetic where the factor allows (0, 1/2, 1), else in binary64."""
        gone = [k for k, e in self.m.items() if e[1] < t]
        for k in gone:
            del self.m[k]
        for e in self.m.values():
            if decay == 0.0:
                e[1] = 0
            elif decay == 0.5:
                e[1] >>= 1
            elif decay != 1.0:
                e[1] = math.floor(e[1] * decay)
        return len(gone)


@pytest.mark.parametrize("admit", [1, 2, 3])
def test_idmap_against_brute_force(admit):
    spec = TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum", admit_threshold=admit)
    tab, ref = oracle.OracleTable(spec), DictTable(admit)
    for step in range(12):
        feats = small_features(100 + step, nfeat=2, batch=9, id_space=25)
        find_only = step % 5 == 4
        r = tab.insert_find(feats, 9, flags=oracle.FIND_ONLY if find_only else 0)
        assert r.status == 0
        want = ref.step(keys_of(feats), find_only)
        got = {int(k): int(row) >= 0 for k, row in zip(r.unique_keys[:r.U], r.unique_rows[:r.U])}
        assert got == {int(k): v for k, v in want.items()}
        if step % 4 == 3:
            assert tab.evict(2) == ref.evict(2)
        ex = tab.export()
        assert [int(k) for k in ex["keys"]] == sorted(int(k) for k in ref.m)
        assert [int(c) for c in ex["counts"]] == [ref.m[k][1] for k in sorted(ref.m)]
        assert [bool(r_ >= 0) for r_ in ex["rows"]] == [ref.m[k][0] for k in sorted(ref.m)]
        rows = ex["rows"][ex["rows"] >= 0]
        assert np.unique(rows).size == rows.size          # bijection key <-> row
        assert tab.rows_in_use() == rows.size


def test_reinsert_is_idempotent_and_counts_add():
    feats = small_features(7)
    tab = oracle.OracleTable(TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum"))
    a = tab.insert_find(feats, 17)
    b = tab.insert_find(feats, 17)
    np.testing.assert_array_equal(a.unique_rows[:a.U], b.unique_rows[:b.U])
    ex = tab.export()
    np.testing.assert_array_equal(ex["counts"], 2 * a.counts[:a.U])


def test_content_independent_of_insertion_order():
    spec = TableSpec(dim=8, dtype="f32", optim="adam", pool="sum", lr=1e-3, eps=1e-8)
    feats = small_features(8, nfeat=1, batch=40, id_space=60)
    keys = feats[0].values
    late = keys[keys >= 30]
    first = [FeatureInput(values=late, bag_offsets=offsets_from_lengths(np.array([late.size])), slot=0)]
    t1, t2 = oracle.OracleTable(spec), oracle.OracleTable(spec)
    t1.insert_find(feats, 40)
    t2.insert_find(first, 1)            # the high keys take the low rows in t2
    t2.insert_find(feats, 40)
    e1, e2 = t1.export(), t2.export()
    np.testing.assert_array_equal(e1["keys"], e2["keys"])
    np.testing.assert_array_equal(e1["params"], e2["params"])
    assert not np.array_equal(e1["rows"], e2["rows"])


def test_capacity_limits():
    spec = TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum")
    feats = [FeatureInput(values=np.arange(10, dtype=np.int64), bag_offsets=np.array([0, 10], np.int32), slot=0)]
    tab = oracle.OracleTable(spec, max_rows=6)
    r = tab.insert_find(feats, 1)
    assert r.status == 3
    assert (r.unique_rows[:10] >= 0).sum() == 6 and tab.size() == 10
    tab = oracle.OracleTable(spec, max_keys=4)
    r = tab.insert_find(feats, 1)
    assert r.status == 3 and tab.size() == 4 and (r.unique_rows[:10] >= 0).sum() == 4


# ------------------------------------------------------------------- forward
def torch_pool(W, feats, batch, pool, r):
    keys = keys_of(feats)
    idx = torch.from_numpy(np.searchsorted(r.unique_keys[:r.U], keys))
    offs = torch.from_numpy(r.merged_offsets[:-1].astype(np.int64))
    out = torch.nn.functional.embedding_bag(idx, torch.from_numpy(W), offs, mode=pool)
    F = len(feats)
    return out.reshape(F, batch, -1).permute(1, 0, 2).reshape(batch, -1).numpy()


@pytest.mark.parametrize("pool", ["sum", "mean"])
@pytest.mark.parametrize("admit", [1, 2])
def test_forward_matches_embedding_bag(pool, admit):
    spec = TableSpec(dim=16, dtype="f32", optim="adagrad", pool=pool, admit_threshold=admit)
    tab = oracle.OracleTable(spec)
    for step in range(3):
        feats = small_features(200 + step, nfeat=3, batch=31, id_space=50)
        r = tab.insert_find(feats, 31)
        out, ab = tab.forward(r, pool, with_abs=True)
        W, _ = canonical_matrix(tab, r.unique_keys[:r.U])
        want = torch_pool(W, feats, 31, pool, r)
        np.testing.assert_allclose(out, want, rtol=0, atol=1e-7)
        np.testing.assert_allclose(ab, torch_pool(np.abs(W), feats, 31, pool, r), rtol=1e-12, atol=0)
        tab.backward_update(r, pool, rng_for(5, step).standard_normal((31, 3 * 16), dtype=np.float32))


def test_forward_none_is_exact_row_copy_bf16():
    spec = TableSpec(dim=8, dtype="bf16", optim="adagrad", pool="none", grad_dtype="bf16")
    tab = oracle.OracleTable(spec)
    feats = small_features(3, nfeat=1, batch=6, id_space=20)
    r = tab.insert_find(feats, 6)
    out = tab.forward(r, "none")
    keys = keys_of(feats)
    want = np.stack([oracle.init_row(spec.seed, int(k), 8) for k in keys])
    want_bits = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(out, want_bits)


# -------------------------------------------------------------------- reduce
@pytest.mark.parametrize("pool", ["sum", "mean", "none"])
def test_reduce_matches_autograd(pool):
    spec = TableSpec(dim=8, dtype="f32", optim="adagrad", pool=pool)
    tab = oracle.OracleTable(spec)
    feats = small_features(11, nfeat=2, batch=19, id_space=15)
    r = tab.insert_find(feats, 19)
    n = r.n
    g = rng_for(6).standard_normal((n, 8) if pool == "none" else (19, 16), dtype=np.float32)
    G = tab.reduce_grads(r, pool, g)
    keys = keys_of(feats)
    idx = torch.from_numpy(np.searchsorted(r.unique_keys[:r.U], keys))
    W = torch.zeros(r.U, 8, dtype=torch.float64, requires_grad=True)
    if pool == "none":
        out = torch.nn.functional.embedding(idx, W, sparse=True)
        out.backward(torch.from_numpy(g.astype(np.float64)))
    else:
        offs = torch.from_numpy(r.merged_offsets[:-1].astype(np.int64))
        out = torch.nn.functional.embedding_bag(idx, W, offs, mode=pool, sparse=True)
        go = torch.from_numpy(g.astype(np.float64)).reshape(19, 2, 8).permute(1, 0, 2).reshape(38, 8)
        out.backward(go)
    want = W.grad.coalesce().to_dense().numpy()
    np.testing.assert_allclose(G, want, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------- optimizers
def _run_against_torch(spec, steps, pool="sum", id_space=30):
    """Run the oracle and torch (float64, stored values rounded to float32 after each
    step as the table stores them) side by side on the dense canonical matrix."""
    tab = oracle.OracleTable(spec)
    universe = np.arange(id_space, dtype=np.int64)  # slot 0
    W = torch.tensor(np.stack([oracle.init_row(spec.seed, int(k), spec.dim) for k in universe]),
                     dtype=torch.float64, requires_grad=True)
    if spec.optim == "adagrad":
        opt = torch.optim.Adagrad([W], lr=spec.lr, eps=spec.eps, initial_accumulator_value=0.0)
    else:
        opt = torch.optim.SparseAdam([W], lr=spec.lr, betas=(spec.beta1, spec.beta2), eps=spec.eps)
    seen = set()
    for step in range(steps):
        rng = rng_for(77, step)
        B = 13
        lens = rng.poisson(2.0, B)
        off = offsets_from_lengths(lens)
        vals = rng.integers(0, id_space // (1 + (step < 2)), int(off[-1]), dtype=np.int64)
        feats = [FeatureInput(values=vals, bag_offsets=off, slot=0)]
        r = tab.insert_find(feats, B)
        g = rng.standard_normal((B, spec.dim), dtype=np.float32)
        assert tab.backward_update(r, pool, g) == 0
        seen.update(int(v) for v in vals)
        opt.zero_grad()
        out = torch.nn.functional.embedding_bag(torch.from_numpy(vals), W,
                                                torch.from_numpy(off[:-1].astype(np.int64)),
                                                mode=pool, sparse=True)
        out.backward(torch.from_numpy(g.astype(np.float64)))
        opt.step()
        with torch.no_grad():        # storage is float32
            W.copy_(W.float().double())
            for st in opt.state[W].values():
                if torch.is_tensor(st) and st.dtype == torch.float64:
                    st.copy_(st.float().double())
    ex = tab.export()
    k = np.array(sorted(seen), dtype=np.int64)
    np.testing.assert_array_equal(ex["keys"], k)
    return ex, W.detach().numpy()[k], opt.state[W], k


def test_adagrad_matches_torch():
    spec = TableSpec(dim=8, dtype="f32", optim="adagrad", pool="sum", lr=0.01, eps=1e-10)
    ex, Wt, st, k = _run_against_torch(spec, 6)
    np.testing.assert_allclose(ex["params"], Wt, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(ex["state"], st["sum"].numpy()[k], rtol=1e-6, atol=1e-12)


def test_sparse_adam_matches_torch():
    spec = TableSpec(dim=8, dtype="f32", optim="adam", pool="mean", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    ex, Wt, st, k = _run_against_torch(spec, 7, pool="mean")
    np.testing.assert_allclose(ex["params"], Wt, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(ex["state"][:, :8], st["exp_avg"].numpy()[k], rtol=1e-5, atol=1e-12)
    np.testing.assert_allclose(ex["state"][:, 8:], st["exp_avg_sq"].numpy()[k], rtol=1e-5, atol=1e-14)


@pytest.mark.parametrize("optim", ["adagrad", "adam"])
def test_first_touch_closed_form(optim):
    spec = TableSpec(dim=8, dtype="f32", optim=optim, pool="sum", lr=0.01 if optim == "adagrad" else 1e-3,
                     eps=1e-10 if optim == "adagrad" else 1e-8)
    tab = oracle.OracleTable(spec)
    # warm the step counter with an unrelated key, then touch fresh keys at step t
    t = 4
    for s in range(t - 1):
        f = [FeatureInput(values=np.array([999], np.int64), bag_offsets=np.array([0, 1], np.int32), slot=0)]
        r = tab.insert_find(f, 1)
        tab.backward_update(r, "sum", np.ones((1, 8), np.float32))
    vals = np.array([1, 2, 2, 3, 3, 3], np.int64)
    f = [FeatureInput(values=vals, bag_offsets=np.array([0, 1, 3, 6], np.int32), slot=0)]
    r = tab.insert_find(f, 3)
    g = rng_for(3).standard_normal((3, 8), dtype=np.float32)
    tab.backward_update(r, "sum", g)
    G = g.astype(np.float64) * np.array([[1], [2], [3]])
    w0 = np.stack([oracle.init_row(spec.seed, k, 8) for k in (1, 2, 3)]).astype(np.float64)
    if optim == "adagrad":
        want = w0 - spec.lr * G / (np.abs(G) + spec.eps)
    else:
        b1, b2 = spec.beta1, spec.beta2
        want = w0 - spec.lr * np.sqrt(1 - b2**t) / (1 - b1**t) * (1 - b1) * G / (np.sqrt(1 - b2) * np.abs(G) + spec.eps)
    ex = tab.export()
    np.testing.assert_allclose(ex["params"][:3], want.astype(np.float32), rtol=2e-7, atol=1e-9)


def test_zero_gradient_touch_still_updates_adam():
    spec = TableSpec(dim=4, dtype="f32", optim="adam", pool="sum", lr=1e-3, eps=1e-8)
    tab = oracle.OracleTable(spec)
    f = [FeatureInput(values=np.array([5], np.int64), bag_offsets=np.array([0, 1], np.int32), slot=0)]
    r = tab.insert_find(f, 1)
    tab.backward_update(r, "sum", np.ones((1, 4), np.float32))
    before = tab.export()
    r = tab.insert_find(f, 1)
    tab.backward_update(r, "sum", np.zeros((1, 4), np.float32))
    after = tab.export()
    assert np.all(after["params"] != before["params"])
    np.testing.assert_allclose(after["state"][:, :4], 0.9 * before["state"][:, :4], rtol=1e-6)


def test_bf16_update_rounds_once():
    spec = TableSpec(dim=8, dtype="bf16", optim="adagrad", pool="none", lr=0.01, eps=1e-10, grad_dtype="bf16")
    tab = oracle.OracleTable(spec)
    vals = np.array([4, 4, 9, 4, 9, 1], np.int64)
    f = [FeatureInput(values=vals, bag_offsets=np.array([0, 3, 6], np.int32), slot=0)]
    r = tab.insert_find(f, 2)
    g = to_bf16_bits(rng_for(8).standard_normal((6, 8), dtype=np.float32))
    gf = torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).double().numpy()
    tab.backward_update(r, "none", g, "bf16")
    ex = tab.export()
    for i, k in enumerate((1, 4, 9)):
        w0 = torch.tensor(oracle.init_row(spec.seed, k, 8)).to(torch.bfloat16).double().numpy()
        G = gf[vals == k].sum(0)
        a = np.float32(G * G).astype(np.float64)  # state stored as float32
        want = w0 - spec.lr * G / (np.sqrt(G * G) + spec.eps)
        np.testing.assert_array_equal(ex["state"][i], a.astype(np.float32))
        wb = oracle.round_bf16(want)
        got = ex["params"][i].view(np.uint32) >> 16
        np.testing.assert_array_equal(got, wb)


def test_bf16_update_rounds_once_at_a_tie_of_the_float_rounding():
    """Adagrad with eps = 0 from a row written to exactly 1.0: the new value is
    exactly 1 - lr in binary64 (lr * g / |g| = lr exactly).  Each lr puts
    1 - lr a quarter of a float32 unit above (or below) a midpoint between two
    bfloat16 neighbours.  Rounded once, it goes to the neighbour on its side;
    rounded to float32 first, it would land on the midpoint and tie to the even
    neighbour.  The expected bits are fixed by that construction, not by the
    oracle's own rounding routine."""
    cases = []  # (lr, expected bf16 bits of 1 - lr)
    for k in (100, 37, 64, 3):
        lo = 0.5 + k * 2.0**-8            # bf16 neighbours in [0.5, 1): spacing 2^-8
        mid = lo + 2.0**-9
        even_is_lo = k % 2 == 0
        # a quarter float32 unit on the odd neighbour's side of the midpoint:
        # single rounding gives the odd neighbour, double rounding the even one
        want = mid + (2.0**-26 if even_is_lo else -2.0**-26)
        odd = lo + 2.0**-8 if even_is_lo else lo
        bits = int(np.array([odd], np.float32).view(np.uint32)[0] >> 16)
        assert np.array([odd], np.float32).view(np.uint32)[0] & 0xFFFF == 0
        cases.append((1.0 - want, bits))
    for lr, bits in cases:
        spec = TableSpec(dim=8, dtype="bf16", optim="adagrad", pool="none", lr=lr, eps=0.0, grad_dtype="bf16")
        tab = oracle.OracleTable(spec)
        assert tab.writeback(np.array([11], np.int64), np.ones((1, 8), np.float32)) == 0
        f = [FeatureInput(values=np.array([11], np.int64), bag_offsets=np.array([0, 1], np.int32), slot=0)]
        r = tab.insert_find(f, 1)
        g = to_bf16_bits(np.full((1, 8), 0.75, np.float32))
        assert tab.backward_update(r, "none", g, "bf16") == 0
        got = tab.export()["params"][0].view(np.uint32) >> 16
        np.testing.assert_array_equal(got, np.full(8, bits, np.uint32))


def test_stale_lookup_acts_on_current_rows():
    """A lookup's backward after an eviction pass and a later insert: the
    evicted key gets nothing, and the key that took over its row keeps its
    initial values; the surviving key gets the closed-form Adagrad step."""
    spec = TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum", lr=0.01, eps=1e-10)
    tab = oracle.OracleTable(spec)
    f = [FeatureInput(values=np.array([1, 1, 2], np.int64), bag_offsets=np.array([0, 2, 3], np.int32), slot=0)]
    ra = tab.insert_find(f, 2)                       # key 1 twice, key 2 once
    assert tab.evict(2) == 1                         # key 2 leaves, its row is freed
    fb = [FeatureInput(values=np.array([7], np.int64), bag_offsets=np.array([0, 1], np.int32), slot=0)]
    tab.insert_find(fb, 1)                           # key 7 takes the freed row
    g = np.array([[1, -2, 3, -4], [5, 6, -7, 8]], np.float32)
    assert tab.backward_update(ra, "sum", g) == 0
    ex = tab.export()
    assert list(ex["keys"]) == [1, 7]
    G1 = 2.0 * g[0].astype(np.float64)               # key 1 sits twice in bag 0
    w1 = oracle.init_row(spec.seed, 1, 4).astype(np.float64)
    np.testing.assert_allclose(ex["params"][0], (w1 - spec.lr * G1 / (np.abs(G1) + spec.eps)).astype(np.float32),
                               rtol=2e-7)
    np.testing.assert_array_equal(ex["params"][1], oracle.init_row(spec.seed, 7, 4))
    np.testing.assert_array_equal(ex["state"][1], np.zeros(4, np.float32))


@pytest.mark.parametrize("decay", [0.0, 0.5, 1.0, 0.3])
def test_evict_decay_against_brute_force(decay):
    """Eviction passes whose survivors keep floor(count * decay), with
    admission at 2: the evicted sets, counts, admissions and rows step by step
    against the dict."""
    spec = TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum", admit_threshold=2)
    tab, ref = oracle.OracleTable(spec), DictTable(2)
    for step in range(14):
        feats = small_features(300 + step, nfeat=2, batch=9, id_space=30)
        r = tab.insert_find(feats, 9)
        assert r.status == 0
        want = ref.step(keys_of(feats), False)
        got = {int(k): int(row) >= 0 for k, row in zip(r.unique_keys[:r.U], r.unique_rows[:r.U])}
        assert got == {int(k): v for k, v in want.items()}
        if step % 3 == 2:
            assert tab.evict(3, decay) == ref.evict(3, decay)
        ex = tab.export()
        assert [int(k) for k in ex["keys"]] == sorted(int(k) for k in ref.m)
        assert [int(c) for c in ex["counts"]] == [ref.m[k][1] for k in sorted(ref.m)]
        assert [bool(r_ >= 0) for r_ in ex["rows"]] == [ref.m[k][0] for k in sorted(ref.m)]


@pytest.mark.parametrize("cap", [0, 15, 40, 10**6])
def test_evict_lru_against_brute_force(cap):
    """LRU-bounded passes (at most `cap` keys kept, youngest lookups first)
    mixed with admission at 2 and a FIND_ONLY lookup, against the dict."""
    spec = TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum", admit_threshold=2)
    tab, ref = oracle.OracleTable(spec), DictTable(2)
    for step in range(16):
        feats = small_features(500 + step, nfeat=2, batch=7, id_space=40)
        find_only = step % 7 == 6
        r = tab.insert_find(feats, 7, flags=oracle.FIND_ONLY if find_only else 0)
        assert r.status == 0
        want = ref.step(keys_of(feats), find_only)
        got = {int(k): int(row) >= 0 for k, row in zip(r.unique_keys[:r.U], r.unique_rows[:r.U])}
        assert got == {int(k): v for k, v in want.items()}
        if step % 3 == 1:
            n = tab.evict_lru(cap)
            assert n == ref.evict_lru(cap)
            assert tab.size() <= cap
        ex = tab.export()
        assert [int(k) for k in ex["keys"]] == sorted(int(k) for k in ref.m)
        assert [int(c) for c in ex["counts"]] == [ref.m[k][1] for k in sorted(ref.m)]
        assert [bool(r_ >= 0) for r_ in ex["rows"]] == [ref.m[k][0] for k in sorted(ref.m)]


def test_evict_lru_keeps_exactly_the_latest_lookup():
    """A bound equal to the latest lookup's distinct keys keeps exactly those."""
    spec = TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum")
    tab = oracle.OracleTable(spec)
    for step in range(4):
        feats = small_features(600 + step, nfeat=1, batch=7, id_space=50)
        assert tab.insert_find(feats, 7).status == 0
    last = np.unique(keys_of(feats))
    n_before = tab.size()
    assert tab.evict_lru(last.size) == n_before - last.size
    np.testing.assert_array_equal(tab.export()["keys"], last)


def _fmix64(x):
    """MurmurHash3's 64-bit finalizer, restated in Python."""
    m = (1 << 64) - 1
    x ^= x >> 33
    x = (x * 0xFF51AFD7ED558CCD) & m
    x ^= x >> 33
    x = (x * 0xC4CEB9FE1A85EC53) & m
    x ^= x >> 33
    return x


class SketchDict:
    """Brute force of count-min sketch admission: a dict of admitted keys
    (key -> [has_row, count]) and a list-of-lists sketch for the rest."""

    def __init__(self, admit, bits):
        self.m, self.admit, self.bits = {}, admit, bits
        self.sk = [[0] * (1 << bits) for _ in range(4)]

    def idx(self, key, r):
        salt = (0x9E3779B97F4A7C15 * (2 * r + 1)) & ((1 << 64) - 1)
        return _fmix64((int(key) & ((1 << 64) - 1)) ^ salt) >> (64 - self.bits)

    def step(self, keys):
        u, c = np.unique(keys, return_counts=True)
        for k, n in zip(u, c):       # all adds first
            if k not in self.m:
                for r in range(4):
                    i = self.idx(k, r)
                    self.sk[r][i] = (self.sk[r][i] + int(n)) & 0xFFFFFFFF
        out = {}
        for k, n in zip(u, c):
            if k in self.m:
                e = self.m[k]
                e[1] += int(n)
            else:
                est = min(self.sk[r][self.idx(k, r)] for r in range(4))
                if est < self.admit:
                    out[k] = False
                    continue
                e = self.m[k] = [False, est]
            if not e[0] and e[1] >= self.admit:
                e[0] = True
            out[k] = e[0]
        return out

    def evict(self, t):
        gone = [k for k, e in self.m.items() if e[1] < t]
        for k in gone:
            del self.m[k]
        for e in self.m.values():
            e[1] = 0
        self.sk = [[0] * (1 << self.bits) for _ in range(4)]
        return len(gone)


@pytest.mark.parametrize("bits", [1, 4, 12])
def test_sketch_admission_against_brute_force(bits):
    """Count-min sketch admission at 3, with an eviction pass every fourth
    step: per-step admissions, the admitted keys and their counts."""
    spec = TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum", admit_threshold=3)
    tab, ref = oracle.OracleTable(spec), SketchDict(3, bits)
    tab.set_sketch(bits)
    for step in range(12):
        feats = small_features(700 + step, nfeat=2, batch=9, id_space=60)
        r = tab.insert_find(feats, 9)
        assert r.status == 0
        want = ref.step(keys_of(feats))
        got = {int(k): int(row) >= 0 for k, row in zip(r.unique_keys[:r.U], r.unique_rows[:r.U])}
        assert got == {int(k): v for k, v in want.items()}
        if step % 4 == 3:
            assert tab.evict(2) == ref.evict(2)
        ex = tab.export()
        assert [int(k) for k in ex["keys"]] == sorted(int(k) for k in ref.m)
        assert [int(c) for c in ex["counts"]] == [ref.m[k][1] for k in sorted(ref.m)]


def test_sketch_without_collisions_admits_as_the_exact_counts():
    """With a sketch far larger than the keys (no shared counters), a key is
    admitted in the same step as with exact counts, with the same count; the
    keys still waiting simply stay out of the map."""
    spec = TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum", admit_threshold=3)
    exact, sk = oracle.OracleTable(spec), oracle.OracleTable(spec)
    sk.set_sketch(20)
    for step in range(10):
        feats = small_features(800 + step, nfeat=2, batch=9, id_space=60)
        a, b = exact.insert_find(feats, 9), sk.insert_find(feats, 9)
        np.testing.assert_array_equal(a.unique_rows[:a.U] >= 0, b.unique_rows[:b.U] >= 0)
        ea, eb = exact.export(), sk.export()
        has = ea["rows"] >= 0
        np.testing.assert_array_equal(eb["keys"], ea["keys"][has])
        np.testing.assert_array_equal(eb["counts"], ea["counts"][has])


def test_sketch_never_admits_later_than_exact_counts():
    """A count-min estimate never falls below the true count: with a tiny
    sketch (many collisions) every key the exact counts admit is admitted."""
    spec = TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum", admit_threshold=4)
    exact, sk = oracle.OracleTable(spec), oracle.OracleTable(spec)
    sk.set_sketch(2)
    for step in range(10):
        feats = small_features(900 + step, nfeat=2, batch=9, id_space=80)
        a, b = exact.insert_find(feats, 9), sk.insert_find(feats, 9)
        assert np.all((a.unique_rows[:a.U] >= 0) <= (b.unique_rows[:b.U] >= 0))


def test_evict_decay_one_keeps_running_totals():
    """decay = 1 and no key evicted: every count is the key's total number of
    occurrences since it was first seen (np.unique over all inputs)."""
    spec = TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum")
    tab = oracle.OracleTable(spec)
    seen = []
    for step in range(6):
        feats = small_features(400 + step, nfeat=2, batch=9, id_space=30)
        assert tab.insert_find(feats, 9).status == 0
        seen.append(keys_of(feats))
        assert tab.evict(1, 1.0) == 0
    keys, counts = np.unique(np.concatenate(seen), return_counts=True)
    ex = tab.export()
    np.testing.assert_array_equal(ex["keys"], keys)
    np.testing.assert_array_equal(ex["counts"], counts)


# --------------------------------------------------------------------- evict
def test_evict_frees_and_reuses_rows():
    spec = TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum")
    tab = oracle.OracleTable(spec)
    f = [FeatureInput(values=np.array([1, 1, 2, 3, 3, 3], np.int64), bag_offsets=np.array([0, 6], np.int32), slot=0)]
    tab.insert_find(f, 1)
    assert tab.rows_in_use() == 3
    assert tab.evict(2) == 1             # key 2 seen once
    assert tab.rows_in_use() == 2
    ex = tab.export()
    assert list(ex["keys"]) == [1, 3] and list(ex["counts"]) == [0, 0]
    f = [FeatureInput(values=np.array([7], np.int64), bag_offsets=np.array([0, 1], np.int32), slot=0)]
    tab.insert_find(f, 1)
    assert tab.rows_in_use() == 3
    ex = tab.export()
    np.testing.assert_array_equal(ex["params"][-1], oracle.init_row(spec.seed, 7, 4))


# ----------------------------------------------------------------- writeback
def test_writeback_is_eta1_sgd_and_last_writer_wins():
    spec = TableSpec(dim=8, dtype="f32", optim="none", pool="none")
    tab = oracle.OracleTable(spec)
    keys = np.array([5, 9, 5, 2, 9, 9], np.int64)
    e = rng_for(9).standard_normal((6, 8), dtype=np.float32)
    assert tab.writeback(keys[:2], e[:2]) == 0          # unique keys: the SGD identity
    M = torch.tensor(np.stack([oracle.init_row(spec.seed, k, 8) for k in (5, 9)]), dtype=torch.float64,
                     requires_grad=True)
    opt = torch.optim.SGD([M], lr=1.0)
    (0.5 * ((M - torch.from_numpy(e[:2].astype(np.float64))) ** 2).sum()).backward()
    opt.step()
    ex = tab.export()
    np.testing.assert_array_equal(ex["params"], M.detach().float().numpy())
    assert tab.writeback(keys, e) == 0
    last = {}
    for i, k in enumerate(keys):
        last[int(k)] = e[i]
    ex = tab.export()
    for i, k in enumerate(ex["keys"]):
        np.testing.assert_array_equal(ex["params"][i], last[int(k)])


def test_writeback_bf16_is_rne():
    spec = TableSpec(dim=16, dtype="bf16", optim="none", pool="none")
    tab = oracle.OracleTable(spec)
    keys = np.arange(50, dtype=np.int64) * 7
    e = rng_for(10).standard_normal((50, 16), dtype=np.float32)
    tab.writeback(keys, e)
    ex = tab.export()
    want = torch.from_numpy(e).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ex["params"], want)


# ------------------------------------------------- merged tables are separate
def test_merged_table_equals_separate_tables():
    spec = TableSpec(dim=8, dtype="f32", optim="adam", pool="mean", lr=1e-3, eps=1e-8)
    merged = oracle.OracleTable(spec)
    parts = [oracle.OracleTable(spec) for _ in range(3)]
    for step in range(3):
        feats = small_features(300 + step, nfeat=3, batch=11, id_space=12)
        g = rng_for(12, step).standard_normal((11, 24), dtype=np.float32)
        r = merged.insert_find(feats, 11)
        out = merged.forward(r, "mean")
        merged.backward_update(r, "mean", g)
        for f, t in enumerate(parts):
            rf = t.insert_find([feats[f]], 11)
            np.testing.assert_array_equal(t.forward(rf, "mean"), out[:, f * 8:(f + 1) * 8])
            t.backward_update(rf, "mean", np.ascontiguousarray(g[:, f * 8:(f + 1) * 8]))
    em = merged.export()
    es = [t.export() for t in parts]
    np.testing.assert_array_equal(em["keys"], np.concatenate([e["keys"] for e in es]))
    np.testing.assert_array_equal(em["params"], np.concatenate([e["params"] for e in es]))
    np.testing.assert_array_equal(em["state"], np.concatenate([e["state"] for e in es]))


def test_bucketize_feature_in_a_table():
    rng = rng_for(13)
    f0 = bucketize_feature(rng, 20, 9, slot=2)
    tab = oracle.OracleTable(TableSpec(dim=4, dtype="f32", optim="adagrad", pool="sum"))
    r = tab.insert_find([f0], 20)
    assert r.status == 0
    want = np.unique((2 << 48) | np.searchsorted(f0.boundaries, f0.values, side="right"))
    np.testing.assert_array_equal(r.unique_keys[:r.U], want)


def test_tiny_workload_runs():
    spec = TableSpec(dim=16, dtype="f32", optim="adagrad", pool="sum")
    tab = oracle.OracleTable(spec)
    for step in range(3):
        b = tiny_batch(step)
        r = tab.insert_find(b.features, b.batch)
        assert r.status == 0
        tab.forward(r, "sum")
        assert tab.backward_update(r, "sum", b.grad) == 0
