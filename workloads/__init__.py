"""Seeded synthetic inputs for the dynamic-embedding hot path.

This module only *draws inputs*: raw feature IDs, bag layouts, upstream
gradients and table settings.  It holds none of the method's arithmetic (no
ID hash, no dedup, no lookup, no pooling, no optimizer); both the HIP path and
the CPU oracle consume the arrays it returns, byte for byte.

Workload shapes follow the five configurations the RecIS engine is measured
on (one small table; a 26-feature CTR batch; a 1000-long behaviour
sequence; a 200M-row capacity stress; five merged tables with eviction plus
an item-cache writeback).  Where a law is not fixed by those descriptions the
plainest reading is taken and named in the function docstring.

Every array is a pure function of (config, step, feature) through
``numpy.random.SeedSequence``; nothing here depends on the GPU.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

# Transform bits of a feature: the values the C ABI header declares for
# RECIS_OP_HASH / RECIS_OP_MOD / RECIS_OP_BUCKETIZE.
OP_HASH = 1
OP_MOD = 2
OP_BUCKETIZE = 4

ID_SPACE_2_40 = 1 << 40


# --------------------------------------------------------------------------
# Plain containers
# --------------------------------------------------------------------------
@dataclass
class FeatureInput:
    """One sparse feature of a batch, in CSR form.

    values      int64 [n]     raw IDs (or raw numeric values for Bucketize)
    bag_offsets int32 [B + 1] sample i owns values[bag_offsets[i]:bag_offsets[i+1]]
    slot        feature tag placed in bits 48..62 of the table key
    ops         OP_* bitmask applied to each value before tagging
    mod         modulus for OP_MOD
    boundaries  strictly increasing int64 boundaries for OP_BUCKETIZE
    """
    values: np.ndarray
    bag_offsets: np.ndarray
    slot: int
    ops: int = 0
    mod: int = 0
    boundaries: Optional[np.ndarray] = None

    @property
    def n(self) -> int:
        return int(self.values.shape[0])


@dataclass
class TableSpec:
    """Attributes of one logical (merged) table and of the step run on it."""
    dim: int
    dtype: str            # "f32" | "bf16"  (parameter storage)
    optim: str            # "adagrad" | "adam" | "none"
    pool: str             # "sum" | "mean" | "none"
    lr: float = 0.01
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-10
    seed: int = 20250925
    init_bound: float = 0.05
    admit_threshold: int = 1
    grad_dtype: str = "f32"


@dataclass
class Batch:
    features: List[FeatureInput]
    batch: int
    grad: np.ndarray                  # float32: [B, F*D] pooled, [N, D] for pool "none" (None: not drawn)
    meta: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(sum(f.n for f in self.features))

    @property
    def num_feats(self) -> int:
        return len(self.features)


# --------------------------------------------------------------------------
# Random laws
# --------------------------------------------------------------------------
def rng_for(*words: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(w) for w in words]))


def zipf_truncated(rng: np.random.Generator, alpha: float, m: int, size: int) -> np.ndarray:
    """Ranks in 1..m with P(k) proportional to k**-alpha (numpy Zipf, rejection-truncated)."""
    out = np.empty(size, dtype=np.int64)
    filled = 0
    while filled < size:
        need = size - filled
        draw = rng.zipf(alpha, size=need + need // 3 + 16)
        draw = draw[draw <= m]
        take = min(need, draw.size)
        out[filled:filled + take] = draw[:take]
        filled += take
    return out


def poisson_bags(rng: np.random.Generator, batch: int, mean: float, min_len: int) -> np.ndarray:
    lens = rng.poisson(mean, size=batch).astype(np.int64)
    if min_len > 0:
        lens = np.maximum(lens, min_len)
    return lens


def offsets_from_lengths(lens: np.ndarray) -> np.ndarray:
    off = np.zeros(lens.shape[0] + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    assert off[-1] < 2**31
    return off.astype(np.int32)


# --------------------------------------------------------------------------
# Rank -> ID bijections (inputs only: they decide which raw ID a Zipf rank
# names, so that hot IDs are scattered over the ID space)
# --------------------------------------------------------------------------
_M1 = np.uint64(0x9E3779B97F4A7C15)
_M2 = np.uint64(0xD6E8FEB86659FD93)


def _feistel(x: np.ndarray, bits: int, key: int, rounds: int = 4) -> np.ndarray:
    half = bits // 2
    mask = np.uint64((1 << half) - 1)
    x = x.astype(np.uint64)
    left = x >> np.uint64(half)
    right = x & mask
    k = np.uint64(key & 0xFFFFFFFFFFFFFFFF)
    with np.errstate(over="ignore"):
        for r in range(rounds):
            t = (right + k + np.uint64(r)) * _M1
            t ^= t >> np.uint64(31)
            t *= _M2
            t ^= t >> np.uint64(29)
            left, right = right, left ^ (t & mask)
    return (left << np.uint64(half)) | right


def permute_2_40(x: np.ndarray, key: int) -> np.ndarray:
    """Bijection of [0, 2**40) (balanced 20/20-bit Feistel, 4 rounds)."""
    return _feistel(x, 40, key).astype(np.int64)


def permute_below(x: np.ndarray, m: int, key: int) -> np.ndarray:
    """Bijection of [0, m): a Feistel permutation of the enclosing even power of two,
    cycle-walked until the value falls below m."""
    bits = max(2, int(m - 1).bit_length())
    bits += bits & 1
    y = _feistel(x, bits, key)
    out = y.copy()
    bad = out >= np.uint64(m)
    while bad.any():
        out[bad] = _feistel(out[bad], bits, key)
        bad = out >= np.uint64(m)
    return out.astype(np.int64)


def feature_key(config: int, table: int, feature: int) -> int:
    ss = np.random.SeedSequence([7919, config, table, feature])
    return int(ss.generate_state(1, dtype=np.uint64)[0])


# --------------------------------------------------------------------------
# Table settings for the five workloads
# --------------------------------------------------------------------------
INIT_SEED = 20250925


def spec_tiny() -> TableSpec:
    return TableSpec(dim=16, dtype="f32", optim="adagrad", pool="sum", lr=0.01, eps=1e-10,
                     seed=INIT_SEED)


def spec_ctr() -> TableSpec:
    return TableSpec(dim=64, dtype="f32", optim="adam", pool="mean", lr=1e-3,
                     beta1=0.9, beta2=0.999, eps=1e-8, seed=INIT_SEED)


def spec_seq() -> TableSpec:
    return TableSpec(dim=128, dtype="bf16", optim="adagrad", pool="none", lr=0.01, eps=1e-10,
                     seed=INIT_SEED, grad_dtype="bf16")


def spec_capacity() -> TableSpec:
    return TableSpec(dim=64, dtype="f32", optim="adam", pool="sum", lr=1e-3,
                     beta1=0.9, beta2=0.999, eps=1e-8, seed=INIT_SEED)


MULTI_DIMS = (8, 16, 32, 64, 128)


def spec_multi(table: int) -> TableSpec:
    return TableSpec(dim=MULTI_DIMS[table], dtype="f32", optim="adagrad", pool="mean",
                     lr=0.01, eps=1e-10, seed=INIT_SEED + table, admit_threshold=2)


def spec_cache() -> TableSpec:
    return TableSpec(dim=256, dtype="bf16", optim="none", pool="none", seed=INIT_SEED + 5)


# --------------------------------------------------------------------------
# Batches
# --------------------------------------------------------------------------
def _grad(config: int, step: int, shape) -> np.ndarray:
    rng = rng_for(config, step, 1_000_000)
    return rng.standard_normal(size=shape, dtype=np.float32)


def tiny_batch(step: int, batch: int = 256, id_space: int = 100_000, dim: int = 16) -> Batch:
    """1 feature, bag length max(1, Poisson(4)), IDs uniform on [0, id_space)."""
    rng = rng_for(1, step, 0)
    lens = poisson_bags(rng, batch, 4.0, 1)
    off = offsets_from_lengths(lens)
    vals = rng.integers(0, id_space, size=int(off[-1]), dtype=np.int64)
    f = FeatureInput(values=vals, bag_offsets=off, slot=0)
    return Batch([f], batch, _grad(1, step, (batch, dim)))


def ctr_batch(step: int, batch: int = 8192, num_feats: int = 26, dim: int = 64,
              alpha: float = 1.05, max_len: int = 50, mod: int = 100_000_000, grad: bool = True) -> Batch:
    """26 features; bag length Zipf(alpha) truncated to 1..max_len (the ID law's
    exponent is reused for lengths); raw IDs Zipf(alpha) ranks over 2**40 mapped
    through a per-feature bijection; the features ask for Hash then Mod(mod)."""
    feats = []
    for f in range(num_feats):
        rng = rng_for(2, step, f)
        lens = zipf_truncated(rng, alpha, max_len, batch)
        off = offsets_from_lengths(lens)
        ranks = zipf_truncated(rng, alpha, ID_SPACE_2_40, int(off[-1]))
        vals = permute_2_40(ranks - 1, feature_key(2, 0, f))
        feats.append(FeatureInput(values=vals, bag_offsets=off, slot=f, ops=OP_HASH | OP_MOD, mod=mod))
    return Batch(feats, batch, _grad(2, step, (batch, num_feats * dim)) if grad else None)


def seq_batch(step: int, batch: int = 2048, seq_len: int = 1000, dim: int = 128,
              alpha: float = 1.2, items: int = 100_000_000, grad: bool = True) -> Batch:
    """1 feature of fixed-length sequences; IDs Zipf(alpha) over `items`, ranks
    mapped by a bijection of [0, items); upstream gradient N(0,1) per position."""
    rng = rng_for(3, step, 0)
    off = offsets_from_lengths(np.full(batch, seq_len, dtype=np.int64))
    ranks = zipf_truncated(rng, alpha, items, batch * seq_len)
    vals = permute_below(ranks - 1, items, feature_key(3, 0, 0))
    f = FeatureInput(values=vals, bag_offsets=off, slot=0)
    return Batch([f], batch, _grad(3, step, (batch * seq_len, dim)) if grad else None)


def capacity_resident_keys(num_feats: int = 100, per_feature: int = 2_000_000):
    """Raw IDs pre-populated before the capacity-stress run: the top `per_feature`
    ranks of every feature (feature f's IDs go to slot f)."""
    for f in range(num_feats):
        ranks = np.arange(per_feature, dtype=np.int64)
        yield f, permute_2_40(ranks, feature_key(4, 0, f))


def capacity_batch(step: int, batch: int = 65536, num_feats: int = 100, dim: int = 64,
                   alpha: float = 1.2, resident_per_feature: int = 2_000_000,
                   novel_frac: float = 0.02, grad: bool = True) -> Batch:
    """Bag length Poisson(8) (empty bags allowed); each occurrence is, with
    probability novel_frac, a never-used ID, else a Zipf(alpha) rank truncated to
    the resident ranks; ranks map to IDs through a per-feature bijection of 2**40."""
    feats = []
    for f in range(num_feats):
        rng = rng_for(4, step, f)
        lens = rng.poisson(8.0, size=batch).astype(np.int64)
        off = offsets_from_lengths(lens)
        n = int(off[-1])
        ranks = zipf_truncated(rng, alpha, resident_per_feature, n) - 1
        novel = rng.random(n) < novel_frac
        k = int(novel.sum())
        # never-used ranks: a disjoint range per step above the resident ranks
        ranks[novel] = resident_per_feature + step * (1 << 26) + np.arange(k, dtype=np.int64)
        vals = permute_2_40(ranks, feature_key(4, 0, f))
        feats.append(FeatureInput(values=vals, bag_offsets=off, slot=f))
    return Batch(feats, batch, _grad(4, step, (batch, num_feats * dim)) if grad else None)


def multi_batch(step: int, table: int, batch: int = 32768, num_feats: int = 60,
                alpha: float = 1.1, grad: bool = True) -> Batch:
    """One of the five merged tables: bag length max(1, Poisson(4)); IDs Zipf(alpha)
    over 2**40 through a per-(table, feature) bijection; slot = feature index."""
    dim = MULTI_DIMS[table]
    feats = []
    for f in range(num_feats):
        rng = rng_for(5, step, table * 1000 + f)
        lens = poisson_bags(rng, batch, 4.0, 1)
        off = offsets_from_lengths(lens)
        ranks = zipf_truncated(rng, alpha, ID_SPACE_2_40, int(off[-1]))
        vals = permute_2_40(ranks - 1, feature_key(5, table, f))
        feats.append(FeatureInput(values=vals, bag_offsets=off, slot=f))
    return Batch(feats, batch, _grad(5, step * 8 + table, (batch, num_feats * dim)) if grad else None)


def cache_keys(num_keys: int = 10_000_000) -> np.ndarray:
    """Distinct item keys of the in-model cache, spread over [0, 2**40)."""
    return permute_2_40(np.arange(num_keys, dtype=np.int64), feature_key(5, 5, 0))


def cache_writes(step: int, keys: np.ndarray, n: int = 16384, dim: int = 256):
    """One step's writeback batch: n keys drawn uniformly with replacement from
    the cache's keys, and item-tower rows e ~ N(0, 1) in fp32."""
    rng = rng_for(5, step, 9999)
    pick = rng.integers(0, keys.shape[0], size=n)
    rows = rng.standard_normal(size=(n, dim), dtype=np.float32)
    return keys[pick].copy(), rows


def bucketize_feature(rng: np.random.Generator, batch: int, nb: int, mean_len: float = 3.0,
                      slot: int = 0) -> FeatureInput:
    """Numeric feature for Bucketize: values near/at the boundaries to exercise ties."""
    lens = poisson_bags(rng, batch, mean_len, 0)
    off = offsets_from_lengths(lens)
    n = int(off[-1])
    bounds = np.unique(rng.integers(-1000, 1000, size=nb * 2, dtype=np.int64))[:nb]
    vals = rng.integers(-1200, 1200, size=n, dtype=np.int64)
    if n and bounds.size:
        hit = rng.random(n) < 0.3
        vals[hit] = bounds[rng.integers(0, bounds.size, size=int(hit.sum()))]
    return FeatureInput(values=vals, bag_offsets=off, slot=slot, ops=OP_BUCKETIZE, boundaries=bounds)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 inputs to bf16 (RNE) and return the raw uint16 patterns; used to
    hand bf16 upstream gradients to both sides."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)
