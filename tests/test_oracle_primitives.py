"""Pins of the oracle's per-value primitives against things other than itself.

Hash    -> MurmurHash3_x64_128 as shipped (source form) with scikit-learn;
Mod     -> numpy unsigned / floor remainder;
Bucketize -> numpy.searchsorted(side='right');
Philox  -> rocRAND's host-callable philox4x32_10 engine (header-only, run on CPU);
init    -> Kolmogorov-Smirnov against U(-b, b) plus exact range/grid properties;
bf16    -> torch's fp32 -> bf16 conversion on fp32-exact inputs, and exact
           rational brute force for doubles between bf16 neighbours.
No GPU is used.
"""
import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import OP_BUCKETIZE, OP_HASH, OP_MOD

MASK64 = (1 << 64) - 1


# --------------------------------------------------------------------- hash
def _sklearn_murmur_src():
    try:
        import sklearn
    except ImportError:
        return None
    p = os.path.join(os.path.dirname(sklearn.__file__), "utils", "src", "MurmurHash3.cpp")
    return p if os.path.exists(p) else None


@pytest.fixture(scope="module")
def murmur_x64_128(tmp_path_factory):
    src = _sklearn_murmur_src()
    if src is None:
        pytest.skip("scikit-learn's MurmurHash3 source is not installed")
    d = tmp_path_factory.mktemp("murmur")
    so = str(d / "libmm3.so")
    subprocess.check_call(["g++", "-O1", "-shared", "-fPIC", "-I", os.path.dirname(src), src, "-o", so])
    L = ctypes.CDLL(so)
    L.MurmurHash3_x64_128.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p]

    def h(data: bytes, seed: int):
        out = (ctypes.c_uint64 * 2)()
        buf = ctypes.create_string_buffer(data, max(len(data), 1))
        L.MurmurHash3_x64_128(buf, len(data), seed, out)
        return int(out[0]), int(out[1])
    return h


def test_fmix64_pinned_by_murmur3_x64_128(murmur_x64_128):
    # With an empty input and seed s, MurmurHash3_x64_128 finalises
    # h1 = fmix64(2s), h2 = fmix64(3s) and outputs (h1 + h2, h1 + 2 h2), so
    # fmix64(2s) = 2*out1 - out2 and fmix64(3s) = out2 - out1 (mod 2^64).
    rng = np.random.default_rng(1)
    seeds = [0, 1, 2, 3, 0x7FFFFFFF, 0xFFFFFFFF] + [int(s) for s in rng.integers(0, 2**32, 200)]
    xs, want = [], []
    for s in seeds:
        o1, o2 = murmur_x64_128(b"", s)
        xs += [2 * s, 3 * s]
        want += [(2 * o1 - o2) & MASK64, (o2 - o1) & MASK64]
    got = oracle.fmix64(np.array(xs, dtype=np.uint64))
    assert [int(v) for v in got] == want


def test_fmix64_special_cases_and_bijection():
    assert int(oracle.fmix64(np.array([0], np.uint64))[0]) == 0
    rng = np.random.default_rng(2)
    x = np.unique(rng.integers(0, 2**63, 200_000, dtype=np.int64).astype(np.uint64))
    y = oracle.fmix64(x)
    assert np.unique(y).size == x.size  # a bijection cannot collide


# ---------------------------------------------------------------- mod / tag
def test_hash_mod_tag_against_numpy():
    rng = np.random.default_rng(3)
    v = rng.integers(-2**63, 2**63 - 1, 5000, dtype=np.int64)
    for mod in (100_000_000, 1, 7, (1 << 48)):
        st, keys = oracle.transform(v, OP_HASH | OP_MOD, mod, slot=25)
        assert st == 0
        h = oracle.fmix64(v.view(np.uint64))
        want = (np.uint64(25) << np.uint64(48)) | (h % np.uint64(mod))
        np.testing.assert_array_equal(keys.view(np.uint64), want)


def test_raw_mod_is_floor_remainder():
    v = np.array([-7, -1, 0, 1, 6, 7, 8, -2**63, 2**63 - 1], dtype=np.int64)
    st, keys = oracle.transform(v, OP_MOD, 7, slot=3)
    assert st == 0
    np.testing.assert_array_equal(keys, (3 << 48) | np.mod(v, 7))


def test_bucketize_against_searchsorted():
    rng = np.random.default_rng(4)
    b = np.unique(rng.integers(-500, 500, 40, dtype=np.int64))
    v = np.concatenate([rng.integers(-600, 600, 3000, dtype=np.int64), b, b - 1, b + 1])
    st, keys = oracle.transform(v, OP_BUCKETIZE, boundaries=b, slot=1)
    assert st == 0
    np.testing.assert_array_equal(keys, (1 << 48) | np.searchsorted(b, v, side="right"))
    st, keys = oracle.transform(v, OP_BUCKETIZE, boundaries=np.zeros(0, np.int64))
    assert st == 0 and np.all(keys == 0)


def test_transform_errors():
    assert oracle.transform(np.array([1 << 48]))[0] == 4            # id past the 48-bit field
    assert oracle.transform(np.array([-1]))[0] == 4                 # raw negative id
    assert oracle.transform(np.array([5]), slot=1 << 15)[0] == 4    # slot past 15 bits
    assert oracle.transform(np.array([5]), OP_HASH)[0] == 4         # 64-bit hash, no Mod
    assert oracle.transform(np.array([5]), OP_MOD, 0)[0] == 1       # Mod 0
    assert oracle.transform(np.array([5]), OP_BUCKETIZE, boundaries=np.array([3, 3]))[0] == 1
    assert oracle.transform(np.array([5]), OP_BUCKETIZE | OP_HASH, boundaries=np.array([3]))[0] == 1
    assert oracle.transform(np.array([(1 << 48) - 1]))[0] == 0


# ------------------------------------------------------------------- philox
@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    inc = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if not os.path.exists(inc) or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("rocRAND headers / hipcc not present")
    d = tmp_path_factory.mktemp("philox")
    src = d / "ph.cpp"
    # Reads (seed, subsequence, offset) triples on stdin and prints the first four
    # outputs of rocRAND's engine; subsequence s and offset 4g place the counter at
    # (g, 0, s_lo, s_hi) and the key at (seed_lo, seed_hi).
    src.write_text(
        "#include <rocrand/rocrand_philox4x32_10.h>\n#include <cstdio>\n"
        "int main(){unsigned long long a,b,c;\n"
        " while(scanf(\"%llu %llu %llu\",&a,&b,&c)==3){\n"
        "  rocrand_device::philox4x32_10_engine e(a,b,c);\n"
        "  unsigned x0=e(),x1=e(),x2=e(),x3=e(); printf(\"%u %u %u %u\\n\",x0,x1,x2,x3);}}\n")
    exe = str(d / "ph")
    subprocess.check_call(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "--cuda-host-only", "-O1",
                           str(src), "-o", exe])

    def run(triples):
        inp = "".join(f"{a} {b} {c}\n" for a, b, c in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [tuple(int(t) for t in line.split()) for line in out.strip().splitlines()]
    return run


def test_philox_against_rocrand(rocrand_philox):
    rng = np.random.default_rng(5)
    triples = [(0, 0, 0), (2**64 - 1, 2**64 - 1, 4 * (2**32 - 1))]
    for _ in range(300):
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        key = int(rng.integers(0, 2**63))
        g = int(rng.integers(0, 64))
        triples.append((seed, key, 4 * g))
    want = rocrand_philox(triples)
    for (seed, key, off), w in zip(triples, want):
        g = off // 4
        ctr = [g & 0xFFFFFFFF, 0, key & 0xFFFFFFFF, key >> 32]
        got = oracle.philox4x32_10(ctr, [seed & 0xFFFFFFFF, seed >> 32])
        assert tuple(int(x) for x in got) == w


def test_init_rows_are_uniform_on_the_bound():
    from scipy import stats
    vals = np.concatenate([oracle.init_row(20250925, k, 64) for k in range(4000)])
    assert vals.min() >= -0.05 and vals.max() < 0.05
    assert stats.kstest(vals, stats.uniform(loc=-0.05, scale=0.1).cdf).pvalue > 1e-3
    assert abs(vals.mean()) < 2e-3 and abs(vals.var() - 0.1**2 / 12) < 5e-5
    # the values sit on the 2^-24 grid of the interval, one rounding of an exact product
    grid = vals.astype(np.float64) / (0.05 * 2.0**-23)
    assert np.all(np.abs(grid - np.round(grid)) < 1e-3 * np.abs(grid).clip(1))


def test_init_rows_depend_on_seed_and_key_only():
    a = oracle.init_row(7, 123, 16)
    np.testing.assert_array_equal(a, oracle.init_row(7, 123, 16))
    np.testing.assert_array_equal(a[:8], oracle.init_row(7, 123, 8))   # prefix-stable in dim
    assert not np.array_equal(a, oracle.init_row(8, 123, 16))
    assert not np.array_equal(a, oracle.init_row(7, 124, 16))


# --------------------------------------------------------------------- bf16
def test_bf16_rounding_matches_torch_on_fp32_values():
    import torch
    rng = np.random.default_rng(6)
    x32 = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0**rng.integers(-6, 6, 20000),
                          np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 3e38, -3e38, 1e-40],
                                   dtype=np.float32)]).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.round_bf16(x32.astype(np.float64)), want)


def test_bf16_rounding_is_single_from_double():
    # x = midpoint of two bf16 neighbours +- 2^-30: an fp32 detour would land on the
    # midpoint and round to even; one rounding from the double must not.
    def nearest_bf16(v: Fraction):
        import math
        e = math.floor(math.log2(abs(v)))
        ulp = Fraction(2) ** (e - 7)
        lo = (v // ulp) * ulp
        hi = lo + ulp
        pick = lo if (v - lo) < (hi - v) else hi
        if v - lo == hi - v:
            pick = lo if (lo / ulp) % 2 == 0 else hi
        return float(pick)
    xs = []
    for base in (1.0, 1.5, 0.75, 3.0, 1.0 + 2**-7):
        mid = base + 2**-8 * (1 if base < 2 else 2)
        for d in (2.0**-30, -(2.0**-30), 0.0):
            xs.append(mid + d)
    got = oracle.round_bf16(np.array(xs))
    for x, g in zip(xs, got):
        want = np.float32(nearest_bf16(Fraction(x))).view(np.uint32) >> 16
        assert int(g) == int(want), x
