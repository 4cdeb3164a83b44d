// oracle.cpp -- TEST INFRASTRUCTURE ONLY.
//
// A plain, sequential CPU statement of what the dynamic-embedding hot path
// computes.  Only the test suite, the smoke check and the benchmark's CPU
// baseline leg may load it; the product path never does.  It shares no code
// with the HIP library: it has its own hash, counter-based RNG, rounding,
// map and loops, and it does every sum in double precision.
//
// Pages followed (title, then section):
//   [README] "RecIS (Recommendation Intelligence System)" README mirror of
//            alibaba/RecIS v1.1.0:
//              Core architecture > Feature Engine (Hash / Mod / Bucketize),
//              Core architecture > Embedding Engine (collision-free KV table,
//                merged tables, eviction and admission),
//              Key optimisations > Efficient dynamic Embedding (IDMap of
//                ID -> Offset; EmbeddingBlocks holding parameters and
//                optimizer state),
//              Key optimisations > Distributed optimisation > request merge
//                and dedup,
//              Key optimisations > Operator implementation (reductions).
//   [ML]     "Memory Layer: Train the In-Model Cache for Recommendation
//            Models" (Pith review): What carries the argument; Referee
//            Report > Summary (Writeback = exact assignment, done as an
//            eta = 1 SGD step); Assumptions (EXACT_SGD, eta = 1).
//
// Where the pages leave a step open, the reading taken is stated at the
// function.  Nothing here is tuned for speed.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <unordered_map>
#include <vector>

namespace {

enum : int { ST_OK = 0, ST_INVALID = 1, ST_CAPACITY = 3, ST_KEY_RANGE = 4, ST_UNSUPPORTED = 6 };
enum : uint32_t { OP_HASH = 1, OP_MOD = 2, OP_BUCKETIZE = 4 };
enum : int { DT_F32 = 0, DT_BF16 = 1 };
enum : int { OPT_NONE = 0, OPT_ADAGRAD = 1, OPT_ADAM = 2 };
enum : int { POOL_SUM = 0, POOL_MEAN = 1, POOL_NONE = 2 };
enum : uint32_t { FLAG_FIND_ONLY = 1 };

const int64_t kIdLimit = int64_t(1) << 48;   // raw ID must fit below the feature tag
const uint32_t kSlotLimit = 1u << 15;        // keys stay non-negative int64

// ---------------------------------------------------------------------------
// Hash.  [README] Feature Engine names a Hash transform without saying which;
// the workload calls it murmur64.  Reading: the 64-bit finalizer of
// MurmurHash3 (Appleby), applied to the ID's two's-complement bit pattern.
// It is a bijection of uint64, so it adds no collision before Mod.
// ---------------------------------------------------------------------------
uint64_t murmur3_fmix64(uint64_t h) {
  h ^= h >> 33;
  h *= 0xff51afd7ed558ccdULL;
  h ^= h >> 33;
  h *= 0xc4ceb9fe1a85ec53ULL;
  h ^= h >> 33;
  return h;
}

// Transform one raw value and tag it with its feature slot.
// [README] Feature Engine: Hash / Mod / Bucketize.  [README] Embedding Engine
// and Distributed optimisation: same-attribute tables are merged into one
// logical table.  Readings: Hash then Mod in that order; Mod after Hash is an
// unsigned remainder, Mod on a raw signed value is a floor remainder in
// [0, m); Bucketize returns how many boundaries are <= x and excludes Hash;
// the merged key is (slot << 48) | id so equal IDs of different features stay
// different rows.
int transform_key(int64_t value, uint32_t ops, uint64_t mod, const int64_t* bounds, int64_t nb,
                  uint32_t slot, int64_t* key) {
  int64_t id;
  if (ops & OP_BUCKETIZE) {
    int64_t c = 0;
    for (int64_t i = 0; i < nb; ++i)
      if (bounds[i] <= value) c = i + 1;
    id = c;
  } else if (ops & OP_HASH) {
    uint64_t h = murmur3_fmix64(static_cast<uint64_t>(value));
    if (ops & OP_MOD) h = h % mod;
    if (h >= static_cast<uint64_t>(kIdLimit)) return ST_KEY_RANGE;
    id = static_cast<int64_t>(h);
  } else if (ops & OP_MOD) {
    int64_t m = static_cast<int64_t>(mod);
    int64_t r = value % m;
    if (r < 0) r += m;
    id = r;
  } else {
    id = value;
  }
  if (id < 0 || id >= kIdLimit || slot >= kSlotLimit) return ST_KEY_RANGE;
  *key = (static_cast<int64_t>(slot) << 48) | id;
  return ST_OK;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies with the
// Weyl-sequence key schedule.
// ---------------------------------------------------------------------------
void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint64_t p0 = uint64_t(0xD2511F53u) * c[0];
    uint64_t p1 = uint64_t(0xCD9E8D57u) * c[2];
    uint32_t hi0 = uint32_t(p0 >> 32), lo0 = uint32_t(p0);
    uint32_t hi1 = uint32_t(p1 >> 32), lo1 = uint32_t(p1);
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
  for (int i = 0; i < 4; ++i) out[i] = c[i];
}

// Initial value of element e of the row of `key`.  [README] tables have an
// "initializer" attribute; the rows must not depend on the offset they land
// at, so the value is a pure function of (seed, key, e).  Reading: Philox
// block g = e / 4 with counter (g, 0, key_lo, key_hi) and key (seed_lo,
// seed_hi); word w = e % 4 gives k = w >> 8 (24 bits) and the value
// fl32((k - 2^23) * fl32(bound) * 2^-23), which is uniform on [-bound, bound)
// and rounded once.
float init_value(uint64_t seed, int64_t key, int e, float bound) {
  uint32_t ctr[4] = {uint32_t(e / 4), 0u, uint32_t(uint64_t(key)), uint32_t(uint64_t(key) >> 32)};
  uint32_t k[2] = {uint32_t(seed), uint32_t(seed >> 32)};
  uint32_t w[4];
  philox4x32_10(ctr, k, w);
  int64_t centred = int64_t(w[e % 4] >> 8) - (int64_t(1) << 23);
  double scale = std::ldexp(double(bound), -23);      // exact
  return static_cast<float>(double(centred) * scale);  // exact product, one rounding
}

// Round a double once to the nearest bfloat16 (ties to even) and return the
// value as a float (every bfloat16 is a float).
float round_to_bf16(double x) {
  if (std::isnan(x)) return std::numeric_limits<float>::quiet_NaN();
  if (x == 0.0 || std::isinf(x)) return static_cast<float>(x);
  int e = std::ilogb(x);
  if (e < -126) e = -126;                          // bfloat16 subnormals share fp32's range
  double scaled = std::ldexp(x, 7 - e);            // 8 significant bits left of the point
  double r = std::nearbyint(scaled);               // default mode: nearest, ties to even
  double y = std::ldexp(r, e - 7);
  const double bf16_max = std::ldexp(255.0, 120);  // (2 - 2^-7) * 2^127
  if (std::fabs(y) > bf16_max) return x > 0 ? INFINITY : -INFINITY;
  return static_cast<float>(y);
}

uint16_t bf16_bits(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  return uint16_t(u >> 16);
}

float bf16_value(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float v;
  std::memcpy(&v, &u, 4);
  return v;
}

// ---------------------------------------------------------------------------
// The table.  [README] Efficient dynamic Embedding: level one maps a feature
// ID to an Offset; level two holds, per offset, the parameters and the
// optimizer state.  Here: std::unordered_map key -> {row, count} and plain
// vectors indexed by row.  A key may sit in the map without a row while it
// waits for admission ([README] Embedding Engine: eviction and admission).
// ---------------------------------------------------------------------------
struct Entry {
  int64_t row;        // -1: no row (not yet admitted, or refused for capacity)
  uint32_t count;     // occurrences since the last eviction pass
  uint32_t last_use;  // the counting lookup that last saw the key (Table::step)
};

struct Table {
  int dim, dtype, optim;
  uint64_t seed;
  float bound;
  int64_t max_rows, max_keys;
  uint32_t admit;
  int slots_per_elem;               // optimizer state words per element
  std::unordered_map<int64_t, Entry> idmap;
  std::vector<float> params;        // [rows * dim], each value exact in the storage dtype
  std::vector<float> state;         // [rows * slots_per_elem * dim]
  std::vector<int64_t> free_rows;   // rows released by eviction, reused last-in first-out
  int64_t next_row = 0;
  int64_t adam_step = 0;
  uint32_t step = 0;                // counting lookups so far (insert_find without FIND_ONLY)
  // count-min sketch admission (sketch_bits > 0): kSketchRows rows of
  // 2^sketch_bits counters for the keys not yet in the map
  int sketch_bits = 0;
  std::vector<uint32_t> sketch;
};

// The sketch's counter of `key` in row r: the top sketch_bits bits of
// MurmurHash3's finalizer of the key xor a per-row salt (odd multiples of
// the 64-bit golden ratio).  Counters are 32-bit and wrap.
constexpr int kSketchRows = 4;
size_t sketch_index(const Table& t, int64_t key, int r) {
  const uint64_t salt = 0x9E3779B97F4A7C15ull * uint64_t(2 * r + 1);
  const uint64_t h = murmur3_fmix64(uint64_t(key) ^ salt);
  return size_t(r) * (size_t(1) << t.sketch_bits) + size_t(h >> (64 - t.sketch_bits));
}

float store_param(const Table& t, double v) {
  return t.dtype == DT_BF16 ? round_to_bf16(v) : static_cast<float>(v);
}

// Give `key` a fresh row: parameters from the initializer, optimizer state 0.
int64_t allocate_row(Table& t, int64_t key) {
  int64_t row;
  if (!t.free_rows.empty()) {
    row = t.free_rows.back();
    t.free_rows.pop_back();
  } else {
    if (t.next_row >= t.max_rows) return -1;
    row = t.next_row++;
    t.params.resize(size_t(t.next_row) * t.dim);
    t.state.resize(size_t(t.next_row) * t.slots_per_elem * t.dim);
  }
  for (int e = 0; e < t.dim; ++e)
    t.params[size_t(row) * t.dim + e] = store_param(t, init_value(t.seed, key, e, t.bound));
  for (int s = 0; s < t.slots_per_elem * t.dim; ++s)
    t.state[size_t(row) * t.slots_per_elem * t.dim + s] = 0.0f;
  return row;
}

}  // namespace

extern "C" {

uint64_t orc_fmix64(uint64_t x) { return murmur3_fmix64(x); }

void orc_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
  philox4x32_10(ctr, key, out);
}

void orc_init_row(uint64_t seed, int64_t key, int dim, float bound, float* out) {
  for (int e = 0; e < dim; ++e) out[e] = init_value(seed, key, e, bound);
}

// Round each double to bfloat16 once; writes the bit patterns.
void orc_round_bf16(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits(round_to_bf16(x[i]));
}

// Transform + tag of n values of one feature (the per-occurrence step).
int orc_transform(const int64_t* values, int64_t n, uint32_t ops, uint64_t mod,
                  const int64_t* bounds, int64_t nb, uint32_t slot, int64_t* keys) {
  if ((ops & OP_MOD) && mod == 0) return ST_INVALID;
  if ((ops & OP_MOD) && !(ops & OP_HASH) && mod > uint64_t(INT64_MAX)) return ST_INVALID;
  if ((ops & OP_BUCKETIZE) && (ops & (OP_HASH | OP_MOD))) return ST_INVALID;
  for (int64_t i = 1; i < nb; ++i)
    if (!(bounds[i - 1] < bounds[i])) return ST_INVALID;
  for (int64_t i = 0; i < n; ++i) {
    int st = transform_key(values[i], ops, mod, bounds, nb, slot, &keys[i]);
    if (st != ST_OK) return st;
  }
  return ST_OK;
}

void* orc_create(int dim, int dtype, int optim, uint64_t seed, float bound, int64_t max_rows,
                 int64_t max_keys, uint32_t admit_threshold) {
  if (dim <= 0 || (dtype != DT_F32 && dtype != DT_BF16) || optim < OPT_NONE || optim > OPT_ADAM)
    return nullptr;
  Table* t = new Table();
  t->dim = dim;
  t->dtype = dtype;
  t->optim = optim;
  t->seed = seed;
  t->bound = bound;
  t->max_rows = max_rows;
  t->max_keys = max_keys;
  t->admit = admit_threshold == 0 ? 1 : admit_threshold;
  t->slots_per_elem = optim == OPT_ADAM ? 2 : (optim == OPT_ADAGRAD ? 1 : 0);
  return t;
}

void orc_destroy(void* h) { delete static_cast<Table*>(h); }

// Count-min sketch admission ([README] Embedding Engine: admission
// strategies).  Reading: with bits > 0, a key not in the map is counted in a
// sketch of kSketchRows x 2^bits counters and enters the map only when its
// estimate reaches admit_threshold; eviction passes clear the sketch.
int orc_set_sketch(void* h, int bits) {
  Table& t = *static_cast<Table*>(h);
  if (bits < 0 || bits > 30) return ST_INVALID;
  t.sketch_bits = bits;
  t.sketch.assign(bits > 0 ? size_t(kSketchRows) << bits : 0, 0u);
  return ST_OK;
}

// One lookup of a batch of `nfeat` features with `batch` samples each.
//   values        int64 [N]  the features' values, feature after feature
//   feat_n        int64 [nfeat]
//   bag_offsets   int32 [nfeat * (batch + 1)], each feature's own CSR from 0
//   slots, ops, mods, bounds (concatenated), nbounds: per-feature transform
// Outputs (caller-sized for N): unique_keys, unique_rows, inverse, counts,
// merged_offsets [nfeat * batch + 1], *num_unique.
//
// Steps, in the pages' order:
//  1. transform + tag each value ([README] Feature Engine);
//  2. merge the features of the logical table, feature-major, so bag
//     f * batch + i is sample i of feature f ([README] Distributed
//     optimisation: requests of same-attribute tables are merged);
//  3. dedup: the sorted distinct keys, each occurrence's index among them and
//     the occurrence count of each ([README] same passage: merged requests
//     are deduplicated);
//  4. IDMap: each distinct key, in ascending order, finds its row; on a miss
//     (unless FIND_ONLY) it is inserted; its count grows by its occurrences;
//     once the count reaches the admission threshold it gets a row initialised
//     from the initializer with zero optimizer state ([README] Efficient
//     dynamic Embedding; Embedding Engine: eviction and admission).
//     FIND_ONLY neither inserts nor counts: an absent key reports row -1.
int orc_insert_find(void* h, int32_t nfeat, int32_t batch, const int64_t* values,
                    const int64_t* feat_n, const int32_t* bag_offsets, const uint32_t* slots,
                    const uint32_t* ops, const uint64_t* mods, const int64_t* bounds,
                    const int64_t* nbounds, uint32_t flags, int64_t* unique_keys,
                    int64_t* unique_rows, int32_t* inverse, int32_t* counts,
                    int32_t* merged_offsets, int64_t* num_unique) {
  Table& t = *static_cast<Table*>(h);
  int64_t n_total = 0;
  for (int32_t f = 0; f < nfeat; ++f) n_total += feat_n[f];

  // 1 + 2: transform every occurrence, feature-major; merged bag offsets.
  std::vector<int64_t> keys(static_cast<size_t>(n_total));
  int64_t base = 0, bound_base = 0;
  for (int32_t f = 0; f < nfeat; ++f) {
    const int32_t* off = bag_offsets + size_t(f) * (batch + 1);
    if (off[0] != 0 || off[batch] != feat_n[f]) return ST_INVALID;
    for (int32_t i = 0; i < batch; ++i) {
      if (off[i + 1] < off[i]) return ST_INVALID;
      merged_offsets[size_t(f) * batch + i] = int32_t(base + off[i]);
    }
    int st = orc_transform(values + base, feat_n[f], ops[f], mods[f], bounds + bound_base,
                           nbounds[f], slots[f], keys.data() + base);
    if (st != ST_OK) return st;
    base += feat_n[f];
    bound_base += nbounds[f];
  }
  merged_offsets[size_t(nfeat) * batch] = int32_t(n_total);

  // 3: dedup.
  std::vector<int64_t> uniq(keys);
  std::sort(uniq.begin(), uniq.end());
  uniq.erase(std::unique(uniq.begin(), uniq.end()), uniq.end());
  const int64_t u_count = int64_t(uniq.size());
  for (int64_t u = 0; u < u_count; ++u) {
    unique_keys[u] = uniq[u];
    counts[u] = 0;
  }
  for (int64_t j = 0; j < n_total; ++j) {
    int64_t u = std::lower_bound(uniq.begin(), uniq.end(), keys[j]) - uniq.begin();
    inverse[j] = int32_t(u);
    counts[u] += 1;
  }
  *num_unique = u_count;

  // 4: IDMap.
  int status = ST_OK;
  const bool find_only = (flags & FLAG_FIND_ONLY) != 0;
  if (!find_only) ++t.step;
  // count-min sketch admission, phase 1: every key of this call that is not
  // in the map adds its occurrences to its counters (all of them before any
  // estimate is read, so the order of the keys does not matter)
  const bool sketching = !find_only && t.sketch_bits > 0;
  if (sketching)
    for (int64_t u = 0; u < u_count; ++u)
      if (t.idmap.find(uniq[u]) == t.idmap.end())
        for (int r = 0; r < kSketchRows; ++r) t.sketch[sketch_index(t, uniq[u], r)] += uint32_t(counts[u]);
  for (int64_t u = 0; u < u_count; ++u) {
    const int64_t key = uniq[u];
    auto it = t.idmap.find(key);
    if (find_only) {
      unique_rows[u] = (it == t.idmap.end()) ? -1 : it->second.row;
      continue;
    }
    uint64_t add = uint64_t(counts[u]);
    if (it == t.idmap.end()) {
      if (sketching) {
        // phase 2: the key enters the map (with its estimate as its count)
        // only once the estimate -- the smallest of its counters -- reaches
        // the admission threshold; until then it has no slot and no row
        uint32_t est = 0xFFFFFFFFu;
        for (int r = 0; r < kSketchRows; ++r) est = std::min(est, t.sketch[sketch_index(t, key, r)]);
        if (est < t.admit) {
          unique_rows[u] = -1;
          continue;
        }
        add = est;
      }
      if (int64_t(t.idmap.size()) >= t.max_keys) {
        status = ST_CAPACITY;
        unique_rows[u] = -1;
        continue;
      }
      it = t.idmap.emplace(key, Entry{-1, 0, 0}).first;
    }
    Entry& e = it->second;
    e.last_use = t.step;
    uint64_t c = uint64_t(e.count) + add;
    e.count = c > 0xFFFFFFFFull ? 0xFFFFFFFFu : uint32_t(c);
    if (e.row < 0 && e.count >= t.admit) {
      e.row = allocate_row(t, key);
      if (e.row < 0) status = ST_CAPACITY;
    }
    unique_rows[u] = e.row;
  }
  return status;
}

// Forward.  out[i, f*dim + d] = sum over the bag (f, i) of the rows' element d
// (SUM), or that sum divided by the bag length (MEAN); an empty bag gives 0;
// a key without a row adds a zero vector but still counts in the length.
// With POOL_NONE every occurrence j gets its row copied to out[j] in the
// storage dtype.  Sums are taken in double and rounded once.  `abs_out`
// (optional, pooled modes) receives the same pooling of |row| values, used by
// the tests as the scale of the summation-order tolerance.
// [README] Operator implementation (reduction); pooling mode from the
// workloads (sum / mean / gather only).
int orc_forward(void* h, const int64_t* unique_rows, const int32_t* inverse,
                const int32_t* merged_offsets, int32_t nfeat, int32_t batch, int32_t pool,
                void* out, double* abs_out) {
  const Table& t = *static_cast<Table*>(h);
  const int D = t.dim;
  const int64_t nbags = int64_t(nfeat) * batch;
  const int64_t n_total = merged_offsets[nbags];
  if (pool == POOL_NONE) {
    for (int64_t j = 0; j < n_total; ++j) {
      int64_t row = unique_rows[inverse[j]];
      for (int d = 0; d < D; ++d) {
        float v = row >= 0 ? t.params[size_t(row) * D + d] : 0.0f;
        if (t.dtype == DT_BF16)
          static_cast<uint16_t*>(out)[size_t(j) * D + d] = bf16_bits(v);
        else
          static_cast<float*>(out)[size_t(j) * D + d] = v;
      }
    }
    return ST_OK;
  }
  if (pool != POOL_SUM && pool != POOL_MEAN) return ST_INVALID;
  float* o = static_cast<float*>(out);
  std::vector<double> acc(D), aacc(D);
  for (int32_t f = 0; f < nfeat; ++f) {
    for (int32_t i = 0; i < batch; ++i) {
      const int64_t b = int64_t(f) * batch + i;
      const int64_t lo = merged_offsets[b], hi = merged_offsets[b + 1];
      std::fill(acc.begin(), acc.end(), 0.0);
      std::fill(aacc.begin(), aacc.end(), 0.0);
      for (int64_t j = lo; j < hi; ++j) {
        int64_t row = unique_rows[inverse[j]];
        if (row < 0) continue;
        for (int d = 0; d < D; ++d) {
          double v = t.params[size_t(row) * D + d];
          acc[d] += v;
          aacc[d] += std::fabs(v);
        }
      }
      const double len = double(hi - lo);
      for (int d = 0; d < D; ++d) {
        double v = acc[d], a = aacc[d];
        if (pool == POOL_MEAN && hi > lo) {
          v /= len;
          a /= len;
        }
        size_t idx = size_t(i) * nfeat * D + size_t(f) * D + d;
        o[idx] = static_cast<float>(v);
        if (abs_out) abs_out[idx] = a;
      }
    }
  }
  return ST_OK;
}

// Duplicate-gradient reduce.  G[u] = sum over occurrences j with inverse[j]
// == u of g_j, where g_j is the upstream gradient of j's bag (divided by the
// bag length for MEAN) or, for POOL_NONE, of j itself.  Summed in double.
// grad_dtype 0: float32; 1: bfloat16 bit patterns.  `abs_out` (optional)
// receives sum |g_j| per element.
// [README] Operator implementation: the reduction that merges duplicates
// before the atomically-sensitive update.
int orc_reduce_grads(void* h, const int32_t* inverse, const int32_t* merged_offsets,
                     int64_t num_unique, int32_t nfeat, int32_t batch, int32_t pool,
                     const void* grad, int32_t grad_dtype, double* G, double* abs_out) {
  const Table& t = *static_cast<Table*>(h);
  const int D = t.dim;
  std::fill(G, G + size_t(num_unique) * D, 0.0);
  if (abs_out) std::fill(abs_out, abs_out + size_t(num_unique) * D, 0.0);
  auto grad_at = [&](size_t idx) -> double {
    if (grad_dtype == DT_BF16) return bf16_value(static_cast<const uint16_t*>(grad)[idx]);
    return static_cast<const float*>(grad)[idx];
  };
  const int64_t nbags = int64_t(nfeat) * batch;
  for (int32_t f = 0; f < nfeat; ++f) {
    for (int32_t i = 0; i < batch; ++i) {
      const int64_t b = int64_t(f) * batch + i;
      const int64_t lo = merged_offsets[b], hi = merged_offsets[b + 1];
      for (int64_t j = lo; j < hi; ++j) {
        const int64_t u = inverse[j];
        for (int d = 0; d < D; ++d) {
          double g;
          if (pool == POOL_NONE) {
            g = grad_at(size_t(j) * D + d);
          } else {
            g = grad_at(size_t(i) * nfeat * D + size_t(f) * D + d);
            if (pool == POOL_MEAN) g /= double(hi - lo);
          }
          G[size_t(u) * D + d] += g;
          if (abs_out) abs_out[size_t(u) * D + d] += std::fabs(g);
        }
      }
    }
  }
  (void)nbags;
  return ST_OK;
}

// Sparse optimizer update of every distinct key of the step that has a row
// (a touched row whose G is exactly zero still updates).  [README] Efficient
// dynamic Embedding: optimizer state lives beside the parameters.  Readings
// (PyTorch semantics, since RecIS builds on PyTorch):
//   ADAGRAD: a += G^2;  w -= lr * G / (sqrt(a) + eps)      (no lr decay)
//   ADAM (lazy, as torch.optim.SparseAdam): one step counter t per table,
//     +1 per update call; m = b1 m + (1-b1) G; v = b2 v + (1-b2) G^2;
//     w -= lr * sqrt(1-b2^t) / (1-b1^t) * m / (sqrt(v) + eps).
// Computed in double on the stored values; each stored quantity is rounded
// once (state to float, parameters to the storage dtype).
// `only` (optional) restricts the update to the marked distinct keys.
int orc_apply_update(void* h, const int64_t* unique_rows, int64_t num_unique, const double* G,
                     double lr, double beta1, double beta2, double eps, const uint8_t* only) {
  Table& t = *static_cast<Table*>(h);
  const int D = t.dim;
  if (t.optim == OPT_NONE) return ST_UNSUPPORTED;
  if (t.optim == OPT_ADAM) t.adam_step += 1;
  const double step = double(t.adam_step);
  for (int64_t u = 0; u < num_unique; ++u) {
    const int64_t row = unique_rows[u];
    if (row < 0 || (only && !only[u])) continue;
    float* w = &t.params[size_t(row) * D];
    float* s = &t.state[size_t(row) * t.slots_per_elem * D];
    for (int d = 0; d < D; ++d) {
      const double g = G[size_t(u) * D + d];
      if (t.optim == OPT_ADAGRAD) {
        const double a = double(s[d]) + g * g;
        const double nw = double(w[d]) - lr * g / (std::sqrt(a) + eps);
        s[d] = static_cast<float>(a);
        w[d] = store_param(t, nw);
      } else {
        const double m = beta1 * double(s[d]) + (1.0 - beta1) * g;
        const double v = beta2 * double(s[D + d]) + (1.0 - beta2) * g * g;
        const double bc1 = 1.0 - std::pow(beta1, step);
        const double bc2 = 1.0 - std::pow(beta2, step);
        const double step_size = lr * std::sqrt(bc2) / bc1;
        const double nw = double(w[d]) - step_size * m / (std::sqrt(v) + eps);
        s[d] = static_cast<float>(m);
        s[D + d] = static_cast<float>(v);
        w[d] = store_param(t, nw);
      }
    }
  }
  return ST_OK;
}

// Backward of one step = duplicate reduce, then the sparse update.
int orc_backward_update(void* h, const int64_t* unique_rows, const int32_t* inverse,
                        const int32_t* merged_offsets, int64_t num_unique, int32_t nfeat,
                        int32_t batch, int32_t pool, const void* grad, int32_t grad_dtype,
                        double lr, double beta1, double beta2, double eps) {
  const Table& t = *static_cast<Table*>(h);
  std::vector<double> G(size_t(num_unique) * t.dim);
  int st = orc_reduce_grads(h, inverse, merged_offsets, num_unique, nfeat, batch, pool, grad,
                            grad_dtype, G.data(), nullptr);
  if (st != ST_OK) return st;
  return orc_apply_update(h, unique_rows, num_unique, G.data(), lr, beta1, beta2, eps, nullptr);
}

// Eviction pass.  [README] Embedding Engine: feature eviction and admission.
// Reading: every key (with or without a row) whose count since the last pass
// is below min_count leaves the map and releases its row; the surviving keys
// keep floor(count * decay) of their count (decay in [0, 1]: 0 restarts the
// window, 1 keeps the running total, in between the counts decay with time).
// Returns the number of keys removed.
int64_t orc_evict_decay(void* h, uint32_t min_count, double decay) {
  Table& t = *static_cast<Table*>(h);
  std::fill(t.sketch.begin(), t.sketch.end(), 0u);  // the sketch's window restarts with every pass
  std::vector<int64_t> gone;
  for (auto& kv : t.idmap) {
    if (kv.second.count < min_count) gone.push_back(kv.first);
    else kv.second.count = uint32_t(std::floor(double(kv.second.count) * decay));
  }
  std::sort(gone.begin(), gone.end());
  for (int64_t key : gone) {
    auto it = t.idmap.find(key);
    if (it->second.row >= 0) t.free_rows.push_back(it->second.row);
    t.idmap.erase(it);
  }
  return int64_t(gone.size());
}

int64_t orc_evict(void* h, uint32_t min_count) { return orc_evict_decay(h, min_count, 0.0); }

// LRU-bounded capacity (one of the richer eviction strategies the README's
// Embedding Engine leaves open).  Reading: a key's age is the number of
// counting lookups since one last counted it (0: the latest), with every age
// of 255 or more taken as 255.  The pass keeps the youngest ages whole, as
// many of them as fit in max_keys keys together, and removes every older key
// (releasing its row); counts are untouched.  Returns the number removed.
int64_t orc_evict_lru(void* h, int64_t max_keys) {
  Table& t = *static_cast<Table*>(h);
  std::fill(t.sketch.begin(), t.sketch.end(), 0u);
  std::vector<int64_t> hist(256, 0);
  auto age = [&](const Entry& e) { return std::min<uint32_t>(t.step - e.last_use, 255u); };
  for (auto& kv : t.idmap) hist[age(kv.second)] += 1;
  int64_t keep = 0;
  int oldest_kept = -1;
  for (int a = 0; a < 256 && keep + hist[a] <= max_keys; ++a) {
    keep += hist[a];
    oldest_kept = a;
  }
  std::vector<int64_t> gone;
  for (auto& kv : t.idmap)
    if (int(age(kv.second)) > oldest_kept) gone.push_back(kv.first);
  std::sort(gone.begin(), gone.end());
  for (int64_t key : gone) {
    auto it = t.idmap.find(key);
    if (it->second.row >= 0) t.free_rows.push_back(it->second.row);
    t.idmap.erase(it);
  }
  return int64_t(gone.size());
}

// Writeback.  [ML] What carries the argument / Summary: the item tower's
// output e is written into the cache row M[key] as an exact assignment (the
// eta = 1 SGD step on (M - e) lands exactly on e).  Reading for repeated keys
// in one batch: the writes happen in batch order, so the last one stays.  An
// absent key is inserted and given a row at once (no admission wait, count
// untouched, last use = the latest lookup); the stored value is e rounded
// once to the storage dtype.
int orc_writeback(void* h, const int64_t* keys, int64_t n, const float* rows) {
  Table& t = *static_cast<Table*>(h);
  const int D = t.dim;
  int status = ST_OK;
  for (int64_t i = 0; i < n; ++i) {
    if (keys[i] < 0) return ST_KEY_RANGE;
    auto it = t.idmap.find(keys[i]);
    if (it == t.idmap.end()) {
      if (int64_t(t.idmap.size()) >= t.max_keys) {
        status = ST_CAPACITY;
        continue;
      }
      it = t.idmap.emplace(keys[i], Entry{-1, 0, t.step}).first;
    }
    if (it->second.row < 0) {
      it->second.row = allocate_row(t, keys[i]);
      if (it->second.row < 0) {
        status = ST_CAPACITY;
        continue;
      }
    }
    for (int d = 0; d < D; ++d)
      t.params[size_t(it->second.row) * D + d] = store_param(t, double(rows[size_t(i) * D + d]));
  }
  return status;
}

// The rows the map holds now for `keys` (-1: absent, or present without a
// row).  A lookup's forward and backward act on the rows its keys hold when
// they run: the IDMap is the map from ID to offset ([README] Efficient
// dynamic Embedding), so a key evicted since the lookup has no row, and a
// row never moves while its key stays.
int orc_current_rows(void* h, const int64_t* keys, int64_t n, int64_t* rows) {
  const Table& t = *static_cast<Table*>(h);
  for (int64_t i = 0; i < n; ++i) {
    auto it = t.idmap.find(keys[i]);
    rows[i] = it == t.idmap.end() ? -1 : it->second.row;
  }
  return ST_OK;
}

int64_t orc_size(void* h) { return int64_t(static_cast<Table*>(h)->idmap.size()); }
int64_t orc_rows_in_use(void* h) {
  const Table& t = *static_cast<Table*>(h);
  return t.next_row - int64_t(t.free_rows.size());
}

// Canonical view: every key in ascending order with its row flag, count,
// parameters (as float values, exact in the storage dtype) and optimizer
// state; keys without a row report zeros.
int64_t orc_export(void* h, int64_t cap, int64_t* keys, int64_t* rows, uint32_t* counts,
                   float* params, float* state) {
  const Table& t = *static_cast<Table*>(h);
  std::vector<int64_t> ks;
  ks.reserve(t.idmap.size());
  for (const auto& kv : t.idmap) ks.push_back(kv.first);
  std::sort(ks.begin(), ks.end());
  const int D = t.dim, S = t.slots_per_elem * t.dim;
  int64_t n = std::min<int64_t>(cap, int64_t(ks.size()));
  for (int64_t i = 0; i < n; ++i) {
    const Entry& e = t.idmap.at(ks[i]);
    keys[i] = ks[i];
    rows[i] = e.row;
    counts[i] = e.count;
    for (int d = 0; d < D; ++d) params[size_t(i) * D + d] = e.row >= 0 ? t.params[size_t(e.row) * D + d] : 0.0f;
    for (int s = 0; s < S; ++s) state[size_t(i) * S + s] = e.row >= 0 ? t.state[size_t(e.row) * S + s] : 0.0f;
  }
  return int64_t(ks.size());
}

int64_t orc_adam_step(void* h) { return static_cast<Table*>(h)->adam_step; }

}  // extern "C"
