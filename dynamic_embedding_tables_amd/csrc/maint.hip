// maint.hip -- table maintenance kernels: slot fills, IDMap rebuild (growth
// and after eviction), the eviction pass, the cache writeback, and export.
//
// Pages: "RecIS (Recommendation Intelligence System)" README --
//   Core architecture > Embedding Engine (eviction and admission);
//   Key optimisations > Efficient dynamic Embedding (blocks grow on demand);
// "Memory Layer: Train the In-Model Cache for Recommendation Models" --
//   What carries the argument / Referee Report > Summary (Writeback: the
//   item tower's output is assigned exactly into the cache row).
#include "internal.h"

namespace recis {

namespace {

__global__ void k_fill_slots(Slot* slots, long long cap) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < cap;
       i += (long long)gridDim.x * blockDim.x) {
    Slot s;
    s.key = kEmptyKey;
    s.row = -1;
    s.count = 0;
    slots[i] = s;
  }
}

__global__ void k_fill_dedup(DedupSlot* dd, long long cap) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < cap;
       i += (long long)gridDim.x * blockDim.x) {
    DedupSlot s;
    s.key = kEmptyKey;
    s.count = 0;
    s.uidx = -1;
    dd[i] = s;
  }
}

// Insert `key` (absent, unique among concurrent inserters) into t's IDMap.
__device__ __forceinline__ long long claim_slot(const TableDev& t, long long key) {
  unsigned long long p = slot_of(key, t.slot_shift);
  for (unsigned long long n = 0; n <= t.region_mask; ++n) {
    const long long cur = t.slots[p].key;
    if (cur == kEmptyKey) {
      const long long old = (long long)atomicCAS((unsigned long long*)&t.slots[p].key,
                                                 (unsigned long long)kEmptyKey, (unsigned long long)key);
      if (old == kEmptyKey) return (long long)p;
    }
    p = next_slot(t, p);
  }
  return -1;
}

__global__ void k_rehash(const Slot* old_slots, const unsigned* old_last_use, long long old_cap, TableDev t) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < old_cap;
       i += (long long)gridDim.x * blockDim.x) {
    const Slot s = old_slots[i];
    if (s.key < 0) continue;
    const long long p = claim_slot(t, s.key);
    if (p < 0) {
      atomicOr(&t.ctr->error, kErrCapacity);
      continue;
    }
    t.slots[p].row = s.row;
    t.slots[p].count = s.count;
    if (t.last_use) t.last_use[p] = old_last_use[i];
  }
}

__device__ __forceinline__ long long wave_add(unsigned long long* ctr, bool take) {
  const unsigned long long m = __ballot(take);
  if (!m) return -1;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)m) - 1;
  unsigned long long base = 0;
  if (lane == leader) base = atomicAdd(ctr, (unsigned long long)__popcll(m));
  base = (unsigned long long)__shfl((long long)base, leader);
  const unsigned long long below = m & ((1ull << lane) - 1ull);
  return take ? (long long)(base + __popcll(below)) : -1;
}

__global__ void k_set_scratch(DevCounters* c) { c->scratch_count = 0; }

// A key's age for the LRU pass: counting lookups since one last counted it,
// ages from kAgeBins - 1 on taken as one.
constexpr int kAgeBins = 256;
constexpr long long kAgeSpan = 1 << 16;
__device__ __forceinline__ int age_of(const TableDev& t, long long i) {
  const unsigned a = t.step - t.last_use[i];
  return a < (unsigned)kAgeBins ? (int)a : kAgeBins - 1;
}

// Eviction: keys whose window count is below min_count leave (their slot is
// marked gone and the IDMap is rebuilt afterwards); their rows go to the free
// list; survivors keep floor(count * decay) (0: the window restarts).  A
// block takes kEvictSpan slots and gathers its freed rows in LDS (wave-wide
// counters), then reserves its share of the free list with one atomic:
// device atomics on one address execute one after another at the memory
// side, so one per wave would serialise the pass.
constexpr int kEvictSpan = 4096;
__global__ __launch_bounds__(256) void k_evict_mark(TableDev t, unsigned min_count, double decay,
                                                    const int* lru_cut) {
  __shared__ int s_rows[kEvictSpan];
  __shared__ int s_nfree, s_ngone;
  __shared__ long long s_base;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x == 0) {
    s_nfree = 0;
    s_ngone = 0;
  }
  __syncthreads();
  const int cut = lru_cut ? *lru_cut : 0;  // LRU pass: the oldest age kept; counts stay as they are
  const long long b0 = (long long)blockIdx.x * kEvictSpan;
  for (int k0 = 0; k0 < kEvictSpan; k0 += 256) {
    const long long i = b0 + k0 + threadIdx.x;
    bool gone = false;
    int row = -1;
    if (i <= (long long)t.slot_mask) {
      const Slot s = t.slots[i];
      if (s.key >= 0 && lru_cut) {
        if (age_of(t, i) > cut) {
          gone = true;
          row = s.row < 0 ? -1 : (s.row & ~kPendingRow);
          t.slots[i].key = kGoneKey;
        }
      } else if (s.key >= 0) {
        if (s.count < min_count) {
          gone = true;
          row = s.row < 0 ? -1 : (s.row & ~kPendingRow);
          t.slots[i].key = kGoneKey;
        } else {
          t.slots[i].count = decay == 0.0 ? 0u : (unsigned)floor((double)s.count * decay);
        }
      }
    }
    const bool frees = row >= 0;
    const unsigned long long mf = __ballot(frees), mg = __ballot(gone);
    int base = 0;
    if (lane == 0) {
      if (mf) base = atomicAdd(&s_nfree, __popcll(mf));
      if (mg) atomicAdd(&s_ngone, __popcll(mg));
    }
    base = __shfl(base, 0);
    if (frees) s_rows[base + __popcll(mf & ((1ull << lane) - 1ull))] = row;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    s_base = s_nfree ? (long long)atomicAdd((unsigned long long*)&t.ctr->free_top, (unsigned long long)s_nfree) : 0;
    if (s_ngone) atomicAdd(&t.ctr->scratch_count, (unsigned long long)s_ngone);
  }
  __syncthreads();
  for (int k = threadIdx.x; k < s_nfree; k += 256) t.free_list[s_base + k] = s_rows[k];
}

__global__ void k_evict_done(DevCounters* c, long long* num_evicted) {
  c->num_keys -= c->scratch_count;
  if (num_evicted) *num_evicted = (long long)c->scratch_count;
}

// Writeback, step 1: dedup the keys; the slot keeps the last occurrence index.
__global__ __launch_bounds__(256) void k_wb_dedup(TableDev t, const long long* keys, long long n,
                                                  DedupSlot* dd, unsigned long long mask, int shift,
                                                  long long* wb_keys, int* uslot) {
  __shared__ int s_new;
  __shared__ long long s_base;
  if (threadIdx.x == 0) s_new = 0;
  __syncthreads();
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  int p = -1, nidx = -1;
  long long key = 0;
  if (i < n) {
    key = keys[i];
    if (key < 0) {
      atomicOr(&t.ctr->error, kErrKeyRange);
    } else {
      unsigned long long q = ((unsigned long long)key * 0x9E3779B97F4A7C15ull) >> shift;
      bool won = false;
      while (true) {
        const long long cur = dd[q].key;
        if (cur == key) break;
        if (cur == kEmptyKey) {
          const long long old = (long long)atomicCAS((unsigned long long*)&dd[q].key,
                                                     (unsigned long long)kEmptyKey, (unsigned long long)key);
          if (old == kEmptyKey) {
            won = true;
            break;
          }
          if (old == key) break;
        }
        q = (q + 1) & mask;
      }
      p = (int)q;
      atomicMax(&dd[p].count, (int)i);
      if (won) nidx = atomicAdd(&s_new, 1);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && s_new > 0)
    s_base = (long long)atomicAdd(&t.ctr->scratch_count, (unsigned long long)s_new);
  __syncthreads();
  if (nidx >= 0) {
    const long long u = s_base + nidx;
    wb_keys[u] = key;
    uslot[u] = p;
    dd[p].uidx = (int)u;
  }
}

__device__ long long alloc_one_row(const TableDev& t) {
  long long top = t.ctr->free_top;
  while (top > 0) {
    const long long seen = (long long)atomicCAS((unsigned long long*)&t.ctr->free_top,
                                                (unsigned long long)top, (unsigned long long)(top - 1));
    if (seen == top) return t.free_list[top - 1];
    top = seen;
  }
  const long long r = (long long)atomicAdd(&t.ctr->next_row, 1ull);
  if (r >= t.rows_limit) {
    atomicAdd(&t.ctr->next_row, ~0ull);  // give the number back
    return -1;
  }
  return r;
}

// Writeback: find or insert key in the IDMap and give it a row if it has
// none (a pending row becomes written).  row = -1 on a full IDMap or row
// space (the error is raised); fresh = 1 when the row's state starts at zero.
__device__ void wb_find_row(const TableDev& t, long long key, long long& row, int& fresh) {
  row = -1;
  fresh = 0;
  unsigned long long p = slot_of(key, t.slot_shift);
  long long at = -1;
  bool inserted = false;
  for (unsigned long long n = 0; n <= t.region_mask; ++n) {
    const long long cur = t.slots[p].key;
    if (cur == key) {
      at = (long long)p;
      break;
    }
    if (cur == kEmptyKey) {
      const long long old = (long long)atomicCAS((unsigned long long*)&t.slots[p].key,
                                                 (unsigned long long)kEmptyKey, (unsigned long long)key);
      if (old == kEmptyKey) {
        at = (long long)p;
        inserted = true;
        break;
      }
      if (old == key) {
        at = (long long)p;
        break;
      }
    }
    p = next_slot(t, p);
  }
  if (at < 0) {
    atomicOr(&t.ctr->error, kErrCapacity);
  } else {
    if (inserted) {
      atomicAdd(&t.ctr->num_keys, 1ull);
      if (t.last_use) t.last_use[at] = t.step;
    }
    row = inserted ? -1 : t.slots[at].row;
    if (row >= 0 && (row & kPendingRow)) {  // allocated, never written: written now
      row &= ~(long long)kPendingRow;
      t.slots[at].row = (int)row;
      fresh = 1;
    } else if (row < 0) {
      row = alloc_one_row(t);
      if (row < 0) atomicOr(&t.ctr->error, kErrCapacity);
      else {
        t.slots[at].row = (int)row;
        fresh = 1;
      }
    }
  }
}

// Writeback, step 2: one wave per distinct key: find or insert it, give it a
// row if it has none, and store the last occurrence's values.
template <typename TP>
__global__ __launch_bounds__(256) void k_wb_apply(TableDev t, const float* rows, DedupSlot* dd,
                                                  const long long* wb_keys, const int* uslot) {
  const long long U = (long long)t.ctr->scratch_count;
  const int lane = threadIdx.x & 63;
  for (long long u = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); u < U; u += (long long)gridDim.x * 4) {
    const long long key = wb_keys[u];
    DedupSlot* d = &dd[uslot[u]];
    const int last = d->count;
    long long row = -1;
    int fresh = 0;
    if (lane == 0) wb_find_row(t, key, row, fresh);
    row = __shfl(row, 0);
    fresh = __shfl(fresh, 0);
    if (row >= 0) {
      char* rp = row_ptr(t.rs, row);
      const float* src = rows + (long long)last * t.dim;
      for (int e = lane; e < t.dim; e += 64) {
        if (sizeof(TP) == 2) reinterpret_cast<unsigned short*>(rp)[e] = f32_to_bf16(src[e]);
        else reinterpret_cast<float*>(rp)[e] = src[e];
      }
      if (fresh) {
        float* st = reinterpret_cast<float*>(rp + (long long)t.dim * (long long)sizeof(TP));
        for (int e = lane; e < t.state_words * t.dim; e += 64) st[e] = 0.f;
      }
    }
    if (lane == 0) {
      d->key = kEmptyKey;
      d->count = 0;
    }
  }
}

// Writeback, step 2, for rows 16-byte aligned: sixteen lanes per distinct
// key, four keys per wave, so that one round of waves covers a batch of
// cache writes.  Each group loads its key's last row before its leader looks
// the key up, so the row's fetch overlaps the IDMap round trips.
template <typename TP>
__global__ __launch_bounds__(256) void k_wb_apply_vec(TableDev t, const float* rows, DedupSlot* dd,
                                                      const long long* wb_keys, const int* uslot) {
  constexpr int G = 16;              // lanes per key
  constexpr int MAXC = 256 / 4 / G;  // 16-byte chunks per lane at the largest dim
  const long long U = (long long)t.ctr->scratch_count;
  const int lane = threadIdx.x & 63, gl = lane & (G - 1), lead = lane & ~(G - 1);
  const int nc = t.dim >> 2;
  const long long ngroups = (long long)gridDim.x * (blockDim.x / G);
  // a group's lanes share u, so every shuffle below reads an active leader
  for (long long u = ((long long)blockIdx.x * blockDim.x + threadIdx.x) / G; u < U; u += ngroups) {
    const long long key = wb_keys[u];
    DedupSlot* d = &dd[uslot[u]];
    const float4* src = reinterpret_cast<const float4*>(rows + (long long)d->count * t.dim);
    float4 v[MAXC];
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (gl + j * G < nc) v[j] = src[gl + j * G];
    }
    long long row = -1;
    int fresh = 0;
    if (gl == 0) wb_find_row(t, key, row, fresh);
    row = __shfl(row, lead);
    fresh = __shfl(fresh, lead);
    if (row >= 0) {
      char* rp = row_ptr(t.rs, row);
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        const int c = gl + j * G;
        if (c >= nc) continue;
        if (sizeof(TP) == 2)
          reinterpret_cast<uint2*>(rp)[c] =
              make_uint2((unsigned)f32_to_bf16(v[j].x) | ((unsigned)f32_to_bf16(v[j].y) << 16),
                         (unsigned)f32_to_bf16(v[j].z) | ((unsigned)f32_to_bf16(v[j].w) << 16));
        else
          reinterpret_cast<float4*>(rp)[c] = v[j];
      }
      if (fresh) {
        float4* st = reinterpret_cast<float4*>(rp + (long long)t.dim * (long long)sizeof(TP));
        for (int c = gl; c < (t.state_words * t.dim) >> 2; c += G) st[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    if (gl == 0) {
      d->key = kEmptyKey;
      d->count = 0;
    }
  }
}

// Export step 1: compact the occupied slots.
__global__ void k_export(TableDev t, long long cap, long long* keys, long long* rows, unsigned* counts) {
  for (long long i0 = (long long)blockIdx.x * blockDim.x; i0 <= (long long)t.slot_mask;
       i0 += (long long)gridDim.x * blockDim.x) {
    const long long i = i0 + threadIdx.x;
    Slot s;
    s.key = kEmptyKey;
    if (i <= (long long)t.slot_mask) s = t.slots[i];
    const long long at = wave_add(&t.ctr->scratch_count, s.key >= 0);
    if (at >= 0 && at < cap) {
      keys[at] = s.key;
      rows[at] = s.row;
      counts[at] = s.count;
    }
  }
}

// Export step 2: one wave per exported key copies params and state; a pending
// row reports its initial values and zero state.  rows[] is left without the
// pending mark.
__global__ void k_export_rows(TableDev t, long long n, const long long* keys, long long* rows, char* params,
                              float* state) {
  const int lane = threadIdx.x & 63;
  const int es = t.dtype == RECIS_DTYPE_BF16 ? 2 : 4;
  const long long pbytes = (long long)t.dim * es;
  const int sw = t.state_words * t.dim;
  const int pchunks = (int)(pbytes >> 4), schunks = state ? sw >> 2 : 0;  // 16-byte chunks (rows are 16-aligned)
  const int cpr = pchunks + schunks;
  constexpr int kCopy = 4;
  for (long long k0 = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64; k0 < n;
       k0 += (long long)gridDim.x * 4 * 64) {
    // one key per lane: its row, without the pending mark
    const long long k = k0 + lane;
    long long r = k < n ? rows[k] : -1;
    const bool pending = r >= 0 && (r & kPendingRow);
    if (pending) r &= ~(long long)kPendingRow;
    const long long key = k < n ? keys[k] : 0;
    // then the wave's rows as one list of 16-byte chunks (key j, chunk c);
    // a pending row is the initializer's, a key without a row gets zeros
    for (int i0 = 0; i0 < 64 * cpr; i0 += 64 * kCopy) {
      uint4 v[kCopy];
      uint4* dst[kCopy];
#pragma unroll
      for (int x = 0; x < kCopy; ++x) {
        const int idx = i0 + x * 64 + lane;
        const int j = idx / cpr, c = idx - j * cpr;
        const int js = j < 64 ? j : 0;
        const long long rj = __shfl(r, js);
        const bool pj = __shfl((int)pending, js) != 0;
        const long long keyj = __shfl(key, js);
        const long long kj = k0 + j;
        v[x] = make_uint4(0, 0, 0, 0);
        dst[x] = nullptr;
        if (idx >= 64 * cpr || kj >= n) continue;
        dst[x] = c < pchunks ? reinterpret_cast<uint4*>(params) + kj * pchunks + c
                             : reinterpret_cast<uint4*>(state) + kj * schunks + (c - pchunks);
        if (rj >= 0 && pj) {
          if (c < pchunks) v[x] = init_chunk(t, keyj, c);
        } else if (rj >= 0) {
          v[x] = reinterpret_cast<const uint4*>(row_ptr(t.rs, rj))[c];
        }
      }
#pragma unroll
      for (int x = 0; x < kCopy; ++x)
        if (dst[x]) *dst[x] = v[x];
    }
    if (k < n) rows[k] = r;
  }
}

// Import (the inverse of export, into an empty table).  One key per lane:
// it is entered into the IDMap with its count (a key already there is an
// input error), and the keys that had a row get the next rows of the bump
// pointer, one atomic per wave.  Then the wave copies its keys' rows, 16
// bytes per lane: the parameters as given (storage dtype), then the state.
__global__ __launch_bounds__(256) void k_import(TableDev t, long long n, const long long* keys,
                                                const long long* rows_in, const unsigned* counts,
                                                const char* params, const float* state) {
  const int lane = threadIdx.x & 63;
  const int es = t.dtype == RECIS_DTYPE_BF16 ? 2 : 4;
  const long long pbytes = (long long)t.dim * es;
  const long long sbytes = (long long)t.state_words * t.dim * 4;
  const int pchunks = (int)(pbytes >> 4), schunks = (int)(sbytes >> 4);
  for (long long k0 = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64; k0 < n;
       k0 += (long long)gridDim.x * 4 * 64) {
    const long long k = k0 + lane;
    long long at = -1;
    bool want_row = false;
    unsigned err = 0;
    if (k < n) {
      const long long key = keys[k];
      if (key < 0) {
        err = kErrKeyRange;
      } else {
        unsigned long long p = slot_of(key, t.slot_shift);
        for (unsigned long long q = 0; q <= t.region_mask; ++q) {
          const long long cur = t.slots[p].key;
          if (cur == key) {
            err = kErrInvalid;  // the key is in the input twice
            break;
          }
          if (cur == kEmptyKey) {
            const long long old = (long long)atomicCAS((unsigned long long*)&t.slots[p].key,
                                                       (unsigned long long)kEmptyKey, (unsigned long long)key);
            if (old == kEmptyKey) {
              at = (long long)p;
              break;
            }
            if (old == key) {
              err = kErrInvalid;
              break;
            }
          }
          p = next_slot(t, p);
        }
        if (at < 0 && !err) err = kErrCapacity;
      }
      want_row = at >= 0 && rows_in[k] >= 0;
    }
    const long long row = wave_add(&t.ctr->next_row, want_row);
    (void)wave_add(&t.ctr->num_keys, at >= 0);
    long long r = -1;
    if (at >= 0) {
      t.slots[at].count = counts[k];
      if (t.last_use) t.last_use[at] = t.step;
      if (want_row && row < t.rows_limit) r = row;
      else if (want_row) err |= kErrCapacity;
      t.slots[at].row = r >= 0 ? (int)r : -1;
    }
    if (err) atomicOr(&t.ctr->error, err);
    // the wave's rows as one list of 16-byte chunks (row j, chunk c), kCopy
    // loads in flight per lane
    constexpr int kCopy = 4;
    const int cpr = pchunks + schunks;
    for (int i0 = 0; i0 < 64 * cpr; i0 += 64 * kCopy) {
      uint4 v[kCopy];
      long long rr[kCopy];
      int cc[kCopy];
#pragma unroll
      for (int x = 0; x < kCopy; ++x) {
        const int idx = i0 + x * 64 + lane;
        const int j = idx / cpr, c = idx - j * cpr;
        rr[x] = __shfl(r, j < 64 ? j : 0);
        cc[x] = c;
        if (idx >= 64 * cpr) rr[x] = -1;
        v[x] = make_uint4(0, 0, 0, 0);
        if (rr[x] >= 0) {
          const long long kj = k0 + j;
          v[x] = c < pchunks ? reinterpret_cast<const uint4*>(params + kj * pbytes)[c]
                             : reinterpret_cast<const uint4*>(state + kj * (sbytes >> 2))[c - pchunks];
        }
      }
#pragma unroll
      for (int x = 0; x < kCopy; ++x)
        if (rr[x] >= 0) reinterpret_cast<uint4*>(row_ptr(t.rs, rr[x]))[cc[x]] = v[x];
    }
  }
}

// LRU-bounded eviction.  A key's age is the number of counting lookups since
// one last counted it, with ages from 255 on taken as 255.  k_age_hist: per
// block of kAgeSpan slots, the histogram of ages in LDS, written as that
// block's row of `work`.  k_age_cut: one block sums the rows and finds the
// oldest age that can stay: the youngest ages are kept whole while their
// keys fit in max_keys.  k_evict_mark then removes every older key.

__global__ __launch_bounds__(256) void k_age_hist(TableDev t, int* work) {
  __shared__ int s_h[kAgeBins];
  s_h[threadIdx.x] = 0;
  __syncthreads();
  const long long b0 = (long long)blockIdx.x * kAgeSpan;
  for (long long k = threadIdx.x; k < kAgeSpan; k += 256) {
    const long long i = b0 + k;
    if (i > (long long)t.slot_mask) break;
    if (t.slots[i].key >= 0) atomicAdd(&s_h[age_of(t, i)], 1);
  }
  __syncthreads();
  work[(long long)blockIdx.x * kAgeBins + threadIdx.x] = s_h[threadIdx.x];
}

// work[nblocks * kAgeBins] holds the cut afterwards: the oldest age kept (-1: none)
__global__ __launch_bounds__(256) void k_age_cut(int* work, long long nblocks, long long max_keys) {
  __shared__ long long s_c[kAgeBins];
  long long c = 0;
  for (long long b = 0; b < nblocks; ++b) c += work[b * kAgeBins + threadIdx.x];
  s_c[threadIdx.x] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long keep = 0;
    int oldest = -1;
    for (int a = 0; a < kAgeBins && keep + s_c[a] <= max_keys; ++a) {
      keep += s_c[a];
      oldest = a;
    }
    work[nblocks * kAgeBins] = oldest;
  }
}

// ------------------------------------------------------ hot-tier placement
// Rows [0, H) live in HBM blocks, the rest in host blocks.  A key's class is
// floor(log2(count)) + 1 (0 for a zero count); the top classes whose keys fit
// H rows together are hot.  Six launches: per-block class histograms; the
// cut (one block); per-block counts of the two lists (hot keys on host rows,
// cooler keys on HBM rows); their scan (one block); the lists, each block's
// part at its scanned base; then one wave per pair swaps the two rows and
// their IDMap entries.  No global atomics.
constexpr int kTierBins = 33;
constexpr long long kTierSpan = 1 << 16;  // IDMap slots per block
__device__ __forceinline__ int tier_class(unsigned c) { return 32 - __clz((int)c); }

struct TierWork {
  int* hist;         // [nb][kTierBins]
  int* cnt;          // [2][nb]: per-block list sizes, then (scanned) bases
  long long* ctl;    // [0] hot class cut, [1] pairs, [2] list A size, [3] list B size
  unsigned* list_a;  // [H] slots of hot keys holding host rows
  unsigned* list_b;  // [H] slots of cooler keys holding HBM rows
};
__host__ __device__ inline long long tier_blocks(long long slot_cap) { return (slot_cap + kTierSpan - 1) / kTierSpan; }
inline TierWork tier_work(int* w, long long slot_cap, long long H) {
  const long long nb = tier_blocks(slot_cap);
  TierWork tw;
  tw.hist = w;
  tw.cnt = w + nb * kTierBins;
  const long long ctl_at = (nb * kTierBins + 2 * nb + 1) & ~1ll;  // 8-byte aligned (the scratch is)
  tw.ctl = reinterpret_cast<long long*>(w + ctl_at);
  tw.list_a = reinterpret_cast<unsigned*>(w + ctl_at + 8);
  tw.list_b = tw.list_a + H;
  return tw;
}

__global__ __launch_bounds__(256) void k_tier_hist(TableDev t, TierWork w) {
  __shared__ int s_h[kTierBins];
  if (threadIdx.x < kTierBins) s_h[threadIdx.x] = 0;
  __syncthreads();
  const long long b0 = (long long)blockIdx.x * kTierSpan;
  for (long long k = threadIdx.x; k < kTierSpan; k += 256) {
    const long long i = b0 + k;
    if (i > (long long)t.slot_mask) break;
    const Slot sl = t.slots[i];
    if (sl.key >= 0 && sl.row >= 0) atomicAdd(&s_h[tier_class(sl.count)], 1);
  }
  __syncthreads();
  if (threadIdx.x < kTierBins) w.hist[(long long)blockIdx.x * kTierBins + threadIdx.x] = s_h[threadIdx.x];
}

__global__ __launch_bounds__(256) void k_tier_cut(TierWork w, long long nb, long long H) {
  __shared__ long long s_tot[kTierBins];
  if (threadIdx.x < kTierBins) s_tot[threadIdx.x] = 0;
  __syncthreads();
  long long v[kTierBins];  // this thread's blocks, every class
#pragma unroll
  for (int j = 0; j < kTierBins; ++j) v[j] = 0;
  for (long long b = threadIdx.x; b < nb; b += 256)
#pragma unroll
    for (int j = 0; j < kTierBins; ++j) v[j] += w.hist[b * kTierBins + j];
#pragma unroll
  for (int j = 0; j < kTierBins; ++j)
    if (v[j]) atomicAdd((unsigned long long*)&s_tot[j], (unsigned long long)v[j]);
  __syncthreads();
  if (threadIdx.x == 0) {
    // the lowest class such that it and the classes above fit in H rows
    long long acc = 0;
    int cut = 0;
    for (int j = kTierBins - 1; j >= 0; --j) {
      acc += s_tot[j];
      if (acc > H) {
        cut = j + 1;
        break;
      }
    }
    w.ctl[0] = cut;
  }
}

// Which list slot i of the IDMap goes to: 1 (A: hot on a host row), 2 (B: not
// hot on an HBM row), 0 none.
__device__ __forceinline__ int tier_list(const TableDev& t, long long i, int cut, long long H) {
  const Slot sl = t.slots[i];
  if (sl.key < 0 || sl.row < 0) return 0;
  const long long r = sl.row & ~kPendingRow;
  const bool hot = tier_class(sl.count) >= cut;
  if (hot && r >= H) return 1;
  if (!hot && r < H) return 2;
  return 0;
}

// Per block: list sizes (COUNT) or the lists at the scanned bases (PLACE),
// in slot order within the block.
template <bool PLACE>
__global__ __launch_bounds__(256) void k_tier_lists(TableDev t, TierWork w, long long nb, long long H) {
  __shared__ int s_w[2][4];
  __shared__ int s_run[2];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int cut = (int)w.ctl[0];
  if (threadIdx.x < 2) s_run[threadIdx.x] = 0;
  const long long b0 = (long long)blockIdx.x * kTierSpan;
  const long long base_a = PLACE ? w.cnt[blockIdx.x] : 0, base_b = PLACE ? w.cnt[nb + blockIdx.x] : 0;
  for (long long k0 = 0; k0 < kTierSpan; k0 += 256) {
    const long long i = b0 + k0 + threadIdx.x;
    const int which = i <= (long long)t.slot_mask ? tier_list(t, i, cut, H) : 0;
    const unsigned long long ma = __ballot(which == 1), mb = __ballot(which == 2);
    __syncthreads();  // the previous round's reads of s_w are done
    if (lane == 0) {
      s_w[0][wid] = __popcll(ma);
      s_w[1][wid] = __popcll(mb);
    }
    __syncthreads();
    int pa = s_run[0], pb = s_run[1];
    for (int x = 0; x < wid; ++x) {
      pa += s_w[0][x];
      pb += s_w[1][x];
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    if (PLACE && which == 1) w.list_a[base_a + pa + __popcll(ma & below)] = (unsigned)i;
    if (PLACE && which == 2) w.list_b[base_b + pb + __popcll(mb & below)] = (unsigned)i;
    __syncthreads();
    if (threadIdx.x == 0) {
      s_run[0] += s_w[0][0] + s_w[0][1] + s_w[0][2] + s_w[0][3];
      s_run[1] += s_w[1][0] + s_w[1][1] + s_w[1][2] + s_w[1][3];
    }
  }
  __syncthreads();
  if (!PLACE && threadIdx.x == 0) {
    w.cnt[blockIdx.x] = s_run[0];
    w.cnt[nb + blockIdx.x] = s_run[1];
  }
}

// One block: exclusive scans of the two per-block size arrays (each thread
// a contiguous run of blocks, its loads in flight together); the pairs are
// as many as the shorter list.
__global__ __launch_bounds__(1024) void k_tier_scan(TierWork w, long long nb) {
  __shared__ long long s_w[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const long long per = (nb + 1023) / 1024, b0 = (long long)tid * per;
  for (int l = 0; l < 2; ++l) {
    int* c = w.cnt + l * nb;
    long long sum = 0;
    for (long long b = b0; b < b0 + per && b < nb; ++b) sum += c[b];
    long long x = sum;  // inclusive scan over the wave
    for (int d = 1; d < 64; d <<= 1) {
      const long long y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane == 63) s_w[l][wid] = x;
    __syncthreads();
    long long run = x - sum, all = 0;
    for (int q = 0; q < 16; ++q) {
      run += q < wid ? s_w[l][q] : 0;
      all += s_w[l][q];
    }
    for (long long b = b0; b < b0 + per && b < nb; ++b) {
      const int v = c[b];
      c[b] = (int)run;
      run += v;
    }
    if (tid == 0) w.ctl[2 + l] = all;
    __syncthreads();
  }
  if (tid == 0) w.ctl[1] = w.ctl[2] < w.ctl[3] ? w.ctl[2] : w.ctl[3];
}

// One wave per pair: key a (hot, host row) and key b (cooler, HBM row)
// exchange rows -- each written row's bytes copied to the other row first
// (a row never written moves as its pending mark alone) -- and IDMap
// entries.
__global__ __launch_bounds__(256) void k_tier_swap(TableDev t, TierWork w, long long* num_moved) {
  const long long np = w.ctl[1];
  const int lane = threadIdx.x & 63;
  const int nc = (int)(t.rs.stride >> 4);  // 16-byte chunks per row
  for (long long q = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); q < np; q += (long long)gridDim.x * 4) {
    const unsigned sa = w.list_a[q], sb = w.list_b[q];
    const int rowa = t.slots[sa].row, rowb = t.slots[sb].row;
    const int pa = rowa & kPendingRow, pb = rowb & kPendingRow;
    const int ra = rowa & ~kPendingRow, rb = rowb & ~kPendingRow;
    uint4* A = reinterpret_cast<uint4*>(row_ptr(t.rs, ra));
    uint4* B = reinterpret_cast<uint4*>(row_ptr(t.rs, rb));
    for (int c0 = 0; c0 < nc; c0 += 64) {
      const int c = c0 + lane;
      uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
      if (c < nc) {
        if (!pa) va = A[c];
        if (!pb) vb = B[c];
      }
      if (c < nc) {
        if (!pa) B[c] = va;
        if (!pb) A[c] = vb;
      }
    }
    if (lane == 0) {
      t.slots[sa].row = rb | pa;
      t.slots[sb].row = ra | pb;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && num_moved) *num_moved = np;
}

unsigned grid_for(long long n, int threads) {
  long long g = (n + threads - 1) / threads;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

void launch_fill_slots(Slot* slots, long long cap, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_slots, dim3(grid_for(cap, 256)), dim3(256), 0, s, slots, cap);
}

// Ages of given keys for a save (set: stamps from saved ages for a restore).
// An age counts the counting lookups since one last counted the key; absent
// keys report ~0u (and are skipped when setting).
__global__ void k_key_ages(TableDev t, const long long* keys, long long n, unsigned* ages, int set) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    const long long key = keys[i];
    long long at = -1;
    if (key >= 0) {
      unsigned long long p = slot_of(key, t.slot_shift);
      for (unsigned long long q = 0; q <= t.region_mask; ++q) {
        const long long cur = t.slots[p].key;
        if (cur == key) {
          at = (long long)p;
          break;
        }
        if (cur == kEmptyKey) break;
        p = next_slot(t, p);
      }
    }
    if (set) {
      if (at >= 0) t.last_use[at] = t.step - ages[i];
    } else {
      ages[i] = at >= 0 ? t.step - t.last_use[at] : ~0u;
    }
  }
}

__global__ void k_zero_u32(unsigned* p, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = 0u;
}

void launch_key_ages(const TableDev& t, const long long* keys, long long n, unsigned* ages, bool set, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_key_ages, dim3(grid_for(n, 256)), dim3(256), 0, s, t, keys, n, ages, set ? 1 : 0);
}

void launch_zero_u32(unsigned* p, long long n, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_u32, dim3(grid_for(n, 256)), dim3(256), 0, s, p, n);
}

void launch_fill_dedup(DedupSlot* dd, long long cap, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_dedup, dim3(grid_for(cap, 256)), dim3(256), 0, s, dd, cap);
}

void launch_rehash(const Slot* old_slots, const unsigned* old_last_use, long long old_cap, const TableDev& t,
                   hipStream_t s) {
  hipLaunchKernelGGL(k_rehash, dim3(grid_for(old_cap, 256)), dim3(256), 0, s, old_slots, old_last_use, old_cap, t);
}

void launch_evict(const TableDev& t, unsigned min_count, double decay, long long* num_evicted, hipStream_t s) {
  hipLaunchKernelGGL(k_set_scratch, dim3(1), dim3(1), 0, s, t.ctr);
  const long long nb = ((long long)t.slot_mask + kEvictSpan) / kEvictSpan;
  hipLaunchKernelGGL(k_evict_mark, dim3((unsigned)nb), dim3(256), 0, s, t, min_count, decay, (const int*)nullptr);
  hipLaunchKernelGGL(k_evict_done, dim3(1), dim3(1), 0, s, t.ctr, num_evicted);
}

long long retier_words(long long slot_cap, long long hbm_rows) {
  const long long nb = tier_blocks(slot_cap);
  return ((nb * kTierBins + 2 * nb + 1) & ~1ll) + 8 + 2 * hbm_rows + 2;
}

void launch_retier(const TableDev& t, long long hbm_rows, int* work, long long* num_moved, hipStream_t s) {
  const long long nb = tier_blocks((long long)t.slot_mask + 1);
  const TierWork w = tier_work(work, (long long)t.slot_mask + 1, hbm_rows);
  hipLaunchKernelGGL(k_tier_hist, dim3((unsigned)nb), dim3(256), 0, s, t, w);
  hipLaunchKernelGGL(k_tier_cut, dim3(1), dim3(256), 0, s, w, nb, hbm_rows);
  hipLaunchKernelGGL((k_tier_lists<false>), dim3((unsigned)nb), dim3(256), 0, s, t, w, nb, hbm_rows);
  hipLaunchKernelGGL(k_tier_scan, dim3(1), dim3(1024), 0, s, w, nb);
  hipLaunchKernelGGL((k_tier_lists<true>), dim3((unsigned)nb), dim3(256), 0, s, t, w, nb, hbm_rows);
  hipLaunchKernelGGL(k_tier_swap, dim3(grid_for(hbm_rows, 4)), dim3(256), 0, s, t, w, num_moved);
}

long long age_hist_words(long long slot_cap) { return (slot_cap + kAgeSpan - 1) / kAgeSpan * kAgeBins + 1; }

void launch_evict_lru(const TableDev& t, long long max_keys, int* work, long long* num_evicted, hipStream_t s) {
  const long long hb = ((long long)t.slot_mask + kAgeSpan) / kAgeSpan;
  hipLaunchKernelGGL(k_set_scratch, dim3(1), dim3(1), 0, s, t.ctr);
  hipLaunchKernelGGL(k_age_hist, dim3((unsigned)hb), dim3(256), 0, s, t, work);
  hipLaunchKernelGGL(k_age_cut, dim3(1), dim3(256), 0, s, work, hb, max_keys);
  const long long nb = ((long long)t.slot_mask + kEvictSpan) / kEvictSpan;
  hipLaunchKernelGGL(k_evict_mark, dim3((unsigned)nb), dim3(256), 0, s, t, 0u, 0.0,
                     (const int*)(work + hb * kAgeBins));
  hipLaunchKernelGGL(k_evict_done, dim3(1), dim3(1), 0, s, t.ctr, num_evicted);
}

void launch_writeback(const TableDev& t, const long long* keys, long long n, const float* rows,
                      DedupSlot* dd, unsigned long long dd_mask, int dd_shift, long long* wb_keys,
                      int* uslot, hipStream_t s) {
  hipLaunchKernelGGL(k_set_scratch, dim3(1), dim3(1), 0, s, t.ctr);
  if (n == 0) return;
  hipLaunchKernelGGL(k_wb_dedup, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, t, keys, n, dd,
                     dd_mask, dd_shift, wb_keys, uslot);
  if ((reinterpret_cast<uintptr_t>(rows) & 15) == 0) {  // sixteen keys per block
    const unsigned g = grid_for(n, 16);
    if (t.dtype == RECIS_DTYPE_BF16)
      hipLaunchKernelGGL(k_wb_apply_vec<unsigned short>, dim3(g), dim3(256), 0, s, t, rows, dd, wb_keys, uslot);
    else
      hipLaunchKernelGGL(k_wb_apply_vec<float>, dim3(g), dim3(256), 0, s, t, rows, dd, wb_keys, uslot);
    return;
  }
  const unsigned g = grid_for(n, 4);
  if (t.dtype == RECIS_DTYPE_BF16)
    hipLaunchKernelGGL(k_wb_apply<unsigned short>, dim3(g), dim3(256), 0, s, t, rows, dd, wb_keys, uslot);
  else
    hipLaunchKernelGGL(k_wb_apply<float>, dim3(g), dim3(256), 0, s, t, rows, dd, wb_keys, uslot);
}

void launch_export(const TableDev& t, long long cap, long long* keys, long long* rows, unsigned* counts,
                   hipStream_t s) {
  hipLaunchKernelGGL(k_set_scratch, dim3(1), dim3(1), 0, s, t.ctr);
  hipLaunchKernelGGL(k_export, dim3(grid_for((long long)t.slot_mask + 1, 256)), dim3(256), 0, s, t, cap,
                     keys, rows, counts);
}

void launch_import(const TableDev& t, long long n, const long long* keys, const long long* rows,
                   const unsigned* counts, const void* params, const float* state, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_import, dim3(grid_for((n + 63) / 64, 4)), dim3(256), 0, s, t, n, keys, rows, counts,
                     static_cast<const char*>(params), state);
}

void launch_export_rows(const TableDev& t, long long n, const long long* keys, long long* rows, void* params,
                        float* state, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_export_rows, dim3(grid_for((n + 63) / 64, 4)), dim3(256), 0, s, t, n, keys, rows,
                     static_cast<char*>(params), state);
}

}  // namespace recis
