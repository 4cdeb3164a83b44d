// lookup.hip -- insert_find: fused transform + dedup, IDMap probe / insert,
// row allocation, and the per-key grouping of occurrences.
//
// Pages: "RecIS (Recommendation Intelligence System)" README --
//   Core architecture > Feature Engine (Hash / Mod / Bucketize, fused);
//   Key optimisations > Distributed optimisation (merged requests, dedup);
//   Key optimisations > Efficient dynamic Embedding (IDMap -> Offset ->
//   EmbeddingBlocks with parameters and optimizer state);
//   Core architecture > Embedding Engine (admission).
//
// Kernel sequence of one call (all on one stream, no host read-back):
//   k_prep      merged bag offsets, offset validation, per-call counters
//   k_dedup     per occurrence: transform + tag, dedup within the block in
//               LDS (rank among equal keys), then one insert into the call's
//               dedup table and one count atomic per distinct key per block
//               (hot keys never serialise on one address)
//   k_key_probe per distinct key: IDMap probe / CAS insert, count, admission
//               decision; block sums of (occurrences, rows to allocate)
//   k_key_scan  one block: exclusive scan of the block sums; rows come from
//               the free list first, then from the bump pointer -- by prefix
//               sum, not by atomics
//   k_key_finalize  per distinct key: group offsets, row assignment (the new
//               row is marked pending, not written: its values are the
//               initializer's until its first update), backward plan for
//               long keys, dedup-table reset
//   k_group     per occurrence: inverse index, the grouped bag / occurrence
//               list used by the backward reduction, and the occurrence's row
//               reference used by the forward
// Memory accesses that do not depend on each other are issued as one batch
// per thread (all loads of a phase before any use), so that each thread
// waits once per phase rather than once per item.
#include "internal.h"

namespace recis {

namespace {

__device__ __forceinline__ long long shfl64(long long v, int src) {
  int lo = __shfl((int)(unsigned long long)v, src);
  int hi = __shfl((int)((unsigned long long)v >> 32), src);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// Block-wide exclusive scan of one uint64 per thread; returns the prefix and
// writes the block total to *total.  kThreads = 256 = 4 waves.
__device__ unsigned long long block_exclusive_scan(unsigned long long v, unsigned long long* total) {
  __shared__ unsigned long long s_w[kThreads / 64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  unsigned long long x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    unsigned long long y = (unsigned long long)shfl64((long long)x, lane >= d ? lane - d : lane);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_w[wid] = x;
  __syncthreads();
  unsigned long long before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wid) before += s_w[w];
    all += s_w[w];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

__device__ __forceinline__ int find_feature(const FeatDev* feats, int F, long long blk) {
  int lo = 0, hi = F - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (feats[mid].tile_base <= blk) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Hash -> Mod, or Bucketize, then the feature tag.
__device__ __forceinline__ long long transform_value(long long v, const FeatDev& fd,
                                                     const long long* bnd, unsigned& err) {
  unsigned long long id;
  if (fd.ops & RECIS_OP_BUCKETIZE) {
    const long long* b = bnd + fd.bnd_off;
    int lo = 0, hi = fd.nb;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (b[mid] <= v) lo = mid + 1;
      else hi = mid;
    }
    id = (unsigned long long)lo;
  } else if (fd.ops & RECIS_OP_HASH) {
    id = fmix64((unsigned long long)v);
    if (fd.ops & RECIS_OP_MOD) id %= fd.mod;
  } else if (fd.ops & RECIS_OP_MOD) {
    const long long m = (long long)fd.mod;
    long long r = v % m;
    if (r < 0) r += m;
    id = (unsigned long long)r;
  } else {
    if (v < 0) {
      err |= kErrKeyRange;
      return kBadKey;
    }
    id = (unsigned long long)v;
  }
  if (id >= (1ull << 48)) {
    err |= kErrKeyRange;
    return kBadKey;
  }
  return (long long)(((unsigned long long)fd.slot << 48) | id);
}

// --------------------------------------------------------------- k_prep
__global__ __launch_bounds__(kThreads) void k_prep(LookupLaunch L, TableDev t) {
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long nb = (long long)L.F * L.B;
  if (idx == 0) {
    *L.res.num_unique = 0;
    L.res.plan[0] = 0;  // long keys
    L.res.plan[1] = 0;  // chunks
  }
  if (idx > nb) return;
  if (idx == nb) {
    L.res.bag_offsets[nb] = (int)L.N;
    return;
  }
  const int f = (int)(idx / L.B), i = (int)(idx - (long long)f * L.B);
  const FeatDev fd = L.feats[f];
  const int o = fd.offs[i], o1 = fd.offs[i + 1];
  bool bad = o1 < o || o < 0 || (long long)o1 > fd.n;
  if (i == 0 && o != 0) bad = true;
  if (i == L.B - 1 && (long long)o1 != fd.n) bad = true;
  if (bad) atomicOr(&t.ctr->error, kErrInvalid);
  const long long oc = o < 0 ? 0 : ((long long)o > fd.n ? fd.n : o);
  L.res.bag_offsets[idx] = (int)(fd.base + oc);
}

// -------------------------------------------------------------- k_dedup
// A block takes kOccTile occurrences of one feature.  Their keys are first
// deduplicated in an LDS table (64-bit CAS in LDS), which also gives each
// occurrence its rank among the block's equal keys; only then does each
// distinct key of the block touch the call's global dedup table -- one probe,
// at most one CAS and one count atomic per block, instead of one per
// occurrence, so the hot keys of a Zipf feature do not serialise thousands
// of atomics on one address.  Each thread issues the global accesses of all
// its entries together, so a phase costs one round trip.
constexpr int kDistPerThread = kOccTile / kThreads;  // list entries a thread resolves

__global__ __launch_bounds__(kThreads) void k_dedup(LookupLaunch L, TableDev t) {
  __shared__ unsigned long long s_key[kLdsTab];  // block's distinct keys; then their dedup slots
  __shared__ int s_cnt[kLdsTab];                 // occurrences in the block; then the rank base
  __shared__ unsigned short s_list[kOccTile];    // entries of s_key in use
  __shared__ int s_nd, s_new;
  __shared__ long long s_ubase;
  __shared__ unsigned s_err;
  const int tid = threadIdx.x;
  const long long blk = blockIdx.x;
  const FeatDev fd = L.feats[find_feature(L.feats, L.F, blk)];
  const long long j0 = (blk - fd.tile_base) * kOccTile;
  for (int i = tid; i < kLdsTab; i += kThreads) {
    s_key[i] = (unsigned long long)kEmptyKey;
    s_cnt[i] = 0;
  }
  if (tid == 0) {
    s_nd = 0;
    s_new = 0;
    s_err = 0;
  }
  long long keyv[kOccPerThread];
  bool valid[kOccPerThread];
  unsigned err = 0;
  // values, all loads issued together; then the transform
#pragma unroll
  for (int k = 0; k < kOccPerThread; ++k) {
    const long long j = j0 + tid + (long long)k * kThreads;
    valid[k] = j < fd.n;
    keyv[k] = valid[k] ? fd.values[j] : 0;
  }
#pragma unroll
  for (int k = 0; k < kOccPerThread; ++k)
    if (valid[k]) keyv[k] = transform_value(keyv[k], fd, L.bnd_pool, err);
  if (err) atomicOr(&s_err, err);
  __syncthreads();  // LDS table initialised
  // block-local dedup: entry and rank of each occurrence
  unsigned short ent[kOccPerThread];
  int rank[kOccPerThread];
#pragma unroll
  for (int k = 0; k < kOccPerThread; ++k) {
    ent[k] = 0;
    rank[k] = 0;
    if (!valid[k]) continue;
    const unsigned long long key = (unsigned long long)keyv[k];
    unsigned h = (unsigned)((key * 0x9E3779B97F4A7C15ull) >> (64 - kLdsTabBits));
    while (true) {
      const unsigned long long o = atomicCAS(&s_key[h], (unsigned long long)kEmptyKey, key);
      if (o == (unsigned long long)kEmptyKey) {
        s_list[atomicAdd(&s_nd, 1)] = (unsigned short)h;
        break;
      }
      if (o == key) break;
      h = (h + 1) & (kLdsTab - 1);
    }
    ent[k] = (unsigned short)h;
    rank[k] = atomicAdd(&s_cnt[h], 1);
  }
  __syncthreads();
  // the block's distinct keys against the global dedup table
  const int nd = s_nd;
  int hh[kDistPerThread];
  unsigned long long key[kDistPerThread], p[kDistPerThread];
  long long cur[kDistPerThread];
#pragma unroll
  for (int m = 0; m < kDistPerThread; ++m) {
    const int i = tid + m * kThreads;
    hh[m] = i < nd ? (int)s_list[i] : -1;
    key[m] = hh[m] >= 0 ? s_key[hh[m]] : 0;
    p[m] = (key[m] * 0x9E3779B97F4A7C15ull) >> L.dd_shift;
    cur[m] = hh[m] >= 0 ? L.dd[p[m]].key : 0;  // a stale empty is settled by the CAS
  }
  long long old[kDistPerThread];
#pragma unroll
  for (int m = 0; m < kDistPerThread; ++m) {
    old[m] = 0;
    if (hh[m] >= 0 && cur[m] == kEmptyKey)
      old[m] = (long long)atomicCAS((unsigned long long*)&L.dd[p[m]].key, (unsigned long long)kEmptyKey, key[m]);
  }
  bool won[kDistPerThread];
#pragma unroll
  for (int m = 0; m < kDistPerThread; ++m) {
    won[m] = false;
    if (hh[m] < 0) continue;
    const long long kv = (long long)key[m];
    if (cur[m] == kv) continue;
    if (cur[m] == kEmptyKey) {
      if (old[m] == kEmptyKey) {
        won[m] = true;
        continue;
      }
      if (old[m] == kv) continue;
    }
    // the first slot holds another key: linear probing (the table has twice
    // as many slots as the call has occurrences, so this is uncommon)
    unsigned long long q = (p[m] + 1) & L.dd_mask;
    while (true) {
      const long long c = L.dd[q].key;
      if (c == kv) break;
      if (c == kEmptyKey) {
        const long long o = (long long)atomicCAS((unsigned long long*)&L.dd[q].key,
                                                 (unsigned long long)kEmptyKey, (unsigned long long)kv);
        if (o == kEmptyKey) {
          won[m] = true;
          break;
        }
        if (o == kv) break;
      }
      q = (q + 1) & L.dd_mask;
    }
    p[m] = q;
  }
  int base[kDistPerThread], nidx[kDistPerThread];
#pragma unroll
  for (int m = 0; m < kDistPerThread; ++m) {
    base[m] = 0;
    nidx[m] = -1;
    if (hh[m] < 0) continue;
    base[m] = atomicAdd(&L.dd[p[m]].count, s_cnt[hh[m]]);  // base of this block's ranks
    if (won[m]) nidx[m] = atomicAdd(&s_new, 1);
  }
  __syncthreads();
  if (tid == 0) {
    if (s_new > 0)
      s_ubase = (long long)atomicAdd((unsigned long long*)L.res.num_unique, (unsigned long long)s_new);
    if (s_err) atomicOr(&t.ctr->error, s_err);
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kDistPerThread; ++m) {
    if (hh[m] < 0) continue;
    if (nidx[m] >= 0) {
      const long long u = s_ubase + nidx[m];
      L.dd[p[m]].uidx = (int)u;
      L.res.unique_keys[u] = (long long)key[m];
      L.uslot[u] = (int)p[m];
    }
    s_key[hh[m]] = p[m];
    s_cnt[hh[m]] = base[m];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kOccPerThread; ++k) {
    if (!valid[k]) continue;
    const long long gj = fd.base + j0 + tid + (long long)k * kThreads;
    L.occ_slot[gj] = (int)s_key[ent[k]];
    L.occ_rank[gj] = s_cnt[ent[k]] + rank[k];
  }
}

// ---------------------------------------------------------- k_key_probe
// One distinct key per thread.  The first probe loads the whole 16-byte slot,
// so a hit costs one dependent access after the key itself.
__global__ __launch_bounds__(kThreads) void k_key_probe(LookupLaunch L, TableDev t) {
  __shared__ unsigned s_ins;
  __shared__ unsigned s_err;
  const long long U = *L.res.num_unique;
  const long long t0 = (long long)blockIdx.x * kKeyTile;
  if (t0 >= U) {
    if (threadIdx.x == 0) L.blk_sums[blockIdx.x] = 0;
    return;
  }
  if (threadIdx.x == 0) {
    s_ins = 0;
    s_err = 0;
  }
  __syncthreads();
  const bool find_only = (L.flags & RECIS_FIND_ONLY) != 0;
  unsigned* idslot = reinterpret_cast<unsigned*>(L.res.plan + plan_layout(L.res.capacity).o_idslot);
  unsigned long long acc = 0;
  unsigned ins = 0, err = 0;
  const long long u = t0 + threadIdx.x;
  if (u < U) {
    const long long key = L.res.unique_keys[u];
    const int us = L.uslot[u];
    const int c = L.dd[us].count;
    L.res.counts[u] = c;
    long long row = -1;
    unsigned sl = 0xFFFFFFFFu;
    int need = 0;
    if (key >= 0) {
      unsigned long long p = slot_of(key, t.slot_shift);
      Slot s = t.slots[p];
      bool found = false, inserted = false;
      for (unsigned long long n = 0; n <= t.slot_mask; ++n) {
        if (n > 0) s = t.slots[p];
        if (s.key == key) {
          found = true;
          break;
        }
        if (s.key == kEmptyKey) {
          if (find_only) break;
          const long long o = (long long)atomicCAS((unsigned long long*)&t.slots[p].key,
                                                   (unsigned long long)kEmptyKey, (unsigned long long)key);
          if (o == kEmptyKey) {
            inserted = true;
            break;
          }
          if (o == key) {  // not expected: keys are distinct within a call
            s = t.slots[p];
            found = true;
            break;
          }
        }
        p = (p + 1) & t.slot_mask;
      }
      if (!found && !inserted) {
        if (!find_only) err |= kErrCapacity;
      } else if (find_only) {
        row = s.row;
        sl = (unsigned)p;
      } else {
        const unsigned c0 = inserted ? 0u : s.count;
        const unsigned long long cs = (unsigned long long)c0 + (unsigned)c;
        const unsigned cnt = cs > 0xFFFFFFFFull ? 0xFFFFFFFFu : (unsigned)cs;
        t.slots[p].count = cnt;
        const int r = inserted ? -1 : s.row;
        if (r < 0 && cnt >= t.admit) need = 1;
        else row = r;
        sl = (unsigned)p;
        ins = inserted ? 1u : 0u;
      }
    }
    // a pending row is reported with the fresh mark (its values may still be
    // the initializer's); -2 marks a key that needs a row from this call
    if (row >= 0 && (row & kPendingRow)) row = (row & ~(long long)kPendingRow) | kFreshRow;
    L.res.unique_rows[u] = need ? -2 : row;
    idslot[u] = sl;
    acc = ((unsigned long long)need << 32) | (unsigned)c;
  }
  if (ins) atomicAdd(&s_ins, ins);
  if (err) atomicOr(&s_err, err);
  unsigned long long total;
  block_exclusive_scan(acc, &total);
  if (threadIdx.x == 0) {
    L.blk_sums[blockIdx.x] = total;
    if (s_ins) atomicAdd(&t.ctr->num_keys, (unsigned long long)s_ins);
    if (s_err) atomicOr(&t.ctr->error, s_err);
  }
}

// ----------------------------------------------------------- k_key_scan
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void k_key_scan(LookupLaunch L, TableDev t) {
  __shared__ unsigned long long s_w[kScanThreads / 64];
  const long long U = *L.res.num_unique;
  const long long nblk = (U + kKeyTile - 1) / kKeyTile;
  const long long per = (nblk + kScanThreads - 1) / kScanThreads;
  const long long b0 = (long long)threadIdx.x * per;
  unsigned long long sum = 0;
  for (long long b = b0; b < b0 + per && b < nblk; ++b) sum += L.blk_sums[b];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  unsigned long long x = sum;
  for (int d = 1; d < 64; d <<= 1) {
    unsigned long long y = (unsigned long long)shfl64((long long)x, lane >= d ? lane - d : lane);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_w[wid] = x;
  __syncthreads();
  unsigned long long before = 0, all = 0;
  for (int w = 0; w < kScanThreads / 64; ++w) {
    if (w < wid) before += s_w[w];
    all += s_w[w];
  }
  unsigned long long run = before + x - sum;
  for (long long b = b0; b < b0 + per && b < nblk; ++b) {
    const unsigned long long v = L.blk_sums[b];
    L.blk_sums[b] = run;
    run += v;
  }
  if (threadIdx.x == 0) {
    const long long R = (long long)(all >> 32);
    const long long Fr = t.ctr->free_top > 0 ? t.ctr->free_top : 0;
    const long long take = R < Fr ? R : Fr;
    const long long base = (long long)t.ctr->next_row;
    long long next = base + (R - take);
    if (next > t.rows_limit) next = base > t.rows_limit ? base : t.rows_limit;
    t.ctr->take_free = take;
    t.ctr->free_top_old = Fr;
    t.ctr->bump_base = base;
    t.ctr->free_top = Fr - take;
    t.ctr->next_row = (unsigned long long)next;
    L.res.unique_offsets[U] = (int)(all & 0xFFFFFFFFull);
  }
}

// ------------------------------------------------------- k_key_finalize
__global__ __launch_bounds__(kThreads) void k_key_finalize(LookupLaunch L, TableDev t) {
  __shared__ unsigned s_err;
  const long long U = *L.res.num_unique;
  const long long t0 = (long long)blockIdx.x * kKeyTile;
  if (t0 >= U) return;
  if (threadIdx.x == 0) s_err = 0;
  const long long u = t0 + threadIdx.x;
  const bool valid = u < U;
  int cnt = 0, us = 0;
  long long mark = -1;
  if (valid) {
    cnt = L.res.counts[u];
    mark = L.res.unique_rows[u];
    us = L.uslot[u];
  }
  const unsigned long long acc = valid ? (((unsigned long long)(mark == -2) << 32) | (unsigned)cnt) : 0ull;
  unsigned long long total;
  const unsigned long long run = block_exclusive_scan(acc, &total) + L.blk_sums[blockIdx.x];
  unsigned err = 0;
  if (valid) {
    const PlanLayout pl = plan_layout(L.res.capacity);
    int* plan = L.res.plan;
    const unsigned* idslot = reinterpret_cast<const unsigned*>(plan + pl.o_idslot);
    const long long take = t.ctr->take_free, ftop = t.ctr->free_top_old, base = t.ctr->bump_base;
    L.res.unique_offsets[u] = (int)(run & 0xFFFFFFFFull);
    long long row = mark;
    if (row == -2) {
      const long long i = (long long)(run >> 32);
      row = i < take ? (long long)t.free_list[ftop - 1 - i] : base + (i - take);
      if (row >= t.rows_limit) {
        row = -1;
        err |= kErrCapacity;
        L.res.unique_rows[u] = -1;
      } else {
        // allocated but not written: its first update materialises it
        t.slots[idslot[u]].row = (int)row | kPendingRow;
        L.res.unique_rows[u] = row | kFreshRow;
      }
    }
    if (cnt > kShortMax && row >= 0) {
      const int idx = atomicAdd(&plan[0], 1);
      const int nch = (cnt + kChunk - 1) / kChunk;
      const int cb = atomicAdd(&plan[1], nch);
      plan[pl.o_long_u + idx] = (int)u;
      plan[pl.o_long_base + idx] = cb;
      plan[pl.o_long_nch + idx] = nch;
      for (int q = 0; q < nch; ++q) plan[pl.o_chunk_owner + cb + q] = idx;
    }
    DedupSlot* d = &L.dd[us];
    d->key = kEmptyKey;
    d->count = 0;
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  if (threadIdx.x == 0 && s_err) atomicOr(&t.ctr->error, s_err);
}

// -------------------------------------------------------------- k_group
__global__ __launch_bounds__(kThreads) void k_group(LookupLaunch L, TableDev t) {
  constexpr int kLdsOff = 4096;
  __shared__ int s_off[kLdsOff];
  __shared__ int s_blo, s_bhi;
  const int tid = threadIdx.x;
  const long long blk = blockIdx.x;
  const int f = find_feature(L.feats, L.F, blk);
  const FeatDev fd = L.feats[f];
  const long long j0 = (blk - fd.tile_base) * kOccTile;
  const bool by_occ = (L.flags & RECIS_GROUP_BY_OCCURRENCE) != 0;
  const int B = L.B;
  long long* occref = reinterpret_cast<long long*>(L.res.plan + plan_layout(L.res.capacity).o_occref);
  if (!by_occ) {
    if (tid < 2) {
      // bag containing occurrence j: the last i with offs[i] <= j, clamped to [0, B)
      const long long j = tid == 0 ? j0 : ((j0 + kOccTile < fd.n ? j0 + kOccTile : fd.n) - 1);
      int lo = 0, hi = B;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((long long)fd.offs[mid] <= j) lo = mid + 1;
        else hi = mid;
      }
      int b = lo - 1;
      b = b < 0 ? 0 : (b > B - 1 ? B - 1 : b);
      if (tid == 0) s_blo = b;
      else s_bhi = b;
    }
    __syncthreads();
    const int cnt = s_bhi - s_blo + 2;
    if (cnt <= kLdsOff && cnt > 0)
      for (int i = tid; i < cnt; i += kThreads) s_off[i] = fd.offs[s_blo + i];
    __syncthreads();
  }
  // phase 1: this thread's occurrences (coalesced)
  int p[kOccPerThread], rk[kOccPerThread];
#pragma unroll
  for (int k = 0; k < kOccPerThread; ++k) {
    const long long j = j0 + tid + (long long)k * kThreads;
    p[k] = -1;
    if (j < fd.n) {
      p[k] = L.occ_slot[fd.base + j];
      rk[k] = L.occ_rank[fd.base + j];
    }
  }
  // phase 2: distinct-key index of each
  int u[kOccPerThread];
#pragma unroll
  for (int k = 0; k < kOccPerThread; ++k) u[k] = p[k] >= 0 ? L.dd[p[k]].uidx : 0;
  // phase 3: group offset, row and key of each distinct key
  int uo[kOccPerThread];
  long long r[kOccPerThread], key[kOccPerThread];
#pragma unroll
  for (int k = 0; k < kOccPerThread; ++k) {
    if (p[k] < 0) continue;
    uo[k] = L.res.unique_offsets[u[k]];
    r[k] = L.res.unique_rows[u[k]];
    key[k] = L.res.unique_keys[u[k]];
  }
  // phase 4: outputs
#pragma unroll
  for (int k = 0; k < kOccPerThread; ++k) {
    if (p[k] < 0) continue;
    const long long j = j0 + tid + (long long)k * kThreads;
    const long long gj = fd.base + j;
    int gval;
    if (by_occ) {
      gval = (int)gj;
    } else {
      const int blo = s_blo, cnt = s_bhi - s_blo + 2;
      int lo, hi;
      if (cnt <= kLdsOff && cnt > 0) {
        lo = 0;
        hi = cnt - 1;  // search offsets[blo .. bhi]
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((long long)s_off[mid] <= j) lo = mid + 1;
          else hi = mid;
        }
        lo += blo;
      } else {
        lo = 0;
        hi = B;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((long long)fd.offs[mid] <= j) lo = mid + 1;
          else hi = mid;
        }
      }
      int i = lo - 1;
      i = i < 0 ? 0 : (i > B - 1 ? B - 1 : i);
      gval = f * B + i;
    }
    L.res.inverse[gj] = u[k];
    L.res.grouped[uo[k] + rk[k]] = gval;
    occref[gj] = r[k] < 0 ? kOccNoRow
                          : ((r[k] & kFreshRow) ? (long long)(kOccPendingBit | (unsigned long long)key[k]) : r[k]);
  }
}

}  // namespace

void launch_lookup(const LookupLaunch& L, const TableDev& t, hipStream_t s) {
  const long long nb = (long long)L.F * L.B + 1;
  hipLaunchKernelGGL(k_prep, dim3((unsigned)((nb + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                     L, t);
  if (L.N > 0) {
    hipLaunchKernelGGL(k_dedup, dim3((unsigned)L.occ_tiles), dim3(kThreads), 0, s, L, t);
    hipLaunchKernelGGL(k_key_probe, dim3((unsigned)L.key_tiles), dim3(kThreads), 0, s, L, t);
  }
  hipLaunchKernelGGL(k_key_scan, dim3(1), dim3(kScanThreads), 0, s, L, t);
  if (L.N > 0) {
    hipLaunchKernelGGL(k_key_finalize, dim3((unsigned)L.key_tiles), dim3(kThreads), 0, s, L, t);
    hipLaunchKernelGGL(k_group, dim3((unsigned)L.occ_tiles), dim3(kThreads), 0, s, L, t);
  }
}

}  // namespace recis
