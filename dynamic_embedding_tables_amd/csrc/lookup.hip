// lookup.hip -- insert_find: fused transform + dedup, IDMap probe / insert,
// row allocation and initialisation, and the per-key grouping of occurrences.
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
//   k_dedup     per occurrence: transform + tag, insert into the call's dedup
//               table; per-block LDS aggregation gives each occurrence its rank
//               among equal keys with one global atomic per distinct key per
//               block (hot keys never serialise on one address)
//   k_key_probe per distinct key: IDMap probe / CAS insert, count, admission
//               decision; block sums of (occurrences, rows to allocate)
//   k_key_scan  one block: exclusive scan of the block sums; rows come from
//               the free list first, then from the bump pointer -- by prefix
//               sum, not by atomics
//   k_key_finalize  per distinct key: group offsets, row assignment, backward
//               plan for long keys, row initialisation (wave-cooperative),
//               dedup-table reset
//   k_group     per occurrence: inverse index and the grouped bag / occurrence
//               list used by the backward reduction
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
__global__ __launch_bounds__(kThreads) void k_dedup(LookupLaunch L, TableDev t) {
  __shared__ int s_pos[kLdsTab];
  __shared__ int s_cnt[kLdsTab];
  __shared__ int s_new;
  __shared__ long long s_ubase;
  __shared__ unsigned s_err;
  const int tid = threadIdx.x;
  const long long blk = blockIdx.x;
  const FeatDev fd = L.feats[find_feature(L.feats, L.F, blk)];
  const long long j0 = (blk - fd.tile_base) * kOccTile;
  for (int i = tid; i < kLdsTab; i += kThreads) {
    s_pos[i] = -1;
    s_cnt[i] = 0;
  }
  if (tid == 0) {
    s_new = 0;
    s_err = 0;
  }
  __syncthreads();

  int pos[kOccPerThread], ent[kOccPerThread], rank[kOccPerThread], nidx[kOccPerThread];
  long long keyv[kOccPerThread];
  unsigned err = 0;
#pragma unroll
  for (int k = 0; k < kOccPerThread; ++k) {
    const long long j = j0 + tid + (long long)k * kThreads;
    pos[k] = -1;
    nidx[k] = -1;
    keyv[k] = 0;
    ent[k] = 0;
    rank[k] = 0;
    if (j < fd.n) {
      const long long key = transform_value(fd.values[j], fd, L.bnd_pool, err);
      keyv[k] = key;
      unsigned long long p = ((unsigned long long)key * 0x9E3779B97F4A7C15ull) >> L.dd_shift;
      bool won = false;
      while (true) {
        const long long cur = L.dd[p].key;  // a stale empty is settled by the CAS
        if (cur == key) break;
        if (cur == kEmptyKey) {
          const long long old = (long long)atomicCAS((unsigned long long*)&L.dd[p].key,
                                                     (unsigned long long)kEmptyKey,
                                                     (unsigned long long)key);
          if (old == kEmptyKey) {
            won = true;
            break;
          }
          if (old == key) break;
        }
        p = (p + 1) & L.dd_mask;
      }
      pos[k] = (int)p;
      unsigned h = ((unsigned)p * 2654435761u) >> 20;  // 12 bits: kLdsTab = 4096
      while (true) {
        const int old = atomicCAS(&s_pos[h], -1, (int)p);
        if (old == -1 || old == (int)p) break;
        h = (h + 1) & (kLdsTab - 1);
      }
      ent[k] = (int)h;
      rank[k] = atomicAdd(&s_cnt[h], 1);
      if (won) nidx[k] = atomicAdd(&s_new, 1);
    }
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  for (int i = tid; i < kLdsTab; i += kThreads) {
    const int p = s_pos[i];
    if (p >= 0) s_cnt[i] = atomicAdd(&L.dd[p].count, s_cnt[i]);  // base of this block's ranks
  }
  if (tid == 0) {
    if (s_new > 0)
      s_ubase = (long long)atomicAdd((unsigned long long*)L.res.num_unique, (unsigned long long)s_new);
    if (s_err) atomicOr(&t.ctr->error, s_err);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kOccPerThread; ++k) {
    if (pos[k] < 0) continue;
    const long long gj = fd.base + j0 + tid + (long long)k * kThreads;
    L.occ_slot[gj] = pos[k];
    L.occ_rank[gj] = s_cnt[ent[k]] + rank[k];
    if (nidx[k] >= 0) {
      const long long u = s_ubase + nidx[k];
      L.dd[pos[k]].uidx = (int)u;
      L.res.unique_keys[u] = keyv[k];
      L.uslot[u] = pos[k];
    }
  }
}

// ---------------------------------------------------------- k_key_probe
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
  unsigned long long acc = 0;
  unsigned ins = 0, err = 0;
  for (int k = 0; k < kKeyPerThread; ++k) {
    const long long u = t0 + (long long)threadIdx.x * kKeyPerThread + k;
    if (u >= U) break;
    const long long key = L.res.unique_keys[u];
    const int c = L.dd[L.uslot[u]].count;
    L.res.counts[u] = c;
    long long row = -1;
    unsigned sl = 0xFFFFFFFFu;
    int need = 0;
    if (key >= 0) {
      unsigned long long p = slot_of(key, t.slot_shift);
      bool found = false, inserted = false;
      for (unsigned long long n = 0; n <= t.slot_mask; ++n) {
        const long long cur = t.slots[p].key;
        if (cur == key) {
          found = true;
          break;
        }
        if (cur == kEmptyKey) {
          if (find_only) break;
          const long long old = (long long)atomicCAS((unsigned long long*)&t.slots[p].key,
                                                     (unsigned long long)kEmptyKey,
                                                     (unsigned long long)key);
          if (old == kEmptyKey) {
            inserted = true;
            break;
          }
          if (old == key) {
            found = true;
            break;
          }
        }
        p = (p + 1) & t.slot_mask;
      }
      if (!found && !inserted) {
        if (!find_only) err |= kErrCapacity;
      } else if (find_only) {
        row = t.slots[p].row;
      } else {
        const unsigned c0 = inserted ? 0u : t.slots[p].count;
        const unsigned long long cs = (unsigned long long)c0 + (unsigned)c;
        const unsigned cnt = cs > 0xFFFFFFFFull ? 0xFFFFFFFFu : (unsigned)cs;
        t.slots[p].count = cnt;
        const int r = inserted ? -1 : t.slots[p].row;
        if (r < 0 && cnt >= t.admit) need = 1;
        else row = r;
        sl = (unsigned)p;
        ins += inserted ? 1u : 0u;
      }
    }
    L.res.unique_rows[u] = need ? -2 : row;
    L.idslot[u] = sl;
    acc += ((unsigned long long)need << 32) | (unsigned)c;
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
__device__ void init_row(const TableDev& t, long long r, long long key, int lane) {
  char* rp = row_ptr(t.rs, r);
  const int pbytes = t.dim * (t.dtype == RECIS_DTYPE_BF16 ? 2 : 4);
  const int chunks = (int)(t.rs.stride >> 4);
  for (int c = lane; c < chunks; c += 64) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (c * 16 < pbytes) {
      if (t.dtype == RECIS_DTYPE_BF16) {
        const float4 a = init4(t.seed, key, 2u * c, t.init_scale);
        const float4 b = init4(t.seed, key, 2u * c + 1u, t.init_scale);
        v.x = (unsigned)f32_to_bf16(a.x) | ((unsigned)f32_to_bf16(a.y) << 16);
        v.y = (unsigned)f32_to_bf16(a.z) | ((unsigned)f32_to_bf16(a.w) << 16);
        v.z = (unsigned)f32_to_bf16(b.x) | ((unsigned)f32_to_bf16(b.y) << 16);
        v.w = (unsigned)f32_to_bf16(b.z) | ((unsigned)f32_to_bf16(b.w) << 16);
      } else {
        const float4 a = init4(t.seed, key, (unsigned)c, t.init_scale);
        v = make_uint4(__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z),
                       __float_as_uint(a.w));
      }
    }
    reinterpret_cast<uint4*>(rp)[c] = v;
  }
}

__global__ __launch_bounds__(kThreads) void k_key_finalize(LookupLaunch L, TableDev t) {
  __shared__ unsigned s_err;
  const long long U = *L.res.num_unique;
  const long long t0 = (long long)blockIdx.x * kKeyTile;
  if (t0 >= U) return;
  if (threadIdx.x == 0) s_err = 0;
  const int lane = threadIdx.x & 63;
  int cnt[kKeyPerThread];
  long long mark[kKeyPerThread];
  unsigned long long acc = 0;
  for (int k = 0; k < kKeyPerThread; ++k) {
    const long long u = t0 + (long long)threadIdx.x * kKeyPerThread + k;
    cnt[k] = 0;
    mark[k] = -1;
    if (u < U) {
      cnt[k] = L.res.counts[u];
      mark[k] = L.res.unique_rows[u];
      acc += ((unsigned long long)(mark[k] == -2) << 32) | (unsigned)cnt[k];
    }
  }
  unsigned long long total;
  unsigned long long run = block_exclusive_scan(acc, &total) + L.blk_sums[blockIdx.x];
  const long long take = t.ctr->take_free, ftop = t.ctr->free_top_old, base = t.ctr->bump_base;
  const PlanLayout pl = plan_layout(L.res.capacity);
  int* plan = L.res.plan;
  unsigned err = 0;
  long long newrow[kKeyPerThread], keyv[kKeyPerThread];
  for (int k = 0; k < kKeyPerThread; ++k) {
    const long long u = t0 + (long long)threadIdx.x * kKeyPerThread + k;
    newrow[k] = -1;
    keyv[k] = 0;
    if (u >= U) continue;
    L.res.unique_offsets[u] = (int)(run & 0xFFFFFFFFull);
    long long row = mark[k];
    if (row == -2) {
      const long long i = (long long)(run >> 32);
      row = i < take ? (long long)t.free_list[ftop - 1 - i] : base + (i - take);
      if (row >= t.rows_limit) {
        row = -1;
        err |= kErrCapacity;
      } else {
        t.slots[L.idslot[u]].row = (int)row;
        newrow[k] = row;
        keyv[k] = L.res.unique_keys[u];
      }
      L.res.unique_rows[u] = row;
    }
    run += ((unsigned long long)(mark[k] == -2) << 32) | (unsigned)cnt[k];
    if (cnt[k] > kShortMax && row >= 0) {
      const int idx = atomicAdd(&plan[0], 1);
      const int nch = (cnt[k] + kChunk - 1) / kChunk;
      const int cb = atomicAdd(&plan[1], nch);
      plan[pl.o_long_u + idx] = (int)u;
      plan[pl.o_long_base + idx] = cb;
      plan[pl.o_long_nch + idx] = nch;
      plan[pl.o_long_done + idx] = 0;
      for (int q = 0; q < nch; ++q) plan[pl.o_chunk_owner + cb + q] = idx;
    }
    DedupSlot* d = &L.dd[L.uslot[u]];
    d->key = kEmptyKey;
    d->count = 0;
  }
  // initialise the new rows, one row per pass of the whole wave
  for (int k = 0; k < kKeyPerThread; ++k) {
    unsigned long long m = __ballot(newrow[k] >= 0);
    while (m) {
      const int src = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const long long r = shfl64(newrow[k], src);
      const long long key = shfl64(keyv[k], src);
      init_row(t, r, key, lane);
    }
  }
  if (err) {
    atomicOr(&s_err, err);
  }
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
  for (int k = 0; k < kOccPerThread; ++k) {
    const long long j = j0 + tid + (long long)k * kThreads;
    if (j >= fd.n) break;
    const long long gj = fd.base + j;
    const int p = L.occ_slot[gj];
    const int u = L.dd[p].uidx;
    L.res.inverse[gj] = u;
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
    L.res.grouped[L.res.unique_offsets[u] + L.occ_rank[gj]] = gval;
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
