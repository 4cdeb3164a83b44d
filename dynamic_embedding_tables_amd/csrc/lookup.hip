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
//   k_tile      transform + tag every occurrence and deduplicate each tile of
//               kTileOcc consecutive occurrences in LDS: the tile's distinct
//               keys with their counts (its pairs), each occurrence's index
//               among them, and per partition block a histogram of the
//               pairs' hash buckets (the top bits of the key's hash)
//   k_part_colscan / k_scan_small / k_pair_scatter
//               the pairs partitioned by hash bucket (one radix-sort pass);
//               the column scan also cuts heavy buckets into slices
//   k_bucket    one bucket per block, twice around a scan of the per-bucket
//               distinct counts and occurrences: dedup of the bucket's pairs
//               in LDS, counts (summed over the pairs), distinct-key indices,
//               group offsets; in the second launch also the IDMap probe /
//               insert of every distinct key (count, admission decision,
//               without global atomics: the block owns the bucket's IDMap
//               regions), then for each pair its distinct-key index, forward
//               reference and span of its key's group, at the pair's slot
//               (a bucket that overflows the LDS table, from colliding inputs,
//               uses a global one; a heavy bucket is counted slice by slice
//               and its pairs are resolved by k_key_scan's other blocks)
//   k_key_scan  block 0: exclusive scan of the per-bucket sums; rows come
//               from the free list first, then from the bump pointer -- by
//               prefix sum, not by atomics
//   k_key_finalize  per bucket: row assignment (the new row is marked
//               pending, not written: its values are the initializer's until
//               its first update), backward plan for long keys
//   k_occ_tile  per tile: every occurrence's inverse index, forward reference
//               and grouped entry, from its pair's resolved record
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

// Block-wide exclusive scan of one uint64 per thread of an NT-thread block;
// returns the prefix and writes the block total to *total.
template <int NT = kThreads>
__device__ unsigned long long block_exclusive_scan(unsigned long long v, unsigned long long* total) {
  __shared__ unsigned long long s_w[NT / 64];
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
  for (int w = 0; w < NT / 64; ++w) {
    if (w < wid) before += s_w[w];
    all += s_w[w];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// Adds 1 to a[h] for every lane with `act`, returning the value a[h] had
// before this lane's add (lanes of one index get consecutive values).  The
// index of the first active lane is served by one atomic for all the lanes
// that share it: a hot key fills most lanes of a wave, and thousands of LDS
// atomics on one address would queue.  Call with the whole wave converged.
__device__ __forceinline__ int lds_add1(int* a, unsigned h, bool act) {
  const unsigned long long am = __ballot(act);
  int res = 0;
  if (am) {
    const int lead = __ffsll((long long)am) - 1;
    const unsigned hl = (unsigned)__builtin_amdgcn_readlane((int)h, lead);
    const unsigned long long same = __ballot(act && h == hl);
    if (__popcll(same) > 1) {
      int base = 0;
      if ((int)(threadIdx.x & 63) == lead) base = atomicAdd(&a[hl], __popcll(same));
      base = __builtin_amdgcn_readlane(base, lead);
      if (act && h == hl) {
        res = base + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(same >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((unsigned)same, 0u));
        act = false;
      }
    }
  }
  if (act) res = atomicAdd(&a[h], 1);
  return res;
}

// x mod d with inv = floor((2^64 - 1) / d): the quotient estimate
// floor(x * inv / 2^64) is at most 2 below floor(x / d), so at most two
// subtractions finish the remainder (division by an invariant integer through
// multiplication, after Granlund and Montgomery).  A generic 64-bit
// remainder is a long instruction sequence on this GPU.
__device__ __forceinline__ unsigned long long mod_by(unsigned long long x, unsigned long long d,
                                                    unsigned long long inv) {
  const unsigned long long q = __umul64hi(x, inv);
  unsigned long long r = x - q * d;
  if (r >= d) r -= d;
  if (r >= d) r -= d;
  return r;
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
    if (fd.ops & RECIS_OP_MOD) id = mod_by(id, fd.mod, fd.mod_inv);
  } else if (fd.ops & RECIS_OP_MOD) {
    // the floor remainder in [0, mod) (mod <= 2^63 - 1 here): a negative v
    // through -(v + 1), which cannot overflow
    id = v >= 0 ? mod_by((unsigned long long)v, fd.mod, fd.mod_inv)
                : fd.mod - 1 - mod_by((unsigned long long)(-(v + 1)), fd.mod, fd.mod_inv);
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
  if (L.hot_ok && idx < L.F) {  // F <= kFeatBins <= the grid here (B >= 1 when N > 0)
    L.res.plan[plan_layout(L.res.capacity).o_fbin + idx] = (int)(L.feats[idx].slot & (kFeatBins - 1));
  }
  if (idx == 0) {
    *L.res.num_unique = 0;
    L.res.plan[0] = 0;  // long keys
    L.res.plan[1] = 0;  // chunks
    L.res.plan[kPlanHotOk] = L.hot_ok;
    L.hslice[0] = 0;    // heavy slices (listed by k_part_colscan)
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
  // the tiles whose first occurrence falls in this bag (a bag is rarely
  // longer than a tile): with valid offsets every tile gets exactly one
  const long long oc1 = o1 < 0 ? 0 : ((long long)o1 > fd.n ? fd.n : o1);
  const long long m0 = fd.base + oc, m1 = fd.base + oc1;
  for (long long tl = (m0 + kTileOcc - 1) / kTileOcc; tl * kTileOcc < m1; ++tl) L.tile_bag[tl] = (int)idx;
}

// ------------------------------------------------------ hash partition
// The call's tile-distinct keys (pairs) are partitioned by the top bits of
// their key's Fibonacci hash into nbk buckets (see part_geom), like one pass
// of a radix sort: k_tile counts per (partition block, bucket), the column
// scan and a small scan turn the counts into positions, and k_pair_scatter
// writes every pair to its bucket's range.  Each bucket is then
// deduplicated by one block entirely in LDS (k_bucket), so the dedup needs
// no global atomics at all: on this GPU those are performed at the memory
// side and would bound the step.
__device__ __forceinline__ unsigned long long fib_mix(long long key) {
  return (unsigned long long)key * 0x9E3779B97F4A7C15ull;
}
__device__ __forceinline__ int bucket_of(long long key, int bits) {
  return bits == 0 ? 0 : (int)(fib_mix(key) >> (64 - bits));
}

// Feature of merged occurrence j (F small: a scan of the bases).
__device__ __forceinline__ int feature_of(const FeatDev* feats, int F, long long j) {
  int lo = 0, hi = F - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (feats[mid].base <= j) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Key of merged occurrence j; the feature descriptor is cached across calls
// of one thread (its occurrences rarely change feature).
struct FeatCursor {
  FeatDev fd;
  long long lo = 1, hi = 0;  // [lo, hi) of the cached feature
};
__device__ __forceinline__ void cursor_to(const LookupLaunch& L, FeatCursor& c, long long j) {
  if (j < c.lo || j >= c.hi) {
    c.fd = L.feats[feature_of(L.feats, L.F, j)];
    c.lo = c.fd.base;
    c.hi = c.fd.base + c.fd.n;
  }
}

// First-level dedup, one tile of kTileOcc consecutive occurrences at a time
// (a partition block takes tiles_per_block of them): transform + tag every
// occurrence, deduplicate the tile in an LDS table, note each occurrence's
// index among the tile's distinct keys, and write the tile's distinct keys
// with their counts (its pairs) from the tile's start in tkey / tcnt.  The
// block's histogram counts pairs per hash bucket.  Skewed inputs repeat
// keys within a tile (0.27 pairs per occurrence on the capacity workload),
// so everything up to the last pass handles pairs, not occurrences.
__global__ __launch_bounds__(kPartThreads) void k_tile(LookupLaunch L, TableDev t) {
  constexpr int kPer = kTileOcc / kPartThreads;
  __shared__ long long s_key[kTileTab];
  __shared__ int s_cnt[kTileTab];
  __shared__ unsigned short s_idx[kTileTab];
  __shared__ unsigned short s_list[kTileOcc];
  __shared__ int s_h[kMaxBuckets];
  __shared__ int s_nd;
  __shared__ unsigned s_err;
  const int tid = threadIdx.x;
  const int pb = xcd_block((int)blockIdx.x, (int)gridDim.x);  // partition block
  const long long t0 = (long long)pb * L.tiles_per_block;
  const long long t1 = t0 + L.tiles_per_block < L.ntiles ? t0 + L.tiles_per_block : L.ntiles;
  for (int b = tid; b < L.nbk; b += kPartThreads) s_h[b] = 0;
  if (tid == 0) s_err = 0;
  // The raw IDs of the next tile are loaded while this one is deduplicated:
  // the addresses first (the feature cursor may have to wait for a feature's
  // descriptor), then the loads together, so that each thread has all of
  // them in flight at once.  fl follows the loads, fu the transforms.
  FeatCursor fl, fu;
  unsigned err = 0;
  long long nraw[kPer];
  auto load_tile = [&](long long tl) {
    const long long a0 = tl * kTileOcc;
    const long long a1 = a0 + kTileOcc < L.N ? a0 + kTileOcc : L.N;
    const long long* src[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const long long j = a0 + tid + (long long)k * kPartThreads;
      src[k] = nullptr;
      if (j < a1) {
        cursor_to(L, fl, j);
        src[k] = fl.fd.values + (j - fl.fd.base);
      }
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) nraw[k] = src[k] ? *gread<long long>(src[k]) : 0;
  };
  if (t0 < t1) load_tile(t0);
  for (long long tile = t0; tile < t1; ++tile) {
    for (int i = tid; i < kTileTab; i += kPartThreads) {
      s_key[i] = kEmptyKey;
      s_cnt[i] = 0;
    }
    if (tid == 0) s_nd = 0;
    __syncthreads();
    const long long j0 = tile * kTileOcc;
    const long long j1 = j0 + kTileOcc < L.N ? j0 + kTileOcc : L.N;
    long long raw[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) raw[k] = nraw[k];
    long long key[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const long long j = j0 + tid + (long long)k * kPartThreads;
      key[k] = 0;
      if (j < j1) {
        cursor_to(L, fu, j);
        key[k] = transform_value(raw[k], fu.fd, L.bnd_pool, err);
      }
    }
    // after the transforms: the wait at the end of a cursor update would
    // otherwise wait for these loads too
    if (tile + 1 < t1) load_tile(tile + 1);
    unsigned h[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const bool act = j0 + tid + (long long)k * kPartThreads < j1;
      h[k] = 0;
      if (act) {
        unsigned q = (unsigned)(fib_mix(key[k]) >> 32) & (kTileTab - 1);
        while (true) {  // at most kTileOcc keys in kTileTab slots: a free slot is always found
          const long long o = (long long)atomicCAS((unsigned long long*)&s_key[q], (unsigned long long)kEmptyKey,
                                                   (unsigned long long)key[k]);
          if (o == kEmptyKey) {
            const int l = atomicAdd(&s_nd, 1);
            s_list[l] = (unsigned short)q;
            s_idx[q] = (unsigned short)l;
            break;
          }
          if (o == key[k]) break;
          q = (q + 1) & (kTileTab - 1);
        }
        h[k] = q;
      }
      lds_add1(s_cnt, h[k], act);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const long long j = j0 + tid + (long long)k * kPartThreads;
      if (j < j1) L.occ_local[j] = s_idx[h[k]];
    }
    const int nd = s_nd;
    for (int l = tid; l < nd; l += kPartThreads) {
      const int q = s_list[l];
      const long long kk = s_key[q];
      L.tkey[j0 + l] = kk;
      L.tcnt[j0 + l] = s_cnt[q];
      atomicAdd(&s_h[bucket_of(kk, L.nbits)], 1);
    }
    if (tid == 0) L.tile_n[tile] = nd;
    __syncthreads();  // the next tile reuses the table
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  int* row = L.hist + (long long)pb * L.nbk;
  for (int b = tid; b < L.nbk; b += kPartThreads) row[b] = s_h[b];
  if (tid == 0 && s_err) atomicOr(&t.ctr->error, s_err);
}

// Per bucket, the exclusive prefix of its counts over the partition blocks
// (in place) and its total.  A block takes 64 buckets (one per lane); its 16
// waves split the partition blocks.
__global__ __launch_bounds__(kPartThreads) void k_part_colscan(LookupLaunch L) {
  __shared__ int s_part[kPartThreads / 64][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int W = kPartThreads / 64;
  const int b = blockIdx.x * 64 + lane;
  const int G = L.part_blocks;
  const int per = (G + W - 1) / W;
  const int g0 = w * per, g1 = g0 + per < G ? g0 + per : G;
  int sum = 0;
  if (b < L.nbk)
    for (int g = g0; g < g1; ++g) sum += L.hist[(long long)g * L.nbk + b];
  s_part[w][lane] = sum;
  __syncthreads();
  int run = 0, all = 0;
#pragma unroll
  for (int x = 0; x < W; ++x) {
    run += x < w ? s_part[x][lane] : 0;
    all += s_part[x][lane];
  }
  if (b < L.nbk) {
    for (int g = g0; g < g1; ++g) {
      int* p = L.hist + (long long)g * L.nbk + b;
      const int v = *p;
      *p = run;
      run += v;
    }
  }
  if (w == 0) {
    int ns = 0, e0 = 0;
    if (b < L.nbk) {
      L.bbase[b] = all;  // total, scanned by k_scan_small
      L.ubase[b] = 0;    // a light bucket's block writes these, a heavy one's slices add to them
      L.obase[b] = 0;
      if (all > kHeavyOcc) {  // a heavy bucket: its slices (few buckets, so one atomic each)
        ns = (all + kSliceOcc - 1) / kSliceOcc;
        e0 = atomicAdd(&L.hslice[0], ns);
      }
    }
    // the wave lists each heavy bucket's slices together (a hot key's bucket
    // has hundreds)
    unsigned long long hv = __ballot(ns > 0);
    while (hv) {
      const int l = __ffsll((long long)hv) - 1;
      hv &= hv - 1;
      const int nsl = __shfl(ns, l), e0l = __shfl(e0, l), bl = __shfl(b, l);
      for (int q = lane; q < nsl; q += 64) {
        L.hslice[1 + 2 * (e0l + q)] = bl;
        L.hslice[2 + 2 * (e0l + q)] = q;
      }
    }
  }
}

// In-place exclusive scan of a[0..n) (n <= kMaxBuckets), a[n] = total, and
// the total also to *total_ll when given.  Bucket positions (bbase), and the
// distinct-key and occurrence bases of the buckets (ubase, obase: the second
// array, scanned by the same launch).  Both arrays' loads are issued before
// either scan, so the launch waits for memory once.
constexpr int kSmallPer = kMaxBuckets / kPartThreads;  // n <= kMaxBuckets
__device__ void scan_small(int* a, const int (&v)[kSmallPer], int n, long long* total_ll);
__global__ __launch_bounds__(kPartThreads) void k_scan_small(int* a, int* a2, int n, long long* total_ll) {
  const int b0 = threadIdx.x * kSmallPer;
  const int* src2 = a2 ? a2 : a;  // without a second array: a second read of a, unused
  int v[kSmallPer], v2[kSmallPer];
#pragma unroll
  for (int k = 0; k < kSmallPer; ++k) {  // from indices clamped into range: no load in a branch of its own
    const int i = b0 + k < n ? b0 + k : 0;
    v[k] = a[i];
    v2[k] = src2[i];
  }
#pragma unroll
  for (int k = 0; k < kSmallPer; ++k) {
    v[k] = b0 + k < n ? v[k] : 0;
    v2[k] = b0 + k < n ? v2[k] : 0;
  }
  scan_small(a, v, n, total_ll);
  if (a2) {
    __syncthreads();
    scan_small(a2, v2, n, nullptr);
  }
}
__device__ void scan_small(int* a, const int (&v)[kSmallPer], int n, long long* total_ll) {
  constexpr int kPer = kSmallPer;
  __shared__ int s_w[kPartThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b0 = tid * kPer;
  int sum = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) sum += v[k];
  int x = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl(x, lane >= d ? lane - d : lane);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_w[w] = x;
  __syncthreads();
  int run = x - sum, all = 0;
#pragma unroll
  for (int q = 0; q < kPartThreads / 64; ++q) {
    run += q < w ? s_w[q] : 0;
    all += s_w[q];
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (b0 + k < n) a[b0 + k] = run;
    run += v[k];
  }
  if (tid == 0) {
    a[n] = all;
    if (total_ll) *total_ll = all;
  }
}

// Every pair of the block's tiles to its bucket's range (the same partition
// block as in k_tile; the blocks of one XCD write neighbouring records of
// every bucket).
__global__ __launch_bounds__(kPartThreads) void k_pair_scatter(LookupLaunch L) {
  constexpr int kPer = kTileOcc / kPartThreads;
  __shared__ int s_h[kMaxBuckets];
  const int tid = threadIdx.x;
  const int pb = xcd_block((int)blockIdx.x, (int)gridDim.x);
  const long long t0 = (long long)pb * L.tiles_per_block;
  const long long t1 = t0 + L.tiles_per_block < L.ntiles ? t0 + L.tiles_per_block : L.ntiles;
  const int* row = L.hist + (long long)pb * L.nbk;
  for (int b = tid; b < L.nbk; b += kPartThreads) s_h[b] = L.bbase[b] + row[b];
  __syncthreads();
  for (long long tile = t0; tile < t1; ++tile) {
    const int nd = L.tile_n[tile];
    const long long p0 = tile * kTileOcc;
    long long key[kPer];
    int w[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int l = tid + k * kPartThreads;
      key[k] = l < nd ? L.tkey[p0 + l] : 0;
      w[k] = l < nd ? L.tcnt[p0 + l] : 0;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int l = tid + k * kPartThreads;
      if (l >= nd) continue;
      const int pos = atomicAdd(&s_h[bucket_of(key[k], L.nbits)], 1);
      PartEntry e;
      e.key = key[k];
      e.pid = (int)(p0 + l);
      e.w = w[k];
      L.part[pos] = e;
    }
  }
}

// ------------------------------------------------ IDMap probe / insert
struct ProbeOut {
  long long row = -1;   // the key's row (pending rows with kFreshRow), or -1
  unsigned sl = 0xFFFFFFFFu;
  int need = 0;         // no row yet and the count reached the admission threshold
  int ins = 0;          // inserted by this call
  unsigned err = 0;
};

// One distinct key with `c` occurrences in this call: probe its region of the
// IDMap; on a miss (unless find_only) take an empty slot that claim(p) grants
// this thread, and write the slot whole; add c to its count (saturating).  The
// caller's block owns the key's region, so the slot stores need no atomics.
template <typename Claim>
__device__ __forceinline__ ProbeOut idmap_probe(const TableDev& t, long long key, int c, bool find_only,
                                                Claim claim, bool sketching = false) {
  ProbeOut o;
  if (key < 0) return o;  // a failed transform
  // count-min admission: an absent key enters only once its estimate (all of
  // this call's counts are in the sketch already) reaches the threshold, and
  // then with the estimate as its count
  unsigned est = 0;
  if (sketching) est = sketch_estimate(t, key);
  const bool admit_absent = !sketching || est >= t.admit;
  unsigned long long p = slot_of(key, t.slot_shift);
  bool found = false, inserted = false, stop = false;
  Slot sv;
  // kProbeBatch consecutive slots per round trip, examined in probe order: at
  // the table's load a linear probe ends within the first few slots, so one
  // round trip usually settles the key instead of one per slot
  constexpr int kProbeBatch = 4;
  for (unsigned long long n = 0; n <= t.region_mask && !stop; n += kProbeBatch) {
    unsigned long long q[kProbeBatch];
    Slot v[kProbeBatch];
    q[0] = p;
#pragma unroll
    for (int k = 1; k < kProbeBatch; ++k) q[k] = next_slot(t, q[k - 1]);
#pragma unroll
    for (int k = 0; k < kProbeBatch; ++k) v[k] = t.slots[q[k]];
#pragma unroll
    for (int k = 0; k < kProbeBatch; ++k) {
      if (stop) continue;
      if (n + k > t.region_mask) {  // the whole region seen
        stop = true;
        continue;
      }
      if (v[k].key == key) {
        found = stop = true;
        p = q[k];
        sv = v[k];
      } else if (v[k].key == kEmptyKey) {
        if (find_only || !admit_absent) {
          stop = true;
        } else if (claim(q[k])) {
          inserted = stop = true;
          p = q[k];
        }
      }
    }
    p = stop ? p : next_slot(t, q[kProbeBatch - 1]);
  }
  if (!found && !inserted) {
    if (!find_only && admit_absent) o.err = kErrCapacity;  // the key's region is full
    return o;  // (or a key the sketch does not admit yet: no slot, no row)
  }
  o.sl = (unsigned)p;
  if (find_only) {
    o.row = sv.row;
  } else {
    const unsigned c0 = inserted ? 0u : sv.count;
    const unsigned long long cs = (unsigned long long)c0 + (inserted && sketching ? est : (unsigned)c);
    const unsigned cnt = cs > 0xFFFFFFFFull ? 0xFFFFFFFFu : (unsigned)cs;
    if (inserted) {
      Slot ns;
      ns.key = key;
      ns.row = -1;
      ns.count = cnt;
      t.slots[p] = ns;
    } else {
      t.slots[p].count = cnt;
    }
    const int r = inserted ? -1 : sv.row;
    if (r < 0 && cnt >= t.admit) o.need = 1;
    else o.row = r;
    o.ins = inserted ? 1 : 0;
  }
  // a pending row is reported with the fresh mark (its values may still be
  // the initializer's)
  if (o.row >= 0 && (o.row & kPendingRow)) o.row = (o.row & ~(long long)kPendingRow) | kFreshRow;
  return o;
}

// Count-min admission, phase 1 (the count launch): a distinct key of the
// call that is not in the IDMap adds its c occurrences to its counters.
__device__ __forceinline__ void sketch_count(const TableDev& t, long long key, int c) {
  if (key < 0 || c <= 0) return;
  const ProbeOut o = idmap_probe(t, key, 0, true, [](unsigned long long) { return false; });
  if (o.sl == 0xFFFFFFFFu) sketch_add(t, key, (unsigned)c);
}

// The forward's reference for the occurrences of a key (see kOccNoRow).
__device__ __forceinline__ long long occ_ref(const TableDev& t, const ProbeOut& o, long long key) {
  if (o.need || (o.row >= 0 && (o.row & kFreshRow))) return (long long)(kOccPendingBit | (unsigned long long)key);
  if (o.row < 0) return kOccNoRow;
  return (long long)row_ptr(t.rs, o.row);
}

// Per-key outputs of the probe, and its share of the bucket's sums: rows to
// allocate << 32 | keys inserted, and long keys << 32 | their chunks.
__device__ __forceinline__ void key_outputs(const LookupLaunch& L, long long u, int c, const ProbeOut& o,
                                            unsigned long long& sum, unsigned long long& sum_long) {
  unsigned* idslot = reinterpret_cast<unsigned*>(L.res.plan + plan_layout(L.res.capacity).o_idslot);
  L.res.unique_rows[u] = o.need ? -2 : o.row;  // -2: needs a row from this call
  idslot[u] = o.sl;
  // the key's last use (tables that keep it; counting calls only)
  if (L.last_use && o.sl != 0xFFFFFFFFu) L.last_use[o.sl] = L.step;
  sum += ((unsigned long long)o.need << 32) | (unsigned)o.ins;
  // a key with more than kShortMax occurrences is reduced in chunks by the
  // backward (also one without a row now: a later lookup may give it one
  // before this lookup's backward runs, which then re-probes its keys)
  if (c > kShortMax) sum_long += (1ull << 32) | (unsigned)long_chunks(c);
}

// A bucket whose distinct keys overflow the LDS table (only inputs built to
// collide in the hash's top bits get here) is done by its block with an
// open-addressing table in global memory -- the bucket's own region of the
// dedup table, 2 slots per occurrence -- and atomics.  Slow but bounded.
// COUNT inserts the bucket's keys and counts them (the distinct count goes to
// ubase[b]); EMIT (after the scan) writes the distinct keys' outputs and the
// occurrences' grouped entries and resolved records, then empties the
// region again.
__device__ __forceinline__ long long ld_key(const DedupSlot* d) {
  return (long long)__hip_atomic_load(reinterpret_cast<const unsigned long long*>(&d->key), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_int(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_int(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reference of an occurrence of distinct key u from its final row entry.
__device__ __forceinline__ long long ref_of_row(const TableDev& t, long long v, long long key) {
  if (v == -2 || (v >= 0 && (v & kFreshRow))) return (long long)(kOccPendingBit | (unsigned long long)key);
  if (v < 0) return kOccNoRow;
  return (long long)row_ptr(t.rs, v);
}

// The resolved pair `pid` (tile * kTileOcc + its index among the tile's
// distinct keys): written at its pair slot, so that k_occ_tile reads a
// tile's resolved pairs contiguously.
__device__ __forceinline__ void put_out(const LookupLaunch& L, int pid, long long ref, int u, int gpos) {
  PartOut o;
  o.ref = ref;
  o.u = u;
  o.gpos = gpos;
  L.pout[pid] = o;
}

template <bool EMIT, int NT>
__device__ void bucket_global(const LookupLaunch& L, const TableDev& t, int b, int& s_nd, int& s_cursor,
                              unsigned long long& s_sum, unsigned long long& s_sum_long,
                              unsigned long long& s_claims) {
  const int tid = threadIdx.x;
  const int s = L.bbase[b], m = L.bbase[b + 1] - s;
  DedupSlot* R = L.dd + 2ll * s;
  const unsigned long long cap = 2ull * (unsigned long long)m;
  __syncthreads();
  if (tid == 0) {
    s_nd = 0;
    s_cursor = 0;
    s_sum = 0;
    s_sum_long = 0;
    s_claims = 0;
  }
  __syncthreads();
  if (!EMIT) {
    int wsum = 0;  // the bucket's occurrences
    for (int i = tid; i < m; i += NT) {
      const PartEntry e = L.part[s + i];
      const long long key = e.key;
      wsum += e.w;
      unsigned long long h = (fib_mix(key) >> 20) % cap;
      while (true) {
        const long long c = ld_key(&R[h]);
        if (c == key) break;
        if (c == kEmptyKey) {
          const long long o = (long long)atomicCAS((unsigned long long*)&R[h].key, (unsigned long long)kEmptyKey,
                                                   (unsigned long long)key);
          if (o == kEmptyKey || o == key) break;
        }
        h = h + 1 == cap ? 0 : h + 1;
      }
      atomicAdd(&R[h].count, e.w);
    }
    atomicAdd(&s_cursor, wsum);
    __syncthreads();
    for (unsigned long long h = tid; h < cap; h += NT) {
      const long long key = ld_key(&R[h]);
      if (key == kEmptyKey) continue;
      atomicAdd(&s_nd, 1);
      if (L.sketching) sketch_count(t, key, ld_int(&R[h].count));
    }
    __syncthreads();
    if (tid == 0) {
      L.ubase[b] = s_nd;
      L.obase[b] = s_cursor;
    }
    return;
  }
  const long long ub = L.ubase[b];
  const int ob = L.obase[b];  // the bucket's first grouped position
  const bool find_only = (L.flags & RECIS_FIND_ONLY) != 0;
  unsigned long long sum = 0, sum_long = 0, claims = 0;
  unsigned err = 0;
  for (unsigned long long h = tid; h < cap; h += NT) {
    const long long key = ld_key(&R[h]);
    if (key == kEmptyKey) continue;
    const long long u = ub + atomicAdd(&s_nd, 1);
    const int c = ld_int(&R[h].count);
    const int o = atomicAdd(&s_cursor, c);
    L.res.unique_keys[u] = key;
    L.res.counts[u] = c;
    st_int(&L.res.unique_offsets[u], ob + o);
    st_int(&R[h].uidx, (int)u);
    // an empty IDMap slot goes to whichever thread's CAS takes it
    auto claim = [&](unsigned long long q) {
      const bool won = atomicCAS((unsigned long long*)&t.slots[q].key, (unsigned long long)kEmptyKey,
                                 (unsigned long long)key) == (unsigned long long)kEmptyKey;
      claims += (1ull << 32) | (won ? 0u : 1u);
      return won;
    };
    const ProbeOut po = idmap_probe(t, key, c, find_only, claim, L.sketching != 0);
    err |= po.err;
    key_outputs(L, u, c, po, sum, sum_long);
  }
  if (err) atomicOr(&t.ctr->error, err);
  if (sum) atomicAdd(&s_sum, sum);
  if (sum_long) atomicAdd(&s_sum_long, sum_long);
  if (claims) atomicAdd(&s_claims, claims);
  __syncthreads();
  if (tid == 0) {
    L.blk_sums[b] = s_sum;
    L.blk_long[b] = s_sum_long;
    L.blk_claim[b] = s_claims;
  }
  for (int i = tid; i < m; i += NT) {
    const PartEntry e = L.part[s + i];
    unsigned long long h = (fib_mix(e.key) >> 20) % cap;
    while (ld_key(&R[h]) != e.key) h = h + 1 == cap ? 0 : h + 1;
    const int u = ld_int(&R[h].uidx);
    const int pos = atomicSub(&R[h].count, e.w) - e.w;  // the group is filled from its end
    const long long v = (long long)__hip_atomic_load(reinterpret_cast<unsigned long long*>(&L.res.unique_rows[u]),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    put_out(L, e.pid, ref_of_row(t, v, e.key), u, ld_int(&L.res.unique_offsets[u]) + pos);
  }
  __syncthreads();
  for (unsigned long long h = tid; h < cap; h += NT) {
    R[h].key = kEmptyKey;
    R[h].count = 0;
  }
}

// Heavy buckets (more than kHeavyOcc occurrences: a hot key's bucket).  One
// block would take the whole bucket, so it is cut into slices of kSliceOcc,
// each deduplicated in LDS by its own block; the slices meet in the bucket's
// region of the dedup table (2 slots per occurrence):
//  - COUNT, per slice: each of the slice's distinct keys is added to the
//    region with its count; the slice whose CAS enters a key lists it (the
//    next index of the bucket's distinct count -> klist);
//  - EMIT, one block per bucket: the listed keys in list order get their
//    index, group offset (a block scan of their counts) and IDMap probe /
//    insert (empty slots taken by CAS: the bucket's keys are spread over
//    its block and the slices);
//  - k_bucket_occ, per slice: each distinct key reserves its slice's span of
//    the key's group (one atomic per key and slice), then every occurrence
//    takes a position in it;
//  - k_key_finalize empties the region again.
// Only the keys that many slices share (the hot ones) meet in global atomics,
// once per slice.

// Region probe of a heavy bucket's dedup table: the slot of `key` (entered
// by the count pass), or cap if it is not there (never: bounded all the same).
__device__ __forceinline__ unsigned long long dd_find(const DedupSlot* R, unsigned long long cap, long long key) {
  unsigned long long h = (fib_mix(key) >> 20) % cap;
  for (unsigned long long n = 0; n < cap; ++n) {
    if (R[h].key == key) return h;
    h = h + 1 == cap ? 0 : h + 1;
  }
  return cap;
}

// The slice [s0, s1) of a heavy bucket into the LDS table: its distinct keys
// (s_list) with their counts in the slice.
template <int TAB, int NT>
__device__ __forceinline__ void slice_dedup(const LookupLaunch& L, int s0, int s1, int hs, long long* s_key,
                                            int* s_cnt, unsigned short* s_list, int& s_nd) {
  const int tid = threadIdx.x;
  for (int i0 = s0; i0 < s1; i0 += NT) {
    const int i = i0 + tid;
    const bool act = i < s1;
    unsigned h = 0;
    int w = 0;
    if (act) {
      const PartEntry e = L.part[i];
      const long long key = e.key;
      w = e.w;
      h = (unsigned)(fib_mix(key) >> hs) & (TAB - 1);
      while (true) {  // a slice has fewer distinct keys than the table has free slots
        const long long o = (long long)atomicCAS((unsigned long long*)&s_key[h], (unsigned long long)kEmptyKey,
                                                 (unsigned long long)key);
        if (o == kEmptyKey) {
          s_list[atomicAdd(&s_nd, 1)] = (unsigned short)h;
          break;
        }
        if (o == key) break;
        h = (h + 1) & (TAB - 1);
      }
    }
    if (act) atomicAdd(&s_cnt[h], w);
  }
}

// Block size of the bucket kernels when the buckets average more than
// kSmallTabOcc occurrences (the 2048-entry table).  More threads put more of a bucket's IDMap probes in
// flight at once; 512 measured faster than 256 and 1024 on the capacity
// workload (1024: registers allow one block per CU).
constexpr int kBigBucketThreads = 512;

// One bucket per block, in two launches around a scan of the per-bucket
// distinct counts (so the distinct keys get dense indices without a global
// counter, which thousands of blocks would serialise on).  Both launches
// deduplicate the bucket in an LDS table of TAB entries (at most 3/4 full; a
// bucket with more distinct keys takes bucket_global instead).  COUNT writes
// the bucket's distinct count.  EMIT writes the distinct keys (index
// ubase[b] + their order in the table), counts and group offsets inside the
// bucket's range; probes the IDMap for each of them -- the block owns every
// IDMap region of its bucket, so empty slots are shared out through an LDS
// set instead of global atomics -- and writes its row and the bucket's sums
// (rows to allocate, keys inserted, long keys, chunks); then every
// occurrence's grouped-list entry, and its distinct-key index and forward
// reference at the pair's slot.
// COUNT's grid has the heavy slices after the buckets; a heavy bucket's own
// block skips COUNT and does EMIT's key pass (see above).
template <int TAB, bool EMIT, int NT>
__global__ __launch_bounds__(NT) void k_bucket(LookupLaunch L, TableDev t) {
  constexpr int kMaxDistinct = TAB / 4 * 3;
  constexpr int kTabBits = TAB == 1024 ? 10 : (TAB == 2048 ? 11 : 0);
  static_assert(kTabBits > 0, "TAB is 1024 or 2048");
  static_assert(kSliceOcc <= kMaxDistinct, "a slice fits the LDS table");
  __shared__ long long s_key[TAB];
  __shared__ int s_cnt[TAB];
  __shared__ int s_u[EMIT ? TAB : 1];
  __shared__ long long s_ref[EMIT ? TAB : 1];
  __shared__ unsigned s_claim[EMIT ? TAB : 1];  // IDMap slots taken by this block (~0u: free)
  __shared__ unsigned short s_list[kMaxDistinct];
  __shared__ int s_nd, s_over, s_cursor;
  __shared__ unsigned long long s_sum, s_sum_long, s_claims;
  __shared__ unsigned s_err;
  const int tid = threadIdx.x;
  // the bits below the bucket bits index the table
  const int hs = 64 - L.nbits - kTabBits;
  if (!EMIT && (int)blockIdx.x >= L.nbk) {  // heavy slices, a share of them per block
    const int H = L.hslice[0], nsb = (int)gridDim.x - L.nbk;
    for (int e = (int)blockIdx.x - L.nbk; e < H; e += nsb) {
    const int b = L.hslice[1 + 2 * e], k = L.hslice[2 + 2 * e];
    const int s = L.bbase[b], m = L.bbase[b + 1] - s;
    const int s0 = s + k * kSliceOcc, s1 = s0 + kSliceOcc < s + m ? s0 + kSliceOcc : s + m;
    for (int i = tid; i < TAB; i += NT) {
      s_key[i] = kEmptyKey;
      s_cnt[i] = 0;
    }
    if (tid == 0) s_nd = 0;
    __syncthreads();
    slice_dedup<TAB, NT>(L, s0, s1, hs, s_key, s_cnt, s_list, s_nd);
    if (tid == 0) s_cursor = 0;
    __syncthreads();
    DedupSlot* R = L.dd + 2ll * s;
    const unsigned long long cap = 2ull * (unsigned long long)m;
    for (int idx = tid; idx < s_nd; idx += NT) {
      const int hl = s_list[idx];
      const long long key = s_key[hl];
      atomicAdd(&s_cursor, s_cnt[hl]);  // the slice's occurrences
      unsigned long long h = (fib_mix(key) >> 20) % cap;
      while (true) {
        const long long c = ld_key(&R[h]);
        if (c == key) break;
        if (c == kEmptyKey) {
          const long long o = (long long)atomicCAS((unsigned long long*)&R[h].key, (unsigned long long)kEmptyKey,
                                                   (unsigned long long)key);
          if (o == kEmptyKey) {
            const int lidx = atomicAdd(&L.ubase[b], 1);
            st_int(&R[h].uidx, lidx);
            L.klist[s + lidx] = (int)h;
            break;
          }
          if (o == key) break;
        }
        h = h + 1 == cap ? 0 : h + 1;
      }
      atomicAdd(&R[h].count, s_cnt[hl]);
      if (L.sketching) sketch_count(t, key, s_cnt[hl]);
    }
    __syncthreads();  // the LDS table is reused by the next slice
    if (tid == 0) atomicAdd(&L.obase[b], s_cursor);
    }
    return;
  }
  const int b = blockIdx.x;
  const int s = L.bbase[b], m = L.bbase[b + 1] - s;
  if (m == 0) {
    if (tid == 0) {
      if (!EMIT) L.ubase[b] = L.obase[b] = 0;
      else L.blk_sums[b] = L.blk_long[b] = L.blk_claim[b] = 0;
    }
    return;
  }
  if (m > kHeavyOcc) {
    if (!EMIT) return;  // its slices count it
    // EMIT's key pass of a heavy bucket: the listed keys in list order
    const long long ub = L.ubase[b], nd = L.ubase[b + 1] - ub;
    const int ob = L.obase[b];
    const DedupSlot* R = L.dd + 2ll * s;
    const bool find_only = (L.flags & RECIS_FIND_ONLY) != 0;
    unsigned long long sum = 0, sum_long = 0, run = 0, claims = 0;
    unsigned err = 0;
    if (tid == 0) {
      s_sum = 0;
      s_sum_long = 0;
      s_claims = 0;
      s_err = 0;
    }
    __syncthreads();
    for (long long c0 = 0; c0 < nd; c0 += NT) {
      const long long idx = c0 + tid;
      const bool valid = idx < nd;
      long long key = 0;
      int c = 0;
      if (valid) {
        const int h = L.klist[s + idx];
        key = R[h].key;
        c = R[h].count;
      }
      unsigned long long tot;
      const long long o = (long long)(block_exclusive_scan<NT>((unsigned long long)c, &tot) + run);
      run += tot;
      if (!valid) continue;
      const long long u = ub + idx;
      L.res.unique_keys[u] = key;
      L.res.counts[u] = c;
      L.res.unique_offsets[u] = (int)(ob + o);
      // an empty IDMap slot goes to whichever thread's CAS takes it
      auto claim = [&](unsigned long long q) {
        const bool won = atomicCAS((unsigned long long*)&t.slots[q].key, (unsigned long long)kEmptyKey,
                                   (unsigned long long)key) == (unsigned long long)kEmptyKey;
        claims += (1ull << 32) | (won ? 0u : 1u);
        return won;
      };
      const ProbeOut po = idmap_probe(t, key, c, find_only, claim, L.sketching != 0);
      err |= po.err;
      key_outputs(L, u, c, po, sum, sum_long);
    }
    if (err) atomicOr(&s_err, err);
    if (sum) atomicAdd(&s_sum, sum);
    if (sum_long) atomicAdd(&s_sum_long, sum_long);
    if (claims) atomicAdd(&s_claims, claims);
    __syncthreads();
    if (tid == 0) {
      L.blk_sums[b] = s_sum;
      L.blk_long[b] = s_sum_long;
      L.blk_claim[b] = s_claims;
      if (s_err) atomicOr(&t.ctr->error, s_err);
    }
    return;
  }
  for (int i = tid; i < TAB; i += NT) {
    s_key[i] = kEmptyKey;
    s_cnt[i] = 0;
    if (EMIT) s_claim[i] = ~0u;
  }
  if (tid == 0) {
    s_nd = 0;
    s_over = 0;
    s_cursor = 0;
    s_sum = 0;
    s_sum_long = 0;
    s_claims = 0;
    s_err = 0;
  }
  // EMIT: the bucket's first distinct-key index and grouped position, loaded
  // now so that they arrive during the dedup
  long long ub_pre = 0;
  int ob_pre = 0;
  if (EMIT) {
    ub_pre = L.ubase[b];
    ob_pre = L.obase[b];
  }
  // a bucket that one pass of the block covers keeps each pair's table slot
  // and weight in registers for EMIT's last pass
  const bool one_pass = m <= NT * kBucketPer;
  unsigned hk[kBucketPer];
  int wk[kBucketPer], pk[kBucketPer];
  __syncthreads();
  for (int i0 = 0; i0 < m; i0 += NT * kBucketPer) {
    long long key[kBucketPer];
    int w[kBucketPer], pid[kBucketPer];
#pragma unroll
    for (int k = 0; k < kBucketPer; ++k) {
      const int i = i0 + tid + k * NT;
      PartEntry e;
      e.key = 0;
      e.pid = 0;
      e.w = 0;
      if (i < m) e = L.part[s + i];
      key[k] = e.key;
      w[k] = e.w;
      pid[k] = e.pid;
    }
#pragma unroll
    for (int k = 0; k < kBucketPer; ++k) {
      const bool act = i0 + tid + k * NT < m;
      unsigned h = 0;
      bool counted = false;
      if (act) {
        h = (unsigned)(fib_mix(key[k]) >> hs) & (TAB - 1);
        int steps = 0;
        while (true) {
          const long long o = (long long)atomicCAS((unsigned long long*)&s_key[h], (unsigned long long)kEmptyKey,
                                                   (unsigned long long)key[k]);
          if (o == kEmptyKey) {
            const int idx = atomicAdd(&s_nd, 1);
            if (idx < kMaxDistinct) s_list[idx] = (unsigned short)h;
            else s_over = 1;
            break;
          }
          if (o == key[k]) break;
          h = (h + 1) & (TAB - 1);
          if (++steps == TAB) {  // full: only after the distinct limit was passed
            s_over = 1;
            break;
          }
        }
        counted = steps < TAB;
      }
      if (counted) atomicAdd(&s_cnt[h], w[k]);
      hk[k] = h;
      wk[k] = act ? w[k] : 0;
      pk[k] = pid[k];
    }
  }
  __syncthreads();
  if (s_over) {  // rare: colliding inputs only
    bucket_global<EMIT, NT>(L, t, b, s_nd, s_cursor, s_sum, s_sum_long, s_claims);
    return;
  }
  if (!EMIT) {
    for (int idx = tid; idx < s_nd; idx += NT) {
      const int c = s_cnt[s_list[idx]];
      atomicAdd(&s_cursor, c);  // the bucket's occurrences
      if (L.sketching) sketch_count(t, s_key[s_list[idx]], c);
    }
    __syncthreads();
    if (tid == 0) {
      L.ubase[b] = s_nd;
      L.obase[b] = s_cursor;
    }
    return;
  }
  const int nd = s_nd;
  const long long ub = ub_pre;
  const int ob = ob_pre;  // the bucket's first grouped position
  const bool find_only = (L.flags & RECIS_FIND_ONLY) != 0;
  // an empty IDMap slot goes to the first thread that enters it in the set
  // (slot indices are below 2^32; the last index of a 2^32-slot table, equal
  // to the set's free mark, is never handed out)
  unsigned long long claims = 0;  // attempts << 32 | lost
  auto claim = [&](unsigned long long p) {
    const unsigned v = (unsigned)p;
    if (v == ~0u) return false;
    claims += 1ull << 32;
    unsigned h = (unsigned)((p * 0x9E3779B97F4A7C15ull) >> (64 - kTabBits));
    for (int n = 0; n < TAB; ++n) {
      const unsigned o = atomicCAS(&s_claim[h], ~0u, v);
      if (o == ~0u) return true;
      if (o == v) {
        claims += 1;
        return false;
      }
      h = (h + 1) & (TAB - 1);
    }
    return false;  // not reached: fewer claims than kMaxDistinct
  };
  unsigned long long sum = 0, sum_long = 0;
  unsigned err = 0;
  for (int idx = tid; idx < nd; idx += NT) {
    const int h = s_list[idx];
    const long long u = ub + idx;
    const long long key = s_key[h];
    const int c = s_cnt[h];
    const int o = atomicAdd(&s_cursor, c);
    L.res.unique_keys[u] = key;
    L.res.counts[u] = c;
    L.res.unique_offsets[u] = ob + o;
    s_u[h] = (int)u;
    s_cnt[h] = o;  // from here on: the next free position of the key's group
    const ProbeOut po = idmap_probe(t, key, c, find_only, claim, L.sketching != 0);
    err |= po.err;
    key_outputs(L, u, c, po, sum, sum_long);
    s_ref[h] = occ_ref(t, po, key);
  }
  if (err) atomicOr(&s_err, err);
  if (sum) atomicAdd(&s_sum, sum);
  if (sum_long) atomicAdd(&s_sum_long, sum_long);
  if (claims) atomicAdd(&s_claims, claims);
  __syncthreads();
  if (tid == 0) {
    L.blk_sums[b] = s_sum;
    L.blk_long[b] = s_sum_long;
    L.blk_claim[b] = s_claims;
    if (s_err) atomicOr(&t.ctr->error, s_err);
  }
  if (one_pass) {  // the slots and weights kept from the dedup
#pragma unroll
    for (int k = 0; k < kBucketPer; ++k) {
      const bool act = tid + k * NT < m;
      const int pos = act ? atomicAdd(&s_cnt[hk[k]], wk[k]) : 0;
      if (act) put_out(L, pk[k], s_ref[hk[k]], s_u[hk[k]], ob + pos);
    }
    return;
  }
  for (int i0 = 0; i0 < m; i0 += NT * kBucketPer) {
    PartEntry e[kBucketPer];
#pragma unroll
    for (int k = 0; k < kBucketPer; ++k) {
      const int i = i0 + tid + k * NT;
      if (i < m) e[k] = L.part[s + i];
    }
#pragma unroll
    for (int k = 0; k < kBucketPer; ++k) {
      const bool act = i0 + tid + k * NT < m;
      unsigned h = 0;
      if (act) {
        h = (unsigned)(fib_mix(e[k].key) >> hs) & (TAB - 1);
        while (s_key[h] != e[k].key) h = (h + 1) & (TAB - 1);
      }
      const int pos = act ? atomicAdd(&s_cnt[h], e[k].w) : 0;
      if (act) put_out(L, e[k].pid, s_ref[h], s_u[h], ob + pos);
    }
  }
}

// The occurrences of the heavy buckets, slices e0, e0 + step, ... by one block
// of NT threads (after EMIT's key pass): a slice's distinct keys reserve their
// spans of the keys' groups, then every occurrence gets its inverse index,
// grouped-list entry and forward reference.
template <int TAB, int NT>
__device__ void heavy_occ(const LookupLaunch& L, const TableDev& t, int e0, int step) {
  constexpr int kMaxDistinct = TAB / 4 * 3;
  constexpr int kTabBits = TAB == 1024 ? 10 : (TAB == 2048 ? 11 : 0);
  __shared__ long long s_key[TAB];
  __shared__ int s_cnt[TAB];
  __shared__ int s_u[TAB];
  __shared__ long long s_ref[TAB];
  __shared__ unsigned short s_list[kMaxDistinct];
  __shared__ int s_nd;
  const int tid = threadIdx.x;
  const int H = L.hslice[0];
  const int hs = 64 - L.nbits - kTabBits;
  for (int e = e0; e < H; e += step) {
  const int b = L.hslice[1 + 2 * e], k = L.hslice[2 + 2 * e];
  const int s = L.bbase[b], m = L.bbase[b + 1] - s;
  const int s0 = s + k * kSliceOcc, s1 = s0 + kSliceOcc < s + m ? s0 + kSliceOcc : s + m;
  for (int i = tid; i < TAB; i += NT) {
    s_key[i] = kEmptyKey;
    s_cnt[i] = 0;
  }
  if (tid == 0) s_nd = 0;
  __syncthreads();
  slice_dedup<TAB, NT>(L, s0, s1, hs, s_key, s_cnt, s_list, s_nd);
  __syncthreads();
  DedupSlot* R = L.dd + 2ll * s;
  const unsigned long long cap = 2ull * (unsigned long long)m;
  const long long ub = L.ubase[b];
  for (int idx = tid; idx < s_nd; idx += NT) {
    const int hl = s_list[idx];
    const long long key = s_key[hl];
    const int lc = s_cnt[hl];
    const unsigned long long h = dd_find(R, cap, key);
    if (h == cap) {  // not reached
      atomicOr(&t.ctr->error, kErrInvalid);
      s_u[hl] = 0;
      s_ref[hl] = kOccNoRow;
      s_cnt[hl] = s;
      continue;
    }
    const long long u = ub + R[h].uidx;
    const int base = atomicSub(&R[h].count, lc) - lc;  // the group is filled from its end
    s_u[hl] = (int)u;
    s_ref[hl] = ref_of_row(t, L.res.unique_rows[u], key);
    s_cnt[hl] = L.res.unique_offsets[u] + base;  // from here on: the slice's next position
  }
  __syncthreads();
  for (int i0 = s0; i0 < s1; i0 += NT) {
    const int i = i0 + tid;
    const bool act = i < s1;
    PartEntry en;
    unsigned h = 0;
    if (act) {
      en = L.part[i];
      h = (unsigned)(fib_mix(en.key) >> hs) & (TAB - 1);
      while (s_key[h] != en.key) h = (h + 1) & (TAB - 1);
    }
    const int pos = act ? atomicAdd(&s_cnt[h], en.w) : 0;
    if (act) put_out(L, en.pid, s_ref[h], s_u[h], pos);
  }
  __syncthreads();  // the LDS table is reused by the next slice
  }
}

// ----------------------------------------------------------- k_key_scan
constexpr int kScanThreads = 1024;
// In-place exclusive scans of a[0..n) and c[0..n) (n <= kMaxBuckets) by one
// block, every load in flight at once; returns the totals.
__device__ void scan_two(unsigned long long* a, unsigned long long* c, long long n, unsigned long long* ta,
                         unsigned long long* tc) {
  constexpr int kPer = kMaxBuckets / kScanThreads;
  __shared__ unsigned long long s_w[2][kScanThreads / 64];
  const long long b0 = (long long)threadIdx.x * kPer;
  unsigned long long va[kPer], vc[kPer], sa = 0, sc = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    va[k] = b0 + k < n ? a[b0 + k] : 0ull;
    vc[k] = b0 + k < n ? c[b0 + k] : 0ull;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    sa += va[k];
    sc += vc[k];
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  unsigned long long xa = sa, xc = sc;
  for (int d = 1; d < 64; d <<= 1) {
    const unsigned long long ya = (unsigned long long)shfl64((long long)xa, lane >= d ? lane - d : lane);
    const unsigned long long yc = (unsigned long long)shfl64((long long)xc, lane >= d ? lane - d : lane);
    if (lane >= d) {
      xa += ya;
      xc += yc;
    }
  }
  if (lane == 63) {
    s_w[0][wid] = xa;
    s_w[1][wid] = xc;
  }
  __syncthreads();
  unsigned long long ra = xa - sa, rc = xc - sc, alla = 0, allc = 0;
  for (int w = 0; w < kScanThreads / 64; ++w) {
    if (w < wid) {
      ra += s_w[0][w];
      rc += s_w[1][w];
    }
    alla += s_w[0][w];
    allc += s_w[1][w];
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (b0 + k < n) {
      a[b0 + k] = ra;
      c[b0 + k] = rc;
    }
    ra += va[k];
    rc += vc[k];
  }
  *ta = alla;
  *tc = allc;
}

// One block: prefix sums of the buckets' (rows to allocate, keys inserted)
// and (long keys, chunks); the row sources of this call; the key and chunk
// counts of the backward plan.
// Its other blocks write the heavy buckets' occurrences (heavy_occ).
__global__ __launch_bounds__(kScanThreads) void k_key_scan(LookupLaunch L, TableDev t) {
  if (blockIdx.x > 0) {
    heavy_occ<1024, kScanThreads>(L, t, (int)blockIdx.x - 1, (int)gridDim.x - 1);
    return;
  }
  const int tid = threadIdx.x;
  const long long nblk = L.N > 0 ? L.nbk : 0;  // per-bucket sums
  // Loaded before the scan's own loads and kept in flight with them, so
  // that the block waits for memory once: the buckets' IDMap slot claims
  // (attempts << 32 | lost); the table's counters, a word per lane, and the
  // call's distinct-key count in the next lane; the call's pair count.  Each
  // value is a lane's own (a value every lane shared would be moved to a
  // scalar register, which waits for its load at once), from an address
  // clamped into range, outside any branch.  The scratch arrays exist for
  // any call; the values of an empty call go unused.  Nothing else writes
  // these counters during the launch: thread 0 writes them once at the end.
  constexpr int kClaimPer = kMaxBuckets / kScanThreads;
  constexpr int kCtrWords = (int)(sizeof(DevCounters) / 8);
  static_assert(sizeof(DevCounters) % 8 == 0 && kCtrWords < kScanThreads, "the counters are whole words");
  __shared__ DevCounters s_ctr;
  __shared__ long long s_u;
  __shared__ int s_pairs;
  unsigned long long cl[kClaimPer];
#pragma unroll
  for (int j = 0; j < kClaimPer; ++j) {
    const long long b = tid + (long long)j * kScanThreads;
    cl[j] = L.blk_claim[b < nblk ? b : 0];
  }
  const unsigned long long* pre_src =
      tid == kCtrWords ? reinterpret_cast<const unsigned long long*>(L.res.num_unique)
                       : reinterpret_cast<const unsigned long long*>(t.ctr) + (tid < kCtrWords ? tid : 0);
  const unsigned long long pre = *pre_src;
  const int pairs = L.bbase[tid == 0 ? L.nbk : 0];
  unsigned long long all, all_long;
  scan_two(L.blk_sums, L.blk_long, nblk, &all, &all_long);
  // the loads above are complete here: the scan waited for its own
  if (tid < kCtrWords) reinterpret_cast<unsigned long long*>(&s_ctr)[tid] = pre;
  if (tid == kCtrWords) s_u = (long long)pre;
  if (tid == 0) s_pairs = pairs;
  // the call's claims, summed over the buckets; each bucket's figures fit 32
  // bits, the call's total 64
  __shared__ unsigned long long s_cl[2];
  if (tid == 0) s_cl[0] = s_cl[1] = 0;
  __syncthreads();
  unsigned long long ca = 0, cf = 0;
#pragma unroll
  for (int j = 0; j < kClaimPer; ++j) {
    const bool in = tid + (long long)j * kScanThreads < nblk;
    ca += in ? cl[j] >> 32 : 0ull;
    cf += in ? cl[j] & 0xFFFFFFFFull : 0ull;
  }
  if (ca) atomicAdd(&s_cl[0], ca);
  if (cf) atomicAdd(&s_cl[1], cf);
  __syncthreads();
  if (tid == 0) {
    const DevCounters c = s_ctr;
    t.ctr->claim_attempts = c.claim_attempts + s_cl[0];
    t.ctr->claim_failures = c.claim_failures + s_cl[1];
    if (L.N > 0) t.ctr->lookup_pairs = c.lookup_pairs + (unsigned long long)s_pairs;
    const long long R = (long long)(all >> 32);
    const long long Fr = c.free_top > 0 ? c.free_top : 0;
    const long long take = R < Fr ? R : Fr;
    const long long base = (long long)c.next_row;
    long long next = base + (R - take);
    if (next > t.rows_limit) next = base > t.rows_limit ? base : t.rows_limit;
    t.ctr->take_free = take;
    t.ctr->free_top_old = Fr;
    t.ctr->bump_base = base;
    t.ctr->free_top = Fr - take;
    t.ctr->next_row = (unsigned long long)next;
    t.ctr->num_keys = c.num_keys + (all & 0xFFFFFFFFull);
    L.res.unique_offsets[s_u] = (int)L.N;
    L.res.plan[0] = (int)(all_long >> 32);
    L.res.plan[1] = (int)(all_long & 0xFFFFFFFFull);
  }
}

// ------------------------------------------------------- k_key_finalize
// One bucket per block: its distinct keys in index order, 256 at a time; a
// block scan ranks the keys that need a row and the long keys, on top of the
// bucket's prefix from k_key_scan.  Rows come from the free list first, then
// from the bump pointer; a new row is marked pending, not written (its values
// are the initializer's until its first update).  Long keys get their entry
// and chunks in the backward plan.
__global__ __launch_bounds__(kThreads) void k_key_finalize(LookupLaunch L, TableDev t) {
  __shared__ unsigned s_err;
  __shared__ int s_cend[kThreads], s_cidx[kThreads];
  const int b = blockIdx.x;
  const long long ub = L.ubase[b], nd = L.ubase[b + 1] - ub;
  if (nd == 0) return;
  if (threadIdx.x == 0) s_err = 0;
  const PlanLayout pl = plan_layout(L.res.capacity);
  int* plan = L.res.plan;
  const unsigned* idslot = reinterpret_cast<const unsigned*>(plan + pl.o_idslot);
  const long long take = t.ctr->take_free, ftop = t.ctr->free_top_old, base = t.ctr->bump_base;
  unsigned long long run0 = L.blk_sums[b], run0_long = L.blk_long[b];
  unsigned err = 0;
  for (long long c0 = 0; c0 < nd; c0 += kThreads) {
    const long long u = ub + c0 + threadIdx.x;
    const bool valid = c0 + threadIdx.x < nd;
    int cnt = 0;
    long long mark = -1;
    if (valid) {
      cnt = L.res.counts[u];
      mark = L.res.unique_rows[u];
    }
    const unsigned long long acc = valid ? ((unsigned long long)(mark == -2) << 32) : 0ull;
    const bool is_long = valid && cnt > kShortMax;  // as k_bucket counted it
    const int nch = long_chunks(cnt);
    const unsigned long long acc_long = is_long ? ((1ull << 32) | (unsigned long long)nch) : 0ull;
    unsigned long long total, total_long;
    const unsigned long long run = block_exclusive_scan(acc, &total) + run0;
    const unsigned long long run_long = block_exclusive_scan(acc_long, &total_long) + run0_long;
    const int chunk0 = (int)(run0_long & 0xFFFFFFFFull);
    run0 += total;
    run0_long += total_long;
    if (valid && mark == -2) {
      const long long i = (long long)(run >> 32);
      const long long row = i < take ? (long long)t.free_list[ftop - 1 - i] : base + (i - take);
      if (row >= t.rows_limit) {
        err |= kErrCapacity;
        L.res.unique_rows[u] = -1;
      } else {
        t.slots[idslot[u]].row = (int)row | kPendingRow;
        L.res.unique_rows[u] = row | kFreshRow;
      }
    }
    // a failed allocation (row -1) is skipped by the backward
    const int idx = (int)(run_long >> 32);
    const int cb = (int)(run_long & 0xFFFFFFFFull);
    if (is_long) {
      plan[pl.o_long_u + idx] = (int)u;
      plan[pl.o_long_base + idx] = cb;
      plan[pl.o_long_nch + idx] = nch;
    }
    // chunk owners: these keys' chunks are [chunk0, chunk0 + chunks), in
    // thread order; the whole block fills them (a hot key has thousands)
    const int nchunks = (int)(total_long & 0xFFFFFFFFull);
    if (nchunks > 0) {
      s_cend[threadIdx.x] = cb + (is_long ? nch : 0);
      s_cidx[threadIdx.x] = idx;
      __syncthreads();
      for (int j = threadIdx.x; j < nchunks; j += kThreads) {
        const int cj = chunk0 + j;
        int lo = 0, hi = kThreads - 1;  // the first thread whose chunks end after cj
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s_cend[mid] > cj) hi = mid;
          else lo = mid + 1;
        }
        plan[pl.o_chunk_owner + cj] = s_cidx[lo];
      }
      __syncthreads();
    }
  }
  // a heavy bucket empties its region of the dedup table (the slots it listed)
  const int s = L.bbase[b];
  if (L.bbase[b + 1] - s > kHeavyOcc) {
    DedupSlot* R = L.dd + 2ll * s;
    for (long long i = threadIdx.x; i < nd; i += kThreads) {
      const int h = L.klist[s + i];
      R[h].key = kEmptyKey;
      R[h].count = 0;
      R[h].uidx = 0;
    }
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  if (threadIdx.x == 0 && s_err) atomicOr(&t.ctr->error, s_err);
}

// Each occurrence's outputs, one tile per block.  The tile's resolved pairs
// (contiguous at the tile's pair slots) go to LDS;
// then every occurrence takes its pair's distinct-key index and forward
// reference (stored contiguously, in occurrence order) and the next place in
// its pair's span of the key's group, where its grouped entry goes: its bag
// (f * B + i, found by a binary search over the tile's window of merged bag
// offsets, kept in LDS when it fits), or the occurrence itself when grouping
// by occurrence.
constexpr int kOccThreads = 1024;
constexpr int kOccPer = kTileOcc / kOccThreads;
constexpr int kOccBagWin = 3072;  // offsets kept in LDS: two blocks per CU fit
// The tile's resolved pairs to LDS, K per thread, the loads in flight
// together.
template <int K>
__device__ __forceinline__ void occ_pairs(const LookupLaunch& L, long long j0, int nd, long long* s_ref, int* s_u,
                                          int* s_g) {
  const int tid = threadIdx.x;
  const int lastl = nd > 0 ? nd - 1 : 0;
  PartOut o[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int l = tid + k * kOccThreads;
    o[k] = L.pout[j0 + (l < nd ? l : lastl)];
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int l = tid + k * kOccThreads;
    if (l < nd) {
      s_ref[l] = o[k].ref;
      s_u[l] = o[k].u;
      s_g[l] = o[k].gpos;
    }
  }
}
__global__ __launch_bounds__(kOccThreads) void k_occ_tile(LookupLaunch L) {
  __shared__ long long s_ref[kTileOcc];
  __shared__ int s_u[kTileOcc];
  __shared__ int s_g[kTileOcc];
  __shared__ int s_off[kOccBagWin];
  const int tid = threadIdx.x;
  const long long tile = blockIdx.x;
  const long long j0 = tile * kTileOcc;
  const long long j1 = j0 + kTileOcc < L.N ? j0 + kTileOcc : L.N;
  const int nd = L.tile_n[tile];
  const bool by_occ = (L.flags & RECIS_GROUP_BY_OCCURRENCE) != 0;
  const int* off = L.res.bag_offsets;  // merged, F * B + 1 entries
  const int nbags = L.F * L.B;
  // Loads in as few round trips as their dependences allow, each from an
  // index clamped into the tile (a tile has at least one pair and one
  // occurrence) so that none sits in a branch of its own, where the copy
  // out of it would wait for it at once.  The pairs take only as many
  // passes of the block as the tile has pairs for (a uniform choice).
  int loc[kOccPer];
#pragma unroll
  for (int k = 0; k < kOccPer; ++k) {
    const long long j = j0 + tid + k * kOccThreads;
    loc[k] = (int)L.occ_local[j < j1 ? j : j1 - 1];
  }
  const int passes = (nd + kOccThreads - 1) / kOccThreads;
  if (passes <= 1) occ_pairs<1>(L, j0, nd, s_ref, s_u, s_g);
  else if (passes == 2) occ_pairs<2>(L, j0, nd, s_ref, s_u, s_g);
  else occ_pairs<kOccPer>(L, j0, nd, s_ref, s_u, s_g);
  // the bags of the tile's occurrences: from the bag of its first occurrence
  // to that of the next tile's first (k_prep's table), their offsets to LDS
  // when they fit (a tile spans few bags unless most of them are empty).
  // Invalid offsets (reported by k_prep) may leave entries of an earlier
  // call: clamped, they keep every access in bounds.
  int blo = 0, wn = 0;
  if (!by_occ) {
    int b0 = L.tile_bag[tile];
    int b1 = tile + 1 < L.ntiles ? L.tile_bag[tile + 1] : nbags - 1;
    b0 = b0 < 0 ? 0 : (b0 > nbags - 1 ? nbags - 1 : b0);
    b1 = b1 < b0 ? b0 : (b1 > nbags - 1 ? nbags - 1 : b1);
    blo = b0;
    wn = b1 - b0 + 2;
  }
  const bool win = wn > 0 && wn <= kOccBagWin;
  if (win)
    for (int i = tid; i < wn; i += kOccThreads) s_off[i] = off[blo + i];
  __syncthreads();
  long long* occref = reinterpret_cast<long long*>(L.res.plan + plan_layout(L.res.capacity).o_occref);
#pragma unroll
  for (int k = 0; k < kOccPer; ++k) {
    const long long j = j0 + tid + k * kOccThreads;
    if (j >= j1) continue;
    int g;
    if (by_occ) {
      g = (int)j;
    } else {
      int lo, hi;
      if (win) {
        lo = 0;
        hi = wn - 1;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((long long)s_off[mid] <= j) lo = mid + 1;
          else hi = mid;
        }
        lo += blo;
      } else {
        lo = 0;
        hi = nbags;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((long long)off[mid] <= j) lo = mid + 1;
          else hi = mid;
        }
      }
      g = lo - 1;
      g = g < 0 ? 0 : (g > nbags - 1 ? nbags - 1 : g);
    }
    const int l = loc[k];
    const int pos = atomicAdd(&s_g[l], 1);
    L.res.grouped[pos] = g;
    // contiguous, and read back by later launches only: non-temporal
    // (the scattered grouped entries are not -- they merge in the caches)
    __builtin_nontemporal_store(s_u[l], L.res.inverse + j);
    __builtin_nontemporal_store(s_ref[l], occref + j);
  }
}

// A lookup made before the IDMap last changed: each distinct key is probed
// again (find only, no count) and its IDMap slot and row entry rewritten as
// the table holds them now -- a key evicted since gets no slot and row -1, a
// key admitted since gets its row, and a row still pending is reported with
// the fresh mark, as insert_find reports it.
__global__ __launch_bounds__(kThreads) void k_refresh(recis_lookup_result res, TableDev t) {
  const long long U = *res.num_unique;
  unsigned* idslot = reinterpret_cast<unsigned*>(res.plan + plan_layout(res.capacity).o_idslot);
  for (long long u = (long long)blockIdx.x * kThreads + threadIdx.x; u < U; u += (long long)gridDim.x * kThreads) {
    const long long key = res.unique_keys[u];
    const ProbeOut o = idmap_probe(t, key, 0, true, [](unsigned long long) { return false; });
    idslot[u] = o.sl;
    res.unique_rows[u] = o.row;
  }
}

__global__ void k_clear_error(DevCounters* ctr, unsigned bits) {
  if (threadIdx.x == 0) atomicAnd(&ctr->error, ~bits);
}

}  // namespace

void launch_refresh(const recis_lookup_result& res, const TableDev& t, hipStream_t s) {
  // a grid for the largest call; blocks past the distinct count exit at once
  long long nb = (res.n + kThreads - 1) / kThreads;
  nb = nb < 1 ? 1 : (nb > 8192 ? 8192 : nb);
  RECIS_LAUNCH("k_refresh", k_refresh, dim3((unsigned)nb), dim3(kThreads), s, res, t);
}

void launch_clear_error(DevCounters* ctr, unsigned bits, hipStream_t s) {
  RECIS_LAUNCH("k_clear_error", k_clear_error, dim3(1), dim3(64), s, ctr, bits);
}

void launch_lookup(const LookupLaunch& L, const TableDev& t, hipStream_t s) {
  const long long nb = (long long)L.F * L.B + 1;
  RECIS_LAUNCH("k_prep", k_prep, dim3((unsigned)((nb + kThreads - 1) / kThreads)), dim3(kThreads), s,
                     L, t);
  if (L.N > 0) {
    const unsigned G = (unsigned)L.part_blocks;
    RECIS_LAUNCH("k_tile", k_tile, dim3(G), dim3(kPartThreads), s, L, t);
    RECIS_LAUNCH("k_part_colscan", k_part_colscan, dim3((unsigned)((L.nbk + 63) / 64)), dim3(kPartThreads), s, L);
    RECIS_LAUNCH("k_scan_small", k_scan_small, dim3(1), dim3(kPartThreads), s, L.bbase, (int*)nullptr, L.nbk,
                 (long long*)nullptr);
    RECIS_LAUNCH("k_pair_scatter", k_pair_scatter, dim3(G), dim3(kPartThreads), s, L);
    // heavy slices: at most kHeavyBlocks blocks, each taking every kHeavyBlocks-th slice
    const long long hb = L.hmax < kHeavyBlocks ? L.hmax : kHeavyBlocks;
    const dim3 nb_grid((unsigned)L.nbk), count_grid((unsigned)(L.nbk + hb));
    if (L.big_tab)
      RECIS_LAUNCH("k_bucket_count", (k_bucket<2048, false, kBigBucketThreads>), count_grid,
                   dim3(kBigBucketThreads), s, L, t);
    else
      RECIS_LAUNCH("k_bucket_count", (k_bucket<1024, false, kThreads>), count_grid, dim3(kThreads), s, L, t);
    RECIS_LAUNCH("k_scan_small", k_scan_small, dim3(1), dim3(kPartThreads), s, L.ubase, L.obase, L.nbk,
                 reinterpret_cast<long long*>(L.res.num_unique));
    if (L.big_tab)
      RECIS_LAUNCH("k_bucket_emit", (k_bucket<2048, true, kBigBucketThreads>), nb_grid,
                   dim3(kBigBucketThreads), s, L, t);
    else
      RECIS_LAUNCH("k_bucket_emit", (k_bucket<1024, true, kThreads>), nb_grid, dim3(kThreads), s, L, t);
  }
  // block 0 scans; the others (N > 0 only) resolve the heavy buckets' pairs
  const long long kb = L.N > 0 ? 1 + (L.hmax < kHeavyBlocks / 4 ? L.hmax : kHeavyBlocks / 4) : 1;
  RECIS_LAUNCH("k_key_scan", k_key_scan, dim3((unsigned)kb), dim3(kScanThreads), s, L, t);
  if (L.N > 0) {
    RECIS_LAUNCH("k_key_finalize", k_key_finalize, dim3((unsigned)L.nbk), dim3(kThreads), s, L, t);
    RECIS_LAUNCH("k_occ_tile", k_occ_tile, dim3((unsigned)L.ntiles), dim3(kOccThreads), s, L);
  }
}

}  // namespace recis
