// internal.h -- shared declarations of the recis HIP library (not installed).
//
// Memory layout in HBM (one table):
//   IDMap        Slot[slot_cap]      16 B per slot: key, row, count; linear
//                                    probing from a multiplicative hash.
//   EmbeddingBlocks  block_rows rows per block; row r lives in block r >> lb at
//                    byte (r & mb) * stride; a row is [dim params in the storage
//                    dtype | slots * dim float32 optimizer state].
//   free list    int32 rows released by eviction.
//   DevCounters  bump pointer, free-list top, key count, error word.
//   scratch      per-step dedup table and per-occurrence / per-key arrays.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "recis.h"

namespace recis {

constexpr long long kEmptyKey = -1;  // free slot
constexpr long long kBadKey = -2;    // an occurrence whose transform failed
constexpr long long kGoneKey = -3;   // evicted, awaiting rebuild

// A row is materialised lazily: insert_find allocates it and marks it
// pending; until its first update (or writeback) its values are the
// initializer's, recomputed from (seed, key) wherever they are read.
constexpr int kPendingRow = 1 << 30;               // in Slot.row
constexpr long long kFreshRow = 1ll << 62;         // in unique_rows: row may be pending
constexpr long long kMaxRows = (1ll << 30) - 1;
// IDMap slot indices are kept in 32 bits with 0xFFFFFFFF meaning "no slot":
// the IDMap never grows past 2^31 slots, so no real index reaches the mark.
constexpr long long kMaxSlots = 1ll << 31;

constexpr unsigned kErrInvalid = 1u << RECIS_ERR_INVALID_ARG;
constexpr unsigned kErrCapacity = 1u << RECIS_ERR_CAPACITY;
constexpr unsigned kErrKeyRange = 1u << RECIS_ERR_KEY_RANGE;

// Occurrence tiling of the per-occurrence kernels.
constexpr int kThreads = 256;
constexpr int kOccPerThread = 8;
constexpr int kOccTile = kThreads * kOccPerThread;  // 2048
constexpr int kLdsTabBits = 12;
constexpr int kLdsTab = 1 << kLdsTabBits;            // block-local dedup table (2 x kOccTile)
static_assert(kLdsTab == 2 * kOccTile, "block-local dedup table at most half full");
// Distinct-key tiling of the per-key kernels: one key per thread, so that the
// dependent probe chains of different keys overlap instead of queueing.
// Backward: keys with more occurrences than kShortMax are split into chunks.
constexpr int kShortMax = 64;
constexpr int kChunk = 64;  // one grouped entry per lane of a wave
// A long key is cut into at most kMaxKeyChunks chunks of a multiple of
// kChunk entries: a hot key's partial sums stay few enough for one wave to
// merge them.
constexpr int kMaxKeyChunks = 1024;
__host__ __device__ inline int long_chunk(int c) {
  const int per = (c + kChunk * kMaxKeyChunks - 1) / (kChunk * kMaxKeyChunks);
  return kChunk * (per > 1 ? per : 1);
}
__host__ __device__ inline int long_chunks(int c) {
  const int z = long_chunk(c);
  return (c + z - 1) / z;
}

struct __align__(16) Slot {
  long long key;
  int row;
  unsigned count;
};

struct __align__(16) DedupSlot {
  long long key;
  int count;  // occurrences in this call (writeback: last occurrence index)
  int uidx;   // index of the key among the call's distinct keys
};

// One tile-distinct key in its hash bucket (the lookup deduplicates each
// tile of kTileOcc occurrences first): the key, its pair index (tile *
// kTileOcc + its index among the tile's distinct keys) and its occurrences
// in the tile.
struct __align__(16) PartEntry {
  long long key;
  int pid;
  int w;
};

// What the bucket kernels write for a pair once its key is resolved, at the
// pair's slot (tile * kTileOcc + its index in the tile): the forward
// reference, the distinct-key index, and where the pair's occurrences start
// in the key's group.  The lookup's last kernel reads a tile's contiguously.
struct __align__(16) PartOut {
  long long ref;
  int u;
  int gpos;
};

struct DevCounters {
  unsigned long long next_row;  // bump pointer over EmbeddingBlocks
  long long free_top;           // entries in the free list
  unsigned long long num_keys;  // keys in the IDMap
  unsigned int error;           // sticky error bits (kErr*)
  unsigned int pad0;
  // written by the scan kernel for the finalize kernel of the same call
  long long take_free;
  long long free_top_old;
  long long bump_base;
  unsigned long long scratch_count;  // writeback distinct keys / export count / evicted
  // IDMap slot claims made by insert_find since creation: attempts, and
  // those that lost the slot to another key (summed per bucket, added by
  // the scan kernel once per call)
  unsigned long long claim_attempts;
  unsigned long long claim_failures;
  // (key, tile) pairs: distinct keys of each tile of kTileOcc consecutive
  // occurrences, summed over the tiles of every insert_find since creation
  unsigned long long lookup_pairs;
  // long keys the backward summed bag-major (hot keys), over every call
  unsigned long long hot_keys;
};

// Device view of one feature of a call.
struct FeatDev {
  const long long* values;
  const int* offs;
  long long n;
  long long base;       // global index of its first occurrence
  unsigned long long mod;
  unsigned long long mod_inv;  // floor((2^64 - 1) / mod), for the remainder by multiplication
  unsigned slot;
  unsigned ops;
  int bnd_off;
  int nb;
};

// Backward work plan header (in recis_lookup_result.plan).
// Feature bins: a key's bin is its feature slot modulo kFeatBins.  The
// backward groups the long keys by bin, and picks the hot keys of each bin.
constexpr int kFeatBins = 4096;

// Plan words 0..3: long keys, chunks, whether the lookup's features have
// distinct bins (kPlanHotOk, with at most kFeatBins features), unused.
// Words o_fbin..: the bin of each feature.
constexpr int kPlanHotOk = 2;
struct PlanLayout {
  long long max_long, max_chunks;
  // word offsets
  long long o_fbin, o_long_u, o_long_base, o_long_nch, o_chunk_owner, o_idslot, o_occref;
  long long words;
};

__host__ __device__ inline PlanLayout plan_layout(long long cap) {
  PlanLayout p;
  p.max_long = cap / kShortMax + 1;
  p.max_chunks = cap / kChunk + p.max_long + 1;
  p.o_fbin = 4;
  p.o_long_u = p.o_fbin + kFeatBins;
  p.o_long_base = p.o_long_u + p.max_long;
  p.o_long_nch = p.o_long_base + p.max_long;
  p.o_chunk_owner = p.o_long_nch + p.max_long;
  p.o_idslot = p.o_chunk_owner + p.max_chunks;  // IDMap slot of each distinct key
  p.o_occref = (p.o_idslot + cap + 2) & ~1ll;   // 8-byte aligned: int64 per occurrence
  p.words = p.o_occref + 2 * cap + 2;
  return p;
}

// Per-occurrence row reference written by insert_find for the forward: the
// row's device address (>= 0; blocks never move, so it stays valid while
// the table lives), kOccNoRow, or kOccPendingBit | key for a row that was
// pending at the lookup (its values are the initializer's of `key`).
constexpr long long kOccNoRow = 1ll << 62;
constexpr unsigned long long kOccPendingBit = 1ull << 63;

struct RowSpace {
  char* const* blocks;  // device array of block base pointers
  int lb;               // log2(block_rows)
  long long mb;         // block_rows - 1
  long long stride;     // bytes per row
};

// Rows are below 2^30, so the block index and the in-block product fit 32-bit
// operands (one 32x32->64 multiply-add).
__device__ __forceinline__ char* row_ptr(const RowSpace& rs, long long r) {
  const unsigned ri = (unsigned)r;
  return rs.blocks[ri >> rs.lb] + (unsigned long long)(ri & (unsigned)rs.mb) * (unsigned)rs.stride;
}

// Global-memory views of pointers that were themselves loaded from memory
// (row addresses, block bases): without the address space the compiler emits
// FLAT accesses, which also count against the LDS wait counter, so every
// wait for an LDS read would wait for the row traffic too.
#define RECIS_GLOBAL __attribute__((address_space(1)))
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ const RECIS_GLOBAL T* gread(const void* p) {
  return (const RECIS_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ RECIS_GLOBAL T* gwrite(void* p) {
  return (RECIS_GLOBAL T*)p;
}

// Multiplicative (Fibonacci) hash of a key to a slot of a 2^k table; shift = 64 - k.
__device__ __forceinline__ unsigned long long slot_of(long long key, int shift) {
  return ((unsigned long long)key * 0x9E3779B97F4A7C15ull) >> shift;
}

// ----------------------------------------------------------------- values
// bfloat16 <-> float; float -> bfloat16 rounds to nearest, ties to even.
__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
  return __uint_as_float((unsigned)b << 16);
}
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))  // NaN stays NaN
    return (unsigned short)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// MurmurHash3's 64-bit finalizer (the Hash transform).
__device__ __forceinline__ unsigned long long fmix64(unsigned long long k) {
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdull;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ull;
  k ^= k >> 33;
  return k;
}

// Philox4x32-10 block (Salmon et al., SC'11).
__device__ __forceinline__ uint4 philox10(uint4 c, uint2 k) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32x32->64 multiply each (v_mad_u64_u32), not separate lo/hi
    const unsigned long long p0 = (unsigned long long)c.x * 0xD2511F53u;
    const unsigned long long p1 = (unsigned long long)c.z * 0xCD9E8D57u;
    c = make_uint4((unsigned)(p1 >> 32) ^ c.y ^ k.x, (unsigned)p1, (unsigned)(p0 >> 32) ^ c.w ^ k.y, (unsigned)p0);
    k.x += 0x9E3779B9u;
    k.y += 0xBB67AE85u;
  }
  return c;
}

// Four initial values of elements 4g..4g+3 of the row of `key`: the top 24
// bits of each Philox word, centred, times bound * 2^-23 (one rounding).
__device__ __forceinline__ float4 init4(unsigned long long seed, long long key, unsigned g,
                                        float scale) {
  const uint4 w = philox10(make_uint4(g, 0u, (unsigned)key, (unsigned)((unsigned long long)key >> 32)),
                           make_uint2((unsigned)seed, (unsigned)(seed >> 32)));
  float4 v;
  v.x = __fmul_rn((float)((int)(w.x >> 8) - (1 << 23)), scale);
  v.y = __fmul_rn((float)((int)(w.y >> 8) - (1 << 23)), scale);
  v.z = __fmul_rn((float)((int)(w.z >> 8) - (1 << 23)), scale);
  v.w = __fmul_rn((float)((int)(w.w >> 8) - (1 << 23)), scale);
  return v;
}

// ------------------------------------------------------------ the table
// The IDMap is open addressing with linear probing, split into 2^region_bits
// regions by the top bits of the key's hash: a key's home slot is the top
// bits of its hash (as for one undivided table) and its probe wraps inside
// the home slot's region.  The lookup partitions a call by the same top bits,
// so one block owns every region its bucket maps to and inserts without
// global atomics.
constexpr int kMinRegionSlotBits = 10;  // regions hold at least 1024 slots

struct TableDev {
  Slot* slots;
  unsigned long long slot_mask;
  int slot_shift;
  int region_bits;
  unsigned long long region_mask;  // slots per region - 1
  DevCounters* ctr;
  int* free_list;
  RowSpace rs;
  int dim, dtype, optim, state_words;  // state_words = slots per element (0, 1, 2)
  unsigned admit;
  unsigned long long seed;
  float init_scale;                    // bound * 2^-23
  long long rows_limit;                // rows covered by blocks
  unsigned* last_use;                  // per IDMap slot: the counting lookup that last saw its key
                                       // (nullptr when the table does not track it)
  unsigned step;                       // counting lookups so far
  unsigned* sketch;                    // count-min admission: kSketchRows x 2^sketch_bits (or nullptr)
  int sketch_bits;
};

// Count-min sketch admission: counter of `key` in row r = the top
// sketch_bits bits of fmix64(key ^ salt_r), salt_r an odd multiple of the
// 64-bit golden ratio.
constexpr int kSketchRows = 4;
__device__ __forceinline__ unsigned long long sketch_at(const TableDev& t, long long key, int r) {
  const unsigned long long salt = 0x9E3779B97F4A7C15ull * (unsigned long long)(2 * r + 1);
  return ((unsigned long long)r << t.sketch_bits) +
         (fmix64((unsigned long long)key ^ salt) >> (64 - t.sketch_bits));
}
__device__ __forceinline__ void sketch_add(const TableDev& t, long long key, unsigned c) {
#pragma unroll
  for (int r = 0; r < kSketchRows; ++r) atomicAdd(&t.sketch[sketch_at(t, key, r)], c);
}
__device__ __forceinline__ unsigned sketch_estimate(const TableDev& t, long long key) {
  unsigned v[kSketchRows];
#pragma unroll
  for (int r = 0; r < kSketchRows; ++r) v[r] = t.sketch[sketch_at(t, key, r)];
  unsigned e = v[0];
#pragma unroll
  for (int r = 1; r < kSketchRows; ++r) e = v[r] < e ? v[r] : e;
  return e;
}

__device__ __forceinline__ unsigned long long next_slot(const TableDev& t, unsigned long long p) {
  return (p & ~t.region_mask) | ((p + 1) & t.region_mask);
}

// Initial values of 16-byte parameter chunk c of the row of `key`, in the
// storage format (4 fp32 or 8 bf16 elements).  Kernels built for one storage
// type take the compile-time form: the other type's code would still count
// toward their registers.
template <bool BF16>
__device__ __forceinline__ uint4 init_chunk_as(const TableDev& t, long long key, int c) {
  if constexpr (BF16) {
    const float4 a = init4(t.seed, key, 2u * c, t.init_scale);
    const float4 b = init4(t.seed, key, 2u * c + 1u, t.init_scale);
    return make_uint4((unsigned)f32_to_bf16(a.x) | ((unsigned)f32_to_bf16(a.y) << 16),
                      (unsigned)f32_to_bf16(a.z) | ((unsigned)f32_to_bf16(a.w) << 16),
                      (unsigned)f32_to_bf16(b.x) | ((unsigned)f32_to_bf16(b.y) << 16),
                      (unsigned)f32_to_bf16(b.z) | ((unsigned)f32_to_bf16(b.w) << 16));
  } else {
    const float4 a = init4(t.seed, key, (unsigned)c, t.init_scale);
    return make_uint4(__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z), __float_as_uint(a.w));
  }
}
__device__ __forceinline__ uint4 init_chunk(const TableDev& t, long long key, int c) {
  return t.dtype == RECIS_DTYPE_BF16 ? init_chunk_as<true>(t, key, c) : init_chunk_as<false>(t, key, c);
}

// Instrumentation: launches of the kernel named `name` are bracketed by the
// two events (see recis_profile_kernel).  The table's probe is made current
// for the duration of each of its calls.
struct KernelProbe {
  char name[64] = {};
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local const KernelProbe* tl_probe;
inline bool probe_on(const char* name) {
  return tl_probe && tl_probe->start && __builtin_strcmp(tl_probe->name, name) == 0;
}
#define RECIS_LAUNCH(NAME, KERNEL, GRID, BLOCK, STREAM, ...)                 \
  do {                                                                       \
    const bool probe_ = probe_on(NAME);                                      \
    if (probe_) (void)hipEventRecord(tl_probe->start, STREAM);               \
    hipLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, STREAM, __VA_ARGS__);         \
    if (probe_) (void)hipEventRecord(tl_probe->stop, STREAM);                \
  } while (0)

}  // namespace recis

struct recis_table {
  recis_table_config cfg;
  recis_allocator alloc;
  bool own_alloc;
  int device;
  int state_words;
  long long row_bytes;
  int lb;

  recis::Slot* slots = nullptr;
  long long slot_cap = 0;
  recis::DevCounters* ctr = nullptr;
  std::vector<char*> blocks;
  char** d_blocks = nullptr;
  long long d_blocks_cap = 0;
  long long rows_alloc = 0;
  int* free_list = nullptr;
  long long free_cap = 0;

  // host-side upper bounds (exact after a sync)
  long long rows_hi = 0;
  long long keys_hi = 0;
  long long adam_step = 0;
  long long bytes = 0;
  // bumped by every call that writes rows or frees them (update, writeback,
  // eviction); a lookup result records the value it was made at
  unsigned long long update_epoch = 1;
  // bumped by every call that can change which key holds which IDMap slot or
  // row: a counting insert_find (inserts, admissions, growth), writeback,
  // import and eviction.  A lookup result records the value after its own
  // insert_find; forward and backward re-probe its keys when it differs.
  unsigned long long map_version = 1;

  recis::KernelProbe probe;

  // per-step scratch, sized for scr_cap occurrences
  long long scr_cap = 0;
  recis::DedupSlot* dd = nullptr;
  long long dd_cap = 0;
  recis::PartEntry* part = nullptr;
  int* hist = nullptr;
  int* bbase = nullptr;
  int* ubase = nullptr;
  int* uslot = nullptr;
  recis::PartOut* pout = nullptr;
  long long* tkey = nullptr;  // tile-distinct keys, their counts, per-tile sizes
  int* tcnt = nullptr;
  int* tile_n = nullptr;
  unsigned short* occ_local = nullptr;  // occurrence -> index among its tile's distinct keys
  unsigned long long* blk_sums = nullptr;
  unsigned* last_use = nullptr;  // [slot_cap] when cfg.track_last_use
  unsigned step = 0;             // counting lookups so far
  unsigned* sketch = nullptr;    // [kSketchRows << cfg.admit_sketch_bits] when sketch admission is on
  long long* wb_keys = nullptr;
  double* partials = nullptr;
  double* hot_partials = nullptr;  // the hot keys' partials: hot_rows rows of dim doubles
  long long hot_rows = 0;
  int* hot_ws = nullptr;  // the hot pass's workspace: hot_ws_len ints
  long long hot_ws_len = 0;

  // pinned staging ring for per-call descriptors
  static constexpr int kRing = 4;
  char* stage_host[kRing] = {};
  char* stage_dev[kRing] = {};
  size_t stage_cap[kRing] = {};
  hipEvent_t stage_ev[kRing] = {};
  int ring_pos = 0;

  recis::TableDev dev() const;
};

namespace recis {

// Launchers (defined in the .hip files; all enqueue on `s`).
void launch_fill_slots(Slot* slots, long long cap, hipStream_t s);
void launch_zero_u32(unsigned* p, long long n, hipStream_t s);
void launch_key_ages(const TableDev& t, const long long* keys, long long n, unsigned* ages, bool set, hipStream_t s);
void launch_fill_dedup(DedupSlot* dd, long long cap, hipStream_t s);
void launch_rehash(const Slot* old_slots, const unsigned* old_last_use, long long old_cap, const TableDev& t,
                   hipStream_t s);

// Logical index of workgroup i of a grid of G.  Workgroups are dealt to the
// 8 XCDs round robin (i mod 8); this gives the workgroups of one XCD
// consecutive logical indices, so that what they write side by side is
// merged in that XCD's L2 before it goes to memory.
__device__ __forceinline__ int xcd_block(int i, int G) {
  const int x = i & 7, k = i >> 3, q = G >> 3, r = G & 7;
  return x * q + (x < r ? x : r) + k;
}

// Hash partition of a lookup call.  Tiles of kTileOcc consecutive
// occurrences are deduplicated in LDS first; their distinct keys (pairs)
// are what the partition and the bucket kernels handle.
constexpr int kTileOcc = 4096;
constexpr int kTileTab = 2 * kTileOcc;  // the tile's LDS table, at most half full
constexpr int kPartThreads = 1024;   // partition kernels' block size
// At most one partition block per CU: k_tile's LDS table allows one block
// per CU anyway, and fewer, longer blocks give k_pair_scatter longer runs of
// records per bucket (each block's records of a bucket are contiguous) and
// the column scan a smaller histogram.
constexpr int kMaxPartBlocks = 256;
// Target occurrences per bucket.  The bucket count is this share rounded up
// to a power of two (then capped), so a call gets 512 to 1024 occurrences per
// bucket until the cap: after the tile-level dedup that is a few hundred
// pairs, enough to keep a bucket block's threads busy past its fixed costs
// (table clear, bases, barriers).
constexpr int kBucketOcc = 1024;
constexpr int kMinBuckets = 256;  // one bucket block per CU for small calls (within the IDMap's regions)
// The bucket blocks' smaller LDS table (1024 entries) holds at most 768
// distinct keys.  A call with more than kSmallTabOcc occurrences per bucket
// on average could give a bucket more than that when most of its keys are
// distinct (a bulk insert of new keys), so it takes the 2048-entry table:
// an overflowing bucket falls back to a global table, several times slower.
constexpr int kSmallTabOcc = 640;
constexpr int kMaxBucketBits = 13;
constexpr int kMaxBuckets = 1 << kMaxBucketBits;
constexpr int kBucketPer = 4;        // occurrences per thread per pass of k_bucket
// A bucket of more than kHeavyOcc occurrences (a hot key's bucket) is cut into
// slices of kSliceOcc (at most 3/4 of the smaller LDS table, so a slice never
// overflows it), each deduplicated by its own block.
constexpr int kHeavyOcc = 16384;
constexpr int kSliceOcc = 768;
constexpr int kHeavyBlocks = 1024;  // blocks that share out the heavy slices

struct LookupLaunch {
  const FeatDev* feats;
  const long long* bnd_pool;
  int F, B;
  long long N;
  unsigned flags;
  recis_lookup_result res;
  DedupSlot* dd;  // empty between calls; regions of it back overflowed buckets
  int nbits, nbk;             // hash buckets: nbk = 2^nbits
  int part_blocks;            // partition blocks
  long long tiles_per_block;  // tiles per partition block
  long long ntiles;           // tiles of the call
  long long* tkey;            // [ntiles * kTileOcc]: each tile's distinct keys, from its start
  int* tcnt;                  // [ntiles * kTileOcc]: their occurrences in the tile
  int* tile_n;                // [ntiles]: distinct keys per tile
  int* tile_bag;              // [ntiles]: the bag of each tile's first occurrence
  unsigned short* occ_local;  // N: each occurrence's index among its tile's distinct keys
  int* obase;                 // nbk + 1: occurrences per bucket, then the first grouped position
  int big_tab;                // buckets average more than kSmallTabOcc occurrences
  int hot_ok;                 // at most kFeatBins features, in distinct feature bins
  int* hist;                  // [part_blocks][nbk]
  int* bbase;                 // nbk + 1: first position of each bucket
  int* ubase;                 // nbk + 1: distinct keys per bucket, then their first index
  PartEntry* part;            // pairs (at most N)
  PartOut* pout;              // [ntiles * kTileOcc]: each pair resolved (emit), at its pair slot
  unsigned long long* blk_sums;  // per key tile: rows to allocate << 32 | keys inserted
  unsigned long long* blk_long;  // per key tile: long keys << 32 | their chunks
  unsigned long long* blk_claim; // per key tile: IDMap slot claims << 32 | claims lost
  int* klist;                    // N: heavy buckets' distinct keys (dedup-table slots), by bucket range
  int* hslice;                   // heavy slices: count, then (bucket, slice) pairs
  long long hmax;                // bound on the heavy slices of the call (their grids)
  unsigned* last_use;            // stamped with `step` for every key the call counts (or nullptr)
  unsigned step;
  int sketching;                 // count-min admission in this (counting) call
};
void launch_lookup(const LookupLaunch& L, const TableDev& t, hipStream_t s);
// Re-probes every distinct key of a lookup (find only): its IDMap slot and
// row as the table holds them now, for a lookup made before the IDMap last
// changed (later inserts, growth, writeback, import or eviction).
void launch_refresh(const recis_lookup_result& res, const TableDev& t, hipStream_t s);
// Clears `bits` of the device error word.
void launch_clear_error(DevCounters* ctr, unsigned bits, hipStream_t s);

// `current`: no update, writeback or eviction ran on the table since the
// lookup, so its fresh marks and per-occurrence row references still hold
// and the IDMap need not be read again.
void launch_forward(const recis_lookup_result& res, const TableDev& t, int pool, void* out,
                    bool current, hipStream_t s);
struct OptConsts {
  float lr, b1, omb1, b2, omb2, eps, step_size;  // omb = 1 - beta, formed in double
};
// reorder: device scratch of reorder_ints ints for the long keys' plan in
// feature order (used when the pooled gradient exceeds kMemCacheBytes, or
// with hot keys).
constexpr double kMemCacheBytes = 256.0 * 1024 * 1024;  // the memory-side (Infinity) cache
// Hot keys (pooled backward, dim 64 or 128): per feature at most
// hot_kmax(dim) long keys with at least hot_min_count(blocks) occurrences
// are summed bag-major, one partial per key and block of kHotBags bags.
// hot_partials: hot_rows rows of dim doubles, at least
// num_feats * hot_kmax(dim) * hot_blocks(batch) for the pass to run.
constexpr int kHotBags = 2048;
__host__ __device__ inline int hot_kmax(int dim) { return dim == 64 || dim == 128 ? 8192 / dim : 0; }
__host__ __device__ inline long long hot_blocks(int batch) { return (batch + kHotBags - 1) / kHotBags; }
// The pass takes a block's bags hot_stage(dim) at a time (kHotBags is a
// multiple of it); per stage the hot occurrences are sorted by key first.
__host__ __device__ inline int hot_stage(int dim) { return dim == 64 || dim == 128 ? 16384 / dim : 1; }
__host__ __device__ inline long long hot_stages(int batch, int dim) {
  return (batch + hot_stage(dim) - 1) / hot_stage(dim);
}
// Its workspace (ints): per bin the count classes, threshold, hot-key count,
// first hot index and placement counter; per distinct key its hot index; per
// occurrence slot a sorted hot entry; per distinct key its hot index (a
// byte); per (feature, stage) the entry count.
constexpr int kHotClasses = 32;
__host__ __device__ inline long long hot_ws_ints(long long n, int num_feats, int batch, int dim) {
  return (long long)kFeatBins * (kHotClasses + 4) + n + (n + 3) / 4 + (long long)num_feats * hot_stages(batch, dim) +
         16;
}
// A hot key's partial rows cost about as much as 4 of its gradient rows
// each; with 8 occurrences per partial the bag-major pass reads fewer bytes.
__host__ __device__ inline int hot_min_count(long long blocks) {
  const long long m = 8 * blocks;
  return m > kShortMax + 1 ? (int)(m < (1 << 30) ? m : (1 << 30)) : kShortMax + 1;
}
recis_status launch_backward(const recis_lookup_result& res, const TableDev& t, int pool,
                             const void* grad, int grad_dtype, const OptConsts& oc,
                             double* partials, int* reorder, long long reorder_ints,
                             double* hot_partials, long long hot_rows, int* hot_ws, long long hot_ws_len,
                             bool current, hipStream_t s);

// The fixed device scratch of the allocation-free backward: the long keys'
// chunk partials, kNoAllocScratchBytes on each GPU the library runs it on,
// held until the process ends and shared by every such call on that GPU.
constexpr long long kNoAllocScratchBytes = 64ll << 20;
// Its address on `device` (which must be current), looked up once per device.
recis_status noalloc_scratch(int device, void** out);

void launch_evict(const TableDev& t, unsigned min_count, double decay, long long* num_evicted, hipStream_t s);
// Hot-tier placement: rows [0, hbm_rows) are in HBM.  `work` holds
// retier_words(slot_cap, hbm_rows) ints of device scratch.
long long retier_words(long long slot_cap, long long hbm_rows);
void launch_retier(const TableDev& t, long long hbm_rows, int* work, long long* num_moved, hipStream_t s);
// LRU-bounded pass: keeps the youngest ages whole within max_keys; `work`
// holds age_hist_words(slot_cap) ints of device scratch.
long long age_hist_words(long long slot_cap);
void launch_evict_lru(const TableDev& t, long long max_keys, int* work, long long* num_evicted, hipStream_t s);
void launch_writeback(const TableDev& t, const long long* keys, long long n, const float* rows,
                      DedupSlot* dd, unsigned long long dd_mask, int dd_shift, long long* wb_keys,
                      int* uslot, hipStream_t s);
void launch_export(const TableDev& t, long long cap, long long* keys, long long* rows,
                   unsigned* counts, hipStream_t s);
void launch_export_rows(const TableDev& t, long long n, const long long* keys, long long* rows, void* params,
                        float* state, hipStream_t s);
void launch_import(const TableDev& t, long long n, const long long* keys, const long long* rows,
                   const unsigned* counts, const void* params, const float* state, hipStream_t s);

}  // namespace recis
