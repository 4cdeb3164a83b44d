/* recis.h -- C ABI of the dynamic-embedding hot path on one MI355X (gfx950).
 *
 * The library implements the embedding engine that the RecIS pages describe
 * (page: "RecIS (Recommendation Intelligence System)" README, mirror of
 * alibaba/RecIS v1.1.0) for one GPU:
 *   - a two-level table: IDMap (feature ID -> Offset) over EmbeddingBlocks that
 *     hold parameters and optimizer state, growing block by block
 *     (section "Key optimisations > Efficient dynamic Embedding");
 *   - collision-free keys, merged same-attribute tables, eviction/admission
 *     (section "Core architecture > Embedding Engine");
 *   - Hash / Mod / Bucketize ID transforms fused into the lookup
 *     (sections "Core architecture > Feature Engine" and "Key optimisations >
 *     GPU concurrency");
 *   - merged, deduplicated requests (section "Key optimisations > Distributed
 *     optimisation > request merge and split");
 *   - duplicate-gradient reduction without hot atomics (section "Key
 *     optimisations > Operator implementation");
 * plus the exact-assignment cache write of the in-model item cache (page:
 * "Memory Layer: Train the In-Model Cache for Recommendation Models", sections
 * "What carries the argument" and "Referee Report > Summary").
 *
 * Conventions shared by every call:
 *   - Every pointer named "device" is GPU memory of the current HIP device;
 *     "host" pointers are CPU memory.  The caller owns every buffer it passes
 *     and keeps it alive until the stream work of the call has completed.  No
 *     call keeps a caller pointer after that.
 *   - The table owns its IDMap, EmbeddingBlocks and per-step scratch, obtained
 *     from the allocator given at creation (hipMalloc / hipFree when NULL).
 *   - All calls are asynchronous and ordered on the stream `s`, except those
 *     documented as synchronising.  A table is used from one stream at a time;
 *     separate tables are independent.
 *   - Argument errors are returned at once and nothing is enqueued.  Errors
 *     found on the GPU (capacity, key range, malformed bag offsets) are
 *     recorded in the table's sticky device error word and returned by
 *     recis_get_error(); the data they concern is then unspecified, but no
 *     kernel reads or writes out of bounds.
 */
#ifndef RECIS_H
#define RECIS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t recis_status;
#define RECIS_OK 0
#define RECIS_ERR_INVALID_ARG 1   /* bad pointer, size, enum, unsorted boundaries, small buffer */
#define RECIS_ERR_OUT_OF_MEMORY 2 /* the allocator returned NULL */
#define RECIS_ERR_CAPACITY 3      /* max_rows, or a key's IDMap region, exhausted (device, sticky) */
#define RECIS_ERR_KEY_RANGE 4     /* transformed id outside [0, 2^48) or slot >= 2^15 (device) */
#define RECIS_ERR_HIP 5           /* a HIP runtime call failed */
#define RECIS_ERR_UNSUPPORTED 6   /* a valid but unimplemented combination */

/* Parameter storage type; optimizer state is always float32. */
#define RECIS_DTYPE_F32 0
#define RECIS_DTYPE_BF16 1

#define RECIS_OPTIM_NONE 0    /* no state; rows change only by writeback */
#define RECIS_OPTIM_ADAGRAD 1 /* 1 state word per element: accumulated G^2 */
#define RECIS_OPTIM_ADAM 2    /* 2 state words per element: m, v */

/* Where the EmbeddingBlocks live (the pages let both tiers sit on the GPU or
 * the CPU: page "RecIS (Recommendation Intelligence System)" README, section
 * "Key optimisations > Efficient dynamic Embedding").  HOST blocks are pinned
 * host memory mapped into the GPU's address space: the kernels read and write
 * rows across the host link, and the table can hold more rows than HBM.  The
 * IDMap and all scratch stay in HBM either way. */
#define RECIS_MEM_DEVICE 0
#define RECIS_MEM_HOST 1

#define RECIS_POOL_SUM 0
#define RECIS_POOL_MEAN 1
#define RECIS_POOL_NONE 2 /* gather only: one output row per occurrence */

/* Per-feature ID transforms (Feature Engine).  HASH is MurmurHash3's 64-bit
 * finalizer of the value's bit pattern; MOD is an unsigned remainder after
 * HASH and a floor remainder in [0, mod) on a raw signed value; BUCKETIZE
 * gives the number of boundaries <= value and excludes HASH and MOD. */
#define RECIS_OP_HASH 1u
#define RECIS_OP_MOD 2u
#define RECIS_OP_BUCKETIZE 4u

/* insert_find flags */
#define RECIS_FIND_ONLY 1u          /* eval: no insert, no count; absent -> row -1 */
#define RECIS_GROUP_BY_OCCURRENCE 2u /* group occurrences for POOL_NONE backward */

typedef struct recis_table recis_table; /* opaque */

typedef struct {
  int32_t dim;              /* elements per row: 8, 16, 32, 64, 128 or 256 */
  int32_t dtype;            /* RECIS_DTYPE_* */
  int32_t optim;            /* RECIS_OPTIM_* */
  uint32_t admit_threshold; /* a key gets a row once its count reaches this (0 or 1: at once) */
  uint64_t seed;            /* initializer seed */
  float init_bound;         /* rows start uniform on [-init_bound, init_bound) */
  float max_load;           /* IDMap occupancy that triggers growth, in (0, 0.75]: the IDMap is
                               split into regions by the top bits of the key hash (each
                               probe stays in its region), and this bound keeps every
                               region from filling unless keys collide in those bits */
  int64_t slot_capacity;    /* initial IDMap slots (rounded up to a power of two) */
  int64_t block_rows;       /* rows per EmbeddingBlock (rounded up to a power of two) */
  int64_t max_rows;         /* hard row limit (<= 2^30 - 1) */
  int64_t reserve_rows;     /* rows allocated at creation (rounded up to whole blocks) */
  int32_t block_memory;     /* RECIS_MEM_DEVICE (from the allocator) or RECIS_MEM_HOST
                               (hipHostMalloc, non-coherent: rows may be cached by the GPU
                               during a call, so the host must not touch them directly) */
  int32_t track_last_use;   /* 1: every counting insert_find stamps the keys it sees (4
                               bytes per IDMap slot), for recis_idmap_evict_lru; 0: off */
  int32_t admit_sketch_bits; /* 0: admission on exact counts kept in the IDMap.  1..30:
                               count-min sketch admission -- a key not in the IDMap is
                               counted in 4 x 2^bits 32-bit counters (its counters gain
                               its occurrences of every counting insert_find, all before
                               any estimate is read) and enters the IDMap, with its
                               estimate (the least of its counters) as its count and a
                               row, once that estimate reaches admit_threshold; until
                               then it takes no slot.  Eviction passes clear the sketch.
                               (Page "RecIS (Recommendation Intelligence System)" README,
                               section "Core architecture > Embedding Engine": admission
                               strategies.) */
  int64_t device_rows;      /* RECIS_MEM_HOST only: the first device_rows rows (rounded up to
                               whole blocks) are EmbeddingBlocks in HBM, the hot tier in front
                               of the pinned host blocks; new rows are handed out from the
                               start, so they fill the HBM tier first, and recis_idmap_retier
                               moves the most frequent keys into it.  0: every block in host
                               memory.  Ignored for RECIS_MEM_DEVICE (every row in HBM). */
  int64_t hot_grad_bytes;   /* the pooled backward sums the gradients of hot long keys
                               bag-major (each bag's gradient row read once for all of them,
                               see recis_table_stats.hot_keys) when the upstream gradient
                               (num_feats * batch * dim elements) holds at least this many
                               bytes: below that it stays in the memory-side cache and the
                               key-by-key sums re-read it cheaply.  0: the library's default,
                               256 MiB; negative: never.  Either way the results agree to
                               the parity bar (the same terms, summed in another order). */
} recis_table_config;

/* Fills `cfg` with defaults (dim 64, f32, Adagrad, seed 20250925, bound 0.05,
 * max_load 0.5, 2^20 slots, 2^20 rows per block, max_rows 2^30-1, reserve 0,
 * blocks in device memory, no last-use stamps, exact admission, no HBM tier,
 * the default gradient size for the bag-major pass).
 * Passage: page "RecIS (Recommendation Intelligence System)" README, section "Key optimisations > Distributed optimisation"
 * (a table's attributes: dimension, initializer). */
void recis_table_config_default(recis_table_config* cfg);

/* Device-memory provider.  alloc returns `bytes` of device memory (256-byte
 * aligned) or NULL; free releases it.  Both may be called with the stream of
 * the call that needs the memory.  The Python binding passes callbacks over
 * torch's caching allocator (the pages build on PyTorch: page "RecIS: Sparse
 * to Dense, A Unified Training Framework for Recommendation Models",
 * abstract), so a table takes its device memory from the same pool as the
 * model; with NULL the library uses hipMalloc / hipFree. */
typedef struct {
  void* ctx;
  void* (*alloc)(void* ctx, size_t bytes, hipStream_t s);
  void (*free)(void* ctx, void* p, hipStream_t s);
} recis_allocator;

/* One sparse feature of a batch, CSR over `batch` samples. */
typedef struct {
  const int64_t* values;      /* device [n] raw values */
  const int32_t* bag_offsets; /* device [batch + 1]: 0 = o[0] <= ... <= o[batch] = n */
  int64_t n;
  uint32_t slot;              /* feature tag, < 2^15; key = (slot << 48) | id */
  uint32_t ops;               /* RECIS_OP_* */
  uint64_t mod;               /* > 0 when RECIS_OP_MOD */
  const int64_t* boundaries;  /* host [nb], strictly increasing, for RECIS_OP_BUCKETIZE */
  int64_t nb;
} recis_feature_desc;

/* Result of one insert_find; all arrays are caller-allocated device memory
 * sized for `capacity` occurrences (N <= capacity) and are filled on the
 * stream.  unique order is unspecified.  Fields after `capacity` are written
 * by insert_find on the host and read by the forward / backward calls. */
typedef struct {
  int64_t* unique_keys;    /* [capacity] distinct keys, first num_unique valid */
  int64_t* unique_rows;    /* [capacity] row of each distinct key, -1 = none; bit 62 set:
                              the row may still hold only its initial values, which
                              the library recomputes from (seed, key) until the
                              row's first update writes it (the backward clears
                              the bit) -- the row offset is the value without it */
  int32_t* inverse;        /* [capacity] occurrence -> index into unique_* */
  int32_t* counts;         /* [capacity] occurrences of each distinct key */
  int32_t* bag_offsets;    /* [bag_capacity + 1]; insert_find writes its first
                              num_feats * batch + 1: merged CSR, bag f*batch + i */
  int64_t* num_unique;     /* [1] */
  int32_t* unique_offsets; /* [capacity + 1] start of each key's group in `grouped` */
  int32_t* grouped;        /* [capacity] bag ids (or occurrence ids) grouped by key */
  int32_t* plan;           /* [recis_plan_words(capacity)] opaque: backward work plan,
                              per-key IDMap slots, per-occurrence row references */
  int64_t capacity;
  int64_t bag_capacity;    /* merged bags bag_offsets has room for: insert_find returns
                              RECIS_ERR_INVALID_ARG, before any work, when
                              num_feats * batch exceeds it */
  int64_t n;               /* occurrences of the last insert_find */
  int32_t num_feats;
  int32_t batch;
  uint32_t flags;
  uint64_t epoch;          /* the table's update count at the lookup: while no update,
                              writeback or eviction has run since, forward and
                              backward use the lookup's row references directly;
                              otherwise they re-read each key's IDMap slot */
  uint64_t map_version;    /* the table's IDMap version after this lookup.  Every call
                              that can move a key to another slot or give it another
                              row bumps it: a counting insert_find (inserts, admissions,
                              growth), writeback, import and every eviction pass.  When
                              it differs at forward / backward, the call first re-probes
                              each distinct key (find only) and rewrites unique_rows and
                              the plan's per-key slots: a stale lookup then computes on
                              the rows its keys hold now (a key evicted since has none) */
} recis_lookup_result;

/* int32 words needed by recis_lookup_result.plan for `capacity` occurrences.
 * (Layout support for the lookup result; no passage of the pages.) */
int64_t recis_plan_words(int64_t capacity);

/* Hyper-parameters in double: the library derives 1 - beta1 and 1 - beta2 in
 * double before rounding them once to the float the kernels use. */
typedef struct {
  double lr, beta1, beta2, eps; /* Adam uses all four; Adagrad lr and eps */
} recis_optim_params;

typedef struct {
  int64_t keys;           /* keys in the IDMap (with or without a row) */
  int64_t rows_in_use;    /* rows held by keys */
  int64_t rows_allocated; /* rows covered by EmbeddingBlocks */
  int64_t blocks;
  int64_t slot_capacity;
  int64_t adam_step;
  int64_t bytes;          /* device bytes owned by the table (host blocks not included) */
  int64_t probationary_keys; /* keys in the IDMap without a row: admission has not
                                given them one yet (keys - rows_in_use) */
  int64_t claim_attempts; /* empty IDMap slots insert_find has tried to claim for a new
                             key since creation (a compare-and-swap: in the bucket's
                             shared-memory claim set, or on the slot itself for
                             overflowed and hot buckets) */
  int64_t claim_failures; /* of those, claims that found the slot already taken by
                             another key of the same call (the probe then moves on) */
  int64_t hbm_rows;       /* rows whose EmbeddingBlocks are in HBM: all of them for
                             RECIS_MEM_DEVICE, the hot tier for RECIS_MEM_HOST */
  int64_t lookup_pairs;   /* insert_find deduplicates each tile of 4096 consecutive
                             occurrences (merged order: feature-major, then bag) on
                             its own first: the distinct keys of each tile, summed
                             over the tiles of every call since creation.  The
                             later passes move one record per such pair, not one
                             per occurrence */
  int64_t hot_keys;       /* long keys (more than 64 occurrences in a call) whose gradient
                             sum the pooled backward took bag-major -- each bag's upstream
                             gradient row read once for all of them -- instead of key by
                             key, summed over every call since creation.  Per call and
                             feature at most 8192 / dim of the keys with the most
                             occurrences (dim 64 or 128; features in distinct feature
                             slots modulo 4096), each with at least 8 occurrences per
                             block of 2048 bags */
} recis_table_stats;

/* Creates a table.  Allocates the IDMap and `reserve_rows` worth of blocks
 * (synchronises `s` once).  Errors: INVALID_ARG (bad config, NULL out),
 * UNSUPPORTED (dim/dtype), OUT_OF_MEMORY, HIP.
 * Passage: page "RecIS (Recommendation Intelligence System)" README, section "Key optimisations > Efficient dynamic Embedding"
 * (a two-level store: IDMap of feature ID -> Offset over EmbeddingBlocks that
 * hold parameters and optimizer state, extended block by block) and section
 * "Key optimisations > Distributed optimisation" (tables of the same
 * attributes -- dimension, initializer -- merged into one). */
recis_status recis_idmap_create(const recis_table_config* cfg, const recis_allocator* alloc,
                                hipStream_t s, recis_table** out);

/* Releases everything the table owns.  No work on `t` may be pending.
 * Passage: page "RecIS (Recommendation Intelligence System)" README, section "Key optimisations > Efficient dynamic Embedding". */
recis_status recis_idmap_destroy(recis_table* t);

/* Lookup of one batch: transform + tag every value, merge the features
 * feature-major (bag f*batch + i), dedup, then per distinct key probe the
 * IDMap, insert on a miss (unless RECIS_FIND_ONLY), add its occurrences to
 * its count, give it a row initialised from (seed, key) with zero optimizer
 * state once the count reaches admit_threshold, and group the occurrences of
 * each key for the backward.  Grows the IDMap or the blocks first when the
 * batch could exceed them (may synchronise `s` then).
 * feats: host array [num_feats].  Errors: INVALID_ARG, OUT_OF_MEMORY, HIP,
 * CAPACITY (max_rows reached, host-detected); device: CAPACITY, KEY_RANGE,
 * INVALID_ARG (bag offsets).
 * Passage: page "RecIS (Recommendation Intelligence System)" README -- section "Core architecture > Feature Engine" (Hash, Mod,
 * Bucketize, fused); section "Key optimisations > Distributed optimisation"
 * (requests to tables of the same attributes merged and deduplicated);
 * section "Core architecture > Embedding Engine" (collision-free table,
 * admission); section "Key optimisations > Efficient dynamic Embedding"
 * (IDMap: feature ID as key, Offset as value). */
recis_status recis_idmap_insert_find(recis_table* t, const recis_feature_desc* feats,
                                     int32_t num_feats, int32_t batch, uint32_t flags,
                                     recis_lookup_result* res, hipStream_t s);

/* Eviction pass: removes every key whose count since the last pass is below
 * min_count (with or without a row), returns its row to the free list, and
 * restarts the surviving counts at 0.  num_evicted: device [1] (may be NULL).
 * Clears a standing CAPACITY error (the pass may have made room).
 * Passage: page "RecIS (Recommendation Intelligence System)" README, section "Core architecture > Embedding Engine" (feature
 * eviction and admission strategies). */
recis_status recis_idmap_evict(recis_table* t, uint32_t min_count, int64_t* num_evicted,
                               hipStream_t s);

/* Eviction pass with time-decayed counts: as recis_idmap_evict, except that
 * the surviving keys keep floor(count * decay) of their count instead of
 * restarting at 0 (decay in [0, 1]; 0 is recis_idmap_evict, 1 keeps running
 * totals).  A key then has to keep being seen to stay, with older
 * occurrences weighing less at every pass: one of the richer eviction and
 * admission strategies the pages leave open (page "RecIS (Recommendation
 * Intelligence System)" README, section "Core architecture > Embedding
 * Engine").  Admission still compares the count with admit_threshold.
 * Errors: INVALID_ARG (decay outside [0, 1]); as recis_idmap_evict. */
recis_status recis_idmap_evict_decay(recis_table* t, uint32_t min_count, double decay,
                                     int64_t* num_evicted, hipStream_t s);

/* LRU-bounded capacity: keeps at most max_keys keys, the most recently used.
 * A key's age is the number of counting insert_find calls (not FIND_ONLY)
 * since one last counted it (writeback and import stamp the keys they add
 * with the latest call); ages of 255 or more count as 255.  The pass keeps
 * the youngest ages whole, as many of them as fit in max_keys keys together,
 * and removes every older key, returning its row to the free list; counts are
 * untouched.  Another of the eviction strategies the pages leave open (page
 * "RecIS (Recommendation Intelligence System)" README, section "Core
 * architecture > Embedding Engine").  Needs track_last_use (else
 * UNSUPPORTED); max_keys >= 0.  num_evicted: device [1] (may be NULL).
 * Synchronises `s`. */
recis_status recis_idmap_evict_lru(recis_table* t, int64_t max_keys, int64_t* num_evicted,
                                   hipStream_t s);

/* Hot-tier placement for a table whose EmbeddingBlocks are in host memory
 * with an HBM tier (device_rows > 0): swaps rows so that the keys with the
 * highest counts hold the HBM rows.  Keys are ranked by their count since the
 * last eviction pass, in classes floor(log2(count)) + 1: the top classes that
 * fit the HBM tier together are hot.  Each hot key holding a host row
 * changes places with a key of a lower class holding an HBM row -- as many
 * pairs as both lists allow -- the two rows' parameters and optimizer state
 * (a row not yet written moves as its pending mark) and their IDMap entries
 * exchanged.  Content is unchanged: only where rows live.  The pages let
 * both levels of the table sit on the GPU or the CPU (page "RecIS
 * (Recommendation Intelligence System)" README, section "Key optimisations >
 * Efficient dynamic Embedding"); this keeps the frequent rows in HBM.
 * num_moved: device [1] (may be NULL), the keys moved into HBM.  Uses
 * 8 bytes per HBM row of temporary device memory from the allocator and
 * synchronises `s`.  Errors: UNSUPPORTED (blocks not in host memory, or no
 * HBM tier), OUT_OF_MEMORY, HIP. */
recis_status recis_idmap_retier(recis_table* t, int64_t* num_moved, hipStream_t s);

/* Forward: SUM / MEAN write float32 out [batch, num_feats * dim] with
 * out[i, f*dim + d] = pooled element d of bag (f, i) (mean divides by the bag
 * length; an empty bag gives 0; a key without a row adds zeros); NONE writes
 * out [N, dim] in the storage dtype, one row per occurrence.  Reads the rows
 * the lookup's keys hold when it runs (see map_version).
 * Passage: page "RecIS (Recommendation Intelligence System)" README, section "Key optimisations > Efficient use of hardware >
 * Operator implementation" (vectorised memory access) and section "Key
 * optimisations > Efficient dynamic Embedding" (the Offset names the row). */
recis_status recis_lookup_pool_fwd(const recis_table* t, const recis_lookup_result* res,
                                   int32_t pool, void* out, hipStream_t s);

/* Backward + update: G[u] = sum of the upstream gradients of u's occurrences
 * (grad_out [batch, num_feats*dim] for SUM / MEAN, divided by the bag length
 * for MEAN; grad_out [N, dim] for NONE, which needs RECIS_GROUP_BY_OCCURRENCE
 * at insert_find), summed in double, then one optimizer step on every
 * distinct key that has a row.  Adam's step counter is the table's and grows
 * by one per call.  grad_dtype: RECIS_DTYPE_F32 or RECIS_DTYPE_BF16.
 * Passage: page "RecIS (Recommendation Intelligence System)" README, section "Key optimisations > Efficient use of hardware >
 * Operator implementation" (reductions merged within a warp rather than by
 * atomics) and section "Key optimisations > Efficient dynamic Embedding"
 * (optimizer state stored in the EmbeddingBlocks beside the parameters). */
recis_status recis_pool_bwd_update(recis_table* t, const recis_lookup_result* res, int32_t pool,
                                   const void* grad_out, int32_t grad_dtype,
                                   const recis_optim_params* opt, hipStream_t s);

/* Allocation-free backward + update, for callers that cannot allocate device
 * memory while they run: code under HIP graph capture, tight training or
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, results and
 * errors as recis_pool_bwd_update, through the same kernels, but it calls no
 * allocator at all (neither hipMalloc nor the table's).  Its one scratch
 * buffer -- the long keys' double-precision chunk partials -- is a fixed array
 * of recis_noalloc_scratch_bytes() bytes (64 MiB) of device memory, one per
 * GPU, held until the process ends.  A call whose partials could exceed it
 * (at most n/32 + 2 chunks of dim doubles for n occurrences, about
 * n * dim / 4 bytes) returns RECIS_ERR_INVALID_ARG at once, before any work
 * (at dim 64: up to about 4.1M occurrences).  Every call on one GPU shares
 * the array, and each chunk's partial is written before it is read, so
 * nothing needs clearing between calls; calls that overlap on one GPU (other
 * streams, other tables) race on it and give undefined results. */
recis_status recis_pool_bwd_update_noalloc(recis_table* t, const recis_lookup_result* res, int32_t pool,
                                           const void* grad_out, int32_t grad_dtype,
                                           const recis_optim_params* opt, hipStream_t s);

/* Bytes of the fixed scratch array of recis_pool_bwd_update_noalloc. */
int64_t recis_noalloc_scratch_bytes(void);

/* Exact-assignment writeback: for i in order, row(keys[i]) <- rows[i] rounded
 * to the storage dtype, so the last occurrence of a repeated key wins.  An
 * absent key is inserted and given a row at once; counts are not touched.
 * keys: device [n] (>= 0); rows: device float32 [n, dim].
 * Passage: page "Memory Layer: Train the In-Model Cache for Recommendation
 * Models", sections "What carries the argument" and "Referee Report >
 * Summary" (the item tower's output written into the cache row by exact
 * assignment). */
recis_status recis_writeback(recis_table* t, const int64_t* keys, int64_t n, const float* rows,
                             hipStream_t s);

/* Copies the table out (synchronises `s`): keys device [cap], rows device
 * [cap] (-1 = no row), counts device [cap], params device [cap, dim] in the
 * storage dtype, state device float32 [cap, slots*dim] (may be NULL when the
 * optimizer has none); params and state 16-byte aligned.  *n receives the
 * number of keys (host); when it exceeds cap only cap entries are written.
 * Order unspecified.
 * Passage: page "RecIS (Recommendation Intelligence System)" README, section "Core architecture > Saver" (sparse parameters
 * stored and delivered as SafeTensors; this call is the device side). */
recis_status recis_idmap_export(recis_table* t, int64_t cap, int64_t* keys, int64_t* rows,
                                uint32_t* counts, void* params, float* state, int64_t* n,
                                hipStream_t s);

/* Restores a table saved from recis_idmap_export into this table, which must
 * never have held a key (else RECIS_ERR_INVALID_ARG at once).  Key i gets the
 * count counts[i] and, when rows[i] >= 0, a row holding params[i] (storage
 * dtype) and state[i] (float32; may be NULL when the optimizer has none);
 * rows[i] < 0 keeps the key without a row, as admission left it.  The row
 * numbers themselves are not kept.  adam_step (>= 0) sets the table's Adam
 * step counter.  keys, rows, counts: device [n]; params device [n, dim];
 * state device [n, slots*dim]; params and state 16-byte aligned.  Keys must be distinct and >= 0: a repeated
 * key records RECIS_ERR_INVALID_ARG and a negative one RECIS_ERR_KEY_RANGE in
 * the device error word.  The pages store and deliver sparse parameters in
 * the SafeTensors format (page "RecIS (Recommendation Intelligence System)"
 * README, section "Core architecture > Saver"); the file itself is written
 * and read above this call. */
recis_status recis_idmap_import(recis_table* t, int64_t n, const int64_t* keys, const int64_t* rows,
                                const uint32_t* counts, const void* params, const float* state,
                                int64_t adam_step, hipStream_t s);

/* The admission state beside the exported keys, so a save of a table that
 * keeps last-use stamps or a count-min sketch restores whole.
 * recis_idmap_key_ages: set 0 writes to ages[i] the age of keys[i] (counting
 * insert_find calls since one last counted it; ~0 for a key not in the
 * table); set 1 gives each key present the stamp that makes its age ages[i].
 * keys device [n], ages device [n].  Needs track_last_use (else UNSUPPORTED).
 * recis_idmap_sketch: set 0 copies the sketch's 4 x 2^admit_sketch_bits
 * counters (row after row) to `counters`; set 1 loads them from there.
 * counters: device.  Needs admit_sketch_bits > 0 (else UNSUPPORTED).
 * Both are stream-ordered; for restoring, call them after recis_idmap_import.
 * Passage: page "RecIS (Recommendation Intelligence System)" README, sections "Core architecture > Saver" and "Core
 * architecture > Embedding Engine" (admission state saved with the table). */
recis_status recis_idmap_key_ages(recis_table* t, const int64_t* keys, int64_t n, uint32_t* ages,
                                  int32_t set, hipStream_t s);
recis_status recis_idmap_sketch(recis_table* t, uint32_t* counters, int32_t set, hipStream_t s);

/* Table statistics (synchronises `s`); st: host.
 * Passage: page "RecIS (Recommendation Intelligence System)" README, section "Key optimisations > Efficient dynamic Embedding"
 * (IDMap, EmbeddingBlocks and where they live). */
recis_status recis_idmap_stats(recis_table* t, recis_table_stats* st, hipStream_t s);

/* Synchronises `s` and returns one error recorded on the device: KEY_RANGE,
 * then INVALID_ARG, each cleared as it is returned; then CAPACITY, which
 * stays (every later call returns it) until an eviction pass clears it.
 * RECIS_OK when none is recorded.  (The pages give no error model; the
 * sticky CAPACITY keeps a full table from being mistaken for a healthy one.) */
recis_status recis_get_error(recis_table* t, hipStream_t s);

/* Text of a status code (no passage of the pages: error reporting). */
const char* recis_status_string(recis_status st);

/* Instrumentation (not part of the method): while set, every launch of the
 * library kernel named `kernel` (e.g. "k_bwd_short", "k_fwd_pool",
 * "k_bucket_emit") made by a call on `t` is bracketed by
 * hipEventRecord(start) / hipEventRecord(stop) on the call's stream, so
 * hipEventElapsedTime(start, stop) is that launch's duration (the last one,
 * when a call launches it twice).  The events are the caller's and must stay
 * valid while set; kernel == NULL clears.  The name is copied.  Errors:
 * INVALID_ARG for a NULL table, or a name with NULL events. */
recis_status recis_profile_kernel(recis_table* t, const char* kernel, hipEvent_t start, hipEvent_t stop);

#ifdef __cplusplus
}
#endif

#endif /* RECIS_H */
