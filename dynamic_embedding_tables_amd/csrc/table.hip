// table.hip -- host side of the recis C ABI: argument checks, table memory
// (IDMap, EmbeddingBlocks, free list, scratch), growth, descriptor staging and
// the launches of each call.
//
// Pages: "RecIS (Recommendation Intelligence System)" README --
//   Key optimisations > Efficient dynamic Embedding: a two-level store whose
//   second level is made of blocks that are added as the table grows;
//   Core architecture > Embedding Engine: collision-free, extensible KV table.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>

#include "internal.h"

using namespace recis;

namespace recis {
thread_local const KernelProbe* tl_probe = nullptr;
}

namespace {

// Makes a table's kernel probe current for one call.
struct ScopedProbe {
  const KernelProbe* prev;
  explicit ScopedProbe(const recis_table* t) : prev(tl_probe) { tl_probe = &t->probe; }
  ~ScopedProbe() { tl_probe = prev; }
};

struct ScopedDevice {
  int prev = -1;
  explicit ScopedDevice(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev) (void)hipSetDevice(dev);
  }
  ~ScopedDevice() {
    int cur;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

void* default_alloc(void*, size_t bytes, hipStream_t) {
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return p;
}

void default_free(void*, void* p, hipStream_t) {
  if (p) (void)hipFree(p);
}

long long next_pow2(long long x) {
  long long p = 1;
  while (p < x) p <<= 1;
  return p;
}

int log2_exact(long long x) {
  int k = 0;
  while ((1ll << k) < x) ++k;
  return k;
}

bool valid_dim(int d) { return d == 8 || d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

void* tab_alloc(recis_table* t, size_t bytes, hipStream_t s) {
  if (bytes == 0) bytes = 256;
  void* p = t->alloc.alloc(t->alloc.ctx, bytes, s);
  if (p) t->bytes += (long long)bytes;
  return p;
}

void tab_free(recis_table* t, void* p, size_t bytes, hipStream_t s) {
  if (!p) return;
  t->alloc.free(t->alloc.ctx, p, s);
  t->bytes -= (long long)(bytes == 0 ? 256 : bytes);
}

#define HIP_TRY(x)                              \
  do {                                          \
    if ((x) != hipSuccess) {                    \
      (void)hipGetLastError();                  \
      return RECIS_ERR_HIP;                     \
    }                                           \
  } while (0)

recis_status check_launch() {
  if (hipPeekAtLastError() != hipSuccess) {
    (void)hipGetLastError();
    return RECIS_ERR_HIP;
  }
  return RECIS_OK;
}

// Adds blocks until at least `rows` rows are covered (capped at max_rows).
// One EmbeddingBlock: device memory from the allocator, or pinned host
// memory mapped for the GPU (non-coherent, so the GPU may cache it within a
// kernel; nothing else writes it while kernels run).
// Block i of a host-memory table goes to HBM while i is below the HBM tier's
// block count.
bool block_in_hbm(const recis_table* t, long long i) {
  if (t->cfg.block_memory != RECIS_MEM_HOST) return true;
  const long long br = t->cfg.block_rows;
  return i < (t->cfg.device_rows + br - 1) / br;
}

char* block_alloc(recis_table* t, size_t bytes, hipStream_t s) {
  if (block_in_hbm(t, (long long)t->blocks.size())) return static_cast<char*>(tab_alloc(t, bytes, s));
  void* h = nullptr;
  if (hipHostMalloc(&h, bytes, hipHostMallocMapped | hipHostMallocNonCoherent) != hipSuccess) return nullptr;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess || d != h) {  // one address for both sides
    (void)hipHostFree(h);
    return nullptr;
  }
  return static_cast<char*>(h);
}

void block_free(recis_table* t, long long i, char* b, hipStream_t s) {
  if (block_in_hbm(t, i)) {
    tab_free(t, b, (size_t)(t->cfg.block_rows * t->row_bytes), s);
    return;
  }
  (void)hipHostFree(b);
}

recis_status grow_rows(recis_table* t, long long rows, hipStream_t s) {
  rows = std::min<long long>(rows, t->cfg.max_rows);
  if (rows <= t->rows_alloc) return RECIS_OK;
  const long long br = t->cfg.block_rows;
  const long long nblocks = (rows + br - 1) / br;
  HIP_TRY(hipStreamSynchronize(s));
  // block pointer table
  if (nblocks > t->d_blocks_cap) {
    long long cap = std::max<long long>(16, t->d_blocks_cap);
    while (cap < nblocks) cap *= 2;
    char** nb = static_cast<char**>(tab_alloc(t, cap * sizeof(char*), s));
    if (!nb) return RECIS_ERR_OUT_OF_MEMORY;
    if (t->d_blocks) tab_free(t, t->d_blocks, t->d_blocks_cap * sizeof(char*), s);
    t->d_blocks = nb;
    t->d_blocks_cap = cap;
  }
  while ((long long)t->blocks.size() < nblocks) {
    char* b = block_alloc(t, (size_t)(br * t->row_bytes), s);
    if (!b) return RECIS_ERR_OUT_OF_MEMORY;
    t->blocks.push_back(b);
  }
  HIP_TRY(hipMemcpyAsync(t->d_blocks, t->blocks.data(), t->blocks.size() * sizeof(char*),
                         hipMemcpyHostToDevice, s));
  const long long new_rows = (long long)t->blocks.size() * br;
  // free list must hold every row
  if (new_rows > t->free_cap) {
    int* nf = static_cast<int*>(tab_alloc(t, (size_t)new_rows * sizeof(int), s));
    if (!nf) return RECIS_ERR_OUT_OF_MEMORY;
    if (t->free_list) {
      HIP_TRY(hipMemcpyAsync(nf, t->free_list, (size_t)t->free_cap * sizeof(int), hipMemcpyDeviceToDevice, s));
      HIP_TRY(hipStreamSynchronize(s));
      tab_free(t, t->free_list, (size_t)t->free_cap * sizeof(int), s);
    }
    t->free_list = nf;
    t->free_cap = new_rows;
  }
  HIP_TRY(hipStreamSynchronize(s));
  t->rows_alloc = std::min<long long>(new_rows, t->cfg.max_rows);
  return RECIS_OK;
}

// Rebuilds the IDMap into `new_cap` slots (growth or after eviction).
recis_status rebuild_idmap(recis_table* t, long long new_cap, hipStream_t s) {
  Slot* old = t->slots;
  unsigned* old_lu = t->last_use;
  const long long old_cap = t->slot_cap;
  Slot* ns = static_cast<Slot*>(tab_alloc(t, (size_t)new_cap * sizeof(Slot), s));
  if (!ns) return RECIS_ERR_OUT_OF_MEMORY;
  unsigned* nlu = nullptr;
  if (old_lu) {  // last-use stamps move with their keys
    nlu = static_cast<unsigned*>(tab_alloc(t, (size_t)new_cap * sizeof(unsigned), s));
    if (!nlu) {
      tab_free(t, ns, (size_t)new_cap * sizeof(Slot), s);
      return RECIS_ERR_OUT_OF_MEMORY;
    }
  }
  launch_fill_slots(ns, new_cap, s);
  t->slots = ns;
  t->last_use = nlu;
  t->slot_cap = new_cap;
  launch_rehash(old, old_lu, old_cap, t->dev(), s);
  recis_status st = check_launch();
  HIP_TRY(hipStreamSynchronize(s));
  tab_free(t, old, (size_t)old_cap * sizeof(Slot), s);
  if (old_lu) tab_free(t, old_lu, (size_t)old_cap * sizeof(unsigned), s);
  return st;
}

recis_status read_counters(recis_table* t, DevCounters* c, hipStream_t s) {
  HIP_TRY(hipStreamSynchronize(s));
  HIP_TRY(hipMemcpy(c, t->ctr, sizeof(DevCounters), hipMemcpyDeviceToHost));
  return RECIS_OK;
}

// Makes room for a call that may add up to n keys and n rows.
recis_status ensure_capacity(recis_table* t, long long n, hipStream_t s) {
  const long long max_keys = (long long)(t->cfg.max_load * (double)t->slot_cap);
  const bool rows_tight = t->rows_hi + n > t->rows_alloc && t->rows_alloc < t->cfg.max_rows;
  const bool keys_tight = t->keys_hi + n > max_keys;
  if (rows_tight || keys_tight) {
    DevCounters c;
    recis_status st = read_counters(t, &c, s);
    if (st != RECIS_OK) return st;
    t->rows_hi = (long long)c.next_row;
    t->keys_hi = (long long)c.num_keys;
    const long long free_rows = c.free_top > 0 ? c.free_top : 0;
    const long long need_rows = t->rows_hi + std::max<long long>(0, n - free_rows);
    if (need_rows > t->rows_alloc) {
      st = grow_rows(t, need_rows + t->cfg.block_rows, s);
      if (st != RECIS_OK) return st;
    }
    long long cap = t->slot_cap;
    while ((long long)(t->cfg.max_load * (double)cap) < t->keys_hi + n) cap *= 2;
    if (cap != t->slot_cap) {
      if (cap > kMaxSlots) return RECIS_ERR_CAPACITY;
      st = rebuild_idmap(t, cap, s);
      if (st != RECIS_OK) return st;
    }
  }
  t->rows_hi += n;
  t->keys_hi += n;
  return RECIS_OK;
}

// IDMap regions: as many as the lookup's buckets can be (kMaxBuckets), but
// none smaller than 2^kMinRegionSlotBits slots.
int region_bits_for(long long slot_cap) {
  const int sb = log2_exact(slot_cap);
  return std::max(0, std::min(kMaxBucketBits, sb - kMinRegionSlotBits));
}

// Hash-partition geometry of a call with n occurrences: buckets of about
// kBucketOcc occurrences, but at least kMinBuckets of them (a small call's
// bucket blocks then spread over the CUs instead of queueing a few long
// chains), a power of two, at most kMaxBuckets; tiles of kTileOcc
// occurrences, partition blocks of whole tiles (at most kMaxPartBlocks).
struct PartGeom {
  int nbits, nbk, blocks, big;
  long long ntiles, tiles_per_block;
};
// Buckets never outnumber the IDMap's regions (max_bits), so that each
// bucket's block owns whole regions.
PartGeom part_geom(long long n, int max_bits = kMaxBucketBits) {
  PartGeom g;
  const long long want = std::max<long long>(kMinBuckets, (n + kBucketOcc - 1) / kBucketOcc);
  g.nbk = (int)std::min<long long>(next_pow2(want), 1ll << max_bits);
  g.nbits = log2_exact(g.nbk);
  g.ntiles = std::max<long long>(1, (n + kTileOcc - 1) / kTileOcc);
  g.tiles_per_block = (g.ntiles + kMaxPartBlocks - 1) / kMaxPartBlocks;
  g.blocks = (int)((g.ntiles + g.tiles_per_block - 1) / g.tiles_per_block);
  g.big = n > (long long)g.nbk * kSmallTabOcc ? 1 : 0;
  return g;
}

// Bytes of each per-step scratch array for cap occurrences.
struct ScratchSizes {
  size_t dd, part, hist, bbase, uslot, pout, blk, wb, partials, tkey, tcnt, tile_n, occ_local;
};
ScratchSizes scratch_sizes(long long cap, int dim) {
  ScratchSizes z;
  const PartGeom g = part_geom(cap);
  z.dd = (size_t)(2 * cap) * sizeof(DedupSlot);
  z.part = (size_t)cap * sizeof(PartEntry);
  // a call of n <= cap occurrences has at most min(kMaxPartBlocks, its tiles)
  // partition blocks and at most cap's buckets
  z.hist = (size_t)std::min<long long>(kMaxPartBlocks, g.ntiles) * (size_t)g.nbk * 4;
  z.bbase = (size_t)(kMaxBuckets + 1) * 4 * 3;  // bbase, ubase, obase
  z.uslot = (size_t)cap * 4;
  const size_t tiled = (size_t)g.ntiles * kTileOcc;  // pair slots, whole tiles
  z.pout = tiled * sizeof(PartOut);
  z.tkey = tiled * 8;
  z.tcnt = tiled * 4;
  z.tile_n = (size_t)(g.ntiles + 1) * 4 * 2;  // tile_n, then tile_bag
  z.occ_local = (size_t)cap * 2;
  z.blk = (size_t)(kMaxBuckets + 2) * 8 * 3;  // per-bucket sums: blk_sums, blk_long, blk_claim
  z.wb = (size_t)cap * 8;
  z.partials = (size_t)plan_layout(cap).max_chunks * (size_t)dim * 8;
  return z;
}

void free_scratch(recis_table* t, hipStream_t s) {
  if (!t->scr_cap) return;
  const ScratchSizes z = scratch_sizes(t->scr_cap, t->cfg.dim);
  tab_free(t, t->dd, z.dd, s);
  tab_free(t, t->part, z.part, s);
  tab_free(t, t->hist, z.hist, s);
  tab_free(t, t->bbase, z.bbase, s);
  tab_free(t, t->uslot, z.uslot, s);
  tab_free(t, t->pout, z.pout, s);
  tab_free(t, t->blk_sums, z.blk, s);
  tab_free(t, t->wb_keys, z.wb, s);
  tab_free(t, t->partials, z.partials, s);
  tab_free(t, t->tkey, z.tkey, s);
  tab_free(t, t->tcnt, z.tcnt, s);
  tab_free(t, t->tile_n, z.tile_n, s);
  tab_free(t, t->occ_local, z.occ_local, s);
  t->tkey = nullptr;
  t->tcnt = t->tile_n = nullptr;
  t->occ_local = nullptr;
  t->dd = nullptr;
  t->part = nullptr;
  t->hist = t->bbase = t->ubase = t->uslot = nullptr;
  t->pout = nullptr;
  t->blk_sums = nullptr;
  t->wb_keys = nullptr;
  t->partials = nullptr;
  t->scr_cap = 0;
  t->dd_cap = 0;
}

// Per-step scratch sized for n occurrences.
recis_status ensure_scratch(recis_table* t, long long n, hipStream_t s) {
  if (n <= t->scr_cap && t->dd) return RECIS_OK;
  const long long cap = std::max<long long>(next_pow2(std::max<long long>(n, 1)), 4096);
  HIP_TRY(hipStreamSynchronize(s));
  free_scratch(t, s);
  const ScratchSizes z = scratch_sizes(cap, t->cfg.dim);
  t->scr_cap = cap;  // sizes of whatever is allocated below, for free_scratch
  t->dd_cap = 2 * cap;
  t->dd = static_cast<DedupSlot*>(tab_alloc(t, z.dd, s));
  t->part = static_cast<PartEntry*>(tab_alloc(t, z.part, s));
  t->hist = static_cast<int*>(tab_alloc(t, z.hist, s));
  t->bbase = static_cast<int*>(tab_alloc(t, z.bbase, s));
  t->ubase = t->bbase ? t->bbase + (kMaxBuckets + 1) : nullptr;
  t->uslot = static_cast<int*>(tab_alloc(t, z.uslot, s));
  t->pout = static_cast<recis::PartOut*>(tab_alloc(t, z.pout, s));
  t->blk_sums = static_cast<unsigned long long*>(tab_alloc(t, z.blk, s));
  t->wb_keys = static_cast<long long*>(tab_alloc(t, z.wb, s));
  t->partials = static_cast<double*>(tab_alloc(t, z.partials, s));
  t->tkey = static_cast<long long*>(tab_alloc(t, z.tkey, s));
  t->tcnt = static_cast<int*>(tab_alloc(t, z.tcnt, s));
  t->tile_n = static_cast<int*>(tab_alloc(t, z.tile_n, s));
  t->occ_local = static_cast<unsigned short*>(tab_alloc(t, z.occ_local, s));
  if (!t->dd || !t->part || !t->hist || !t->bbase || !t->uslot || !t->pout || !t->blk_sums || !t->wb_keys ||
      !t->partials || !t->tkey || !t->tcnt || !t->tile_n || !t->occ_local) {
    free_scratch(t, s);
    return RECIS_ERR_OUT_OF_MEMORY;
  }
  launch_fill_dedup(t->dd, t->dd_cap, s);
  return check_launch();
}

// Copies `bytes` of host data to device memory through the pinned ring.
recis_status stage(recis_table* t, const void* src, size_t bytes, hipStream_t s, void** dev_out) {
  const int k = t->ring_pos;
  t->ring_pos = (t->ring_pos + 1) % recis_table::kRing;
  if (t->stage_ev[k]) HIP_TRY(hipEventSynchronize(t->stage_ev[k]));
  if (bytes > t->stage_cap[k]) {
    size_t cap = std::max<size_t>(bytes, 4096);
    if (t->stage_host[k]) (void)hipHostFree(t->stage_host[k]);
    if (t->stage_dev[k]) tab_free(t, t->stage_dev[k], t->stage_cap[k], s);
    t->stage_host[k] = nullptr;
    t->stage_dev[k] = nullptr;
    t->stage_cap[k] = 0;
    HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&t->stage_host[k]), cap, hipHostMallocDefault));
    t->stage_dev[k] = static_cast<char*>(tab_alloc(t, cap, s));
    if (!t->stage_dev[k]) return RECIS_ERR_OUT_OF_MEMORY;
    t->stage_cap[k] = cap;
  }
  if (!t->stage_ev[k]) HIP_TRY(hipEventCreateWithFlags(&t->stage_ev[k], hipEventDisableTiming));
  std::memcpy(t->stage_host[k], src, bytes);
  HIP_TRY(hipMemcpyAsync(t->stage_dev[k], t->stage_host[k], bytes, hipMemcpyHostToDevice, s));
  HIP_TRY(hipEventRecord(t->stage_ev[k], s));
  *dev_out = t->stage_dev[k];
  return RECIS_OK;
}

// Rows whose blocks are in HBM (the allocated ones).
long long hbm_rows(const recis_table* t) {
  if (t->cfg.block_memory != RECIS_MEM_HOST) return t->rows_alloc;
  const long long br = t->cfg.block_rows;
  const long long nb = std::min<long long>((long long)t->blocks.size(), (t->cfg.device_rows + br - 1) / br);
  return std::min<long long>(nb * br, t->rows_alloc);
}

}  // namespace

TableDev recis_table::dev() const {
  TableDev d;
  d.slots = slots;
  d.slot_mask = (unsigned long long)(slot_cap - 1);
  d.slot_shift = 64 - log2_exact(slot_cap);
  d.region_bits = region_bits_for(slot_cap);
  d.region_mask = (unsigned long long)((slot_cap >> d.region_bits) - 1);
  d.ctr = ctr;
  d.free_list = free_list;
  d.rs.blocks = d_blocks;
  d.rs.lb = lb;
  d.rs.mb = cfg.block_rows - 1;
  d.rs.stride = row_bytes;
  d.dim = cfg.dim;
  d.dtype = cfg.dtype;
  d.optim = cfg.optim;
  d.state_words = state_words;
  d.admit = cfg.admit_threshold == 0 ? 1u : cfg.admit_threshold;
  d.seed = cfg.seed;
  d.init_scale = std::ldexp(cfg.init_bound, -23);
  d.rows_limit = rows_alloc;
  d.last_use = last_use;
  d.step = step;
  d.sketch = sketch;
  d.sketch_bits = cfg.admit_sketch_bits;
  return d;
}

extern "C" {

void recis_table_config_default(recis_table_config* c) {
  if (!c) return;
  std::memset(c, 0, sizeof(*c));
  c->dim = 64;
  c->dtype = RECIS_DTYPE_F32;
  c->optim = RECIS_OPTIM_ADAGRAD;
  c->admit_threshold = 1;
  c->seed = 20250925ull;
  c->init_bound = 0.05f;
  c->max_load = 0.5f;
  c->slot_capacity = 1ll << 20;
  c->block_rows = 1ll << 20;
  c->max_rows = kMaxRows;
  c->reserve_rows = 0;
}

int64_t recis_plan_words(int64_t capacity) {
  if (capacity < 0) return -1;
  return plan_layout(capacity).words;
}

recis_status recis_idmap_create(const recis_table_config* cfg, const recis_allocator* alloc, hipStream_t s,
                                recis_table** out) {
  if (!cfg || !out) return RECIS_ERR_INVALID_ARG;
  *out = nullptr;
  if (cfg->dtype != RECIS_DTYPE_F32 && cfg->dtype != RECIS_DTYPE_BF16) return RECIS_ERR_INVALID_ARG;
  if (cfg->optim < RECIS_OPTIM_NONE || cfg->optim > RECIS_OPTIM_ADAM) return RECIS_ERR_INVALID_ARG;
  if (!(cfg->max_load > 0.f && cfg->max_load <= 0.75f)) return RECIS_ERR_INVALID_ARG;
  if (!std::isfinite(cfg->init_bound) || cfg->init_bound < 0.f) return RECIS_ERR_INVALID_ARG;
  if (cfg->slot_capacity < 1 || cfg->slot_capacity > kMaxSlots) return RECIS_ERR_INVALID_ARG;
  if (cfg->block_rows < 1 || cfg->block_rows > (1ll << 30)) return RECIS_ERR_INVALID_ARG;
  if (cfg->max_rows < 1 || cfg->max_rows > kMaxRows) return RECIS_ERR_INVALID_ARG;
  if (cfg->reserve_rows < 0) return RECIS_ERR_INVALID_ARG;
  if (cfg->block_memory != RECIS_MEM_DEVICE && cfg->block_memory != RECIS_MEM_HOST) return RECIS_ERR_INVALID_ARG;
  if (cfg->track_last_use != 0 && cfg->track_last_use != 1) return RECIS_ERR_INVALID_ARG;
  if (cfg->admit_sketch_bits < 0 || cfg->admit_sketch_bits > 30) return RECIS_ERR_INVALID_ARG;
  if (cfg->device_rows < 0) return RECIS_ERR_INVALID_ARG;
  if (alloc && (!alloc->alloc || !alloc->free)) return RECIS_ERR_INVALID_ARG;
  if (!valid_dim(cfg->dim)) return RECIS_ERR_UNSUPPORTED;

  recis_table* t = new (std::nothrow) recis_table();
  if (!t) return RECIS_ERR_OUT_OF_MEMORY;
  t->cfg = *cfg;
  t->cfg.block_rows = std::max<long long>(next_pow2(cfg->block_rows), 64);
  t->lb = log2_exact(t->cfg.block_rows);
  t->own_alloc = alloc == nullptr;
  if (alloc) t->alloc = *alloc;
  else t->alloc = recis_allocator{nullptr, default_alloc, default_free};
  t->state_words = cfg->optim == RECIS_OPTIM_ADAM ? 2 : (cfg->optim == RECIS_OPTIM_ADAGRAD ? 1 : 0);
  t->row_bytes = (long long)cfg->dim * (cfg->dtype == RECIS_DTYPE_BF16 ? 2 : 4) +
                 (long long)t->state_words * cfg->dim * 4;

  auto fail = [&](recis_status st) {
    recis_idmap_destroy(t);
    return st;
  };
  t->ctr = static_cast<DevCounters*>(tab_alloc(t, sizeof(DevCounters), s));
  if (!t->ctr) return fail(RECIS_ERR_OUT_OF_MEMORY);
  if (hipGetDevice(&t->device) != hipSuccess) return fail(RECIS_ERR_HIP);
  DevCounters zero;
  std::memset(&zero, 0, sizeof(zero));
  if (hipMemcpyAsync(t->ctr, &zero, sizeof(zero), hipMemcpyHostToDevice, s) != hipSuccess) return fail(RECIS_ERR_HIP);
  t->slot_cap = std::max<long long>(next_pow2(cfg->slot_capacity), 64);
  t->slots = static_cast<Slot*>(tab_alloc(t, (size_t)t->slot_cap * sizeof(Slot), s));
  if (!t->slots) return fail(RECIS_ERR_OUT_OF_MEMORY);
  if (cfg->admit_sketch_bits > 0) {
    const long long n = (long long)kSketchRows << cfg->admit_sketch_bits;
    t->sketch = static_cast<unsigned*>(tab_alloc(t, (size_t)n * sizeof(unsigned), s));
    if (!t->sketch) return fail(RECIS_ERR_OUT_OF_MEMORY);
    launch_zero_u32(t->sketch, n, s);
  }
  if (cfg->track_last_use) {  // stamped whenever a key enters; empty slots' stamps are never read
    t->last_use = static_cast<unsigned*>(tab_alloc(t, (size_t)t->slot_cap * sizeof(unsigned), s));
    if (!t->last_use) return fail(RECIS_ERR_OUT_OF_MEMORY);
  }
  launch_fill_slots(t->slots, t->slot_cap, s);
  if (check_launch() != RECIS_OK) return fail(RECIS_ERR_HIP);
  recis_status st = grow_rows(t, std::max<long long>(cfg->reserve_rows, 1), s);
  if (st != RECIS_OK) return fail(st);
  if (hipStreamSynchronize(s) != hipSuccess) return fail(RECIS_ERR_HIP);
  *out = t;
  return RECIS_OK;
}

recis_status recis_idmap_destroy(recis_table* t) {
  if (!t) return RECIS_ERR_INVALID_ARG;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  hipStream_t s = nullptr;
  (void)hipDeviceSynchronize();
  for (size_t i = 0; i < t->blocks.size(); ++i) block_free(t, (long long)i, t->blocks[i], s);
  tab_free(t, t->d_blocks, t->d_blocks_cap * sizeof(char*), s);
  tab_free(t, t->free_list, (size_t)t->free_cap * 4, s);
  tab_free(t, t->slots, (size_t)t->slot_cap * sizeof(Slot), s);
  tab_free(t, t->last_use, (size_t)t->slot_cap * sizeof(unsigned), s);
  tab_free(t, t->sketch, (size_t)((long long)kSketchRows << t->cfg.admit_sketch_bits) * sizeof(unsigned), s);
  tab_free(t, t->ctr, sizeof(DevCounters), s);
  tab_free(t, t->hot_partials, (size_t)t->hot_rows * (size_t)t->cfg.dim * 8, s);
  tab_free(t, t->hot_ws, (size_t)t->hot_ws_len * 4, s);
  free_scratch(t, s);
  for (int k = 0; k < recis_table::kRing; ++k) {
    if (t->stage_host[k]) (void)hipHostFree(t->stage_host[k]);
    if (t->stage_dev[k]) tab_free(t, t->stage_dev[k], t->stage_cap[k], s);
    if (t->stage_ev[k]) (void)hipEventDestroy(t->stage_ev[k]);
  }
  delete t;
  return RECIS_OK;
}

recis_status recis_idmap_insert_find(recis_table* t, const recis_feature_desc* feats, int32_t num_feats,
                                     int32_t batch, uint32_t flags, recis_lookup_result* res, hipStream_t s) {
  if (!t || !res || num_feats < 0 || batch < 0) return RECIS_ERR_INVALID_ARG;
  if (num_feats > 0 && !feats) return RECIS_ERR_INVALID_ARG;
  if (flags & ~(RECIS_FIND_ONLY | RECIS_GROUP_BY_OCCURRENCE)) return RECIS_ERR_INVALID_ARG;
  if ((long long)num_feats * batch >= (1ll << 31) - 1) return RECIS_ERR_INVALID_ARG;
  long long N = 0, nbounds = 0;
  for (int f = 0; f < num_feats; ++f) {
    const recis_feature_desc& d = feats[f];
    if (d.n < 0 || (d.n > 0 && !d.values) || !d.bag_offsets) return RECIS_ERR_INVALID_ARG;
    if (batch == 0 && d.n != 0) return RECIS_ERR_INVALID_ARG;
    if (d.slot >= (1u << 15)) return RECIS_ERR_INVALID_ARG;
    if (d.ops & ~(RECIS_OP_HASH | RECIS_OP_MOD | RECIS_OP_BUCKETIZE)) return RECIS_ERR_INVALID_ARG;
    if ((d.ops & RECIS_OP_BUCKETIZE) && (d.ops & (RECIS_OP_HASH | RECIS_OP_MOD))) return RECIS_ERR_INVALID_ARG;
    if ((d.ops & RECIS_OP_MOD) && d.mod == 0) return RECIS_ERR_INVALID_ARG;
    if ((d.ops & RECIS_OP_MOD) && !(d.ops & RECIS_OP_HASH) && d.mod > (uint64_t)INT64_MAX)
      return RECIS_ERR_INVALID_ARG;
    if (d.ops & RECIS_OP_BUCKETIZE) {
      if (d.nb < 0 || (d.nb > 0 && !d.boundaries) || d.nb > (1 << 30)) return RECIS_ERR_INVALID_ARG;
      for (long long i = 1; i < d.nb; ++i)
        if (!(d.boundaries[i - 1] < d.boundaries[i])) return RECIS_ERR_INVALID_ARG;
      nbounds += d.nb;
    }
    N += d.n;
  }
  if (N > (1ll << 30) || N > res->capacity) return RECIS_ERR_INVALID_ARG;
  if ((long long)num_feats * batch > res->bag_capacity) return RECIS_ERR_INVALID_ARG;
  if (!res->bag_offsets || !res->num_unique || !res->unique_offsets || !res->plan) return RECIS_ERR_INVALID_ARG;
  if (N > 0 && (!res->unique_keys || !res->unique_rows || !res->inverse || !res->counts || !res->grouped))
    return RECIS_ERR_INVALID_ARG;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);

  recis_status st = ensure_scratch(t, N, s);
  if (st != RECIS_OK) return st;
  if (!(flags & RECIS_FIND_ONLY)) {
    st = ensure_capacity(t, N, s);
    if (st != RECIS_OK) return st;
  }

  // descriptors + boundary pool, staged in one copy
  std::vector<char> host(sizeof(FeatDev) * (size_t)std::max(num_feats, 1) + 8 * (size_t)nbounds + 16);
  FeatDev* fd = reinterpret_cast<FeatDev*>(host.data());
  long long* pool = reinterpret_cast<long long*>(host.data() + sizeof(FeatDev) * (size_t)std::max(num_feats, 1));
  long long base = 0, boff = 0;
  for (int f = 0; f < num_feats; ++f) {
    const recis_feature_desc& d = feats[f];
    fd[f].values = reinterpret_cast<const long long*>(d.values);
    fd[f].offs = d.bag_offsets;
    fd[f].n = d.n;
    fd[f].base = base;
    fd[f].mod = d.mod;
    fd[f].mod_inv = (d.ops & RECIS_OP_MOD) ? ~0ull / d.mod : 0;
    fd[f].slot = d.slot;
    fd[f].ops = d.ops;
    fd[f].bnd_off = (int)boff;
    fd[f].nb = (d.ops & RECIS_OP_BUCKETIZE) ? (int)d.nb : 0;
    if (d.ops & RECIS_OP_BUCKETIZE) {
      std::memcpy(pool + boff, d.boundaries, (size_t)d.nb * 8);
      boff += d.nb;
    }
    base += d.n;
  }
  void* dev = nullptr;
  st = stage(t, host.data(), host.size(), s, &dev);
  if (st != RECIS_OK) return st;

  res->n = N;
  res->num_feats = num_feats;
  res->batch = batch;
  res->flags = flags;
  res->epoch = t->update_epoch;
  if (!(flags & RECIS_FIND_ONLY)) t->map_version += 1;  // inserts, admissions, growth
  res->map_version = t->map_version;

  LookupLaunch L;
  L.feats = static_cast<const FeatDev*>(dev);
  L.bnd_pool = reinterpret_cast<const long long*>(static_cast<char*>(dev) + sizeof(FeatDev) * (size_t)std::max(num_feats, 1));
  L.F = num_feats;
  L.B = batch;
  L.N = N;
  L.flags = flags;
  L.res = *res;
  L.dd = t->dd;
  const PartGeom g = part_geom(N, region_bits_for(t->slot_cap));
  L.nbits = g.nbits;
  L.nbk = g.nbk;
  L.part_blocks = g.blocks;
  L.tiles_per_block = g.tiles_per_block;
  L.ntiles = g.ntiles;
  L.tkey = t->tkey;
  L.tcnt = t->tcnt;
  L.tile_n = t->tile_n;
  L.tile_bag = t->tile_n + (g.ntiles + 1);
  L.occ_local = t->occ_local;
  L.obase = t->bbase + 2 * (kMaxBuckets + 1);
  L.big_tab = g.big;
  // the backward's hot-key pass needs each feature's own bin
  L.hot_ok = 0;
  if (!(flags & RECIS_GROUP_BY_OCCURRENCE) && num_feats <= kFeatBins && N > 0) {
    std::vector<unsigned char> used(kFeatBins, 0);
    L.hot_ok = 1;
    for (int f = 0; f < num_feats && L.hot_ok; ++f) {
      const unsigned bin = feats[f].slot & (kFeatBins - 1);
      if (used[bin]) L.hot_ok = 0;
      used[bin] = 1;
    }
  }
  L.hist = t->hist;
  L.bbase = t->bbase;
  L.ubase = t->ubase;
  L.part = t->part;
  L.pout = t->pout;
  L.blk_sums = t->blk_sums;
  L.blk_long = t->blk_sums + (kMaxBuckets + 2);
  L.blk_claim = t->blk_sums + 2 * (kMaxBuckets + 2);
  // heavy-bucket bookkeeping lives in the writeback scratch (the two never
  // share a call): the distinct-key list in uslot (N ints), the slice list in
  // wb_keys (2 N ints)
  L.klist = t->uslot;
  L.hslice = reinterpret_cast<int*>(t->wb_keys);
  L.hmax = N / kSliceOcc + N / kHeavyOcc + 1;
  const bool counting = (flags & RECIS_FIND_ONLY) == 0;
  if (counting) t->step += 1;
  L.last_use = counting ? t->last_use : nullptr;
  L.step = t->step;
  L.sketching = counting && t->sketch ? 1 : 0;
  launch_lookup(L, t->dev(), s);
  return check_launch();
}

recis_status recis_idmap_evict_decay(recis_table* t, uint32_t min_count, double decay, int64_t* num_evicted,
                                     hipStream_t s) {
  if (!t || !(decay >= 0.0 && decay <= 1.0)) return RECIS_ERR_INVALID_ARG;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  t->update_epoch += 1;
  t->map_version += 1;
  if (t->sketch) launch_zero_u32(t->sketch, (long long)kSketchRows << t->cfg.admit_sketch_bits, s);
  launch_evict(t->dev(), min_count, decay, reinterpret_cast<long long*>(num_evicted), s);
  recis_status st = check_launch();
  if (st != RECIS_OK) return st;
  st = rebuild_idmap(t, t->slot_cap, s);
  if (st != RECIS_OK) return st;
  launch_clear_error(t->ctr, kErrCapacity, s);  // the pass may have made room
  DevCounters c;
  st = read_counters(t, &c, s);
  if (st != RECIS_OK) return st;
  t->rows_hi = (long long)c.next_row;
  t->keys_hi = (long long)c.num_keys;
  return RECIS_OK;
}

recis_status recis_idmap_evict(recis_table* t, uint32_t min_count, int64_t* num_evicted, hipStream_t s) {
  return recis_idmap_evict_decay(t, min_count, 0.0, num_evicted, s);
}

recis_status recis_idmap_evict_lru(recis_table* t, int64_t max_keys, int64_t* num_evicted, hipStream_t s) {
  if (!t || max_keys < 0) return RECIS_ERR_INVALID_ARG;
  if (!t->last_use) return RECIS_ERR_UNSUPPORTED;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  const size_t wbytes = (size_t)age_hist_words(t->slot_cap) * sizeof(int);
  int* work = static_cast<int*>(tab_alloc(t, wbytes, s));
  if (!work) return RECIS_ERR_OUT_OF_MEMORY;
  t->update_epoch += 1;
  t->map_version += 1;
  if (t->sketch) launch_zero_u32(t->sketch, (long long)kSketchRows << t->cfg.admit_sketch_bits, s);
  launch_evict_lru(t->dev(), max_keys, work, reinterpret_cast<long long*>(num_evicted), s);
  recis_status st = check_launch();
  if (st == RECIS_OK) st = rebuild_idmap(t, t->slot_cap, s);  // synchronises: work is idle after
  tab_free(t, work, wbytes, s);
  if (st != RECIS_OK) return st;
  launch_clear_error(t->ctr, kErrCapacity, s);  // the pass may have made room
  DevCounters c;
  st = read_counters(t, &c, s);
  if (st != RECIS_OK) return st;
  t->rows_hi = (long long)c.next_row;
  t->keys_hi = (long long)c.num_keys;
  return RECIS_OK;
}

recis_status recis_idmap_retier(recis_table* t, int64_t* num_moved, hipStream_t s) {
  if (!t) return RECIS_ERR_INVALID_ARG;
  if (t->cfg.block_memory != RECIS_MEM_HOST || t->cfg.device_rows <= 0) return RECIS_ERR_UNSUPPORTED;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  const long long H = hbm_rows(t);
  const size_t wbytes = (size_t)retier_words(t->slot_cap, H) * sizeof(int);
  int* work = static_cast<int*>(tab_alloc(t, wbytes, s));
  if (!work) return RECIS_ERR_OUT_OF_MEMORY;
  t->update_epoch += 1;  // rows move: lookups made before re-probe their keys
  t->map_version += 1;
  launch_retier(t->dev(), H, work, reinterpret_cast<long long*>(num_moved), s);
  recis_status st = check_launch();
  if (hipStreamSynchronize(s) != hipSuccess) st = RECIS_ERR_HIP;
  tab_free(t, work, wbytes, s);
  return st;
}

recis_status recis_lookup_pool_fwd(const recis_table* t, const recis_lookup_result* res, int32_t pool, void* out,
                                   hipStream_t s) {
  if (!t || !res) return RECIS_ERR_INVALID_ARG;
  if (pool != RECIS_POOL_SUM && pool != RECIS_POOL_MEAN && pool != RECIS_POOL_NONE) return RECIS_ERR_INVALID_ARG;
  const long long outn = pool == RECIS_POOL_NONE ? res->n : (long long)res->num_feats * res->batch;
  if (outn > 0 && !out) return RECIS_ERR_INVALID_ARG;
  if (res->n > res->capacity || res->n < 0) return RECIS_ERR_INVALID_ARG;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  const bool moved = res->map_version != t->map_version;
  if (moved && res->n > 0) launch_refresh(*res, t->dev(), s);
  launch_forward(*res, t->dev(), pool, out, !moved && res->epoch == t->update_epoch, s);
  return check_launch();
}

namespace {

// The backward of both entry points.  noalloc: the long keys' chunk partials
// go to the library's fixed device scratch instead of the table's (grown on
// demand), and the long keys keep the lookup's order (the feature-ordered
// plan needs scratch of its own; the order changes no sum).
recis_status pool_bwd_update(recis_table* t, const recis_lookup_result* res, int32_t pool, const void* grad_out,
                             int32_t grad_dtype, const recis_optim_params* opt, hipStream_t s, bool noalloc) {
  if (!t || !res || !opt) return RECIS_ERR_INVALID_ARG;
  if (pool != RECIS_POOL_SUM && pool != RECIS_POOL_MEAN && pool != RECIS_POOL_NONE) return RECIS_ERR_INVALID_ARG;
  if (grad_dtype != RECIS_DTYPE_F32 && grad_dtype != RECIS_DTYPE_BF16) return RECIS_ERR_INVALID_ARG;
  const bool by_occ = (res->flags & RECIS_GROUP_BY_OCCURRENCE) != 0;
  if ((pool == RECIS_POOL_NONE) != by_occ) return RECIS_ERR_INVALID_ARG;
  if (res->n < 0 || res->n > res->capacity) return RECIS_ERR_INVALID_ARG;
  if (res->n > 0 && !grad_out) return RECIS_ERR_INVALID_ARG;
  if (t->cfg.optim == RECIS_OPTIM_NONE) return RECIS_ERR_UNSUPPORTED;
  if (!(opt->lr >= 0.0) || !(opt->eps >= 0.0)) return RECIS_ERR_INVALID_ARG;
  const bool adam = t->cfg.optim == RECIS_OPTIM_ADAM;
  if (adam && !(opt->beta1 >= 0.0 && opt->beta1 < 1.0 && opt->beta2 >= 0.0 && opt->beta2 < 1.0))
    return RECIS_ERR_INVALID_ARG;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  double* partials = t->partials;
  int* reorder = reinterpret_cast<int*>(t->wb_keys);  // the writeback scratch is free during a backward
  long long reorder_ints = 2 * t->scr_cap;
  if (noalloc) {
    // every chunk partial the call can have: max_chunks(n) rows of dim doubles
    const long long need = plan_layout(res->n).max_chunks * (long long)t->cfg.dim * (long long)sizeof(double);
    if (need > kNoAllocScratchBytes) return RECIS_ERR_INVALID_ARG;
    void* p = nullptr;
    recis_status st = noalloc_scratch(t->device, &p);
    if (st != RECIS_OK) return st;
    partials = static_cast<double*>(p);
    reorder = nullptr;
    reorder_ints = 0;
  } else if (res->n > t->scr_cap) {
    recis_status st = ensure_scratch(t, res->n, s);
    if (st != RECIS_OK) return st;
    partials = t->partials;
    reorder = reinterpret_cast<int*>(t->wb_keys);
    reorder_ints = 2 * t->scr_cap;
  }
  // the hot keys' partials (not in the allocation-free call: its long keys
  // keep the chunked plan)
  double* hot_partials = nullptr;
  long long hot_rows = 0;
  int* hot_ws = nullptr;
  long long hot_ws_len = 0;
  const double grad_bytes =
      (double)res->num_feats * res->batch * t->cfg.dim * (grad_dtype == RECIS_DTYPE_BF16 ? 2 : 4);
  const double hot_from = t->cfg.hot_grad_bytes == 0 ? kMemCacheBytes : (double)t->cfg.hot_grad_bytes;
  if (!noalloc && pool != RECIS_POOL_NONE && hot_kmax(t->cfg.dim) > 0 && res->num_feats <= kFeatBins &&
      res->n > 0 && t->cfg.hot_grad_bytes >= 0 && grad_bytes >= hot_from) {
    const long long rows = (long long)res->num_feats * hot_kmax(t->cfg.dim) * hot_blocks(res->batch);
    const long long ws = hot_ws_ints(res->n, res->num_feats, res->batch, t->cfg.dim);
    if (rows <= INT32_MAX / 2) {
      if (rows > t->hot_rows || ws > t->hot_ws_len) {
        HIP_TRY(hipStreamSynchronize(s));
        if (rows > t->hot_rows) {
          tab_free(t, t->hot_partials, (size_t)t->hot_rows * (size_t)t->cfg.dim * 8, s);
          t->hot_rows = 0;
          t->hot_partials = static_cast<double*>(tab_alloc(t, (size_t)rows * (size_t)t->cfg.dim * 8, s));
          if (t->hot_partials) t->hot_rows = rows;
        }
        if (ws > t->hot_ws_len) {
          tab_free(t, t->hot_ws, (size_t)t->hot_ws_len * 4, s);
          t->hot_ws_len = 0;
          t->hot_ws = static_cast<int*>(tab_alloc(t, (size_t)ws * 4, s));
          if (t->hot_ws) t->hot_ws_len = ws;
        }
      }
      if (t->hot_partials && t->hot_ws) {
        hot_partials = t->hot_partials;
        hot_rows = t->hot_rows;
        hot_ws = t->hot_ws;
        hot_ws_len = t->hot_ws_len;
      }
    }
  }
  OptConsts oc;
  oc.lr = (float)opt->lr;
  oc.eps = (float)opt->eps;
  oc.b1 = (float)opt->beta1;
  oc.b2 = (float)opt->beta2;
  oc.omb1 = (float)(1.0 - opt->beta1);
  oc.omb2 = (float)(1.0 - opt->beta2);
  oc.step_size = 0.f;
  if (adam) {
    t->adam_step += 1;
    const double n = (double)t->adam_step;
    oc.step_size = (float)(opt->lr * std::sqrt(1.0 - std::pow(opt->beta2, n)) / (1.0 - std::pow(opt->beta1, n)));
  }
  const bool moved = res->map_version != t->map_version;
  if (moved && res->n > 0) launch_refresh(*res, t->dev(), s);
  const bool current = !moved && res->epoch == t->update_epoch;
  t->update_epoch += 1;
  recis_status st = launch_backward(*res, t->dev(), pool, grad_out, grad_dtype, oc, partials, reorder, reorder_ints,
                                    hot_partials, hot_rows, hot_ws, hot_ws_len, current, s);
  if (st != RECIS_OK) return st;
  return check_launch();
}

}  // namespace

recis_status recis_pool_bwd_update(recis_table* t, const recis_lookup_result* res, int32_t pool,
                                   const void* grad_out, int32_t grad_dtype, const recis_optim_params* opt,
                                   hipStream_t s) {
  return pool_bwd_update(t, res, pool, grad_out, grad_dtype, opt, s, false);
}

recis_status recis_pool_bwd_update_noalloc(recis_table* t, const recis_lookup_result* res, int32_t pool,
                                           const void* grad_out, int32_t grad_dtype,
                                           const recis_optim_params* opt, hipStream_t s) {
  return pool_bwd_update(t, res, pool, grad_out, grad_dtype, opt, s, true);
}

int64_t recis_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

recis_status recis_writeback(recis_table* t, const int64_t* keys, int64_t n, const float* rows, hipStream_t s) {
  if (!t || n < 0 || (n > 0 && (!keys || !rows)) || n > (1ll << 30)) return RECIS_ERR_INVALID_ARG;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  recis_status st = ensure_scratch(t, n, s);
  if (st != RECIS_OK) return st;
  st = ensure_capacity(t, n, s);
  if (st != RECIS_OK) return st;
  t->update_epoch += 1;
  t->map_version += 1;
  launch_writeback(t->dev(), reinterpret_cast<const long long*>(keys), n, rows, t->dd,
                   (unsigned long long)(t->dd_cap - 1), 64 - log2_exact(t->dd_cap), t->wb_keys, t->uslot, s);
  return check_launch();
}

recis_status recis_idmap_import(recis_table* t, int64_t n, const int64_t* keys, const int64_t* rows,
                                const uint32_t* counts, const void* params, const float* state, int64_t adam_step,
                                hipStream_t s) {
  if (!t || n < 0 || adam_step < 0 || n > (1ll << 31) - 1) return RECIS_ERR_INVALID_ARG;
  if (n > 0 && (!keys || !rows || !counts || !params)) return RECIS_ERR_INVALID_ARG;
  if (n > 0 && t->state_words > 0 && !state) return RECIS_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(params) | reinterpret_cast<uintptr_t>(state)) & 15) return RECIS_ERR_INVALID_ARG;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  if (t->keys_hi > 0 || t->rows_hi > 0) {  // the bounds say it may hold keys: ask the device
    DevCounters c;
    recis_status st = read_counters(t, &c, s);
    if (st != RECIS_OK) return st;
    if (c.num_keys != 0 || c.next_row != 0) return RECIS_ERR_INVALID_ARG;
    t->keys_hi = t->rows_hi = 0;
  }
  recis_status st = ensure_capacity(t, n, s);
  if (st != RECIS_OK) return st;
  t->update_epoch += 1;
  t->map_version += 1;
  t->adam_step = adam_step;
  launch_import(t->dev(), n, reinterpret_cast<const long long*>(keys), reinterpret_cast<const long long*>(rows),
                counts, params, t->state_words > 0 ? state : nullptr, s);
  return check_launch();
}

recis_status recis_idmap_key_ages(recis_table* t, const int64_t* keys, int64_t n, uint32_t* ages, int32_t set,
                                  hipStream_t s) {
  if (!t || n < 0 || (n > 0 && (!keys || !ages)) || (set != 0 && set != 1)) return RECIS_ERR_INVALID_ARG;
  if (!t->last_use) return RECIS_ERR_UNSUPPORTED;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  launch_key_ages(t->dev(), reinterpret_cast<const long long*>(keys), n, ages, set != 0, s);
  return check_launch();
}

recis_status recis_idmap_sketch(recis_table* t, uint32_t* counters, int32_t set, hipStream_t s) {
  if (!t || !counters || (set != 0 && set != 1)) return RECIS_ERR_INVALID_ARG;
  if (!t->sketch) return RECIS_ERR_UNSUPPORTED;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  const size_t bytes = ((size_t)kSketchRows << t->cfg.admit_sketch_bits) * sizeof(unsigned);
  HIP_TRY(hipMemcpyAsync(set ? t->sketch : counters, set ? counters : t->sketch, bytes, hipMemcpyDeviceToDevice, s));
  return RECIS_OK;
}

recis_status recis_idmap_export(recis_table* t, int64_t cap, int64_t* keys, int64_t* rows, uint32_t* counts,
                                void* params, float* state, int64_t* n, hipStream_t s) {
  if (!t || !n || cap < 0) return RECIS_ERR_INVALID_ARG;
  if (cap > 0 && (!keys || !rows || !counts || !params)) return RECIS_ERR_INVALID_ARG;
  if (cap > 0 && t->state_words > 0 && !state) return RECIS_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(params) | reinterpret_cast<uintptr_t>(state)) & 15) return RECIS_ERR_INVALID_ARG;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  launch_export(t->dev(), cap, reinterpret_cast<long long*>(keys), reinterpret_cast<long long*>(rows), counts, s);
  recis_status st = check_launch();
  if (st != RECIS_OK) return st;
  DevCounters c;
  st = read_counters(t, &c, s);
  if (st != RECIS_OK) return st;
  *n = (int64_t)c.scratch_count;
  const long long m = std::min<long long>(cap, (long long)c.scratch_count);
  launch_export_rows(t->dev(), m, reinterpret_cast<const long long*>(keys), reinterpret_cast<long long*>(rows), params,
                     t->state_words > 0 ? state : nullptr, s);
  st = check_launch();
  if (st != RECIS_OK) return st;
  HIP_TRY(hipStreamSynchronize(s));
  return RECIS_OK;
}

recis_status recis_idmap_stats(recis_table* t, recis_table_stats* out, hipStream_t s) {
  if (!t || !out) return RECIS_ERR_INVALID_ARG;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  DevCounters c;
  recis_status st = read_counters(t, &c, s);
  if (st != RECIS_OK) return st;
  out->keys = (int64_t)c.num_keys;
  out->rows_in_use = (int64_t)c.next_row - (c.free_top > 0 ? c.free_top : 0);
  out->rows_allocated = t->rows_alloc;
  out->blocks = (int64_t)t->blocks.size();
  out->slot_capacity = t->slot_cap;
  out->adam_step = t->adam_step;
  out->bytes = t->bytes;
  out->probationary_keys = out->keys - out->rows_in_use;
  out->hbm_rows = hbm_rows(t);
  out->claim_attempts = (int64_t)c.claim_attempts;
  out->claim_failures = (int64_t)c.claim_failures;
  out->lookup_pairs = (int64_t)c.lookup_pairs;
  out->hot_keys = (int64_t)c.hot_keys;
  return RECIS_OK;
}

recis_status recis_get_error(recis_table* t, hipStream_t s) {
  if (!t) return RECIS_ERR_INVALID_ARG;
  ScopedDevice sd(t->device);
  ScopedProbe sp(t);
  HIP_TRY(hipStreamSynchronize(s));
  unsigned err = 0;
  HIP_TRY(hipMemcpy(&err, &t->ctr->error, sizeof(err), hipMemcpyDeviceToHost));
  // One error per call.  KEY_RANGE and INVALID_ARG are cleared as they are
  // returned, and come first, so that a standing CAPACITY never hides them;
  // CAPACITY stays until an eviction pass clears it.
  const unsigned bit = (err & kErrKeyRange) ? kErrKeyRange : ((err & kErrInvalid) ? kErrInvalid : 0u);
  if (bit) {
    const unsigned keep = err & ~bit;
    HIP_TRY(hipMemcpy(&t->ctr->error, &keep, sizeof(keep), hipMemcpyHostToDevice));
    return bit == kErrKeyRange ? RECIS_ERR_KEY_RANGE : RECIS_ERR_INVALID_ARG;
  }
  return (err & kErrCapacity) ? RECIS_ERR_CAPACITY : RECIS_OK;
}

recis_status recis_profile_kernel(recis_table* t, const char* kernel, hipEvent_t start, hipEvent_t stop) {
  if (!t) return RECIS_ERR_INVALID_ARG;
  if (!kernel) {
    t->probe = KernelProbe();
    return RECIS_OK;
  }
  if (!start || !stop || std::strlen(kernel) >= sizeof(t->probe.name)) return RECIS_ERR_INVALID_ARG;
  std::memset(t->probe.name, 0, sizeof(t->probe.name));
  std::memcpy(t->probe.name, kernel, std::strlen(kernel));
  t->probe.start = start;
  t->probe.stop = stop;
  return RECIS_OK;
}

const char* recis_status_string(recis_status st) {
  switch (st) {
    case RECIS_OK: return "ok";
    case RECIS_ERR_INVALID_ARG: return "invalid argument";
    case RECIS_ERR_OUT_OF_MEMORY: return "out of device memory";
    case RECIS_ERR_CAPACITY: return "table capacity exceeded";
    case RECIS_ERR_KEY_RANGE: return "key outside the 48-bit id / 15-bit slot range";
    case RECIS_ERR_HIP: return "HIP runtime error";
    case RECIS_ERR_UNSUPPORTED: return "unsupported combination";
    default: return "unknown status";
  }
}

}  // extern "C"
