// fwd_bwd.hip -- gather + bag pooling forward, and the backward: duplicate-
// gradient reduction fused with the sparse optimizer row update.
//
// Pages: "RecIS (Recommendation Intelligence System)" README --
//   Key optimisations > Operator implementation: vectorised memory access,
//   reductions that merge inside a warp to avoid atomics;
//   Key optimisations > Efficient dynamic Embedding: optimizer state is kept
//   next to the parameters in the EmbeddingBlocks.
//
// Work layout: a row is split into 16-byte chunks (4 fp32 or 8 bf16
// elements); a "group" of lanes of one 64-lane wavefront owns one bag
// (forward, C = row_bytes / 16 lanes) or one distinct key (backward, one
// chunk per lane), so a wave moves whole rows with full 16-byte loads.  A
// forward group fetches the references of up to C occurrences at once (one
// lane each), then walks them with cross-lane broadcasts, several row loads
// in flight per group.
//
// Rows allocated by insert_find stay pending until their first update: their
// values are the initializer's, recomputed here from (seed, key) instead of
// being read, and the update writes the row once (parameters and state).
//
// Backward, no atomics on data: each key's occurrences were grouped by
// insert_find.  Keys with more than kShortMax occurrences take two launches:
// one wave per chunk of kChunk occurrences (more for a hot key) writes a
// double-precision partial sum, then one wave per key sums its partials in a
// fixed order and applies the
// update (a launch boundary instead of fences and completion counters, which
// serialise on the per-XCD L2 writeback).  The other keys take a third
// launch: a block stages the metadata and gradient references of 256
// consecutive keys in LDS, then each group of KL lanes reduces and updates
// one key at a time with all of the key's loads in flight together.
#include <mutex>
#include <type_traits>

#include "internal.h"

namespace recis {

// ------------------------------------------- allocation-free backward scratch
// The long keys' chunk partials of recis_pool_bwd_update_noalloc.  Host code
// never passes the array's name to a kernel (in host code it is a stand-in,
// not a device address): it passes the address hipGetSymbolAddress gives for
// the current device, looked up once per device and kept.
static __device__ __align__(256) double scratch[kNoAllocScratchBytes / sizeof(double)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

recis_status noalloc_scratch(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return RECIS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return RECIS_ERR_HIP;
    }
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return RECIS_OK;
}

namespace {

template <typename TP>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int E = 4;
  static constexpr bool kBF16 = false;
  __device__ static void load(const void* p, float (&v)[4]) {
    const f32x4 x = *gread<f32x4>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  __device__ static void unpack(uint4 x, float (&v)[4]) {
    v[0] = __uint_as_float(x.x); v[1] = __uint_as_float(x.y);
    v[2] = __uint_as_float(x.z); v[3] = __uint_as_float(x.w);
  }
  // Row stores are non-temporal: an updated row is not read again within the
  // step, and streaming it past the caches keeps them for the reads.
  __device__ static void store(void* p, const float (&v)[4]) {
    const f32x4 x = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(x, gwrite<f32x4>(p));
  }
};
struct bf16_t {
  unsigned short bits;
};
template <>
struct Vec<bf16_t> {
  static constexpr int E = 8;
  static constexpr bool kBF16 = true;
  __device__ static void unpack(uint4 x, float (&v)[8]) {
    const unsigned w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static void load(const void* p, float (&v)[8]) {
    const u32x4 x = *gread<u32x4>(p);
    unpack(make_uint4(x.x, x.y, x.z, x.w), v);
  }
  __device__ static void store(void* p, const float (&v)[8]) {
    uint4 x;
    x.x = (unsigned)f32_to_bf16(v[0]) | ((unsigned)f32_to_bf16(v[1]) << 16);
    x.y = (unsigned)f32_to_bf16(v[2]) | ((unsigned)f32_to_bf16(v[3]) << 16);
    x.z = (unsigned)f32_to_bf16(v[4]) | ((unsigned)f32_to_bf16(v[5]) << 16);
    x.w = (unsigned)f32_to_bf16(v[6]) | ((unsigned)f32_to_bf16(v[7]) << 16);
    const u32x4 y = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(y, gwrite<u32x4>(p));
  }
};

__device__ __forceinline__ long long shfl64(long long v, int src) {
  const int lo = __shfl((int)(unsigned long long)v, src);
  const int hi = __shfl((int)((unsigned long long)v >> 32), src);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double shfl_d(double v, int src) {
  return __longlong_as_double(shfl64(__double_as_longlong(v), src));
}
__device__ __forceinline__ double shfl_xor_d(double v, int m) {
  const unsigned long long b = __double_as_longlong(v);
  const int lo = __shfl_xor((int)(unsigned)b, m), hi = __shfl_xor((int)(unsigned)(b >> 32), m);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Gradient loads of E consecutive elements (E = 4 or 8) in either dtype.
template <int E>
__device__ __forceinline__ void load_grad(const void* base, long long elem, int gdt, float (&g)[E]) {
  if (gdt == RECIS_DTYPE_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const float4 x = p[i];
      g[4 * i] = x.x; g[4 * i + 1] = x.y; g[4 * i + 2] = x.z; g[4 * i + 3] = x.w;
    }
  } else {
    const uint2* p = reinterpret_cast<const uint2*>(static_cast<const unsigned short*>(base) + elem);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const uint2 x = p[i];
      g[4 * i] = __uint_as_float(x.x << 16);
      g[4 * i + 1] = __uint_as_float(x.x & 0xFFFF0000u);
      g[4 * i + 2] = __uint_as_float(x.y << 16);
      g[4 * i + 3] = __uint_as_float(x.y & 0xFFFF0000u);
    }
  }
}

// Where the values of distinct key u live: >= 0 a written row, -1 no row,
// -2 a pending row (values = initializer of `key`).
__device__ __forceinline__ long long resolve_row(const TableDev& t, const long long* urows,
                                                 const long long* ukeys, const unsigned* idslot,
                                                 long long u, long long& key) {
  long long r = urows[u];
  if (r < 0) return -1;
  if (r & kFreshRow) {
    r &= ~kFreshRow;
    if (t.slots[idslot[u]].row & kPendingRow) {
      key = ukeys[u];
      return -2;
    }
  }
  return r;
}

// ------------------------------------------------------------- forward
struct FwdArgs {
  const int* off;
  const int* inverse;
  const long long* urows;
  const long long* ukeys;
  const unsigned* idslot;
  const long long* occref;
  long long N;
  long long nbags;
  int F, B, pool, current;
  void* out;
  TableDev t;
};

// Reference to the values of occurrence j: the device address of its row
// (>= 0), kOccNoRow (zeros), or kOccPendingBit | key for a row that still
// holds its initial values.  While the lookup is current this is the
// occurrence's reference written by insert_find (one load); otherwise the
// distinct key's row and IDMap slot are read.
__device__ __forceinline__ long long occurrence_ref(const FwdArgs& a, long long j) {
  if (a.current) return a.occref[j];
  long long key = 0;
  const long long r = resolve_row(a.t, a.urows, a.ukeys, a.idslot, a.inverse[j], key);
  if (r == -1) return kOccNoRow;
  if (r == -2) return (long long)(kOccPendingBit | (unsigned long long)key);
  return (long long)row_ptr(a.t.rs, r);
}

// Value of lane x of this lane's group of C lanes (x uniform).  A group of 16
// is one DPP row: row_newbcast copies lane x of every row to the whole row in
// one VALU move; other widths go through LDS (ds_bpermute).  A source lane
// that is off yields `old`.
template <int C>
__device__ __forceinline__ int group_bcast(int v, int x, int gbase, int old) {
  if constexpr (C == 16) {
    switch (x) {
      case 0: return __builtin_amdgcn_update_dpp(old, v, 0x150, 0xF, 0xF, false);
      case 1: return __builtin_amdgcn_update_dpp(old, v, 0x151, 0xF, 0xF, false);
      case 2: return __builtin_amdgcn_update_dpp(old, v, 0x152, 0xF, 0xF, false);
      case 3: return __builtin_amdgcn_update_dpp(old, v, 0x153, 0xF, 0xF, false);
      case 4: return __builtin_amdgcn_update_dpp(old, v, 0x154, 0xF, 0xF, false);
      case 5: return __builtin_amdgcn_update_dpp(old, v, 0x155, 0xF, 0xF, false);
      case 6: return __builtin_amdgcn_update_dpp(old, v, 0x156, 0xF, 0xF, false);
      case 7: return __builtin_amdgcn_update_dpp(old, v, 0x157, 0xF, 0xF, false);
      case 8: return __builtin_amdgcn_update_dpp(old, v, 0x158, 0xF, 0xF, false);
      case 9: return __builtin_amdgcn_update_dpp(old, v, 0x159, 0xF, 0xF, false);
      case 10: return __builtin_amdgcn_update_dpp(old, v, 0x15A, 0xF, 0xF, false);
      case 11: return __builtin_amdgcn_update_dpp(old, v, 0x15B, 0xF, 0xF, false);
      case 12: return __builtin_amdgcn_update_dpp(old, v, 0x15C, 0xF, 0xF, false);
      case 13: return __builtin_amdgcn_update_dpp(old, v, 0x15D, 0xF, 0xF, false);
      case 14: return __builtin_amdgcn_update_dpp(old, v, 0x15E, 0xF, 0xF, false);
      default: return __builtin_amdgcn_update_dpp(old, v, 0x15F, 0xF, 0xF, false);
    }
  } else {
    return __shfl(v, gbase + x);
  }
}
template <int C>
__device__ __forceinline__ long long group_bcast64(long long v, int x, int gbase, long long old) {
  const int lo = group_bcast<C>((int)(unsigned long long)v, x, gbase, (int)(unsigned long long)old);
  const int hi = group_bcast<C>((int)((unsigned long long)v >> 32), x, gbase, (int)((unsigned long long)old >> 32));
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// Pooling: a group of C = D / E lanes per bag, GPW = 64 / C bags per wave.
// A block takes BB consecutive bags, ranks them by length in LDS and deals
// them out in that order, GPB at a time (one per group), so the groups of a
// wave walk bags of about the same length and few lanes idle while the
// longest one finishes.  Each round a group reads the references of its
// bag's next C occurrences, one per lane, and walks them BF at a time with
// those rows' loads in flight together, summing in occurrence order.  Rows
// still pending (values = the initializer's) are left out of the walk and
// queued per wave in LDS; as soon as GPW are queued the wave computes them in
// one pass, one row per group, and each row's group adds it.  The
// initializer then runs once per GPW pending rows; run inside the walk it
// would cost the whole wave a pass each time any one group met a pending
// row.  The order of the additions depends only on the data, so runs repeat
// exactly.
constexpr int kFwdBatch = 4;

template <int C>
struct FwdShape {
  static constexpr int GPW = 64 / C;                    // bags per wave at a time
  static constexpr int GPB = 256 / C;                   // bags per block at a time
  static constexpr int BB = GPB > 64 ? GPB : 64;        // bags per block
  static constexpr int NSTEP = BB / GPB;                // bags per group
};

template <int D, typename TP>
__global__ __launch_bounds__(256) void k_fwd_pool(FwdArgs a) {
  constexpr int E = Vec<TP>::E;
  constexpr int C = D / E;  // lanes per bag
  using S = FwdShape<C>;
  constexpr int GPW = S::GPW, GPB = S::GPB, BB = S::BB;
  constexpr int BF = kFwdBatch < C ? kFwdBatch : C;
  constexpr int QL = 128;  // queue ring (at most GPW - 1 + 64 entries wait)
  __shared__ int s_lo[BB], s_len[BB];
  __shared__ unsigned short s_order[BB];
  __shared__ long long s_qkey[4][QL];
  __shared__ unsigned char s_qown[4][QL];
  __shared__ uint4 s_stage[4][GPW * C];
  const int tid = threadIdx.x, wid = tid >> 6, wl = tid & 63;
  const int lane = wl % C, g = wl / C, gbase = wl - lane;
  long long* qkey = s_qkey[wid];
  unsigned char* qown = s_qown[wid];
  uint4* stage = s_stage[wid];
  const long long b0 = (long long)blockIdx.x * BB;
  for (int t = tid; t < BB; t += 256) {
    const long long b = b0 + t;
    long long lo = 0, hi = -1;  // past the last bag: length -1, ranked last
    if (b < a.nbags) {
      lo = a.off[b];
      hi = a.off[b + 1];
      lo = lo < 0 ? 0 : (lo > a.N ? a.N : lo);
      hi = hi < lo ? lo : (hi > a.N ? a.N : hi);
    }
    s_lo[t] = (int)lo;
    s_len[t] = (int)(hi - lo);
  }
  __syncthreads();
  for (int t = tid; t < BB; t += 256) {  // rank: longer first, then by index
    const int L = s_len[t];
    int rk = 0;
    for (int k = 0; k < BB; ++k) {
      const int Lk = s_len[k];
      rk += (Lk > L || (Lk == L && k < t)) ? 1 : 0;
    }
    s_order[rk] = (unsigned short)t;
  }
  __syncthreads();
  int qhead = 0, qlen = 0;  // uniform
  float acc[E];
  // the first `take` queued rows: group g computes row g, then every row's
  // group adds it, in queue order
  auto pass = [&](int take) {
    const long long key = qkey[(qhead + (g < take ? g : 0)) & (QL - 1)];
    if (g < take) stage[g * C + lane] = init_chunk_as<Vec<TP>::kBF16>(a.t, key, lane);
    for (int k = 0; k < take; ++k) {
      if (qown[(qhead + k) & (QL - 1)] == g) {
        float v[E];
        Vec<TP>::unpack(stage[k * C + lane], v);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += v[e];
      }
    }
    qhead = (qhead + take) & (QL - 1);
    qlen -= take;
  };
  // every lane stays to the end: the wave's broadcasts, ballots and passes
  // need all of them; a group without a bag has no occurrences
  for (int st = 0; st < S::NSTEP; ++st) {
    const int t = s_order[st * GPB + tid / C];
    const long long bag = b0 + t;
    const long long lo = s_lo[t];
    const long long hi = lo + (s_len[t] > 0 ? s_len[t] : 0);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (long long base = lo;; base += C) {
      const int cnt = (int)(hi - base < C ? (hi - base > 0 ? hi - base : 0) : C);
      if (__ballot(cnt > 0) == 0) break;
      const long long ref = lane < cnt ? occurrence_ref(a, base + lane) : kOccNoRow;
      const bool pend = ref < 0;  // kOccPendingBit
      const unsigned long long pm = __ballot(pend);
      if (pend) {
        const int at =
            (qhead + qlen +
             (int)__builtin_amdgcn_mbcnt_hi((unsigned)(pm >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)pm, 0u))) &
            (QL - 1);
        qkey[at] = (long long)((unsigned long long)ref & ~kOccPendingBit);
        qown[at] = (unsigned char)g;
      }
      qlen += __popcll(pm);
      while (qlen >= GPW) pass(GPW);
      int cmax = cnt;
#pragma unroll
      for (int m = C; m < 64; m <<= 1) {
        const int o = __shfl_xor(cmax, m);
        cmax = o > cmax ? o : cmax;
      }
      cmax = __builtin_amdgcn_readfirstlane(cmax);
#pragma unroll
      for (int q = 0; q < C; q += BF) {  // unrolled: broadcast sources are constants
        if (q >= cmax) break;
        long long r[BF];
        float v[BF][E];
#pragma unroll
        for (int x = 0; x < BF; ++x) {
          r[x] = group_bcast64<C>(ref, q + x, gbase, kOccNoRow);
          if (q + x >= cnt) r[x] = kOccNoRow;
#pragma unroll
          for (int e = 0; e < E; ++e) v[x][e] = 0.f;
        }
        // the loads write v only: a branch that also wrote v would have to
        // wait for every load in flight
#pragma unroll
        for (int x = 0; x < BF; ++x)
          if (r[x] >= 0 && r[x] != kOccNoRow) Vec<TP>::load(reinterpret_cast<const char*>(r[x]) + lane * 16, v[x]);
#pragma unroll
        for (int x = 0; x < BF; ++x)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] += v[x][e];
      }
    }
    if (qlen > 0) pass(qlen);  // the bags change: settle the queue
    if (bag < a.nbags) {
      if (a.pool == RECIS_POOL_MEAN && hi > lo) {
        const float len = (float)(hi - lo);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = acc[e] / len;
      }
      // non-temporal: the step does not read the output again
      const int f = (int)(bag / a.B), i = (int)(bag - (long long)f * a.B);
      float* o = static_cast<float*>(a.out) + ((long long)i * a.F + f) * D + lane * E;
#pragma unroll
      for (int q = 0; q < E / 4; ++q)
        __builtin_nontemporal_store(f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]},
                                    reinterpret_cast<f32x4*>(o) + q);
    }
  }
}

// Gather (no pooling): a group of C lanes copies kGatherPer consecutive
// occurrences' rows, all their loads in flight together; the output is
// written with non-temporal stores (it is not read again by this step).
constexpr int kGatherPer = 4;

template <int D, typename TP>
__global__ __launch_bounds__(256) void k_fwd_gather(FwdArgs a) {
  constexpr int E = Vec<TP>::E;
  constexpr int C = D / E;
  constexpr int GPB = 256 / C;
  const int lane = threadIdx.x % C;
  const long long j0 = ((long long)blockIdx.x * GPB + threadIdx.x / C) * kGatherPer;
  if (j0 >= a.N) return;
  long long r[kGatherPer];
#pragma unroll
  for (int x = 0; x < kGatherPer; ++x) r[x] = j0 + x < a.N ? occurrence_ref(a, j0 + x) : kOccNoRow;
  u32x4 v[kGatherPer];
#pragma unroll
  for (int x = 0; x < kGatherPer; ++x) {
    v[x] = u32x4{0u, 0u, 0u, 0u};
    // loads write v only after its zeros (never under an else: that would
    // wait for every load in flight)
    if (r[x] >= 0 && r[x] != kOccNoRow) v[x] = *gread<u32x4>(reinterpret_cast<const char*>(r[x]) + lane * 16);
  }
#pragma unroll
  for (int x = 0; x < kGatherPer; ++x) {
    if (j0 + x >= a.N) break;
    u32x4 y = v[x];
    if (r[x] < 0) {
      const uint4 p = init_chunk_as<Vec<TP>::kBF16>(a.t, (long long)((unsigned long long)r[x] & ~kOccPendingBit), lane);
      y = u32x4{p.x, p.y, p.z, p.w};
    }
    __builtin_nontemporal_store(y, gwrite<u32x4>(static_cast<char*>(a.out) + ((j0 + x) * D * (long long)sizeof(TP)) + lane * 16));
  }
}

// ------------------------------------------------------------ backward
struct BwdArgs {
  const int* off;       // merged bag offsets
  const int* grouped;
  const int* uoff;
  const int* counts;
  long long* urows;
  const long long* ukeys;
  const long long* num_unique;
  const int* plan;
  const unsigned* idslot;
  PlanLayout pl;
  // the long-key plan: per long key its distinct index, first chunk and
  // chunk count, and per chunk its key (the lookup's, or the same reordered
  // feature by feature)
  const int* long_u;
  const int* long_base;
  const int* long_nch;
  const int* owner;
  int F, B, pool, gdt;
  const void* grad;
  OptConsts oc;
  TableDev t;
  double* partials;
  int current;  // no update since the lookup: a fresh row is still pending
  // the chunks of the long-key plan when it was rebuilt here (else plan[1])
  const int* nchunks;
  // hot keys (hot != 0): per bin the count-class histogram of the eligible
  // long keys, the class threshold, hot-key count, first hot index and
  // placement counter; per distinct key its index among its bin's hot keys
  // (-1: none); per occurrence the same (-1: none); the hot keys' partials,
  // hot index * hot_nc + bag block, D doubles each
  int hot, hot_nc, hot_min;
  unsigned* hot_cls;
  int* hot_thr;
  int* hot_n;
  int* hot_base;
  int* hot_cnt;
  unsigned char* hot_of;  // kHotNone: no hot index
  unsigned* hot_ent;  // per (feature, stage): its hot occurrences sorted by key, (key << 16 | bag),
                      // from the stage's first occurrence slot on
  int* hot_scnt;      // per (feature, stage): that entry count
  int hot_spf;        // stages per feature
  long long n_occ;    // occurrences of the lookup
  double* hot_partials;
};

constexpr int kBwdKeys = kThreads;  // distinct keys per block tile (short path)
constexpr int kBwdStage = 1024;     // gradient entries staged in LDS per tile
#ifndef RECIS_BWD_LANES
#define RECIS_BWD_LANES 64
#endif
constexpr int kBwdLanes = RECIS_BWD_LANES;  // lanes per key in the short path (at most)
#ifndef RECIS_BWD_BATCH
#define RECIS_BWD_BATCH 8
#endif
constexpr int kBwdBatchElems = RECIS_BWD_BATCH;  // gradient elements per lane in flight (short path)

// Upstream-gradient row of grouped entry gval (a bag, or an occurrence for
// POOL_NONE) and the scale it enters with (1 / bag length for mean pooling).
template <int D>
__device__ __forceinline__ void grad_ref(const BwdArgs& a, int gval, int& grow, double& scale) {
  scale = 1.0;
  if (a.pool == RECIS_POOL_NONE) {
    grow = gval;
    return;
  }
  const int f = gval / a.B, i = gval - f * a.B;
  grow = i * a.F + f;
  if (a.pool == RECIS_POOL_MEAN) {
    const int len = a.off[gval + 1] - a.off[gval];
    scale = 1.0 / (double)(len > 0 ? len : 1);
  }
}

// A row is split into NCH 16-byte chunks of E elements; with KL lanes per key
// each lane owns CH = NCH / KL chunks, chunk ch * KL + lane, so that every
// load instruction of a group covers KL * 16 contiguous bytes.
template <int D, typename TP, int KL>
struct RowMap {
  static constexpr int E = Vec<TP>::E;
  static constexpr int NCH = D / E;
  static constexpr int CH = NCH / KL;
  static_assert(CH >= 1 && CH * KL == NCH, "lanes per key must divide the row's chunks");
};

// Row state of this lane's chunks: the stored values, or for a pending row
// the initializer's values and zero optimizer state.
template <int D, typename TP, int OPT, int KL>
__device__ __forceinline__ void load_row(const BwdArgs& a, const char* rp, bool pending, long long key, int lane,
                                         float (&w)[RowMap<D, TP, KL>::CH][Vec<TP>::E],
                                         float (&s0)[RowMap<D, TP, KL>::CH][Vec<TP>::E],
                                         float (&s1)[RowMap<D, TP, KL>::CH][Vec<TP>::E]) {
  constexpr int E = Vec<TP>::E, CH = RowMap<D, TP, KL>::CH;
  if (pending) {
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      Vec<TP>::unpack(init_chunk_as<Vec<TP>::kBF16>(a.t, key, ch * KL + lane), w[ch]);
#pragma unroll
      for (int e = 0; e < E; ++e) s0[ch][e] = s1[ch][e] = 0.f;
    }
    return;
  }
  const float* st = reinterpret_cast<const float*>(rp + D * (int)sizeof(TP));
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int c = ch * KL + lane;
    Vec<TP>::load(rp + c * 16, w[ch]);
    Vec<float>::load(st + c * E, *reinterpret_cast<float(*)[4]>(s0[ch]));
    if constexpr (E == 8) Vec<float>::load(st + c * E + 4, *reinterpret_cast<float(*)[4]>(s0[ch] + 4));
    if constexpr (OPT == RECIS_OPTIM_ADAM) {
      Vec<float>::load(st + D + c * E, *reinterpret_cast<float(*)[4]>(s1[ch]));
      if constexpr (E == 8) Vec<float>::load(st + D + c * E + 4, *reinterpret_cast<float(*)[4]>(s1[ch] + 4));
    }
  }
}

// One optimizer step on this lane's chunks, then their stores.  The square
// root and reciprocal are the hardware's (about 1 ulp each).
template <int D, typename TP, int OPT, int KL>
__device__ __forceinline__ void update_store(const BwdArgs& a, char* rp, int lane,
                                             const double (&G)[RowMap<D, TP, KL>::CH][Vec<TP>::E],
                                             float (&w)[RowMap<D, TP, KL>::CH][Vec<TP>::E],
                                             float (&s0)[RowMap<D, TP, KL>::CH][Vec<TP>::E],
                                             float (&s1)[RowMap<D, TP, KL>::CH][Vec<TP>::E]) {
  constexpr int E = Vec<TP>::E, CH = RowMap<D, TP, KL>::CH;
  float* st = reinterpret_cast<float*>(rp + D * (int)sizeof(TP));
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int c = ch * KL + lane;
    if constexpr (OPT == RECIS_OPTIM_ADAGRAD) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float g = (float)G[ch][e];
        s0[ch][e] = s0[ch][e] + g * g;
        w[ch][e] = w[ch][e] - a.oc.lr * g * __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(s0[ch][e]) + a.oc.eps);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float g = (float)G[ch][e];
        s0[ch][e] = a.oc.b1 * s0[ch][e] + a.oc.omb1 * g;
        s1[ch][e] = a.oc.b2 * s1[ch][e] + a.oc.omb2 * (g * g);
        w[ch][e] = w[ch][e] - a.oc.step_size * s0[ch][e] *
                                  __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(s1[ch][e]) + a.oc.eps);
      }
      Vec<float>::store(st + D + c * E, *reinterpret_cast<float(*)[4]>(s1[ch]));
      if constexpr (E == 8) Vec<float>::store(st + D + c * E + 4, *reinterpret_cast<float(*)[4]>(s1[ch] + 4));
    }
    Vec<float>::store(st + c * E, *reinterpret_cast<float(*)[4]>(s0[ch]));
    if constexpr (E == 8) Vec<float>::store(st + c * E + 4, *reinterpret_cast<float(*)[4]>(s0[ch] + 4));
    Vec<TP>::store(rp + c * 16, w[ch]);
  }
}

// acc += scale * (upstream-gradient row grow), this lane's chunks.
template <int D, typename TP, int KL>
__device__ __forceinline__ void add_grad_row(const BwdArgs& a, int grow, double scale, int lane,
                                             double (&acc)[RowMap<D, TP, KL>::CH][Vec<TP>::E]) {
  constexpr int E = Vec<TP>::E, CH = RowMap<D, TP, KL>::CH;
  float g[CH][E];
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) load_grad<E>(a.grad, (long long)grow * D + (ch * KL + lane) * E, a.gdt, g[ch]);
#pragma unroll
  for (int ch = 0; ch < CH; ++ch)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[ch][e] += (double)g[ch][e] * scale;
}

// Block-wide exclusive scan of one 64-bit value per thread (kThreads = 256).
__device__ __forceinline__ long long block_scan_ll(long long v, long long* total) {
  __shared__ long long s_w[kThreads / 64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  long long x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long y = shfl64(x, lane >= d ? lane - d : lane);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_w[wid] = x;
  __syncthreads();
  long long before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    before += w < wid ? s_w[w] : 0;
    all += s_w[w];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// Long keys, pass 1: one wave per chunk (long_chunk(count) entries: kChunk,
// or a multiple of it for a hot key, so that it has at most kMaxKeyChunks
// chunks).  The chunk is taken kChunk entries at a time, one per lane; each
// group of C = D / E lanes sums a contiguous share of them (up to 8 rows in
// flight), a butterfly across the groups merges the shares, and the chunk's
// double-precision partial is stored.  No atomics and no cross-block waits:
// the finishing pass runs as the next launch.
template <int D, typename TP>
__global__ __launch_bounds__(256) void k_bwd_long_partial(BwdArgs a) {
  constexpr int E = Vec<TP>::E;
  constexpr int C = D / E;
  constexpr int GPW = 64 / C;           // groups per wave
  constexpr int PER = kChunk / GPW;     // entries per group
  constexpr int GF = PER < 8 ? PER : 8;  // gradient rows in flight per group
  const int wl = threadIdx.x & 63;
  const int lane = wl % C, g = wl / C;
  const int nchunks = a.nchunks ? *a.nchunks : a.plan[1];
  const long long nwaves = (long long)gridDim.x * 4;
  const int* long_u = a.long_u;
  const int* long_base = a.long_base;
  const int* owner = a.owner;
  for (long long q = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); q < nchunks; q += nwaves) {
    const int idx = owner[q];
    const int u = long_u[idx], cb = long_base[idx];
    const int o = a.uoff[u], c = a.counts[u];
    const int csz = long_chunk(c);
    const int k0 = (int)(q - cb) * csz;
    const int cend = c - k0 < csz ? c - k0 : csz;
    double acc[1][E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[0][e] = 0.0;
#pragma unroll 1
    for (int s0 = 0; s0 < cend; s0 += kChunk) {
      const int cnt = cend - s0 < kChunk ? cend - s0 : kChunk;
      int gr = 0;
      double scale = 0.0;
      if (wl < cnt) grad_ref<D>(a, a.grouped[o + k0 + s0 + wl], gr, scale);
      // All 64 lanes take part in every shuffle: the trip counts are
      // constants and each group masks its own loads.
#pragma unroll 1
      for (int x0 = 0; x0 < PER; x0 += GF) {
        float gv[GF][E];
        double sv[GF];
#pragma unroll
        for (int x = 0; x < GF; ++x) {
          const int src = g * PER + x0 + x;
          const int sl = src < cnt ? src : 0;
          const int gi = __shfl(gr, sl);
          sv[x] = shfl_d(scale, sl);
#pragma unroll
          for (int e = 0; e < E; ++e) gv[x][e] = 0.f;
          // the loads write gv only after its zeros, never under an else
          // (that would wait for every load in flight)
          if (src < cnt) load_grad<E>(a.grad, (long long)gi * D + lane * E, a.gdt, gv[x]);
        }
#pragma unroll
        for (int x = 0; x < GF; ++x)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[0][e] += (double)gv[x][e] * sv[x];
      }
    }
#pragma unroll
    for (int m = C; m < 64; m <<= 1)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[0][e] += shfl_xor_d(acc[0][e], m);
    if (g == 0) {
      double* pp = a.partials + q * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) pp[e] = acc[0][e];
    }
  }
}

// Long keys, pass 2: the chunk partials of each long key are summed (each
// group of lanes loads kMergeBatch partials at a time, then a butterfly
// across the groups, in a fixed order) and the update applied.  A block
// takes up to four keys at a time.  Those with more partials than a wave loads in
// one round (a hot key has up to kMaxKeyChunks) are summed one after another
// by all four waves, whose sums meet in LDS; then each wave sums its own key
// if it has fewer.  With few long keys a block takes one or two at a time.
// A key's first partial: cb >= 0 a chunk of the chunked plan, cb < 0 the
// row -1 - cb of the hot keys' partials.
template <int D>
__device__ __forceinline__ const double* partial_base(const BwdArgs& a, int cb) {
  return cb >= 0 ? a.partials + (long long)cb * D : a.hot_partials + (long long)(-1 - cb) * D;
}

template <int D, typename TP, int G_STRIDE, int E>
__device__ __forceinline__ void sum_partials(const BwdArgs& a, int cb, int nch, int grp, int lane,
                                             double (&G)[1][E]) {
  constexpr int kMergeBatch = 4;
#pragma unroll
  for (int e = 0; e < E; ++e) G[0][e] = 0.0;
  const double* base = partial_base<D>(a, cb);
  for (int p0 = 0; p0 < nch; p0 += G_STRIDE * kMergeBatch) {
    double part[kMergeBatch][E];
#pragma unroll
    for (int m = 0; m < kMergeBatch; ++m) {
      const int p = p0 + m * G_STRIDE + grp;
      const double* pp = base + (long long)(p < nch ? p : 0) * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) part[m][e] = p < nch ? pp[e] : 0.0;
    }
#pragma unroll
    for (int m = 0; m < kMergeBatch; ++m)
#pragma unroll
      for (int e = 0; e < E; ++e) G[0][e] += part[m][e];
  }
}

// The update of long key u (row entry r >= 0) with its summed gradient, by
// one group of C lanes.
template <int D, typename TP, int OPT>
__device__ __forceinline__ void long_update(const BwdArgs& a, int u, long long r, int lane, bool lead,
                                            double (&G)[1][Vec<TP>::E]) {
  constexpr int E = Vec<TP>::E;
  constexpr int C = D / E;
  const bool fresh = (r & kFreshRow) != 0;
  r &= ~kFreshRow;
  unsigned sl = 0;
  bool pending = false;
  if (fresh) {
    sl = a.idslot[u];
    pending = a.current ? true : (a.t.slots[sl].row & kPendingRow) != 0;
  }
  float wv[1][E], s0[1][E], s1[1][E];
  char* rp = row_ptr(a.t.rs, r);
  load_row<D, TP, OPT, C>(a, rp, pending, pending ? a.ukeys[u] : 0, lane, wv, s0, s1);
  update_store<D, TP, OPT, C>(a, rp, lane, G, wv, s0, s1);
  if (lead && fresh) {
    if (pending) a.t.slots[sl].row = (int)r;
    a.urows[u] = r;
  }
}

template <int D, typename TP, int OPT>
__global__ __launch_bounds__(256) void k_bwd_long_final(BwdArgs a) {
  constexpr int E = Vec<TP>::E;
  constexpr int C = D / E;
  constexpr int GPW = 64 / C;   // groups per wave
  constexpr int GPB = 256 / C;  // groups per block
  constexpr int kWaveMerge = GPW * 4;  // partials one wave sums in one round
  __shared__ double s_g[4][D];
  __shared__ int s_u[4], s_cb[4], s_nch[4];
  __shared__ long long s_r[4];
  const int wl = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lane = wl % C;
  const int nlong = a.plan[0];
  // keys per block and round: 1, 2 or 4, as few as the grid allows, so that
  // the hot keys land in different blocks when there are few long keys
  const int K = nlong <= (int)gridDim.x ? 1 : (nlong <= 2 * (int)gridDim.x ? 2 : 4);
  for (long long q = blockIdx.x; q * K < nlong; q += gridDim.x) {
    const long long idx = q * K + w;
    int u = 0, cb = 0, nch = 0;
    long long r = -1;  // no row (FIND_ONLY miss, or no key): nothing to update
    if (w < K && idx < nlong) {
      u = a.long_u[idx];
      cb = a.long_base[idx];
      nch = a.long_nch[idx];
      r = a.urows[u];
    }
    if (wl == 0) {
      s_u[w] = u;
      s_cb[w] = cb;
      s_nch[w] = nch;
      s_r[w] = r;
    }
    __syncthreads();
    // the block's keys with many partials, one after another by all waves
    for (int k = 0; k < 4; ++k) {
      const long long rk = s_r[k];
      if (rk < 0 || s_nch[k] <= kWaveMerge) continue;  // the same for the whole block
      double G[1][E];
      sum_partials<D, TP, GPB, E>(a, s_cb[k], s_nch[k], (int)threadIdx.x / C, lane, G);
#pragma unroll
      for (int m = C; m < 64; m <<= 1)
#pragma unroll
        for (int e = 0; e < E; ++e) G[0][e] += shfl_xor_d(G[0][e], m);
      if (wl < C)
#pragma unroll
        for (int e = 0; e < E; ++e) s_g[w][lane * E + e] = G[0][e];
      __syncthreads();
      if (w == 0 && wl < C) {
#pragma unroll
        for (int e = 0; e < E; ++e)
          G[0][e] = ((s_g[0][lane * E + e] + s_g[1][lane * E + e]) + s_g[2][lane * E + e]) + s_g[3][lane * E + e];
        long_update<D, TP, OPT>(a, s_u[k], rk, lane, wl == 0, G);
      }
      __syncthreads();  // s_g is reused by the next key
    }
    // the others, each by its own wave
    if (r >= 0 && nch <= kWaveMerge) {
      double G[1][E];
      sum_partials<D, TP, GPW, E>(a, cb, nch, wl / C, lane, G);
#pragma unroll
      for (int m = C; m < 64; m <<= 1)
#pragma unroll
        for (int e = 0; e < E; ++e) G[0][e] += shfl_xor_d(G[0][e], m);
      if (wl < C) long_update<D, TP, OPT>(a, u, r, lane, wl == 0, G);
    }
    __syncthreads();  // the key slots are reused by the next four keys
  }
}

// One key of the short path in flight: its LDS metadata, row state (loaded or
// initial) and its first GB gradient rows.
template <int D, typename TP, int KL, int GB>
struct KeyStage {
  static constexpr int E = Vec<TP>::E, CH = RowMap<D, TP, KL>::CH;
  int k = -1, c = 0, st = 0, base = 0;
  char* prow = nullptr;
  float w[CH][E], s0[CH][E], s1[CH][E];
  float g[GB][CH][E];
};

template <int D, typename TP, int OPT, int KL, int GB>
__device__ __forceinline__ void stage_key(const BwdArgs& a, int q, int nact, int lane, const unsigned char* s_perm,
                                          const int* s_c, const unsigned char* s_st, const int* s_eo,
                                          char* const* s_ptr, const long long* s_key, const int* s_grow,
                                          KeyStage<D, TP, KL, GB>& S) {
  constexpr int E = Vec<TP>::E, CH = RowMap<D, TP, KL>::CH;
  S.k = q < nact ? (int)s_perm[q] : -1;
  if (S.k < 0) {
    S.c = 0;
    return;
  }
  S.c = s_c[S.k];
  S.st = s_st[S.k];
  S.base = s_eo[S.k];
  S.prow = s_ptr[S.k];
  load_row<D, TP, OPT, KL>(a, S.prow, S.st == 2, s_key[S.k], lane, S.w, S.s0, S.s1);
#pragma unroll
  for (int i = 0; i < GB; ++i) {
    const bool in = i < S.c;
    const int gr = in ? s_grow[S.base + i] : 0;
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      if (in) {
        load_grad<E>(a.grad, (long long)gr * D + (ch * KL + lane) * E, a.gdt, S.g[i][ch]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) S.g[i][ch][e] = 0.f;
      }
    }
  }
}

// Short keys (<= kShortMax entries).  A block takes a tile of consecutive
// keys: kBwdKeys, or fewer when there are not enough keys for a full tile
// per block (a call with few distinct keys would otherwise leave most of
// the chip idle).
// Phase 1, one thread per key: metadata and the row's address (the block
// table is read here once, not per update), and one packed block scan that
// gives each key its staged-entry base and its place in an order with the
// pending rows first, so the groups of a wave mostly agree on whether to run
// the initializer.  Phase 2: the keys' gradient references, staged in LDS
// when they fit.  Phase 3: each group of KL lanes walks its keys, the row and
// gradient loads of a key in flight together.
// With one chunk per lane, fp32 rows fit 80 registers without spilling: ask
// for six waves per SIMD there (one more than the allocator picks by itself).
template <int D, typename TP>
constexpr int bwd_short_waves() {
  return Vec<TP>::E == 4 && D <= 64 * Vec<TP>::E ? 6 : 1;
}

template <int D, typename TP, int OPT, int KL>
__global__ __launch_bounds__(256, (bwd_short_waves<D, TP>())) void k_bwd_short(BwdArgs a) {
  constexpr int E = Vec<TP>::E, CH = RowMap<D, TP, KL>::CH;
  constexpr int GPB = 256 / KL;
  constexpr int GB = CH * E >= kBwdBatchElems ? 1 : kBwdBatchElems / (CH * E);  // gradient rows per batch
  const int wl = threadIdx.x & 63;
  const int lane = wl % KL, gbase = wl - lane;
  const int tid = threadIdx.x;
  __shared__ int s_o[kBwdKeys], s_c[kBwdKeys], s_eo[kBwdKeys + 1];
  __shared__ char* s_ptr[kBwdKeys];
  __shared__ int s_r[kBwdKeys];
  __shared__ long long s_key[kBwdKeys];
  __shared__ unsigned s_sl[kBwdKeys];
  __shared__ unsigned char s_st[kBwdKeys];
  __shared__ unsigned char s_perm[kBwdKeys];
  __shared__ int s_grow[kBwdStage];
  __shared__ double s_sc[kBwdStage];
  __shared__ int s_nact;
  const long long U = *a.num_unique;
  // keys per tile: kBwdKeys, or fewer (a multiple of 32) when the call has
  // too few distinct keys to give every block a full tile
  const long long per = (U + gridDim.x - 1) / gridDim.x;
  const int T = per >= kBwdKeys ? kBwdKeys : (per <= 32 ? 32 : (int)((per + 31) & ~31ll));
  for (long long t0 = (long long)blockIdx.x * T; t0 < U; t0 += (long long)gridDim.x * T) {
    const long long u = t0 + tid;
    int c = 0, o = 0, st = 0;  // st: 0 written row, 1 fresh but written, 2 pending
    long long r = -1, key = 0;
    unsigned sl = 0;
    if (tid < T && u < U) {
      c = a.counts[u];
      o = a.uoff[u];
      r = a.urows[u];
      if (r >= 0 && (r & kFreshRow)) {
        r &= ~kFreshRow;
        sl = a.idslot[u];
        key = a.ukeys[u];
        st = a.current ? 2 : ((a.t.slots[sl].row & kPendingRow) ? 2 : 1);
      }
      if (c > kShortMax) r = -1;  // the long-key kernels update it
    }
    const bool act = r >= 0;
    char* rp = act ? row_ptr(a.t.rs, r) : nullptr;
    // fields: entries (bits 0..19), pending keys (20..39), active keys (40..59)
    const long long packed = (act ? (long long)c : 0) | ((long long)(act && st == 2) << 20) | ((long long)act << 40);
    long long all;
    const long long pre = block_scan_ll(packed, &all);
    const int eo = (int)(pre & 0xFFFFF), tot = (int)(all & 0xFFFFF);
    const int npend = (int)((all >> 20) & 0xFFFFF);
    if (act) {
      const int pb = (int)((pre >> 20) & 0xFFFFF), ab = (int)((pre >> 40) & 0xFFFFF);
      s_perm[st == 2 ? pb : npend + (ab - pb)] = (unsigned char)tid;
    }
    s_o[tid] = o;
    s_c[tid] = act ? c : 0;
    s_eo[tid] = eo;
    s_st[tid] = (unsigned char)st;
    s_ptr[tid] = rp;
    s_r[tid] = (int)r;
    s_key[tid] = key;
    s_sl[tid] = sl;
    if (tid == 0) {
      s_eo[kBwdKeys] = tot;
      s_nact = (int)((all >> 40) & 0xFFFFF);
    }
    __syncthreads();
    const bool staged = tot <= kBwdStage;
    if (staged) {
      for (int i = tid; i < tot; i += kThreads) {
        int lo = 0, hi = kBwdKeys;  // the key whose staged range holds i
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_eo[mid] <= i) lo = mid;
          else hi = mid;
        }
        int gr;
        double sc;
        grad_ref<D>(a, a.grouped[s_o[lo] + (i - s_eo[lo])], gr, sc);
        s_grow[i] = gr;
        s_sc[i] = sc;
      }
      __syncthreads();
    }
    const int nact = s_nact;
    if (staged) {
      // one key per group at a time: its row and first GB gradient rows are
      // loaded together, further gradient rows GB at a time
      for (int q = tid / KL; q < nact; q += GPB) {
        KeyStage<D, TP, KL, GB> cur;
        stage_key<D, TP, OPT, KL, GB>(a, q, nact, lane, s_perm, s_c, s_st, s_eo, s_ptr, s_key, s_grow, cur);
        double acc[CH][E];
#pragma unroll
        for (int ch = 0; ch < CH; ++ch)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[ch][e] = 0.0;
#pragma unroll
        for (int i = 0; i < GB; ++i) {
          const double sc = i < cur.c ? s_sc[cur.base + i] : 0.0;
#pragma unroll
          for (int ch = 0; ch < CH; ++ch)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[ch][e] += (double)cur.g[i][ch][e] * sc;
        }
        for (int x0 = GB; x0 < cur.c; x0 += GB) {  // keys with more than GB entries
          float gv[GB][CH][E];
#pragma unroll
          for (int i = 0; i < GB; ++i) {
            const bool in = x0 + i < cur.c;
            const int gr = in ? s_grow[cur.base + x0 + i] : 0;
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) {
              if (in) {
                load_grad<E>(a.grad, (long long)gr * D + (ch * KL + lane) * E, a.gdt, gv[i][ch]);
              } else {
#pragma unroll
                for (int e = 0; e < E; ++e) gv[i][ch][e] = 0.f;
              }
            }
          }
#pragma unroll
          for (int i = 0; i < GB; ++i) {
            const double sc = x0 + i < cur.c ? s_sc[cur.base + x0 + i] : 0.0;
#pragma unroll
            for (int ch = 0; ch < CH; ++ch)
#pragma unroll
              for (int e = 0; e < E; ++e) acc[ch][e] += (double)gv[i][ch][e] * sc;
          }
        }
        update_store<D, TP, OPT, KL>(a, cur.prow, lane, acc, cur.w, cur.s0, cur.s1);
        if (lane == 0 && cur.st != 0) {
          const int row = s_r[cur.k];
          if (cur.st == 2) a.t.slots[s_sl[cur.k]].row = row;
          a.urows[t0 + cur.k] = row;
        }
      }
    } else {
      // more entries than the stage holds: one key at a time, the entries
      // straight from global memory, KL at a time (one per lane)
      for (int q = tid / KL; q < nact; q += GPB) {
        const int k = s_perm[q], c = s_c[k], st = s_st[k];
        char* prow = s_ptr[k];
        float w[CH][E], s0[CH][E], s1[CH][E];
        load_row<D, TP, OPT, KL>(a, prow, st == 2, s_key[k], lane, w, s0, s1);
        double acc[CH][E];
#pragma unroll
        for (int ch = 0; ch < CH; ++ch)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[ch][e] = 0.0;
        const int ko = s_o[k];
        for (int b0 = 0; b0 < c; b0 += KL) {
          const int cnt = c - b0 < KL ? c - b0 : KL;
          int gr = 0;
          double scale = 0.0;
          if (lane < cnt) grad_ref<D>(a, a.grouped[ko + b0 + lane], gr, scale);
          for (int x = 0; x < cnt; ++x)
            add_grad_row<D, TP, KL>(a, __shfl(gr, gbase + x), shfl_d(scale, gbase + x), lane, acc);
        }
        update_store<D, TP, OPT, KL>(a, prow, lane, acc, w, s0, s1);
        if (lane == 0 && st != 0) {
          const int row = s_r[k];
          if (st == 2) a.t.slots[s_sl[k]].row = row;
          a.urows[t0 + k] = row;
        }
      }
    }
    __syncthreads();  // the tile's LDS is reused by the next tile
  }
}

template <int D, typename TP>
void fwd_dispatch(const FwdArgs& a, int pool, hipStream_t s) {
  constexpr int C = D / Vec<TP>::E;
  constexpr int GPB = 256 / C;
  if (pool == RECIS_POOL_NONE) {
    if (a.N == 0) return;
    const long long per_block = (long long)GPB * kGatherPer;
    RECIS_LAUNCH("k_fwd_gather", (k_fwd_gather<D, TP>), dim3((unsigned)((a.N + per_block - 1) / per_block)), dim3(256), s, a);
  } else {
    if (a.nbags == 0) return;
    constexpr int BB = FwdShape<C>::BB;
    RECIS_LAUNCH("k_fwd_pool", (k_fwd_pool<D, TP>), dim3((unsigned)((a.nbags + BB - 1) / BB)), dim3(256), s, a);
  }
}

// The long keys' plan in feature order.  Chunks of one feature then run
// together, and the waves in flight share that feature's rows of the
// upstream gradient in the memory-side cache instead of each fetching its
// own from HBM -- worth it when the gradient is larger than that cache.
// Three launches over the long keys (bin = the key's feature bin):
// k_long_hist counts keys and chunks per bin (block histograms in LDS, one
// global add per bin and block); k_long_scan turns the bins into bases (one
// block); k_long_place gives every key its place and first chunk with one
// 64-bit add on its bin (place << 32 | chunks), so places and chunk bases
// rise together, and writes its chunks' owner.
//
// With hot keys (pooled gradients): before these, k_hot_hist counts the
// eligible long keys of each bin by count class (floor(log2 count)) and
// k_hot_plan picks, per bin, the classes from the top down while they hold
// at most the pass's key limit: those keys are the bin's hot keys.  A hot
// key gets no chunks; k_long_place gives it its index among its bin's hot
// keys and its partial rows (one per block of kHotBags bags), which
// k_bwd_hot writes and the final pass sums like chunk partials.
__global__ void k_zero_u64(unsigned long long* p, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}
__device__ __forceinline__ int feat_bin(const BwdArgs& a, int u) {
  return (int)(((unsigned long long)a.ukeys[u] >> 48) & (kFeatBins - 1));
}
__device__ __forceinline__ int count_class(int c) { return 31 - __clz(c); }
// A long key is eligible when its count is at least hot_min and it is a
// key (not the mark of failed transforms, whose bin is no feature's); it is
// hot when its class reached its bin's threshold (kHotClasses: no hot keys
// in the bin).
__device__ __forceinline__ bool hot_eligible(const BwdArgs& a, int u, int c) {
  return c >= a.hot_min && a.ukeys[u] >= 0;
}
__device__ __forceinline__ bool is_hot(const BwdArgs& a, int u, int bin) {
  if (!a.hot) return false;
  const int c = a.counts[u];
  return hot_eligible(a, u, c) && count_class(c) >= a.hot_thr[bin];
}

__global__ __launch_bounds__(256) void k_hot_hist(BwdArgs a) {
  const int nlong = a.plan[0];
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= nlong || !a.plan[kPlanHotOk]) return;
  const int u = a.plan[a.pl.o_long_u + idx];
  const int c = a.counts[u];
  if (hot_eligible(a, u, c)) atomicAdd(&a.hot_cls[feat_bin(a, u) * kHotClasses + count_class(c)], 1u);
}

// One block: per bin the threshold class and hot-key count, then the bins'
// first hot indices (an exclusive scan).
template <int KMAX>
__global__ __launch_bounds__(1024) void k_hot_plan(BwdArgs a) {
  constexpr int kPer = kFeatBins / 1024;
  __shared__ int s_w[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool ok = a.plan[kPlanHotOk] != 0;
  int n[kPer], run = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = tid * kPer + k;
    unsigned x[kHotClasses];
    const uint4* p = reinterpret_cast<const uint4*>(a.hot_cls + b * kHotClasses);
#pragma unroll
    for (int q = 0; q < kHotClasses / 4; ++q) {
      const uint4 v = p[q];
      x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
    }
    // the classes from the top down while they fit; the lowest one taken
    // (with keys) is the threshold
    int thr = kHotClasses, tot = 0;
    bool open = ok;
#pragma unroll
    for (int c = kHotClasses - 1; c >= 0; --c) {
      open = open && tot + (int)x[c] <= KMAX;
      if (open) {
        tot += (int)x[c];
        if (x[c]) thr = c;
      }
    }
    a.hot_thr[b] = tot ? thr : kHotClasses;
    a.hot_n[b] = tot;
    a.hot_cnt[b] = 0;
    n[k] = tot;
    run += tot;
  }
  int inc = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  int base = inc - run;
  for (int x = 0; x < w; ++x) base += s_w[x];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    a.hot_base[tid * kPer + k] = base;
    base += n[k];
  }
  if (tid == 1023) a.t.ctr->hot_keys += (unsigned long long)base;
}

__global__ __launch_bounds__(256) void k_long_hist(BwdArgs a, unsigned long long* bins) {
  __shared__ unsigned long long s_b[kFeatBins];
  const int nlong = a.plan[0];
  if ((long long)blockIdx.x * 256 >= nlong) return;
  for (int i = threadIdx.x; i < kFeatBins; i += 256) s_b[i] = 0;
  __syncthreads();
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx < nlong) {
    const int u = a.plan[a.pl.o_long_u + idx], nch = a.plan[a.pl.o_long_nch + idx];
    const int bin = feat_bin(a, u);
    atomicAdd(&s_b[bin], (1ull << 32) | (unsigned)(is_hot(a, u, bin) ? 0 : nch));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kFeatBins; i += 256)
    if (s_b[i]) atomicAdd(&bins[i], s_b[i]);
}

// In place: bins[i] becomes the exclusive prefix of (keys << 32 | chunks);
// the chunks in all to *nchunks.
__global__ __launch_bounds__(1024) void k_long_scan(unsigned long long* bins, int* nchunks) {
  constexpr int kPer = kFeatBins / 1024;
  __shared__ unsigned long long s_w[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  unsigned long long v[kPer], run = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    v[k] = bins[tid * kPer + k];
    run += v[k];
  }
  unsigned long long inc = run;  // inclusive over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const unsigned long long y = (unsigned long long)__shfl_up((long long)inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  unsigned long long base = inc - run;
  for (int x = 0; x < w; ++x) base += s_w[x];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    bins[tid * kPer + k] = base;
    base += v[k];
  }
  if (tid == 1023) *nchunks = (int)(base & 0xFFFFFFFFull);
}

__global__ __launch_bounds__(256) void k_long_place(BwdArgs a, unsigned long long* bins, int* out_u, int* out_base,
                                                    int* out_nch, int* out_owner) {
  const int nlong = a.plan[0];
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= nlong) return;
  const int u = a.plan[a.pl.o_long_u + idx], nch = a.plan[a.pl.o_long_nch + idx];
  const int bin = feat_bin(a, u);
  const bool hot = is_hot(a, u, bin);
  const unsigned long long at = atomicAdd(&bins[bin], (1ull << 32) | (unsigned)(hot ? 0 : nch));
  const int pos = (int)(at >> 32), cb = (int)(at & 0xFFFFFFFFull);
  out_u[pos] = u;
  if (hot) {
    const int h = atomicAdd(&a.hot_cnt[bin], 1);  // below hot_n[bin]: the same test counted it
    a.hot_of[u] = (unsigned char)h;
    out_nch[pos] = a.hot_nc;
    out_base[pos] = -1 - (a.hot_base[bin] + h) * a.hot_nc;
    return;
  }
  out_nch[pos] = nch;
  out_base[pos] = cb;
  for (int k = 0; k < nch; ++k) out_owner[cb + k] = pos;
}

// Per distinct key: no hot index yet (a byte each, the hot indices being
// below hot_kmax <= kHotNone).
constexpr unsigned char kHotNone = 255;
__global__ __launch_bounds__(256) void k_hot_fill(BwdArgs a) {
  const long long U = *a.num_unique;
  for (long long u = (long long)blockIdx.x * 256 + threadIdx.x; u < U; u += (long long)gridDim.x * 256)
    a.hot_of[u] = kHotNone;
}

// Hot keys, bag-major, in two launches.  A stage is STAGE consecutive bags
// of one feature.
//  - k_hot_sort, one block per stage: the stage's occurrences that belong to
//    a hot key, sorted by hot index (a counting sort in LDS), written as
//    (key << 16 | bag within the stage) from the stage's first occurrence
//    slot on, and their count.  This launch does the per-occurrence lookups
//    (occurrence -> distinct key -> hot index), with little LDS per block and
//    so many blocks in flight to hide them.
//  - k_bwd_hot, one block per (block of kHotBags bags, feature): the bags'
//    gradient rows are read once and staged in LDS a stage at a time, with
//    the stage's sorted entries; the waves split the entries evenly and sum
//    each run of one key in double precision in registers, adding the run to
//    the key's LDS sum at its end (an LDS double add; runs of one key meet
//    only where a wave's share starts or ends).  The block writes one partial
//    per hot key of its feature's bin, zero where the key does not occur.
//    The next stage's rows and entries are loaded while one is summed.
// A key's gradient sum is the same set of terms (row * scale, the scale 1 /
// bag length for mean pooling) as in the chunked plan, in another order.
constexpr int kHotThreads = 1024;
constexpr int kHotUnroll = 8;
constexpr int kHotEnt = 4096;  // sorted entries staged at a time (a stage has more only with long bags)
template <int D>
struct HotShape {
  static constexpr int E = D / 64;        // gradient elements per lane (D = 64 or 128)
  static constexpr int KMAX = 8192 / D;   // hot keys per bin: 64 KB of sums (hot_kmax)
  static constexpr int STAGE = 16384 / D; // bags staged at a time: 64 KB of fp32 rows (hot_stage)
  static constexpr int LOADS = STAGE * D / 4 / kHotThreads;  // 4-element loads per thread and stage
  static constexpr int EPT = kHotEnt / kHotThreads;          // staged entries per thread
};

constexpr int kSortThreads = 256;
constexpr int kSortPer = 4;
template <int D>
__global__ __launch_bounds__(kSortThreads) void k_hot_sort(BwdArgs a, const int* inverse) {
  constexpr int STAGE = HotShape<D>::STAGE, KMAX = HotShape<D>::KMAX;
  constexpr int BATCH = kSortThreads * kSortPer;
  static_assert(STAGE <= 256, "a bag within the stage fits a byte");
  static_assert(KMAX <= kHotNone, "a hot index fits a byte below kHotNone");
  __shared__ int s_off[STAGE + 1];
  __shared__ unsigned char s_obag[BATCH];
  __shared__ int s_kc[KMAX];
  __shared__ int s_ks[KMAX + 1];
  if (!a.plan[kPlanHotOk]) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = blockIdx.x;
  const int f = g / a.hot_spf, st = g - f * a.hot_spf;
  const int nh = a.hot_n[a.plan[a.pl.o_fbin + f]];
  if (nh == 0) return;  // the same for the whole block
  const int i0 = st * STAGE;
  const int sn = a.B - i0 < STAGE ? a.B - i0 : STAGE;
  const long long fb = (long long)f * a.B + i0;
  for (int i = tid; i <= sn; i += kSortThreads) s_off[i] = a.off[fb + i];
  for (int i = tid; i < KMAX; i += kSortThreads) s_kc[i] = 0;
  __syncthreads();
  const int jlo = s_off[0], jhi = s_off[sn];
  int count = 0;
  for (int jb = jlo; jb < jhi; jb += BATCH) {
    const int je = jhi - jb < BATCH ? jhi : jb + BATCH;
    // each bag of the stage marks its occurrences in the batch
    for (int t = tid; t < sn; t += kSortThreads) {
      int j = s_off[t], j1 = s_off[t + 1];
      j = j > jb ? j : jb;
      j1 = j1 < je ? j1 : je;
      for (; j < j1; ++j) s_obag[j - jb] = (unsigned char)t;
    }
    // hot indices, every load from an index inside the batch
    int u[kSortPer], h[kSortPer], rk[kSortPer];
#pragma unroll
    for (int k = 0; k < kSortPer; ++k) {
      const int j = jb + tid + k * kSortThreads;
      u[k] = inverse[j < je ? j : je - 1];
    }
#pragma unroll
    for (int k = 0; k < kSortPer; ++k) {
      const int x = a.hot_of[u[k]];
      h[k] = x == kHotNone ? -1 : x;
    }
#pragma unroll
    for (int k = 0; k < kSortPer; ++k) {
      if (jb + tid + k * kSortThreads >= je) h[k] = -1;
      rk[k] = h[k] >= 0 ? atomicAdd(&s_kc[h[k]], 1) : 0;
    }
    __syncthreads();
    if (w == 0) {  // exclusive scan of the per-key counts; the counts back to zero
      constexpr int P = (KMAX + 63) / 64;
      int v[P], sum = 0;
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int x = lane * P + q;
        v[q] = x < nh ? s_kc[x] : 0;
        if (x < KMAX) s_kc[x] = 0;
        sum += v[q];
      }
      int inc = sum;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d);
        if (lane >= d) inc += y;
      }
      int run = inc - sum;
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int x = lane * P + q;
        if (x < nh) s_ks[x] = run;
        run += v[q];
      }
      if (lane == 63) s_ks[nh] = inc;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSortPer; ++k)
      if (h[k] >= 0)
        a.hot_ent[(long long)jlo + count + s_ks[h[k]] + rk[k]] =
            ((unsigned)h[k] << 16) | (unsigned)s_obag[tid + k * kSortThreads];
    count += s_ks[nh];
    __syncthreads();  // s_obag and s_ks are reused by the next batch
  }
  if (tid == 0) a.hot_scnt[g] = count;
}

template <int D>
__global__ __launch_bounds__(kHotThreads) void k_bwd_hot(BwdArgs a) {
  using S = HotShape<D>;
  constexpr int E = S::E, KMAX = S::KMAX, STAGE = S::STAGE, LOADS = S::LOADS, EPT = S::EPT;
  static_assert(LOADS >= 1 && STAGE * D == LOADS * 4 * kHotThreads, "a stage is whole loads");
  static_assert(kHotBags % STAGE == 0, "a block is whole stages");
  __shared__ double s_acc[KMAX * D];
  __shared__ float s_grad[(STAGE + 1) * D];  // row STAGE stays zero: the padding entries' row
  __shared__ double s_scale[STAGE + 1];
  __shared__ unsigned s_list[kHotEnt];
  __shared__ int s_off[kHotBags + 1];
  if (!a.plan[kPlanHotOk]) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = blockIdx.x, f = blockIdx.y;
  const int bin = a.plan[a.pl.o_fbin + f];
  const int nh = a.hot_n[bin];
  if (nh == 0) return;  // the same for the whole block
  const int hb = a.hot_base[bin];
  const int i0 = c * kHotBags;
  const int nb = a.B - i0 < kHotBags ? a.B - i0 : kHotBags;
  const long long fb = (long long)f * a.B + i0;  // merged index of the first bag
  const int g0 = f * a.hot_spf + c * (kHotBags / STAGE);  // the block's first stage
  const bool mean = a.pool == RECIS_POOL_MEAN;
  for (int i = tid; i < nh * D; i += kHotThreads) s_acc[i] = 0.0;
  for (int i = tid; i <= nb; i += kHotThreads) s_off[i] = a.off[fb + i];
  if (tid < D) s_grad[STAGE * D + tid] = 0.f;
  if (tid == 0) s_scale[STAGE] = 0.0;
  __syncthreads();
  // a stage's loads: LOADS gradient quads and the first kHotEnt of its
  // sorted entries, from indices clamped into range
  float gq[LOADS][4];
  unsigned ge[EPT];
  int gcnt = 0;
  auto load_stage = [&](int sb0) {
    const int sn = nb - sb0 < STAGE ? nb - sb0 : STAGE;
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const int x = tid + k * kHotThreads;  // quad x: bag x / (D / 4), quad x % (D / 4)
      int bl = x / (D / 4);
      bl = bl < sn ? bl : sn - 1;
      const long long i = i0 + sb0 + bl;  // bag within the feature
      load_grad<4>(a.grad, (i * a.F + f) * D + (x % (D / 4)) * 4, a.gdt, gq[k]);
    }
    gcnt = a.hot_scnt[g0 + sb0 / STAGE];
    const long long jlo = s_off[sb0];
    const int last = gcnt > 0 ? gcnt - 1 : 0;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = tid + k * kHotThreads;
      // an entry of the stage; with none, the stage's first occurrence slot
      // (or slot 0 past the last occurrence): read, never used
      const long long j = gcnt > 0 ? jlo + (e < gcnt ? e : last) : (jlo < a.n_occ ? jlo : 0);
      ge[k] = a.hot_ent[j];
    }
  };
  // The share [r0, r1) of one wave in entries [0, ne) of s_list, 64 entries
  // at a time: each lane reads one entry, its row's place and (mean pooling)
  // its bag's scale, and notes whether a run ends there (the next entry has
  // another key, or it is the last one); one ballot gives the wave those
  // ends, and the wave takes the entries one by one from those lanes, the
  // 64 positions unrolled.  Per entry that is one LDS read, a conversion and
  // a double add on the vector side and one bit test on the scalar side (the
  // CU's one scalar unit, shared by all its waves, would otherwise bound the
  // pass); a run's end is a branch the wave takes or skips.  Entries past the
  // share read the zero row.
  auto accumulate = [&](int ne, auto mean_tag) __attribute__((always_inline)) {
    constexpr bool MEAN = decltype(mean_tag)::value;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int r0 = __builtin_amdgcn_readfirstlane((int)((long long)ne * wu / (kHotThreads / 64)));
    const int r1 = __builtin_amdgcn_readfirstlane((int)((long long)ne * (wu + 1) / (kHotThreads / 64)));
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    for (int rb = r0; rb < r1; rb += 64) {
      const int cnt = r1 - rb < 64 ? r1 - rb : 64;
      const bool valid = lane < cnt;
      const unsigned my_en = s_list[valid ? rb + lane : r1 - 1];
      const int my_key = (int)(my_en >> 16);
      const int my_bag = valid ? (int)(my_en & 0xFFFFu) : STAGE;
      const int my_row = my_bag * D;
      double my_sc = 1.0;
      if constexpr (MEAN) my_sc = s_scale[my_bag];
      const int my_lo = __double2loint(my_sc), my_hi = __double2hiint(my_sc);
      const int next_key = __shfl_down(my_key, 1);
      const unsigned long long ends = __ballot(valid && (lane == cnt - 1 || next_key != my_key));
#pragma unroll
      for (int gi = 0; gi < 64 / kHotUnroll; ++gi) {
        if (gi * kHotUnroll >= cnt) break;  // the same for the whole wave
        float gv[kHotUnroll][E];
#pragma unroll
        for (int v = 0; v < kHotUnroll; ++v) {
          const int row = __builtin_amdgcn_readlane(my_row, gi * kHotUnroll + v);
#pragma unroll
          for (int e = 0; e < E; ++e) gv[v][e] = s_grad[row + e * 64 + lane];
        }
#pragma unroll
        for (int v = 0; v < kHotUnroll; ++v) {
          const int q = gi * kHotUnroll + v;
          if constexpr (MEAN) {
            const double sc =
                __hiloint2double(__builtin_amdgcn_readlane(my_hi, q), __builtin_amdgcn_readlane(my_lo, q));
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += (double)gv[v][e] * sc;
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += (double)gv[v][e];
          }
          if (ends & (1ull << q)) {
            const int h = __builtin_amdgcn_readlane(my_key, q);
#pragma unroll
            for (int e = 0; e < E; ++e) {
              atomicAdd(&s_acc[h * D + e * 64 + lane], acc[e]);
              acc[e] = 0.0;
            }
          }
        }
      }
    }
  };
  auto accumulate_any = [&](int ne) __attribute__((always_inline)) {
    if (mean) accumulate(ne, std::true_type{});
    else accumulate(ne, std::false_type{});
  };
  if (nb > 0) load_stage(0);
  for (int sb0 = 0; sb0 < nb; sb0 += STAGE) {
    const int sn = nb - sb0 < STAGE ? nb - sb0 : STAGE;
    const int cnt = gcnt;
    const long long jlo = s_off[sb0];
    __syncthreads();  // the previous stage's rows and entries are no longer read
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const int x = tid + k * kHotThreads;
      const int bl = x / (D / 4), q = x % (D / 4);
      if (bl < sn)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_grad[bl * D + q * 4 + e] = gq[k][e];
    }
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = tid + k * kHotThreads;
      if (e < cnt) s_list[e] = ge[k];
    }
    if (tid < sn) {
      const int len = s_off[sb0 + tid + 1] - s_off[sb0 + tid];
      s_scale[tid] = mean ? 1.0 / (double)(len > 0 ? len : 1) : 1.0;
    }
    __syncthreads();
    if (sb0 + STAGE < nb) load_stage(sb0 + STAGE);  // in flight while this stage is summed
    accumulate_any(cnt < kHotEnt ? cnt : kHotEnt);
    // a stage with more entries than s_list holds (long bags): the rest, a
    // part at a time (their loads also wait for the prefetch: rare)
    for (int e0 = kHotEnt; e0 < cnt; e0 += kHotEnt) {
      const int ne = cnt - e0 < kHotEnt ? cnt - e0 : kHotEnt;
      __syncthreads();
      for (int e = tid; e < ne; e += kHotThreads) s_list[e] = a.hot_ent[jlo + e0 + e];
      __syncthreads();
      accumulate_any(ne);
    }
  }
  __syncthreads();
  // partial (hb + h) * hot_nc + c of each hot key h of the bin
  for (int i = tid; i < nh * D; i += kHotThreads) {
    const int h = i / D, d = i - h * D;
    a.hot_partials[((long long)(hb + h) * a.hot_nc + c) * D + d] = s_acc[i];
  }
}

template <int D, typename TP, int OPT>
void bwd_dispatch(BwdArgs a, long long n, hipStream_t s) {
  constexpr int NCH = D / Vec<TP>::E;
  constexpr int KL = NCH < kBwdLanes ? NCH : kBwdLanes;
  long long lb = (n / kChunk + 4) / 4;
  lb = lb > 2048 ? 2048 : (lb < 1 ? 1 : lb);
  RECIS_LAUNCH("k_bwd_long_partial", (k_bwd_long_partial<D, TP>), dim3((unsigned)lb), dim3(256), s, a);
  if constexpr (D == 64 || D == 128) {
    if (a.hot)
      RECIS_LAUNCH("k_bwd_hot", k_bwd_hot<D>, dim3((unsigned)a.hot_nc, (unsigned)a.F), dim3(kHotThreads), s, a);
  }
  long long fb = (n / (kShortMax + 1) + 4) / 4;  // long keys <= n / (kShortMax + 1), four per block
  fb = fb > 2048 ? 2048 : (fb < 1 ? 1 : fb);
  RECIS_LAUNCH("k_bwd_long_final", (k_bwd_long_final<D, TP, OPT>), dim3((unsigned)fb), dim3(256), s, a);
  long long sb = (n + kBwdKeys - 1) / kBwdKeys;
  sb = sb > 4096 ? 4096 : (sb < 1 ? 1 : sb);
  RECIS_LAUNCH("k_bwd_short", (k_bwd_short<D, TP, OPT, KL>), dim3((unsigned)sb), dim3(256), s, a);
}

template <typename TP, int OPT>
void bwd_dim(const BwdArgs& a, int dim, long long n, hipStream_t s) {
  switch (dim) {
    case 8: bwd_dispatch<8, TP, OPT>(a, n, s); break;
    case 16: bwd_dispatch<16, TP, OPT>(a, n, s); break;
    case 32: bwd_dispatch<32, TP, OPT>(a, n, s); break;
    case 64: bwd_dispatch<64, TP, OPT>(a, n, s); break;
    case 128: bwd_dispatch<128, TP, OPT>(a, n, s); break;
    case 256: bwd_dispatch<256, TP, OPT>(a, n, s); break;
  }
}

template <typename TP>
void fwd_dim(const FwdArgs& a, int dim, int pool, hipStream_t s) {
  switch (dim) {
    case 8: fwd_dispatch<8, TP>(a, pool, s); break;
    case 16: fwd_dispatch<16, TP>(a, pool, s); break;
    case 32: fwd_dispatch<32, TP>(a, pool, s); break;
    case 64: fwd_dispatch<64, TP>(a, pool, s); break;
    case 128: fwd_dispatch<128, TP>(a, pool, s); break;
    case 256: fwd_dispatch<256, TP>(a, pool, s); break;
  }
}

}  // namespace

void launch_forward(const recis_lookup_result& res, const TableDev& t, int pool, void* out,
                    bool current, hipStream_t s) {
  FwdArgs a;
  const PlanLayout pl = plan_layout(res.capacity);
  a.off = res.bag_offsets;
  a.inverse = res.inverse;
  a.urows = reinterpret_cast<const long long*>(res.unique_rows);
  a.ukeys = reinterpret_cast<const long long*>(res.unique_keys);
  a.idslot = reinterpret_cast<const unsigned*>(res.plan + pl.o_idslot);
  a.occref = reinterpret_cast<const long long*>(res.plan + pl.o_occref);
  a.current = current ? 1 : 0;
  a.N = res.n;
  a.nbags = (long long)res.num_feats * res.batch;
  a.F = res.num_feats;
  a.B = res.batch;
  a.pool = pool;
  a.out = out;
  a.t = t;
  if (t.dtype == RECIS_DTYPE_BF16) fwd_dim<bf16_t>(a, t.dim, pool, s);
  else fwd_dim<float>(a, t.dim, pool, s);
}

recis_status launch_backward(const recis_lookup_result& res, const TableDev& t, int pool,
                             const void* grad, int grad_dtype, const OptConsts& oc,
                             double* partials, int* reorder, long long reorder_ints,
                             double* hot_partials, long long hot_rows, int* hot_ws, long long hot_ws_len,
                             bool current, hipStream_t s) {
  if (res.n == 0) return RECIS_OK;
  BwdArgs a;
  a.current = current ? 1 : 0;
  a.off = res.bag_offsets;
  a.grouped = res.grouped;
  a.uoff = res.unique_offsets;
  a.counts = res.counts;
  a.urows = reinterpret_cast<long long*>(res.unique_rows);
  a.ukeys = reinterpret_cast<const long long*>(res.unique_keys);
  a.num_unique = reinterpret_cast<const long long*>(res.num_unique);
  a.plan = res.plan;
  a.pl = plan_layout(res.capacity);
  a.idslot = reinterpret_cast<const unsigned*>(res.plan + a.pl.o_idslot);
  a.F = res.num_feats;
  a.B = res.batch;
  a.pool = pool;
  a.gdt = grad_dtype;
  a.grad = grad;
  a.oc = oc;
  a.t = t;
  a.partials = partials;
  a.long_u = res.plan + a.pl.o_long_u;
  a.long_base = res.plan + a.pl.o_long_base;
  a.long_nch = res.plan + a.pl.o_long_nch;
  a.owner = res.plan + a.pl.o_chunk_owner;
  a.nchunks = nullptr;
  a.hot = 0;
  a.hot_nc = (int)hot_blocks(res.batch);
  a.hot_min = hot_min_count(a.hot_nc);
  a.hot_partials = hot_partials;
  // The long keys' plan is rebuilt feature by feature (see k_long_place) for
  // pooled gradients larger than the memory-side cache, and whenever hot keys
  // are summed bag-major (the hot pass needs room for every feature's hot
  // keys, and the plan room for its hot indices).
  const bool pooled = pool != RECIS_POOL_NONE;
  const int kmax = hot_kmax(t.dim);
  bool hot = pooled && kmax > 0 && hot_partials && hot_ws && res.num_feats <= kFeatBins &&
             (long long)res.num_feats * kmax * a.hot_nc <= hot_rows &&
             hot_ws_ints(res.n, res.num_feats, res.batch, t.dim) <= hot_ws_len;
  a.hot_spf = (int)hot_stages(res.batch, t.dim);
  a.n_occ = res.n;
  const double grad_bytes = (double)res.num_feats * res.batch * t.dim * (grad_dtype == RECIS_DTYPE_BF16 ? 2 : 4);
  const long long maxl = res.n / (kShortMax + 1) + 1, maxc = res.n / kChunk + maxl + 1;
  const long long bins_at = (3 * maxl + maxc + 1) & ~1ll;  // 8-byte aligned (the scratch is)
  const long long plain_need = bins_at + 2 * (long long)kFeatBins + 2;
  if (pooled && reorder_ints > 0 && (hot || grad_bytes > kMemCacheBytes) && plain_need <= reorder_ints) {
    int* ou = reorder;
    int* ob = ou + maxl;
    int* on = ob + maxl;
    int* oo = on + maxl;
    unsigned long long* bins = reinterpret_cast<unsigned long long*>(reorder + bins_at);
    int* ncold = reorder + bins_at + 2 * kFeatBins;
    const unsigned kb = (unsigned)((maxl + 255) / 256);
    RECIS_LAUNCH("k_long_zero", k_zero_u64, dim3(kFeatBins / 256), dim3(256), s, bins, (long long)kFeatBins);
    if (hot) {
      a.hot = 1;
      a.hot_cls = reinterpret_cast<unsigned*>(hot_ws);  // 16-byte aligned: k_hot_plan reads it by 4
      a.hot_thr = hot_ws + (long long)kFeatBins * kHotClasses;
      a.hot_n = a.hot_thr + kFeatBins;
      a.hot_base = a.hot_n + kFeatBins;
      a.hot_cnt = a.hot_base + kFeatBins;
      a.hot_ent = reinterpret_cast<unsigned*>(a.hot_cnt + kFeatBins);
      a.hot_of = reinterpret_cast<unsigned char*>(a.hot_ent + res.n);
      a.hot_scnt = reinterpret_cast<int*>(a.hot_of) + (res.n + 3) / 4;
      const long long cls_u64 = (long long)kFeatBins * kHotClasses / 2;
      RECIS_LAUNCH("k_long_zero", k_zero_u64, dim3((unsigned)((cls_u64 + 255) / 256)), dim3(256), s,
                   reinterpret_cast<unsigned long long*>(a.hot_cls), cls_u64);
      const long long fg = std::min<long long>(4096, res.n / 256 + 1);
      RECIS_LAUNCH("k_hot_fill", k_hot_fill, dim3((unsigned)fg), dim3(256), s, a);
      RECIS_LAUNCH("k_hot_hist", k_hot_hist, dim3(kb), dim3(256), s, a);
      if (kmax == hot_kmax(64))
        RECIS_LAUNCH("k_hot_plan", k_hot_plan<HotShape<64>::KMAX>, dim3(1), dim3(1024), s, a);
      else
        RECIS_LAUNCH("k_hot_plan", k_hot_plan<HotShape<128>::KMAX>, dim3(1), dim3(1024), s, a);
    }
    RECIS_LAUNCH("k_long_hist", k_long_hist, dim3(kb), dim3(256), s, a, bins);
    RECIS_LAUNCH("k_long_scan", k_long_scan, dim3(1), dim3(1024), s, bins, ncold);
    RECIS_LAUNCH("k_long_place", k_long_place, dim3(kb), dim3(256), s, a, bins, ou, ob, on, oo);
    if (hot) {
      const unsigned sg = (unsigned)((long long)res.num_feats * a.hot_spf);
      if (t.dim == 64)
        RECIS_LAUNCH("k_hot_sort", k_hot_sort<64>, dim3(sg), dim3(kSortThreads), s, a, res.inverse);
      else
        RECIS_LAUNCH("k_hot_sort", k_hot_sort<128>, dim3(sg), dim3(kSortThreads), s, a, res.inverse);
    }
    a.long_u = ou;
    a.long_base = ob;
    a.long_nch = on;
    a.owner = oo;
    a.nchunks = ncold;
  }
  if (t.dtype == RECIS_DTYPE_BF16) {
    if (t.optim == RECIS_OPTIM_ADAGRAD) bwd_dim<bf16_t, RECIS_OPTIM_ADAGRAD>(a, t.dim, res.n, s);
    else bwd_dim<bf16_t, RECIS_OPTIM_ADAM>(a, t.dim, res.n, s);
  } else {
    if (t.optim == RECIS_OPTIM_ADAGRAD) bwd_dim<float, RECIS_OPTIM_ADAGRAD>(a, t.dim, res.n, s);
    else bwd_dim<float, RECIS_OPTIM_ADAM>(a, t.dim, res.n, s);
  }
  return RECIS_OK;
}

}  // namespace recis
