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
// elements); a "group" of C = row_bytes / 16 lanes of one 64-lane wavefront
// owns one bag (forward) or one distinct key (backward), so a wave moves
// 64 / C rows per instruction with full 16-byte loads.
// Backward, no atomics on data: each key's occurrences were grouped by
// insert_find.  Keys with <= kShortMax occurrences are reduced by one group
// and updated at once; longer keys are cut into kChunk-occurrence chunks, one
// wave per chunk sums its share across its groups with cross-lane shuffles,
// writes a double-precision partial, and the last chunk to finish (one
// counter per key) sums the partials in chunk order and applies the update.
#include "internal.h"

namespace recis {

namespace {

struct FwdArgs {
  const int* off;
  const int* inverse;
  const long long* urows;
  long long N;
  long long nbags;
  int F, B, pool;
  void* out;
  RowSpace rs;
};

template <typename TP>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int E = 4;
  __device__ static void load(const void* p, float (&v)[4]) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  __device__ static void store(void* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
struct bf16_t {
  unsigned short bits;
};
template <>
struct Vec<bf16_t> {
  static constexpr int E = 8;
  __device__ static void load(const void* p, float (&v)[8]) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const unsigned w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static void store(void* p, const float (&v)[8]) {
    uint4 x;
    x.x = (unsigned)f32_to_bf16(v[0]) | ((unsigned)f32_to_bf16(v[1]) << 16);
    x.y = (unsigned)f32_to_bf16(v[2]) | ((unsigned)f32_to_bf16(v[3]) << 16);
    x.z = (unsigned)f32_to_bf16(v[4]) | ((unsigned)f32_to_bf16(v[5]) << 16);
    x.w = (unsigned)f32_to_bf16(v[6]) | ((unsigned)f32_to_bf16(v[7]) << 16);
    *reinterpret_cast<uint4*>(p) = x;
  }
};

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

// ------------------------------------------------------------- forward
template <int D, typename TP>
__global__ __launch_bounds__(256) void k_fwd_pool(FwdArgs a) {
  constexpr int E = Vec<TP>::E;
  constexpr int C = D / E;  // lanes per bag
  constexpr int GPB = 256 / C;
  const int lane = threadIdx.x % C;
  const long long bag = (long long)blockIdx.x * GPB + threadIdx.x / C;
  if (bag >= a.nbags) return;
  long long lo = a.off[bag], hi = a.off[bag + 1];
  lo = lo < 0 ? 0 : (lo > a.N ? a.N : lo);
  hi = hi < lo ? lo : (hi > a.N ? a.N : hi);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  long long j = lo;
  for (; j + 4 <= hi; j += 4) {
    long long r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = a.urows[a.inverse[j + q]];
    float v[4][E];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (r[q] >= 0) Vec<TP>::load(row_ptr(a.rs, r[q]) + lane * 16, v[q]);
      else
#pragma unroll
        for (int e = 0; e < E; ++e) v[q][e] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += v[q][e];
  }
  for (; j < hi; ++j) {
    const long long r = a.urows[a.inverse[j]];
    if (r >= 0) {
      float v[E];
      Vec<TP>::load(row_ptr(a.rs, r) + lane * 16, v);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += v[e];
    }
  }
  if (a.pool == RECIS_POOL_MEAN && hi > lo) {
    const float len = (float)(hi - lo);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = acc[e] / len;
  }
  const int f = (int)(bag / a.B), i = (int)(bag - (long long)f * a.B);
  float* o = static_cast<float*>(a.out) + ((long long)i * a.F + f) * D + lane * E;
#pragma unroll
  for (int q = 0; q < E / 4; ++q)
    reinterpret_cast<float4*>(o)[q] = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
}

template <int D, typename TP>
__global__ __launch_bounds__(256) void k_fwd_gather(FwdArgs a) {
  constexpr int E = Vec<TP>::E;
  constexpr int C = D / E;
  constexpr int GPB = 256 / C;
  const int lane = threadIdx.x % C;
  const long long j = (long long)blockIdx.x * GPB + threadIdx.x / C;
  if (j >= a.N) return;
  const long long r = a.urows[a.inverse[j]];
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (r >= 0) v = *reinterpret_cast<const uint4*>(row_ptr(a.rs, r) + lane * 16);
  reinterpret_cast<uint4*>(static_cast<char*>(a.out) + (j * D * (long long)sizeof(TP)))[lane] = v;
}

// ------------------------------------------------------------ backward
struct BwdArgs {
  const int* off;       // merged bag offsets
  const int* grouped;
  const int* uoff;
  const int* counts;
  const long long* urows;
  const long long* num_unique;
  const int* plan;
  PlanLayout pl;
  int F, B, pool, gdt;
  const void* grad;
  OptConsts oc;
  RowSpace rs;
  double* partials;
};

// Adds the upstream gradient of one grouped entry (a bag, or an occurrence
// for POOL_NONE) to acc, element chunk `lane`.
template <int D, int E>
__device__ __forceinline__ void add_grad(const BwdArgs& a, int gval, int lane, double (&acc)[E]) {
  float g[E];
  if (a.pool == RECIS_POOL_NONE) {
    load_grad<E>(a.grad, (long long)gval * D + lane * E, a.gdt, g);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += (double)g[e];
  } else {
    const int f = gval / a.B, i = gval - f * a.B;
    load_grad<E>(a.grad, ((long long)i * a.F + f) * D + lane * E, a.gdt, g);
    if (a.pool == RECIS_POOL_MEAN) {
      const int len = a.off[gval + 1] - a.off[gval];
      const double inv = 1.0 / (double)(len > 0 ? len : 1);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += (double)g[e] * inv;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += (double)g[e];
    }
  }
}

// One optimizer step on element chunk `lane` of row r.
template <int D, typename TP, int OPT>
__device__ __forceinline__ void apply_update(const BwdArgs& a, long long r, int lane,
                                             const double (&G)[Vec<TP>::E]) {
  constexpr int E = Vec<TP>::E;
  char* rp = row_ptr(a.rs, r);
  void* wp = rp + lane * 16;
  float* st = reinterpret_cast<float*>(rp + D * (int)sizeof(TP)) + lane * E;
  float w[E], s0[E];
  Vec<TP>::load(wp, w);
  Vec<float>::load(st, *reinterpret_cast<float(*)[4]>(s0));
  if constexpr (E == 8) Vec<float>::load(st + 4, *reinterpret_cast<float(*)[4]>(s0 + 4));
  if constexpr (OPT == RECIS_OPTIM_ADAGRAD) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float g = (float)G[e];
      s0[e] = s0[e] + g * g;
      w[e] = w[e] - a.oc.lr * g / (sqrtf(s0[e]) + a.oc.eps);
    }
  } else {
    float s1[E];
    Vec<float>::load(st + D, *reinterpret_cast<float(*)[4]>(s1));
    if constexpr (E == 8) Vec<float>::load(st + D + 4, *reinterpret_cast<float(*)[4]>(s1 + 4));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float g = (float)G[e];
      s0[e] = a.oc.b1 * s0[e] + a.oc.omb1 * g;
      s1[e] = a.oc.b2 * s1[e] + a.oc.omb2 * (g * g);
      w[e] = w[e] - a.oc.step_size * s0[e] / (sqrtf(s1[e]) + a.oc.eps);
    }
    Vec<float>::store(st + D, *reinterpret_cast<float(*)[4]>(s1));
    if constexpr (E == 8) Vec<float>::store(st + D + 4, *reinterpret_cast<float(*)[4]>(s1 + 4));
  }
  Vec<float>::store(st, *reinterpret_cast<float(*)[4]>(s0));
  if constexpr (E == 8) Vec<float>::store(st + 4, *reinterpret_cast<float(*)[4]>(s0 + 4));
  Vec<TP>::store(wp, w);
}

template <int D, typename TP, int OPT>
__global__ __launch_bounds__(256) void k_bwd_short(BwdArgs a) {
  constexpr int E = Vec<TP>::E;
  constexpr int C = D / E;
  constexpr int GPB = 256 / C;
  const int lane = threadIdx.x % C;
  const long long U = *a.num_unique;
  const long long step = (long long)gridDim.x * GPB;
  for (long long u = (long long)blockIdx.x * GPB + threadIdx.x / C; u < U; u += step) {
    const int c = a.counts[u];
    if (c > kShortMax) continue;
    const long long r = a.urows[u];
    if (r < 0) continue;
    const int o = a.uoff[u];
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    int k = 0;
    for (; k + 4 <= c; k += 4) {
      const int g0 = a.grouped[o + k], g1 = a.grouped[o + k + 1];
      const int g2 = a.grouped[o + k + 2], g3 = a.grouped[o + k + 3];
      add_grad<D, E>(a, g0, lane, acc);
      add_grad<D, E>(a, g1, lane, acc);
      add_grad<D, E>(a, g2, lane, acc);
      add_grad<D, E>(a, g3, lane, acc);
    }
    for (; k < c; ++k) add_grad<D, E>(a, a.grouped[o + k], lane, acc);
    apply_update<D, TP, OPT>(a, r, lane, acc);
  }
}

__device__ __forceinline__ double shfl_xor_d(double v, int m) {
  const unsigned long long b = __double_as_longlong(v);
  const int lo = __shfl_xor((int)(unsigned)b, m), hi = __shfl_xor((int)(unsigned)(b >> 32), m);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

__device__ __forceinline__ double load_coherent(const double* p) {
  const unsigned long long v =
      __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
  return __longlong_as_double((long long)v);
}

template <int D, typename TP, int OPT>
__global__ __launch_bounds__(256) void k_bwd_long(BwdArgs a) {
  constexpr int E = Vec<TP>::E;
  constexpr int C = D / E;
  constexpr int GPW = 64 / C;  // groups per wave
  const int wl = threadIdx.x & 63;
  const int lane = wl % C, g = wl / C;
  const int nchunks = a.plan[1];
  const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long nwaves = (long long)gridDim.x * 4;
  const int* long_u = a.plan + a.pl.o_long_u;
  const int* long_base = a.plan + a.pl.o_long_base;
  const int* long_nch = a.plan + a.pl.o_long_nch;
  int* long_done = const_cast<int*>(a.plan) + a.pl.o_long_done;
  const int* owner = a.plan + a.pl.o_chunk_owner;
  for (long long q = wave; q < nchunks; q += nwaves) {
    const int idx = owner[q];
    const int u = long_u[idx], cb = long_base[idx], nch = long_nch[idx];
    const long long r = a.urows[u];
    const int o = a.uoff[u], c = a.counts[u];
    const int k0 = (int)(q - cb) * kChunk;
    const int k1 = k0 + kChunk < c ? k0 + kChunk : c;
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    for (int k = k0 + g; k < k1; k += GPW) add_grad<D, E>(a, a.grouped[o + k], lane, acc);
#pragma unroll
    for (int m = C; m < 64; m <<= 1)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += shfl_xor_d(acc[e], m);
    if (g == 0) {
      double* pp = a.partials + q * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) pp[e] = acc[e];
    }
    __threadfence();
    int last = 0;
    if (wl == 0) last = atomicAdd(&long_done[idx], 1) == nch - 1;
    last = __shfl(last, 0);
    if (last) {
      __threadfence();
      if (g == 0) {
        double G[E];
#pragma unroll
        for (int e = 0; e < E; ++e) G[e] = 0.0;
        for (int p = 0; p < nch; ++p) {
          const double* pp = a.partials + (long long)(cb + p) * D + lane * E;
#pragma unroll
          for (int e = 0; e < E; ++e) G[e] += load_coherent(pp + e);
        }
        if (r >= 0) apply_update<D, TP, OPT>(a, r, lane, G);
      }
      if (wl == 0) long_done[idx] = 0;
    }
  }
}

template <int D, typename TP>
void fwd_dispatch(const FwdArgs& a, int pool, hipStream_t s) {
  constexpr int C = D / Vec<TP>::E;
  constexpr int GPB = 256 / C;
  if (pool == RECIS_POOL_NONE) {
    if (a.N == 0) return;
    hipLaunchKernelGGL((k_fwd_gather<D, TP>), dim3((unsigned)((a.N + GPB - 1) / GPB)), dim3(256), 0, s, a);
  } else {
    if (a.nbags == 0) return;
    hipLaunchKernelGGL((k_fwd_pool<D, TP>), dim3((unsigned)((a.nbags + GPB - 1) / GPB)), dim3(256), 0, s, a);
  }
}

template <int D, typename TP, int OPT>
void bwd_dispatch(const BwdArgs& a, long long cap, hipStream_t s) {
  constexpr int C = D / Vec<TP>::E;
  constexpr int GPB = 256 / C;
  long long blocks = (cap + GPB - 1) / GPB;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((k_bwd_short<D, TP, OPT>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  long long lb = (cap / kChunk + 4) / 4;
  if (lb > 4096) lb = 4096;
  if (lb < 1) lb = 1;
  hipLaunchKernelGGL((k_bwd_long<D, TP, OPT>), dim3((unsigned)lb), dim3(256), 0, s, a);
}

template <typename TP, int OPT>
void bwd_dim(const BwdArgs& a, int dim, long long cap, hipStream_t s) {
  switch (dim) {
    case 8: bwd_dispatch<8, TP, OPT>(a, cap, s); break;
    case 16: bwd_dispatch<16, TP, OPT>(a, cap, s); break;
    case 32: bwd_dispatch<32, TP, OPT>(a, cap, s); break;
    case 64: bwd_dispatch<64, TP, OPT>(a, cap, s); break;
    case 128: bwd_dispatch<128, TP, OPT>(a, cap, s); break;
    case 256: bwd_dispatch<256, TP, OPT>(a, cap, s); break;
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
                    hipStream_t s) {
  FwdArgs a;
  a.off = res.bag_offsets;
  a.inverse = res.inverse;
  a.urows = reinterpret_cast<const long long*>(res.unique_rows);
  a.N = res.n;
  a.nbags = (long long)res.num_feats * res.batch;
  a.F = res.num_feats;
  a.B = res.batch;
  a.pool = pool;
  a.out = out;
  a.rs = t.rs;
  if (t.dtype == RECIS_DTYPE_BF16) fwd_dim<bf16_t>(a, t.dim, pool, s);
  else fwd_dim<float>(a, t.dim, pool, s);
}

recis_status launch_backward(const recis_lookup_result& res, const TableDev& t, int pool,
                             const void* grad, int grad_dtype, const OptConsts& oc,
                             double* partials, hipStream_t s) {
  BwdArgs a;
  a.off = res.bag_offsets;
  a.grouped = res.grouped;
  a.uoff = res.unique_offsets;
  a.counts = res.counts;
  a.urows = reinterpret_cast<const long long*>(res.unique_rows);
  a.num_unique = reinterpret_cast<const long long*>(res.num_unique);
  a.plan = res.plan;
  a.pl = plan_layout(res.capacity);
  a.F = res.num_feats;
  a.B = res.batch;
  a.pool = pool;
  a.gdt = grad_dtype;
  a.grad = grad;
  a.oc = oc;
  a.rs = t.rs;
  a.partials = partials;
  if (res.n == 0) return RECIS_OK;
  const long long cap = res.n;
  if (t.dtype == RECIS_DTYPE_BF16) {
    if (t.optim == RECIS_OPTIM_ADAGRAD) bwd_dim<bf16_t, RECIS_OPTIM_ADAGRAD>(a, t.dim, cap, s);
    else bwd_dim<bf16_t, RECIS_OPTIM_ADAM>(a, t.dim, cap, s);
  } else {
    if (t.optim == RECIS_OPTIM_ADAGRAD) bwd_dim<float, RECIS_OPTIM_ADAGRAD>(a, t.dim, cap, s);
    else bwd_dim<float, RECIS_OPTIM_ADAM>(a, t.dim, cap, s);
  }
  return RECIS_OK;
}

}  // namespace recis
