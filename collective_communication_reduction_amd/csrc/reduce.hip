// Reduction-family kernels for gfx950: fused all-reduce, reduce-scatter and
// all-gather over N rank buffers resident in one GPU's HBM.
//
// What is computed (DTLM = "Distributed Training for Large Models:
// Collectives, FSDP/ZeRO, DeviceMesh, and Multi-Dimensional Parallelism"):
//   reduce-scatter  owner j gets y_j = sum_i x_{j,i}  (DTLM §2 "Reduce-Scatter")
//   all-gather      every rank gets concat(p_0..p_{N-1}) (DTLM §2 "All-Gather")
//   all-reduce      reduce-scatter then all-gather    (DTLM §2 "All-Reduce")
// The ring fixes the fold order: chunk j is accumulated starting with rank
// j+1's contribution and ending with its owner j's (DTLM §2, N = 4 schedule).
//
// Design.  Every element is independent, so there is no reuse for LDS to
// exploit and no contraction for MFMA: the kernels are pure HBM streams.  The
// grid is chunk-major (tile -> (chunk j, tile t)), which makes the fold's
// starting rank wavefront-uniform, so the N rank pointers are read from the
// kernel arguments with scalar loads and no lane diverges.  Each thread owns U
// 16-byte vectors per tile and issues all N*U loads of a batch before the
// first add, so that enough bytes are in flight to cover HBM latency.  All
// traffic carries the non-temporal hint.  Elements before the first and after
// the last 16-byte-aligned vector of a chunk are handled one by one by tile 0
// of that chunk, in the same order.  Buffers whose relative alignment rules
// out vectors use the element-wise kernels at the end of this file.

#include <algorithm>

#include "device_common.h"
#include "fold.h"
#include "gc_internal.h"

namespace {

using namespace gcdev;

enum Kind { kAllReduce = 0, kReduceScatter = 1 };

template <int P>
struct RedArgs {
  const char* in[P];
  char* out[P];
  uint64_t S;       // elements in the reference index space
  uint64_t c;       // chunk length
  uint32_t N;
  uint32_t ring;
  uint32_t avg;
  uint32_t phase;   // elements before the first aligned vector (0..VE-1)
  uint32_t tpc;     // tiles per chunk
  uint32_t ntiles;  // N * tpc
  float nf;         // (float)N
};

struct ChunkGeom {
  uint64_t lo, hi;    // element range of the chunk
  uint64_t vlo, vhi;  // aligned vectors [vlo, vhi) fully inside the chunk
};

template <int VE, int P>
__device__ __forceinline__ ChunkGeom chunk_geom(const RedArgs<P>& a, uint32_t j) {
  ChunkGeom g;
  g.lo = min(a.S, static_cast<uint64_t>(j) * a.c);
  g.hi = min(a.S, g.lo + a.c);
  const uint64_t ph = a.phase;
  g.vlo = g.lo <= ph ? 0 : (g.lo - ph + VE - 1) / VE;
  g.vhi = g.hi < ph + VE ? 0 : (g.hi - ph) / VE;
  if (g.vhi < g.vlo) g.vhi = g.vlo;
  return g;
}

// Tile layout of the reductions: each wavefront reads a contiguous run of
// U KiB per rank.  Measured on MI355X against the workgroup-strided layout (one
// process, same buffers, 8 x 64 MiB bf16 all-reduce): 5.67-5.77 against
// 5.48-5.54 TB/s on separate per-rank allocations, 6.25-6.29 against
// 6.26-6.28 on the rank arena, equal for the 64-rank reduce-scatter.
#ifndef GC_WAVE_CONTIG
#define GC_WAVE_CONTIG 1
#endif
constexpr bool kWaveContig = GC_WAVE_CONTIG != 0;

template <int U>
__device__ __forceinline__ uint64_t red_tile_vec(uint64_t tv0, int u) {
  return gcdev::tile_vec<U, kWaveContig>(tv0, u);
}

// Element-wise fold of one element E in the chunk's order.
// One tile of U vectors per thread: fold, epilogue, store.  GUARD is false for
// tiles that lie wholly inside the chunk (no predicates anywhere, so the
// compiler keeps every load of a batch in flight together); the chunk's last,
// partial tile sets GUARD: lanes past the last vector reload that vector and
// skip their stores.
template <int KIND, class In, class Out, int NF, int U, bool GUARD, bool WIRE, int P>
__device__ __forceinline__ void reduce_tile(const RedArgs<P>& a, uint32_t N, uint32_t j, uint32_t first,
                                            const ChunkGeom& g, uint64_t tv0) {
  constexpr int VE = In::VE;
  typedef typename In::Acc Acc;
  uint64_t off[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t v = GUARD ? min(red_tile_vec<U>(tv0, u), g.vhi - 1) : red_tile_vec<U>(tv0, u);
    off[u] = (a.phase + v * VE) * In::ES;
  }
  Acc acc[U][VE];
  fold_vec<In, NF, U, WIRE>(a.in, first, N, off, acc);
  const bool avg = a.avg != 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t v = red_tile_vec<U>(tv0, u);
    Acc o[VE];
#pragma unroll
    for (int l = 0; l < VE; ++l) o[l] = finish(acc[u][l], avg, a.nf);
    const Words<Out, VE> w = pack<Out, VE>(o);
    const uint64_t e0 = a.phase + v * VE;
    if constexpr (KIND == kReduceScatter && Words<Out, VE>::NW == 8) {
      // bf16 -> fp32: 1 KiB lane-contiguous stores (every lane takes part in the regrouping)
      const uint32_t lane = threadIdx.x & 63;
      const uint64_t vw = v - lane;
      u32x4 h0, h1;
      wave_halves32<Out, VE>(w, h0, h1);
      char* base = a.out[j] + (a.phase + vw * VE - g.lo) * Out::ES;
      if (!GUARD || vw + (lane >> 1) < g.vhi) st16(base + 16 * lane, h0);
      if (!GUARD || vw + 32 + (lane >> 1) < g.vhi) st16(base + 1024 + 16 * lane, h1);
    } else if (!GUARD || v < g.vhi) {
      if constexpr (KIND == kAllReduce) {
        for (uint32_t q = 0; q < N; ++q) put<Out, VE>(a.out[q] + e0 * Out::ES, w);
      } else {
        put<Out, VE>(a.out[j] + (e0 - g.lo) * Out::ES, w);
      }
    }
  }
}

// Fused all-reduce (KIND == kAllReduce: fold N inputs, write N outputs) and
// reduce-scatter (KIND == kReduceScatter: fold N inputs, write the owner's).
// NF > 0 fixes N at compile time (N <= 8); NF == 0 reads it from the
// arguments and folds in batches of eight ranks.  WIRE rounds each forwarded
// partial to the input type (bf16 ring communicating in bf16).
template <int KIND, class In, class Out, int NF, int U, bool WIRE, int P>
__global__ void __launch_bounds__(kThreads) reduce_vec_kernel(const RedArgs<P> a) {
  constexpr int VE = In::VE;
  constexpr int TV = kThreads * U;
  typedef typename In::Acc Acc;
  const uint32_t N = NF ? NF : a.N;
  const bool avg = a.avg != 0;

  for (uint32_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const uint32_t j = tile / a.tpc;
    const uint32_t t = tile - j * a.tpc;
    const ChunkGeom g = chunk_geom<VE>(a, j);
    const uint32_t first = a.ring ? next_rank(j, N) : 0;
    const uint64_t tv0 = g.vlo + static_cast<uint64_t>(t) * TV;
    if (tv0 + TV <= g.vhi) {
      reduce_tile<KIND, In, Out, NF, U, false, WIRE>(a, N, j, first, g, tv0);
    } else if (tv0 < g.vhi) {
      reduce_tile<KIND, In, Out, NF, U, true, WIRE>(a, N, j, first, g, tv0);
    }

    if (t == 0) {
      // Elements of the chunk outside the aligned vectors: at most 2*VE - 2.
      const bool has_vec = g.vhi > g.vlo;
      const uint64_t head_end = has_vec ? a.phase + g.vlo * VE : g.hi;
      const uint64_t tail_beg = has_vec ? a.phase + g.vhi * VE : g.hi;
      const uint64_t nhead = head_end - g.lo;
      const uint64_t nscalar = nhead + (g.hi - tail_beg);
      if (threadIdx.x < nscalar) {
        const uint64_t E = threadIdx.x < nhead ? g.lo + threadIdx.x : tail_beg + (threadIdx.x - nhead);
        const Acc x = finish(fold_one<In, WIRE>(a.in, first, N, E), avg, a.nf);
        if constexpr (KIND == kAllReduce) {
          for (uint32_t q = 0; q < N; ++q) put_one<Out>(a.out[q], E, x);
        } else {
          put_one<Out>(a.out[j], E - g.lo, x);
        }
      }
    }
  }
}

// Element-wise variant for buffers whose relative alignment rules out vectors.
template <int KIND, class In, class Out, bool WIRE, int P>
__global__ void __launch_bounds__(kThreads) reduce_elem_kernel(const RedArgs<P> a) {
  constexpr int TE = kThreads * 4;
  const uint32_t N = a.N;
  const bool avg = a.avg != 0;
  for (uint32_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const uint32_t j = tile / a.tpc;
    const uint32_t t = tile - j * a.tpc;
    const uint64_t lo = min(a.S, static_cast<uint64_t>(j) * a.c);
    const uint64_t hi = min(a.S, lo + a.c);
    const uint32_t first = a.ring ? next_rank(j, N) : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t E = lo + static_cast<uint64_t>(t) * TE + u * kThreads + threadIdx.x;
      if (E < hi) {
        const typename In::Acc x = finish(fold_one<In, WIRE>(a.in, first, N, E), avg, a.nf);
        if constexpr (KIND == kAllReduce) {
          for (uint32_t r = 0; r < N; ++r) put_one<Out>(a.out[r], E, x);
        } else {
          put_one<Out>(a.out[j], E - lo, x);
        }
      }
    }
  }
}

// All-gather: shard j's element E is read once and written to every rank.
// Same full-tile / guarded-tile split as the reductions.
// The all-gather keeps the workgroup-strided layout: the wavefront-contiguous
// one measured equal (64-rank layer all-gather, 6.67 TB/s either way).
#ifndef GC_GATHER_WAVE_CONTIG
#define GC_GATHER_WAVE_CONTIG 0
#endif
constexpr bool kGatherWave = GC_GATHER_WAVE_CONTIG != 0;

template <int ES, int U, bool GUARD, int P>
__device__ __forceinline__ void gather_tile(const RedArgs<P>& a, uint32_t N, const char* src, const ChunkGeom& g,
                                            uint64_t tv0) {
  constexpr int VE = 16 / ES;
  u32x4 raw[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t v = GUARD ? min(gcdev::tile_vec<U, kGatherWave>(tv0, u), g.vhi - 1)
                             : gcdev::tile_vec<U, kGatherWave>(tv0, u);
    raw[u] = ld16(src + (a.phase + v * VE - g.lo) * ES);
  }
  for (uint32_t d = 0; d < N; ++d) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t v = gcdev::tile_vec<U, kGatherWave>(tv0, u);
      if (!GUARD || v < g.vhi) st16(a.out[d] + (a.phase + v * VE) * ES, raw[u]);
    }
  }
}

template <int ES, int U, int P>
__global__ void __launch_bounds__(kThreads) gather_vec_kernel(const RedArgs<P> a) {
  constexpr int VE = 16 / ES;
  constexpr int TV = kThreads * U;
  const uint32_t N = a.N;
  for (uint32_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const uint32_t j = tile / a.tpc;
    const uint32_t t = tile - j * a.tpc;
    const ChunkGeom g = chunk_geom<VE>(a, j);
    const uint64_t tv0 = g.vlo + static_cast<uint64_t>(t) * TV;
    const char* src = a.in[j];
    if (tv0 + TV <= g.vhi) {
      gather_tile<ES, U, false>(a, N, src, g, tv0);
    } else if (tv0 < g.vhi) {
      gather_tile<ES, U, true>(a, N, src, g, tv0);
    }
    if (t == 0) {
      const bool has_vec = g.vhi > g.vlo;
      const uint64_t head_end = has_vec ? a.phase + g.vlo * VE : g.hi;
      const uint64_t tail_beg = has_vec ? a.phase + g.vhi * VE : g.hi;
      const uint64_t nhead = head_end - g.lo;
      const uint64_t nscalar = nhead + (g.hi - tail_beg);
      if (threadIdx.x < nscalar) {
        const uint64_t E = threadIdx.x < nhead ? g.lo + threadIdx.x : tail_beg + (threadIdx.x - nhead);
        if constexpr (ES == 2) {
          const uint16_t x = reinterpret_cast<const uint16_t*>(src)[E - g.lo];
          for (uint32_t d = 0; d < N; ++d) reinterpret_cast<uint16_t*>(a.out[d])[E] = x;
        } else {
          const uint32_t x = reinterpret_cast<const uint32_t*>(src)[E - g.lo];
          for (uint32_t d = 0; d < N; ++d) reinterpret_cast<uint32_t*>(a.out[d])[E] = x;
        }
      }
    }
  }
}

template <int ES, int P>
__global__ void __launch_bounds__(kThreads) gather_elem_kernel(const RedArgs<P> a) {
  constexpr int TE = kThreads * 4;
  const uint32_t N = a.N;
  for (uint32_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const uint32_t j = tile / a.tpc;
    const uint32_t t = tile - j * a.tpc;
    const uint64_t lo = min(a.S, static_cast<uint64_t>(j) * a.c);
    const uint64_t hi = min(a.S, lo + a.c);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t E = lo + static_cast<uint64_t>(t) * TE + u * kThreads + threadIdx.x;
      if (E < hi) {
        if constexpr (ES == 2) {
          const uint16_t x = reinterpret_cast<const uint16_t*>(a.in[j])[E - lo];
          for (uint32_t d = 0; d < N; ++d) reinterpret_cast<uint16_t*>(a.out[d])[E] = x;
        } else {
          const uint32_t x = reinterpret_cast<const uint32_t*>(a.in[j])[E - lo];
          for (uint32_t d = 0; d < N; ++d) reinterpret_cast<uint32_t*>(a.out[d])[E] = x;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host side

#ifndef GC_RED_MAX_GRID
#define GC_RED_MAX_GRID (1u << 20)
#endif
#ifndef GC_RED_U
#define GC_RED_U 2
#endif

constexpr uint32_t kMaxGrid = GC_RED_MAX_GRID;

uint64_t addr(const void* p) { return reinterpret_cast<uint64_t>(p); }

template <int P>
RedArgs<P> make_args(const gci::ReduceCall& c) {
  RedArgs<P> a{};
  for (int i = 0; i < c.nranks; ++i) {
    a.in[i] = static_cast<const char*>(c.in[i]);
    a.out[i] = static_cast<char*>(c.out[i]);
  }
  a.S = c.S;
  a.c = c.c;
  a.N = static_cast<uint32_t>(c.nranks);
  a.ring = c.ring ? 1u : 0u;
  a.avg = c.avg ? 1u : 0u;
  a.nf = static_cast<float>(c.nranks);
  return a;
}

template <class K, class A>
gc_status launch(K kernel, const A& args, uint32_t ntiles, hipStream_t stream) {
  const uint32_t grid = std::max(1u, std::min(ntiles, kMaxGrid));
  void* params[] = {const_cast<A*>(&args)};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(kThreads),
                                       params, 0, stream);
  return gci::hip_status(e);
}

// Phase (in elements) that puts every pointer in `ptrs` on a 16-byte boundary,
// or -1 if no common phase exists.
int common_phase(const void* const* ptrs, int n, size_t es) {
  const uint64_t mis = addr(ptrs[0]) & 15;
  for (int i = 1; i < n; ++i)
    if ((addr(ptrs[i]) & 15) != mis) return -1;
  if (mis % es) return -1;
  return static_cast<int>(((16 - mis) & 15) / es);
}

struct Plan {
  bool vec;
  uint32_t phase;
  uint32_t tpc;
};

// Tiles per chunk: enough for the chunk with the most aligned vectors (or
// elements, when vectors are ruled out).  Never 0: tile 0 of every chunk also
// owns the chunk's unaligned edges.
uint32_t tiles_per_chunk(const gci::ReduceCall& c, int VE, int TV, bool vec, uint32_t phase) {
  if (!vec) return static_cast<uint32_t>(std::max<uint64_t>(1, (c.c + kThreads * 4 - 1) / (kThreads * 4)));
  uint64_t most = 0;
  for (int j = 0; j < c.nranks; ++j) {
    const uint64_t lo = std::min<uint64_t>(c.S, static_cast<uint64_t>(j) * c.c);
    const uint64_t hi = std::min<uint64_t>(c.S, lo + c.c);
    const uint64_t vlo = lo <= phase ? 0 : (lo - phase + VE - 1) / VE;
    const uint64_t vhi = hi < phase + static_cast<uint64_t>(VE) ? 0 : (hi - phase) / VE;
    if (vhi > vlo) most = std::max(most, vhi - vlo);
  }
  return static_cast<uint32_t>(std::max<uint64_t>(1, (most + TV - 1) / TV));
}

template <int KIND, class In, class Out, int U, bool WIRE>
gc_status dispatch_reduce(const gci::ReduceCall& c, const Plan& pl) {
  const int N = c.nranks;
  const uint32_t ntiles = static_cast<uint32_t>(N) * pl.tpc;
  if (N <= 8) {
    RedArgs<8> a = make_args<8>(c);
    a.phase = pl.phase;
    a.tpc = pl.tpc;
    a.ntiles = ntiles;
    if (!pl.vec) return launch(reduce_elem_kernel<KIND, In, Out, WIRE, 8>, a, ntiles, c.stream);
    switch (N) {
      case 2: return launch(reduce_vec_kernel<KIND, In, Out, 2, U, WIRE, 8>, a, ntiles, c.stream);
      case 4: return launch(reduce_vec_kernel<KIND, In, Out, 4, U, WIRE, 8>, a, ntiles, c.stream);
      case 8: return launch(reduce_vec_kernel<KIND, In, Out, 8, U, WIRE, 8>, a, ntiles, c.stream);
      default: return launch(reduce_vec_kernel<KIND, In, Out, 0, U, WIRE, 8>, a, ntiles, c.stream);
    }
  }
  RedArgs<GC_MAX_RANKS> a = make_args<GC_MAX_RANKS>(c);
  a.phase = pl.phase;
  a.tpc = pl.tpc;
  a.ntiles = ntiles;
  if (!pl.vec) return launch(reduce_elem_kernel<KIND, In, Out, WIRE, GC_MAX_RANKS>, a, ntiles, c.stream);
  return launch(reduce_vec_kernel<KIND, In, Out, 0, U, WIRE, GC_MAX_RANKS>, a, ntiles, c.stream);
}

// The wire-rounding kernels exist for bf16 inputs only; for the other types
// the rounding is an identity and the plain ring kernels run.
template <int KIND, class In, class Out, int U>
gc_status dispatch_wire(const gci::ReduceCall& c, const Plan& pl) {
  if constexpr (In::ES == 2) {
    if (c.wire) return dispatch_reduce<KIND, In, Out, U, true>(c, pl);
  }
  return dispatch_reduce<KIND, In, Out, U, false>(c, pl);
}

constexpr int kU = GC_RED_U;
// Below this many tiles (with U vectors per thread) launches use one vector per
// thread, doubling the workgroup count.  Measured per operation on MI355X
// (same buffers, one process): at 512 tiles the fused all-reduce is faster
// with U (4 x 1M fp32: 6.97 vs 7.65 us; 8 x 2M bf16: 11.9 vs 14.6 us), the
// reduce-scatter (4 x 1M fp32: 5.23 vs 5.81 us) and the all-gather (64 ranks:
// 47.9 vs 50.7 us) with one vector; below 256 tiles one vector wins for all.
constexpr uint64_t kSmallTilesAR = 512;
constexpr uint64_t kSmallTiles = 1024;

template <int KIND, class In, class Out>
gc_status run_reduce(const gci::ReduceCall& c) {
  constexpr int VE = In::VE;
  const int N = c.nranks;
  // Inputs: one common phase across all N buffers.
  const int ph = common_phase(c.in, N, In::ES);
  bool vec = ph >= 0;
  if (vec && KIND == kAllReduce) {
    // Outputs are addressed with the same element index as the inputs.
    for (int r = 0; r < N && vec; ++r)
      if (((addr(c.out[r]) + static_cast<uint64_t>(ph) * Out::ES) & 15) != 0) vec = false;
  }
  if (vec && KIND == kReduceScatter) {
    // Output j receives element E at out[j] + (E - lo_j): its first aligned
    // vector must land on a boundary of the output vector width.
    const uint64_t wb = std::min<uint64_t>(16, Out::vec_bytes(VE));
    for (int j = 0; j < N && vec; ++j) {
      const uint64_t lo = std::min<uint64_t>(c.S, static_cast<uint64_t>(j) * c.c);
      if (lo == std::min<uint64_t>(c.S, lo + c.c)) continue;  // empty chunk: its output is never touched
      const uint64_t vlo = lo <= static_cast<uint64_t>(ph) ? 0 : (lo - ph + VE - 1) / VE;
      const uint64_t first = ph + vlo * VE;
      if (((addr(c.out[j]) + (first - lo) * Out::ES) % wb) != 0) vec = false;
    }
  }
  const uint32_t phase = vec ? static_cast<uint32_t>(ph) : 0u;
  Plan pl{vec, phase, tiles_per_chunk(c, VE, kThreads * kU, vec, phase)};
  // Small messages: with too few workgroups to cover every CU several times,
  // one vector per thread doubles the workgroup count.
  const uint64_t small = KIND == kAllReduce ? kSmallTilesAR : kSmallTiles;
  if (vec && kU > 1 && static_cast<uint64_t>(pl.tpc) * N < small) {
    pl.tpc = tiles_per_chunk(c, VE, kThreads, vec, phase);
    return dispatch_wire<KIND, In, Out, 1>(c, pl);
  }
  return dispatch_wire<KIND, In, Out, kU>(c, pl);
}

template <int KIND>
gc_status run_typed(const gci::ReduceCall& c) {
  if (c.in_t == GC_BF16 && c.out_t == GC_BF16) return run_reduce<KIND, InBf16, OutBf16>(c);
  if (c.in_t == GC_FP32 && c.out_t == GC_FP32) return run_reduce<KIND, InF32, OutF32>(c);
  if (c.in_t == GC_INT32 && c.out_t == GC_INT32) return run_reduce<KIND, InI32, OutI32>(c);
  if (KIND == kReduceScatter) {
    if (c.in_t == GC_BF16 && c.out_t == GC_FP32) return run_reduce<KIND, InBf16, OutF32>(c);
    if (c.in_t == GC_FP32 && c.out_t == GC_BF16) return run_reduce<KIND, InF32, OutBf16>(c);
  }
  return GC_ERR_UNSUPPORTED;
}

template <int ES>
gc_status run_gather(const gci::ReduceCall& c) {
  constexpr int VE = 16 / ES;
  const int N = c.nranks;
  const int ph = common_phase(c.out, N, ES);
  bool vec = ph >= 0;
  for (int j = 0; j < N && vec; ++j) {
    const uint64_t lo = std::min<uint64_t>(c.S, static_cast<uint64_t>(j) * c.c);
    if (lo == std::min<uint64_t>(c.S, lo + c.c)) continue;  // empty shard: never read
    const uint64_t vlo = lo <= static_cast<uint64_t>(ph) ? 0 : (lo - ph + VE - 1) / VE;
    const uint64_t first = ph + vlo * VE;
    if (((addr(c.in[j]) + (first - lo) * ES) & 15) != 0) vec = false;
  }
  uint32_t tpc = tiles_per_chunk(c, VE, kThreads * kU, vec, vec ? static_cast<uint32_t>(ph) : 0u);
  const bool small = vec && kU > 1 && static_cast<uint64_t>(tpc) * N < kSmallTiles;
  if (small) tpc = tiles_per_chunk(c, VE, kThreads, vec, static_cast<uint32_t>(ph));
  const uint32_t ntiles = static_cast<uint32_t>(N) * tpc;
  auto fill = [&](auto& a) {
    a.phase = vec ? static_cast<uint32_t>(ph) : 0u;
    a.tpc = tpc;
    a.ntiles = ntiles;
  };
  if (N <= 8) {
    RedArgs<8> a = make_args<8>(c);
    fill(a);
    if (small) return launch(gather_vec_kernel<ES, 1, 8>, a, ntiles, c.stream);
    return vec ? launch(gather_vec_kernel<ES, kU, 8>, a, ntiles, c.stream)
               : launch(gather_elem_kernel<ES, 8>, a, ntiles, c.stream);
  }
  RedArgs<GC_MAX_RANKS> a = make_args<GC_MAX_RANKS>(c);
  fill(a);
  if (small) return launch(gather_vec_kernel<ES, 1, GC_MAX_RANKS>, a, ntiles, c.stream);
  return vec ? launch(gather_vec_kernel<ES, kU, GC_MAX_RANKS>, a, ntiles, c.stream)
             : launch(gather_elem_kernel<ES, GC_MAX_RANKS>, a, ntiles, c.stream);
}

}  // namespace

namespace gci {

gc_status launch_all_reduce(const ReduceCall& c) { return run_typed<kAllReduce>(c); }

gc_status launch_reduce_scatter(const ReduceCall& c) { return run_typed<kReduceScatter>(c); }

gc_status launch_all_gather(const ReduceCall& c) {
  return elem_bytes(c.in_t) == 2 ? run_gather<2>(c) : run_gather<4>(c);
}

}  // namespace gci
