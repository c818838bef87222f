// Two-level (hierarchical) all-reduce and the HSDP gradient reduce-scatter
// for gfx950 (AIG6 Table 6-2: hierarchical all-reduce, two-level aggregation
// matching the topology; AIG6 §6.3.6: HSDP on nodes of 8 GPUs; DTLM §4: an
// HSDP mesh has a shard dimension and a replicate dimension).
//
// N = R * S ranks form R groups of S; rank g * S + i is member i of group g.
// Across GPUs the schedule is three rings: reduce-scatter inside each group
// (member i gets chunk i of its group's sum), all-reduce of chunk i across
// the R groups, all-gather inside each group.  On one GPU the three phases
// collapse into one pass that reads every input once and writes every output
// once, folding each element in exactly the order the schedule produces:
//
//   element E lies in chunk i = [i*c1, ...) of the S chunks and in piece h of
//   that chunk's R pieces; the groups are folded in ring order from h+1, each
//   group's S members in ring order from i+1 (GC_ORDER_RANK: 0, 1, ... at
//   both levels); fp32 partials throughout; one epilogue (avg divides by N).
//   With the bf16 wire (DTLM §11: low-precision communication, fp32
//   arithmetic) every partial is rounded to bf16 where the schedule sends it:
//   inside a group before the next member adds its term, across groups before
//   the next group adds its own (unrounded) partial.
//
// The grid walks cells (i, h); a tile holds U 16-byte vectors per thread of
// one cell, so both fold starts are wavefront-uniform; the rank pointers are
// read from an LDS copy with wavefront-uniform addresses.

#include <algorithm>

#include "fold.h"
#include "gc_internal.h"

namespace {

using namespace gcdev;

enum HierKind { kHierAllReduce = 0, kHsdpReduceScatter = 1 };

// Each wavefront reads a contiguous run of U KiB per rank (measured on MI355X,
// 16 x 64 MiB bf16 two-level all-reduce, one process: 6.31-6.34 against
// 6.28-6.30 TB/s for the workgroup-strided layout on the rank arena).
#ifndef GC_HIER_WAVE_CONTIG
#define GC_HIER_WAVE_CONTIG 1
#endif
constexpr bool kHierWave = GC_HIER_WAVE_CONTIG != 0;

template <int P>
struct HierArgs {
  const char* in[P];
  char* out[P];
  uint64_t count;   // elements per rank
  uint64_t c1;      // chunk length inside a group
  uint32_t S, R, N;
  uint32_t ring;
  uint32_t avg;
  uint32_t phase;   // elements before the first aligned vector
  uint32_t tpc;     // tiles per cell
  uint32_t ntiles;  // S * R * tpc
  float nf;
};

struct CellGeom {
  uint64_t clo;       // first element of the chunk (shard offset for the HSDP outputs)
  uint64_t lo, hi;    // element range of the cell
  uint64_t vlo, vhi;  // aligned vectors wholly inside the cell
};

template <int VE, int P>
__device__ __forceinline__ CellGeom cell_geom(const HierArgs<P>& a, uint32_t i, uint32_t h) {
  CellGeom g;
  g.clo = min(a.count, static_cast<uint64_t>(i) * a.c1);
  const uint64_t L = min(a.count, g.clo + a.c1) - g.clo;
  const uint64_t c2 = (L + a.R - 1) / a.R;
  g.lo = g.clo + min(L, static_cast<uint64_t>(h) * c2);
  g.hi = g.clo + min(L, static_cast<uint64_t>(h + 1) * c2);
  const uint64_t ph = a.phase;
  g.vlo = g.lo <= ph ? 0 : (g.lo - ph + VE - 1) / VE;
  g.vhi = g.hi < ph + VE ? 0 : (g.hi - ph) / VE;
  if (g.vhi < g.vlo) g.vhi = g.vlo;
  return g;
}

// Two-level fold of U vectors: groups from g0, members from m0 (mod R, S).
// `in` is the workgroup's LDS copy of the rank pointers: indexing the kernel
// arguments inside the runtime loop over groups made the compiler copy the
// whole argument block to scratch memory.
template <class In, int NS, int U, bool WIRE, int P>
__device__ __forceinline__ void fold2_vec(const HierArgs<P>& a, const char* const* in, uint32_t g0, uint32_t m0,
                                          const uint64_t (&off)[U], typename In::Acc (&acc)[U][In::VE]) {
  constexpr int VE = In::VE;
  typedef typename In::Acc Acc;
  const uint32_t S = NS ? NS : a.S;
  uint32_t g = g0;
  fold_vec<In, NS, U, WIRE>(in, m0, S, off, acc, g * S);
  for (uint32_t q = 1; q < a.R; ++q) {
    g = next_rank(g, a.R);
    Acc part[U][VE];
    fold_vec<In, NS, U, WIRE>(in, m0, S, off, part, g * S);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int l = 0; l < VE; ++l) acc[u][l] = on_wire<In, WIRE>(acc[u][l]) + part[u][l];
  }
}

template <class In, bool WIRE, int P>
__device__ __forceinline__ typename In::Acc fold2_one(const HierArgs<P>& a, const char* const* in, uint32_t g0,
                                                      uint32_t m0, uint64_t E) {
  uint32_t g = g0;
  typename In::Acc acc = fold_one<In, WIRE>(in, m0, a.S, E, g * a.S);
  for (uint32_t q = 1; q < a.R; ++q) {
    g = next_rank(g, a.R);
    acc = on_wire<In, WIRE>(acc) + fold_one<In, WIRE>(in, m0, a.S, E, g * a.S);
  }
  return acc;
}

// The rank pointers, copied once per workgroup into LDS.
template <int P>
__device__ __forceinline__ void load_rank_pointers(const HierArgs<P>& a, const char** s_in) {
  for (uint32_t r = threadIdx.x; r < a.N; r += kThreads) s_in[r] = a.in[r];
  __syncthreads();
}

template <int KIND, class In, class Out, int NS, int U, bool GUARD, bool WIRE, int P>
__device__ __forceinline__ void hier_tile(const HierArgs<P>& a, const char* const* in, uint32_t i, uint32_t g0,
                                          uint32_t m0, const CellGeom& c, uint64_t tv0) {
  constexpr int VE = In::VE;
  typedef typename In::Acc Acc;
  uint64_t off[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t v = GUARD ? min(tile_vec<U, kHierWave>(tv0, u), c.vhi - 1) : tile_vec<U, kHierWave>(tv0, u);
    off[u] = (a.phase + v * VE) * In::ES;
  }
  Acc acc[U][VE];
  fold2_vec<In, NS, U, WIRE>(a, in, g0, m0, off, acc);
  const bool avg = a.avg != 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t v = tile_vec<U, kHierWave>(tv0, u);
    Acc o[VE];
#pragma unroll
    for (int l = 0; l < VE; ++l) o[l] = finish(acc[u][l], avg, a.nf);
    const Words<Out, VE> w = pack<Out, VE>(o);
    const uint64_t e0 = a.phase + v * VE;
    if constexpr (KIND == kHsdpReduceScatter && Words<Out, VE>::NW == 8) {
      // bf16 -> fp32: 1 KiB lane-contiguous stores to every holder (all lanes take part)
      const uint32_t lane = threadIdx.x & 63;
      const uint64_t vw = v - lane;
      u32x4 h0, h1;
      wave_halves32<Out, VE>(w, h0, h1);
      const bool ok0 = !GUARD || vw + (lane >> 1) < c.vhi;
      const bool ok1 = !GUARD || vw + 32 + (lane >> 1) < c.vhi;
      const uint64_t off = (a.phase + vw * VE - c.clo) * Out::ES;
      for (uint32_t g = 0; g < a.R; ++g) {
        char* base = a.out[g * a.S + i] + off;
        if (ok0) st16(base + 16 * lane, h0);
        if (ok1) st16(base + 1024 + 16 * lane, h1);
      }
    } else if (!GUARD || v < c.vhi) {
      if constexpr (KIND == kHierAllReduce) {
        for (uint32_t q = 0; q < a.N; ++q) put<Out, VE>(a.out[q] + e0 * Out::ES, w);
      } else {
        for (uint32_t g = 0; g < a.R; ++g) put<Out, VE>(a.out[g * a.S + i] + (e0 - c.clo) * Out::ES, w);
      }
    }
  }
}

template <int KIND, class In, class Out, int NS, int U, bool WIRE, int P>
__global__ void __launch_bounds__(kThreads) hier_vec_kernel(const HierArgs<P> a) {
  constexpr int VE = In::VE;
  constexpr int TV = kThreads * U;
  typedef typename In::Acc Acc;
  __shared__ const char* s_in[P];
  load_rank_pointers(a, s_in);
  const bool avg = a.avg != 0;
  for (uint32_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const uint32_t cell = tile / a.tpc;
    const uint32_t t = tile - cell * a.tpc;
    const uint32_t i = cell / a.R;
    const uint32_t h = cell - i * a.R;
    const CellGeom c = cell_geom<VE>(a, i, h);
    const uint32_t g0 = a.ring ? next_rank(h, a.R) : 0;
    const uint32_t m0 = a.ring ? next_rank(i, a.S) : 0;
    const uint64_t tv0 = c.vlo + static_cast<uint64_t>(t) * TV;
    if (tv0 + TV <= c.vhi) {
      hier_tile<KIND, In, Out, NS, U, false, WIRE>(a, s_in, i, g0, m0, c, tv0);
    } else if (tv0 < c.vhi) {
      hier_tile<KIND, In, Out, NS, U, true, WIRE>(a, s_in, i, g0, m0, c, tv0);
    }
    if (t == 0) {
      // Elements of the cell outside its aligned vectors: at most 2*VE - 2.
      const bool has_vec = c.vhi > c.vlo;
      const uint64_t head_end = has_vec ? a.phase + c.vlo * VE : c.hi;
      const uint64_t tail_beg = has_vec ? a.phase + c.vhi * VE : c.hi;
      const uint64_t nhead = head_end - c.lo;
      const uint64_t nscalar = nhead + (c.hi - tail_beg);
      if (threadIdx.x < nscalar) {
        const uint64_t E = threadIdx.x < nhead ? c.lo + threadIdx.x : tail_beg + (threadIdx.x - nhead);
        const Acc x = finish(fold2_one<In, WIRE>(a, s_in, g0, m0, E), avg, a.nf);
        if constexpr (KIND == kHierAllReduce) {
          for (uint32_t q = 0; q < a.N; ++q) put_one<Out>(a.out[q], E, x);
        } else {
          for (uint32_t g = 0; g < a.R; ++g) put_one<Out>(a.out[g * a.S + i], E - c.clo, x);
        }
      }
    }
  }
}

// Element-wise variant for buffers whose relative alignment rules out vectors.
template <int KIND, class In, class Out, bool WIRE, int P>
__global__ void __launch_bounds__(kThreads) hier_elem_kernel(const HierArgs<P> a) {
  constexpr int TE = kThreads * 4;
  __shared__ const char* s_in[P];
  load_rank_pointers(a, s_in);
  const bool avg = a.avg != 0;
  for (uint32_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const uint32_t cell = tile / a.tpc;
    const uint32_t t = tile - cell * a.tpc;
    const uint32_t i = cell / a.R;
    const uint32_t h = cell - i * a.R;
    const CellGeom c = cell_geom<1>(a, i, h);
    const uint32_t g0 = a.ring ? next_rank(h, a.R) : 0;
    const uint32_t m0 = a.ring ? next_rank(i, a.S) : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t E = c.lo + static_cast<uint64_t>(t) * TE + u * kThreads + threadIdx.x;
      if (E < c.hi) {
        const typename In::Acc x = finish(fold2_one<In, WIRE>(a, s_in, g0, m0, E), avg, a.nf);
        if constexpr (KIND == kHierAllReduce) {
          for (uint32_t q = 0; q < a.N; ++q) put_one<Out>(a.out[q], E, x);
        } else {
          for (uint32_t g = 0; g < a.R; ++g) put_one<Out>(a.out[g * a.S + i], E - c.clo, x);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host side

#ifndef GC_HIER_MAX_GRID
#define GC_HIER_MAX_GRID (1u << 20)
#endif
#ifndef GC_HIER_U
#define GC_HIER_U 2
#endif

constexpr uint32_t kMaxGrid = GC_HIER_MAX_GRID;
constexpr int kU = GC_HIER_U;
constexpr uint64_t kSmallTiles = 1024;

uint64_t addr(const void* p) { return reinterpret_cast<uint64_t>(p); }

int common_phase(const void* const* ptrs, int n, size_t es) {
  const uint64_t mis = addr(ptrs[0]) & 15;
  for (int i = 1; i < n; ++i)
    if ((addr(ptrs[i]) & 15) != mis) return -1;
  if (mis % es) return -1;
  return static_cast<int>(((16 - mis) & 15) / es);
}

// Most aligned vectors (or elements) in any cell, for the tiles-per-cell count.
uint64_t most_in_cell(const gci::HierCall& c, int VE, uint32_t phase, bool vec) {
  const uint64_t c1 = (c.count + c.group - 1) / c.group;
  const int R = c.nranks / c.group;
  uint64_t most = 0;
  for (int i = 0; i < c.group; ++i) {
    const uint64_t clo = std::min<uint64_t>(c.count, static_cast<uint64_t>(i) * c1);
    const uint64_t L = std::min<uint64_t>(c.count, clo + c1) - clo;
    const uint64_t c2 = (L + R - 1) / R;
    for (int h = 0; h < R; ++h) {
      const uint64_t lo = clo + std::min<uint64_t>(L, h * c2), hi = clo + std::min<uint64_t>(L, (h + 1) * c2);
      if (!vec) {
        most = std::max(most, hi - lo);
        continue;
      }
      const uint64_t vlo = lo <= phase ? 0 : (lo - phase + VE - 1) / VE;
      const uint64_t vhi = hi < phase + static_cast<uint64_t>(VE) ? 0 : (hi - phase) / VE;
      if (vhi > vlo) most = std::max(most, vhi - vlo);
    }
  }
  return most;
}

template <class K, class A>
gc_status launch(K kernel, const A& args, uint32_t ntiles, hipStream_t stream) {
  const uint32_t grid = std::max(1u, std::min(ntiles, kMaxGrid));
  void* params[] = {const_cast<A*>(&args)};
  return gci::hip_status(hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(kThreads), params,
                                         0, stream));
}

template <int P>
HierArgs<P> make_args(const gci::HierCall& c) {
  HierArgs<P> a{};
  for (int r = 0; r < c.nranks; ++r) {
    a.in[r] = static_cast<const char*>(c.in[r]);
    a.out[r] = static_cast<char*>(c.out[r]);
  }
  a.count = c.count;
  a.c1 = (c.count + c.group - 1) / c.group;
  a.S = static_cast<uint32_t>(c.group);
  a.R = static_cast<uint32_t>(c.nranks / c.group);
  a.N = static_cast<uint32_t>(c.nranks);
  a.ring = c.ring ? 1u : 0u;
  a.avg = c.avg ? 1u : 0u;
  a.nf = static_cast<float>(c.nranks);
  return a;
}

template <int KIND, class In, class Out, int U, bool WIRE, int P>
gc_status run_p(const gci::HierCall& c, bool vec, uint32_t phase, uint32_t tpc) {
  HierArgs<P> a = make_args<P>(c);
  a.phase = phase;
  a.tpc = tpc;
  a.ntiles = static_cast<uint32_t>(c.nranks) * tpc;  // S * R cells
  if (!vec) return launch(hier_elem_kernel<KIND, In, Out, WIRE, P>, a, a.ntiles, c.stream);
  if (c.group == 8) return launch(hier_vec_kernel<KIND, In, Out, 8, U, WIRE, P>, a, a.ntiles, c.stream);
  if (c.group == 4) return launch(hier_vec_kernel<KIND, In, Out, 4, U, WIRE, P>, a, a.ntiles, c.stream);
  return launch(hier_vec_kernel<KIND, In, Out, 0, U, WIRE, P>, a, a.ntiles, c.stream);
}

// The wire-rounding kernels exist for bf16 inputs only; for the other types
// the rounding is an identity and the plain kernels run.
template <int KIND, class In, class Out, int U, int P>
gc_status run_w(const gci::HierCall& c, bool vec, uint32_t phase, uint32_t tpc) {
  if constexpr (In::ES == 2) {
    if (c.wire) return run_p<KIND, In, Out, U, true, P>(c, vec, phase, tpc);
  }
  return run_p<KIND, In, Out, U, false, P>(c, vec, phase, tpc);
}

template <int KIND, class In, class Out>
gc_status run(const gci::HierCall& c) {
  constexpr int VE = In::VE;
  const int N = c.nranks;
  const int ph = common_phase(c.in, N, In::ES);
  bool vec = ph >= 0;
  const uint64_t c1 = (c.count + c.group - 1) / c.group;
  if (vec && KIND == kHierAllReduce) {
    for (int r = 0; r < N && vec; ++r)
      if (((addr(c.out[r]) + static_cast<uint64_t>(ph) * Out::ES) & 15) != 0) vec = false;
  }
  if (vec && KIND == kHsdpReduceScatter) {
    // Output (g, i) receives element E at out + (E - lo_i): its first aligned
    // vector must land on a boundary of the output vector width.
    const uint64_t wb = std::min<uint64_t>(16, Out::vec_bytes(VE));
    for (int i = 0; i < c.group && vec; ++i) {
      const uint64_t lo = std::min<uint64_t>(c.count, static_cast<uint64_t>(i) * c1);
      if (lo == std::min<uint64_t>(c.count, lo + c1)) continue;
      const uint64_t vlo = lo <= static_cast<uint64_t>(ph) ? 0 : (lo - ph + VE - 1) / VE;
      const uint64_t first = ph + vlo * VE;
      for (int g = 0; g < N / c.group && vec; ++g)
        if (((addr(c.out[g * c.group + i]) + (first - lo) * Out::ES) % wb) != 0) vec = false;
    }
  }
  const uint32_t phase = vec ? static_cast<uint32_t>(ph) : 0u;
  const uint64_t most = most_in_cell(c, VE, phase, vec);
  const uint64_t per_tile = vec ? static_cast<uint64_t>(kThreads) * kU : kThreads * 4;
  uint32_t tpc = static_cast<uint32_t>(std::max<uint64_t>(1, (most + per_tile - 1) / per_tile));
  const bool small = vec && kU > 1 && static_cast<uint64_t>(tpc) * N < kSmallTiles;
  if (small) {
    tpc = static_cast<uint32_t>(std::max<uint64_t>(1, (most + kThreads - 1) / kThreads));
    return N <= 8 ? run_w<KIND, In, Out, 1, 8>(c, vec, phase, tpc)
                  : run_w<KIND, In, Out, 1, GC_MAX_RANKS>(c, vec, phase, tpc);
  }
  return N <= 8 ? run_w<KIND, In, Out, kU, 8>(c, vec, phase, tpc)
                : run_w<KIND, In, Out, kU, GC_MAX_RANKS>(c, vec, phase, tpc);
}

template <int KIND>
gc_status run_typed(const gci::HierCall& c) {
  if (c.in_t == GC_BF16 && c.out_t == GC_BF16) return run<KIND, InBf16, OutBf16>(c);
  if (c.in_t == GC_FP32 && c.out_t == GC_FP32) return run<KIND, InF32, OutF32>(c);
  if (c.in_t == GC_INT32 && c.out_t == GC_INT32) return run<KIND, InI32, OutI32>(c);
  if (KIND == kHsdpReduceScatter) {
    if (c.in_t == GC_BF16 && c.out_t == GC_FP32) return run<KIND, InBf16, OutF32>(c);
    if (c.in_t == GC_FP32 && c.out_t == GC_BF16) return run<KIND, InF32, OutBf16>(c);
  }
  return GC_ERR_UNSUPPORTED;
}

}  // namespace

namespace gci {

gc_status launch_hier_all_reduce(const HierCall& c) { return run_typed<kHierAllReduce>(c); }

gc_status launch_hsdp_reduce_scatter(const HierCall& c) { return run_typed<kHsdpReduceScatter>(c); }

}  // namespace gci
