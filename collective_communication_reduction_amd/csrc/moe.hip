// Expert-parallel MoE data flow around the all-to-all, for gfx950 (DTLM §8
// "专家并行和 MoE 通信": router top-k, pack by target expert / rank, dispatch,
// local experts, combine back, restore token order).
//
//   route     the routing plan, on the device: from each source's top-k expert
//             ids to the split table and, per (token, k), the rank and row its
//             copy occupies in the receive layout (by local expert, then
//             source, then token).  Three small kernels: a stable in-tile rank
//             per route (lanes matched by expert with one ballot per id bit),
//             a per-destination scan of the tile totals, and the final rows
//             (each tile adds the counts of the source's earlier tiles).
//   dispatch  the pack fused into the all-to-all: each token row is read once
//             and written to its K destinations (an HBM stream, no arithmetic).
//   combine   the inverse all-to-all fused with the weighted un-permute: each
//             output row gathers its K expert rows, sums w_k * y_k in fp32
//             (k = 0 first, every product rounded to fp32), rounds once.
//
// Route entries whose rank or row falls outside the destination buffers are
// skipped by dispatch and combine, so malformed plans cannot fault.

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "fold.h"
#include "gc_internal.h"

namespace {

using namespace gcdev;

// ------------------------------------------------------------ routing plan

constexpr int kWave = 64;

template <int P>
struct RouteArgs {
  const int32_t* experts[P];  // [routes_s] global expert ids, token-major (t * K + k)
  int2* dest[P];              // [routes_s] (rank, row); (expert, in-tile rank) in between kernels
  int64_t routes[P];          // tokens_s * K
  int32_t tile0[P + 1];       // first tile of each source
  int32_t* counts;            // [tiles][nbins] per-tile counts, then exclusive prefixes over tiles
  int32_t* roff;              // [N][nbins] receive-row offset of block (s, expert)
  int64_t* splits;            // [N][N][E]
  int32_t tile;               // routes per tile
  int32_t N, E, nbins;
  int32_t nbits;              // bits of the largest expert id, nbins - 1
};

template <int P>
__device__ __forceinline__ int source_of(const int32_t (&first)[P + 1], int N, int32_t b) {
  int s = 0;
  while (s + 1 < N && first[s + 1] <= b) ++s;
  return s;
}

// Rank of each route of one 64-route chunk among the earlier routes to the
// same expert.  Each lane finds the lanes holding its expert with one ballot
// per bit of the expert id (nbits ballots, however many experts the chunk
// holds); its rank is the running count `cnt` (LDS) plus the matching lanes
// below it, and the lowest lane of each group advances the count.  Within a
// wavefront the LDS read completes before the write is issued.
__device__ __forceinline__ int32_t rank_in_chunk(int32_t g, bool valid, int32_t* cnt, int lane, int nbits) {
  const uint64_t below = (uint64_t(1) << lane) - 1;
  uint64_t same = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool set = (g >> bit) & 1;
    const uint64_t b = __ballot(set);
    same &= set ? b : ~b;
  }
  const int32_t base = cnt[valid ? g : 0];
  if (!valid) return -1;
  const uint64_t mine = same & below;
  if (mine == 0) cnt[g] = base + __popcll(same);
  return base + __popcll(mine);
}

// Tiles of kMoeRouteTile routes while the experts fit the tile: each of the
// four wavefronts ranks its share of the routes with the expert ids of all its
// chunks loaded up front, then the wavefronts' per-expert counts are scanned in LDS and each
// rank is offset by the counts of the wavefronts before it.  Writes (expert,
// rank in tile) per route and the tile's count per expert.
constexpr int kRouteWaves = 4;
constexpr int kRouteChunks = gci::kMoeRouteTile / (kRouteWaves * kWave);  // 64-route chunks per wavefront
static_assert(kRouteChunks * kRouteWaves * kWave == gci::kMoeRouteTile, "tile = whole chunks per wavefront");

template <int P>
__global__ void __launch_bounds__(kWave * kRouteWaves) route_count_kernel(const RouteArgs<P> a) {
  extern __shared__ int32_t cnt[];  // [kRouteWaves][nbins]
  const int32_t b = blockIdx.x;
  const int s = source_of<P>(a.tile0, a.N, b);
  const int64_t lo = static_cast<int64_t>(b - a.tile0[s]) * a.tile;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t wlo = lo + static_cast<int64_t>(w) * kWave * kRouteChunks;
  const int64_t n = max<int64_t>(0, min<int64_t>(kWave * kRouteChunks, a.routes[s] - wlo));
  for (int i = threadIdx.x; i < kRouteWaves * a.nbins; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  int32_t g[kRouteChunks], rank[kRouteChunks];
#pragma unroll
  for (int c = 0; c < kRouteChunks; ++c) {
    const int64_t i = c * kWave + lane;
    g[c] = i < n ? a.experts[s][wlo + i] : -1;
  }
#pragma unroll
  for (int c = 0; c < kRouteChunks; ++c) {
    const bool valid = g[c] >= 0 && g[c] < a.nbins;
    rank[c] = rank_in_chunk(g[c], valid, cnt + w * a.nbins, lane, a.nbits);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.nbins; e += blockDim.x) {
    int32_t run = 0;
    for (int q = 0; q < kRouteWaves; ++q) {
      const int32_t v = cnt[q * a.nbins + e];
      cnt[q * a.nbins + e] = run;
      run += v;
    }
    a.counts[static_cast<int64_t>(b) * a.nbins + e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kRouteChunks; ++c) {
    const int64_t i = c * kWave + lane;
    if (i >= n) continue;
    const bool valid = g[c] >= 0 && g[c] < a.nbins;
    const int32_t before = cnt[w * a.nbins + (valid ? g[c] : 0)];  // routes of earlier wavefronts
    a.dest[s][wlo + i] = valid ? make_int2(g[c], rank[c] + before) : make_int2(-1, -1);
  }
}

// More experts than kMoeRouteTile: one wavefront per tile of a.tile routes
// (at least one route per expert), chunk by chunk.
template <int P>
__global__ void __launch_bounds__(kWave) route_count_wide_kernel(const RouteArgs<P> a) {
  extern __shared__ int32_t cnt[];
  const int32_t b = blockIdx.x;
  const int s = source_of<P>(a.tile0, a.N, b);
  const int64_t lo = static_cast<int64_t>(b - a.tile0[s]) * a.tile;
  const int64_t n = min<int64_t>(a.tile, a.routes[s] - lo);
  const int lane = threadIdx.x;
  for (int i = lane; i < a.nbins; i += kWave) cnt[i] = 0;
  __syncthreads();
  for (int64_t c0 = 0; c0 < n; c0 += kWave) {
    const int64_t i = c0 + lane;
    const bool in = i < n;
    const int32_t g = in ? a.experts[s][lo + i] : -1;
    const bool valid = in && g >= 0 && g < a.nbins;
    const int32_t rank = rank_in_chunk(g, valid, cnt, lane, a.nbits);
    if (in) a.dest[s][lo + i] = valid ? make_int2(g, rank) : make_int2(-1, -1);
  }
  __syncthreads();
  for (int i = lane; i < a.nbins; i += kWave) a.counts[static_cast<int64_t>(b) * a.nbins + i] = cnt[i];
}

// Exclusive scan of one value per thread over a workgroup of kThreads.
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* lds, int32_t& total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  int32_t x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) lds[wid] = x;
  __syncthreads();
  int32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) {
    const int32_t t = lds[w];
    off += w < wid ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + x - v;
}

// Sum of counts[t][g] over tiles [t0, t1): independent loads, eight in flight.
__device__ __forceinline__ int32_t sum_tiles(const int32_t* counts, int32_t nbins, int32_t g, int32_t t0, int32_t t1) {
  int32_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int32_t t = t0;
  for (; t + 8 <= t1; t += 8) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += counts[static_cast<int64_t>(t + k) * nbins + g];
  }
  for (; t < t1; ++t) acc[0] += counts[static_cast<int64_t>(t) * nbins + g];  // integer sums: any order
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

// One workgroup per destination d: each (source, local expert) block's total
// over the tiles is its split; the receive offsets follow by scanning the
// blocks in (expert, source) order.
template <int P>
__global__ void __launch_bounds__(kThreads) route_scan_kernel(const RouteArgs<P> a) {
  __shared__ int32_t lds[kThreads / kWave];
  const int d = blockIdx.x;
  const int items = a.E * a.N;
  int32_t carry = 0;
  for (int base = 0; base < items; base += kThreads) {
    const int i = base + threadIdx.x;
    int32_t total = 0;
    int s = 0, g = 0;
    if (i < items) {
      const int e = i / a.N;
      s = i - e * a.N;
      g = d * a.E + e;
      total = sum_tiles(a.counts, a.nbins, g, a.tile0[s], a.tile0[s + 1]);
      a.splits[(static_cast<int64_t>(s) * a.N + d) * a.E + e] = total;
    }
    int32_t sum;
    const int32_t excl = block_exclusive_scan(total, lds, sum);
    if (i < items) a.roff[static_cast<int64_t>(s) * a.nbins + g] = carry + excl;
    carry += sum;
  }
}

// One workgroup per tile: the first receive row of each expert's routes in
// this tile (block offset plus the counts of the source's earlier tiles),
// then row = that + rank in tile, rank = expert / E.
template <int P>
__global__ void __launch_bounds__(kThreads) route_final_kernel(const RouteArgs<P> a) {
  extern __shared__ int32_t first_row[];  // [nbins]
  const int32_t b = blockIdx.x;
  const int s = source_of<P>(a.tile0, a.N, b);
  for (int g = threadIdx.x; g < a.nbins; g += kThreads)
    first_row[g] = a.roff[static_cast<int64_t>(s) * a.nbins + g] + sum_tiles(a.counts, a.nbins, g, a.tile0[s], b);
  __syncthreads();
  const int64_t lo = static_cast<int64_t>(b - a.tile0[s]) * a.tile;
  const int64_t n = min<int64_t>(a.tile, a.routes[s] - lo);
  for (int64_t i = threadIdx.x; i < n; i += kThreads) {
    const int2 p = a.dest[s][lo + i];
    if (p.x < 0) continue;
    a.dest[s][lo + i] = make_int2(p.x / a.E, first_row[p.x] + p.y);
  }
}

// ------------------------------------------------------- dispatch / combine
//
// Rows are cut into units (a 16-byte vector, or one element / byte when the
// rows or buffers are not 16-byte aligned).  S = 2^lanes_log2 lanes work on a
// row, kMoeU units per lane per step (all loads of a step issued before the
// first store); a workgroup holds kThreads / S rows.
//
// Dispatch with WROW (S >= 64): every wavefront lies inside one row, so a
// route's (rank, row) entry is the same on all of its lanes.  It is moved to
// scalar registers, and the destination's base pointer and row count then
// come from the kernel arguments by scalar loads: one vector round trip per
// batch of routes instead of three dependent ones per route.

#ifndef GC_MOE_UNITS
#define GC_MOE_UNITS 4
#endif
constexpr int kMoeU = GC_MOE_UNITS;

template <int P>
struct DispatchArgs {
  const char* tok[P];      // [tokens_s][R units]
  const int2* dest[P];     // [tokens_s * K] (rank, row)
  char* recv[P];           // [recv_rows_d][R units]
  int64_t recv_rows[P];
  int64_t ntok[P];
  int32_t grp0[P + 1];     // first row group of each source
  uint64_t R;              // units per row
  int32_t N, K, lanes_log2;
  int32_t cb;              // column blocks per row (workgroups sharing one row)
};

template <class T>
__device__ __forceinline__ T ld_unit(const T* p) {
  if constexpr (sizeof(T) == 16) return ld16(p);
  else return __builtin_nontemporal_load(p);
}
template <int POL = gci::kStoreNT, class T>
__device__ __forceinline__ void st_unit(T* p, T v) {
  if constexpr (sizeof(T) == 16) st16p<POL>(p, v);
  else __builtin_nontemporal_store(v, p);
}

// Cache policy of the combine's 16-byte output stores: device scope measured
// 514.5 against 517.8 us for the 8-rank top-2 combine (the dispatch, which
// writes K rows per row read, was equal with it, or slower without the
// non-temporal hint).
#ifndef GC_COMBINE_STORE
#define GC_COMBINE_STORE gci::kStoreDevNT
#endif

// A route's (rank, row) entry as a unit pointer into its destination, or
// nullptr when the entry lies outside the destination buffers.  Branch-free:
// the rank index is clamped so that the base pointer and row count are always
// loaded (in bounds) and the loads of several routes issue together.  With
// WROW the entry is first made wavefront-uniform, so both are scalar loads.
template <class T, bool WROW, int P>
__device__ __forceinline__ T* route_row(char* const (&buf)[P], const int64_t (&rows)[P], int N, int2 p,
                                        uint64_t R) {
  if constexpr (WROW) p = make_int2(__builtin_amdgcn_readfirstlane(p.x), __builtin_amdgcn_readfirstlane(p.y));
  const int q = min(max(p.x, 0), N - 1);
  const int64_t nrows = rows[q];
  char* const base = buf[q];
  const bool ok = p.x >= 0 && p.x < N && p.y >= 0 && p.y < nrows;
  return ok ? reinterpret_cast<T*>(base) + static_cast<uint64_t>(p.y) * R : nullptr;
}

// Routes resolved per batch: all K at once when K is known at compile time, else four.
template <int KT>
constexpr int route_batch() { return KT > 0 ? KT : 4; }

// KT > 0: K == KT known at compile time.  The K destinations of a step are
// resolved together, after its loads are issued and before any store, so no
// route waits on the previous route's stores.
template <class T, int KT, bool WROW, int P>
__global__ void __launch_bounds__(kThreads) dispatch_kernel(const DispatchArgs<P> a) {
  constexpr int KB = route_batch<KT>();
  const int K = KT > 0 ? KT : a.K;
  const int S = 1 << a.lanes_log2;
  const int sub = threadIdx.x >> a.lanes_log2, lane = threadIdx.x & (S - 1);
  const int G = kThreads >> a.lanes_log2;
  const int32_t ngroups = a.grp0[a.N];
  const uint64_t span = static_cast<uint64_t>(kMoeU) * S;  // units a row group covers per step
  for (int32_t b = blockIdx.x; b < ngroups; b += gridDim.x) {
    const int s = source_of<P>(a.grp0, a.N, b);
    const int32_t local = b - a.grp0[s];
    const int64_t t = static_cast<int64_t>(local / a.cb) * G + sub;
    if (t >= a.ntok[s]) continue;
    const uint64_t cbeg = static_cast<uint64_t>(local % a.cb) * span;
    const uint64_t cend = a.cb > 1 ? min(a.R, cbeg + span) : a.R;
    const T* src = reinterpret_cast<const T*>(a.tok[s]) + static_cast<uint64_t>(t) * a.R;
    const int2* dst = a.dest[s] + t * K;
    for (uint64_t c = cbeg + lane; c < cend; c += span) {
      T v[kMoeU];
#pragma unroll
      for (int j = 0; j < kMoeU; ++j) {
        const uint64_t cj = c + static_cast<uint64_t>(j) * S;
        v[j] = ld_unit(src + (cj < cend ? cj : c));  // clamped: no exec-masked load
      }
      for (int k0 = 0; k0 < K; k0 += KB) {
        int2 e[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i) e[i] = KT > 0 || k0 + i < K ? dst[k0 + i] : make_int2(-1, -1);
        T* out[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i) out[i] = route_row<T, WROW, P>(a.recv, a.recv_rows, a.N, e[i], a.R);
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          if (!out[i]) continue;
#pragma unroll
          for (int j = 0; j < kMoeU; ++j) {
            const uint64_t cj = c + static_cast<uint64_t>(j) * S;
            if (j == 0 || cj < cend) st_unit(out[i] + cj, v[j]);
          }
        }
      }
    }
  }
}

template <int P>
struct CombineArgs {
  char* y[P];              // expert outputs in the receive layout (read only)
  int64_t y_rows[P];
  const int2* dest[P];     // [tokens_s * K]
  const float* w[P];       // [tokens_s * K] gate weights
  char* out[P];            // [tokens_s][R units]
  int64_t ntok[P];
  int32_t grp0[P + 1];
  uint64_t R;
  int32_t N, K, lanes_log2;
  int32_t cb;
};

// One unit of K weighted rows: 16-byte vectors of In::VE elements, or single elements.
template <class In, bool VEC>
struct Unit;

template <class In>
struct Unit<In, true> {
  typedef u32x4 T;
  static constexpr int VE = In::VE;
  __device__ static __forceinline__ void widen(const T& v, float (&x)[VE]) { unpack<In>(v, x); }
  __device__ static __forceinline__ T narrow(const float (&x)[VE]) {
    const Words<typename std::conditional<In::ES == 2, OutBf16, OutF32>::type, VE> r =
        pack<typename std::conditional<In::ES == 2, OutBf16, OutF32>::type, VE>(x);
    return u32x4{r.w[0], r.w[1], r.w[2], r.w[3]};
  }
};

template <>
struct Unit<InBf16, false> {
  typedef uint16_t T;
  static constexpr int VE = 1;
  __device__ static __forceinline__ void widen(const T& v, float (&x)[1]) {
    x[0] = __uint_as_float(static_cast<uint32_t>(v) << 16);
  }
  __device__ static __forceinline__ T narrow(const float (&x)[1]) { return static_cast<T>(bf16_bits(x[0])); }
};

template <>
struct Unit<InF32, false> {
  typedef uint32_t T;
  static constexpr int VE = 1;
  __device__ static __forceinline__ void widen(const T& v, float (&x)[1]) { x[0] = __uint_as_float(v); }
  __device__ static __forceinline__ T narrow(const float (&x)[1]) { return __float_as_uint(x[0]); }
};

// acc = w * y (first valid route) or acc + w * y, each product rounded to fp32.
template <int VE>
__device__ __forceinline__ void accumulate(float (&acc)[VE], const float (&y)[VE], float w, bool first) {
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    const float p = w * y[e];
    acc[e] = first ? p : acc[e] + p;
  }
}

// KT > 0: K == KT known at compile time (all K loads of a step in flight at once).
// Routes are looked up per lane even when a wavefront lies in one row: the
// combine's row reads scatter over every expert block, and on MI355X issuing
// them sooner through the scalar lookup made it slower (529 vs 506 us for 8 x
// 16384 tokens x 8 KiB rows, top-2), unlike the dispatch.
template <class In, bool VEC, int KT, int P>
__global__ void __launch_bounds__(kThreads) combine_kernel(const CombineArgs<P> a) {
  typedef Unit<In, VEC> U;
  typedef typename U::T T;
  constexpr int VE = U::VE;
  constexpr int KB = KT > 0 ? KT : 1;  // routes held per batch
  const int K = KT > 0 ? KT : a.K;
  const int S = 1 << a.lanes_log2;
  const int sub = threadIdx.x >> a.lanes_log2, lane = threadIdx.x & (S - 1);
  const int G = kThreads >> a.lanes_log2;
  const int32_t ngroups = a.grp0[a.N];
  const uint64_t span = static_cast<uint64_t>(kMoeU) * S;
  for (int32_t b = blockIdx.x; b < ngroups; b += gridDim.x) {
    const int s = source_of<P>(a.grp0, a.N, b);
    const int32_t local = b - a.grp0[s];
    const int64_t t = static_cast<int64_t>(local / a.cb) * G + sub;
    if (t >= a.ntok[s]) continue;
    const uint64_t cbeg = static_cast<uint64_t>(local % a.cb) * span;
    const uint64_t cend = a.cb > 1 ? min(a.R, cbeg + span) : a.R;
    const int2* routes = a.dest[s] + t * K;
    const float* wt = a.w[s] + t * K;
    T* out = reinterpret_cast<T*>(a.out[s]) + static_cast<uint64_t>(t) * a.R;
    for (uint64_t c = cbeg + lane; c < cend; c += span) {
      uint64_t cu[kMoeU];
#pragma unroll
      for (int u = 0; u < kMoeU; ++u) {
        const uint64_t cj = c + static_cast<uint64_t>(u) * S;
        cu[u] = cj < cend ? cj : c;  // clamped: no exec-masked load
      }
      float acc[kMoeU][VE];
      bool any = false;
      for (int k0 = 0; k0 < K; k0 += KB) {
        T v[KB][kMoeU];
        bool ok[KB];
        float wk[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          const T* row = route_row<T, false, P>(a.y, a.y_rows, a.N, routes[k0 + j], a.R);
          ok[j] = row != nullptr;
          wk[j] = wt[k0 + j];
          if (ok[j]) {
#pragma unroll
            for (int u = 0; u < kMoeU; ++u) v[j][u] = ld_unit(row + cu[u]);
          }
        }
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          if (!ok[j]) continue;
#pragma unroll
          for (int u = 0; u < kMoeU; ++u) {
            float y[VE];
            U::widen(v[j][u], y);
            accumulate(acc[u], y, wk[j], !any);
          }
          any = true;
        }
      }
      if (!any) {
#pragma unroll
        for (int u = 0; u < kMoeU; ++u)
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[u][e] = 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kMoeU; ++u) {
        const uint64_t cj = c + static_cast<uint64_t>(u) * S;
        if (u == 0 || cj < cend) st_unit<GC_COMBINE_STORE>(out + cj, U::narrow(acc[u]));
      }
    }
  }
}

// ------------------------------------------------------------ host side

#ifndef GC_MOE_MAX_GRID
#define GC_MOE_MAX_GRID (1u << 20)
#endif

template <class Kern, class A>
gc_status launch(Kern kernel, const A& args, uint32_t grid, uint32_t threads, size_t lds, hipStream_t stream) {
  void* params[] = {const_cast<A*>(&args)};
  return gci::hip_status(hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(std::max(1u, grid)),
                                         dim3(threads), params, lds, stream));
}

uint64_t addr(const void* p) { return reinterpret_cast<uint64_t>(p); }

// Lanes per row: the row's units over kMoeU, rounded up to a power of two, 1..kThreads.
int lanes_log2_for(uint64_t R) {
  int l = 0;
  while (l < 8 && (uint64_t(1) << l) * kMoeU < R) ++l;
  return l;
}

// Column blocks per row: rows longer than one workgroup step are shared by
// several workgroups (each writes a few KiB per row), shorter ones are not.
#ifndef GC_MOE_SPLIT_ROWS
#define GC_MOE_SPLIT_ROWS 1
#endif
int32_t column_blocks(uint64_t R, int lanes_log2, const int64_t* tokens, int N) {
  const uint64_t span = static_cast<uint64_t>(kMoeU) << lanes_log2;
  if (!GC_MOE_SPLIT_ROWS || lanes_log2 < 8 || R <= span) return 1;
  const uint64_t cb = (R + span - 1) / span;
  uint64_t groups = 0;  // one row per group here (a full workgroup per row)
  for (int s = 0; s < N; ++s) groups += static_cast<uint64_t>(tokens[s]) * cb;
  return groups < (uint64_t(1) << 31) ? static_cast<int32_t>(cb) : 1;  // group indices are int32
}

template <int P>
void fill_groups(int32_t (&grp0)[P + 1], int64_t (&ntok)[P], const int64_t* tokens, int N, int G, int32_t cb) {
  int64_t run = 0;
  for (int s = 0; s < N; ++s) {
    grp0[s] = static_cast<int32_t>(run);
    ntok[s] = tokens[s];
    run += (tokens[s] + G - 1) / G * cb;
  }
  for (int s = N; s <= P; ++s) grp0[s] = static_cast<int32_t>(run);
}

template <int P>
gc_status route_impl(const gci::MoeRouteCall& c) {
  RouteArgs<P> a{};
  int32_t tiles = 0;
  for (int s = 0; s < c.nranks; ++s) {
    a.experts[s] = c.experts[s];
    a.dest[s] = reinterpret_cast<int2*>(c.dest[s]);
    a.routes[s] = c.routes[s];
    a.tile0[s] = tiles;
    tiles += static_cast<int32_t>((c.routes[s] + c.tile - 1) / c.tile);
  }
  for (int s = c.nranks; s <= P; ++s) a.tile0[s] = tiles;
  a.counts = c.counts;
  a.roff = c.roff;
  a.splits = c.splits;
  a.tile = c.tile;
  a.N = c.nranks;
  a.E = c.experts_per_rank;
  a.nbins = c.nranks * c.experts_per_rank;
  a.nbits = 0;
  while ((1 << a.nbits) < a.nbins) ++a.nbits;
  const size_t lds = static_cast<size_t>(a.nbins) * sizeof(int32_t);
  const bool wide = a.tile != kRouteWaves * kRouteChunks * kWave;
  if (tiles > 0) {
    const gc_status st = wide ? launch(route_count_wide_kernel<P>, a, tiles, kWave, lds, c.stream)
                              : launch(route_count_kernel<P>, a, tiles, kWave * kRouteWaves, kRouteWaves * lds,
                                       c.stream);
    if (st != GC_OK) return st;
  }
  gc_status st = launch(route_scan_kernel<P>, a, c.nranks, kThreads, 0, c.stream);
  if (st != GC_OK || tiles == 0) return st;
  return launch(route_final_kernel<P>, a, tiles, kThreads, lds, c.stream);
}

template <class T, bool WROW, int P>
gc_status launch_dispatch(const DispatchArgs<P>& a, int topk, uint32_t grid, hipStream_t stream) {
  switch (topk) {
    case 1: return launch(dispatch_kernel<T, 1, WROW, P>, a, grid, kThreads, 0, stream);
    case 2: return launch(dispatch_kernel<T, 2, WROW, P>, a, grid, kThreads, 0, stream);
    default: return launch(dispatch_kernel<T, 0, WROW, P>, a, grid, kThreads, 0, stream);
  }
}

template <class T, int P>
gc_status dispatch_impl(const gci::MoeMoveCall& c, uint64_t R) {
  DispatchArgs<P> a{};
  for (int s = 0; s < c.nranks; ++s) {
    a.tok[s] = static_cast<const char*>(c.src[s]);
    a.dest[s] = reinterpret_cast<const int2*>(c.dest[s]);
    a.recv[s] = static_cast<char*>(c.dst[s]);
    a.recv_rows[s] = c.dst_rows[s];
  }
  a.R = R;
  a.N = c.nranks;
  a.K = c.topk;
  a.lanes_log2 = lanes_log2_for(R);
  a.cb = column_blocks(R, a.lanes_log2, c.tokens, c.nranks);
  fill_groups<P>(a.grp0, a.ntok, c.tokens, c.nranks, kThreads >> a.lanes_log2, a.cb);
  if (a.grp0[c.nranks] == 0) return GC_OK;
  const uint32_t grid = std::min<uint32_t>(a.grp0[c.nranks], GC_MOE_MAX_GRID);
  if (a.lanes_log2 >= 6) return launch_dispatch<T, true, P>(a, c.topk, grid, c.stream);
  return launch_dispatch<T, false, P>(a, c.topk, grid, c.stream);
}

template <class In, bool VEC, int P>
gc_status launch_combine(const CombineArgs<P>& a, int topk, uint32_t grid, hipStream_t stream) {
  switch (topk) {
    case 1: return launch(combine_kernel<In, VEC, 1, P>, a, grid, kThreads, 0, stream);
    case 2: return launch(combine_kernel<In, VEC, 2, P>, a, grid, kThreads, 0, stream);
    default: return launch(combine_kernel<In, VEC, 0, P>, a, grid, kThreads, 0, stream);
  }
}

template <class In, bool VEC, int P>
gc_status combine_impl(const gci::MoeMoveCall& c, uint64_t R) {
  CombineArgs<P> a{};
  for (int s = 0; s < c.nranks; ++s) {
    a.y[s] = static_cast<char*>(const_cast<void*>(c.src[s]));
    a.y_rows[s] = c.src_rows[s];
    a.dest[s] = reinterpret_cast<const int2*>(c.dest[s]);
    a.w[s] = c.weights[s];
    a.out[s] = static_cast<char*>(c.dst[s]);
  }
  a.R = R;
  a.N = c.nranks;
  a.K = c.topk;
  a.lanes_log2 = lanes_log2_for(R);
  a.cb = column_blocks(R, a.lanes_log2, c.tokens, c.nranks);
  fill_groups<P>(a.grp0, a.ntok, c.tokens, c.nranks, kThreads >> a.lanes_log2, a.cb);
  if (a.grp0[c.nranks] == 0) return GC_OK;
  const uint32_t grid = std::min<uint32_t>(a.grp0[c.nranks], GC_MOE_MAX_GRID);
  return launch_combine<In, VEC, P>(a, c.topk, grid, c.stream);
}

template <int P>
gc_status dispatch_any(const gci::MoeMoveCall& c) {
  uint64_t m = c.row_bytes;
  for (int s = 0; s < c.nranks; ++s) m |= addr(c.src[s]) | addr(c.dst[s]);
  if ((m & 15) == 0) return dispatch_impl<u32x4, P>(c, c.row_bytes / 16);
  if ((m & 3) == 0) return dispatch_impl<uint32_t, P>(c, c.row_bytes / 4);
  if ((m & 1) == 0) return dispatch_impl<uint16_t, P>(c, c.row_bytes / 2);
  return dispatch_impl<uint8_t, P>(c, c.row_bytes);
}

template <int P>
gc_status combine_any(const gci::MoeMoveCall& c) {
  uint64_t m = c.row_bytes;
  for (int s = 0; s < c.nranks; ++s) m |= addr(c.src[s]) | addr(c.dst[s]);
  const bool vec = (m & 15) == 0;
  if (c.t == GC_BF16)
    return vec ? combine_impl<InBf16, true, P>(c, c.row_bytes / 16) : combine_impl<InBf16, false, P>(c, c.row_bytes / 2);
  return vec ? combine_impl<InF32, true, P>(c, c.row_bytes / 16) : combine_impl<InF32, false, P>(c, c.row_bytes / 4);
}

}  // namespace

// Scratch of the routing plan for gc_moe_route_noalloc: one copy per GPU the
// library runs on, held until the process ends.  Host code never uses the
// array's name as an address (on the host it names a stand-in, not device
// memory): the kernels get the per-device address hipGetSymbolAddress
// returns, looked up once per device with that device current.
static __device__ __align__(256) char scratch[GC_MOE_ROUTE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace gci {

gc_status moe_route_static_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return GC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return hip_status(e);
    if (!p || reinterpret_cast<uintptr_t>(p) % 256) return GC_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return GC_OK;
}

gc_status launch_moe_route(const MoeRouteCall& c) {
  return c.nranks <= 8 ? route_impl<8>(c) : route_impl<64>(c);
}

gc_status launch_moe_dispatch(const MoeMoveCall& c) {
  return c.nranks <= 8 ? dispatch_any<8>(c) : dispatch_any<64>(c);
}

gc_status launch_moe_combine(const MoeMoveCall& c) {
  return c.nranks <= 8 ? combine_any<8>(c) : combine_any<64>(c);
}

}  // namespace gci
