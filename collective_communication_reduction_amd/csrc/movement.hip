// Pure data-movement kernels for gfx950: the segment copy behind DDP bucket
// pack / unpack (AIG6 §6.2.4 and NXMR §5.1 gradient buckets; DTLM §4 FSDP1
// FlatParameter layout) and the all-to-all(v) block permutation of MoE
// dispatch (DTLM §2 "All-to-All", DTLM §8 All-to-AllV).
//
// Both are HBM streams with no arithmetic.  Work is cut into equal-byte tiles
// across all segments or rows, so a launch that mixes one huge tensor with
// many tiny ones, or a skewed all-to-all where most rows go to one rank, still
// gives every workgroup the same number of bytes.

#include <algorithm>

#include "device_common.h"
#include "gc_internal.h"

namespace {

using namespace gcdev;

// ------------------------------------------------------------ segment copy

constexpr int kMaxSeg = 48;
constexpr int kSegU = 4;                          // 16-byte vectors per thread per tile
constexpr uint64_t kSegTileVec = kThreads * kSegU;

struct SegArgs {
  const char* src[kMaxSeg];  // nullptr: fill with zeros
  char* dst[kMaxSeg];
  uint64_t bytes[kMaxSeg];
  uint32_t tile0[kMaxSeg + 1];  // first tile of each segment; tile0[nseg] = total
  uint32_t nseg;
};

__device__ __forceinline__ uint32_t find_segment(const SegArgs& a, uint32_t tile) {
  uint32_t lo = 0, hi = a.nseg;  // last s with tile0[s] <= tile
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) / 2;
    if (a.tile0[mid] <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

// Segments whose source and destination agree modulo 16 bytes: byte head up
// to the first 16-byte boundary of the destination, 16-byte body, byte tail.
__global__ void __launch_bounds__(kThreads) segment_vec_kernel(const SegArgs a) {
  const uint32_t ntiles = a.tile0[a.nseg];
  for (uint32_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const uint32_t s = find_segment(a, tile);
    const uint32_t t = tile - a.tile0[s];
    const char* src = a.src[s];
    char* dst = a.dst[s];
    const uint64_t n = a.bytes[s];
    const uint64_t head = min<uint64_t>(n, (16 - (reinterpret_cast<uint64_t>(dst) & 15)) & 15);
    const uint64_t nvec = (n - head) / 16;
    const uint64_t tail_beg = head + nvec * 16;
    const uint64_t v0 = static_cast<uint64_t>(t) * kSegTileVec + threadIdx.x;
    if (static_cast<uint64_t>(t) * kSegTileVec < nvec) {
      // Lanes past the last vector reload it (no exec-masked loads) and skip the store.
      u32x4 buf[kSegU];
#pragma unroll
      for (int u = 0; u < kSegU; ++u) {
        const uint64_t v = min(v0 + u * kThreads, nvec - 1);
        buf[u] = src ? ld16(src + head + 16 * v) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kSegU; ++u) {
        const uint64_t v = v0 + u * kThreads;
        if (v < nvec) st16(dst + head + 16 * v, buf[u]);
      }
    }
    if (t == 0) {
      const uint64_t nedge = head + (n - tail_beg);  // < 32 bytes
      if (threadIdx.x < nedge) {
        const uint64_t b = threadIdx.x < head ? threadIdx.x : tail_beg + (threadIdx.x - head);
        dst[b] = src ? src[b] : 0;
      }
    }
  }
}

// Segments with mismatched alignment: W-byte elements (W divides both
// addresses and the length).
template <typename T>
__global__ void __launch_bounds__(kThreads) segment_narrow_kernel(const SegArgs a) {
  const uint32_t ntiles = a.tile0[a.nseg];
  constexpr uint64_t TE = kThreads * 8;
  for (uint32_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const uint32_t s = find_segment(a, tile);
    const uint32_t t = tile - a.tile0[s];
    const T* src = reinterpret_cast<const T*>(a.src[s]);
    T* dst = reinterpret_cast<T*>(a.dst[s]);
    const uint64_t n = a.bytes[s] / sizeof(T);
    if (static_cast<uint64_t>(t) * TE >= n) continue;
    T buf[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint64_t e = min(static_cast<uint64_t>(t) * TE + u * kThreads + threadIdx.x, n - 1);
      buf[u] = src ? src[e] : T(0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint64_t e = static_cast<uint64_t>(t) * TE + u * kThreads + threadIdx.x;
      if (e < n) dst[e] = buf[u];
    }
  }
}

// ------------------------------------------------------------ all-to-all

constexpr int kA2AMax = gci::kA2AMaxBlocks;
static_assert(2 * kThreads >= kA2AMax, "the block scans hold two entries per thread");

struct A2AArgs {
  const char* send[GC_MAX_RANKS];
  char* recv[GC_MAX_RANKS];
  uint64_t row_bytes;
  int32_t N, E, d0, Dg;
  uint32_t rows_per_tile;
  int32_t send_base[GC_MAX_RANKS];
  int32_t rows[kA2AMax];  // block (s, dl, e) at (s * Dg + dl) * E + e
};

// Exclusive prefix sums of up to 512 values held two per thread (elements 2t
// and 2t+1), across the workgroup.  Returns the prefix of element 2t; *total
// gets the sum of everything.  Uses wavefront shuffles and one LDS exchange.
__device__ int32_t scan_pairs(int32_t v0, int32_t v1, int32_t* s_wave, int32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int32_t x = v0 + v1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wave) before += s_wave[w];
    all += s_wave[w];
  }
  __syncthreads();
  *total = all;
  return before + x - (v0 + v1);
}

template <typename V>
__device__ __forceinline__ V ld_any(const char* p) {
  if constexpr (sizeof(V) == 16) return ld16(p);
  else return *reinterpret_cast<const V*>(p);
}
template <typename V>
__device__ __forceinline__ void st_any(char* p, V v) {
  if constexpr (sizeof(V) == 16) st16(p, v);
  else *reinterpret_cast<V*>(p) = v;
}

// Each workgroup first derives, in LDS, every block's first row in the
// launch's work order (source-major) and its source and destination row
// addresses; then it copies whole tiles of rows_per_tile rows, each lane
// resolving its row's block by binary search.
template <typename V, int UNR>
__global__ void __launch_bounds__(kThreads) a2a_kernel(const A2AArgs a) {
  __shared__ int32_t s_pre[kA2AMax + 1];   // work-order first row of each block
  __shared__ const char* s_src[kA2AMax];   // address of the block's first row in send[s]
  __shared__ char* s_dst[kA2AMax];         // address of the block's first row in recv[d]
  __shared__ int32_t s_rpre[kA2AMax];      // destination-order first row of each block
  __shared__ int32_t s_wave[kThreads / 64];

  const int nblk = a.N * a.Dg * a.E;
  const int t2 = 2 * threadIdx.x;

  // Work order (s, dl, e): prefix over rows.
  {
    const int32_t v0 = t2 < nblk ? a.rows[t2] : 0;
    const int32_t v1 = t2 + 1 < nblk ? a.rows[t2 + 1] : 0;
    int32_t total;
    const int32_t p = scan_pairs(v0, v1, s_wave, &total);
    if (t2 < nblk) s_pre[t2] = p;
    if (t2 + 1 < nblk) s_pre[t2 + 1] = p + v0;
    if (threadIdx.x == 0) s_pre[nblk] = total;
  }
  __syncthreads();
  // Source rows: blocks of source s are contiguous in send[s], starting at send_base[s].
  for (int b = threadIdx.x; b < nblk; b += kThreads) {
    const int s = b / (a.Dg * a.E);
    const int64_t row = a.send_base[s] + (s_pre[b] - s_pre[s * a.Dg * a.E]);
    s_src[b] = a.send[s] + row * static_cast<int64_t>(a.row_bytes);
  }
  // Destination rows: at rank d0+dl, blocks are laid out by (e, s).
  {
    const int NE = a.N * a.E;
    auto value = [&](int q) -> int32_t {  // q = (dl * E + e) * N + s
      if (q >= nblk) return 0;
      const int s = q % a.N;
      const int de = q / a.N;  // dl * E + e
      const int dl = de / a.E;
      const int e = de - dl * a.E;
      return a.rows[(s * a.Dg + dl) * a.E + e];
    };
    const int32_t v0 = value(t2), v1 = value(t2 + 1);
    int32_t total;
    const int32_t p = scan_pairs(v0, v1, s_wave, &total);
    // Each thread holds the prefixes of q = t2 and t2 + 1; the offset within
    // destination dl subtracts the prefix at q = dl * NE, which another thread
    // owns, so the exclusive prefixes go through LDS first.
    if (t2 < nblk) s_rpre[t2] = p;
    if (t2 + 1 < nblk) s_rpre[t2 + 1] = p + v0;
    __syncthreads();
    for (int q = threadIdx.x; q < nblk; q += kThreads) {
      const int s = q % a.N;
      const int de = q / a.N;
      const int dl = de / a.E;
      const int e = de - dl * a.E;
      const int64_t row = s_rpre[q] - s_rpre[dl * NE];
      s_dst[(s * a.Dg + dl) * a.E + e] = a.recv[a.d0 + dl] + row * static_cast<int64_t>(a.row_bytes);
    }
  }
  __syncthreads();

  const int64_t total_rows = s_pre[nblk];
  const uint64_t vpr = a.row_bytes / sizeof(V);
  const int64_t ntiles = (total_rows + a.rows_per_tile - 1) / a.rows_per_tile;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t row0 = tile * a.rows_per_tile;
    const int64_t row1 = min<int64_t>(total_rows, row0 + a.rows_per_tile);
    const uint64_t nv = static_cast<uint64_t>(row1 - row0) * vpr;
    for (uint64_t base = 0; base < nv; base += static_cast<uint64_t>(kThreads) * UNR) {
      V buf[UNR];
      char* dptr[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        // Lanes past the tile's end reload its last vector and skip the store.
        const uint64_t idx = min(base + u * kThreads + threadIdx.x, nv - 1);
        const int64_t row = row0 + static_cast<int64_t>(idx / vpr);
        const uint64_t col = idx - static_cast<uint64_t>(row - row0) * vpr;
        int lo = 0, hi = nblk;  // last block with s_pre[b] <= row (never an empty block)
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_pre[mid] <= row) lo = mid; else hi = mid;
        }
        const uint64_t off = static_cast<uint64_t>(row - s_pre[lo]) * a.row_bytes + col * sizeof(V);
        buf[u] = ld_any<V>(s_src[lo] + off);
        dptr[u] = s_dst[lo] + off;
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        if (base + u * kThreads + threadIdx.x < nv) st_any<V>(dptr[u], buf[u]);
    }
  }
}

// ------------------------------------------------------------ host side

#ifndef GC_SEG_MAX_GRID
#define GC_SEG_MAX_GRID (1u << 20)
#endif
#ifndef GC_A2A_MAX_GRID
#define GC_A2A_MAX_GRID (1u << 20)
#endif
#ifndef GC_A2A_TILE_BYTES
#define GC_A2A_TILE_BYTES 32768
#endif
#ifndef GC_A2A_UNR
#define GC_A2A_UNR 4
#endif

constexpr uint32_t kMaxGrid = GC_SEG_MAX_GRID;
constexpr uint32_t kA2AMaxGrid = GC_A2A_MAX_GRID;

template <class K, class A>
gc_status launch(K kernel, const A& args, uint32_t grid, hipStream_t stream) {
  void* params[] = {const_cast<A*>(&args)};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(std::max(1u, grid)),
                                       dim3(kThreads), params, 0, stream);
  return gci::hip_status(e);
}

uint64_t addr(const void* p) { return reinterpret_cast<uint64_t>(p); }

// Largest power-of-two width (<= 8) dividing the segment's addresses and length.
int narrow_width(const gci::Segment& s) {
  const uint64_t m = (s.src ? addr(s.src) : 0) | addr(s.dst) | s.bytes;
  if ((m & 7) == 0) return 8;
  if ((m & 3) == 0) return 4;
  if ((m & 1) == 0) return 2;
  return 1;
}

bool vec_ok(const gci::Segment& s) { return !s.src || ((addr(s.src) ^ addr(s.dst)) & 15) == 0; }

// Launch one batch of segments of one class (width 16 = vector kernel).
gc_status launch_batch(const gci::Segment* segs, int n, int width, hipStream_t stream) {
  SegArgs a{};
  uint32_t tiles = 0;
  for (int i = 0; i < n; ++i) {
    a.src[i] = static_cast<const char*>(segs[i].src);
    a.dst[i] = static_cast<char*>(segs[i].dst);
    a.bytes[i] = segs[i].bytes;
    a.tile0[i] = tiles;
    uint64_t units;
    if (width == 16) {
      const uint64_t head = std::min<uint64_t>(segs[i].bytes, (16 - (addr(segs[i].dst) & 15)) & 15);
      units = (segs[i].bytes - head) / 16;
      tiles += static_cast<uint32_t>(std::max<uint64_t>(1, (units + kSegTileVec - 1) / kSegTileVec));
    } else {
      units = segs[i].bytes / width;
      tiles += static_cast<uint32_t>(std::max<uint64_t>(1, (units + kThreads * 8 - 1) / (kThreads * 8)));
    }
  }
  a.tile0[n] = tiles;
  a.nseg = static_cast<uint32_t>(n);
  const uint32_t grid = std::min(tiles, kMaxGrid);
  switch (width) {
    case 16: return launch(segment_vec_kernel, a, grid, stream);
    case 8: return launch(segment_narrow_kernel<uint64_t>, a, grid, stream);
    case 4: return launch(segment_narrow_kernel<uint32_t>, a, grid, stream);
    case 2: return launch(segment_narrow_kernel<uint16_t>, a, grid, stream);
    default: return launch(segment_narrow_kernel<uint8_t>, a, grid, stream);
  }
}

}  // namespace

namespace gci {

gc_status launch_segment_copy(const Segment* segs, size_t nseg, hipStream_t stream) {
  // Group by copy class, then launch in batches of at most kMaxSeg.
  for (int width : {16, 8, 4, 2, 1}) {
    Segment batch[kMaxSeg];
    int n = 0;
    for (size_t i = 0; i < nseg; ++i) {
      const Segment& s = segs[i];
      if (s.bytes == 0) continue;
      const int w = vec_ok(s) ? 16 : narrow_width(s);
      if (w != width) continue;
      batch[n++] = s;
      if (n == kMaxSeg) {
        const gc_status st = launch_batch(batch, n, width, stream);
        if (st != GC_OK) return st;
        n = 0;
      }
    }
    if (n) {
      const gc_status st = launch_batch(batch, n, width, stream);
      if (st != GC_OK) return st;
    }
  }
  return GC_OK;
}

gc_status launch_all_to_all(const A2ACall& c) {
  A2AArgs a{};
  int64_t total = 0;
  for (int s = 0; s < c.nranks; ++s) {
    a.send[s] = static_cast<const char*>(c.send[s]);
    a.recv[s] = static_cast<char*>(c.recv[s]);
    a.send_base[s] = c.send_base[s];
  }
  const int nblk = c.nranks * c.dcount * c.experts;
  for (int b = 0; b < nblk; ++b) {
    a.rows[b] = c.rows[b];
    total += c.rows[b];
  }
  if (total == 0) return GC_OK;
  a.row_bytes = c.row_bytes;
  a.N = c.nranks;
  a.E = c.experts;
  a.d0 = c.d0;
  a.Dg = c.dcount;
  // Fixed payload per tile (GC_A2A_TILE_BYTES, at least one row).
  a.rows_per_tile = static_cast<uint32_t>(
      std::max<uint64_t>(1, std::min<uint64_t>(1u << 20, GC_A2A_TILE_BYTES / c.row_bytes)));
  const int64_t ntiles = (total + a.rows_per_tile - 1) / a.rows_per_tile;
  const uint32_t grid = static_cast<uint32_t>(std::min<int64_t>(ntiles, kA2AMaxGrid));
  uint64_t m = c.row_bytes;
  for (int s = 0; s < c.nranks; ++s) m |= addr(c.send[s]) | addr(c.recv[s]);
  if ((m & 15) == 0) return launch(a2a_kernel<u32x4, GC_A2A_UNR>, a, grid, c.stream);
  if ((m & 3) == 0) return launch(a2a_kernel<uint32_t, 8>, a, grid, c.stream);
  return launch(a2a_kernel<uint8_t, 8>, a, grid, c.stream);
}

}  // namespace gci
