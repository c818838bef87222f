// The segment copy for gfx950: a batch of (source, destination, bytes)
// copies in one launch.  It carries DDP bucket pack / unpack (AIG6 §6.2.4 and
// NXMR §5.1 gradient buckets; DTLM §4 FSDP1 FlatParameter layout) and the
// all-to-all(v) block permutation (DTLM §2 "All-to-All", DTLM §8
// All-to-AllV), whose (source, destination, expert) blocks are contiguous on
// both sides, so each block is one segment.
//
// An HBM stream with no arithmetic.  Work is cut into equal-byte tiles across
// all segments, so a launch that mixes one huge tensor with many tiny ones, or
// a skewed all-to-all where most rows go to one rank, still gives every
// workgroup the same number of bytes.

#include <algorithm>
#include <cstdint>

#include "device_common.h"
#include "gc_internal.h"

namespace {

using namespace gcdev;

// ------------------------------------------------------------ segment copy

constexpr int kMaxSeg = 128;  // kernel arguments: 3.6 KiB of the 4 KiB limit
constexpr int kSegGroup = 16;                     // segments per lookup group
constexpr int kSegGroups = kMaxSeg / kSegGroup;
#ifndef GC_SEG_U
#define GC_SEG_U 1
#endif
constexpr int kSegU = GC_SEG_U;                   // 16-byte vectors per thread per tile
constexpr uint64_t kSegTileVec = kThreads * kSegU;

struct SegDesc {
  const char* src;  // nullptr: fill with zeros
  char* dst;
  uint64_t bytes;
};

struct SegArgs {
  SegDesc seg[kMaxSeg];
  uint32_t tile0[kMaxSeg];         // first tile of each segment; UINT32_MAX past the last
  uint32_t coarse[kSegGroups];     // tile0[kSegGroup * g]; UINT32_MAX for unused groups
  uint32_t nseg, ntiles;
};
static_assert(sizeof(SegArgs) <= 4096, "segment table must fit the kernel argument limit");

// Launch-wide lookup state, read once per workgroup before its first tile:
// with these the segment of a tile takes at most two dependent scalar loads
// (the tile starts of its group of 16 segments, then its descriptor), and a
// one-segment launch none.  A workgroup copies only 4 KiB, so its life is
// about one HBM round trip; a binary search over the tile table (seven
// dependent loads at 128 segments) kept fewer bytes in flight.
struct SegLookup {
  uint32_t ntiles, nseg;
  uint32_t coarse[kSegGroups];
  SegDesc first;
};

__device__ __forceinline__ SegLookup seg_lookup(const SegArgs& a) {
  SegLookup l;
  l.ntiles = a.ntiles;
  l.nseg = a.nseg;
#pragma unroll
  for (int i = 0; i < kSegGroups; ++i) l.coarse[i] = a.coarse[i];
  l.first = a.seg[0];
  return l;
}

// Segment of `tile` and the tile's index inside it.
__device__ __forceinline__ SegDesc find_segment(const SegArgs& a, const SegLookup& l, uint32_t tile, uint32_t& t) {
  if (l.nseg == 1) {
    t = tile;
    return l.first;
  }
  // Group g: the last whose first tile is <= tile (selects only: a dynamic
  // index into a local array would put it, and the argument block, in scratch).
  uint32_t g = 0, start = l.coarse[0];
#pragma unroll
  for (int i = 1; i < kSegGroups; ++i) {
    if (l.coarse[i] <= tile) {
      g = i;
      start = l.coarse[i];
    }
  }
  uint32_t j = 0;
#pragma unroll
  for (int i = 1; i < kSegGroup; ++i) {
    const uint32_t v = a.tile0[g * kSegGroup + i];  // ascending; UINT32_MAX past the last segment
    if (v <= tile) {
      j = i;
      start = v;
    }
  }
  t = tile - start;
  return a.seg[g * kSegGroup + j];
}

// Segments whose source and destination agree modulo 16 bytes: byte head up
// to the first 16-byte boundary of the destination, 16-byte body, byte tail.
// POL is the body stores' cache policy (gci::StorePolicy).
template <int POL>
__global__ void __launch_bounds__(kThreads) segment_vec_kernel(const SegArgs a) {
  const SegLookup l = seg_lookup(a);
  // The grid never exceeds the tile count, so every workgroup has a first tile
  // (no guard ahead of it: all lookup loads issue together).
  uint32_t tile = blockIdx.x;
  do {
    uint32_t t;
    const SegDesc d = find_segment(a, l, tile, t);
    const char* src = d.src;
    char* dst = d.dst;
    const uint64_t n = d.bytes;
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
        if (v < nvec) st16p<POL>(dst + head + 16 * v, buf[u]);
      }
    }
    if (t == 0) {
      const uint64_t nedge = head + (n - tail_beg);  // < 32 bytes
      if (threadIdx.x < nedge) {
        const uint64_t b = threadIdx.x < head ? threadIdx.x : tail_beg + (threadIdx.x - head);
        dst[b] = src ? src[b] : 0;
      }
    }
    tile += gridDim.x;
  } while (tile < l.ntiles);
}

// Segments with mismatched alignment: W-byte elements (W divides both
// addresses and the length).
template <typename T>
__global__ void __launch_bounds__(kThreads) segment_narrow_kernel(const SegArgs a) {
  const SegLookup l = seg_lookup(a);
  constexpr uint64_t TE = kThreads * 8;
  uint32_t tile = blockIdx.x;  // the grid never exceeds the tile count
  do {
    uint32_t t;
    const SegDesc d = find_segment(a, l, tile, t);
    const T* src = reinterpret_cast<const T*>(d.src);
    T* dst = reinterpret_cast<T*>(d.dst);
    const uint64_t n = d.bytes / sizeof(T);
    if (static_cast<uint64_t>(t) * TE < n) {
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
    tile += gridDim.x;
  } while (tile < l.ntiles);
}

// ------------------------------------------------------------ host side

#ifndef GC_SEG_MAX_GRID
#define GC_SEG_MAX_GRID (1u << 20)
#endif
constexpr uint32_t kMaxGrid = GC_SEG_MAX_GRID;

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
gc_status launch_batch(const gci::Segment* segs, int n, int width, gci::StorePolicy pol, hipStream_t stream) {
  SegArgs a{};
  std::fill(a.tile0, a.tile0 + kMaxSeg, UINT32_MAX);
  std::fill(a.coarse, a.coarse + kSegGroups, UINT32_MAX);
  uint32_t tiles = 0;
  for (int i = 0; i < n; ++i) {
    a.seg[i] = SegDesc{static_cast<const char*>(segs[i].src), static_cast<char*>(segs[i].dst), segs[i].bytes};
    a.tile0[i] = tiles;
    if (i % kSegGroup == 0) a.coarse[i / kSegGroup] = tiles;
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
  a.ntiles = tiles;
  a.nseg = static_cast<uint32_t>(n);
  const uint32_t grid = std::min(tiles, kMaxGrid);
  switch (width) {
    case 16:
      switch (pol) {
        case gci::kStoreDevNT: return launch(segment_vec_kernel<gci::kStoreDevNT>, a, grid, stream);
        case gci::kStoreDev: return launch(segment_vec_kernel<gci::kStoreDev>, a, grid, stream);
        default: return launch(segment_vec_kernel<gci::kStoreNT>, a, grid, stream);
      }
    case 8: return launch(segment_narrow_kernel<uint64_t>, a, grid, stream);
    case 4: return launch(segment_narrow_kernel<uint32_t>, a, grid, stream);
    case 2: return launch(segment_narrow_kernel<uint16_t>, a, grid, stream);
    default: return launch(segment_narrow_kernel<uint8_t>, a, grid, stream);
  }
}

}  // namespace

namespace gci {

gc_status launch_segment_copy(const Segment* segs, size_t nseg, StorePolicy pol, hipStream_t stream) {
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
        const gc_status st = launch_batch(batch, n, width, pol, stream);
        if (st != GC_OK) return st;
        n = 0;
      }
    }
    if (n) {
      const gc_status st = launch_batch(batch, n, width, pol, stream);
      if (st != GC_OK) return st;
    }
  }
  return GC_OK;
}

}  // namespace gci
