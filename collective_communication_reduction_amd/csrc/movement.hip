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

#include "device_common.h"
#include "gc_internal.h"

namespace {

using namespace gcdev;

// ------------------------------------------------------------ segment copy

constexpr int kMaxSeg = 128;  // kernel arguments: 3.6 KiB of the 4 KiB limit
#ifndef GC_SEG_U
#define GC_SEG_U 1
#endif
constexpr int kSegU = GC_SEG_U;                   // 16-byte vectors per thread per tile
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

}  // namespace gci
