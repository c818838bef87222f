// Access-pattern ceilings for bench.py --patterns: unordered kernels that move
// the same bytes as the library's collectives, in the same tiles, with none of
// their semantics (no fold order, no floating point, no epilogue).  Comparing
// a collective with the pattern of its own reads and writes on the same
// buffers separates what the memory system allows from what the kernel adds.
// Measurement infrastructure only: nothing in the library links it.
//
// One pattern = nsrc source streams and ndst destination streams of nvec
// 16-byte vectors each, in tiles of 256 threads x 2 vectors, each wavefront
// reading a contiguous 2 KiB per stream (the library's tile layout).  For
// every vector position the sources are summed as uint32 lanes, then
//   mode 0 (all-reduce shape)    the sum is stored to every destination at the
//                                same position (ndst = 0: nothing is stored,
//                                the fold's reads alone);
//   mode 1 (reduce-scatter shape) position v belongs to chunk j = v / chunk_vecs
//                                of nch = nvec / chunk_vecs chunks, and out_mult
//                                vectors are stored at (v - j * chunk_vecs) *
//                                out_mult in dst[j + c * nch] for each of the
//                                ndst / nch copies c (out_mult = 2: the 32 bytes
//                                of fp32 output per 16 bytes of bf16 input; two
//                                copies: both holders of an HSDP shard).
// nsrc = 0 stores a pattern of the position (writes alone).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMax = 64;
constexpr int kThreads = 256;
constexpr int kU = 2;

struct PatArgs {
  const char* src[kMax];
  char* dst[kMax];
  uint64_t nvec;
  uint64_t chunk_vecs;
  uint32_t nsrc, ndst, mode, out_mult, nch;
  uint32_t* sink;
};

__global__ void __launch_bounds__(kThreads) pattern_kernel(const PatArgs a) {
  const uint64_t tv0 = static_cast<uint64_t>(blockIdx.x) * (kThreads * kU);
  uint64_t v[kU], vl[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    v[u] = tv0 + (threadIdx.x >> 6) * (64 * kU) + u * 64 + (threadIdx.x & 63);
    vl[u] = v[u] < a.nvec ? v[u] : a.nvec - 1;  // loads stay in bounds without predicates
  }
  u32x4 acc[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) acc[u] = u32x4{0, 0, 0, 0};
  for (uint32_t s = 0; s < a.nsrc; s += 8) {  // batches of eight streams, every load in flight together
    u32x4 x[8][kU];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int u = 0; u < kU; ++u)
        x[k][u] = s + k < a.nsrc
                      ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.src[s + k]) + vl[u])
                      : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int u = 0; u < kU; ++u) acc[u] += x[k][u];
  }
  if (a.nsrc == 0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) acc[u] = u32x4{static_cast<uint32_t>(v[u]), 1u, 2u, 3u};
  }
  if (a.ndst == 0) {
    // keep the reads: store only for a sum no input here produces
    if (acc[0].x == 0x9E3779B9u && acc[kU - 1].w == 0x7F4A7C15u) a.sink[threadIdx.x] = acc[0].y;
    return;
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if (v[u] >= a.nvec) continue;
    if (a.mode == 0) {
      for (uint32_t d = 0; d < a.ndst; ++d)
        __builtin_nontemporal_store(acc[u], reinterpret_cast<u32x4*>(a.dst[d]) + v[u]);
    } else {
      // A wavefront's 64 positions produce 64 * out_mult contiguous output vectors.  Where they all
      // lie in one chunk, lane l stores vectors l, l + 64, ... of that run (every store instruction
      // writes 1 KiB contiguously, as the library's regrouped stores do; which lane's sum lands where
      // does not matter here).  A wavefront across a chunk edge or the end stores its own out_mult
      // vectors per lane.
      const uint64_t lane = threadIdx.x & 63, vw = v[u] - lane;
      const uint64_t j = v[u] / a.chunk_vecs;
      const bool whole = vw / a.chunk_vecs == (vw + 63) / a.chunk_vecs && vw + 63 < a.nvec;
      const uint64_t off = whole ? (vw - j * a.chunk_vecs) * a.out_mult + lane : (v[u] - j * a.chunk_vecs) * a.out_mult;
      const uint64_t step = whole ? 64 : 1;
      for (uint32_t c = j; c < a.ndst; c += a.nch) {
        u32x4* out = reinterpret_cast<u32x4*>(a.dst[c]) + off;
        for (uint32_t m = 0; m < a.out_mult; ++m) __builtin_nontemporal_store(acc[u] ^ m, out + m * step);
      }
    }
  }
}

}  // namespace

// Returns 0 on success, 1 for invalid arguments (nothing launched), 3 if the
// launch failed.  Buffers are device pointers of at least nvec vectors each
// (mode 1: each dst holds chunk_vecs * out_mult vectors); sink holds 256 uint32.
extern "C" int bp_pattern(const void* const* src, int nsrc, void* const* dst, int ndst, uint64_t nvec,
                          uint64_t chunk_vecs, int mode, int out_mult, uint32_t* sink, hipStream_t stream) {
  if (nsrc < 0 || nsrc > kMax || ndst < 0 || ndst > kMax || nvec == 0 || !sink) return 1;
  if ((nsrc > 0 && !src) || (ndst > 0 && !dst) || (nsrc == 0 && ndst == 0)) return 1;
  if (mode != 0 && mode != 1) return 1;
  uint64_t nch = 0;
  if (mode == 1) {
    if (out_mult < 1 || out_mult > 4 || chunk_vecs == 0 || nvec % chunk_vecs) return 1;
    nch = nvec / chunk_vecs;
    if (ndst == 0 || nch > static_cast<uint64_t>(ndst) || ndst % nch) return 1;
  }
  PatArgs a = {};
  for (int i = 0; i < nsrc; ++i) {
    if (!src[i] || reinterpret_cast<uintptr_t>(src[i]) % 16) return 1;
    a.src[i] = static_cast<const char*>(src[i]);
  }
  for (int i = 0; i < ndst; ++i) {
    if (!dst[i] || reinterpret_cast<uintptr_t>(dst[i]) % 16) return 1;
    a.dst[i] = static_cast<char*>(dst[i]);
  }
  a.nvec = nvec;
  a.chunk_vecs = chunk_vecs;
  a.nsrc = static_cast<uint32_t>(nsrc);
  a.ndst = static_cast<uint32_t>(ndst);
  a.mode = static_cast<uint32_t>(mode);
  a.out_mult = static_cast<uint32_t>(out_mult);
  a.nch = static_cast<uint32_t>(nch);
  a.sink = sink;
  const uint64_t grid = (nvec + kThreads * kU - 1) / (kThreads * kU);
  if (grid > 0x7fffffffull) return 1;
  void* params[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(pattern_kernel), dim3(static_cast<uint32_t>(grid)),
                         dim3(kThreads), params, 0, stream) == hipSuccess ? 0 : 3;
}
