// Zero-copy bucketed all-reduce for gfx950 (DDP with gradient_as_bucket_view,
// AIG6 = "AI Infra Guide" ch. 6, §6.2.4): the bucket is never materialised.
// The reduction runs directly over the N ranks' gradient tensors, in place,
// and every element is folded in the order its position in the packed bucket
// gives it (owner chunk j of ceil(bucket/N) elements, ranks j+1, ..., j;
// DTLM = "Distributed Training for Large Models", §2 "Reduce-Scatter").  The
// result is therefore bit-identical to packing the bucket, all-reducing it and
// unpacking it, with a third of the HBM traffic: 2*N*B bytes instead of 6*N*B.
//
// With the bf16 wire order every forwarded partial is rounded to bf16 before
// the next rank adds its term, as a ring that communicates in the gradients'
// type would (DTLM §11), so the result stays bit-identical to pack ->
// all-reduce (wire order) -> unpack.
//
// The host cuts the bucket into pieces (tensor x owner chunk); each piece has
// one pointer set, one fold start and one alignment phase, so the inner loop
// is the fused all-reduce's: 16-byte vectors, all of a batch's loads issued
// before the first add, predicate-free full tiles.
//
// Optionally the epilogue also accumulates the sum of squares of the results
// (as stored) into a device double, for gradient-norm clipping after the sync:
// wavefront shuffles reduce each wavefront's partial, LDS combines the
// wavefronts, then one atomic add per workgroup.  The atomics' order is not fixed, so the norm's last bits may
// vary between runs; the gradients themselves never do.

#include <algorithm>

#include "device_common.h"
#include "fold.h"
#include "gc_internal.h"

namespace {

using namespace gcdev;

// Cache policy of the in-place results' 16-byte stores: device scope measured
// 34.55 against 34.77 ms for the 226 buckets of the 8-rank DDP step.
#ifndef GC_BUCKET_STORE
#define GC_BUCKET_STORE gci::kStoreDevNT
#endif

constexpr int kMaxPieces = 40;

// Each wavefront reads a contiguous run of U KiB per rank (measured on MI355X,
// the zero-copy all-reduce of a 37-tensor Llama-7B prefix, one process: 5.66-5.70
// against 5.49-5.51 TB/s for the workgroup-strided layout).
#ifndef GC_BUCKET_WAVE_CONTIG
#define GC_BUCKET_WAVE_CONTIG 1
#endif
constexpr bool kBucketWave = GC_BUCKET_WAVE_CONTIG != 0;

struct PieceDev {
  uint64_t lo;      // first element of the piece (tensor-local index)
  uint64_t len;     // elements
  uint32_t slot;    // row of the pointer table
  uint32_t first;   // first rank of the fold
  uint32_t phase;   // elements before the first 16-byte-aligned vector, or len (no vectors)
  uint32_t tile0;   // first tile of the piece
  uint32_t vec;     // 1: vector path; 0: element path (pointers disagree modulo 16)
  uint32_t pad;
};

template <int P, int MAXS>
struct BucketArgs {
  char* ptr[MAXS][P];
  PieceDev piece[kMaxPieces];
  uint32_t npieces;
  uint32_t ntiles;
  uint32_t N;
  uint32_t avg;
  float nf;
};

template <int P, int MAXS>
__device__ __forceinline__ uint32_t find_piece(const BucketArgs<P, MAXS>& a, uint32_t tile) {
  uint32_t lo = 0, hi = a.npieces;  // last piece with tile0 <= tile
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) / 2;
    if (a.piece[mid].tile0 <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

// Value of a stored result, as the tensor holds it, widened to double.
template <class Out>
__device__ __forceinline__ double stored_value(float x) {
  if constexpr (Out::ES == 2) return static_cast<double>(__uint_as_float(bf16_bits(x) << 16));
  else return static_cast<double>(x);
}

// Workgroup sum of v (wavefront shuffles, then the wavefronts' partials in a
// fixed order through LDS), added to *dst with one atomic per workgroup.
// Every thread of the workgroup must call it.
__device__ __forceinline__ void group_atomic_add(double* dst, double v) {
  __shared__ double s_part[kThreads / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) t += s_part[w];
    if (t != 0.0) atomicAdd(dst, t);
  }
}

template <class In, class Out, int NF, int U, bool GUARD, bool SUMSQ, bool WIRE, int P, int MAXS>
__device__ __forceinline__ double bucket_tile(const BucketArgs<P, MAXS>& a, const PieceDev& pc, uint32_t N,
                                              uint64_t tv0, uint64_t nvec) {
  constexpr int VE = In::VE;
  typedef typename In::Acc Acc;
  const char* const* in = reinterpret_cast<const char* const*>(a.ptr[pc.slot]);
  uint64_t off[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t v = GUARD ? min(tile_vec<U, kBucketWave>(tv0, u), nvec - 1) : tile_vec<U, kBucketWave>(tv0, u);
    off[u] = (pc.lo + pc.phase + v * VE) * In::ES;
  }
  Acc acc[U][VE];
  fold_vec<In, NF, U, WIRE>(in, pc.first, N, off, acc);
  const bool avg = a.avg != 0;
  double sq = 0.0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t v = tile_vec<U, kBucketWave>(tv0, u);
    Acc o[VE];
#pragma unroll
    for (int l = 0; l < VE; ++l) o[l] = finish(acc[u][l], avg, a.nf);
    const Words<Out, VE> w = pack<Out, VE>(o);
    if (!GUARD || v < nvec) {
      for (uint32_t q = 0; q < N; ++q) put<Out, VE, GC_BUCKET_STORE>(a.ptr[pc.slot][q] + off[u], w);
      if constexpr (SUMSQ) {
#pragma unroll
        for (int l = 0; l < VE; ++l) {
          const double y = stored_value<Out>(o[l]);
          sq += y * y;
        }
      }
    }
  }
  return sq;
}

template <class In, class Out, int NF, int U, bool SUMSQ, bool WIRE, int P, int MAXS>
__global__ void __launch_bounds__(kThreads) bucket_ar_kernel(const BucketArgs<P, MAXS> a, double* sumsq) {
  constexpr int VE = In::VE;
  constexpr int TV = kThreads * U;
  constexpr int TE = kThreads * 4;
  typedef typename In::Acc Acc;
  const uint32_t N = NF ? NF : a.N;
  const bool avg = a.avg != 0;
  double sq = 0.0;
  for (uint32_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const PieceDev& pc = a.piece[find_piece(a, tile)];
    const uint32_t t = tile - pc.tile0;
    const char* const* in = reinterpret_cast<const char* const*>(a.ptr[pc.slot]);
    if (pc.vec) {
      const uint64_t nvec = pc.len > pc.phase ? (pc.len - pc.phase) / VE : 0;
      const uint64_t tv0 = static_cast<uint64_t>(t) * TV;
      if (tv0 + TV <= nvec) {
        sq += bucket_tile<In, Out, NF, U, false, SUMSQ, WIRE>(a, pc, N, tv0, nvec);
      } else if (tv0 < nvec) {
        sq += bucket_tile<In, Out, NF, U, true, SUMSQ, WIRE>(a, pc, N, tv0, nvec);
      }
      if (t == 0) {
        // elements before the first and after the last aligned vector: < 2 * VE
        const uint64_t nhead = min(pc.phase, pc.len);
        const uint64_t tail_beg = nvec ? pc.phase + nvec * VE : nhead;
        const uint64_t nscalar = nhead + (pc.len - tail_beg);
        if (threadIdx.x < nscalar) {
          const uint64_t E = pc.lo + (threadIdx.x < nhead ? threadIdx.x : tail_beg + (threadIdx.x - nhead));
          const Acc x = finish(fold_one<In, WIRE>(in, pc.first, N, E), avg, a.nf);
          for (uint32_t q = 0; q < N; ++q) put_one<Out>(a.ptr[pc.slot][q], E, x);
          if constexpr (SUMSQ) {
            const double y = stored_value<Out>(x);
            sq += y * y;
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint64_t e = static_cast<uint64_t>(t) * TE + u * kThreads + threadIdx.x;
        if (e < pc.len) {
          const uint64_t E = pc.lo + e;
          const Acc x = finish(fold_one<In, WIRE>(in, pc.first, N, E), avg, a.nf);
          for (uint32_t q = 0; q < N; ++q) put_one<Out>(a.ptr[pc.slot][q], E, x);
          if constexpr (SUMSQ) {
            const double y = stored_value<Out>(x);
            sq += y * y;
          }
        }
      }
    }
  }
  if constexpr (SUMSQ) group_atomic_add(sumsq, sq);
}

// ------------------------------------------------------------------ host side

constexpr int kU = 2;

uint64_t addr(const void* p) { return reinterpret_cast<uint64_t>(p); }

template <class K, class A>
gc_status launch(K kernel, const A& args, double* sumsq, hipStream_t stream) {
  void* params[] = {const_cast<A*>(&args), &sumsq};
  const uint32_t grid = std::max(1u, args.ntiles);
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(kThreads), params, 0,
                                       stream);
  return gci::hip_status(e);
}

template <class In, class Out, int P, int MAXS, bool SUMSQ, bool WIRE>
gc_status dispatch(const BucketArgs<P, MAXS>& a, double* sumsq, hipStream_t s) {
  if constexpr (P == 8) {
    switch (a.N) {
      case 2: return launch(bucket_ar_kernel<In, Out, 2, kU, SUMSQ, WIRE, P, MAXS>, a, sumsq, s);
      case 4: return launch(bucket_ar_kernel<In, Out, 4, kU, SUMSQ, WIRE, P, MAXS>, a, sumsq, s);
      case 8: return launch(bucket_ar_kernel<In, Out, 8, kU, SUMSQ, WIRE, P, MAXS>, a, sumsq, s);
      default: break;
    }
  }
  return launch(bucket_ar_kernel<In, Out, 0, kU, SUMSQ, WIRE, P, MAXS>, a, sumsq, s);
}

// The wire-rounding instantiations exist for bf16 data only (fp32 and int32
// partials travel unrounded, so the plain kernels run).
template <class In, class Out, int P, int MAXS, bool SUMSQ>
gc_status dispatch_wire(const BucketArgs<P, MAXS>& a, bool wire, double* sumsq, hipStream_t s) {
  if constexpr (In::ES == 2) {
    if (wire) return dispatch<In, Out, P, MAXS, SUMSQ, true>(a, sumsq, s);
  }
  return dispatch<In, Out, P, MAXS, SUMSQ, false>(a, sumsq, s);
}

// One launch over pieces [p0, p1), whose slots are [s0, s1).
template <class In, class Out, int P, int MAXS>
gc_status run_batch(const gci::BucketCall& c, int p0, int p1, int s0, int s1) {
  constexpr int VE = In::VE;
  const int N = c.nranks;
  BucketArgs<P, MAXS> a{};
  for (int s = s0; s < s1; ++s)
    for (int r = 0; r < N; ++r) a.ptr[s - s0][r] = static_cast<char*>(c.slot_ptrs[static_cast<size_t>(s) * N + r]);
  uint32_t tiles = 0;
  for (int i = p0; i < p1; ++i) {
    const gci::BucketPiece& bp = c.pieces[i];
    PieceDev& d = a.piece[i - p0];
    d.lo = bp.lo;
    d.len = bp.len;
    d.slot = bp.slot - s0;
    d.first = bp.first;
    d.tile0 = tiles;
    // common 16-byte phase of element lo across the N tensors
    const uint64_t mis = (addr(a.ptr[d.slot][0]) + bp.lo * In::ES) & 15;
    bool same = mis % In::ES == 0;
    for (int r = 1; r < N && same; ++r) same = ((addr(a.ptr[d.slot][r]) + bp.lo * In::ES) & 15) == mis;
    d.vec = same ? 1u : 0u;
    if (same) {
      d.phase = static_cast<uint32_t>(std::min<uint64_t>(bp.len, ((16 - mis) & 15) / In::ES));
      const uint64_t nvec = bp.len > d.phase ? (bp.len - d.phase) / VE : 0;
      tiles += static_cast<uint32_t>(std::max<uint64_t>(1, (nvec + kThreads * kU - 1) / (kThreads * kU)));
    } else {
      d.phase = 0;
      tiles += static_cast<uint32_t>(std::max<uint64_t>(1, (bp.len + kThreads * 4 - 1) / (kThreads * 4)));
    }
  }
  a.npieces = static_cast<uint32_t>(p1 - p0);
  a.ntiles = tiles;
  a.N = static_cast<uint32_t>(N);
  a.avg = c.avg ? 1u : 0u;
  a.nf = static_cast<float>(N);
  if constexpr (__is_same(typename In::Acc, float)) {
    if (c.sumsq) return dispatch_wire<In, Out, P, MAXS, true>(a, c.wire, c.sumsq, c.stream);
  }
  return dispatch_wire<In, Out, P, MAXS, false>(a, c.wire, nullptr, c.stream);
}

template <class In, class Out, int P, int MAXS>
gc_status run_all(const gci::BucketCall& c) {
  // Batches of consecutive pieces touching at most MAXS slots and kMaxPieces pieces.
  int p0 = 0;
  while (p0 < c.npieces) {
    const int s0 = static_cast<int>(c.pieces[p0].slot);
    int p1 = p0;
    while (p1 < c.npieces && p1 - p0 < kMaxPieces && static_cast<int>(c.pieces[p1].slot) - s0 < MAXS) ++p1;
    const int s1 = static_cast<int>(c.pieces[p1 - 1].slot) + 1;
    const gc_status st = run_batch<In, Out, P, MAXS>(c, p0, p1, s0, s1);
    if (st != GC_OK) return st;
    p0 = p1;
  }
  return GC_OK;
}

template <class In, class Out>
gc_status run_typed(const gci::BucketCall& c) {
  if (c.nranks <= 8) return run_all<In, Out, 8, 24>(c);
  return run_all<In, Out, GC_MAX_RANKS, 3>(c);
}

}  // namespace

namespace gci {

gc_status launch_bucket_all_reduce(const BucketCall& c) {
  if (c.npieces == 0) return GC_OK;
  switch (c.t) {
    case GC_BF16: return run_typed<InBf16, OutBf16>(c);
    case GC_FP32: return run_typed<InF32, OutF32>(c);
    default: return run_typed<InI32, OutI32>(c);
  }
}

}  // namespace gci
