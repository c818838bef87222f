// Internal interface between the C ABI layer (api.cpp: validation, planning)
// and the kernel launchers (reduce.hip, movement.hip).  Not installed.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gc.h"

namespace gci {

inline size_t elem_bytes(gc_dtype t) { return t == GC_BF16 ? 2 : 4; }

// Maps a HIP result to a status, remembering a failure for gc_last_hip_error().
gc_status hip_status(hipError_t e);

// Geometry shared by the three reduction-family launches.  The reference index
// space has S elements cut into N chunks [j*c, min(S, (j+1)*c)).
//
//   all_reduce:      in[i]  = rank i's buffer        (element E at in[i] + E)
//                    out[r] = rank r's buffer        (element E at out[r] + E)
//   reduce_scatter:  in[i]  = rank i's full buffer   (element E at in[i] + E)
//                    out[j] = chunk j's destination  (element E at out[j] + E - j*c)
//   all_gather:      in[i]  = shard i                (element E at in[i] + E - i*c)
//                    out[d] = rank d's full buffer   (element E at out[d] + E)
struct ReduceCall {
  const void* const* in;
  void* const* out;
  int nranks;
  uint64_t S;
  uint64_t c;
  gc_dtype in_t;
  gc_dtype out_t;
  bool avg;
  bool ring;
  hipStream_t stream;
  bool wire = false;  // ring whose forwarded partials are rounded to the input type
};

gc_status launch_all_reduce(const ReduceCall& call);

// Two-level reduction over nranks = R * group ranks (rank g * group + i is
// member i of group g).  in[r]: rank r's count elements.  All-reduce: out[r]
// rank r's count elements.  HSDP reduce-scatter: out[r] member i's shard of
// count / group elements.
struct HierCall {
  const void* const* in;
  void* const* out;
  int nranks;
  int group;
  uint64_t count;
  gc_dtype in_t;
  gc_dtype out_t;
  bool avg;
  bool ring;
  hipStream_t stream;
  bool wire = false;  // ring whose forwarded partials are rounded to the input type (both levels)
};

gc_status launch_hier_all_reduce(const HierCall& call);
gc_status launch_hsdp_reduce_scatter(const HierCall& call);
gc_status launch_reduce_scatter(const ReduceCall& call);
gc_status launch_all_gather(const ReduceCall& call);

// Zero-copy bucket all-reduce.  A piece is the part of one tensor that falls
// inside one owner chunk of the bucket's packed index space: elements
// [lo, lo + len) of the tensor in `slot`, folded starting at rank `first`.
struct BucketPiece {
  uint64_t lo;
  uint64_t len;
  uint32_t slot;
  uint32_t first;
};

struct BucketCall {
  void* const* slot_ptrs;  // [nslots * nranks], slot-major: rank r's tensor of slot s at [s * nranks + r]
  int nslots;
  int nranks;
  const BucketPiece* pieces;  // ordered by slot
  int npieces;
  gc_dtype t;
  bool avg;
  double* sumsq;  // device accumulator for the sum of squared results, or nullptr
  hipStream_t stream;
  bool wire = false;  // ring whose forwarded partials are rounded to the input type
};

gc_status launch_bucket_all_reduce(const BucketCall& call);

// Cache policy of a kernel's 16-byte stores.  kStoreNT: the non-temporal hint
// alone.  kStoreDevNT: device scope (sc1) plus the hint: the line is written
// through the XCD's L2 rather than left there dirty.  kStoreDev: device scope
// without the hint, so the line may stay in the MALL for the kernel that reads
// it next.
enum StorePolicy : int { kStoreNT = 0, kStoreDevNT = 1, kStoreDev = 2 };

// One contiguous copy; src == nullptr writes zeros.
struct Segment {
  const void* src;
  void* dst;
  uint64_t bytes;
};

gc_status launch_segment_copy(const Segment* segs, size_t nseg, StorePolicy pol, hipStream_t stream);


// MoE routing plan (see gc_moe_route).  Routes of source s are cut into tiles
// of `tile` routes; counts holds [tiles][nranks * experts_per_rank] int32 and
// roff [nranks][nranks * experts_per_rank] int32 of scratch.
struct MoeRouteCall {
  const int32_t* const* experts;
  int32_t* const* dest;
  const int64_t* routes;  // [nranks] tokens * topk
  int nranks;
  int experts_per_rank;
  int32_t tile;
  int32_t* counts;
  int32_t* roff;
  int64_t* splits;
  hipStream_t stream;
};

// MoE dispatch (src = token rows, dst = receive buffers) or combine
// (src = expert outputs in the receive layout, dst = token rows).
struct MoeMoveCall {
  const void* const* src;
  const int64_t* src_rows;     // rows of each src buffer
  const int32_t* const* dest;  // per source: [tokens * topk] (rank, row) pairs
  const float* const* weights; // combine only
  void* const* dst;
  const int64_t* dst_rows;     // rows of each dst buffer
  const int64_t* tokens;       // [nranks] tokens per source
  int nranks;
  int topk;
  uint64_t row_bytes;
  gc_dtype t;                  // combine only
  hipStream_t stream;
};

// Routes per routing-plan tile while the experts fit it (four wavefronts).
#ifndef GC_MOE_ROUTE_TILE
#define GC_MOE_ROUTE_TILE 1024
#endif
constexpr int32_t kMoeRouteTile = GC_MOE_ROUTE_TILE;

gc_status launch_moe_route(const MoeRouteCall& call);

// Device address of the routing plan's static scratch array on the device that
// runs `stream` (the current device for the null stream), looked up once per
// device; GC_ERR_HIP if the lookup fails.
gc_status moe_route_static_scratch(hipStream_t stream, void** ptr);
gc_status launch_moe_dispatch(const MoeMoveCall& call);
gc_status launch_moe_combine(const MoeMoveCall& call);

}  // namespace gci
