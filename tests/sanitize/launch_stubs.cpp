// Host-only stand-ins for the kernel launchers of libgc, for the sanitizer
// build of the C ABI layer (api.cpp).  Nothing here touches a GPU: each stub
// checks that every byte range the launch would read or write lies inside a
// buffer the caller declared (registered by the harness with the extent the
// header's contract gives it), counts the launch and returns GC_OK.
#include "stubs.h"

#include <cstdio>
#include <cstdlib>
#include <vector>

#include "gc_internal.h"

namespace stub {

uint64_t addr(const void* p) { return reinterpret_cast<uint64_t>(p); }

namespace {
struct Buf {
  uint64_t lo, hi;
};
std::vector<Buf> g_bufs;
long g_launches = 0;
long g_bad = 0;

void need(uint64_t lo, uint64_t bytes, const char* what) {
  if (bytes == 0) return;
  for (const Buf& b : g_bufs)
    if (b.lo <= lo && lo <= b.hi && bytes <= b.hi - lo) return;
  std::fprintf(stderr, "launch touches undeclared memory: %s at %#llx + %llu\n", what,
               static_cast<unsigned long long>(lo), static_cast<unsigned long long>(bytes));
  ++g_bad;
}
void need(const void* p, uint64_t bytes, const char* what) { need(addr(p), bytes, what); }
}  // namespace

void reset() { g_bufs.clear(); }
void declare(const void* p, uint64_t bytes) {
  if (p && bytes) g_bufs.push_back(Buf{addr(p), addr(p) + bytes});
}
long launches() { return g_launches; }
long violations() { return g_bad; }

}  // namespace stub

namespace gci {

using stub::need;

static gc_status reduce_like(const ReduceCall& c, uint64_t in_bytes_each, uint64_t out_bytes_each, bool per_chunk_in,
                             bool per_chunk_out) {
  const uint64_t ei = elem_bytes(c.in_t), eo = elem_bytes(c.out_t);
  for (int r = 0; r < c.nranks; ++r) {
    const uint64_t lo = std::min<uint64_t>(c.S, static_cast<uint64_t>(r) * c.c);
    const uint64_t hi = std::min<uint64_t>(c.S, lo + c.c);
    need(c.in[r], per_chunk_in ? (hi - lo) * ei : in_bytes_each, "reduce input");
    need(c.out[r], per_chunk_out ? (hi - lo) * eo : out_bytes_each, "reduce output");
  }
  ++stub::g_launches;
  return GC_OK;
}

gc_status launch_all_reduce(const ReduceCall& c) {
  return reduce_like(c, c.S * elem_bytes(c.in_t), c.S * elem_bytes(c.out_t), false, false);
}
gc_status launch_reduce_scatter(const ReduceCall& c) {
  return reduce_like(c, c.S * elem_bytes(c.in_t), 0, false, true);
}
gc_status launch_all_gather(const ReduceCall& c) {
  return reduce_like(c, 0, c.S * elem_bytes(c.out_t), true, false);
}

static gc_status hier_like(const HierCall& c, bool hsdp) {
  const uint64_t ei = elem_bytes(c.in_t), eo = elem_bytes(c.out_t);
  for (int r = 0; r < c.nranks; ++r) {
    need(c.in[r], c.count * ei, "two-level input");
    need(c.out[r], (hsdp ? c.count / c.group : c.count) * eo, "two-level output");
  }
  ++stub::g_launches;
  return GC_OK;
}
gc_status launch_hier_all_reduce(const HierCall& c) { return hier_like(c, false); }
gc_status launch_hsdp_reduce_scatter(const HierCall& c) { return hier_like(c, true); }

gc_status launch_bucket_all_reduce(const BucketCall& c) {
  const uint64_t es = elem_bytes(c.t);
  for (int i = 0; i < c.npieces; ++i) {
    const BucketPiece& p = c.pieces[i];
    if (static_cast<int>(p.slot) >= c.nslots || static_cast<int>(p.first) >= c.nranks) ++stub::g_bad;
    for (int r = 0; r < c.nranks; ++r)
      need(stub::addr(c.slot_ptrs[static_cast<size_t>(p.slot) * c.nranks + r]) + p.lo * es, p.len * es,
           "bucket piece");
  }
  if (c.sumsq) need(c.sumsq, 8, "sum of squares");
  ++stub::g_launches;
  return GC_OK;
}

gc_status launch_segment_copy(const Segment* segs, size_t nseg, StorePolicy, hipStream_t) {
  for (size_t i = 0; i < nseg; ++i) {
    if (segs[i].src) need(segs[i].src, segs[i].bytes, "segment source");
    need(segs[i].dst, segs[i].bytes, "segment destination");
  }
  ++stub::g_launches;
  return GC_OK;
}

gc_status launch_moe_route(const MoeRouteCall& c) {
  const int64_t nbins = static_cast<int64_t>(c.nranks) * c.experts_per_rank;
  int64_t tiles = 0;
  for (int s = 0; s < c.nranks; ++s) {
    need(c.experts[s], c.routes[s] * 4, "route experts");
    need(c.dest[s], c.routes[s] * 8, "route dest");
    tiles += (c.routes[s] + c.tile - 1) / c.tile;
  }
  need(c.counts, static_cast<uint64_t>(tiles * nbins * 4), "route counts");
  need(c.roff, static_cast<uint64_t>(c.nranks * nbins * 4), "route offsets");
  need(c.splits, static_cast<uint64_t>(c.nranks * nbins * 8), "splits");
  ++stub::g_launches;
  return GC_OK;
}

static gc_status move_like(const MoeMoveCall& c) {
  for (int r = 0; r < c.nranks; ++r) {
    need(c.src[r], c.src_rows[r] * c.row_bytes, "moe source rows");
    need(c.dst[r], c.dst_rows[r] * c.row_bytes, "moe destination rows");
    need(c.dest[r], c.tokens[r] * c.topk * 8, "moe dest table");
    if (c.weights) need(c.weights[r], c.tokens[r] * c.topk * 4, "moe weights");
  }
  ++stub::g_launches;
  return GC_OK;
}
gc_status launch_moe_dispatch(const MoeMoveCall& c) { return move_like(c); }
gc_status launch_moe_combine(const MoeMoveCall& c) { return move_like(c); }

// The static scratch of gc_moe_route_noalloc: a stand-in address, declared so
// that launches into it pass the extent check.
gc_status moe_route_static_scratch(hipStream_t, void** ptr) {
  static const uint64_t kFake = 0x7e0000000000ull;
  *ptr = reinterpret_cast<void*>(kFake);
  stub::declare(*ptr, GC_MOE_ROUTE_NOALLOC_SCRATCH_BYTES);
  return GC_OK;
}

}  // namespace gci
