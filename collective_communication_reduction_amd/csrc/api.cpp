// C ABI of libgc: argument validation, aliasing rules, chunk / bucket /
// all-to-all planning on the host, then the kernel launches.  Every check runs
// before anything is enqueued, so a non-OK status means no work was launched.

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <new>
#include <vector>

#include "gc.h"
#include "gc_internal.h"

namespace {

using gci::elem_bytes;

bool valid_dtype(gc_dtype t) { return t == GC_INT32 || t == GC_FP32 || t == GC_BF16; }
bool valid_op(gc_op op) { return op == GC_SUM || op == GC_AVG; }
bool valid_order(gc_order o) { return o == GC_ORDER_RING || o == GC_ORDER_RANK || o == GC_ORDER_RING_WIRE; }

uint64_t addr(const void* p) { return reinterpret_cast<uint64_t>(p); }

// Byte interval [lo, hi) of a buffer.
struct Span {
  uint64_t lo, hi;
  bool empty() const { return hi <= lo; }
};

Span span(const void* p, uint64_t bytes) { return Span{addr(p), addr(p) + bytes}; }

// Largest extent of one buffer: 2^40 bytes, beyond any one GPU's memory
// (MI355X: 288 GB of HBM).  With it, and a call's total copy volume bounded by
// kMaxCopyBytes, every tile count the planners derive (2 KiB or more per
// tile) stays below 2^32.
constexpr uint64_t kMaxExtent = uint64_t(1) << 40;
constexpr uint64_t kMaxCopyBytes = uint64_t(1) << 42;

// True if `bytes` bytes at p are a possible buffer: at most kMaxExtent and
// ending inside the 64-bit address space.  Every buffer extent a call derives
// is checked with it before any span is formed, so spans never wrap and the
// addresses handed to the kernels never overflow.
bool fits(const void* p, uint64_t bytes) { return bytes <= kMaxExtent && bytes <= UINT64_MAX - addr(p); }

// Address `off` bytes past p, computed on integers (the extent holding it was checked with fits).
void* at(const void* p, uint64_t off) { return reinterpret_cast<void*>(addr(p) + off); }

bool overlaps(const Span& a, const Span& b) { return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi; }

// True if any two spans of `w` overlap.
bool any_overlap(std::vector<Span> w) {
  std::sort(w.begin(), w.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
  uint64_t reach = 0;
  bool first = true;
  for (const Span& s : w) {
    if (s.empty()) continue;
    if (!first && s.lo < reach) return true;
    reach = first ? s.hi : std::max(reach, s.hi);
    first = false;
  }
  return false;
}

bool mul_overflows(uint64_t a, uint64_t b) { return b != 0 && a > UINT64_MAX / b; }

gc_status check_ranks(int nranks) {
  if (nranks < 1) return GC_ERR_INVALID_ARG;
  if (nranks > GC_MAX_RANKS) return GC_ERR_UNSUPPORTED;
  return GC_OK;
}

// n non-null pointers aligned to the element size, each holding `bytes` bytes.
gc_status check_ptrs(const void* const* p, int n, size_t es, uint64_t bytes) {
  if (!p) return GC_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (!p[i] || addr(p[i]) % es || !fits(p[i], bytes)) return GC_ERR_INVALID_ARG;
  return GC_OK;
}

// Store policy of each use of the segment copy (measured on MI355X in one
// process on the same buffers).  Device-scope stores speed up these one-stream
// copies: the 8-rank MoE all-to-all went from 677 to 653 us (659 without the
// non-temporal hint).  The pack leaves out the hint so that the bucket can stay
// in the MALL for the all-reduce that reads it next: the 226-bucket DDP step
// went from 102.4 to 95.6 ms (99.4 with the hint; the unpack's choice moved it
// by 0.3 %).
#ifndef GC_A2A_STORE
#define GC_A2A_STORE gci::kStoreDevNT
#endif
#ifndef GC_PACK_STORE
#define GC_PACK_STORE gci::kStoreDev
#endif
#ifndef GC_UNPACK_STORE
#define GC_UNPACK_STORE gci::kStoreDevNT
#endif
constexpr gci::StorePolicy kA2aStore = GC_A2A_STORE;
constexpr gci::StorePolicy kPackStore = GC_PACK_STORE;
constexpr gci::StorePolicy kUnpackStore = GC_UNPACK_STORE;

#define GC_TRY(expr)                    \
  do {                                  \
    const gc_status _s = (expr);        \
    if (_s != GC_OK) return _s;         \
  } while (0)

// ------------------------------------------------------------ GC_DEBUG checks
// With GC_DEBUG set to a value other than "0" in the environment, every launch
// first checks the tables the host planners built for it: copy segments write
// disjoint ranges and none of them reads what another writes; a bucket's
// pieces cover each tensor exactly once, in owner-chunk order, with a valid
// fold start.  These are invariants of the library's own planning (arguments
// were validated before), so a failure is a library bug: it is reported on
// stderr and the call returns GC_ERR_INVALID_ARG with nothing launched.

bool debug_on() {
  static const bool on = [] {
    const char* v = std::getenv("GC_DEBUG");
    return v && *v && !(v[0] == '0' && v[1] == 0);
  }();
  return on;
}

gc_status debug_fail(const char* what) {
  std::fprintf(stderr, "libgc GC_DEBUG: %s\n", what);
  return GC_ERR_INVALID_ARG;
}

gc_status debug_segments(const gci::Segment* segs, size_t n) {
  if (!debug_on()) return GC_OK;
  std::vector<Span> dst, src;
  for (size_t i = 0; i < n; ++i) {
    if (!segs[i].bytes || !segs[i].dst) return debug_fail("empty or null copy segment");
    if (!fits(segs[i].dst, segs[i].bytes) || (segs[i].src && !fits(segs[i].src, segs[i].bytes)))
      return debug_fail("copy segment wraps the address space");
    dst.push_back(span(segs[i].dst, segs[i].bytes));
    if (segs[i].src) src.push_back(span(segs[i].src, segs[i].bytes));
  }
  if (any_overlap(dst)) return debug_fail("two copy segments write overlapping ranges");
  for (const Span& d : dst)
    for (const Span& r : src)
      if (overlaps(d, r)) return debug_fail("a copy segment writes what another reads");
  return GC_OK;
}

}  // namespace

// --------------------------------------------------------------------- status

extern "C" const char* gc_status_string(gc_status s) {
  switch (s) {
    case GC_OK: return "GC_OK";
    case GC_ERR_INVALID_ARG: return "GC_ERR_INVALID_ARG";
    case GC_ERR_UNSUPPORTED: return "GC_ERR_UNSUPPORTED";
    case GC_ERR_HIP: return "GC_ERR_HIP";
    case GC_ERR_NO_MEMORY: return "GC_ERR_NO_MEMORY";
  }
  return "GC_ERR_UNKNOWN";
}

extern "C" int gc_version(void) { return 100; }

namespace {
thread_local int g_last_hip_error = 0;
}  // namespace

gc_status gci::hip_status(hipError_t e) {
  if (e == hipSuccess) return GC_OK;
  g_last_hip_error = static_cast<int>(e);
  return GC_ERR_HIP;
}

extern "C" int gc_last_hip_error(void) { return g_last_hip_error; }

// ------------------------------------------------------------- reduce-scatter

extern "C" gc_status gc_reduce_scatter(const void* const* send, void* const* recv, size_t recv_count,
                                       int nranks, gc_dtype in_t, gc_dtype out_t, gc_op op,
                                       gc_order order, hipStream_t stream) {
  GC_TRY(check_ranks(nranks));
  if (!valid_dtype(in_t) || !valid_dtype(out_t) || !valid_op(op) || !valid_order(order) || !send || !recv)
    return GC_ERR_INVALID_ARG;
  if ((in_t == GC_INT32) != (out_t == GC_INT32)) return GC_ERR_UNSUPPORTED;
  if (op == GC_AVG && in_t == GC_INT32) return GC_ERR_UNSUPPORTED;
  const uint64_t N = static_cast<uint64_t>(nranks);
  if (mul_overflows(recv_count, N) || mul_overflows(recv_count * N, 4)) return GC_ERR_INVALID_ARG;
  if (recv_count == 0) return GC_OK;
  const size_t ei = elem_bytes(in_t), eo = elem_bytes(out_t);
  GC_TRY(check_ptrs(send, nranks, ei, N * recv_count * ei));
  GC_TRY(check_ptrs(const_cast<const void* const*>(recv), nranks, eo, recv_count * eo));

  // Aliasing: recv[r] may sit exactly on chunk r of send[r] when types match;
  // recv spans must not overlap each other nor any other part of any send.
  std::vector<Span> outs;
  for (int r = 0; r < nranks; ++r) outs.push_back(span(recv[r], recv_count * eo));
  if (any_overlap(outs)) return GC_ERR_INVALID_ARG;
  for (int r = 0; r < nranks; ++r) {
    const bool in_place = in_t == out_t && addr(recv[r]) == addr(send[r]) + r * recv_count * ei;
    for (int i = 0; i < nranks; ++i) {
      const Span in = span(send[i], N * recv_count * ei);
      if (!overlaps(outs[r], in)) continue;
      if (in_place && i == r) continue;
      return GC_ERR_INVALID_ARG;
    }
  }
  gci::ReduceCall c{send, recv, nranks, N * recv_count, recv_count, in_t, out_t,
                    op == GC_AVG, order != GC_ORDER_RANK, stream};
  c.wire = order == GC_ORDER_RING_WIRE;
  return gci::launch_reduce_scatter(c);
}

// ----------------------------------------------------------------- all-gather

extern "C" gc_status gc_all_gather(const void* const* send, void* const* recv, size_t count, int nranks,
                                   gc_dtype t, hipStream_t stream) {
  GC_TRY(check_ranks(nranks));
  if (!valid_dtype(t) || !send || !recv) return GC_ERR_INVALID_ARG;
  const uint64_t N = static_cast<uint64_t>(nranks);
  if (mul_overflows(count, N) || mul_overflows(count * N, 4)) return GC_ERR_INVALID_ARG;
  if (count == 0) return GC_OK;
  const size_t es = elem_bytes(t);
  GC_TRY(check_ptrs(send, nranks, es, count * es));
  GC_TRY(check_ptrs(const_cast<const void* const*>(recv), nranks, es, N * count * es));

  // Aliasing: send[r] may sit exactly on slot r of recv[r]; otherwise no overlap.
  std::vector<Span> outs;
  for (int r = 0; r < nranks; ++r) outs.push_back(span(recv[r], N * count * es));
  if (any_overlap(outs)) return GC_ERR_INVALID_ARG;
  for (int i = 0; i < nranks; ++i) {
    const Span in = span(send[i], count * es);
    const bool in_place = addr(send[i]) == addr(recv[i]) + i * count * es;
    for (int r = 0; r < nranks; ++r) {
      if (!overlaps(outs[r], in)) continue;
      if (in_place && r == i) continue;
      return GC_ERR_INVALID_ARG;
    }
  }
  gci::ReduceCall c{send, recv, nranks, N * count, count, t, t, false, false, stream};
  return gci::launch_all_gather(c);
}

// ----------------------------------------------------------------- all-reduce

namespace {

uint64_t chunk_len(uint64_t count, int nranks) { return (count + nranks - 1) / nranks; }

}  // namespace

extern "C" size_t gc_all_reduce_scratch_bytes(size_t count, int nranks, gc_dtype t, gc_ar_algo algo) {
  if (algo != GC_AR_RS_AG || !valid_dtype(t) || nranks < 1) return 0;
  if (mul_overflows(count, 4)) return 0;
  return (count * elem_bytes(t) + 255) / 256 * 256;
}

extern "C" gc_status gc_all_reduce(const void* const* send, void* const* recv, size_t count, int nranks,
                                   gc_dtype t, gc_op op, gc_order order, gc_ar_algo algo, void* scratch,
                                   size_t scratch_bytes, hipStream_t stream) {
  GC_TRY(check_ranks(nranks));
  if (!valid_dtype(t) || !valid_op(op) || !valid_order(order) || !send || !recv) return GC_ERR_INVALID_ARG;
  if (algo != GC_AR_FUSED && algo != GC_AR_RS_AG) return GC_ERR_INVALID_ARG;
  if (op == GC_AVG && t == GC_INT32) return GC_ERR_UNSUPPORTED;
  if (mul_overflows(count, 4)) return GC_ERR_INVALID_ARG;
  if (count == 0) return GC_OK;
  const size_t es = elem_bytes(t);
  const uint64_t bytes = count * es;
  GC_TRY(check_ptrs(send, nranks, es, bytes));
  GC_TRY(check_ptrs(const_cast<const void* const*>(recv), nranks, es, bytes));

  // Aliasing: each recv[r] is disjoint from every send[i] or equal to it.
  std::vector<Span> outs;
  for (int r = 0; r < nranks; ++r) outs.push_back(span(recv[r], bytes));
  if (any_overlap(outs)) return GC_ERR_INVALID_ARG;
  for (int r = 0; r < nranks; ++r)
    for (int i = 0; i < nranks; ++i)
      if (overlaps(outs[r], span(send[i], bytes)) && addr(recv[r]) != addr(send[i])) return GC_ERR_INVALID_ARG;

  const uint64_t c = chunk_len(count, nranks);
  if (algo == GC_AR_FUSED) {
    gci::ReduceCall call{send, recv, nranks, count, c, t, t, op == GC_AVG, order != GC_ORDER_RANK, stream};
    call.wire = order == GC_ORDER_RING_WIRE;
    return gci::launch_all_reduce(call);
  }

  if (!scratch || addr(scratch) % es || scratch_bytes < gc_all_reduce_scratch_bytes(count, nranks, t, algo) ||
      !fits(scratch, scratch_bytes))
    return GC_ERR_INVALID_ARG;
  const Span sc = span(scratch, bytes);
  for (int r = 0; r < nranks; ++r)
    if (overlaps(sc, outs[r]) || overlaps(sc, span(send[r], bytes))) return GC_ERR_INVALID_ARG;

  // Owner chunk j lives at scratch + j*c elements: reduce-scatter writes it
  // (averaged and rounded), all-gather reads it back out to every rank.
  std::vector<void*> shard_out(nranks);
  std::vector<const void*> shard_in(nranks);
  for (int j = 0; j < nranks; ++j) {
    const uint64_t lo = std::min<uint64_t>(count, static_cast<uint64_t>(j) * c);
    shard_out[j] = at(scratch, lo * es);
    shard_in[j] = shard_out[j];
  }
  gci::ReduceCall rs{send, shard_out.data(), nranks, count, c, t, t, op == GC_AVG, order != GC_ORDER_RANK, stream};
  rs.wire = order == GC_ORDER_RING_WIRE;
  GC_TRY(gci::launch_reduce_scatter(rs));
  gci::ReduceCall ag{shard_in.data(), recv, nranks, count, c, t, t, false, false, stream};
  return gci::launch_all_gather(ag);
}

// ----------------------------------------------------------------- all-to-all

extern "C" gc_status gc_all_to_all(const void* const* send, void* const* recv, const int64_t* splits,
                                   int nranks, int experts_per_rank, size_t row_bytes, hipStream_t stream) {
  GC_TRY(check_ranks(nranks));
  if (!send || !recv || !splits || experts_per_rank < 1 || row_bytes == 0) return GC_ERR_INVALID_ARG;
  const int N = nranks, E = experts_per_rank;
  if (static_cast<int64_t>(N) * N * E > (int64_t(1) << 24)) return GC_ERR_UNSUPPORTED;

  std::vector<int64_t> send_rows(N, 0), recv_rows(N, 0);
  for (int s = 0; s < N; ++s)
    for (int d = 0; d < N; ++d)
      for (int e = 0; e < E; ++e) {
        const int64_t v = splits[(static_cast<int64_t>(s) * N + d) * E + e];
        if (v < 0) return GC_ERR_INVALID_ARG;
        send_rows[s] += v;
        recv_rows[d] += v;
        if (send_rows[s] >= (int64_t(1) << 31) || recv_rows[d] >= (int64_t(1) << 31)) return GC_ERR_UNSUPPORTED;
      }
  int64_t total = 0;
  for (int s = 0; s < N; ++s) total += send_rows[s];
  if (total >= (int64_t(1) << 31)) return GC_ERR_UNSUPPORTED;
  for (int s = 0; s < N; ++s)
    if (mul_overflows(static_cast<uint64_t>(send_rows[s]), row_bytes) ||
        mul_overflows(static_cast<uint64_t>(recv_rows[s]), row_bytes))
      return GC_ERR_INVALID_ARG;
  if (total == 0) return GC_OK;

  std::vector<Span> all;
  for (int r = 0; r < N; ++r) {
    if ((send_rows[r] && !send[r]) || (recv_rows[r] && !recv[r])) return GC_ERR_INVALID_ARG;
    if (!fits(send[r], send_rows[r] * row_bytes) || !fits(recv[r], recv_rows[r] * row_bytes))
      return GC_ERR_INVALID_ARG;
    all.push_back(span(recv[r], recv_rows[r] * row_bytes));
  }
  if (any_overlap(all)) return GC_ERR_INVALID_ARG;
  for (int r = 0; r < N; ++r)
    for (int s = 0; s < N; ++s)
      if (overlaps(all[r], span(send[s], send_rows[s] * row_bytes))) return GC_ERR_INVALID_ARG;
  if (mul_overflows(static_cast<uint64_t>(total), row_bytes) || static_cast<uint64_t>(total) * row_bytes > kMaxCopyBytes)
    return GC_ERR_UNSUPPORTED;

  // Every (s, d, e) block is contiguous in send[s] and in recv[d]: the
  // all-to-all is one contiguous copy per non-empty block, done by the
  // segment-copy kernel in equal-byte tiles across blocks.
  std::vector<int64_t> roff(static_cast<size_t>(N) * N * E, 0);
  for (int d = 0; d < N; ++d) {
    int64_t run = 0;
    for (int e = 0; e < E; ++e)
      for (int s = 0; s < N; ++s) {
        const size_t b = (static_cast<size_t>(s) * N + d) * E + e;
        roff[b] = run;
        run += splits[b];
      }
  }
  std::vector<gci::Segment> segs;
  for (int s = 0; s < N; ++s) {
    int64_t run = 0;
    for (int d = 0; d < N; ++d)
      for (int e = 0; e < E; ++e) {
        const size_t b = (static_cast<size_t>(s) * N + d) * E + e;
        const int64_t v = splits[b];
        if (v)
          segs.push_back(gci::Segment{at(send[s], run * row_bytes), at(recv[d], roff[b] * row_bytes),
                                      v * row_bytes});
        run += v;
      }
  }
  GC_TRY(debug_segments(segs.data(), segs.size()));
  return gci::launch_segment_copy(segs.data(), segs.size(), kA2aStore, stream);
}

// ------------------------------------------------------- two-level / HSDP

namespace {

gc_status check_mesh(int nranks, int group_size) {
  GC_TRY(check_ranks(nranks));
  if (group_size < 1 || nranks % group_size) return GC_ERR_INVALID_ARG;
  return GC_OK;
}

}  // namespace

extern "C" gc_status gc_hier_all_reduce(const void* const* send, void* const* recv, size_t count, int nranks,
                                        int group_size, gc_dtype t, gc_op op, gc_order order, hipStream_t stream) {
  if (!valid_dtype(t) || !valid_op(op) || !valid_order(order) || !send || !recv) return GC_ERR_INVALID_ARG;
  GC_TRY(check_mesh(nranks, group_size));
  if (op == GC_AVG && t == GC_INT32) return GC_ERR_UNSUPPORTED;
  if (mul_overflows(count, 4)) return GC_ERR_INVALID_ARG;
  if (count == 0) return GC_OK;
  const size_t es = elem_bytes(t);
  const uint64_t bytes = count * es;
  GC_TRY(check_ptrs(send, nranks, es, bytes));
  GC_TRY(check_ptrs(const_cast<const void* const*>(recv), nranks, es, bytes));
  // Aliasing as gc_all_reduce: each recv[r] is disjoint from every send[i] or equal to it.
  std::vector<Span> outs;
  for (int r = 0; r < nranks; ++r) outs.push_back(span(recv[r], bytes));
  if (any_overlap(outs)) return GC_ERR_INVALID_ARG;
  for (int r = 0; r < nranks; ++r)
    for (int i = 0; i < nranks; ++i)
      if (overlaps(outs[r], span(send[i], bytes)) && addr(recv[r]) != addr(send[i])) return GC_ERR_INVALID_ARG;
  gci::HierCall call{send, recv, nranks, group_size, count, t, t, op == GC_AVG, order != GC_ORDER_RANK, stream};
  call.wire = order == GC_ORDER_RING_WIRE;
  return gci::launch_hier_all_reduce(call);
}

extern "C" gc_status gc_hsdp_reduce_scatter(const void* const* send, void* const* recv, size_t recv_count,
                                            int nranks, int group_size, gc_dtype in_t, gc_dtype out_t, gc_op op,
                                            gc_order order, hipStream_t stream) {
  if (!valid_dtype(in_t) || !valid_dtype(out_t) || !valid_op(op) || !valid_order(order) || !send || !recv)
    return GC_ERR_INVALID_ARG;
  GC_TRY(check_mesh(nranks, group_size));
  if ((in_t == GC_INT32) != (out_t == GC_INT32)) return GC_ERR_UNSUPPORTED;
  if (op == GC_AVG && in_t == GC_INT32) return GC_ERR_UNSUPPORTED;
  const uint64_t S = static_cast<uint64_t>(group_size);
  if (mul_overflows(recv_count, S) || mul_overflows(recv_count * S, 4)) return GC_ERR_INVALID_ARG;
  if (recv_count == 0) return GC_OK;
  const size_t ei = elem_bytes(in_t), eo = elem_bytes(out_t);
  GC_TRY(check_ptrs(send, nranks, ei, S * recv_count * ei));
  GC_TRY(check_ptrs(const_cast<const void* const*>(recv), nranks, eo, recv_count * eo));
  // Aliasing: recv[r] may sit exactly on member i's chunk of send[r] (i = r mod
  // group) when the types match; no other overlap.
  std::vector<Span> outs;
  for (int r = 0; r < nranks; ++r) outs.push_back(span(recv[r], recv_count * eo));
  if (any_overlap(outs)) return GC_ERR_INVALID_ARG;
  for (int r = 0; r < nranks; ++r) {
    const uint64_t i = static_cast<uint64_t>(r % group_size);
    const bool in_place = in_t == out_t && addr(recv[r]) == addr(send[r]) + i * recv_count * ei;
    for (int q = 0; q < nranks; ++q) {
      if (!overlaps(outs[r], span(send[q], S * recv_count * ei))) continue;
      if (in_place && q == r) continue;
      return GC_ERR_INVALID_ARG;
    }
  }
  gci::HierCall call{send, recv, nranks, group_size, S * recv_count, in_t, out_t, op == GC_AVG,
                     order != GC_ORDER_RANK, stream};
  call.wire = order == GC_ORDER_RING_WIRE;
  return gci::launch_hsdp_reduce_scatter(call);
}

// ------------------------------------------------------------- FSDP2 Shard(0)

namespace {

// Rows of rank r's dim-0 shard of a parameter with `rows` rows (torch.chunk rule).
struct RowShard {
  uint64_t lo, hi;
};

RowShard row_shard(uint64_t rows, int nranks, int r) {
  const uint64_t c = (rows + nranks - 1) / nranks;
  return RowShard{std::min<uint64_t>(rows, r * c), std::min<uint64_t>(rows, (r + 1) * c)};
}

// A buffer of parameter p on rank r; `in_place` marks an output that may hold
// the same (p, r) input inside it (or sit inside it) at the shard's offset.
struct Tagged {
  Span s;
  int p, r;
  bool in_place;
};

// True if two outputs overlap, or an output overlaps an input other than its
// own in-place partner.  Outputs are sorted once; each input is matched
// against the outputs it can reach by binary search.
bool tagged_conflict(const std::vector<Tagged>& outs, const std::vector<Tagged>& ins) {
  std::vector<Span> os;
  std::vector<Tagged> sorted;
  for (const Tagged& o : outs) {
    os.push_back(o.s);
    if (!o.s.empty()) sorted.push_back(o);
  }
  if (any_overlap(os)) return true;
  std::sort(sorted.begin(), sorted.end(), [](const Tagged& a, const Tagged& b) { return a.s.lo < b.s.lo; });
  for (const Tagged& i : ins) {
    if (i.s.empty()) continue;
    // Disjoint outputs sorted by start are sorted by end too: skip those ending at or before i.lo.
    auto it = std::partition_point(sorted.begin(), sorted.end(), [&](const Tagged& o) { return o.s.hi <= i.s.lo; });
    for (; it != sorted.end() && it->s.lo < i.s.hi; ++it) {
      if (it->in_place && it->p == i.p && it->r == i.r) continue;
      return true;
    }
  }
  return false;
}

// Shared checks of the per-parameter calls.  full[r * P + p] holds rows[p] *
// cols[p] elements of es_full bytes, part[r * P + p] rank r's shard of es_part
// bytes (NULL allowed when empty).  `outputs_are_parts` picks which side is
// written; with `in_place_ok` a shard may sit exactly at its offset inside
// the same rank's full buffer.
gc_status fsdp2_check(const void* const* full, const void* const* part, const size_t* rows, const size_t* cols,
                      int P, int N, size_t es_full, size_t es_part, bool outputs_are_parts, bool in_place_ok) {
  GC_TRY(check_ranks(N));
  if (!full || !part || !rows || !cols || P < 0) return GC_ERR_INVALID_ARG;
  std::vector<Tagged> outs, ins;
  for (int p = 0; p < P; ++p) {
    if (mul_overflows(rows[p], cols[p]) || mul_overflows(rows[p] * cols[p], 4)) return GC_ERR_INVALID_ARG;
    const uint64_t S = rows[p] * cols[p];
    if (S == 0) continue;
    for (int r = 0; r < N; ++r) {
      const void* f = full[static_cast<size_t>(r) * P + p];
      const void* q = part[static_cast<size_t>(r) * P + p];
      const RowShard sh = row_shard(rows[p], N, r);
      const uint64_t n = (sh.hi - sh.lo) * cols[p];
      if (!f || addr(f) % es_full || !fits(f, S * es_full)) return GC_ERR_INVALID_ARG;
      if (n && (!q || addr(q) % es_part || !fits(q, n * es_part))) return GC_ERR_INVALID_ARG;
      const bool in_place = in_place_ok && n && addr(q) == addr(f) + sh.lo * cols[p] * es_full;
      const Tagged ft{span(f, S * es_full), p, r, in_place};
      const Tagged qt{span(n ? q : nullptr, n * es_part), p, r, in_place};
      (outputs_are_parts ? outs : ins).push_back(qt);
      (outputs_are_parts ? ins : outs).push_back(ft);
    }
  }
  return tagged_conflict(outs, ins) ? GC_ERR_INVALID_ARG : GC_OK;
}

}  // namespace

extern "C" gc_status gc_fsdp2_reduce_scatter(const void* const* grads, void* const* shards, const size_t* rows,
                                             const size_t* cols, int nparams, int nranks, gc_dtype in_t,
                                             gc_dtype out_t, gc_op op, gc_order order, hipStream_t stream) {
  GC_TRY(check_ranks(nranks));
  if (!valid_dtype(in_t) || !valid_dtype(out_t) || !valid_op(op) || !valid_order(order)) return GC_ERR_INVALID_ARG;
  if ((in_t == GC_INT32) != (out_t == GC_INT32)) return GC_ERR_UNSUPPORTED;
  if (op == GC_AVG && in_t == GC_INT32) return GC_ERR_UNSUPPORTED;
  const size_t ei = elem_bytes(in_t), eo = elem_bytes(out_t);
  GC_TRY(fsdp2_check(grads, const_cast<const void* const*>(shards), rows, cols, nparams, nranks, ei, eo, true,
                     in_t == out_t));
  const int N = nranks, P = nparams;
  std::vector<const void*> in(N);
  std::vector<void*> out(N);
  for (int p = 0; p < P; ++p) {
    const uint64_t S = rows[p] * cols[p];
    if (S == 0) continue;
    for (int r = 0; r < N; ++r) {
      in[r] = grads[static_cast<size_t>(r) * P + p];
      out[r] = shards[static_cast<size_t>(r) * P + p];
    }
    const uint64_t c = (rows[p] + N - 1) / N * cols[p];
    gci::ReduceCall call{in.data(), out.data(), N, S, c, in_t, out_t, op == GC_AVG, order != GC_ORDER_RANK, stream};
    call.wire = order == GC_ORDER_RING_WIRE;
    GC_TRY(gci::launch_reduce_scatter(call));
  }
  return GC_OK;
}

extern "C" gc_status gc_fsdp2_all_gather(const void* const* shards, void* const* params, const size_t* rows,
                                         const size_t* cols, int nparams, int nranks, gc_dtype t,
                                         hipStream_t stream) {
  GC_TRY(check_ranks(nranks));
  if (!valid_dtype(t)) return GC_ERR_INVALID_ARG;
  const size_t es = elem_bytes(t);
  GC_TRY(fsdp2_check(const_cast<const void* const*>(params), shards, rows, cols, nparams, nranks, es, es, false,
                     true));
  const int N = nranks, P = nparams;
  std::vector<const void*> in(N);
  std::vector<void*> out(N);
  for (int p = 0; p < P; ++p) {
    const uint64_t S = rows[p] * cols[p];
    if (S == 0) continue;
    for (int r = 0; r < N; ++r) {
      in[r] = shards[static_cast<size_t>(r) * P + p];
      out[r] = params[static_cast<size_t>(r) * P + p];
    }
    const uint64_t c = (rows[p] + N - 1) / N * cols[p];
    gci::ReduceCall call{in.data(), out.data(), N, S, c, t, t, false, false, stream};
    GC_TRY(gci::launch_all_gather(call));
  }
  return GC_OK;
}

// ------------------------------------------------------------------------ MoE

namespace {

constexpr int kMoeMaxTopk = 8;
constexpr int kMoeMaxBins = 8192;

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// Tiling of the routing plan: routes per tile, total tiles, scratch bytes.
struct MoeRouteGeom {
  int32_t tile = 0;
  int64_t tiles = 0;
  int64_t routes = 0;
  uint64_t counts_bytes = 0;
  uint64_t bytes = 0;
};

gc_status moe_route_geom(const int64_t* ntokens, int nranks, int topk, int E, MoeRouteGeom& g) {
  GC_TRY(check_ranks(nranks));
  if (!ntokens || topk < 1 || E < 1) return GC_ERR_INVALID_ARG;
  if (topk > kMoeMaxTopk || static_cast<int64_t>(nranks) * E > kMoeMaxBins) return GC_ERR_UNSUPPORTED;
  const int64_t nbins = static_cast<int64_t>(nranks) * E;
  // Tiles of kMoeRouteTile routes (four wavefronts) while the experts fit;
  // beyond, one wavefront per tile of at least one route per expert.
  g.tile = static_cast<int32_t>(std::max<int64_t>(gci::kMoeRouteTile, (nbins + 63) / 64 * 64));
  for (int s = 0; s < nranks; ++s) {
    if (ntokens[s] < 0) return GC_ERR_INVALID_ARG;
    if (ntokens[s] >= (int64_t(1) << 31)) return GC_ERR_UNSUPPORTED;
    const int64_t r = ntokens[s] * topk;
    g.routes += r;
    if (g.routes >= (int64_t(1) << 31)) return GC_ERR_UNSUPPORTED;
    g.tiles += (r + g.tile - 1) / g.tile;
  }
  g.counts_bytes = align256(static_cast<uint64_t>(g.tiles) * nbins * 4);
  g.bytes = g.counts_bytes + align256(static_cast<uint64_t>(nbins) * nranks * 4);
  return GC_OK;
}

}  // namespace

extern "C" size_t gc_moe_route_scratch_bytes(const int64_t* ntokens, int nranks, int topk, int experts_per_rank) {
  MoeRouteGeom g;
  return moe_route_geom(ntokens, nranks, topk, experts_per_rank, g) == GC_OK ? g.bytes : 0;
}

namespace {

// Checks shared by gc_moe_route and gc_moe_route_noalloc; the scratch span is
// empty for the variant whose scratch is the library's own.  Nothing here
// allocates (fixed-size span lists: at most 2 + nranks outputs and nranks
// inputs), so the variant without a scratch argument allocates nothing at all.
gc_status moe_route_check(const int32_t* const* experts, const int64_t* ntokens, int nranks, int topk,
                          int experts_per_rank, const int64_t* splits, int32_t* const* dest, Span scratch) {
  const int N = nranks, E = experts_per_rank;
  if (!experts || !dest || !splits || addr(splits) % 8) return GC_ERR_INVALID_ARG;
  if (!fits(splits, static_cast<uint64_t>(N) * N * E * 8)) return GC_ERR_INVALID_ARG;
  Span outs[GC_MAX_RANKS + 2], ins[GC_MAX_RANKS];
  int nout = 0, nin = 0;
  outs[nout++] = span(splits, static_cast<uint64_t>(N) * N * E * 8);
  outs[nout++] = scratch;
  for (int s = 0; s < N; ++s) {
    const int64_t routes = ntokens[s] * topk;
    if (!routes) continue;
    if (!experts[s] || addr(experts[s]) % 4 || !dest[s] || addr(dest[s]) % 8) return GC_ERR_INVALID_ARG;
    if (!fits(experts[s], routes * 4) || !fits(dest[s], routes * 8)) return GC_ERR_INVALID_ARG;
    ins[nin++] = span(experts[s], routes * 4);
    outs[nout++] = span(dest[s], routes * 8);
  }
  std::sort(outs, outs + nout, [](const Span& a, const Span& b) { return a.lo < b.lo; });
  for (int k = 1; k < nout; ++k)
    if (overlaps(outs[k - 1], outs[k])) return GC_ERR_INVALID_ARG;  // sorted: any overlap shows between neighbours
  for (int o = 0; o < nout; ++o)
    for (int i = 0; i < nin; ++i)
      if (overlaps(outs[o], ins[i])) return GC_ERR_INVALID_ARG;
  return GC_OK;
}

gc_status moe_route_launch(const int32_t* const* experts, const int64_t* ntokens, int nranks, int topk,
                           int experts_per_rank, int64_t* splits, int32_t* const* dest, void* scratch,
                           const MoeRouteGeom& g, hipStream_t stream) {
  int64_t routes[GC_MAX_RANKS];
  for (int s = 0; s < nranks; ++s) routes[s] = ntokens[s] * topk;
  char* base = static_cast<char*>(scratch);
  gci::MoeRouteCall call{experts, dest, routes, nranks, experts_per_rank, g.tile,
                         reinterpret_cast<int32_t*>(base), reinterpret_cast<int32_t*>(base + g.counts_bytes),
                         splits, stream};
  return gci::launch_moe_route(call);
}

}  // namespace

extern "C" gc_status gc_moe_route(const int32_t* const* experts, const int64_t* ntokens, int nranks, int topk,
                                  int experts_per_rank, int64_t* splits, int32_t* const* dest, void* scratch,
                                  size_t scratch_bytes, hipStream_t stream) {
  MoeRouteGeom g;
  GC_TRY(moe_route_geom(ntokens, nranks, topk, experts_per_rank, g));
  if (!scratch || addr(scratch) % 256 || scratch_bytes < g.bytes || !fits(scratch, scratch_bytes))
    return GC_ERR_INVALID_ARG;
  GC_TRY(moe_route_check(experts, ntokens, nranks, topk, experts_per_rank, splits, dest, span(scratch, g.bytes)));
  return moe_route_launch(experts, ntokens, nranks, topk, experts_per_rank, splits, dest, scratch, g, stream);
}

extern "C" gc_status gc_moe_route_noalloc(const int32_t* const* experts, const int64_t* ntokens, int nranks,
                                          int topk, int experts_per_rank, int64_t* splits, int32_t* const* dest,
                                          hipStream_t stream) {
  MoeRouteGeom g;
  GC_TRY(moe_route_geom(ntokens, nranks, topk, experts_per_rank, g));
  if (g.bytes > GC_MOE_ROUTE_NOALLOC_SCRATCH_BYTES) return GC_ERR_UNSUPPORTED;
  GC_TRY(moe_route_check(experts, ntokens, nranks, topk, experts_per_rank, splits, dest, Span{0, 0}));
  void* scratch = nullptr;
  GC_TRY(gci::moe_route_static_scratch(stream, &scratch));
  return moe_route_launch(experts, ntokens, nranks, topk, experts_per_rank, splits, dest, scratch, g, stream);
}

namespace {

// Checks shared by dispatch and combine: row buffers of src (src_rows each),
// dst (dst_rows each) and the per-source route tables.
gc_status moe_move_check(const void* const* src, const int64_t* src_rows, void* const* dst, const int64_t* dst_rows,
                         const int32_t* const* dest, const float* const* weights, const int64_t* ntokens,
                         int nranks, int topk, uint64_t row_bytes) {
  GC_TRY(check_ranks(nranks));
  if (!src || !src_rows || !dst || !dst_rows || !dest || !ntokens || topk < 1 || row_bytes == 0)
    return GC_ERR_INVALID_ARG;
  if (topk > kMoeMaxTopk) return GC_ERR_UNSUPPORTED;
  std::vector<Span> outs, ins;
  int64_t routes = 0;
  for (int r = 0; r < nranks; ++r) {
    if (ntokens[r] < 0 || src_rows[r] < 0 || dst_rows[r] < 0) return GC_ERR_INVALID_ARG;
    if (ntokens[r] >= (int64_t(1) << 31) || src_rows[r] >= (int64_t(1) << 31) || dst_rows[r] >= (int64_t(1) << 31))
      return GC_ERR_UNSUPPORTED;
    routes += ntokens[r] * topk;
    if (routes >= (int64_t(1) << 31)) return GC_ERR_UNSUPPORTED;
    if (mul_overflows(static_cast<uint64_t>(src_rows[r]), row_bytes) ||
        mul_overflows(static_cast<uint64_t>(dst_rows[r]), row_bytes))
      return GC_ERR_INVALID_ARG;
    if ((src_rows[r] && !src[r]) || (dst_rows[r] && !dst[r])) return GC_ERR_INVALID_ARG;
    if (!fits(src[r], src_rows[r] * row_bytes) || !fits(dst[r], dst_rows[r] * row_bytes)) return GC_ERR_INVALID_ARG;
    outs.push_back(span(dst[r], dst_rows[r] * row_bytes));
    ins.push_back(span(src[r], src_rows[r] * row_bytes));
    if (ntokens[r]) {
      if (!dest[r] || addr(dest[r]) % 8 || !fits(dest[r], ntokens[r] * topk * 8)) return GC_ERR_INVALID_ARG;
      ins.push_back(span(dest[r], ntokens[r] * topk * 8));
      if (weights) {
        if (!weights[r] || addr(weights[r]) % 4 || !fits(weights[r], ntokens[r] * topk * 4)) return GC_ERR_INVALID_ARG;
        ins.push_back(span(weights[r], ntokens[r] * topk * 4));
      }
    }
  }
  if (any_overlap(outs)) return GC_ERR_INVALID_ARG;
  for (const Span& o : outs)
    for (const Span& i : ins)
      if (overlaps(o, i)) return GC_ERR_INVALID_ARG;
  return GC_OK;
}

}  // namespace

extern "C" gc_status gc_moe_dispatch(const void* const* tokens, const int64_t* ntokens, const int32_t* const* dest,
                                     int nranks, int topk, size_t row_bytes, void* const* recv,
                                     const int64_t* recv_rows, hipStream_t stream) {
  GC_TRY(moe_move_check(tokens, ntokens, recv, recv_rows, dest, nullptr, ntokens, nranks, topk, row_bytes));
  gci::MoeMoveCall call{tokens, ntokens, dest, nullptr, recv, recv_rows, ntokens, nranks, topk, row_bytes,
                        GC_BF16, stream};
  return gci::launch_moe_dispatch(call);
}

extern "C" gc_status gc_moe_combine(const void* const* expert_out, const int64_t* expert_rows,
                                    const int32_t* const* dest, const float* const* weights,
                                    const int64_t* ntokens, int nranks, int topk, size_t hidden, gc_dtype t,
                                    void* const* out, hipStream_t stream) {
  if (!valid_dtype(t) || !weights) return GC_ERR_INVALID_ARG;
  if (t == GC_INT32) return GC_ERR_UNSUPPORTED;
  if (hidden == 0 || mul_overflows(hidden, elem_bytes(t))) return GC_ERR_INVALID_ARG;
  const uint64_t row_bytes = hidden * elem_bytes(t);
  GC_TRY(moe_move_check(expert_out, expert_rows, out, ntokens, dest, weights, ntokens, nranks, topk, row_bytes));
  for (int r = 0; r < nranks; ++r)
    if ((expert_rows[r] && addr(expert_out[r]) % elem_bytes(t)) || (ntokens[r] && addr(out[r]) % elem_bytes(t)))
      return GC_ERR_INVALID_ARG;
  gci::MoeMoveCall call{expert_out, expert_rows, dest, weights, out, ntokens, ntokens, nranks, topk, row_bytes,
                        t, stream};
  return gci::launch_moe_combine(call);
}

// ---------------------------------------------------------------- bucket plan

namespace {
// Largest padding multiple a plan accepts (FlatParameter pads to the rank count).
constexpr size_t kMaxPadTo = size_t(1) << 20;
}  // namespace

struct gc_bucket_plan {
  gc_dtype t;
  size_t es;
  std::vector<size_t> numel;
  std::vector<int> tensor_bucket;
  std::vector<size_t> tensor_offset;
  std::vector<std::vector<int>> buckets;  // tensor indices in packing order
  std::vector<size_t> used;               // elements of real data per bucket
  std::vector<size_t> padded;             // elements after zero padding
};

extern "C" gc_status gc_bucket_plan_create(const size_t* numels, int ntensors, gc_dtype t, size_t cap_bytes,
                                           int reverse, size_t pad_to, gc_bucket_plan** out) {
  if (!out) return GC_ERR_INVALID_ARG;
  *out = nullptr;
  if (ntensors < 0 || (ntensors > 0 && !numels) || !valid_dtype(t) || pad_to == 0 || pad_to > kMaxPadTo)
    return GC_ERR_INVALID_ARG;
  gc_bucket_plan* p = new (std::nothrow) gc_bucket_plan;
  if (!p) return GC_ERR_NO_MEMORY;
  try {
    p->t = t;
    p->es = elem_bytes(t);
    p->numel.assign(numels, numels + ntensors);
    p->tensor_bucket.assign(ntensors, -1);
    p->tensor_offset.assign(ntensors, 0);
    std::vector<int> cur;
    size_t cur_elems = 0;
    bool too_big = false;  // a bucket larger than any one GPU's buffer
    auto close = [&]() {
      size_t run = 0;
      for (int ti : cur) {
        p->tensor_bucket[ti] = static_cast<int>(p->buckets.size());
        p->tensor_offset[ti] = run;
        run += p->numel[ti];
      }
      p->buckets.push_back(cur);
      p->used.push_back(run);
      p->padded.push_back((run + pad_to - 1) / pad_to * pad_to);
      if (p->padded.back() * p->es > kMaxExtent) too_big = true;
      cur.clear();
      cur_elems = 0;
    };
    for (int k = 0; k < ntensors; ++k) {
      const int ti = reverse ? ntensors - 1 - k : k;
      // A bucket's bytes must stay representable: every size the plan hands out is
      // elements * element size (and padded up to pad_to elements).
      if (mul_overflows(p->numel[ti], 4) || cur_elems + p->numel[ti] < cur_elems ||
          mul_overflows(cur_elems + p->numel[ti] + pad_to, 4)) {
        delete p;
        return GC_ERR_INVALID_ARG;
      }
      cur.push_back(ti);
      cur_elems += p->numel[ti];
      if (cap_bytes != SIZE_MAX && cur_elems * p->es >= cap_bytes) close();
    }
    if (!cur.empty()) close();
    if (too_big) {
      delete p;
      return GC_ERR_INVALID_ARG;
    }
  } catch (const std::bad_alloc&) {
    delete p;
    return GC_ERR_NO_MEMORY;
  }
  *out = p;
  return GC_OK;
}

extern "C" gc_status gc_bucket_plan_query(const gc_bucket_plan* p, int* nbuckets, size_t* bucket_numel,
                                          int* tensor_bucket, size_t* tensor_offset) {
  if (!p) return GC_ERR_INVALID_ARG;
  if (nbuckets) *nbuckets = static_cast<int>(p->buckets.size());
  if (bucket_numel) std::copy(p->padded.begin(), p->padded.end(), bucket_numel);
  if (tensor_bucket) std::copy(p->tensor_bucket.begin(), p->tensor_bucket.end(), tensor_bucket);
  if (tensor_offset) std::copy(p->tensor_offset.begin(), p->tensor_offset.end(), tensor_offset);
  return GC_OK;
}

extern "C" void gc_bucket_plan_destroy(gc_bucket_plan* p) { delete p; }

namespace {

// Segments of one bucket for every rank; pack copies tensor -> bucket (plus
// zero padding), unpack copies bucket -> tensor.
gc_status bucket_segments(const gc_bucket_plan* p, int bucket, const void* const* tensors,
                          void* const* tensor_out, const void* const* bufs_in, void* const* bufs_out,
                          int nranks, bool packing, std::vector<gci::Segment>* segs) {
  GC_TRY(check_ranks(nranks));
  if (!p || bucket < 0 || bucket >= static_cast<int>(p->buckets.size())) return GC_ERR_INVALID_ARG;
  const size_t T = p->numel.size();
  const std::vector<int>& b = p->buckets[bucket];
  const size_t es = p->es;
  std::vector<Span> writes, reads;
  for (int r = 0; r < nranks; ++r) {
    const void* buf_r = packing ? static_cast<const void*>(bufs_out[r]) : bufs_in[r];
    if (p->padded[bucket] && (!buf_r || addr(buf_r) % es || !fits(buf_r, p->padded[bucket] * es)))
      return GC_ERR_INVALID_ARG;
    const Span bspan = span(buf_r, p->padded[bucket] * es);
    (packing ? writes : reads).push_back(bspan);
    for (int ti : b) {
      const size_t n = p->numel[ti];
      if (!n) continue;
      const void* tp = packing ? tensors[r * T + ti] : static_cast<const void*>(tensor_out[r * T + ti]);
      if (!tp || addr(tp) % es || !fits(tp, n * es)) return GC_ERR_INVALID_ARG;
      (packing ? reads : writes).push_back(span(tp, n * es));
      void* bb = at(buf_r, p->tensor_offset[ti] * es);
      if (packing) segs->push_back(gci::Segment{tp, bb, n * es});
      else segs->push_back(gci::Segment{bb, const_cast<void*>(tp), n * es});
    }
    if (packing && p->padded[bucket] > p->used[bucket])
      segs->push_back(gci::Segment{nullptr, at(bufs_out[r], p->used[bucket] * es),
                                   (p->padded[bucket] - p->used[bucket]) * es});
  }
  if (any_overlap(writes)) return GC_ERR_INVALID_ARG;
  for (const Span& w : writes)
    for (const Span& rd : reads)
      if (overlaps(w, rd)) return GC_ERR_INVALID_ARG;
  return GC_OK;
}

}  // namespace

extern "C" gc_status gc_bucket_all_reduce(const gc_bucket_plan* p, int bucket, void* const* tensors, int nranks,
                                          gc_op op, gc_order order, double* sumsq, hipStream_t stream) {
  GC_TRY(check_ranks(nranks));
  if (!p || !tensors || bucket < 0 || bucket >= static_cast<int>(p->buckets.size()) || !valid_op(op) ||
      !valid_order(order))
    return GC_ERR_INVALID_ARG;
  if (p->t == GC_INT32 && (op == GC_AVG || sumsq)) return GC_ERR_UNSUPPORTED;
  if (sumsq && (addr(sumsq) % 8 || !fits(sumsq, 8))) return GC_ERR_INVALID_ARG;
  const size_t T = p->numel.size();
  const size_t es = p->es;
  const std::vector<int>& b = p->buckets[bucket];
  const uint64_t count = p->padded[bucket];
  const uint64_t c = chunk_len(count, nranks);

  std::vector<Span> spans;
  std::vector<void*> slot_ptrs;
  std::vector<gci::BucketPiece> pieces;
  uint32_t slot = 0;
  for (int ti : b) {
    const uint64_t n = p->numel[ti];
    if (!n) continue;
    for (int r = 0; r < nranks; ++r) {
      void* tp = tensors[static_cast<size_t>(r) * T + ti];
      if (!tp || addr(tp) % es || !fits(tp, n * es)) return GC_ERR_INVALID_ARG;
      spans.push_back(span(tp, n * es));
      slot_ptrs.push_back(tp);
    }
    // the tensor's packed range [o, o + n) cut at owner-chunk boundaries
    const uint64_t o = p->tensor_offset[ti];
    for (uint64_t lo = o; lo < o + n;) {
      const uint64_t j = lo / c;
      const uint64_t hi = std::min(o + n, (j + 1) * c);
      const uint32_t first = order != GC_ORDER_RANK ? static_cast<uint32_t>((j + 1) % nranks) : 0u;
      pieces.push_back(gci::BucketPiece{lo - o, hi - lo, slot, first});
      lo = hi;
    }
    ++slot;
  }
  if (any_overlap(spans)) return GC_ERR_INVALID_ARG;
  if (sumsq) {
    const Span sq = span(sumsq, sizeof(double));
    for (const Span& t : spans)
      if (overlaps(sq, t)) return GC_ERR_INVALID_ARG;
  }
  if (debug_on()) {
    // pieces of each slot: consecutive, starting at 0, ending at the tensor's length, each inside one owner
    // chunk of the packed bucket and folded from that chunk's first rank
    size_t k = 0;
    uint32_t sl = 0;
    for (int ti : b) {
      const uint64_t n = p->numel[ti];
      if (!n) continue;
      uint64_t at_ = 0;
      for (; k < pieces.size() && pieces[k].slot == sl; ++k) {
        const gci::BucketPiece& pc = pieces[k];
        const uint64_t g0 = p->tensor_offset[ti] + pc.lo;
        if (pc.lo != at_ || !pc.len || g0 / c != (g0 + pc.len - 1) / c ||
            (order != GC_ORDER_RANK && pc.first != (g0 / c + 1) % nranks) || pc.first >= static_cast<uint32_t>(nranks))
          return debug_fail("bucket pieces do not tile a tensor by owner chunks");
        at_ += pc.len;
      }
      if (at_ != n) return debug_fail("bucket pieces do not cover a tensor");
      ++sl;
    }
    if (k != pieces.size()) return debug_fail("bucket piece outside every tensor");
  }
  gci::BucketCall call{slot_ptrs.data(), static_cast<int>(slot), nranks, pieces.data(),
                       static_cast<int>(pieces.size()), p->t, op == GC_AVG, sumsq, stream};
  call.wire = order == GC_ORDER_RING_WIRE;
  return gci::launch_bucket_all_reduce(call);
}

extern "C" gc_status gc_bucket_pack(const gc_bucket_plan* p, int bucket, const void* const* tensors,
                                    void* const* bucket_bufs, int nranks, hipStream_t stream) {
  if (!tensors || !bucket_bufs) return GC_ERR_INVALID_ARG;
  std::vector<gci::Segment> segs;
  GC_TRY(bucket_segments(p, bucket, tensors, nullptr, nullptr, bucket_bufs, nranks, true, &segs));
  GC_TRY(debug_segments(segs.data(), segs.size()));
  return gci::launch_segment_copy(segs.data(), segs.size(), kPackStore, stream);
}

extern "C" gc_status gc_bucket_unpack(const gc_bucket_plan* p, int bucket, const void* const* bucket_bufs,
                                      void* const* tensors, int nranks, hipStream_t stream) {
  if (!tensors || !bucket_bufs) return GC_ERR_INVALID_ARG;
  std::vector<gci::Segment> segs;
  GC_TRY(bucket_segments(p, bucket, nullptr, tensors, bucket_bufs, nullptr, nranks, false, &segs));
  GC_TRY(debug_segments(segs.data(), segs.size()));
  return gci::launch_segment_copy(segs.data(), segs.size(), kUnpackStore, stream);
}
