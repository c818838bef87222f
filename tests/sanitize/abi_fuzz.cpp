// Seeded argument fuzz of libgc's C ABI, built for the host only with
// AddressSanitizer and UndefinedBehaviorSanitizer (api.cpp linked against the
// launch stubs of launch_stubs.cpp; nothing touches a GPU).
//
// Every call gets host arrays of exactly the length its contract names (so an
// over-read is an ASan report) and stand-in device addresses, each buffer
// declared to the stubs with the extent the contract gives it.  Arguments are
// drawn mostly valid, with a few per call perturbed: null or misaligned
// pointers, buffers aliasing each other, invalid enums, rank counts out of
// range, sizes near the 64-bit limits, negative splits.  Checked per call:
//   * the status is one of the gc_status values;
//   * a non-OK status launched nothing (validation precedes every launch);
//   * every launch stays inside the declared buffers (checked by the stubs);
//   * the library's GC_DEBUG checks of its own plan tables never fire;
// and over the run, every entry point returned GC_OK at least once and was
// refused at least once.  Exit status 0 means all held; the sanitizers abort
// the run on their first report.
//
// usage: abi_fuzz [iterations] [seed]

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "gc.h"
#include "stubs.h"

namespace {

std::mt19937_64 g_rng;
int g_failures = 0;

uint64_t rnd(uint64_t n) { return n ? g_rng() % n : 0; }
bool coin(double p) { return std::uniform_real_distribution<double>(0.0, 1.0)(g_rng) < p; }

// Stand-in device addresses: buffer k of a call sits at (k + 1) << 40, so
// buffers up to 2^40 bytes never overlap unless a perturbation makes them.
struct Mem {
  uint64_t next = 1;
  std::vector<std::pair<uint64_t, uint64_t>> made;  // (address, bytes) of every buffer of this call

  // A buffer of `bytes`, now and then perturbed: null, misaligned, an alias
  // into an earlier buffer of the call, or shifted.  Whatever address the
  // caller ends up passing is declared with the full extent: a caller's buffer
  // is valid memory of that size wherever it sits, and only the library's own
  // rules (alignment, overlap) may refuse it.
  void* buf(uint64_t bytes, double rate = 0.02) {
    uint64_t a = (next++) << 40;
    if (coin(rate)) {
      switch (rnd(4)) {
        case 0: a = 0; break;
        case 1: a += 1 + rnd(3); break;
        case 2:
          if (!made.empty()) {
            const auto& o = made[rnd(made.size())];
            a = o.first + (o.second ? rnd(o.second) & ~uint64_t(15) : 0);
          }
          break;
        default: a += 16 * rnd(1024); break;
      }
    }
    if (a && bytes && a + bytes > a) stub::declare(reinterpret_cast<void*>(a), bytes);  // never a wrapping extent
    made.push_back({a, bytes});
    return reinterpret_cast<void*>(a);
  }
};



int pick_ranks() {
  const uint64_t r = rnd(100);
  if (r < 3) return static_cast<int>(rnd(3)) - 2;  // -2 .. 0
  if (r < 6) return 64 + static_cast<int>(rnd(3));  // 64 .. 66
  if (r < 20) return 1 + static_cast<int>(rnd(64));
  return 1 + static_cast<int>(rnd(9));
}

uint64_t pick_count() {
  const uint64_t r = rnd(100);
  if (r < 5) return 0;
  if (r < 75) return rnd(3000);
  if (r < 90) return rnd(1u << 20);
  switch (rnd(5)) {
    case 0: return UINT64_MAX - rnd(8);
    case 1: return (uint64_t(1) << 62) - rnd(64);
    case 2: return uint64_t(1) << (32 + rnd(30));
    case 3: return (UINT64_MAX / 4) + rnd(4);
    default: return (uint64_t(1) << 40) + rnd(1000);
  }
}

template <class E>
E pick_enum(int valid) {
  return static_cast<E>(coin(0.03) ? static_cast<int>(rnd(20)) - 5 : static_cast<int>(rnd(valid)));
}

size_t es(gc_dtype t) { return t == GC_BF16 ? 2 : 4; }
bool valid_dtype(gc_dtype t) { return t == GC_INT32 || t == GC_FP32 || t == GC_BF16; }

// A byte extent that saturates instead of wrapping (the buffer a caller would need).
uint64_t ext(uint64_t a, uint64_t b) { return (b && a > UINT64_MAX / b) ? UINT64_MAX : a * b; }
uint64_t ext3(uint64_t a, uint64_t b, uint64_t c) { return ext(ext(a, b), c); }

struct Tally {
  long ok = 0, refused = 0;
};
std::vector<std::pair<std::string, Tally>> g_tally;

Tally& tally(const char* name) {
  for (auto& t : g_tally)
    if (t.first == name) return t.second;
  g_tally.push_back({name, Tally{}});
  return g_tally.back().second;
}

void check(const char* name, gc_status st, long launches_before, uint64_t iter) {
  Tally& t = tally(name);
  if (st < GC_OK || st > GC_ERR_NO_MEMORY) {
    std::fprintf(stderr, "iteration %llu %s: status %d out of range\n", (unsigned long long)iter, name, (int)st);
    ++g_failures;
  }
  if (st != GC_OK && stub::launches() != launches_before) {
    std::fprintf(stderr, "iteration %llu %s: status %s after a launch\n", (unsigned long long)iter, name,
                 gc_status_string(st));
    ++g_failures;
  }
  (st == GC_OK ? t.ok : t.refused)++;
}

// ---------------------------------------------------------------- one call each

void fuzz_reduce(uint64_t it) {
  Mem m;
  const int N = pick_ranks();
  const int n = N > 0 ? N : 0;
  const uint64_t count = pick_count();
  const gc_dtype ti = pick_enum<gc_dtype>(3), to = coin(0.5) ? ti : pick_enum<gc_dtype>(3);
  const gc_op op = pick_enum<gc_op>(2);
  const gc_order order = pick_enum<gc_order>(3);
  const size_t ei = valid_dtype(ti) ? es(ti) : 4, eo = valid_dtype(to) ? es(to) : 4;
  const int which = static_cast<int>(rnd(3));
  std::vector<const void*> send(n);
  std::vector<void*> recv(n);
  const uint64_t in_b = which == 0 ? ext3(n, count, ei) : which == 1 ? ext(count, ei) : ext(count, ei);
  const uint64_t out_b = which == 0 ? ext(count, eo) : which == 1 ? ext3(n, count, ei) : ext(count, ei);
  for (int r = 0; r < n; ++r) send[r] = m.buf(in_b);
  for (int r = 0; r < n; ++r) recv[r] = m.buf(out_b);
  if (which == 2 && coin(0.2))
    for (int r = 0; r < n; ++r) recv[r] = const_cast<void*>(send[r]);  // all-reduce in place
  const long before = stub::launches();
  gc_status st;
  if (which == 0) {
    st = gc_reduce_scatter(n ? send.data() : nullptr, n ? recv.data() : nullptr, count, N, ti, to, op, order,
                           nullptr);
    check("gc_reduce_scatter", st, before, it);
  } else if (which == 1) {
    st = gc_all_gather(n ? send.data() : nullptr, n ? recv.data() : nullptr, count, N, ti, nullptr);
    check("gc_all_gather", st, before, it);
  } else {
    const gc_ar_algo algo = pick_enum<gc_ar_algo>(2);
    uint64_t sb = gc_all_reduce_scratch_bytes(count, N, ti, algo);
    if (coin(0.05)) sb = sb ? sb - 1 : 0;
    void* scratch = m.buf(sb ? sb : 1);
    st = gc_all_reduce(n ? send.data() : nullptr, n ? recv.data() : nullptr, count, N, ti, op, order, algo,
                       scratch, sb, nullptr);
    check("gc_all_reduce", st, before, it);
  }
}

void fuzz_mesh(uint64_t it) {
  Mem m;
  const int N = pick_ranks();
  const int n = N > 0 ? N : 0;
  int group = n ? 1 + static_cast<int>(rnd(n)) : 1;
  if (coin(0.7))
    for (int g = group; g >= 1; --g)
      if (n % g == 0) {
        group = g;
        break;
      }
  if (coin(0.03)) group = static_cast<int>(rnd(3)) - 1;
  const uint64_t count = pick_count();
  const gc_dtype ti = pick_enum<gc_dtype>(3), to = coin(0.5) ? ti : pick_enum<gc_dtype>(3);
  const gc_op op = pick_enum<gc_op>(2);
  const gc_order order = pick_enum<gc_order>(3);
  const size_t ei = valid_dtype(ti) ? es(ti) : 4, eo = valid_dtype(to) ? es(to) : 4;
  const bool hsdp = coin(0.5);
  std::vector<const void*> send(n);
  std::vector<void*> recv(n);
  const uint64_t g = group > 0 ? static_cast<uint64_t>(group) : 1;
  for (int r = 0; r < n; ++r) send[r] = m.buf(hsdp ? ext3(g, count, ei) : ext(count, ei));
  for (int r = 0; r < n; ++r) recv[r] = m.buf(ext(count, hsdp ? eo : ei));
  const long before = stub::launches();
  if (hsdp) {
    check("gc_hsdp_reduce_scatter",
          gc_hsdp_reduce_scatter(n ? send.data() : nullptr, n ? recv.data() : nullptr, count, N, group, ti, to, op,
                                 order, nullptr),
          before, it);
  } else {
    check("gc_hier_all_reduce",
          gc_hier_all_reduce(n ? send.data() : nullptr, n ? recv.data() : nullptr, count, N, group, ti, op, order,
                             nullptr),
          before, it);
  }
}

void fuzz_a2a(uint64_t it) {
  Mem m;
  const int N = pick_ranks();
  const int n = N > 0 ? N : 0;
  const int E = coin(0.03) ? static_cast<int>(rnd(3)) - 1 : 1 + static_cast<int>(rnd(4));
  const int e = E > 0 ? E : 0;
  uint64_t rb = coin(0.05) ? pick_count() : 1 + rnd(300);
  std::vector<int64_t> splits(static_cast<size_t>(n) * n * e);
  std::vector<uint64_t> srows(n, 0), rrows(n, 0);
  for (int s = 0; s < n; ++s)
    for (int d = 0; d < n; ++d)
      for (int k = 0; k < e; ++k) {
        int64_t v = static_cast<int64_t>(rnd(40));
        if (coin(0.002)) v = -1 - static_cast<int64_t>(rnd(3));
        if (coin(0.001)) v = int64_t(1) << (20 + rnd(40));
        splits[(static_cast<size_t>(s) * n + d) * e + k] = v;
        if (v > 0) {
          srows[s] += v;
          rrows[d] += v;
        }
      }
  std::vector<const void*> send(n);
  std::vector<void*> recv(n);
  for (int r = 0; r < n; ++r) send[r] = m.buf(ext(srows[r], rb));
  for (int r = 0; r < n; ++r) recv[r] = m.buf(ext(rrows[r], rb));
  const long before = stub::launches();
  check("gc_all_to_all",
        gc_all_to_all(n ? send.data() : nullptr, n ? recv.data() : nullptr, n ? splits.data() : nullptr, N, E, rb,
                      nullptr),
        before, it);
}

// torch.chunk rule for dim-0 shards: rank r holds rows [min(rows, r c), min(rows, (r + 1) c)).
uint64_t shard_rows(uint64_t rows, int N, int r) {
  const uint64_t c = (rows + N - 1) / N;
  const uint64_t lo = std::min<uint64_t>(rows, ext(r, c)), hi = std::min<uint64_t>(rows, ext(r + 1, c));
  return hi - lo;
}

void fuzz_fsdp2(uint64_t it) {
  Mem m;
  const int N = pick_ranks();
  const int n = N > 0 ? N : 0;
  const int P = coin(0.03) ? -1 : static_cast<int>(rnd(6));
  const int p = P > 0 ? P : 0;
  std::vector<size_t> rows(p), cols(p);
  for (int k = 0; k < p; ++k) {
    rows[k] = coin(0.05) ? pick_count() : rnd(200);
    cols[k] = coin(0.05) ? pick_count() : rnd(40);
  }
  const gc_dtype ti = pick_enum<gc_dtype>(3), to = coin(0.5) ? ti : pick_enum<gc_dtype>(3);
  const size_t ei = valid_dtype(ti) ? es(ti) : 4, eo = valid_dtype(to) ? es(to) : 4;
  const bool rs = coin(0.5);
  std::vector<void*> full(static_cast<size_t>(n) * p);
  std::vector<void*> part(static_cast<size_t>(n) * p);
  for (int r = 0; r < n; ++r)
    for (int k = 0; k < p; ++k) {
      const size_t i = static_cast<size_t>(r) * p + k;
      full[i] = m.buf(ext3(rows[k], cols[k], rs ? ei : ei));
      const uint64_t sr = n ? shard_rows(rows[k], n, r) : 0;
      part[i] = sr && cols[k] ? m.buf(ext3(sr, cols[k], rs ? eo : ei)) : nullptr;
    }
  const long before = stub::launches();
  if (rs) {
    check("gc_fsdp2_reduce_scatter",
          gc_fsdp2_reduce_scatter(full.data(), part.data(), rows.data(), cols.data(), P, N, ti, to,
                                  pick_enum<gc_op>(2), pick_enum<gc_order>(3), nullptr),
          before, it);
  } else {
    check("gc_fsdp2_all_gather",
          gc_fsdp2_all_gather(part.data(), full.data(), rows.data(), cols.data(), P, N, ti, nullptr),
          before, it);
  }
}

void fuzz_moe(uint64_t it) {
  Mem m;
  const int N = pick_ranks();
  const int n = N > 0 ? N : 0;
  const int K = coin(0.05) ? static_cast<int>(rnd(12)) - 1 : 1 + static_cast<int>(rnd(3));
  const int E = coin(0.03) ? 5000 : 1 + static_cast<int>(rnd(8));
  std::vector<int64_t> ntok(n);
  for (int s = 0; s < n; ++s) ntok[s] = coin(0.01) ? -1 : coin(0.01) ? (int64_t(1) << 31) : rnd(3000);
  const uint64_t kk = K > 0 ? K : 0;
  std::vector<const int32_t*> experts(n);
  std::vector<int32_t*> dest(n);
  for (int s = 0; s < n; ++s) {
    const uint64_t routes = ntok[s] > 0 ? ext(ntok[s], kk) : 0;
    experts[s] = static_cast<const int32_t*>(m.buf(ext(routes, 4)));
    dest[s] = static_cast<int32_t*>(m.buf(ext(routes, 8)));
  }
  const int64_t NE = static_cast<int64_t>(n) * (E > 0 ? E : 0);
  int64_t* splits = static_cast<int64_t*>(m.buf(ext3(n, NE, 8)));
  const long before = stub::launches();
  const int kind = static_cast<int>(rnd(4));
  if (kind == 0) {
    const size_t need = gc_moe_route_scratch_bytes(n ? ntok.data() : nullptr, N, K, E);
    size_t sb = coin(0.05) && need ? need - 1 : need;
    void* scratch = m.buf(sb);
    check("gc_moe_route", gc_moe_route(n ? experts.data() : nullptr, n ? ntok.data() : nullptr, N, K, E, splits,
                                       n ? dest.data() : nullptr, scratch, sb, nullptr),
          before, it);
  } else if (kind == 1) {
    check("gc_moe_route_noalloc", gc_moe_route_noalloc(n ? experts.data() : nullptr, n ? ntok.data() : nullptr, N,
                                                       K, E, splits, n ? dest.data() : nullptr, nullptr),
          before, it);
  } else {
    const uint64_t rb = coin(0.05) ? pick_count() : 2 * (1 + rnd(64));
    std::vector<int64_t> rows(n);
    std::vector<const void*> src(n);
    std::vector<void*> dst(n);
    std::vector<const float*> w(n);
    for (int r = 0; r < n; ++r) rows[r] = coin(0.01) ? -1 : rnd(5000);
    for (int r = 0; r < n; ++r) {
      const uint64_t srows = kind == 2 ? (ntok[r] > 0 ? ntok[r] : 0) : (rows[r] > 0 ? rows[r] : 0);
      const uint64_t drows = kind == 2 ? (rows[r] > 0 ? rows[r] : 0) : (ntok[r] > 0 ? ntok[r] : 0);
      src[r] = m.buf(ext(srows, rb));
      dst[r] = m.buf(ext(drows, rb));
      w[r] = static_cast<const float*>(m.buf(ext(ntok[r] > 0 ? ntok[r] : 0, 4 * kk)));
    }
    if (kind == 2) {
      check("gc_moe_dispatch",
            gc_moe_dispatch(n ? src.data() : nullptr, n ? ntok.data() : nullptr,
                            n ? const_cast<const int32_t* const*>(dest.data()) : nullptr, N, K, rb,
                            n ? dst.data() : nullptr, n ? rows.data() : nullptr, nullptr),
            before, it);
    } else {
      const gc_dtype t = pick_enum<gc_dtype>(3);
      const uint64_t hidden = valid_dtype(t) ? rb / es(t) : rb;
      check("gc_moe_combine",
            gc_moe_combine(n ? src.data() : nullptr, n ? rows.data() : nullptr,
                           n ? const_cast<const int32_t* const*>(dest.data()) : nullptr, n ? w.data() : nullptr,
                           n ? ntok.data() : nullptr, N, K, hidden, t, n ? dst.data() : nullptr, nullptr),
            before, it);
    }
  }
}

void fuzz_buckets(uint64_t it) {
  const int T = coin(0.02) ? -1 : static_cast<int>(rnd(12));
  const int t = T > 0 ? T : 0;
  std::vector<size_t> numels(t);
  for (int k = 0; k < t; ++k) numels[k] = coin(0.03) ? pick_count() : rnd(5000);
  const gc_dtype dt = pick_enum<gc_dtype>(3);
  const size_t cap = coin(0.1) ? SIZE_MAX : rnd(40000);
  const size_t pad = coin(0.03) ? pick_count() : 1 + rnd(9);
  gc_bucket_plan* plan = nullptr;
  const long before = stub::launches();
  const gc_status st = gc_bucket_plan_create(t ? numels.data() : nullptr, T, dt, cap, static_cast<int>(rnd(2)), pad,
                                             coin(0.01) ? nullptr : &plan);
  check("gc_bucket_plan_create", st, before, it);
  if (st != GC_OK) return;
  int nb = 0;
  gc_bucket_plan_query(plan, &nb, nullptr, nullptr, nullptr);
  std::vector<size_t> bn(nb + 1);
  std::vector<int> tb(t + 1);
  std::vector<size_t> toff(t + 1);
  gc_bucket_plan_query(plan, &nb, bn.data(), tb.data(), toff.data());
  const size_t e = es(dt);
  for (int rep = 0; rep < 3; ++rep) {
    Mem m;
    const int N = pick_ranks();
    const int n = N > 0 ? N : 0;
    const int b = coin(0.03) ? nb + static_cast<int>(rnd(3)) : (nb ? static_cast<int>(rnd(nb)) : 0);
    std::vector<void*> tensors(static_cast<size_t>(n) * t);
    for (int r = 0; r < n; ++r)
      for (int k = 0; k < t; ++k) tensors[static_cast<size_t>(r) * t + k] = m.buf(ext(numels[k], e));
    std::vector<void*> bufs(n);
    for (int r = 0; r < n; ++r) bufs[r] = m.buf(ext(b < nb ? bn[b] : 0, e));
    const long b0 = stub::launches();
    const int kind = static_cast<int>(rnd(3));
    if (kind == 0) {
      check("gc_bucket_pack", gc_bucket_pack(plan, b, const_cast<const void* const*>(tensors.data()), bufs.data(), N,
                                             nullptr),
            b0, it);
    } else if (kind == 1) {
      check("gc_bucket_unpack", gc_bucket_unpack(plan, b, const_cast<const void* const*>(bufs.data()),
                                                 tensors.data(), N, nullptr),
            b0, it);
    } else {
      double* sq = coin(0.5) ? static_cast<double*>(m.buf(8)) : nullptr;
      check("gc_bucket_all_reduce", gc_bucket_all_reduce(plan, b, tensors.data(), N, pick_enum<gc_op>(2),
                                                         pick_enum<gc_order>(3), sq, nullptr),
            b0, it);
    }
  }
  gc_bucket_plan_destroy(plan);
}

}  // namespace

int main(int argc, char** argv) {
  // the library's own plan-table checks run before every launch (a failure is printed and refuses the call)
  setenv("GC_DEBUG", "1", 1);
  const uint64_t iters = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 20000;
  const uint64_t seed = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1;
  g_rng.seed(seed);
  for (uint64_t it = 0; it < iters; ++it) {
    stub::reset();
    switch (rnd(7)) {
      case 0:
      case 1: fuzz_reduce(it); break;
      case 2: fuzz_mesh(it); break;
      case 3: fuzz_a2a(it); break;
      case 4: fuzz_fsdp2(it); break;
      case 5: fuzz_moe(it); break;
      default: fuzz_buckets(it); break;
    }
  }
  if (stub::violations()) {
    std::fprintf(stderr, "%ld launches touched undeclared memory\n", stub::violations());
    ++g_failures;
  }
  for (const auto& t : g_tally) {
    std::printf("%-26s ok %6ld  refused %6ld\n", t.first.c_str(), t.second.ok, t.second.refused);
    if (!t.second.ok || !t.second.refused) {
      std::fprintf(stderr, "%s: never %s\n", t.first.c_str(), t.second.ok ? "refused" : "accepted");
      ++g_failures;
    }
  }
  std::printf("%llu iterations, seed %llu, %ld launches, %d failures\n", (unsigned long long)iters,
              (unsigned long long)seed, stub::launches(), g_failures);
  return g_failures ? 1 : 0;
}
