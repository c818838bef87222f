/*
 * A plain C program that uses libgc through include/gc.h alone: device memory
 * from hipMalloc, one HIP stream, no Python and no PyTorch.  It runs the
 * collectives on N rank buffers in one GPU and checks every output against a
 * closed form computed here on the host.  The inputs are chosen so that the
 * closed form is exact whatever the fold order:
 *   - int32 sums wrap modulo 2^32 (any order gives the same bits);
 *   - fp32 and bf16 inputs are small integers, whose sums stay below 2^24, and
 *     GC_AVG divides by a power of two, so every partial and result is exact;
 *   - data movement (all-gather, all-to-all, bucket pack / unpack) is compared
 *     bit for bit with the definition of where each element goes.
 * Error returns are checked for a few invalid calls (nothing may be launched).
 *
 * Exit status 0 when every check passes; the first failing check prints what
 * differed and the program exits with status 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gc.h"

static int g_checks = 0;

#define HIP_OK(call)                                                                         \
  do {                                                                                       \
    hipError_t e_ = (call);                                                                  \
    if (e_ != hipSuccess) {                                                                  \
      fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
      exit(1);                                                                               \
    }                                                                                        \
  } while (0)

#define GC_EXPECT(call, want)                                                                       \
  do {                                                                                              \
    gc_status s_ = (call);                                                                          \
    if (s_ != (want)) {                                                                             \
      fprintf(stderr, "%s:%d: %s -> %s, expected %s\n", __FILE__, __LINE__, #call, gc_status_string(s_), \
              gc_status_string(want));                                                              \
      exit(1);                                                                                      \
    }                                                                                               \
  } while (0)

static void* dalloc(size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes ? bytes : 1));
  return p;
}

static void* halloc(size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p) {
    fprintf(stderr, "host allocation of %zu bytes failed\n", bytes);
    exit(1);
  }
  return p;
}

static void compare(const char* what, const void* got, const void* want, size_t n, size_t es) {
  const unsigned char* g = (const unsigned char*)got;
  const unsigned char* w = (const unsigned char*)want;
  for (size_t i = 0; i < n; ++i) {
    if (memcmp(g + i * es, w + i * es, es) != 0) {
      uint32_t gv = 0, wv = 0;
      memcpy(&gv, g + i * es, es < 4 ? es : 4);
      memcpy(&wv, w + i * es, es < 4 ? es : 4);
      fprintf(stderr, "%s: element %zu differs: got 0x%08x, want 0x%08x\n", what, i, gv, wv);
      exit(1);
    }
  }
  ++g_checks;
}

/* A small integer in [-lim, lim] from (rank, element). */
static int small_int(int r, size_t e, int lim) {
  uint32_t h = (uint32_t)e * 2654435761u ^ (uint32_t)(r + 1) * 0x9E3779B9u;
  h ^= h >> 15;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  return (int)(h % (uint32_t)(2 * lim + 1)) - lim;
}

/* bf16 bits of a float whose low 16 bits are zero (small integers are). */
static uint16_t bf16_bits_exact(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* int32 all-reduce (sum, wrapping) in both orders and both algorithms. */
static void check_all_reduce_int32(hipStream_t st) {
  enum { N = 5 };
  const size_t S = 100003;
  void *send[N], *recv[N];
  int32_t* host = (int32_t*)halloc(S * 4);
  uint32_t* want = (uint32_t*)halloc(S * 4);
  memset(want, 0, S * 4);
  for (int r = 0; r < N; ++r) {
    for (size_t e = 0; e < S; ++e) {
      uint32_t v = (uint32_t)e * 2246822519u + (uint32_t)r * 3266489917u;
      host[e] = (int32_t)v;
      want[e] += v;
    }
    send[r] = dalloc(S * 4);
    recv[r] = dalloc(S * 4);
    HIP_OK(hipMemcpy(send[r], host, S * 4, hipMemcpyHostToDevice));
  }
  const size_t scratch_bytes = gc_all_reduce_scratch_bytes(S, N, GC_INT32, GC_AR_RS_AG);
  void* scratch = dalloc(scratch_bytes);
  const gc_order orders[2] = {GC_ORDER_RING, GC_ORDER_RANK};
  for (int o = 0; o < 2; ++o) {
    for (int a = 0; a < 2; ++a) {
      const gc_ar_algo algo = a ? GC_AR_RS_AG : GC_AR_FUSED;
      GC_EXPECT(gc_all_reduce((const void* const*)send, recv, S, N, GC_INT32, GC_SUM, orders[o], algo,
                              a ? scratch : NULL, a ? scratch_bytes : 0, st),
                GC_OK);
      HIP_OK(hipStreamSynchronize(st));
      for (int r = 0; r < N; ++r) {
        HIP_OK(hipMemcpy(host, recv[r], S * 4, hipMemcpyDeviceToHost));
        compare(a ? "all-reduce int32 rs_ag" : "all-reduce int32 fused", host, want, S, 4);
      }
    }
  }
  for (int r = 0; r < N; ++r) {
    HIP_OK(hipFree(send[r]));
    HIP_OK(hipFree(recv[r]));
  }
  HIP_OK(hipFree(scratch));
  free(host);
  free(want);
}

/* fp32 all-reduce, avg over 8 ranks, in place. */
static void check_all_reduce_fp32_avg(hipStream_t st) {
  enum { N = 8 };
  const size_t S = 65541;
  void* buf[N];
  float* host = (float*)halloc(S * 4);
  float* want = (float*)halloc(S * 4);
  int32_t* sum = (int32_t*)halloc(S * 4);
  memset(sum, 0, S * 4);
  for (int r = 0; r < N; ++r) {
    for (size_t e = 0; e < S; ++e) {
      const int v = small_int(r, e, 500);
      host[e] = (float)v;
      sum[e] += v;
    }
    buf[r] = dalloc(S * 4);
    HIP_OK(hipMemcpy(buf[r], host, S * 4, hipMemcpyHostToDevice));
  }
  for (size_t e = 0; e < S; ++e) want[e] = (float)sum[e] / 8.0f;
  GC_EXPECT(gc_all_reduce((const void* const*)buf, buf, S, N, GC_FP32, GC_AVG, GC_ORDER_RING, GC_AR_FUSED, NULL, 0,
                          st),
            GC_OK);
  HIP_OK(hipStreamSynchronize(st));
  for (int r = 0; r < N; ++r) {
    HIP_OK(hipMemcpy(host, buf[r], S * 4, hipMemcpyDeviceToHost));
    compare("all-reduce fp32 avg in place", host, want, S, 4);
    HIP_OK(hipFree(buf[r]));
  }
  free(host);
  free(want);
  free(sum);
}

/* Reduce-scatter bf16 -> fp32, avg over 64 ranks (the FSDP gradient step). */
static void check_reduce_scatter_bf16_fp32(hipStream_t st) {
  enum { N = 64 };
  const size_t rc = 1000, S = N * rc;
  void *send[N], *recv[N];
  uint16_t* host = (uint16_t*)halloc(S * 2);
  int32_t* sum = (int32_t*)halloc(S * 4);
  float* got = (float*)halloc(rc * 4);
  float* want = (float*)halloc(rc * 4);
  memset(sum, 0, S * 4);
  for (int r = 0; r < N; ++r) {
    for (size_t e = 0; e < S; ++e) {
      const int v = small_int(r, e, 100); /* |v| <= 100: exact in bf16 */
      host[e] = bf16_bits_exact((float)v);
      sum[e] += v;
    }
    send[r] = dalloc(S * 2);
    recv[r] = dalloc(rc * 4);
    HIP_OK(hipMemcpy(send[r], host, S * 2, hipMemcpyHostToDevice));
  }
  GC_EXPECT(gc_reduce_scatter((const void* const*)send, recv, rc, N, GC_BF16, GC_FP32, GC_AVG, GC_ORDER_RING, st),
            GC_OK);
  HIP_OK(hipStreamSynchronize(st));
  for (int j = 0; j < N; ++j) {
    for (size_t k = 0; k < rc; ++k) want[k] = (float)sum[j * rc + k] / 64.0f;
    HIP_OK(hipMemcpy(got, recv[j], rc * 4, hipMemcpyDeviceToHost));
    compare("reduce-scatter bf16 -> fp32 avg", got, want, rc, 4);
  }
  for (int r = 0; r < N; ++r) {
    HIP_OK(hipFree(send[r]));
    HIP_OK(hipFree(recv[r]));
  }
  free(host);
  free(sum);
  free(got);
  free(want);
}

/* All-gather of raw bf16 bit patterns (NaN and Inf patterns included). */
static void check_all_gather_bf16(hipStream_t st) {
  enum { N = 6 };
  const size_t count = 1001;
  void *send[N], *recv[N];
  uint16_t* shard = (uint16_t*)halloc(count * 2);
  uint16_t* want = (uint16_t*)halloc(N * count * 2);
  uint16_t* got = (uint16_t*)halloc(N * count * 2);
  for (int i = 0; i < N; ++i) {
    for (size_t k = 0; k < count; ++k) shard[k] = (uint16_t)(k * 40503u + (unsigned)i * 7919u);
    memcpy(want + i * count, shard, count * 2);
    send[i] = dalloc(count * 2);
    recv[i] = dalloc(N * count * 2);
    HIP_OK(hipMemcpy(send[i], shard, count * 2, hipMemcpyHostToDevice));
  }
  GC_EXPECT(gc_all_gather((const void* const*)send, recv, count, N, GC_BF16, st), GC_OK);
  HIP_OK(hipStreamSynchronize(st));
  for (int d = 0; d < N; ++d) {
    HIP_OK(hipMemcpy(got, recv[d], N * count * 2, hipMemcpyDeviceToHost));
    compare("all-gather bf16", got, want, N * count, 2);
  }
  for (int i = 0; i < N; ++i) {
    HIP_OK(hipFree(send[i]));
    HIP_OK(hipFree(recv[i]));
  }
  free(shard);
  free(want);
  free(got);
}

/* All-to-all(v) with two experts per rank and uneven (some empty) blocks. */
static void check_all_to_all(hipStream_t st) {
  enum { N = 3, E = 2 };
  const size_t row_bytes = 24;
  int64_t splits[N][N][E];
  int64_t send_rows[N] = {0}, recv_rows[N] = {0};
  for (int s = 0; s < N; ++s)
    for (int d = 0; d < N; ++d)
      for (int e = 0; e < E; ++e) {
        splits[s][d][e] = (s * 7 + d * 3 + e * 5) % 6; /* 0..5 rows, zeros included */
        send_rows[s] += splits[s][d][e];
        recv_rows[d] += splits[s][d][e];
      }
  void *send[N], *recv[N];
  unsigned char* sendh[N];
  for (int s = 0; s < N; ++s) {
    const size_t b = (size_t)send_rows[s] * row_bytes;
    sendh[s] = (unsigned char*)halloc(b);
    for (size_t i = 0; i < b; ++i) sendh[s][i] = (unsigned char)(i * 31u + (unsigned)s * 101u);
    send[s] = dalloc(b);
    HIP_OK(hipMemcpy(send[s], sendh[s], b, hipMemcpyHostToDevice));
  }
  for (int d = 0; d < N; ++d) recv[d] = dalloc((size_t)recv_rows[d] * row_bytes);
  GC_EXPECT(gc_all_to_all((const void* const*)send, recv, &splits[0][0][0], N, E, row_bytes, st), GC_OK);
  HIP_OK(hipStreamSynchronize(st));
  for (int d = 0; d < N; ++d) {
    /* receive layout: by local expert e, then by source s; send layout: by destination, then expert */
    const size_t b = (size_t)recv_rows[d] * row_bytes;
    unsigned char* want = (unsigned char*)halloc(b);
    unsigned char* got = (unsigned char*)halloc(b);
    size_t at = 0;
    for (int e = 0; e < E; ++e)
      for (int s = 0; s < N; ++s) {
        size_t from = 0;
        for (int dd = 0; dd < N; ++dd)
          for (int ee = 0; ee < E; ++ee)
            if (dd < d || (dd == d && ee < e)) from += (size_t)splits[s][dd][ee];
        const size_t n = (size_t)splits[s][d][e] * row_bytes;
        memcpy(want + at, sendh[s] + from * row_bytes, n);
        at += n;
      }
    HIP_OK(hipMemcpy(got, recv[d], b, hipMemcpyDeviceToHost));
    compare("all-to-all(v) with experts", got, want, b, 1);
    free(want);
    free(got);
  }
  for (int r = 0; r < N; ++r) {
    HIP_OK(hipFree(send[r]));
    HIP_OK(hipFree(recv[r]));
    free(sendh[r]);
  }
}

/* Bucket plan: pack -> all-reduce -> unpack, and the zero-copy bucket all-reduce with
 * the sum of squares, on fp32 tensors holding small integers. */
static void check_buckets(hipStream_t st) {
  enum { N = 4, T = 5 };
  const size_t numels[T] = {1000, 37, 4096, 8, 513};
  gc_bucket_plan* plan = NULL;
  GC_EXPECT(gc_bucket_plan_create(numels, T, GC_FP32, 6000, 1, 1, &plan), GC_OK);
  int nb = 0;
  GC_EXPECT(gc_bucket_plan_query(plan, &nb, NULL, NULL, NULL), GC_OK);
  size_t* bnumel = (size_t*)halloc((size_t)nb * sizeof(size_t));
  int tbucket[T];
  size_t toff[T];
  GC_EXPECT(gc_bucket_plan_query(plan, &nb, bnumel, tbucket, toff), GC_OK);

  void* tens[N * T];   /* the pack path's tensors (kept as inputs) */
  void* zc[N * T];     /* the zero-copy path's tensors (reduced in place) */
  void* out[N * T];    /* the pack path's unpacked results */
  float* want[T];
  double want_sumsq = 0.0;
  for (int t = 0; t < T; ++t) {
    want[t] = (float*)halloc(numels[t] * 4);
    int32_t* sum = (int32_t*)halloc(numels[t] * 4);
    memset(sum, 0, numels[t] * 4);
    float* h = (float*)halloc(numels[t] * 4);
    for (int r = 0; r < N; ++r) {
      for (size_t k = 0; k < numels[t]; ++k) {
        const int v = small_int(r, k + 10000u * (size_t)t, 1000);
        h[k] = (float)v;
        sum[k] += v;
      }
      tens[r * T + t] = dalloc(numels[t] * 4);
      zc[r * T + t] = dalloc(numels[t] * 4);
      out[r * T + t] = dalloc(numels[t] * 4);
      HIP_OK(hipMemcpy(tens[r * T + t], h, numels[t] * 4, hipMemcpyHostToDevice));
      HIP_OK(hipMemcpy(zc[r * T + t], h, numels[t] * 4, hipMemcpyHostToDevice));
    }
    for (size_t k = 0; k < numels[t]; ++k) {
      want[t][k] = (float)sum[k];
      want_sumsq += (double)sum[k] * (double)sum[k];
    }
    free(sum);
    free(h);
  }
  double* sumsq = (double*)dalloc(sizeof(double));
  const double zero = 0.0;
  HIP_OK(hipMemcpy(sumsq, &zero, sizeof(double), hipMemcpyHostToDevice));
  for (int b = 0; b < nb; ++b) {
    void* bufs[N];
    for (int r = 0; r < N; ++r) bufs[r] = dalloc(bnumel[b] * 4);
    GC_EXPECT(gc_bucket_pack(plan, b, (const void* const*)tens, bufs, N, st), GC_OK);
    GC_EXPECT(gc_all_reduce((const void* const*)bufs, bufs, bnumel[b], N, GC_FP32, GC_SUM, GC_ORDER_RING, GC_AR_FUSED,
                            NULL, 0, st),
              GC_OK);
    GC_EXPECT(gc_bucket_unpack(plan, b, (const void* const*)bufs, out, N, st), GC_OK);
    GC_EXPECT(gc_bucket_all_reduce(plan, b, zc, N, GC_SUM, GC_ORDER_RING, sumsq, st), GC_OK);
    HIP_OK(hipStreamSynchronize(st));
    for (int r = 0; r < N; ++r) HIP_OK(hipFree(bufs[r]));
  }
  for (int t = 0; t < T; ++t) {
    float* got = (float*)halloc(numels[t] * 4);
    for (int r = 0; r < N; ++r) {
      HIP_OK(hipMemcpy(got, out[r * T + t], numels[t] * 4, hipMemcpyDeviceToHost));
      compare("bucket pack -> all-reduce -> unpack", got, want[t], numels[t], 4);
      HIP_OK(hipMemcpy(got, zc[r * T + t], numels[t] * 4, hipMemcpyDeviceToHost));
      compare("zero-copy bucket all-reduce", got, want[t], numels[t], 4);
    }
    free(got);
  }
  double got_sumsq = -1.0;
  HIP_OK(hipMemcpy(&got_sumsq, sumsq, sizeof(double), hipMemcpyDeviceToHost));
  /* every square and partial sum is an integer below 2^53: exact in any order */
  compare("zero-copy bucket all-reduce sum of squares", &got_sumsq, &want_sumsq, 1, sizeof(double));
  for (int i = 0; i < N * T; ++i) {
    HIP_OK(hipFree(tens[i]));
    HIP_OK(hipFree(zc[i]));
    HIP_OK(hipFree(out[i]));
  }
  for (int t = 0; t < T; ++t) free(want[t]);
  HIP_OK(hipFree(sumsq));
  free(bnumel);
  gc_bucket_plan_destroy(plan);
}

/* Refused calls return their status and launch nothing (the output keeps its sentinel). */
static void check_errors(hipStream_t st) {
  enum { N = 2 };
  const size_t S = 64;
  void *send[N], *recv[N];
  for (int r = 0; r < N; ++r) {
    send[r] = dalloc(S * 4);
    recv[r] = dalloc(S * 4);
    HIP_OK(hipMemset(send[r], 0x11, S * 4));
    HIP_OK(hipMemset(recv[r], 0x5A, S * 4));
  }
  GC_EXPECT(gc_all_reduce(NULL, recv, S, N, GC_FP32, GC_SUM, GC_ORDER_RING, GC_AR_FUSED, NULL, 0, st),
            GC_ERR_INVALID_ARG);
  GC_EXPECT(gc_all_reduce((const void* const*)send, recv, S, 65, GC_FP32, GC_SUM, GC_ORDER_RING, GC_AR_FUSED, NULL, 0,
                          st),
            GC_ERR_UNSUPPORTED);
  GC_EXPECT(gc_all_reduce((const void* const*)send, recv, S, N, GC_INT32, GC_AVG, GC_ORDER_RING, GC_AR_FUSED, NULL, 0,
                          st),
            GC_ERR_UNSUPPORTED);
  GC_EXPECT(gc_all_reduce((const void* const*)send, recv, S, N, GC_FP32, GC_SUM, GC_ORDER_RING, GC_AR_RS_AG, NULL, 0,
                          st),
            GC_ERR_INVALID_ARG); /* RS_AG without its scratch */
  void* overlap[N] = {recv[0], (char*)recv[0] + 4};
  GC_EXPECT(gc_all_reduce((const void* const*)send, overlap, S, N, GC_FP32, GC_SUM, GC_ORDER_RING, GC_AR_FUSED, NULL,
                          0, st),
            GC_ERR_INVALID_ARG);
  HIP_OK(hipStreamSynchronize(st));
  unsigned char* h = (unsigned char*)halloc(S * 4);
  unsigned char* sentinel = (unsigned char*)halloc(S * 4);
  memset(sentinel, 0x5A, S * 4);
  for (int r = 0; r < N; ++r) {
    HIP_OK(hipMemcpy(h, recv[r], S * 4, hipMemcpyDeviceToHost));
    compare("refused calls leave the output untouched", h, sentinel, S * 4, 1);
  }
  if (gc_status_string(GC_ERR_HIP) == NULL || gc_version() <= 0 || gc_last_hip_error() != 0) {
    fprintf(stderr, "status string, version or last HIP error unexpected\n");
    exit(1);
  }
  ++g_checks;
  free(h);
  free(sentinel);
  for (int r = 0; r < N; ++r) {
    HIP_OK(hipFree(send[r]));
    HIP_OK(hipFree(recv[r]));
  }
}

int main(void) {
  hipStream_t st;
  HIP_OK(hipSetDevice(0));
  HIP_OK(hipStreamCreate(&st));
  check_all_reduce_int32(st);
  check_all_reduce_fp32_avg(st);
  check_reduce_scatter_bf16_fp32(st);
  check_all_gather_bf16(st);
  check_all_to_all(st);
  check_buckets(st);
  check_errors(st);
  HIP_OK(hipStreamDestroy(st));
  printf("abi_demo: %d checks passed (libgc version %d)\n", g_checks, gc_version());
  return 0;
}
