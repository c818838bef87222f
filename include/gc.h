/*
 * gc.h — gradient-synchronisation collectives on one MI355X (gfx950).
 *
 * The N "ranks" of a data-parallel group are N buffers in one GPU's HBM; a
 * collective is the reduction and data movement it performs on them, done by
 * hand-written HIP kernels.  Semantics follow the pages cited per call:
 *
 *   DTLM  "Distributed Training for Large Models: Collectives, FSDP/ZeRO,
 *         DeviceMesh, and Multi-Dimensional Parallelism" (zexinliu.github.io)
 *   AIG6  "AI Infra Guide", chapter 6 "分布式训练基础" (theaiera.top)
 *   NXMR  the nxmr.cn article on collective communication and model
 *         parallelism (news/160867), by its own section numbers
 *
 * Conventions for every call
 *   - Buffers are DEVICE pointers owned by the caller; arrays of pointers,
 *     split tables and size lists are HOST arrays, read before the call returns.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without synchronising; results are visible to later work on that stream.
 *   - Arguments are validated on the host first: GC_ERR_INVALID_ARG and
 *     GC_ERR_UNSUPPORTED mean nothing was enqueued.  GC_ERR_HIP means a launch
 *     failed; a call that issues several launches (one per parameter, per
 *     batch of segments, per phase) may have enqueued the ones before it, so
 *     its outputs are then incomplete.  Faults inside a kernel surface at the
 *     caller's next synchronisation.
 *   - No call allocates device memory.  The bucket plan is a host object.
 *   - No call memsets, copies through the host or synchronises, so calls can
 *     be captured into a HIP graph and replayed (validation runs at capture).
 *   - nranks is 1..GC_MAX_RANKS.  Element counts are per rank.
 *   - Every buffer extent a call derives from its counts is at most 2^40
 *     bytes (more than one GPU holds) and ends inside the address space;
 *     otherwise GC_ERR_INVALID_ARG.  An all-to-all moves at most 2^42 bytes
 *     per call (GC_ERR_UNSUPPORTED above).
 *   - Calls are reentrant; concurrent calls on different streams must not
 *     write overlapping memory.
 *
 * Reduction arithmetic (AIG6 §6.3.4, reduce_dtype=float32): bf16 and fp32
 * inputs are summed in fp32, int32 inputs with wrap-around.  GC_AVG divides
 * the fp32 sum by nranks with one IEEE division, then the result is rounded to
 * the output type (bf16: round to nearest, ties to even; NaN stays NaN;
 * subnormals kept).
 *
 * Fold order.  GC_ORDER_RING folds chunk j (owned by rank j) starting from
 * rank j+1's contribution and ending with rank j's, the order the ring
 * reduce-scatter produces (DTLM §2 "Reduce-Scatter", N = 4 schedule; NXMR
 * §2.2).  GC_ORDER_RANK folds ranks 0, 1, ..., N-1 for every element.  Each
 * fold starts from its first operand, never from zero.
 *
 * GC_ORDER_RING_WIRE is the ring order of a ring that communicates in the
 * gradient's type (DTLM §11 "精度和分布式通信的关系": low-precision
 * communication, fp32 arithmetic): every partial a rank forwards is rounded to
 * the input type (bf16: nearest, ties to even) before the next rank adds its
 * own term in fp32; the owner's last add and the epilogue are as above.  For
 * fp32 and int32 inputs it equals GC_ORDER_RING.  Every reduction accepts it;
 * in the two-level calls both levels forward bf16 partials (inside a group
 * before the next member adds its term, across groups before the next group
 * adds its own partial).
 *
 * Debug checks.  With GC_DEBUG set to a value other than "0" in the
 * environment (read once), each call also checks the launch tables the host
 * planned from its arguments (copy segments write disjoint ranges that no other
 * segment reads; bucket pieces tile every tensor by owner chunk) and refuses
 * the call with GC_ERR_INVALID_ARG and a message on stderr if one fails.
 */
#ifndef GC_H
#define GC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GC_MAX_RANKS 64

typedef enum {
  GC_OK = 0,
  GC_ERR_INVALID_ARG = 1,   /* null pointer, bad enum, size mismatch, illegal overlap        */
  GC_ERR_UNSUPPORTED = 2,   /* valid request outside this library's limits (e.g. N > 64)     */
  GC_ERR_HIP = 3,           /* a HIP runtime call failed (launch, device query)               */
  GC_ERR_NO_MEMORY = 4      /* host allocation failed (bucket plan)                           */
} gc_status;

typedef enum { GC_INT32 = 0, GC_FP32 = 1, GC_BF16 = 2 } gc_dtype;
typedef enum { GC_SUM = 0, GC_AVG = 1 } gc_op;                 /* GC_AVG: floating types only */
typedef enum { GC_ORDER_RING = 0, GC_ORDER_RANK = 1, GC_ORDER_RING_WIRE = 2 } gc_order;
typedef enum { GC_AR_FUSED = 0, GC_AR_RS_AG = 1 } gc_ar_algo;

/*
 * Reduce-scatter (DTLM §2 "Reduce-Scatter"; FSDP gradient sync, DTLM §4 FSDP1).
 *   send[i]  rank i's full buffer, nranks*recv_count elements of in_t
 *            (chunk j = elements [j*recv_count, (j+1)*recv_count)).
 *   recv[j]  owner j's shard, recv_count elements of out_t:
 *            recv[j][k] = op over i of send[i][j*recv_count + k].
 *   Types: bf16->bf16, bf16->fp32, fp32->fp32, fp32->bf16, int32->int32.
 *   The caller pads so that nranks divides the full length, as FSDP pads its
 *   FlatParameter (DTLM §4 FSDP1).
 *   In place is allowed only as recv[r] == send[r] + r*recv_count elements with
 *   in_t == out_t; any other overlap is rejected with GC_ERR_INVALID_ARG.
 */
gc_status gc_reduce_scatter(const void* const* send, void* const* recv, size_t recv_count,
                            int nranks, gc_dtype in_t, gc_dtype out_t, gc_op op, gc_order order,
                            hipStream_t stream);

/*
 * All-gather (DTLM §2 "All-Gather"; FSDP parameter unshard, DTLM §4 FSDP1).
 *   send[i]  shard i, count elements of t.
 *   recv[d]  nranks*count elements: recv[d][i*count + k] = send[i][k] for every d.
 *   Pure data movement (bit-exact).  In place is allowed only as
 *   send[r] == recv[r] + r*count elements.
 */
gc_status gc_all_gather(const void* const* send, void* const* recv, size_t count, int nranks,
                        gc_dtype t, hipStream_t stream);

/*
 * Scratch bytes gc_all_reduce needs for `algo` (0 for GC_AR_FUSED; for
 * GC_AR_RS_AG one owner-shard buffer of count elements, 256-byte aligned).
 */
size_t gc_all_reduce_scratch_bytes(size_t count, int nranks, gc_dtype t, gc_ar_algo algo);

/*
 * All-reduce (DTLM §2 "All-Reduce": All-Reduce = Reduce-Scatter + All-Gather;
 * DDP gradient sync, AIG6 §6.2.4).
 *   send[i], recv[i]  count elements of t each; any count (the ring's owner
 *   chunks are c = ceil(count/nranks) elements, trailing chunks short or empty).
 *   recv[r][e] = op over i of send[i][e] for every r, folded in `order`.
 *   GC_AR_FUSED   one pass: every element's N inputs are read once and the
 *                 result is written to all N outputs.
 *   GC_AR_RS_AG   reduce-scatter into `scratch` (owner shards, already
 *                 averaged and rounded), then all-gather from it; the result is
 *                 bit-identical to GC_AR_FUSED.  scratch_bytes must be at least
 *                 gc_all_reduce_scratch_bytes(); scratch may be NULL for FUSED.
 *   In place (recv[r] == send[r]) is allowed; recv[r] may also equal any send[i]
 *   exactly.  Partial overlaps, overlapping recv buffers, or scratch
 *   overlapping a buffer are rejected.
 */
gc_status gc_all_reduce(const void* const* send, void* const* recv, size_t count, int nranks,
                        gc_dtype t, gc_op op, gc_order order, gc_ar_algo algo,
                        void* scratch, size_t scratch_bytes, hipStream_t stream);

/*
 * All-to-all(v) with an expert dimension (DTLM §2 "All-to-All"; MoE dispatch
 * and All-to-AllV, DTLM §8).
 *   splits   HOST int64 array [nranks][nranks][experts_per_rank]: splits[s][d][e]
 *            rows go from rank s to local expert e of rank d.
 *   send[s]  rows grouped by destination d, then expert e (block (s,d,e) at row
 *            offset sum of splits[s][d'][e'] over (d',e') before (d,e)).
 *   recv[d]  rows grouped by expert e, then source s (block (s,d,e) at row
 *            offset sum of splits[s'][d][e'] over (e',s') before (e,s)); rows of
 *            a block keep their order.  With experts_per_rank == 1 this is
 *            plain all_to_all_v ordered by source.
 *   row_bytes bytes per row (any value >= 1).  Row counts per rank must be
 *            below 2^31; nranks^2 * experts_per_rank at most 2^24.  Pure data
 *            movement (bit-exact); buffers must not overlap.  Each non-empty
 *            block is one contiguous copy; the copies run in equal-byte tiles,
 *            up to 128 blocks per launch.
 */
gc_status gc_all_to_all(const void* const* send, void* const* recv, const int64_t* splits,
                        int nranks, int experts_per_rank, size_t row_bytes, hipStream_t stream);

/*
 * Two-level (hierarchical) all-reduce and HSDP (AIG6 Table 6-2: hierarchical
 * all-reduce, two-level aggregation matched to the topology; AIG6 §6.3.6:
 * HSDP on nodes of 8 GPUs; DTLM §4: an HSDP mesh has a shard dimension and a
 * replicate dimension).  nranks = R * group_size ranks form R groups; rank
 * g * group_size + i is member i of group g (the mesh's shard index).
 *
 * The result is bit-identical to the three-ring schedule: inside each group a
 * ring reduce-scatter over its members (member i keeps chunk i of the group's
 * sum, chunks c1 = ceil(count / group_size) long, fp32 partials), then for
 * each i a ring all-reduce of chunk i across the R groups (chunk i cut into R
 * pieces of ceil(len_i / R); piece h folded from group h+1 around to group h),
 * then an all-gather inside each group.  The epilogue runs once at the end
 * (GC_AVG divides by nranks).  GC_ORDER_RANK folds members 0.. and groups 0..
 * instead.  GC_ORDER_RING_WIRE is the same schedule with every forwarded
 * partial rounded to bf16 at both levels (for fp32 and int32 it is the ring).
 * One pass: every input is read once and every output written once.  Types
 * and aliasing as gc_all_reduce.
 */
gc_status gc_hier_all_reduce(const void* const* send, void* const* recv, size_t count, int nranks, int group_size,
                             gc_dtype t, gc_op op, gc_order order, hipStream_t stream);

/*
 * HSDP gradient reduce-scatter: the first two phases of gc_hier_all_reduce.
 *   send[r]  rank r's full gradient, group_size * recv_count elements of in_t.
 *   recv[r]  recv_count elements of out_t: chunk i = r mod group_size of the
 *            reduction over all nranks ranks, the same on every group.
 * Types, op and padding as gc_reduce_scatter (group_size divides the length).
 * recv[r] may sit exactly on chunk i of send[r] when in_t == out_t.
 */
gc_status gc_hsdp_reduce_scatter(const void* const* send, void* const* recv, size_t recv_count, int nranks,
                                 int group_size, gc_dtype in_t, gc_dtype out_t, gc_op op, gc_order order,
                                 hipStream_t stream);

/*
 * FSDP2 per-parameter Shard(0) (DTLM §4 "FSDP2: DTensor / DeviceMesh"): each of
 * nparams parameters, rows[p] x cols[p] elements stored row-major, is its own
 * sharded tensor.  Rank r's shard of parameter p is rows [min(R, r*c),
 * min(R, (r+1)*c)), R = rows[p], c = ceil(R / nranks), stored contiguously:
 * the torch.chunk rule, so trailing ranks may hold fewer rows or none.
 * Pointer arrays are HOST arrays of nranks * nparams device pointers, rank-major
 * (entry r * nparams + p); a shard pointer may be NULL when its shard is empty.
 *
 * gc_fsdp2_reduce_scatter: grads[r*nparams + p] is rank r's full gradient of p;
 *   shards[j*nparams + p] receives rank j's rows of the reduction over ranks.
 *   Types, op and order as gc_reduce_scatter, with each parameter's row
 *   shards as the owner chunks (ring order folds shard j from rank j+1 around
 *   to rank j).  A shard may sit in place at its offset in the same rank's
 *   gradient when in_t == out_t; no other overlap is allowed.
 * gc_fsdp2_all_gather: params[d*nparams + p] receives the full parameter p on
 *   every rank d, assembled from the shards by offset (bit-exact).  A shard
 *   may sit in place at its offset in the same rank's parameter buffer.
 * One launch per non-empty parameter.
 */
gc_status gc_fsdp2_reduce_scatter(const void* const* grads, void* const* shards, const size_t* rows,
                                  const size_t* cols, int nparams, int nranks, gc_dtype in_t, gc_dtype out_t,
                                  gc_op op, gc_order order, hipStream_t stream);

gc_status gc_fsdp2_all_gather(const void* const* shards, void* const* params, const size_t* rows,
                              const size_t* cols, int nparams, int nranks, gc_dtype t, hipStream_t stream);

/*
 * Expert-parallel MoE around the all-to-all (DTLM §8 "专家并行和 MoE 通信": the
 * router picks top-k experts per token, tokens are packed by target expert /
 * rank and dispatched with All-to-AllV, the local experts run, a second
 * All-to-AllV brings the results back and the token order is restored).
 * Ranks hold E = experts_per_rank experts each; global expert g lives on rank
 * g / E as local expert g % E.  The router and the experts are the caller's.
 *
 * A route is one (token, k) pair of a source rank, numbered t * topk + k.
 * Its destination row in rank d's receive buffer follows gc_all_to_all's
 * receive layout: blocks by local expert, then by source, and inside a block
 * the routes in ascending route number (the order a source sends them in,
 * by global expert, then token).
 */

/*
 * Scratch bytes gc_moe_route needs, nbins = nranks * E: each source's routes
 * are cut into tiles of max(1024, nbins rounded up to 64) routes, and the
 * plan keeps one int32 per tile and global expert, plus nranks * nbins int32.
 */
size_t gc_moe_route_scratch_bytes(const int64_t* ntokens, int nranks, int topk, int experts_per_rank);

/*
 * Routing plan, computed on the device.
 *   experts[s]  DEVICE int32 [ntokens[s] * topk]: global expert of each route of
 *               source s (token-major).  Ids outside [0, nranks * E) mark a
 *               dropped route: it is not counted and its dest entry is (-1, -1).
 *   ntokens     HOST int64 [nranks] tokens per source (0 allowed).
 *   splits      DEVICE int64 [nranks][nranks][E] out: routes of source s to local
 *               expert e of rank d, the table gc_all_to_all takes (copy it to the
 *               host to size the receive buffers).
 *   dest[s]     DEVICE int32 pairs [ntokens[s] * topk][2] out: (rank, row) of
 *               each route's copy in the receive buffers.
 *   scratch     DEVICE, 256-byte aligned, at least gc_moe_route_scratch_bytes().
 * 1 <= topk <= 8; nranks * E <= 8192; total routes below 2^31.  Output and
 * scratch buffers must not overlap each other or the inputs.
 */
gc_status gc_moe_route(const int32_t* const* experts, const int64_t* ntokens, int nranks, int topk,
                       int experts_per_rank, int64_t* splits, int32_t* const* dest, void* scratch,
                       size_t scratch_bytes, hipStream_t stream);

/*
 * gc_moe_route for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as gc_moe_route, without the scratch buffer:
 * the plan's scratch is a static array of GC_MOE_ROUTE_NOALLOC_SCRATCH_BYTES
 * in the library, one per GPU, held until the process ends.  The call itself
 * allocates nothing (no hipMalloc / hipFree, no host heap).  Plans that need
 * more scratch than that (gc_moe_route_scratch_bytes()) are refused with
 * GC_ERR_UNSUPPORTED before anything is launched; 4 MiB holds, for example,
 * 8 ranks x 64 experts with up to 16,000 tiles of 1024 routes.  The array
 * belongs to the device of `stream` (the current device for the null stream)
 * and its address is looked up on the first call there (GC_ERR_HIP if that
 * fails).  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (concurrent streams, or host threads) race and must be ordered by
 * the caller.  Nothing has to be cleared between calls: every entry the plan
 * reads was written earlier in the same call.
 */
#define GC_MOE_ROUTE_NOALLOC_SCRATCH_BYTES (4u << 20)

gc_status gc_moe_route_noalloc(const int32_t* const* experts, const int64_t* ntokens, int nranks, int topk,
                               int experts_per_rank, int64_t* splits, int32_t* const* dest, hipStream_t stream);

/*
 * Dispatch straight from token order: the pack by expert fused into the
 * all-to-all.  Row t of tokens[s] is read once and copied to recv[d] row r for
 * each of its routes (d, r) = dest[s][t * topk + k].  Equal to packing every
 * source's routes in their send order and calling gc_all_to_all with the
 * splits of gc_moe_route.
 *   tokens[s]   DEVICE [ntokens[s]] rows of row_bytes bytes.
 *   dest[s]     DEVICE int32 pairs, as gc_moe_route writes them.
 *   recv[d]     DEVICE [recv_rows[d]] rows; recv_rows is a HOST int64 [nranks].
 * Entries of dest outside [0, nranks) x [0, recv_rows[d]) are skipped.  Pure
 * data movement (bit-exact); receive buffers must not overlap anything else.
 */
gc_status gc_moe_dispatch(const void* const* tokens, const int64_t* ntokens, const int32_t* const* dest,
                          int nranks, int topk, size_t row_bytes, void* const* recv,
                          const int64_t* recv_rows, hipStream_t stream);

/*
 * Combine: the inverse all-to-all fused with the weighted un-permute back to
 * token order.  For every source s and token t,
 *   out[s][t] = sum over k of weights[s][t * topk + k] * expert_out[d][r],
 *   (d, r) = dest[s][t * topk + k], hidden elements of type t per row.
 * Arithmetic: rows are widened to fp32, each product is rounded to fp32, the
 * products are added in k order starting from k = 0, and the sum is rounded
 * once to the row type (bf16: nearest, ties to even).  Routes whose entry lies
 * outside the expert_out buffers are left out of the sum; a token with no
 * route left gets zeros.
 *   expert_out[d]  DEVICE [expert_rows[d]] rows in rank d's receive layout.
 *   weights[s]     DEVICE fp32 [ntokens[s] * topk] gate weights.
 *   out[s]         DEVICE [ntokens[s]] rows.
 * t is GC_BF16 or GC_FP32.  Output buffers must not overlap anything else.
 */
gc_status gc_moe_combine(const void* const* expert_out, const int64_t* expert_rows, const int32_t* const* dest,
                         const float* const* weights, const int64_t* ntokens, int nranks, int topk,
                         size_t hidden, gc_dtype t, void* const* out, hipStream_t stream);

/*
 * Bucket plan: DDP gradient buckets (AIG6 §6.2.4; NXMR §5.1) and the FSDP
 * FlatParameter layout (DTLM §4 FSDP1).
 *   Tensors are visited in reverse definition order when `reverse` is nonzero
 *   (the order backward produces gradients), else in definition order.  Each
 *   tensor is appended to the open bucket; the bucket closes as soon as its
 *   bytes reach cap_bytes (cap_bytes == SIZE_MAX: one bucket holding all
 *   tensors).  Tensors are never split.  Inside a bucket tensors are
 *   concatenated in visiting order; each bucket's length is padded with zeros
 *   to a multiple of pad_to elements (1: no padding; nranks: FlatParameter;
 *   at most 2^20).  A bucket whose padded bytes would not fit in 64 bits is
 *   rejected with GC_ERR_INVALID_ARG.
 *   The plan is an immutable host object and may be shared across streams.
 */
typedef struct gc_bucket_plan gc_bucket_plan;

gc_status gc_bucket_plan_create(const size_t* numels, int ntensors, gc_dtype t, size_t cap_bytes,
                                int reverse, size_t pad_to, gc_bucket_plan** out);

/*
 * Query a plan.  Every output pointer may be NULL.
 *   nbuckets        number of buckets.
 *   bucket_numel    [nbuckets] padded element count of each bucket.
 *   tensor_bucket   [ntensors] bucket index of each tensor.
 *   tensor_offset   [ntensors] element offset of each tensor in its bucket.
 */
gc_status gc_bucket_plan_query(const gc_bucket_plan* plan, int* nbuckets, size_t* bucket_numel,
                               int* tensor_bucket, size_t* tensor_offset);

/*
 * Pack bucket `bucket` of every rank: bucket_bufs[r][offset_t ...] = tensors[r*ntensors + t]
 * for each tensor t of the bucket, and zeros in the padding.
 *   tensors      HOST array of nranks*ntensors device pointers (rank-major); only
 *                the bucket's tensors are read, others may be NULL.
 *   bucket_bufs  nranks device buffers of at least bucket_numel elements.
 * Pure data movement (bit-exact).  Buffers must not overlap.
 */
gc_status gc_bucket_pack(const gc_bucket_plan* plan, int bucket, const void* const* tensors,
                         void* const* bucket_bufs, int nranks, hipStream_t stream);

/* Inverse of gc_bucket_pack: tensors[r*ntensors + t] = bucket_bufs[r][offset_t ...]. */
gc_status gc_bucket_unpack(const gc_bucket_plan* plan, int bucket, const void* const* bucket_bufs,
                           void* const* tensors, int nranks, hipStream_t stream);

/*
 * Zero-copy bucketed all-reduce: DDP with gradient_as_bucket_view (AIG6
 * §6.2.4), where gradients live in the bucket instead of being copied into it.
 * All-reduces bucket `bucket` directly over the tensors, in place:
 * tensors[r*ntensors + t][k] becomes op over ranks i of tensors[i*ntensors + t][k],
 * for every tensor t of the bucket.  Element k of tensor t sits at
 * offset_t + k of the packed bucket, whose bucket_numel elements (padding
 * included) form the owner chunks that fix the fold order, so the result is
 * bit-identical to gc_bucket_pack, gc_all_reduce over bucket_numel elements
 * with the same op and order, then gc_bucket_unpack; it moves 2*N*B bytes
 * instead of 6*N*B.
 *   tensors  HOST array of nranks*ntensors device pointers (rank-major); only
 *            the bucket's tensors are read; they must not overlap.
 *   sumsq    optional DEVICE pointer to one double (NULL: none; floating types
 *            only).  The sum over the bucket's elements of the squared results,
 *            as stored (rank 0's copy), is ADDED to *sumsq with device atomics,
 *            so callers zero it once and accumulate over buckets for gradient-norm
 *            clipping.  The order of the atomic additions is not fixed: the
 *            norm's last bits may differ between runs.
 */
gc_status gc_bucket_all_reduce(const gc_bucket_plan* plan, int bucket, void* const* tensors, int nranks,
                               gc_op op, gc_order order, double* sumsq, hipStream_t stream);

void gc_bucket_plan_destroy(gc_bucket_plan* plan);

/* Static, human-readable name of a status code. */
const char* gc_status_string(gc_status status);

/* Library version as 10000*major + 100*minor + patch. */
int gc_version(void);

/*
 * hipError_t of the most recent HIP call that failed inside this library on
 * the calling thread (the cause behind a GC_ERR_HIP), or 0 if none has failed.
 */
int gc_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GC_H */
