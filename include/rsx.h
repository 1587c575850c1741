/*
 * rsx -- ring reduce-scatter / all-gather / all-reduce on one MI355X (gfx950).
 *
 * C ABI of librsx.so.  One process drives W "virtual ranks": rank r is a
 * buffer in the one GPU's HBM, and each call takes a host array of W device
 * pointers where a communicator-based library would take one buffer and a
 * communicator.  Every entry point enqueues its kernels on `stream` and
 * returns without synchronising the host.
 *
 * Sources of the semantics (web pages):
 *   [NC] NCCL 1.x src/reduce_scatter.cu (pytorch mirror, "Git at Google"):
 *        ncclReduceScatter, the ring kernel and GetBlock, its host launcher
 *        (count 0 -> success; one device -> plain copy) and its op/type
 *        dispatch (unknown op / type -> an error code).
 *   [DP] "Distributed primitives": reduce-scatter, all-gather, all-reduce,
 *        Ring AllReduce = ReduceScatter + AllGather, bucketed ring all-reduce.
 *   [SG] Apache SINGA src/io/communicator.cc, fusedSynch / synch: tensors
 *        packed back to back into a fusion buffer, all-reduced, unpacked;
 *        in-place all-reduce of a tensor.
 *   [HV] Horovod horovod/common/operations.cc, PerformOperation: memcpy into
 *        the fusion buffer at running offsets, in-place all-reduce, memcpy out.
 *   [MX] "Add scatter reduce for JACCL#3901": naive all-reduce for messages
 *        of at most 32 KB.
 *
 * Common conventions
 *   - Pointer arrays (`sendbufs`, `recvbufs`, `tensors`, `counts`) are HOST
 *     arrays, read during the call only.  The device buffers they point to
 *     are owned by the caller and must stay valid until the stream work ends.
 *   - The library allocates no device or pinned memory and does not
 *     synchronise; it launches kernels on `stream` (0 = the null stream) on
 *     the calling thread's current HIP device, which must hold every buffer.
 *   - Validation (null pointers, rank count, enum ranges, size overflow,
 *     illegal buffer overlap) happens before any HIP call; a rejected call
 *     has no effect.  A failed launch returns RSX_ERR_HIP, and
 *     rsx_status_string(RSX_ERR_HIP) then names the HIP error (per thread).
 *   - Counts are elements, not bytes.  A count of 0 returns RSX_SUCCESS
 *     without launching anything [NC host launcher].
 *   - Every buffer must start at a multiple of its element size (4 for
 *     fp32, 2 for bf16, ...); any other address returns
 *     RSX_ERR_INVALID_ARGUMENT.  Buffers of 16-byte-aligned address take the
 *     dwordx4 kernels (for reduce-scatter blocks and all-gather pieces whose
 *     byte length is a multiple of 4, with dword-aligned loads where they are
 *     not whole 16-byte vectors); other element-aligned addresses are correct
 *     but slower.
 *   - Bit-exact means equal bit patterns, except that NaN payloads are not
 *     specified: where the result is a NaN, any NaN is correct (the pages fix
 *     no NaN propagation rule; bf16 rounding quiets a NaN as sign|0x7FC0).
 *   - The dwordx4 reduction and gather kernels reserve LDS they do not use
 *     (up to 96 KiB per workgroup) to limit how many of their workgroups
 *     share a CU, unless the calling thread turned that off with
 *     rsx_set_occupancy_caps (for launches that overlap other kernels).
 */
#ifndef RSX_H
#define RSX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RSX_VERSION 110          /* 1.1.0 */
#define RSX_MAX_RANKS 16         /* largest W a call accepts */
#define RSX_NAIVE_MAX_BYTES 32768 /* RSX_ALGO_AUTO picks naive at or below this, per rank [MX] */
#define RSX_FUSE_BATCH 248       /* tensors per pack/unpack launch */
#define RSX_SPARSE_SCRATCH_BYTES 134217728 /* 128 MiB: scratch array of rsx_sparse_all_reduce_noalloc, per GPU */

typedef enum {
  RSX_FLOAT32 = 0,   /* fp32 in, fp32 fold, fp32 out */
  RSX_BFLOAT16 = 1,  /* bf16 in, widened exactly to fp32, fp32 fold, one RNE rounding to bf16 out */
  RSX_INT32 = 2,     /* int32, two's-complement wrapping sum and product */
  RSX_FLOAT64 = 3,   /* fp64 in, fp64 fold, fp64 out */
  RSX_FLOAT16 = 4,   /* IEEE half in and out, folded in half: the ring partial is rounded (RNE)
                        to half after every step, as the page's T-typed ring buffers hold it
                        [NC ReduceScatterKernelArgs<T>, ThisBuffer / NextBuffer]; avg divides
                        the half fold by W, the quotient rounded to half */
  RSX_INT64 = 5,     /* int64, wrapping */
  RSX_UINT64 = 6,    /* uint64, wrapping */
  RSX_INT8 = 7,      /* int8 (the page's char), wrapping */
  RSX_FLOAT32_HALF_WIRE = 8 /* fp32 in and out with IEEE half as the wire format
                               [Apache SINGA communicator.cc, synchHalf / fusedSynchHalf]:
                               each input is rounded (RNE) to half, the halves are folded
                               as RSX_FLOAT16 is (half partial at every ring step), and the
                               half result is widened to fp32.  Reductions only:
                               rsx_all_gather rejects it with RSX_ERR_INVALID_TYPE; pack and
                               unpack treat it as fp32.  W = 1 still rounds through half. */
} rsx_dtype_t;

typedef enum {
  RSX_SUM = 0,
  RSX_MAX = 1,       /* compare-select fold: a later value replaces the partial only if greater */
  RSX_MIN = 2,       /* compare-select fold: a later value replaces the partial only if smaller */
  RSX_AVG = 3,       /* sum fold, then one division by W in the fold type (signed: toward zero) */
  RSX_PROD = 4       /* product fold (integers wrap) [NC FuncProd] */
} rsx_op_t;

typedef enum {
  RSX_ALGO_RING = 0,       /* segment k folded in ring order (k+1)%W, ..., k; then gathered, in
                              one pass or two (the faster form for the shape; same bits) */
  RSX_ALGO_NAIVE = 1,      /* every element folded in rank order 0..W-1 [MX] */
  RSX_ALGO_AUTO = 2,       /* NAIVE when count * element size <= RSX_NAIVE_MAX_BYTES, else RING */
  RSX_ALGO_RING_FUSED = 3, /* RING, always as one pass (fold, then store to every rank) */
  RSX_ALGO_RING_SPLIT = 4  /* RING, always as a reduce-scatter, then an all-gather [DP] */
} rsx_algo_t;

typedef enum {
  RSX_SUCCESS = 0,
  RSX_ERR_INVALID_ARGUMENT = 1, /* null or misaligned pointer, rank count out of [1, RSX_MAX_RANKS], bad algo */
  RSX_ERR_INVALID_TYPE = 2,     /* dtype outside rsx_dtype_t [NC: invalid type] */
  RSX_ERR_INVALID_OP = 3,       /* op outside rsx_op_t [NC: invalid operation] */
  RSX_ERR_UNSUPPORTED = 4,      /* sizes whose byte count or launch grid overflows */
  RSX_ERR_ALIASING = 5,         /* buffers overlap in a way other than the in-place forms */
  RSX_ERR_HIP = 6               /* a HIP launch failed; see rsx_status_string */
} rsx_status_t;

/*
 * Reduce-scatter [NC ncclReduceScatter; DP "Reduce-Scatter"].
 *
 * sendbufs[r]  device array of W*recvcount elements, rank r's input.
 * recvbufs[k]  device array of recvcount elements, receives block k:
 *              recvbufs[k][i] = fold of sendbufs[r][k*recvcount + i] over
 *              r = (k+1)%W, (k+2)%W, ..., k, in that order (the ring's order:
 *              block k leaves the position after k at step 0 and ends on
 *              position k at step W-1, per GetBlock with the identity ring).
 * nranks       W, 1..RSX_MAX_RANKS.  W = 1 is a copy (nothing if in place).
 * In place: recvbufs[k] == (char*)sendbufs[k] + k*recvcount*size is allowed.
 * Any other overlap of a recv buffer with a send buffer or another recv
 * buffer returns RSX_ERR_ALIASING.  Send buffers may alias each other only
 * when identical.
 */
rsx_status_t rsx_reduce_scatter(const void* const* sendbufs, void* const* recvbufs,
                                int nranks, size_t recvcount, rsx_dtype_t dtype,
                                rsx_op_t op, hipStream_t stream);

/*
 * All-gather [DP "All-Gather"; the gather half of Ring AllReduce].
 *
 * sendbufs[k]  device array of sendcount elements, rank k's piece.
 * recvbufs[r]  device array of W*sendcount elements; on return
 *              recvbufs[r][k*sendcount + i] = sendbufs[k][i] for every r, k.
 * In place: sendbufs[k] == (char*)recvbufs[k] + k*sendcount*size is allowed.
 * Other overlaps return RSX_ERR_ALIASING.
 */
rsx_status_t rsx_all_gather(const void* const* sendbufs, void* const* recvbufs,
                            int nranks, size_t sendcount, rsx_dtype_t dtype,
                            hipStream_t stream);

/*
 * All-reduce [DP Ring AllReduce = ReduceScatter + AllGather; SG synch; HV
 * PerformOperation].
 *
 * sendbufs[r], recvbufs[r]  device arrays of `count` elements.
 * RSX_ALGO_RING: the `count` elements are split into W segments of
 *   S = ceil(count/W): segment k = [min(kS,count), min((k+1)S,count)), see
 *   rsx_segment_begin.  Segment k is folded in ring order (k+1)%W, ..., k and
 *   written to every rank: the result equals rsx_all_gather applied to the
 *   reduce-scatter output whenever W divides count.  Two forms give the
 *   same bits (the same folds in the same order):
 *   - one pass (RSX_ALGO_RING_FUSED): each lane folds its element of all W
 *     inputs in registers and stores the result to all W outputs;
 *   - two passes (RSX_ALGO_RING_SPLIT): a reduce-scatter writes segment k
 *     into recvbufs[k] at its own offset, then an all-gather copies it from
 *     there to the other W-1 outputs, (2W+1)/(2W) of the one-pass bytes.
 *     W must divide count (else RSX_ERR_UNSUPPORTED); any element-aligned address.
 *   RSX_ALGO_RING takes two passes when W >= 7, W divides count, every
 *   buffer and segment is 16-byte aligned and a rank holds at least 4 MiB
 *   (measured faster there), one pass otherwise.
 * RSX_ALGO_NAIVE: every element folded in rank order 0..W-1 [MX].
 * In place: recvbufs[r] == sendbufs[r] for every r (or a permutation of the
 * send buffers) is allowed; other overlaps return RSX_ERR_ALIASING.
 */
rsx_status_t rsx_all_reduce(const void* const* sendbufs, void* const* recvbufs,
                            int nranks, size_t count, rsx_dtype_t dtype, rsx_op_t op,
                            rsx_algo_t algo, hipStream_t stream);

/*
 * Bucketed all-reduce ["Distributed primitives", In practice: the gradient
 * is all-reduced in buckets, one after another].
 *
 * The `count` elements of every rank are cut into consecutive buckets of
 * bucket_elems elements, the last one shorter: bucket b = [b*bucket_elems,
 * min((b+1)*bucket_elems, count)).  Each bucket is an rsx_all_reduce of its
 * own, with its own segments (S = ceil(len/W), ring order per segment) and
 * its own RSX_ALGO_AUTO choice, launched in bucket order on `stream`.  The
 * result equals rsx_all_reduce on each bucket in turn.  When W divides
 * bucket_elems, the full buckets share one launch per pass (each bucket
 * still folded over its own segments in its own ring order) and the shorter
 * last bucket follows.
 * Arguments, ownership, in-place and aliasing rules: as rsx_all_reduce, on
 * the whole buffers.  bucket_elems = 0: RSX_ERR_INVALID_ARGUMENT.
 * RSX_ALGO_RING_SPLIT needs W to divide every bucket (RSX_ERR_UNSUPPORTED).
 * The whole call is validated before the first launch.
 */
rsx_status_t rsx_all_reduce_bucketed(const void* const* sendbufs, void* const* recvbufs,
                                     int nranks, size_t count, size_t bucket_elems,
                                     rsx_dtype_t dtype, rsx_op_t op, rsx_algo_t algo,
                                     hipStream_t stream);

/*
 * One bucket of a bucketed all-reduce ["Distributed primitives", In
 * practice: each bucket is all-reduced as soon as the backward pass has
 * produced it, on a stream of its own].
 *
 * The all-reduce of bucket `bucket` alone, [bucket*bucket_elems,
 * min((bucket+1)*bucket_elems, count)), with that bucket's own segments and
 * RSX_ALGO_AUTO choice: the result equals what rsx_all_reduce_bucketed
 * stores for it.  For callers that enqueue each bucket when its inputs are
 * ready.  Arguments and validation as rsx_all_reduce_bucketed, on the whole
 * buffers; bucket >= rsx_bucket_count(count, bucket_elems):
 * RSX_ERR_INVALID_ARGUMENT (count = 0: nothing to do, RSX_SUCCESS).
 */
rsx_status_t rsx_all_reduce_bucket(const void* const* sendbufs, void* const* recvbufs,
                                   int nranks, size_t count, size_t bucket_elems, size_t bucket,
                                   rsx_dtype_t dtype, rsx_op_t op, rsx_algo_t algo,
                                   hipStream_t stream);

/* Buckets of a bucketed all-reduce: ceil(count / bucket_elems); 0 when
 * bucket_elems is 0. */
size_t rsx_bucket_count(size_t count, size_t bucket_elems);

/*
 * Tensor-fusion pack [SG fusedSynch(send=false); HV PerformOperation memcpy in].
 *
 * Copies tensors[i] (device, counts[i] elements) to
 * fused + (counts[0] + ... + counts[i-1]) elements: back to back, in list
 * order, with no padding.  `fused` must hold the sum of counts and must not
 * overlap any tensor (RSX_ERR_ALIASING).  ntensors >= 0; zero-count tensors
 * are skipped and may be null.  Launches one kernel per RSX_FUSE_BATCH
 * non-empty tensors (a tensor above 16 GiB counts once per 16 GiB).  The sum
 * of counts times the element size must stay below 2^40 bytes
 * (RSX_ERR_UNSUPPORTED otherwise).
 */
rsx_status_t rsx_fuse_pack(const void* const* tensors, const size_t* counts, int ntensors,
                           void* fused, rsx_dtype_t dtype, hipStream_t stream);

/*
 * Tensor-fusion unpack [SG fusedSynch(send=true) copy-out; HV memcpy out]:
 * the inverse of rsx_fuse_pack, same offsets and rules.
 */
rsx_status_t rsx_fuse_unpack(const void* fused, void* const* tensors, const size_t* counts,
                             int ntensors, rsx_dtype_t dtype, hipStream_t stream);

/*
 * Tensor-fusion all-reduce without a fusion buffer [SG fusedSynch; HV
 * PerformOperation; DP Ring AllReduce].
 *
 * sendtensors[r*ntensors + i], recvtensors[r*ntensors + i]: device arrays of
 * rank r's tensor i, counts[i] elements each (the same count on every rank).
 * The result is, bit for bit, that of rsx_fuse_pack of each rank's list into
 * a buffer of F = counts[0] + ... + counts[n-1] elements, rsx_all_reduce of
 * the W buffers with `algo`, then rsx_fuse_unpack into recvtensors: element
 * j of tensor i sits at fused offset counts[0] + ... + counts[i-1] + j and is
 * folded in the order of the fused segment holding that offset.  No fusion
 * buffer is read or written, so HBM traffic is one all-reduce of the tensors.
 * RSX_ALGO_AUTO picks naive when F * element size <= RSX_NAIVE_MAX_BYTES.
 * Ring order is always one pass here (RSX_ALGO_RING_FUSED and RSX_ALGO_RING
 * alike); RSX_ALGO_RING_SPLIT returns RSX_ERR_UNSUPPORTED.
 * In place: recvtensors[r*n + i] == sendtensors[r2*n + i] (same tensor index)
 * is allowed; any other overlap of a destination returns RSX_ERR_ALIASING.
 * Zero-count tensors are skipped and may be null.  Launches about one kernel
 * per 256 / (2W) tensors (256 / W when every destination is its own source).
 */
rsx_status_t rsx_fused_all_reduce(const void* const* sendtensors, void* const* recvtensors,
                                  const size_t* counts, int ntensors, int nranks,
                                  rsx_dtype_t dtype, rsx_op_t op, rsx_algo_t algo,
                                  hipStream_t stream);

/* Sparsification of rsx_sparse_all_reduce [SG valSparsAllReduce / topKSparsAllReduce]. */
typedef enum {
  RSX_SPARSE_THRESHOLD = 0, /* send the entries with |x| >= threshold (never a zero) */
  RSX_SPARSE_TOPK = 1       /* send the k largest values (not magnitudes); ties by lower index */
} rsx_sparse_mode_t;

/*
 * K of the top-K mode as the page computes it: ceil(fraction * count) with
 * `fraction` a float and `count` converted to float, the product rounded to
 * float [SG topKSparsAllReduce].  Returns 0 when the product is not positive
 * (or NaN).  Host arithmetic only.
 */
size_t rsx_sparse_topk_count(size_t count, float fraction);

/*
 * Bytes of device workspace rsx_sparse_all_reduce needs for these sizes:
 * per-tile counts and offsets, radix histograms and 8 bytes per element per
 * rank (rounded up to whole 4096-element tiles) of per-tile entry slots.
 * The same for both modes and with or without an accumulation.  0 for
 * invalid arguments.
 */
size_t rsx_sparse_workspace_size(int nranks, size_t count, rsx_sparse_mode_t mode, int has_accum);

/*
 * Sparsified all-reduce with error feedback [SG valSparsAllReduce,
 * topKSparsAllReduce, via sparsification / fusedSparsification].
 *
 * For each rank r, with g = grads[r] + accums[r] (one fp32 add; g = grads[r]
 * when accums is NULL):
 *   RSX_SPARSE_THRESHOLD: entry i is sent when |g[i]| >= threshold and
 *     g[i] != 0 (any threshold: a NaN threshold sends nothing, one <= 0
 *     every nonzero entry);
 *   RSX_SPARSE_TOPK: the k largest g[i] are sent (a NaN ranks below every
 *     number, -0 equals +0, equal values are taken by increasing index);
 *   with accums: accums[r][i] = g[i] - (0 + g[i]) where sent, g[i] - 0 where
 *     not (what was not sent; a sent inf leaves NaN);
 *   msg_idx[r][0..nnz[r]), msg_val[r][0..nnz[r]): the sent (zero-based
 *     index, g value) pairs in increasing index order (the page's wire
 *     message; its top-K message holds the same pairs sorted by value).
 * Then every outs[r][i] = the fp32 sum, starting from +0 and taking ranks
 * 0, 1, ..., W-1 in order, of the values sent for index i (+0 if none).
 *
 * grads[r], outs[r], accums[r]: device arrays of `count` fp32, 16-byte
 *   aligned.  accums may be NULL (no error feedback); if not, every entry
 *   must be set.  outs[r] == grads[r] is allowed (in place, as the page
 *   writes the result into the gradient).
 * msg_idx[r], msg_val[r]: device arrays of msg_capacity entries, 4-byte
 *   aligned; msg_capacity >= count (threshold) or >= k (top-K).
 * nnz: device array of nranks uint32, the message lengths (k for top-K).
 * workspace: device memory, 256-byte aligned, of at least
 *   rsx_sparse_workspace_size(...) bytes; its contents are scratch.
 * count <= UINT32_MAX (indices are uint32); k <= count.
 * count 0: nnz is zeroed and nothing else is touched.
 * The outputs may overlap the gradients (they are written after every read
 * of the gradients; e.g. outs[r] == grads[r]) and gradients may overlap each
 * other; any other overlap among grads, accums, outs, messages, nnz and the
 * workspace is RSX_ERR_ALIASING.  Invalid sizes, pointers, alignment, mode or
 * capacity: RSX_ERR_INVALID_ARGUMENT; count > UINT32_MAX: RSX_ERR_UNSUPPORTED.
 * With an accumulation, top-K writes accums[r] twice (a guess of the
 * residual, then its corrections), so accums[r] must not be read by other
 * work meanwhile.  Validation precedes every HIP call.  Enqueues 4 kernels
 * (threshold) or up to 16 (top-K) on `stream`; allocates nothing and does
 * not synchronise.
 */
rsx_status_t rsx_sparse_all_reduce(const float* const* grads, float* const* accums,
                                   float* const* outs, int nranks, size_t count,
                                   rsx_sparse_mode_t mode, float threshold, size_t k,
                                   uint32_t* const* msg_idx, float* const* msg_val,
                                   size_t msg_capacity, uint32_t* nnz, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * The sparsified all-reduce above without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, results,
 * validation and errors as rsx_sparse_all_reduce; it calls no hipMalloc or
 * hipFree and allocates nothing.
 *
 * Its workspace is a library-owned array of RSX_SPARSE_SCRATCH_BYTES in each
 * GPU's memory, held from the first call on that GPU until the process ends.
 * Sizes whose rsx_sparse_workspace_size(...) exceeds RSX_SPARSE_SCRATCH_BYTES
 * return RSX_ERR_UNSUPPORTED (8 bytes per element of every rank plus a little:
 * e.g. W * count up to about 16 M elements).  The kernels initialise what they
 * read of it, so contents left by an earlier call do not matter.  Every call
 * on one GPU uses the same array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and give wrong results;
 * serialise them.  Enqueues on `stream` and does not synchronise.
 */
rsx_status_t rsx_sparse_all_reduce_noalloc(const float* const* grads, float* const* accums,
                                           float* const* outs, int nranks, size_t count,
                                           rsx_sparse_mode_t mode, float threshold, size_t k,
                                           uint32_t* const* msg_idx, float* const* msg_val,
                                           size_t msg_capacity, uint32_t* nnz, hipStream_t stream);

/*
 * Tensor-fusion planner [HV BackgroundThreadLoop, fusion of consecutive
 * all-reduce requests; HorovodGlobalState tensor_fusion_threshold, default
 * 64 MiB, overridden by an environment variable].
 *
 * Groups tensors 0..ntensors-1 in order: a group starts at the first tensor
 * not yet grouped and takes each next tensor while that tensor has the
 * group's dtype and the group's bytes plus its bytes stay <= threshold_bytes.
 * A tensor that does not fit ends the group; none is skipped.  A tensor
 * larger than the threshold is a group of its own.
 * counts[i], dtypes[i]: tensor i's element count and type (host arrays).
 * group_end: host array of at least ntensors ints; group g is tensors
 *   [group_end[g-1], group_end[g]) (group_end[-1] taken as 0).
 * Returns the number of groups (0 for no tensors), or -1 for a null array, a
 * negative ntensors or an invalid dtype.  Host logic only: no HIP call.
 */
int rsx_fusion_plan(const size_t* counts, const rsx_dtype_t* dtypes, int ntensors,
                    size_t threshold_bytes, int* group_end);

/*
 * First element of segment k in RSX_ALGO_RING all-reduce of `count`
 * elements over `nranks` ranks: min(k * ceil(count/nranks), count).
 * k may be 0..nranks (k = nranks gives count).  Returns 0 for nranks < 1.
 */
size_t rsx_segment_begin(size_t count, int nranks, int k);

/* Size in bytes of one element of `dtype`, 0 if it is not a valid dtype. */
size_t rsx_dtype_size(rsx_dtype_t dtype);

/* Static description of a status; for RSX_ERR_HIP the calling thread's last
 * HIP error text.  Never NULL. */
const char* rsx_status_string(rsx_status_t status);

/* RSX_VERSION of the built library. */
int rsx_version(void);

/*
 * Occupancy caps of the calling thread's launches; returns the previous
 * setting (1 on, 0 off).  On by default: the dwordx4 reduction and gather
 * kernels then reserve LDS they do not use, so that fewer of their
 * workgroups share a CU, which keeps HBM busiest when a collective runs by
 * itself (W = 8 reduce-scatter 378 -> 361 us, one-pass all-reduce
 * 769 -> 735 us).  Reserved LDS also keeps other kernels off those CUs:
 * turn the caps off for launches meant to overlap compute on another stream
 * (bucketed all-reduce beside a matmul per bucket: 1,371 us with the caps,
 * 1,185 us without).  Results are the same either way.  Host state only.
 */
int rsx_set_occupancy_caps(int enable);

#ifdef __cplusplus
}
#endif

#endif /* RSX_H */
