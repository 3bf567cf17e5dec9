/*
 * ddp.h -- C ABI of libddp.so: bucketed gradient synchronisation on one
 * MI355X (gfx950), with N virtual ranks whose gradients live in HBM.
 *
 * What the library computes (pages cited by title and section):
 *   [DDP]  "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel)
 *   [TR24] "(24) NCCL通信与分布式数据并行" (tech-renaissance.cn)
 *   [TR16] "(16) DTensor：一张图纸，多卡共享的分布式张量抽象" (tech-renaissance.cn)
 *   [DL]   "DDP分布式训练–数据加载和训练NCCL" (139.9.1.231)
 *
 *   1. plan      parameters are packed, last-registered first, into buckets of
 *                at most bucket_cap bytes ([DDP] 3.2, 4.2), or split into the
 *                two buckets DEEP_COMM / FIRST_COMM ([TR24] 八).
 *   2. flatten   each rank's per-parameter gradients are copied into one
 *                contiguous flat buffer per bucket ([DDP] 4.2, flat_grad).
 *   3. reduce    every bucket element is summed over the N ranks in a fixed
 *                FP32 order: SEQUENTIAL (zero, then ranks 0..N-1; [TR24] 一)
 *                or RING (the ring reduce-scatter order of [DDP] 2.10-2.11:
 *                chunk c = floor(i / ceil(L/N)) starts at rank (c+1) mod N).
 *   4. scale     the sum is multiplied by fl(1/N) ([TR24] 九; [DDP] 4.2),
 *                then stored as float32 or rounded to bf16 (nearest, ties to
 *                even) -- fused into the reduce.
 *   5. unflatten the averaged flat buffer is copied back to the per-parameter
 *                gradient views ([DDP] 4.2, viewed back onto .grad).
 *
 * Conventions for every entry point
 *   - Status codes, never exceptions or aborts.  Arguments are validated on
 *     the host before any GPU work is queued; on a non-OK return nothing has
 *     been enqueued (except DDP_ERR_HIP, returned when a launch fails).
 *   - "stream" is a hipStream_t passed as void*; NULL means the default
 *     stream.  Device work is enqueued on it and runs asynchronously: an OK
 *     return means "enqueued"; faults surface at the caller's next sync.
 *   - Device pointers refer to memory of the current HIP device
 *     (hipSetDevice / torch.cuda.set_device).  The caller owns all gradient
 *     and output memory.  The library allocates device memory only for its
 *     own descriptor tables (plans, bindings) and frees it in *_free.
 *   - Element counts and offsets are int64 everywhere.  A dispatch counts
 *     its grid in 32-bit work-items, so a grid of more than 2^30 work-items
 *     (a one-launch f32 reduce past 2^32 elements, bf16 past 2^33) runs as
 *     consecutive launches on the same stream; results are the same bits.  DDP_ERR_HIP from a later launch may follow earlier
 *     ones already enqueued.  The environment variable DDP_MAX_LAUNCH_ITEMS,
 *     read once per process, lowers the limit (at least 4096, rounded down
 *     to a multiple of 4096), so that tests can split small grids.
 */
#ifndef DDP_H
#define DDP_H

#include <stddef.h>
#include <stdint.h>

/* The library's exported symbols: it is built with hidden visibility, so
 * these declarations are the whole ABI. */
#if defined(__GNUC__)
#define DDP_API __attribute__((visibility("default")))
#else
#define DDP_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define DDP_ABI_VERSION 1
/* Largest number of virtual ranks one call accepts. */
#define DDP_MAX_RANKS 64

typedef enum {
    DDP_OK = 0,
    DDP_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad index/enum */
    DDP_ERR_UNSUPPORTED = 2,   /* dtype pair or rank count the library does not do */
    DDP_ERR_OVERFLOW = 3,      /* a size that does not fit the int64 layout */
    DDP_ERR_ALIAS = 4,         /* output overlaps an input other than exactly */
    DDP_ERR_HIP = 5,           /* a HIP runtime call failed */
    DDP_ERR_NOMEM = 6,         /* host or device allocation failed */
    DDP_ERR_CAPACITY = 7       /* beyond a fixed capacity (the no-allocation
                                  entry point's static buffer) */
} ddp_status_t;

typedef enum { DDP_F32 = 0, DDP_BF16 = 1 } ddp_dtype_t;

typedef enum {
    DDP_ORDER_SEQUENTIAL = 0,  /* acc = +0; acc += x_0; ...; acc += x_{N-1} */
    DDP_ORDER_RING = 1         /* acc = x_s; acc += x_{s+1}; ... (indices mod N) */
} ddp_order_t;

/* Gradient regions of the two-bucket split, in memory order ([TR24] 七:
 * G_BN_BIAS, G_BN_WEIGHT, G_FC_BIAS, G_FC_WEIGHT, G_FIRST_CONV, G_DEEP_CONV). */
typedef enum {
    DDP_REGION_BN_BIAS = 0,
    DDP_REGION_BN_WEIGHT = 1,
    DDP_REGION_FC_BIAS = 2,
    DDP_REGION_FC_WEIGHT = 3,
    DDP_REGION_FIRST = 4,
    DDP_REGION_DEEP = 5
} ddp_region_t;

typedef struct ddp_plan ddp_plan_t;        /* opaque; host data + per-device tables */
typedef struct ddp_binding ddp_binding_t;  /* opaque; one rank's parameter pointers */
typedef struct ddp_param_sync ddp_param_sync_t;  /* opaque; a bound per-parameter sync */

/* ------------------------------------------------------------------ plans
 * Host-only calls: no GPU is touched, no device memory is allocated.
 *
 * Flat layout of a plan: buckets 0..B-1 back to back from element 0; inside
 * a bucket its parameters back to back in "slot" order, with no padding.
 */

/* Cap-mode plan ([DDP] 3.2 and 4.2: parameters reversed, packed into buckets
 * of about bucket_cap_mb; the last layer lands in the first bucket).
 *   numel[n_params]   element count of each parameter, registration order, >= 0
 *   bucket_cap_bytes  cap in bytes of `dtype` elements (25 MiB = 26214400), > 0
 *   dtype             gradient element type (sets bytes per element)
 *   out               receives a new plan; free it with ddp_plan_free
 * Rule: walk parameters from last to first; close the current bucket when it
 * is non-empty and adding the next parameter would exceed the cap; a lone
 * parameter larger than the cap forms its own bucket.
 * Errors: INVALID_ARG (null, n_params < 1, numel < 0, cap <= 0, bad dtype),
 * OVERFLOW (total elements or bytes beyond int64), NOMEM. */
DDP_API ddp_status_t ddp_plan_buckets(const int64_t *numel, int32_t n_params,
                              int64_t bucket_cap_bytes, ddp_dtype_t dtype,
                              ddp_plan_t **out);

/* Two-bucket plan ([TR24] 八, layout of [TR16] 四).
 *   region[n_params]  one ddp_region_t per parameter
 * Bucket 0 = DEEP_COMM: the DEEP parameters in registration order.
 * Bucket 1 = FIRST_COMM: regions BN_BIAS, BN_WEIGHT, FC_BIAS, FC_WEIGHT,
 * FIRST in that order, registration order inside each region.
 * A bucket with no parameters is left out (the plan then has one bucket).
 * Errors: as ddp_plan_buckets, plus INVALID_ARG for an unknown region tag. */
DDP_API ddp_status_t ddp_plan_two_bucket(const int64_t *numel, const uint8_t *region,
                                 int32_t n_params, ddp_dtype_t dtype,
                                 ddp_plan_t **out);

/* Frees the plan and its device tables on every device they were uploaded
 * to.  The caller must make sure no queued work still reads them. NULL is ok. */
DDP_API void ddp_plan_free(ddp_plan_t *plan);

/* Number of buckets, or -1 for a NULL plan. */
DDP_API int32_t ddp_plan_num_buckets(const ddp_plan_t *plan);
/* Total elements of the flat layout, or -1 for a NULL plan. */
DDP_API int64_t ddp_plan_total(const ddp_plan_t *plan);

/* Bucket b: its length, its first element in the flat layout, and the range
 * [first_slot, first_slot + n_slots) of slots it holds.  Any output pointer
 * may be NULL.  Errors: INVALID_ARG (null plan, b out of range). */
DDP_API ddp_status_t ddp_plan_bucket(const ddp_plan_t *plan, int32_t b, int64_t *len,
                             int64_t *base, int32_t *first_slot, int32_t *n_slots);

/* Parameter held by flat slot `slot` (slots count 0..n_params-1 in flat order). */
DDP_API ddp_status_t ddp_plan_slot_param(const ddp_plan_t *plan, int32_t slot, int32_t *param);

/* Bucket of parameter p and its element offset inside that bucket. */
DDP_API ddp_status_t ddp_plan_param(const ddp_plan_t *plan, int32_t p, int32_t *bucket,
                            int64_t *offset);

/* Uploads the plan's device tables (used by ddp_sync_allreduce_avg in RING
 * order) to the current device, synchronously.  Optional: the first RING
 * sync on a device does it by itself; call it beforehand when the sync will
 * be captured into a HIP graph or must not allocate.
 * Errors: INVALID_ARG, HIP, NOMEM. */
DDP_API ddp_status_t ddp_plan_prepare(ddp_plan_t *plan);

/* ddp_plan_prepare, plus the table a RING synchronisation over n_ranks ranks
 * reads: one 32-bit word per tile of the flat layout (4 bytes per 256 f32 or
 * 512 bf16 elements) naming the ring chunks the tile meets.  RING chunks are
 * per bucket and depend on n_ranks, so each rank count has its own table,
 * kept on the device until ddp_plan_free.  Optional like ddp_plan_prepare:
 * the first RING call (ddp_sync_allreduce_avg, ddp_sync_sgd_update) with a
 * new rank count builds it synchronously; call this first when that call
 * will be captured into a HIP graph or must not allocate.
 *   n_ranks  1..DDP_MAX_RANKS (1 prepares only what ddp_plan_prepare does)
 * Errors: INVALID_ARG, HIP, NOMEM. */
DDP_API ddp_status_t ddp_plan_prepare_ranks(ddp_plan_t *plan, int32_t n_ranks);

/* ------------------------------------------------------------------ bindings
 * One rank's per-parameter gradient buffers, resolved once (a static graph
 * fixes every address up front: [DDP] 6.2; [TR24] 十 resolves addresses at
 * capture time).
 *   param_grads[n_params]  device pointer of each parameter's gradient, in
 *                          registration order; each holds numel[p] elements
 *                          of the element type flatten/unflatten are given.
 *                          Pointers must be at least 2-byte aligned.
 *   stream                 unused for now (the table upload is synchronous)
 * The binding copies the pointer array; it does not own the gradients.  It
 * keeps a device table of 32 bytes per 4096 elements of each parameter
 * (rounded up per parameter), plus 16 bytes per parameter with elements and
 * 72 bytes per bucket and element size (2 and 4 bytes) for each 16-byte
 * piece of storage that two parameters share (views carved out of one
 * buffer), until ddp_binding_free.
 * Errors: INVALID_ARG (null plan/array/out, a null pointer for a parameter
 * with numel > 0, misaligned pointer), HIP, NOMEM. */
DDP_API ddp_status_t ddp_bind_params(const ddp_plan_t *plan, void *const *param_grads,
                             void *stream, ddp_binding_t **out);
DDP_API void ddp_binding_free(ddp_binding_t *binding);

/* flat_buf[base_b + offset_p + j] = grad_p[j] for every parameter p of
 * bucket `bucket` (-1: all buckets), elements of `dtype`.  One launch; where
 * a parameter of the range starts, or the range ends, off a 16-byte
 * boundary of flat_buf, the 16-byte pieces that hold two parameters are
 * written by extra blocks at its end (a second, small launch if they do not
 * fit under the per-launch work-item limit).  Bytes of flat_buf outside the
 * range are not written.  flat_buf: device, ddp_plan_total(plan) elements, must not
 * overlap any parameter buffer.  Errors: INVALID_ARG (null, bucket out of
 * range, bad dtype, binding of another plan), HIP. */
DDP_API ddp_status_t ddp_flatten(const ddp_plan_t *plan, const ddp_binding_t *binding,
                         int32_t bucket, void *flat_buf, ddp_dtype_t dtype,
                         void *stream);

/* grad_p[j] = flat_out[base_b + offset_p + j]: the inverse copy, elements of
 * `dtype` (the sync's output type).  One launch; 16-byte pieces of storage
 * that two parameters share (views carved out of one buffer) are written
 * by extra blocks at its end, as in ddp_flatten.  Bytes outside the range's
 * parameters are not written.
 * Same arguments and errors. */
DDP_API ddp_status_t ddp_unflatten(const ddp_plan_t *plan, const ddp_binding_t *binding,
                           int32_t bucket, const void *flat_out, ddp_dtype_t dtype,
                           void *stream);

/* ------------------------------------------------------------------ reduce
 * One bucket's all-reduce + average, the operation of [TR24] 九 (sum with
 * ncclSum, then dst *= 1/world_size) and of [DDP] 4.2 (all_reduce SUM, then
 * flat_grad.div_(world_size)), on N buffers resident in one GPU.
 *   rank_ptrs[n_ranks]  host array of device pointers; rank_ptrs[r] holds
 *                       rank r's `len` elements of in_dtype
 *   n_ranks             N, 1..DDP_MAX_RANKS
 *   len                 elements in the bucket, >= 0 (0: nothing is done and
 *                       the pointers are not looked at)
 *   order               DDP_ORDER_SEQUENTIAL or DDP_ORDER_RING; for RING the
 *                       chunks are C = ceil(len/N) elements from element 0
 *   in_dtype, out_dtype f32->f32, bf16->bf16 or f32->bf16; bf16 inputs are
 *                       widened exactly and summed in FP32
 *   out                 device, `len` elements of out_dtype; every virtual
 *                       rank's result (they are identical, [DDP] 2.5).  It may
 *                       be exactly one of the inputs (in place, as ncclAllReduce
 *                       with send == recv in [TR24] 九) when the dtypes match;
 *                       any other overlap is rejected.
 *   stream              hipStream_t
 * N == 1: the result is the input, bit for bit ([TR24] 九 returns early for
 * world_size <= 1); with out == rank_ptrs[0] nothing is launched.
 * Pointers need only element alignment.  The vector kernel starts after a
 * short per-element head that puts every rank buffer on a 128-byte boundary
 * when they all sit at the same offset from one (a bucket at an unpadded
 * offset into equally aligned flat buffers), else the output; rank buffers
 * at different offsets are then read at their element alignment (a little
 * slower).  Results are identical either way.
 * Errors: INVALID_ARG, UNSUPPORTED, ALIAS, HIP. */
DDP_API ddp_status_t ddp_bucket_allreduce_avg(const void *const *rank_ptrs, int32_t n_ranks,
                                      int64_t len, ddp_order_t order,
                                      ddp_dtype_t in_dtype, ddp_dtype_t out_dtype,
                                      void *out, void *stream);

/* Every bucket of a plan in one launch (the whole synchronisation of one
 * step; bit-identical to calling ddp_bucket_allreduce_avg per bucket on the
 * bucket's sub-ranges).
 *   rank_flat[n_ranks]  host array of device pointers to each rank's flat
 *                       buffer (ddp_plan_total elements of the plan's dtype)
 *   out_flat            device, ddp_plan_total elements of out_dtype
 * RING chunks are computed per bucket (each bucket is its own all-reduce).
 * The first RING call on a device with a given n_ranks uploads the plan's
 * tables synchronously (see ddp_plan_prepare_ranks).  One launch needs
 * out_flat on a 16-byte boundary (rank buffers need only element
 * alignment); otherwise each bucket is launched on its own, as
 * ddp_bucket_allreduce_avg.
 * Errors: as ddp_bucket_allreduce_avg. */
DDP_API ddp_status_t ddp_sync_allreduce_avg(ddp_plan_t *plan, const void *const *rank_flat,
                                    int32_t n_ranks, ddp_order_t order,
                                    ddp_dtype_t out_dtype, void *out_flat,
                                    void *stream);

/* Bucket b of a plan on its own: ddp_bucket_allreduce_avg on the bucket's
 * sub-ranges of the flat buffers (elements [base_b, base_b + len_b) of each
 * rank_flat[r] and of out_flat), with the plan's occupancy policy.  DDP
 * all-reduces each bucket as soon as backward has produced it, last layers
 * first ([DDP] 3.2; [TR24] 十一): a caller runs bucket 0, 1, ... as they
 * become ready.  The buckets of one step together give the bits of one
 * ddp_sync_allreduce_avg.
 *   rank_flat, n_ranks, order, out_dtype, out_flat  as ddp_sync_allreduce_avg
 *   bucket  0..ddp_plan_num_buckets(plan) - 1
 * Errors: as ddp_bucket_allreduce_avg, plus INVALID_ARG for a bucket out of
 * range. */
DDP_API ddp_status_t ddp_sync_allreduce_avg_bucket(ddp_plan_t *plan, int32_t bucket,
                                                   const void *const *rank_flat, int32_t n_ranks,
                                                   ddp_order_t order, ddp_dtype_t out_dtype,
                                                   void *out_flat, void *stream);

/* Every bucket's average folded into one SGD step on the flat parameters,
 * in one launch: the optimizer update [TR24] 九 suggests absorbing the 1/N
 * scale into, with the update rule theta <- theta - eta * g of [DDP] 5.3.
 * Per element, with g the averaged gradient exactly as ddp_sync_allreduce_avg
 * would store it (a bf16 average is rounded, then widened back to f32):
 *     momentum_flat != NULL:  v = fl(fl(momentum * m) + g);  m = v;  g = v
 *     param:                  p = fl(p - fl(lr * g))
 * so the result equals ddp_sync_allreduce_avg followed by that step, bit for
 * bit, while the average never makes a round trip through HBM.
 *   rank_flat, n_ranks, order, out_dtype  as ddp_sync_allreduce_avg
 *   grad_out       device, ddp_plan_total elements of out_dtype, or NULL to
 *                  skip storing the average; may be exactly one of the inputs
 *   param_flat     device, ddp_plan_total f32 parameters in the plan's flat
 *                  layout, updated in place
 *   momentum_flat  device, ddp_plan_total f32 momentum buffer updated in
 *                  place (start from zeros), or NULL for plain SGD
 *   lr, momentum   learning rate and momentum factor (f32)
 * param_flat and momentum_flat may overlap no other buffer (DDP_ERR_ALIAS).
 * N == 1 takes the input as the average, bit for bit.  One launch of the
 * vector kernel (N <= 8 unrolled, N > 8 looped) at any element alignment of
 * every buffer: each is read and written with 16-byte accesses that need
 * not sit on a 16-byte boundary.
 * Errors: as ddp_sync_allreduce_avg. */
DDP_API ddp_status_t ddp_sync_sgd_update(ddp_plan_t *plan, const void *const *rank_flat, int32_t n_ranks,
                                 ddp_order_t order, ddp_dtype_t out_dtype, void *grad_out,
                                 float *param_flat, float *momentum_flat, float lr,
                                 float momentum, void *stream);

/* ------------------------------------------------------------ per-parameter
 * The whole path of one step -- flatten every rank, average every bucket,
 * unflatten ([DDP] 4.2) -- over per-parameter gradient tensors, in one
 * kernel that reads each rank's gradients where they lie and writes the
 * averages straight to per-parameter outputs.  The result equals
 * ddp_flatten (every rank) + ddp_sync_allreduce_avg + ddp_unflatten, bit for
 * bit, including the RING chunks, which follow the flat positions; the
 * bytes moved are those of the sync alone.  It is what bucket views
 * (gradient_as_bucket_view, [DDP] 4.2; [TR24] 八's region layout) give,
 * without asking for that layout.
 *
 * ddp_param_sync_create resolves everything once (a static graph, [DDP] 6.2):
 *   plan               the bucket plan; its dtype is the gradients' dtype
 *   rank_bindings[n_ranks]  host array; rank r's gradients (ddp_bind_params
 *                      with this plan, on the current device)
 *   out_binding        the per-parameter outputs (ddp_bind_params with this
 *                      plan): numel[p] elements of out_dtype each.  It may
 *                      be one of rank_bindings (in place): an output may be
 *                      exactly the same parameter's gradient of one rank
 *                      and may overlap nothing else (DDP_ERR_ALIAS);
 *                      outputs may not overlap each other
 *   order, out_dtype   as ddp_sync_allreduce_avg (N == 1: the input, bit
 *                      for bit, and out_dtype must equal the plan's dtype)
 * It uploads a table, held until ddp_param_sync_free: an 8-byte record per
 * tile of each parameter (256 f32 or 512 bf16 elements; 0.09 % of the 9 KiB
 * an f32 tile of 8 ranks reads and writes) and, per parameter with elements,
 * its n_ranks + 1 addresses and 40 bytes of position, rounded up to 16
 * bytes (Llama-7B, 8 ranks: 105 MB in all).  The bindings' addresses are copied into it: bind
 * again if a gradient moves.  Every tensor is read and written in 16- or
 * 8-byte vectors at its own element alignment (views carved out of one
 * buffer at any offset run as fast as separate tensors, within 2-3 %);
 * tile ends and ring cuts inside a vector take a per-element path (same
 * results).
 * ddp_param_sync_run enqueues the sync on `stream` (current device = the
 * device it was created on); it allocates nothing, so it can be captured.
 * Errors: INVALID_ARG (null arguments, a binding of another plan or device,
 * misaligned pointers), UNSUPPORTED, ALIAS, OVERFLOW, HIP, NOMEM. */
DDP_API ddp_status_t ddp_param_sync_create(const ddp_plan_t *plan,
                                           const ddp_binding_t *const *rank_bindings,
                                           int32_t n_ranks, const ddp_binding_t *out_binding,
                                           ddp_order_t order, ddp_dtype_t out_dtype,
                                           ddp_param_sync_t **out);
DDP_API ddp_status_t ddp_param_sync_run(const ddp_param_sync_t *sync, void *stream);

/* ddp_param_sync_run for buckets [first_bucket, first_bucket + n_buckets)
 * only: DDP's schedule ([DDP] 3.2; [TR24] 十一) averages each bucket as soon
 * as backward has produced its gradients, last layers first, so a caller
 * runs bucket 0, then 1, ..., each when it is ready.  The buckets of one
 * step together give the bits of one ddp_param_sync_run.
 * Errors: INVALID_ARG (range outside the plan's buckets), HIP. */
DDP_API ddp_status_t ddp_param_sync_run_buckets(const ddp_param_sync_t *sync, int32_t first_bucket,
                                                int32_t n_buckets, void *stream);

/* The same average folded into an SGD step on per-parameter f32 parameters:
 * ddp_sync_sgd_update for tensors that are not in the flat layout.  Per
 * element, with g the averaged gradient exactly as ddp_param_sync_run would
 * store it (a bf16 average rounded, then widened back):
 *     momentum != NULL:  v = fl(fl(mu * m) + g);  m = v;  g = v
 *     params:            p = fl(p - fl(lr * g))
 * bit for bit ddp_param_sync_run followed by that step, in one pass.
 *   rank_bindings, n_ranks, order, out_dtype  as ddp_param_sync_create
 *   grad_out   binding of per-parameter outputs for the averaged gradient
 *              (out_dtype), or NULL not to store it; may be one rank's
 *              binding (in place, as ddp_param_sync_create)
 *   params     binding of the f32 parameters (ddp_bind_params with this
 *              plan; numel[p] f32 each), updated in place
 *   momentum   binding of f32 momentum buffers (start from zeros), updated
 *              in place, or NULL for plain SGD
 * params and momentum may overlap no other tensor (DDP_ERR_ALIAS).  The
 * table holds 8 bytes per tile and 8 * (n_ranks + 3) + 40 bytes per
 * parameter, rounded up to 16.
 * ddp_param_sgd_run enqueues one step with learning rate lr and momentum
 * factor mu; it allocates nothing.  A sync made by one create function is
 * refused by the other's run function (DDP_ERR_INVALID_ARG).
 * Errors: as ddp_param_sync_create. */
DDP_API ddp_status_t ddp_param_sgd_create(const ddp_plan_t *plan,
                                          const ddp_binding_t *const *rank_bindings,
                                          int32_t n_ranks, const ddp_binding_t *grad_out,
                                          const ddp_binding_t *params,
                                          const ddp_binding_t *momentum, ddp_order_t order,
                                          ddp_dtype_t out_dtype, ddp_param_sync_t **out);
DDP_API ddp_status_t ddp_param_sgd_run(const ddp_param_sync_t *sync, float lr, float mu,
                                       void *stream);
/* The SGD step of buckets [first_bucket, first_bucket + n_buckets) only, as
 * ddp_param_sync_run_buckets. */
DDP_API ddp_status_t ddp_param_sgd_run_buckets(const ddp_param_sync_t *sync, int32_t first_bucket,
                                               int32_t n_buckets, float lr, float mu,
                                               void *stream);

/* Frees a sync made by ddp_param_sync_create or ddp_param_sgd_create. */
DDP_API void ddp_param_sync_free(ddp_param_sync_t *sync);

/* Local gradient accumulation between synchronisations: the no_sync
 * micro-steps of [DDP] 5.2, where backward adds each micro-batch's gradient
 * into .grad and only the last micro-step synchronises.  For every pair k,
 * in one launch:  dst[k][i] = fl(dst[k][i] + src[k][i])  (bf16: both widened,
 * one f32 add, one round to nearest even).
 *   dst[n_bufs], src[n_bufs]  host arrays of device pointers to len elements
 *                             of dtype; n_bufs 1..DDP_MAX_RANKS (one pair
 *                             per virtual rank)
 * dst[k] may be exactly src[k]; any other overlap between the buffers is
 * rejected (DDP_ERR_ALIAS).  Buffers need only element alignment (one
 * vector kernel for any offset).  len == 0 does nothing.
 * Errors: INVALID_ARG, UNSUPPORTED, OVERFLOW, ALIAS, HIP. */
DDP_API ddp_status_t ddp_accumulate(void *const *dst, const void *const *src, int32_t n_bufs, int64_t len,
                            ddp_dtype_t dtype, void *stream);

/* ------------------------------------------------------------ no allocation
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * ddp_sync_allreduce_avg with the same arguments and the same result, bit
 * for bit, that never allocates device memory and calls no allocating HIP
 * routine.  Where ddp_sync_allreduce_avg reads the plan's device tables
 * (RING order with out_flat on a 16-byte boundary), this call rebuilds them
 * on `stream`, before the reduce, in a static device buffer of
 * DDP_NOALLOC_SCRATCH_BYTES that each device holds from its first such call
 * until the process ends: the bucket bases ((n_buckets + 1) * 8 bytes), a
 * bucket index per 64 tiles and a 4-byte ring word per tile (tiles of 256
 * f32 or 512 bf16 elements), each part rounded up to 256 bytes.  That fits
 * about 16 M tiles: 4.2 G f32 or 8.4 G bf16 elements.  Every other case is
 * ddp_sync_allreduce_avg's own path, which allocates nothing there.
 *
 * Every call on a device shares that device's buffer and leaves its
 * contents behind; calls that overlap on one device (on different streams
 * without an ordering between them) race on it and may give wrong results.
 * Calls on one stream, or ordered by events, are safe.
 * Errors: as ddp_sync_allreduce_avg, plus DDP_ERR_CAPACITY when the plan's
 * tables exceed the buffer (nothing is enqueued), DDP_ERR_UNSUPPORTED for a
 * device index of 64 or more. */
#define DDP_NOALLOC_SCRATCH_BYTES (64ll << 20)
DDP_API ddp_status_t ddp_sync_allreduce_avg_noalloc(ddp_plan_t *plan,
                                                    const void *const *rank_flat,
                                                    int32_t n_ranks, ddp_order_t order,
                                                    ddp_dtype_t out_dtype, void *out_flat,
                                                    void *stream);

/* ------------------------------------------------------------------ occupancy
 * How many blocks of the streaming kernels (reduce, fused SGD step, flatten /
 * unflatten, per-parameter sync) may be resident on one CU.
 *   DDP_OCCUPANCY_TUNED   each launch is capped at the number of resident
 *       blocks per CU measured fastest for its kernel and rank count, by
 *       asking for an unused share of the CU's LDS.  Best for a
 *       synchronisation that has the GPU to itself.
 *   DDP_OCCUPANCY_SHARED  no cap.  The reserved LDS keeps other kernels'
 *       LDS-using blocks (a GEMM's, say) off a CU while the reduce runs
 *       there; when syncs overlap compute on other streams this policy
 *       shortens the overlapped step by a few percent (more for the
 *       per-parameter sync, whose tuned cap is higher).
 *   DDP_OCCUPANCY_DEFAULT (objects only) follow the process-wide policy.
 * The policy is a property of each plan and each per-parameter sync: the
 * launches of a call that takes one (ddp_sync_allreduce_avg[_bucket,
 * _noalloc], ddp_sync_sgd_update, ddp_flatten / ddp_unflatten with that
 * plan; ddp_param_sync_run[_buckets], ddp_param_sgd_run[_buckets]) follow
 * the object's, so that the syncs a caller overlaps with compute and those
 * it runs alone can differ without touching shared state.  A new object
 * has DDP_OCCUPANCY_DEFAULT; calls without an object (ddp_bucket_allreduce_avg,
 * ddp_accumulate) and objects left at DEFAULT follow the process-wide
 * policy, DDP_OCCUPANCY_TUNED unless ddp_set_occupancy changed it.
 * Results do not depend on any of it, only timing. */
typedef enum {
    DDP_OCCUPANCY_TUNED = 0,
    DDP_OCCUPANCY_SHARED = 1,
    DDP_OCCUPANCY_DEFAULT = 2
} ddp_occupancy_t;

/* Process-wide policy (TUNED or SHARED), for launches made after the call.
 * Errors: INVALID_ARG (not TUNED or SHARED). */
DDP_API ddp_status_t ddp_set_occupancy(ddp_occupancy_t policy);
DDP_API ddp_occupancy_t ddp_get_occupancy(void);

/* A plan's own policy (TUNED, SHARED or DEFAULT), for the calls that take
 * the plan, from the next call on.  Errors: INVALID_ARG (null plan, bad
 * value). */
DDP_API ddp_status_t ddp_plan_set_occupancy(ddp_plan_t *plan, ddp_occupancy_t policy);
/* The plan's policy as set (DEFAULT if never set), or DEFAULT for NULL. */
DDP_API ddp_occupancy_t ddp_plan_get_occupancy(const ddp_plan_t *plan);

/* The same for a per-parameter sync or SGD step. */
DDP_API ddp_status_t ddp_param_sync_set_occupancy(ddp_param_sync_t *sync, ddp_occupancy_t policy);
DDP_API ddp_occupancy_t ddp_param_sync_get_occupancy(const ddp_param_sync_t *sync);

/* ------------------------------------------------------------------ misc */
DDP_API const char *ddp_status_string(ddp_status_t status);
/* Text of the last HIP failure seen by this thread ("" if none): the HIP call
 * and the runtime's error string.  Valid until the thread's next failure. */
DDP_API const char *ddp_last_error(void);
DDP_API int32_t ddp_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DDP_H */
