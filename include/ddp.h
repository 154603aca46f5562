/* ddp.h — bucketed gradient reduction for data-parallel training, MI355X (gfx950).
 *
 * C ABI of libddp.so. Plain pointers and sizes only; every function returns
 * an int status (DDP_OK = 0, negative on error, text in ddp_last_error())
 * unless stated otherwise. No exception ever leaves an entry point: host
 * memory exhaustion anywhere in a call is DDP_ERR_NOMEM, and a call that
 * fails that way leaves the reducer as it was before the call (a launch
 * that could not be issued counts as a failed launch, see ddp_mark_ready).
 *
 * Sources (cited by tag and section):
 *   [DDP-ch17]    "PyTorch 训练框架内核深度解析", chapter 17
 *                 "DDP：环形 AllReduce 与梯度桶" (yangyitao.com)
 *   [L15]         CMU 11-868 lecture 15 notes, "分布式训练（二）：PyTorch DDP 的
 *                 设计与实现" (semidirectx.com)
 *   [MegatronDDP] "Megatron DDP：连续 buffer 与通信 overlap" (llm-infra-atlas)
 *   [PTD-notes]   notes on "PyTorch Distributed: Experiences on Accelerating
 *                 Data Parallel Training" (arcsin2.cloud)
 *
 * On one GPU the W data-parallel replicas are W gradient buffers resident in
 * HBM, so a bucket "all-reduce" is one streaming kernel: it reads the bucket
 * from all W replicas, scales by 1/W, sums in the ring all-reduce's order and
 * writes the identical mean back to all W replicas' flat buffers (or, as a
 * reduce-scatter, each ring chunk to its owner only). Built-in bf16 / fp16
 * compression hooks change that arithmetic; unused-parameter detection
 * masks replicas out per gradient.
 *
 * Memory ownership: the caller allocates and owns every device buffer
 * (gradients, flat buffers, workspace) and both streams; they must stay
 * valid until ddp_reducer_destroy returns. The library copies the plan and
 * the pointer tables into its own host memory at creation and writes its
 * device tables into the caller's workspace; it allocates no device memory.
 * With unused-parameter detection it allocates one pinned host staging
 * buffer (hipHostMalloc) of two copies of its segment table, 96 bytes per
 * segment (a segment is the part of one gradient inside one ring chunk, so
 * at most P + B * W of them), freed by ddp_reducer_destroy.
 *
 * Threading: a reducer is used from one thread at a time (hooks fire from
 * one thread, [DDP-ch17 §17.12]); that thread may change between calls, as
 * when autograd runs gradient hooks on its device worker thread while the
 * caller's thread waits in backward and calls ddp_finish afterwards.
 * Calls on different reducers may run concurrently. ddp_last_error() text is
 * per thread: read it on the thread whose call failed.
 */
#ifndef DDP_H
#define DDP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DDP_OK = 0,
    DDP_ERR_INVALID = -1,        /* bad argument or inconsistent plan                                */
    DDP_ERR_ALREADY_READY = -2,  /* a gradient marked ready twice in one backward [DDP-ch17 §17.16];
                                    text "Expected to mark a variable ready only once: ..."        */
    DDP_ERR_UNFINISHED = -3,     /* new iteration while buckets of the last one never launched
                                    [DDP-ch17 §17.6; L15 §4.2]; text "Expected to have finished
                                    reduction in the prior iteration before starting a new one.
                                    Parameter indices which did not receive grad: i j ..."         */
    DDP_ERR_NOT_READY = -4,      /* finish while some buckets still wait for gradients; the text
                                    ends "Parameter indices which did not receive grad: i j ..."
                                    [DDP-ch17 §17.6]                                                */
    DDP_ERR_ORDER = -5,          /* explicit reduce of a bucket whose gradients are not all ready   */
    DDP_ERR_HIP = -6,            /* a HIP runtime call failed (its text is in ddp_last_error)        */
    DDP_ERR_HOOK = -7,           /* a registered communication hook returned non-zero               */
    DDP_ERR_NOMEM = -8           /* host memory ran out (an allocation inside the library failed)  */
};

enum {
    DDP_ORDER_REVERSE = 0,          /* parameters P-1 .. 0: reverse registration order
                                       [DDP-ch17 §17.3.1; L15 §2.2]                                  */
    DDP_ORDER_GIVEN = 1,            /* the caller's order, e.g. the ready order recorded in an
                                       earlier iteration (rebuild) [DDP-ch17 §17.13]                 */
    DDP_ORDER_FWD_THEN_REVERSE = 2  /* form buckets in forward order, then reverse the list of
                                       buckets (layout without a rebuild) [DDP-ch17 §17.13]          */
};

enum {
    DDP_IN_F32_COPY = 0,        /* fp32 per-parameter gradients, copied into the flat buffer while
                                   being reduced [DDP-ch17 §17.5, §17.12]                           */
    DDP_IN_F32_VIEW = 1,        /* the gradients already live in the flat buffer (bucket views),
                                   reduced in place [DDP-ch17 §17.5]                               */
    DDP_IN_BF16_ACCUM_F32 = 2   /* bf16 weight gradients accumulated into the fp32 flat main_grad
                                   buffer, then reduced in place [MegatronDDP §1]                   */
};

/* ---------------------------------------------------------------------------
 * ddp_plan_buckets — assign gradients to buckets. Host only, no device.
 *
 * Walks the parameters in the order the mode selects, appends each one to
 * the open bucket and seals the bucket as soon as its bytes reach the cap
 * (so a bucket may exceed it) [DDP-ch17 §17.2; L15 §2.2, §8 exercise 3].
 * The first bucket formed uses first_cap_bytes (1 MiB after a rebuild in
 * PyTorch), every later one cap_bytes (25 MiB by default) [DDP-ch17 §17.2,
 * §17.13]. cap_bytes = INT64_MAX gives one bucket (PyTorch's first
 * iteration) and 0 one bucket per gradient [L15 §3.2]. Megatron's bucket size
 * max(40 MB, 1 MB x DP) is passed as cap = first cap [MegatronDDP §1].
 *
 * Buckets are numbered in launch order. Inside a bucket, gradients are laid
 * out back to back in append order (bytes, no padding); buckets follow one
 * another in the flat buffer, bucket 0 first.
 *
 *   n_params          P >= 0
 *   param_bytes       [P] bytes of each gradient (>= 0; multiples of 4 for the reducer)
 *   order             [P] permutation of 0..P-1, read only for DDP_ORDER_GIVEN (may be NULL otherwise)
 *   order_mode        DDP_ORDER_*
 *   cap_bytes, first_cap_bytes   >= 0
 * Outputs (caller-allocated, each may be NULL if not wanted):
 *   bucket_of         [P] bucket index of each gradient
 *   offset_in_bucket  [P] byte offset of each gradient inside its bucket
 *   bucket_params     [P] gradient indices bucket by bucket, append order
 *   bucket_nparams    [P] gradients per bucket (first *n_buckets entries used)
 *   bucket_bytes      [P] bytes per bucket (first *n_buckets entries used)
 *   n_buckets         number of buckets (required)
 * Errors: DDP_ERR_INVALID for negative sizes or caps, a missing required
 * array, or an order that is not a permutation.
 * ------------------------------------------------------------------------- */
int ddp_plan_buckets(int32_t n_params, const int64_t *param_bytes, const int32_t *order, int32_t order_mode,
                     int64_t cap_bytes, int64_t first_cap_bytes, int32_t *bucket_of, int64_t *offset_in_bucket,
                     int32_t *bucket_params, int32_t *bucket_nparams, int64_t *bucket_bytes, int32_t *n_buckets);

/* ---------------------------------------------------------------------------
 * Reducer: one model's gradients over W replicas, reduced bucket by bucket.
 * ------------------------------------------------------------------------- */
enum {
    DDP_ALL_REDUCE = 0,      /* every replica receives the whole reduced bucket (DDP) [DDP-ch17 §17.4]     */
    DDP_REDUCE_SCATTER = 1   /* replica c receives only ring chunk c of it (ZeRO-1, distributed optimizer)
                                [MegatronDDP §3]; chunk c = [c*q, min((c+1)*q, n)), q = ceil(n/W). The
                                sum is folded exactly as for DDP_ALL_REDUCE, so the owned shard is bit-identical
                                to the same slice of the all-reduce result; the rest of each replica's flat
                                buffer is left as it was (in-place modes: unreduced input).             */
};

typedef struct ddp_reducer ddp_reducer;   /* opaque, owned by the library */

typedef struct {
    int32_t world;                     /* W replicas, 1 <= W <= 1024 (<= 64 with find_unused)      */
    int32_t n_params;                  /* P >= 0                                                    */
    const int64_t *param_numel;        /* [P] elements per gradient                                 */
    const int32_t *bucket_of;          /* [P] a plan (e.g. from ddp_plan_buckets)                   */
    const int64_t *offset_in_bucket;   /* [P] bytes, multiples of 4; each bucket's gradients must
                                          tile [0, bucket bytes) exactly                            */
    int32_t n_buckets;                 /* every bucket must hold at least one gradient              */
    int32_t input_mode;                /* DDP_IN_*                                                  */
    const void *const *grads;          /* [W*P] device pointers, entry w*P + p = replica w's
                                          gradient p: fp32 (COPY) or bf16 (BF16_ACCUM); unused and
                                          may be NULL for VIEW                                      */
    float *const *flat;                /* [W] device pointers: replica w's flat fp32 buffer of
                                          sum(bucket bytes) bytes, laid out by the plan (the bucket
                                          buffer, or main_grad in BF16_ACCUM mode). NULL: no device
                                          is used and a communication hook must be registered
                                          before any bucket launches                               */
    void *workspace;                   /* device memory of ddp_workspace_bytes() bytes, 256-B
                                          aligned; unused when flat is NULL                         */
    size_t workspace_bytes;
    void *compute_stream;              /* hipStream_t on which gradients are produced               */
    void *comm_stream;                 /* hipStream_t on which bucket reductions run (a side
                                          stream that overlaps backward [PTD-notes §2.3])           */
    int32_t collective;                /* DDP_ALL_REDUCE (0) or DDP_REDUCE_SCATTER                  */
    int32_t find_unused;               /* != 0: per-replica used tables (ddp_set_local_used) decide
                                          which gradients contribute; W <= 64 [DDP-ch17 §17.33]     */
} ddp_reducer_desc;

/* Device workspace the reducer needs for its tables (segments, tiles,
 * pointers): the device-side counterpart of the Reducer's bucket list
 * [DDP-ch17 §17.2]. Returns 0 and sets ddp_last_error() if the desc is
 * invalid (or host memory runs out). */
size_t ddp_workspace_bytes(const ddp_reducer_desc *desc);

/* The Reducer [DDP-ch17 §17.2, §17.14]: built once from the parameter list
 * and its bucket plan, it holds the buckets, each bucket's pending count and
 * the per-gradient ready hooks' state. Validates the desc, copies the plan,
 * builds and uploads the device tables (synchronously) and leaves the
 * reducer ready for its first backward. *out is set only on success.
 * Errors: DDP_ERR_INVALID (bad desc or buffers), DDP_ERR_HIP, DDP_ERR_NOMEM;
 * nothing is left allocated on failure. */
int ddp_reducer_create(const ddp_reducer_desc *desc, ddp_reducer **out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * reducer as ddp_reducer_create, with its device tables in a static table
 * area the library owns instead of a caller-allocated workspace
 * (desc->workspace and desc->workspace_bytes are ignored). The call and the
 * reducer allocate no device memory: the area is a device array of
 * DDP_STATIC_TABLE_BYTES per GPU, which every GPU the library runs on holds
 * until the process ends. The caller still passes the gradient and flat
 * buffers and both streams.
 *  - One area per device, shared by every static reducer on it: creating a
 *    static reducer first waits for the device to drain (so reductions
 *    already queued by an earlier one finish), then rewrites the area; the
 *    earlier static reducer then refuses to launch (DDP_ERR_INVALID). Calls
 *    that overlap on one device (from several host threads) race.
 *  - Unused-parameter detection (desc->find_unused) is not supported: its
 *    mask staging needs pinned host memory (DDP_ERR_INVALID).
 *  - Tables larger than DDP_STATIC_TABLE_BYTES are refused (DDP_ERR_INVALID,
 *    with the size needed); ddp_workspace_bytes gives that size.
 * It also creates the reducer's HIP events and host-side state, as
 * ddp_reducer_create does. Released by ddp_reducer_destroy. */
#define DDP_STATIC_TABLE_BYTES (16u << 20)
int ddp_reducer_create_static(const ddp_reducer_desc *desc, ddp_reducer **out);

/* Ends a Reducer [DDP-ch17 §17.2]: waits for every reduction it queued on
 * its comm stream (as the end of backward waits for each bucket's
 * collective, [DDP-ch17 §17.41]), then releases host state, events and
 * staging; the caller's buffers are untouched and may be freed once this
 * returns. Reductions the caller queued on other streams through
 * ddp_bucket_reduce are the caller's to wait for. NULL is a no-op. The
 * reducer is released even when the wait reports an error (DDP_ERR_HIP). */
int ddp_reducer_destroy(ddp_reducer *r);

/* Resets every bucket's pending count and the per-iteration ready set before
 * a backward [DDP-ch17 §17.12, §17.16]. DDP_ERR_UNFINISHED if gradients were
 * marked since the last reset but the iteration was never finished; the
 * message lists the gradients that got none, ascending [DDP-ch17 §17.6]. A
 * backward in which a launch failed needs no ddp_finish: its error was
 * already returned, and the reset discards its used tables. */
int ddp_prepare_for_backward(ddp_reducer *r);

/* The gradient-ready hook for gradient `param` [DDP-ch17 §17.3, §17.12; L15
 * §2.3; MegatronDDP §2]: decrements its bucket's pending count, then launches
 * bucket groups (ddp_set_bucket_groups; by default one bucket each) strictly
 * in order, from the first unlaunched one, for as long as every count in the
 * group is zero. With unused-parameter detection, the backward's first mark
 * also marks every gradient no replica used. A launch makes the comm stream
 * wait for the work queued so far on the compute stream (no wait is enqueued
 * when that stream has already drained), then runs the registered hook once
 * per bucket or, by default, one bucket-reduce kernel over the launched
 * buckets on the comm stream. May launch 0..B buckets. Inside no_sync the
 * call only checks the index (see ddp_set_require_sync).
 * Errors: DDP_ERR_INVALID (index out of range), DDP_ERR_ALREADY_READY,
 * DDP_ERR_HIP, DDP_ERR_HOOK (a launch failed; the mark itself counts). A
 * failed launch ends the backward's reductions: the buckets from the one
 * that failed on are not reduced, every later launch in the same backward is
 * refused with the same code, and ddp_finish reports the failure.
 * Stream capture: while the compute stream is being recorded into a HIP
 * graph (hipStreamBeginCapture, or a framework's graph capture on that
 * stream), a launch never queries the compute stream. It always waits on it
 * through the reducer's event, which the graph keeps as an edge from the
 * recorded backward to the reduction, and every launch but the one holding
 * the last bucket takes the shape for running beside a backward. Per-launch
 * timing and unused-parameter detection are refused there (DDP_ERR_INVALID,
 * before anything is enqueued, so the capture stays usable): a replay cannot
 * read timing events on the host nor change the replica masks. Create the
 * reducer before the capture begins (creation uploads its tables
 * synchronously). */
int ddp_mark_ready(ddp_reducer *r, int32_t param);

/* ddp_mark_ready for params[0], params[1], ... in that order, in one call
 * (gradients that become ready together, e.g. the weight and bias of one
 * layer, or every gradient at once after a backward without overlap).
 * Buckets completed by the call are launched at its end, in index order;
 * without a registered hook, consecutive ones go out as ONE kernel launch (a
 * coalesced bucket group [MegatronDDP §3]), results identical to separate
 * launches. Stops at the first failing mark and returns its error (buckets
 * completed before it are still launched); *n_done (may be NULL) receives how
 * many marks succeeded. */
int ddp_mark_ready_many(ddp_reducer *r, const int32_t *params, int32_t n, int32_t *n_done);

/* The default communication hook: enqueues the reduction of `bucket` on
 * `stream` (a hipStream_t; NULL is the null stream) without waiting for any
 * other stream. Callable from a registered hook, or on its own for timing.
 * During an iteration it refuses (DDP_ERR_ORDER) a bucket not yet launched by
 * ddp_mark_ready, whose gradients may still be in flight.
 *
 * Per element e of the bucket (n elements, chunk length q = ceil(n/W),
 * chunk c = e / q): t_w = x_w[e] * fp32(1/W) (COPY, VIEW) or
 * (main_w[e] + fp32(wgrad_w[e])) * fp32(1/W) (BF16_ACCUM);
 * acc = t_c, then acc += t_{c+1}, ..., t_{c+W-1} (indices mod W), each an
 * fp32 add rounded to nearest even: the value the ring reduce-scatter leaves
 * for chunk c [DDP-ch17 §17.4, §17.9; MegatronDDP §3]. acc is written to
 * element e of all W flat buffers (the all-gather), or, for
 * DDP_REDUCE_SCATTER, to replica c's flat buffer only. That is the default
 * hook's arithmetic; a compression hook (ddp_register_builtin_hook) changes
 * the term and every add as described there. With unused-parameter
 * detection the reduction applies the replica masks last uploaded (all
 * replicas before the first synchronized backward's first launch); the
 * masks travel in the segment table, which the comm stream rewrites, so on
 * any other stream the reduction is made to wait for the work queued so far
 * on the comm stream, and the comm stream to wait for the reduction (two
 * events; results do not depend on the stream). On a stream being recorded
 * into a HIP graph, a reducer with unused-parameter detection, or with
 * per-launch timing on, refuses (DDP_ERR_INVALID, nothing enqueued). */
int ddp_bucket_reduce(ddp_reducer *r, int32_t bucket, void *stream);

/* End of backward [DDP-ch17 §17.41; MegatronDDP §5]: checks that every bucket
 * launched (DDP_ERR_NOT_READY otherwise, listing the gradients not marked
 * ready), then makes the compute stream wait for the comm stream; with
 * host_blocking != 0 the host also waits for the reductions to complete.
 * If a launch of this backward failed, it returns that launch's error code
 * (DDP_ERR_HOOK or DDP_ERR_HIP), naming the buckets that were not reduced,
 * and ends the backward. While the compute stream is being recorded into a
 * HIP graph, host_blocking != 0 is refused (DDP_ERR_INVALID) and nothing
 * changes; a non-blocking finish records the comm stream's join into the
 * compute stream, which the capture needs before it ends. */
int ddp_finish(ddp_reducer *r, int32_t host_blocking);

/* no_sync [L15 §4.1; PTD-notes §2.2.4]: with sync == 0, the backward passes
 * prepared from now on do not reduce: ddp_mark_ready only checks the index,
 * ddp_finish does nothing, and gradients are left to accumulate locally in
 * the caller's buffers; the next backward prepared with sync != 0 reduces the
 * accumulated sum. The flag is read by ddp_prepare_for_backward. Default 1. */
int ddp_set_require_sync(ddp_reducer *r, int32_t sync);

/* Unused-parameter detection (desc.find_unused) [DDP-ch17 §17.33; L15 §4.2;
 * PTD-notes §2.2.3, §3.2]. used: [W*P] host bytes, entry w*P + p != 0 when
 * replica w produced gradient p in this backward. Call after
 * ddp_prepare_for_backward and before the backward's first ddp_mark_ready.
 * Tables OR together over every backward since the last synchronized one
 * (no_sync passes included). In the next synchronized backward:
 *  - at the first ready mark, gradients no replica used are marked ready;
 *  - a replica that did not use gradient p contributes a zero-filled slice
 *    (its source is not read);
 *  - gradients no replica used are not written (their flat-buffer slices keep
 *    their contents).
 * The reduced tables go to the device once per synchronized backward, on the
 * comm stream, ahead of its first reduction, as a fresh copy of the segment
 * table (48 bytes per segment, each record carrying its gradient's replica
 * mask), unless the masks equal those the device already holds. Without a
 * call every replica
 * counts as having used every gradient. Errors: DDP_ERR_INVALID if detection
 * is off or the backward already started. */
int ddp_set_local_used(ddp_reducer *r, const uint8_t *used);

/* Replaces the default hook [DDP-ch17 §17.9, §17.20; L15 §2.2]: fn(ctx, b)
 * is called for each bucket launch, in launch order, after the comm stream
 * was made to wait on the compute stream. fn = NULL restores the default. */
typedef int (*ddp_comm_hook_fn)(void *ctx, int32_t bucket);
int ddp_register_comm_hook(ddp_reducer *r, ddp_comm_hook_fn fn, void *ctx);

/* Bucket groups [MegatronDDP §3]: consecutive buckets whose reductions are
 * issued together, as one launch, once every bucket of the group is ready
 * and every earlier group was issued. This trades overlap for fewer launches
 * (one launch overhead per group instead of per bucket), which pays at small
 * caps. first_bucket: [n_groups] strictly increasing bucket indices, the
 * first 0; group g = [first_bucket[g], first_bucket[g+1]) (the last group
 * runs to the end). n_groups = 0 (first_bucket may be NULL) restores the
 * default, one group per bucket. The reducer keeps its own copy.
 * Independently of groups, buckets completed by one ready call
 * (ddp_mark_ready_many) always go out as one launch.
 * Errors: DDP_ERR_INVALID for a malformed list; DDP_ERR_UNFINISHED while a
 * backward is in flight. */
int ddp_set_bucket_groups(ddp_reducer *r, const int32_t *first_bucket, int32_t n_groups);

/* Built-in communication hooks [DDP-ch17 §17.9]: the arithmetic every
 * bucket reduction of this reducer uses (the reducer's own launches and
 * ddp_bucket_reduce, also from a callback hook).
 *  DDP_HOOK_ALLREDUCE: the default; each replica's gradient is scaled by
 *    fp32(1/W) and the terms are summed in fp32.
 *  DDP_HOOK_BF16_COMPRESS / DDP_HOOK_FP16_COMPRESS: each replica's bucket
 *    (in bf16 mode: main_grad + wgrad, summed in fp32) is cast to the 16-bit
 *    wire format (round to nearest even) and divided by W in fp32, rounded to
 *    the wire format again; every hop of the ring sum is an fp32 add rounded
 *    to the wire format; the result is widened into the fp32 buckets. These
 *    halve the bytes a collective would send and lose precision; fp16 turns a
 *    gradient beyond its range (|x| >= 65520) into inf.
 * The flat buffers stay fp32 in HBM, so the single-GPU pass moves the same
 * HBM bytes under every hook. Errors: DDP_ERR_INVALID for an unknown hook;
 * DDP_ERR_UNFINISHED while a backward is in flight. */
enum {
    DDP_HOOK_ALLREDUCE = 0,
    DDP_HOOK_BF16_COMPRESS = 1,
    DDP_HOOK_FP16_COMPRESS = 2
};
int ddp_register_builtin_hook(ddp_reducer *r, int32_t hook);

/* Workgroups of one reduction launch that may share a CU. The kernel uses no
 * LDS; a launch reserves LDS only so that the hardware dispatcher keeps at
 * most n of its workgroups on a CU. Fewer tiles in flight keep the 2W
 * streams' windows narrow, which suits HBM: on MI355X this measured 2-8%
 * faster than full occupancy for 3 <= W <= 32. The reserved LDS and the
 * wave slots are unavailable to kernels that share the CUs, such as the
 * backward's GEMMs.
 *   n = 0  automatic (default): none for W <= 2 and for W > 32; two per CU
 *          for the reduce-scatter and for the all-reduce at W = 5..32;
 *          except that the all-reduce at W = 3, 4 runs one per CU (none in
 *          DDP_IN_BF16_ACCUM_F32 mode) and the DDP_IN_BF16_ACCUM_F32
 *          all-reduce at W = 16 runs one per CU. A launch of a managed
 *          backward (ddp_mark_ready*) that does not hold the backward's last
 *          bucket, issued while the compute stream has work queued, runs
 *          beside the backward's remaining kernels [PTD-notes §2.2.3] and
 *          takes at most one per CU; the last launch, which runs after the
 *          backward's final kernels, keeps the rule above;
 *   n < 0  no cap (no LDS reserved; occupancy limited by registers only);
 *   1..8   at most n per CU.
 * At one workgroup per CU (by either rule) the all-reduce at W = 5..8 gives
 * each workgroup two consecutive tiles, so a CU keeps the bytes in flight of
 * the two single-tile workgroups the automatic rule allows, in half the
 * workgroups (BERT-large with bf16 GEMMs as its backward, MI355X: the
 * overlapped step 0.92-1.58 ms shorter than the serial one, median 1.27 ms
 * over six runs, against 0.40-0.49 ms with two single-tile workgroups per CU
 * beside the backward). A managed
 * backward without backward kernels, such as back-to-back reductions marked
 * one bucket at a time, cannot be told apart and takes the same shape: its
 * launches ran 5-7% below the tuned rule.
 * The instance for the DDP_IN_BF16_ACCUM_F32 all-reduce at W = 16 is compiled
 * for one wave per SIMD (all of its loads in flight), so it holds one
 * workgroup per CU whatever n allows.
 * Takes effect at the next launch; results do not depend on it.
 * Errors: DDP_ERR_INVALID for n > 8. ddp_get_launch_lds reports the LDS bytes
 * each workgroup of the next launch will reserve when no backward runs beside
 * it (0: none). */
int ddp_set_workgroups_per_cu(ddp_reducer *r, int32_t n);
int ddp_get_launch_lds(const ddp_reducer *r, int32_t *lds_bytes);

/* Plan introspection (bucket sizes and members, [DDP-ch17 §17.39]). */
int ddp_get_bucket(const ddp_reducer *r, int32_t bucket, int64_t *bytes, int64_t *flat_offset_bytes,
                   int32_t *n_params);
/* params: [n_params of that bucket], in flat-buffer order */
int ddp_get_bucket_params(const ddp_reducer *r, int32_t bucket, int32_t *params);
/* Gradients in the order they were marked ready since the last reset, the
 * input of a rebuild with DDP_ORDER_GIVEN [DDP-ch17 §17.13]. order: [P]. */
int ddp_get_ready_order(const ddp_reducer *r, int32_t *order, int32_t *n);
/* Buckets launched since the last reset. */
int ddp_get_launched(const ddp_reducer *r, int32_t *n_launched);

/* Per-launch timing: while enabled, each default reduction launch (one
 * bucket, or a coalesced group) is bracketed by two HIP events on the stream
 * it runs on (timing-only events, without the system-scope fence). The
 * events form a fixed ring of 256 pairs, created on first use and freed by
 * ddp_reducer_destroy: when launch i reuses the pair of launch i - 256, the
 * host first waits for that launch to complete and copies its duration into
 * a host record (12 bytes per launch). Enabling (again) starts a new record
 * list.
 * ddp_get_timings copies up to `capacity` records (launch order) of the
 * launches since timing was last enabled: the first bucket, the number of
 * buckets the launch covered, and the kernel's duration in ms. With ms
 * non-NULL it waits for the launches it reports to complete. *n = number of
 * records. Any output array may be NULL. */
int ddp_set_timing(ddp_reducer *r, int32_t enable);
int ddp_get_timings(const ddp_reducer *r, int32_t *first_bucket, int32_t *n_buckets, float *ms, int32_t capacity,
                    int32_t *n);

/* Text of the last error on this thread ("" if none). Never NULL. Where the
 * pages give PyTorch's wording of a Reducer error, the text starts with it
 * (DDP_ERR_ALREADY_READY, DDP_ERR_UNFINISHED, DDP_ERR_NOT_READY above:
 * [DDP-ch17 §17.6, §17.16; L15 §4.2]). The pointer stays valid until the
 * next failing call on the same thread. */
const char *ddp_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DDP_H */
