/*
 * pkvs.h -- C ABI of libpkvs: batched attention over a paged KV cache with a
 * sliding-window mask, for AMD Instinct MI355X (gfx950).
 *
 * Sources the operations follow (the web pages, cited by title and section):
 *  [PR31501] sglang PR "[flashinfer] Pass window_left at plan time for the
 *            SWA paged prefill wrapper" -- section "What": window_left must be
 *            fixed when the work is planned, the per-element left-window mask
 *            must always be applied (a per-tile KV-start skip alone leaks), and
 *            the plan/run consistency check must hold.
 *  [FIB]     sglang python/sglang/srt/layers/attention/flashinfer_backend.py --
 *            fast_prefill_plan (plan from host-known CSR layout, no device-to-
 *            host copy), FlashInferAttnBackend.forward_extend / forward_decode
 *            (the run calls: sm_scale, window_left, causal, NHD paged cache,
 *            q viewed as [tokens, heads, head_dim]), _safe_merge_state (the
 *            (v_a, s_a, v_b, s_b) -> (v, s) combine launched over a (token,
 *            head) grid), _full_cg_prefill_workspace_bytes (a fixed grid whose
 *            idle blocks exit early; "increase the workspace" failure at plan),
 *            should_use_tensor_core (grouped heads share each K/V load),
 *            FlashInferIndicesUpdaterPrefill.update_sliding_window and
 *            _build_swa_prefix_custom_mask (the cascade's trimmed prefix
 *            table and its left-window mask).
 *  [PR234]   AMD-Ecosystem/flashinfer PR "fix(rocm): correct AITER decode
 *            backend gaps -- sliding window, CUDA graph, return_lse" --
 *            "Why each fix" 1 (window_left = W: the query at kv_len-1 sees W+1
 *            keys, W = 0 is one key and never "disabled"), 2 (a launch grid
 *            sized from per-plan batch scalars breaks replay with a larger
 *            batch; reject at plan time), 3 (LSE is requested per run call).
 *
 * Conventions shared by every entry point
 *  - Status: 0 (PKVS_OK) or a negative pkvs_status.  Nothing throws across
 *    the ABI; pkvs_last_error() returns a thread-local detail message.
 *  - Device pointers are HIP device memory owned by the caller.  The library
 *    owns only the opaque pkvs_plan (and the pinned host staging buffers it
 *    holds).  run() calls allocate nothing and are asynchronous on `stream`.
 *    q, o, k_cache, v_cache (and a cascade's k_extend, v_extend) and the two
 *    workspaces must be 16-byte aligned (INVALID_ARG otherwise): the kernels
 *    move their rows in 16-byte vectors.
 *  - Layouts (all row-major, contiguous):
 *      q, o        [nnz_qo, num_qo_heads, head_dim]   (decode: nnz_qo = batch)
 *      lse         [nnz_qo, num_qo_heads] float32, natural log of the sum of
 *                  exp(sm_scale * q.k) over the visible keys; -inf if none
 *      k_cache, v_cache  [num_pages, page_size, num_kv_heads, head_dim] ("NHD")
 *      qo_indptr   [batch+1] int32, query tokens of request b are
 *                  qo_indptr[b] .. qo_indptr[b+1]-1
 *      kv_indptr   [batch+1] int32, in pages; kv_indices[kv_indptr[b] + i] is
 *                  the i-th page of request b
 *      kv_last_page_len [batch] int32 in [1, page_size] (0 for a request with
 *                  no pages);  kv_len_b = (npages_b - 1) * page_size + last_b
 *  - Query i of request b sits at position p = kv_len_b - qo_len_b + i (its
 *    keys are already in the cache).  Key j is visible to it iff
 *        j <= p (causal)  and  (window_left < 0  or  j >= p - window_left).
 *    Query head h reads KV head h / (num_qo_heads / num_kv_heads).
 */
#ifndef PKVS_H
#define PKVS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkvs_status {
    PKVS_OK = 0,
    PKVS_ERR_INVALID_ARG = -1,   /* malformed argument or layout */
    PKVS_ERR_UNSUPPORTED = -2,   /* head_dim / page_size / dtype / mode not built */
    PKVS_ERR_WORKSPACE = -3,     /* a workspace is smaller than pkvs_workspace_size() */
    PKVS_ERR_CAPACITY = -4,      /* batch / tokens / keys above the plan's capacity */
    PKVS_ERR_PLAN_MISMATCH = -5, /* run() window_left or causal differs from the plan */
    PKVS_ERR_HIP = -6,           /* HIP runtime or launch failure */
    PKVS_ERR_NOT_PLANNED = -7    /* run() before a device plan was made */
} pkvs_status;

typedef enum pkvs_dtype { PKVS_BF16 = 0, PKVS_FP32 = 1, PKVS_FP16 = 2 } pkvs_dtype;

/* Storage of the K/V cache: the plan's dtype, or OCP 8-bit floats (e4m3,
 * "float8_e4m3fn"; e5m2) holding K / k_scale and V / v_scale ([FIB]
 * forward_extend / forward_decode pass k_scale and v_scale with the cache;
 * should_use_tensor_core names both 8-bit cache types). */
typedef enum pkvs_kv_format {
    PKVS_KV_SAME = 0,
    PKVS_KV_FP8_E4M3 = 1,
    PKVS_KV_FP8_E5M2 = 2
} pkvs_kv_format;

typedef enum pkvs_kind { PKVS_PREFILL = 0, PKVS_DECODE = 1, PKVS_CASCADE = 2 } pkvs_kind;

/* Fixed properties of a plan.  window_left and causal are fixed here, at plan
 * time ([PR31501] "What"); run() must pass the same values.
 *  kind             PKVS_PREFILL, PKVS_DECODE or PKVS_CASCADE (a prefill whose
 *                   new tokens' keys come in a contiguous array and whose cached
 *                   prefix sits in the paged cache; see pkvs_cascade_plan)
 *  num_qo_heads     multiple of num_kv_heads; group = num_qo_heads/num_kv_heads
 *                   must be a power of two <= 16 (bf16 and fp16 paths)
 *  head_dim         64, 128 or 256
 *  page_size        power of two, 1 .. 1024
 *  dtype            q, k_cache, v_cache and o share it: PKVS_BF16, PKVS_FP16
 *                   (IEEE half; the dtype sweep of [PR234] "Tests added") or
 *                   PKVS_FP32; accumulation is fp32 in every case
 *  causal           prefill, cascade: 1, or 0 only with window_left = -1;
 *                   decode: ignored
 *  window_left      -1 (no window) or W >= 0 (W+1 visible keys, [PR234] 1)
 *  fixed_split_size decode: keys per KV chunk (a multiple of 32), or -1 to let
 *                   the planner choose; the partial (o, lse) of the chunks of
 *                   one request are combined by the merge of pkvs_merge_state
 *  disable_split_kv decode: 1 = one chunk per request; prefill, cascade: 1 =
 *                   never split a query tile's keys (see pkvs_prefill_plan)
 *  prefill_variant  prefill kernel shape: 0 = planner's choice (from head_dim,
 *                   page_size and the capacities), 1 = 4 waves x 32 rows, 2 = 8
 *                   waves x 32 rows, 3 = 4 waves x 64 rows, software-pipelined
 *                   (2 and 3: head_dim <= 128), 4 = 8 waves x 32 rows with K/V
 *                   rows loaded straight into LDS, 5 = as 4 with 64-key steps
 *                   and 16-byte loads into a chunk-permuted LDS layout, 6 = as
 *                   5 with 4 waves x 32 rows and two workgroups per CU (4, 5
 *                   and 6: head_dim 128, 16-bit K/V; they hold an item's page
 *                   ids in an LDS table of 2048 entries, 8192 for variant 5, so
 *                   a plan whose capacities let one item span more pages --
 *                   (kv_capacity - 1) / page_size + 1, or with a window
 *                   (window_left + query tile + 2 key tiles - 3) / page_size +
 *                   2 if smaller -- runs variant 2 instead); rows are (query
 *                   token, head) pairs.  The variant is fixed by
 *                   pkvs_plan_create and never changes with the planned batch
 *  batch_capacity   largest batch a plan() call may describe
 *  qo_capacity      prefill, cascade: largest total number of query tokens
 *  kv_capacity      largest kv_len of one request (cascade: the most cached
 *                   keys one request's page table may hold)
 *  kv_format        PKVS_KV_SAME (k_cache / v_cache in dtype) or an 8-bit
 *                   format (dtype bf16 or fp16 only; widened exactly to dtype
 *                   on the way to the matrix cores; prefill variants 1 and 2,
 *                   the planner picks one).  A cascade's new-token K/V stay in
 *                   dtype; only its cache is 8-bit.
 *  decode_waves     decode: waves that share one work item (request, kv
 *                   head, chunk): 1, or 4 (each streams a quarter of the
 *                   chunk's keys and the four combine their partial results
 *                   in LDS, as pkvs_merge_state would); 0 = planner's choice:
 *                   4 when batch_capacity x num_kv_heads x 32 is at most the
 *                   device's resident one-wave items (32 pairs on a 256-CU
 *                   MI355X) and kv_capacity (cut to window_left + 1) exceeds
 *                   2048 keys, else 1.  Fixed for the plan's lifetime (every
 *                   plan() runs the same kernel).
 *  logits_soft_cap  0 (off) or c > 0: every logit x = sm_scale * q.k becomes
 *                   c * tanh(x / c) before the softmax and the LSE ([FIB]
 *                   forward_extend / forward_decode pass logits_soft_cap to
 *                   the wrappers; the tanh cap of the scaled logit is the
 *                   reading taken)
 * The launch grid and the workspaces are sized from these capacities and the
 * device alone, never from one batch ([PR234] 2; [FIB]
 * _full_cg_prefill_workspace_bytes). */
typedef struct pkvs_desc {
    int32_t kind;
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t dtype;
    int32_t causal;
    int32_t window_left;
    int32_t fixed_split_size;
    int32_t disable_split_kv;
    int32_t batch_capacity;
    int32_t prefill_variant;
    int64_t qo_capacity;
    int64_t kv_capacity;
    float logits_soft_cap;
    int32_t kv_format;
    int32_t decode_waves;
} pkvs_desc;

/* Read-only facts about a plan (for callers, tests and profilers). */
typedef struct pkvs_plan_info {
    int64_t num_items;       /* work items of the last plan() */
    int64_t num_merges;      /* (request, kv head) pairs whose chunks are merged; key-split
                                prefill: (query token, kv head) pairs */
    int64_t float_ws_bytes;  /* required float workspace (fp32 partials) */
    int64_t int_ws_bytes;    /* required int workspace (work list) */
    int32_t grid_blocks;     /* fixed grid of the main kernel */
    int32_t block_threads;
    int32_t split_size;      /* decode: keys per chunk chosen by the last plan() */
    int32_t item_words;      /* int32 words per work item */
    int32_t query_tile;      /* prefill: query tokens per item */
    int32_t num_cus;         /* compute units the grid was sized for */
    int32_t prefill_variant; /* prefill: kernel variant the last plan() runs */
    int32_t decode_waves;    /* decode: waves that share one work item */
    int32_t cascade_passes;  /* cascade: 1 (one launch over cached and new keys) or 2 */
    int32_t key_chunks;      /* prefill, cascade: most key chunks per query tile a plan()
                                may cut (1: never; see pkvs_prefill_plan) */
} pkvs_plan_info;

typedef struct pkvs_plan pkvs_plan;

/* Create a plan object for `desc` on the current HIP device ([FIB]
 * _create_full_cg_prefill_wrappers: the wrappers are made once, for the
 * largest batch they will see, and bound to a workspace sized for it; the
 * launch grid, the kernel variant and the workspace sizes are fixed here from
 * the capacities and the device).  Fails with INVALID_ARG / UNSUPPORTED for a
 * descriptor outside the rules above.  Works without a GPU (then only dry
 * plans, with null workspaces, can be made).  The plan is a host object owned
 * by the library until pkvs_plan_destroy. */
int pkvs_plan_create(pkvs_plan **out, const pkvs_desc *desc);

/* Worst-case workspace sizes for the plan's capacities, in bytes ([FIB]
 * _full_cg_prefill_workspace_bytes: the split-KV float workspace is sized for
 * the largest batch the wrapper will run, once).  Callers allocate device
 * buffers at least this large (float_ws may be 0 bytes).
 * int_ws holds the work list that plan() copies in; the decode kernel and the
 * default prefill kernel also keep two work counters in its header, which
 * plan() uploads as 0 and every run() leaves at 0 when it completes, so the
 * same plan can be run (or a captured run replayed) any number of times, one
 * run at a time per workspace. */
int pkvs_workspace_size(const pkvs_plan *plan, size_t *float_ws_bytes, size_t *int_ws_bytes);

/* Worst-case workspace sizes of a descriptor without keeping a plan ([FIB]
 * _full_cg_prefill_workspace_bytes: the split-KV float workspace a wrapper
 * needs for the largest batch, computed before the wrappers exist, so a
 * too-small buffer fails at start-up).  is_decode must agree with desc->kind
 * (1 for PKVS_DECODE, 0 for PKVS_PREFILL or PKVS_CASCADE); max_kv_len > 0
 * replaces desc->kv_capacity, 0 keeps it.  Equal to pkvs_workspace_size of
 * the plan pkvs_plan_create would make for the same descriptor on the current
 * device.  Errors as pkvs_plan_create, INVALID_ARG for a null output or a
 * kind that disagrees with is_decode. */
int pkvs_workspace_bytes(const pkvs_desc *desc, int32_t is_decode, int64_t max_kv_len,
                         size_t *float_ws_bytes, size_t *int_ws_bytes);

/* Plan a causal paged prefill (extend with cached prefix) batch.
 * Host arrays: qo_indptr_h [batch+1], kv_indptr_h [batch+1],
 * kv_last_page_len_h [batch] (the host-known layout of [FIB]
 * fast_prefill_plan; no device-to-host copy happens).  Builds the work list
 * (request, kv head, query tile, first and last key tile after the window
 * skip) and enqueues one host-to-device copy of it into int_ws on `stream`.
 * With int_ws == NULL the plan is built on the host only ("dry plan",
 * inspectable with pkvs_plan_copy_items, not runnable).
 * Key split (split-KV for prefill, the combine of [FIB] _safe_merge_state):
 * on prefill variants 1, 2 and 5 with 16-bit queries, a batch with at most
 * one query tile per two workgroups of the plan's grid may have the key
 * ranges of its longest tiles cut into chunks of whole key tiles, each a
 * work item writing a partial (o, lse) per query token into the float
 * workspace, at most one item per workgroup in all; run() then merges each
 * token's chunks.  A batch is cut when that shortens its longest item by
 * more than the merge costs.  The float workspace holds the partial slots
 * for that (sized from the grid, not the capacities); disable_split_kv = 1
 * turns the split off (float_ws then 0 bytes).
 * Errors: INVALID_ARG (qo_len_b > kv_len_b, last page length outside
 * [1, page_size], decreasing indptr), CAPACITY, WORKSPACE, HIP. */
int pkvs_prefill_plan(pkvs_plan *plan, const int32_t *qo_indptr_h, const int32_t *kv_indptr_h,
                      const int32_t *kv_last_page_len_h, int32_t batch_size, void *float_ws,
                      size_t float_ws_bytes, void *int_ws, size_t int_ws_bytes,
                      hipStream_t stream);

/* Run the planned prefill: o (and lse when non-null) for every query token.
 * k_cache/v_cache hold num_pages pages; kv_indices_d (device, int32) holds
 * kv_indptr_h[batch] page ids in [0, num_pages).  window_left and causal must
 * equal the plan's (PLAN_MISMATCH otherwise, [PR31501] "What").  The exact
 * per-element window mask is always applied.  Keys and values are read as
 * k_scale * k and v_scale * v (positive finite; 1 for an unscaled cache;
 * INVALID_ARG otherwise), k_scale folded into the logit scale and v_scale
 * into the output normalisation, for every cache type.  After a batch whose
 * plan cut key ranges, a second launch merges the chunk partials (under
 * stream capture it is launched whenever the plan can cut, and reads the
 * merge count from the workspace). */
int pkvs_prefill_run(const pkvs_plan *plan, const void *q, const void *k_cache,
                     const void *v_cache, int64_t num_pages, const int32_t *kv_indices_d,
                     void *o, float *lse, float sm_scale, int32_t window_left, int32_t causal,
                     float k_scale, float v_scale, hipStream_t stream);

/* Plan a single-token decode batch (one query per request, at kv_len-1).
 * The window keeps the last min(kv_len, W+1) keys of each request ([FIB]
 * FlashInferIndicesUpdaterDecode.update_sliding_window); those keys are cut
 * into chunks of split_size keys (fixed_split_size or the planner's choice).
 * A request with kv_len 0 yields o = 0, lse = -inf. */
int pkvs_decode_plan(pkvs_plan *plan, const int32_t *kv_indptr_h,
                     const int32_t *kv_last_page_len_h, int32_t batch_size, void *float_ws,
                     size_t float_ws_bytes, void *int_ws, size_t int_ws_bytes,
                     hipStream_t stream);

/* Run the planned decode ([FIB] FlashInferAttnBackend.forward_decode; LSE on
 * request, [PR234] "Why each fix" 3): q, o [batch, num_qo_heads, head_dim],
 * lse [batch, num_qo_heads] (nullable).  Launches the chunk kernel and, when
 * some request was split, the merge of its chunk partials.  window_left must
 * equal the plan's (PLAN_MISMATCH otherwise, [PR31501] "What"); k_scale /
 * v_scale as pkvs_prefill_run. */
int pkvs_decode_run(const pkvs_plan *plan, const void *q, const void *k_cache,
                    const void *v_cache, int64_t num_pages, const int32_t *kv_indices_d,
                    void *o, float *lse, float sm_scale, int32_t window_left, float k_scale,
                    float v_scale, hipStream_t stream);

/* Bytes of the library's device scratch array, one per device, that
 * pkvs_decode_noalloc plans and runs in (64 MiB). */
#define PKVS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate memory at the point of the call (serving
 * loops that must not allocate per step, harnesses that forbid allocation):
 * pkvs_decode_plan followed by pkvs_decode_run, with the plan's int and float
 * workspaces taken from the library's fixed device array of
 * PKVS_NOALLOC_SCRATCH_BYTES instead of caller buffers.  It calls no
 * hipMalloc, hipFree, hipHostMalloc or host allocator: the plan's pinned
 * staging ring and planning buffers were made by pkvs_plan_create.
 *  plan        a PKVS_DECODE plan of bf16 or fp16 queries, created on the
 *              device that is current at the call
 *  kv_indptr_h .. batch_size   the layout, as pkvs_decode_plan (host arrays)
 *  q .. v_scale, stream        as pkvs_decode_run
 * The work list (header with the work counters at 0) is copied into the array
 * on `stream` before the kernels run, so nothing depends on what an earlier
 * call left there.  Every call on one device shares that device's array: calls
 * that overlap on one device (other streams, other plans, other threads)
 * race and must be ordered by the caller.  Not for stream capture: the
 * work-list copy reads a host staging buffer that later calls rewrite.
 * Errors: INVALID_ARG (null or non-decode plan, fp32 plan, plan made for
 * another device than the current one), WORKSPACE (the plan's workspaces
 * for its capacities, int part then float part at the next 256-byte
 * boundary, exceed PKVS_NOALLOC_SCRATCH_BYTES: use pkvs_decode_plan and
 * pkvs_decode_run with caller workspaces), HIP, and those of
 * pkvs_decode_plan / pkvs_decode_run.  After a successful call the plan is
 * planned on the array: a later pkvs_decode_run reruns this batch there. */
int pkvs_decode_noalloc(pkvs_plan *plan, const int32_t *kv_indptr_h,
                        const int32_t *kv_last_page_len_h, int32_t batch_size, const void *q,
                        const void *k_cache, const void *v_cache, int64_t num_pages,
                        const int32_t *kv_indices_d, void *o, float *lse, float sm_scale,
                        int32_t window_left, float k_scale, float v_scale, hipStream_t stream);

/* Plan a cascade prefill ([FIB] FlashInferAttnBackend.forward_extend, the
 * branch for a batch with cached prefixes: a ragged pass over the new tokens'
 * own keys, a paged pass over the cached prefix, and _safe_merge_state of the
 * two (o, lse) pairs).  The plan must have kind PKVS_CASCADE.
 *  qo_indptr_h [batch+1]   new (query) tokens of request b; their keys and
 *                          values are the same rows of k_extend / v_extend
 *  kv_indptr_h, kv_last_page_len_h   the page table of the cached keys that
 *                          precede the new tokens: request b's table holds
 *                          kv_len_b keys, the last kv_len_b before its first
 *                          new token.  It may start anywhere at or before the
 *                          window's reach -- the whole prefix, or only its
 *                          last min(prefix, window_left) keys ([FIB]
 *                          FlashInferIndicesUpdaterPrefill.update_sliding_window
 *                          trims it so); keys beyond the window are skipped.
 * New token i of request b (position kv_len_b + i relative to the table's
 * first key) sees cached key j iff window_left < 0 or j >= kv_len_b + i -
 * window_left ([FIB] _build_swa_prefix_custom_mask), and new key i' iff
 * i' <= i (causal) and (window_left < 0 or i' >= i - window_left).  The
 * result equals pkvs_prefill_run over one page table holding the table's keys
 * followed by the new keys.  Zero new tokens or zero cached keys are legal.
 * The plan is one pass when pkvs_plan_create found that a kernel reading
 * split key ranges serves the combined problem (16-bit K/V in the query dtype;
 * prefill_variant 0, 1, 2 or 5): each request becomes one prefill request
 * over its cached keys followed by its new tokens, one causal sequence whose
 * window mask is exactly the two masks above, and the key split of
 * pkvs_prefill_plan applies to it.  Otherwise two passes
 * (pkvs_plan_info.cascade_passes tells which).  Builds the work list(s) and
 * enqueues the host-to-device copies into int_ws on `stream` (int_ws == NULL:
 * dry plan).  float_ws holds the paged pass's (o, lse) of a two-pass plan, the
 * key split's partials of a one-pass plan (0 bytes when it cannot split).
 * Errors as pkvs_prefill_plan (a request may have more new tokens than cached
 * keys). */
int pkvs_cascade_plan(pkvs_plan *plan, const int32_t *qo_indptr_h, const int32_t *kv_indptr_h,
                      const int32_t *kv_last_page_len_h, int32_t batch_size, void *float_ws,
                      size_t float_ws_bytes, void *int_ws, size_t int_ws_bytes,
                      hipStream_t stream);

/* Run the planned cascade ([FIB] FlashInferAttnBackend.forward_extend, the
 * branch with cached prefixes): q, o [nnz_qo, num_qo_heads, head_dim]; k_extend,
 * v_extend [nnz_qo, num_kv_heads, head_dim] (row r is the key / value of query
 * token r); k_cache, v_cache, num_pages and kv_indices_d as pkvs_prefill_run
 * (they may be NULL / 0 when the planned batch has no cached keys); lse
 * nullable.  Where the plan is one pass (pkvs_plan_info.cascade_passes 1),
 * one launch on `stream` reads each request's cached keys through the page
 * table and its new keys from k_extend / v_extend in one online softmax
 * (followed by the merge of a key-split batch, as pkvs_prefill_run);
 * otherwise two launches: the paged pass writes its (o, lse) into
 * float_ws, then the ragged pass stores the merge_state combine of its own
 * (o, lse) with them into o and lse (the merge runs in its epilogue).
 * window_left must equal the plan's.  k_scale / v_scale apply to the cache
 * (as pkvs_prefill_run); the new tokens' K/V are read unscaled. */
int pkvs_cascade_run(const pkvs_plan *plan, const void *q, const void *k_extend,
                     const void *v_extend, const void *k_cache, const void *v_cache,
                     int64_t num_pages, const int32_t *kv_indices_d, void *o, float *lse,
                     float sm_scale, int32_t window_left, float k_scale, float v_scale,
                     hipStream_t stream);

/* Combine two attention partials over disjoint key sets ([FIB]
 * _safe_merge_state):  s = ln(exp(s_a) + exp(s_b)),
 * v = exp(s_a - s) * v_a + exp(s_b - s) * v_b;  s_a = s_b = -inf gives v = 0,
 * s = -inf.  v_* [num_tokens, num_heads, head_dim] in v_dtype, s_*
 * [num_tokens, num_heads] float32.  The grid runs over (token, head) pairs,
 * so no head count limits the launch.  v_out/s_out may alias v_a/s_a. */
int pkvs_merge_state(const void *v_a, const float *s_a, const void *v_b, const float *s_b,
                     void *v_out, float *s_out, int64_t num_tokens, int32_t num_heads,
                     int32_t head_dim, int32_t v_dtype, hipStream_t stream);

/* Write the batch's new key/value rows into the paged cache ([FIB]
 * forward_extend / forward_decode: token_to_kv_pool.set_kv_buffer with the
 * batch's cache locations, before the paged attention reads them).
 *  k_new, v_new  [num_tokens, num_kv_heads, head_dim] in dtype, 16-byte aligned
 *  loc_d         [num_tokens] int64 (device): the cache slot of each row,
 *                slot = page * page_size + position in the page
 *  k_cache, v_cache  the cache viewed as [num_slots, num_kv_heads, head_dim]
 *                (num_slots = num_pages * page_size), 16-byte aligned, in dtype
 *                (kv_format PKVS_KV_SAME: rows copied bit for bit) or 8-bit
 *                (PKVS_KV_FP8_E4M3 / _E5M2: every element x becomes the 8-bit
 *                value of x / k_scale -- v_scale for values -- computed in fp32,
 *                rounded to dtype, then to the 8-bit format to nearest even;
 *                e4m3 overflow, infinities and NaN give NaN, e5m2 overflow
 *                gives +-inf, as the cast of set_kv_buffer does)
 *  k_scale, v_scale  positive finite; read only for an 8-bit cache
 *  status_d      nullable device int32: the kernel adds the number of rows
 *                whose slot lies outside [0, num_slots) (they are not written)
 * Slots must be distinct (two rows to one slot leave either).  One launch on
 * `stream`, no allocation.  Errors: INVALID_ARG (shape, null or misaligned
 * pointer, kv_format, scales), UNSUPPORTED (dtype, a row not a multiple of 16
 * bytes), HIP. */
int pkvs_append_kv(const void *k_new, const void *v_new, const int64_t *loc_d,
                   int64_t num_tokens, void *k_cache, void *v_cache, int64_t num_slots,
                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype, int32_t kv_format,
                   float k_scale, float v_scale, int32_t *status_d, hipStream_t stream);

/* Build the page table on the device ([FIB] call_begin_forward: kv_indptr is
 * the running sum of the per-request lengths; create_flashinfer_kv_indices_triton
 * gathers, for request b, entries start[b] .. start[b] + len[b] - 1 of row
 * slot[b] of the request-to-token map into kv_indices from kv_indptr[b] on; a
 * sliding-window wrapper passes start = the first key of the window).  With
 * page_size 1 the map holds token slots, as on the pages; with larger pages
 * it holds page ids and start / len count pages.  All arrays are device int32:
 *  page_map_d   [map_rows, map_cols]        slot_d, len_d  [batch_size]
 *  start_d      [batch_size] or NULL (0)    kv_indptr_d    [batch_size + 1] (out)
 *  kv_indices_d [capacity] (out)
 * A negative length counts as 0; an entry whose source lies outside the map
 * is written as -1; entries at or past `capacity` are not written; each adds 1
 * to *status_d when it is given.  Two launches on `stream` (the running sum,
 * then the gather), no allocation.  Errors: INVALID_ARG, HIP. */
int pkvs_build_kv_indices(const int32_t *page_map_d, int64_t map_rows, int64_t map_cols,
                          const int32_t *slot_d, const int32_t *start_d, const int32_t *len_d,
                          int32_t batch_size, int32_t *kv_indptr_d, int32_t *kv_indices_d,
                          int64_t capacity, int32_t *status_d, hipStream_t stream);

/* Facts about the plan (counts refer to the last plan() call).  Library
 * utility, no passage: for callers, tests and profilers. */
int pkvs_plan_get_info(const pkvs_plan *plan, pkvs_plan_info *info);

/* Host copy of the last plan()'s work list: up to max_items items of
 * info.item_words int32 words each into dst; *n_items receives the count.  A
 * cascade lists its ragged pass's items, then its paged pass's.  Library
 * utility, no passage: it exposes the planner's output to tests. */
int pkvs_plan_copy_items(const pkvs_plan *plan, int32_t *dst, int64_t max_items,
                         int64_t *n_items);

/* Destroy a plan (waits for its pending host-to-device copies).  NULL is a
 * no-op.  Library utility, no passage. */
void pkvs_plan_destroy(pkvs_plan *plan);

/* Static description of a status code.  Library utility, no passage. */
const char *pkvs_strerror(int code);

/* Detail message of the last error on this thread ("" if none); the string
 * stays valid until the thread's next libpkvs call.  Library utility, no
 * passage. */
const char *pkvs_last_error(void);

/* The same thread-local detail message as pkvs_last_error (both names are
 * exported).  Library utility, no passage. */
const char *pkvs_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* PKVS_H */
