/*
 * libxattn: plan/run paged attention for AMD Instinct MI355X (gfx950).
 *
 * The operation is softmax attention of ragged, packed queries over a paged KV
 * cache that the library only reads:
 *
 *  - page "mstar.engine.resources.attn.cross", FlashInferCrossManager: non-causal
 *    paged attention over a fixed encoder context; the context is an ordinary paged
 *    KV stream, planned once per step and run once per layer;
 *  - same page, FlashInferCrossManager.plan: the plan result is immutable and opaque;
 *  - same page, FlashInferCrossManager.run: one layer's attention, and nothing is
 *    written to the context cache;
 *  - same page, FlashInferCrossManager.force_double_buffer: a plan staged through a
 *    reused host buffer and a non-blocking host-to-device copy races when the host
 *    runs ahead, so the staging buffers are kept per slot and fenced before reuse;
 *  - same page, QueryPacking: the query side is the requests in packed order plus
 *    the cumulative query lengths (qo_indptr);
 *  - page "mstar.engine.resources.attn.config", AttentionStep.causal: causal
 *    self-attention over a paged cache;
 *  - page "mstar.engine.resources.attn.ragged.base", RaggedBlockCausalAttnManager:
 *    cacheless block-causal self-attention within each span of a packed batch;
 *  - page "mstar.model.components.attention", Attention: grouped-query attention
 *    when num_kv_heads < num_heads.
 *
 * The pages name paging but not its layout. This library reads it as a CSR page
 * table (kv_indptr in pages, kv_page_indices, kv_last_page_len) over K and V pools
 * laid out [num_pages][page_size][num_kv_heads][head_dim] (the per-token
 * (len, heads, head_dim) layout of CrossAttention.compute_kv on the attention page).
 *
 * Conventions shared by every entry point:
 *  - All integers are int32 unless stated; all index arrays are host memory and are
 *    copied before the call returns (the caller may reuse them at once).
 *  - q, out: [qo_indptr[B]][num_qo_heads][head_dim], row-major, in the plan's dtype.
 *  - k_pages, v_pages: [num_pages][page_size][num_kv_heads][head_dim], in the plan's
 *    dtype; they are const and never written.
 *  - lse: [qo_indptr[B]][num_qo_heads] fp32, natural log of the softmax normaliser
 *    of the scaled scores; -inf for a row that sees no key.
 *  - Query row i of request r is the key position kv_len[r] - qo_len[r] + i (the
 *    queries are the last qo_len positions of the context). CAUSAL shows it keys
 *    j <= that position; BLOCK_CAUSAL shows it keys whose block (j / block_size) is
 *    not after its own; NONE shows every key.
 *  - Query head h reads KV head h / (num_qo_heads / num_kv_heads).
 *  - Status codes: XATTN_OK (0) or a negative XATTN_ERR_*; xattn_last_error()
 *    returns a thread-local message for the last failure.
 *  - A handle is not thread-safe; distinct handles are independent.
 */
#ifndef XATTN_H
#define XATTN_H

#include <stdint.h>

#if defined(__GNUC__)
#define XATTN_API __attribute__((visibility("default")))
#else
#define XATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef struct xattn_plan_s* xattn_plan_t;

enum xattn_mask_mode {
  XATTN_MASK_NONE = 0,         /* cross-attention: every key */
  XATTN_MASK_CAUSAL = 1,       /* key j <= the query's position */
  XATTN_MASK_BLOCK_CAUSAL = 2  /* key block <= the query's block, blocks of block_size */
};

enum xattn_dtype {
  XATTN_F32 = 0,  /* fp32 storage and arithmetic; head_dim in {16, 32, 64, 128} */
  XATTN_BF16 = 1  /* bf16 storage, fp32 accumulation; head_dim in {64, 128} */
};

enum xattn_status {
  XATTN_OK = 0,
  XATTN_ERR_INVALID_ARG = -1, /* an argument breaks the contract above */
  XATTN_ERR_UNSUPPORTED = -2, /* valid but not built (e.g. head_dim) */
  XATTN_ERR_HIP = -3,         /* a HIP runtime call failed */
  XATTN_ERR_OOM = -4,         /* device or pinned host allocation failed */
  XATTN_ERR_BUSY = -5         /* reserved: the slot to be planned is still in use */
};

/*
 * xattn_plan: validate the page table and query packing, partition the work into
 * units (splitting long contexts into KV chunks whose partial results are merged
 * on the log-sum-exp), and stage the schedule for xattn_run.
 *
 * Page "mstar.engine.resources.attn.cross", FlashInferCrossManager.plan: one step's
 * query packing (QueryPacking: requests in packed order and cumulative query lengths)
 * becomes an immutable, opaque planned object that every layer's run of the step
 * reuses; FlashInferCrossManager.force_double_buffer: its host staging and non-blocking
 * copy are kept per slot, two slots, so a plan never overwrites what an earlier run
 * still reads.
 *
 * The argument list is the page table and packing of the problem statement
 * (qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, head counts, head_dim,
 * page_size, mask) plus what a C call cannot infer: batch_size, block_size, sm_scale,
 * dtype, stream, and one deliberate addition, num_pages, the size of the K and V
 * pools, so that every page index is checked against the pool before any kernel
 * reads through it (without it a bad index could only be caught by a device fault).
 *
 * plan            in/out. *plan == NULL creates a handle; otherwise the new schedule
 *                 is written into the handle's other slot (two slots: pinned host
 *                 staging + device copy + fp32 split workspace each). Before a slot is
 *                 rewritten the call waits until the slot's previous host-to-device
 *                 copy is done, and until every run that read the slot is done or is
 *                 ordered before the new copy by the stream (runs on the plan's stream
 *                 are; runs on other streams are waited for, and a plan on another
 *                 stream than the slot last used waits for that stream).
 * qo_indptr       [batch_size + 1]; qo_indptr[0] == 0, non-decreasing.
 * kv_indptr       [batch_size + 1]; page counts; kv_indptr[0] == 0, non-decreasing.
 * kv_page_indices [kv_indptr[batch_size]], each in [0, num_pages); NULL means the
 *                 identity table (logical page p of the batch is physical page p), which
 *                 is how cacheless spans are passed: page_size 1, kv_indptr equal to
 *                 the spans' cu_seqlens, and k_pages the packed keys [T][1][H][D].
 * kv_last_page_len [batch_size], each in [1, page_size] for a request with pages;
 *                 NULL means every last page is full.
 * batch_size      number of requests B >= 0.
 * num_qo_heads, num_kv_heads  >= 1, num_qo_heads % num_kv_heads == 0.
 * head_dim        see xattn_dtype.
 * page_size       tokens per page, >= 1.
 * num_pages       pages in the K and V pools; every referenced page must lie below it.
 * mask_mode       an xattn_mask_mode. CAUSAL and BLOCK_CAUSAL need qo_len <= kv_len.
 * block_size      >= 1, read only for BLOCK_CAUSAL.
 * sm_scale        score scale; <= 0 means 1 / sqrt(head_dim); NaN, infinity and scales
 *                 whose product with log2(e) overflows are rejected.
 * dtype           an xattn_dtype.
 * stream          hipStream_t for the host-to-device copy (NULL: the null stream).
 *
 * On error the handle (if any) keeps its previous schedule unchanged.
 */
XATTN_API int xattn_plan(xattn_plan_t* plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
               const int32_t* kv_page_indices, const int32_t* kv_last_page_len,
               int32_t batch_size, int32_t num_qo_heads, int32_t num_kv_heads,
               int32_t head_dim, int32_t page_size, int64_t num_pages, int32_t mask_mode,
               int32_t block_size, float sm_scale, int32_t dtype, void* stream);

enum xattn_plan_flags {
  XATTN_PLAN_GRAPH_STABLE = 1
};

/*
 * xattn_plan_create: an empty handle with flags (xattn_plan creates one with no flags
 * when *plan is NULL). *plan must be NULL on entry.
 *
 * XATTN_PLAN_GRAPH_STABLE (page "mstar.engine.resources.attn.cross",
 * force_double_buffer: the plan keeps two buffers so that a captured graph reads one
 * while the next plan fills the other). Each slot lays its device schedule out by
 * capacities that only grow (with a quarter of headroom when they do), and a run
 * launches every kernel family the slot has held, with grids of the slot's capacity;
 * blocks past the current plan's units exit at once. A run captured into a HIP graph
 * (on the plan's stream, timing off) then replays correctly for any later schedule in
 * the same slot as long as the slot's layout_generation (xattn_plan_info) is unchanged;
 * when it changes, capture again. Keep one graph per slot: consecutive plans alternate
 * slots (xattn_plan_info's `slot`). The q, k_pages, v_pages, out and lse pointers are
 * part of the capture. Costs a few idle blocks per launch; without the flag, grids
 * match each schedule exactly.
 */
XATTN_API int xattn_plan_create(xattn_plan_t* plan, int32_t flags);

/*
 * xattn_run: one layer's attention with the latest schedule (page
 * "mstar.engine.resources.attn.cross", FlashInferCrossManager.run). Launches the
 * attention kernels, and the log-sum-exp merge kernel when a context was split, on
 * `stream`, then records the slot's fence there. Any number of runs (one per layer,
 * each with its own q/k/v/out) may share one plan.
 * When the schedule splits contexts (xattn_plan_info: num_merge_rows > 0) its runs share
 * the slot's fp32 workspace of partial results. A run on another stream than the latest
 * run that used it therefore first waits for that stream (an event recorded there), so
 * runs of a split schedule on several streams execute one after another and never mix
 * their partials; runs on one stream are ordered by the stream and record nothing.
 *
 * q, k_pages, v_pages  device pointers, layouts above, 16-byte aligned; k_pages and
 *                      v_pages are not written.
 * out                  device pointer, caller-allocated, 16-byte aligned.
 * lse                  device pointer (4-byte aligned) or NULL (not written).
 * stream               hipStream_t (NULL: the null stream).
 *
 * Returns XATTN_ERR_INVALID_ARG for a handle with no schedule, a NULL pointer that
 * the schedule needs or a misaligned pointer, XATTN_ERR_HIP for a launch failure.
 * Device faults surface at the caller's next synchronisation. Pointers are borrowed
 * until the stream passes the run. A run on another stream than the plan's waits for
 * the schedule's copy and records an event that the next plan into this slot waits
 * for; a run on the plan's stream records nothing. Streams used by runs must stay
 * valid until the handle's next-but-one xattn_plan or its destruction.
 *
 * Graph capture (page "mstar.engine.resources.attn.cross", force_double_buffer: the plan
 * keeps two buffers so that a captured graph can read one while the next plan fills the
 * other). A run on the plan's own stream with timing off issues kernel launches only, so
 * it may be captured into a HIP graph, provided that the slot's latest run of a split
 * schedule was on that stream too (otherwise the run first waits for an event recorded
 * on the other stream, which a capture cannot take in). A replay repeats the captured
 * schedule with the captured pointers: it stays valid through the handle's next
 * xattn_plan (which fills the other slot) and must not be replayed after the one after
 * that, which reuses (and may reallocate) the slot it reads.
 */
XATTN_API int xattn_run(xattn_plan_t plan, const void* q, const void* k_pages, const void* v_pages,
              void* out, float* lse, void* stream);

/*
 * xattn_run_noalloc: xattn_run for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, layouts and kernels as xattn_run; the split workspace of partial results
 * is instead the library's static device scratch, 32 MiB per GPU (a file-scope device
 * array that each GPU the library runs on holds until the process ends). The call makes
 * no device or host allocation of any kind (no hipMalloc, no event, no timing records).
 *
 * Rules:
 *  - runs on the stream of the handle's latest xattn_plan only (XATTN_ERR_INVALID_ARG
 *    otherwise); the handle's plans still allocate as usual;
 *  - a schedule whose split workspace (workspace_rows x (head_dim + 1) x 4 bytes, the
 *    slot's capacity in a graph-stable handle) exceeds 32 MiB is rejected with
 *    XATTN_ERR_UNSUPPORTED and a message; xattn_run has no such limit;
 *  - every call on one GPU, from any handle, shares that GPU's scratch: calls whose
 *    executions overlap on one GPU (runs on different streams not ordered by events)
 *    race and give wrong results. Calls ordered on one stream are safe. The scratch is
 *    never cleared: each run's kernels write every partial row before its merge reads it.
 */
XATTN_API int xattn_run_noalloc(xattn_plan_t plan, const void* q, const void* k_pages,
                                const void* v_pages, void* out, float* lse, void* stream);

/*
 * xattn_write_kv: the step before the path. Writes each request's context keys and
 * values into its pages once, so that later runs read them (page
 * "mstar.engine.resources.attn.cross": the context is written once by the encode step
 * and then read as an ordinary paged KV stream; page "mstar.model.components.attention",
 * CrossAttention.compute_kv: a request's keys and values come out as (length, heads,
 * head_dim)). Uses the page table of the latest schedule.
 *
 * k_src, v_src      device [sum kv_len, Hkv, D] in the plan's dtype, requests packed in
 *                   order (request r's rows start at kv_len[0] + ... + kv_len[r-1]),
 *                   16-byte aligned; not written.
 * k_pages, v_pages  device pools [num_pages, page_size, Hkv, D], 16-byte aligned.
 *                   Position t of request r goes to slot t % page_size of page
 *                   kv_page_indices[kv_indptr[r] + t / page_size] (identity table:
 *                   page kv_indptr[r] + t / page_size). Slots past a request's kv_len in
 *                   its last page, and pages of no request, are left untouched.
 * stream            hipStream_t; ordered with the plan's copy like xattn_run.
 *
 * Returns XATTN_ERR_INVALID_ARG for a handle with no schedule or a NULL or misaligned
 * pointer, XATTN_ERR_UNSUPPORTED when the contexts hold more than 2^31-1 rows in total,
 * XATTN_ERR_HIP for a launch failure. Pages shared by two requests are written by both,
 * in no fixed order.
 */
XATTN_API int xattn_write_kv(xattn_plan_t plan, const void* k_src, const void* v_src, void* k_pages,
                             void* v_pages, void* stream);

/* 1 if the next xattn_plan on this handle (on the same stream) would not wait, 0 if it
 * would, negative on error. Never blocks. Page "mstar.engine.resources.attn.cross",
 * force_double_buffer: the host runs ahead of the device, and this tells it whether the
 * slot the next plan fills is still in use. */
XATTN_API int xattn_plan_ready(xattn_plan_t plan);

/* Waits on both slot fences, then frees the handle. NULL is ignored.
 * Plumbing of the C boundary (a handle's lifetime); no page passage defines it. */
XATTN_API void xattn_plan_destroy(xattn_plan_t plan);

/* Thread-local message for the last non-OK status of this thread ("" if none).
 * Plumbing of the C boundary (error reporting); no page passage defines it. */
XATTN_API const char* xattn_last_error(void);

/* What a schedule holds (host-side summary, no GPU involved). */
typedef struct xattn_schedule_info {
  int32_t num_units[3];     /* per kernel family: 0 fp32, 1 bf16 decode, 2 bf16 MFMA tile */
  int32_t chunk_tokens[3];  /* KV chunk length per family (0: family unused) */
  int32_t decode_rows;      /* query rows (tokens x grouped heads) per decode unit */
  int32_t num_merge_rows;   /* output rows assembled from split chunks */
  int64_t workspace_rows;   /* fp32 partial rows (head_dim values + 1 lse each) */
  int64_t total_kv_tokens;  /* sum over requests of kv_len */
  int64_t visible_pairs;    /* sum over query rows and heads of visible keys */
  int64_t layout_generation; /* xattn_plan_info: the slot's layout generation (see
                                XATTN_PLAN_GRAPH_STABLE); 0 from xattn_schedule */
  int32_t slot;             /* xattn_plan_info: the slot (0 or 1) the schedule is in */
  int32_t reserved;
} xattn_schedule_info;

/*
 * xattn_schedule: build, on the host only, the schedule xattn_plan would stage for
 * the same arguments (no GPU call, usable without a device). Fills *info. When
 * `units` is not NULL it receives sum(num_units) records of 8 int32 each, families in
 * order: {request, kv_head, row0, nrows, kv_begin, kv_end, workspace_row (-1: written
 * straight to out), cost}. Query row `row` of a request is token row / group of head
 * kv_head * group + row % group. When `merges` is not NULL it receives num_merge_rows
 * records of 4 int32: {out_row = token * num_qo_heads + head, first workspace row,
 * chunk count, workspace row stride between chunks}. Same errors as xattn_plan.
 * Inspection of the plan step (page "mstar.engine.resources.attn.cross",
 * FlashInferCrossManager.plan) without a device; the pages define no such call.
 */
XATTN_API int xattn_schedule(const int32_t* qo_indptr, const int32_t* kv_indptr,
                   const int32_t* kv_page_indices, const int32_t* kv_last_page_len,
                   int32_t batch_size, int32_t num_qo_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t page_size, int64_t num_pages, int32_t mask_mode,
                   int32_t block_size, int32_t dtype, int32_t force_chunk,
                   xattn_schedule_info* info, int32_t* units, int32_t* merges);

/* The summary of the handle's current schedule. Inspection of the opaque plan result
 * (page "mstar.engine.resources.attn.cross", FlashInferCrossManager.plan); the pages
 * define no such call. */
XATTN_API int xattn_plan_info(xattn_plan_t plan, xattn_schedule_info* info);

/*
 * Kernel timing. With every > 0, every `every`-th later xattn_run on this handle
 * launches each kernel with a pair of HIP events that the runtime stamps with that
 * kernel's own start and end on the run's stream (hipExtLaunchKernel; at most 65536
 * pairs are kept; later runs are not recorded until the next collection). Sampling
 * keeps the small cost of the events off most runs.
 * xattn_plan_timing waits for the recorded events, writes the summed milliseconds
 * and the launch count per stage {0 fp32, 1 bf16 decode, 2 bf16 MFMA tile, 3 merge}
 * into ms[4] and launches[4], and clears the records. every <= 0 stops recording.
 * Measurement plumbing; no page passage defines it (the pages publish no timings).
 */
XATTN_API int xattn_plan_set_timing(xattn_plan_t plan, int every);
XATTN_API int xattn_plan_timing(xattn_plan_t plan, double* ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_H */
