/*
 * pod_attn.h -- C ABI of the fused hybrid-batch paged attention library for MI355X (gfx950).
 *
 * One call computes, for a mixed batch, exact causal chunked-prefill attention (a query chunk
 * over its cached prefix plus itself) and decode attention (one query token over its whole
 * context), reading K and V from a paged KV cache through per-sequence block tables.
 *
 * Sources (web pages; sections as printed on them):
 *   [POD] Silicon & Systems digest "POD-Attention hybrid batching": one fused launch whose
 *         software scheduler hands prefill or decode work to each compute unit (section
 *         "Virtual CTAs and per-SM balance"); comparison against separate and stream-concurrent
 *         launches (sections "Why concurrency alone is not enough", "Reproduction and hardware
 *         evaluation"); unsupported shapes fall back and the runtime reports tile choice,
 *         occupancy and fallback reasons (section "Predictable latency and diagnostics").
 *   [W6]  "Week 6: Beyond PyTorch: Custom Kernel과 vLLM": attention equation (section
 *         "Attention에 적용하기"), causal rule ("Non-Causal vs. Causal Attention"), prefill /
 *         extend / decode kinds ("한 스텝에 여러 종류의 request 섞기"), paged blocks and block
 *         tables ("PagedAttention"), padding-free packed batches ("vLLM 내부 구조").
 *   [W4]  "LLMSO - W4 - Optimization & Frameworks": online softmax, split-KV decoding with a
 *         max/sum combine, block-table gather, GQA (section "1-2. 어텐션 최적화").
 *
 * Definition of the result (exact; no approximation):
 *   For query row r of sequence s at absolute position i, query head h, KV head
 *   g = floor(h / (Hq / Hkv)):
 *       out[r][h] = sum_{j <= i} softmax_j(scale * <q[r][h], k_s[j][g]>) * v_s[j][g]
 *   with j running over the sequence's logical tokens 0 .. ctx-1.  A prefill (extend) chunk of
 *   L rows with context ctx holds positions ctx-L .. ctx-1 (its own K/V are already in the
 *   cache); a decode row is at position ctx-1.
 *
 * Buffer formats (all row-major, element type bf16 or fp32 as configured, same for all):
 *   q, out   [total_q][Hq][D]; rows 0 .. P-1 are the prefill chunks back to back in batch order
 *            (P = prefill_q_start[num_prefill]), rows P .. P+num_decode-1 the decode queries.
 *   k_cache  [num_pages][Hkv][D/x][16][x]  with x = 16 bytes / element size (8 for bf16, 4 for
 *            fp32): element (page, g, slot t, dim d) at (((page*Hkv+g)*(D/x) + d/x)*16 + t)*x + d%x.
 *            One (page, head) slab is 16*D*elem bytes, contiguous; every 16-byte chunk holds x
 *            consecutive dims of one token.
 *   v_cache  [num_pages][Hkv][D][16]: element (page, g, t, d) at ((page*Hkv+g)*D + d)*16 + t.
 *            Each 16-byte chunk holds 8 (bf16) or 4 (fp32) consecutive tokens of one dim.
 *   block_tables  int32 [num_prefill + num_decode][block_table_stride], device memory.  Row s
 *            maps logical page t/16 of sequence s to a physical page; rows for the prefill
 *            sequences come first, then one row per decode.  Only entries 0 .. ceil(ctx/16)-1
 *            of a row are read; slots past ctx in the last page are never used in the result.
 *
 * Ownership: the caller owns every device buffer (q, caches, block tables, out, workspace) and
 * every host array.  The handle owns host state only (plus two HIP streams and events for STREAMS
 * mode, timing events, and a small pinned host staging ring).  No call allocates device memory;
 * the library itself holds one fixed scratch array per GPU for pod_attn_run_noalloc.
 *
 * Errors: every call returns a pod_attn_status; on a non-OK status pod_attn_last_error()
 * returns a message for the calling thread.  pod_attn_run is asynchronous on `stream`;
 * argument and launch errors are returned synchronously; device faults surface at the
 * caller's next synchronisation, as for any HIP launch.  A block-table entry outside
 * [0, num_pages_in_pool) is never dereferenced: the kernels read nothing for that page,
 * treat its tokens as absent and set POD_ATTN_DEVICE_ERR_BAD_PAGE in the workspace status word
 * (see pod_attn_read_device_status).
 */
#ifndef POD_ATTN_H
#define POD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  POD_ATTN_OK = 0,
  POD_ATTN_ERR_INVALID_ARG = -1,   /* null pointer, inconsistent metadata, bad sizes          */
  POD_ATTN_ERR_UNSUPPORTED = -2,   /* valid but unsupported shape (head_dim, group size, ...) */
  POD_ATTN_ERR_WORKSPACE = -3,     /* workspace missing or smaller than pod_attn_workspace_size */
  POD_ATTN_ERR_HIP = -4,           /* a HIP runtime call failed (message has the HIP error)    */
  POD_ATTN_ERR_NO_DEVICE = -5      /* no usable gfx950 device for create()                     */
} pod_attn_status;

/* Element types.  FP8_E4M3: q and out are bf16; k_cache and v_cache hold OCP FP8 E4M3 codes
 * (1 byte, x = 16 in the K layout) and every (page, KV head) slab has one float scale for K and
 * one for V: an element's value is decode(code) * scale ([W6] "KV Cache": a low-precision cache
 * such as FP8 halves what each decode step reads).  Runs take the scales through
 * pod_attn_run_scaled. */
typedef enum { POD_ATTN_BF16 = 0, POD_ATTN_FP32 = 1, POD_ATTN_FP8_E4M3 = 2 } pod_attn_dtype;

/* FUSED: one persistent launch, prefill and decode work claimed per compute unit.
 * SEPARATE: prefill kernel, then decode kernel, then the split combine, serially on `stream`.
 * STREAMS: prefill on one internal stream concurrently with decode (+combine) on another;
 * both wait for `stream` and `stream` waits for both.  All modes give the same result up to
 * floating-point rounding order ([POD], "Why concurrency alone is not enough"). */
typedef enum { POD_ATTN_MODE_FUSED = 0, POD_ATTN_MODE_SEPARATE = 1, POD_ATTN_MODE_STREAMS = 2 } pod_attn_mode;

/* Fallback reasons reported in pod_attn_stats.fallback_reason ([POD], "Predictable latency
 * and diagnostics": unsupported-but-valid work is routed to separate kernels, with a reason). */
typedef enum {
  POD_ATTN_FALLBACK_NONE = 0,
  POD_ATTN_FALLBACK_NO_PREFILL = 1,    /* nothing to overlap: fused kernel runs decode only    */
  POD_ATTN_FALLBACK_NO_DECODE = 2,     /* nothing to overlap: fused kernel runs prefill only   */
  POD_ATTN_FALLBACK_OCCUPANCY = 3,     /* fused kernel cannot keep 2 workgroups per CU; ran SEPARATE */
  POD_ATTN_FALLBACK_ENV = 4,           /* mode overridden by POD_ATTN_MODE                      */
  POD_ATTN_NUM_FALLBACK_REASONS = 5
} pod_attn_fallback;

/* Flags */
#define POD_ATTN_FLAG_DEBUG_CLAIMS 1   /* count every work-item claim in the workspace (tests) */
#define POD_ATTN_FLAG_TRACE 2          /* record a timeline entry per work item (pod_attn_read_trace) */

typedef struct pod_attn_config {
  int num_q_heads;          /* Hq >= 1                                                        */
  int num_kv_heads;         /* Hkv >= 1, Hq % Hkv == 0, group Hq/Hkv <= 16                     */
  int head_dim;             /* D: 64 or 128                                                   */
  int page_size;            /* tokens per page: must be 16                                    */
  int dtype;                /* pod_attn_dtype                                                 */
  int mode;                 /* pod_attn_mode                                                  */
  float scale;              /* softmax scale; 0 means 1/sqrt(head_dim)                        */
  int decode_split_tokens;  /* 0: automatic; else tokens per decode work item (multiple of 128) */
  int prefill_split_cap;    /* 0: automatic; else max KV splits of one prefill tile (>= 1)     */
  int wgs_per_cu;           /* 0: automatic; else persistent workgroups per CU in FUSED mode  */
  int flags;                /* POD_ATTN_FLAG_*                                                */
  int extend_max_q;         /* prefill (extend) chunks of at most this many query rows, whose
                               rows x group <= 16, run on the decode path as small-q extends:
                               0 = automatic (16), -1 = never, else 1..256                     */
} pod_attn_config;

/* Batch metadata: host arrays ([W6] "vLLM 내부 구조": padding-free packing with offsets). */
typedef struct pod_attn_batch {
  int num_prefill;                 /* prefill (extend) chunks, >= 0                           */
  const int32_t* prefill_q_start;  /* host [num_prefill+1]: row offsets, [0] = 0, non-decreasing */
  const int32_t* prefill_ctx_len;  /* host [num_prefill]: ctx = chunk offset + chunk length     */
  int num_decode;                  /* decode sequences, >= 0                                   */
  const int32_t* decode_ctx_len;   /* host [num_decode]: context length (>= 1), query at ctx-1  */
  int block_table_stride;          /* int32 entries per block-table row, >= ceil(max ctx / 16) */
  int num_pages_in_pool;           /* pages in k_cache / v_cache                               */
} pod_attn_batch;

typedef struct pod_attn_handle pod_attn_handle;   /* opaque, host-side */

/* Diagnostics of a handle's runs ([POD], "Predictable latency and diagnostics": virtual-CTA
 * ratio, tile choice, occupancy, memory throughput, fallback reason; [POD], "Reproduction and
 * hardware evaluation": the share of iterations that took the fused path and every fallback
 * cause).  The fields up to num_small_extends describe the last run; runs, runs_fused_path and
 * fallback_runs count over the handle's life; kernel_us and the achieved rates are those of the
 * newest run whose attention kernels have completed when pod_attn_get_stats is called (timed_run
 * names it; pod_attn_get_stats never waits for the GPU). */
typedef struct pod_attn_stats {
  int mode_requested;
  int mode_used;
  int fallback_reason;          /* pod_attn_fallback                                          */
  int num_prefill_items;        /* prefill work items (tile x KV head x KV split)             */
  int num_decode_items;         /* decode work items (sequence x KV head x split)             */
  int num_combine_groups;       /* (query tile, KV head) groups whose splits are combined     */
  int prefill_tile_cols;        /* query-head columns per prefill tile (queries x group)      */
  int prefill_tile_queries;     /* query rows per prefill tile                                */
  int prefill_kv_tile;          /* keys per prefill inner iteration                           */
  int prefill_max_splits;       /* largest KV split count of a prefill tile                   */
  int decode_split_tokens;      /* tokens per decode work item                                */
  int decode_max_splits;        /* largest split count of a decode (sequence, KV head)        */
  int grid_wgs;                 /* workgroups launched by the fused kernel (0 otherwise)      */
  int wgs_per_cu;               /* persistent workgroups per CU in FUSED mode                 */
  int num_cus;                  /* compute units of the device                                */
  int lds_bytes_per_wg;         /* LDS of the fused kernel per workgroup                      */
  int vgprs_per_lane;           /* registers of the fused kernel per lane (arch + acc)        */
  size_t workspace_bytes;       /* workspace needed by this batch                             */
  double host_plan_us;          /* host planning time of the last run                         */
  int prefill_wg_budget;        /* FUSED: prefill-role workgroups allowed while decode remains */
  int num_append_units;         /* KV append units of the last run (0 for pod_attn_run)      */
  int num_small_extends;        /* prefill chunks run on the decode path as small-q extends   */
  uint64_t runs;                /* runs (pod_attn_run*) that launched work on this handle      */
  uint64_t runs_fused_path;     /* of them, runs on the fused kernel with both kinds of work  */
  uint64_t fallback_runs[POD_ATTN_NUM_FALLBACK_REASONS];   /* runs per fallback_reason value  */
  double algorithmic_bytes;     /* last run: K and V once per KV head per context token, q in,
                                   out, one block-table entry per page (+ FP8 scales)         */
  double algorithmic_flops;     /* last run: 4*D per visible (query head, key) pair           */
  uint64_t timed_run;           /* run number (1-based) the kernel time below belongs to; 0: none */
  double kernel_us;             /* that run's attention kernels, first start to last end (< 0: none) */
  double achieved_gbps;         /* that run's algorithmic bytes / kernel_us                    */
  double achieved_tflops;       /* that run's algorithmic FLOPs / kernel_us                    */
} pod_attn_stats;

/* Create a handle for one attention configuration on the current HIP device.  Validates the
 * configuration (ERR_INVALID_ARG / ERR_UNSUPPORTED) and queries the device (ERR_NO_DEVICE if
 * it is not a gfx950).  Launches nothing. */
pod_attn_status pod_attn_create(const pod_attn_config* cfg, pod_attn_handle** out);

/* Bytes of device workspace pod_attn_run needs for this batch (work lists, counters, split
 * partials).  Validates the batch metadata. */
pod_attn_status pod_attn_workspace_size(pod_attn_handle* h, const pod_attn_batch* batch, size_t* bytes);

/* Compute the hybrid batch: for every query row, exact causal attention over its sequence's
 * cached keys and values ([W6] "Attention에 적용하기": softmax(Q K^T / sqrt(d_k)) V; [W6]
 * "Non-Causal vs. Causal Attention": a token sees itself and earlier tokens; [W6] "한 스텝에
 * 여러 종류의 request 섞기": extend and decode rows in one batch), read through the block tables
 * ([W6] "PagedAttention"), long key ranges split and merged by their maxima and sums ([W4]
 * "FlashDecoding -- decode 단계의 병렬성 확보").  q, k_cache, v_cache, block_tables, out and
 * workspace are device pointers in the formats above; `stream` is a hipStream_t (NULL = null stream).  Plans the
 * work on the host, copies the plan into `workspace` and launches on `stream` (FUSED: one
 * kernel; SEPARATE: up to three; STREAMS: as SEPARATE on two internal streams joined by
 * events).  Returns before the GPU finishes.  `out` rows are each written exactly once; no
 * other memory than `out` and `workspace` is written. */
pod_attn_status pod_attn_run(pod_attn_handle* h, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables,
                             const pod_attn_batch* batch, void* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* pod_attn_run for an FP8_E4M3 handle: k_scale and v_scale are device float arrays
 * [num_pages_in_pool][Hkv], the scale of each (page, KV head) slab of k_cache / v_cache.  The
 * result is attention over the decoded, scaled cache (value = decode(code) * scale, any finite
 * scale).  Decode rows multiply their fp32 scores by the K scale and their probabilities by the
 * V scale (the row sum takes them unscaled); prefill tiles round each decoded, scaled value to
 * bf16 when they stage it, as a bf16 cache holds it.  Other handles: POD_ATTN_ERR_INVALID_ARG.
 * Everything else as pod_attn_run; pod_attn_run on an FP8_E4M3 handle returns
 * POD_ATTN_ERR_INVALID_ARG (the scales are required) and pod_attn_run_append
 * POD_ATTN_ERR_UNSUPPORTED (writing FP8 needs a quantizer, which stays with the cache's
 * producer). */
pod_attn_status pod_attn_run_scaled(pod_attn_handle* h, const void* q, const void* k_cache,
                                    const void* v_cache, const float* k_scale, const float* v_scale,
                                    const int32_t* block_tables, const pod_attn_batch* batch,
                                    void* out, void* workspace, size_t workspace_bytes, void* stream);

/* KV append, then the hybrid batch: the step's new tokens are first written into the cache and
 * attention then reads them ([W6] "KV Cache": each step adds the new tokens' keys and values to
 * the cache before attending; [W6] "PagedAttention": position p of sequence s is slot p % 16 of
 * page block_tables[s][p / 16]).  k_new and v_new are device buffers [total_q][Hkv][D] of the
 * cache's element type, rows in q's row order; row r's token is written at its query position
 * (a prefill chunk's L rows at ctx-L .. ctx-1, a decode row at ctx-1) into k_cache / v_cache,
 * then the result is exactly that of pod_attn_run on the updated cache.  Only the slots of the
 * new positions are written; every other cache byte is left as it was.  FUSED: the append rides
 * in the plan-upload launch that precedes the persistent attention kernel (no extra launch);
 * SEPARATE and STREAMS: an append kernel of its own runs after the upload, before attention.
 * Slots of the new positions must be distinct: two rows mapping to the same slot give an
 * unspecified byte mix.  A block-table entry outside the pool is not written through and is
 * reported as POD_ATTN_DEVICE_ERR_BAD_PAGE by the attention kernels, which read that page.  Null k_new or
 * v_new, or buffers not 16-byte aligned, give POD_ATTN_ERR_INVALID_ARG; the workspace is sized
 * by pod_attn_workspace_size as for pod_attn_run.  The caller owns every buffer. */
pod_attn_status pod_attn_run_append(pod_attn_handle* h, const void* q, const void* k_new,
                                    const void* v_new, void* k_cache, void* v_cache,
                                    const int32_t* block_tables, const pod_attn_batch* batch,
                                    void* out, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  pod_attn_run, with the workspace taken from a fixed
 * device array that the library holds on every GPU it runs on (POD_ATTN_NOALLOC_SCRATCH_BYTES,
 * 256 MiB, held from the first pod_attn_create on that GPU until the process ends) instead of a
 * caller's buffer.  The caller still passes q, the caches, the block tables and out, in the formats
 * above; the result is bitwise that of pod_attn_run with a workspace of its own (same plan, same
 * kernels).  The call allocates nothing: no device or pinned memory (the handle's pinned staging
 * slots were made by pod_attn_create).  Errors as pod_attn_run, plus POD_ATTN_ERR_WORKSPACE when
 * the batch needs more workspace than the scratch holds (pod_attn_workspace_size tells) or a plan
 * larger than the handle's staging slots (256 KiB each), both before anything is launched.  Every
 * call on a GPU shares that GPU's scratch, which keeps the last call's contents (each run clears
 * the counters it needs): calls that overlap on one GPU -- concurrent streams, or handles used
 * from several threads -- race and must be serialised by the caller.  FP8_E4M3 handles need their
 * scales: POD_ATTN_ERR_INVALID_ARG. */
#define POD_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
pod_attn_status pod_attn_run_noalloc(pod_attn_handle* h, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const pod_attn_batch* batch, void* out, void* stream);

/* Copy the diagnostics of the last run into *st. */
pod_attn_status pod_attn_get_stats(pod_attn_handle* h, pod_attn_stats* st);

/* Debug/test: gather one sequence's K (which = 0) or V (which = 1) for all KV heads into
 * out_contig [ctx][Hkv][D] (same element type), through the same page-address arithmetic the
 * attention kernels use: logical token t is slot t % 16 of the physical page that row `seq` of
 * block_tables names for logical page t / 16 ([W6] "PagedAttention"; [W4] "PagedAttention --
 * 메모리 단편화를 없애는 커널": the kernel follows the block table to the scattered pages).
 * Bit-exact copy; asynchronous on `stream`.  FP8_E4M3 handles also take which = 2 (K) / 3 (V):
 * each code decoded to bf16 (unscaled) by the kernels' conversion.  A block-table entry outside
 * [0, num_pages_in_pool) is not read: its tokens come out as zeros and, when device_status (a
 * device int32, may be NULL) is given, POD_ATTN_DEVICE_ERR_BAD_PAGE is OR-ed into it.  Errors:
 * POD_ATTN_ERR_INVALID_ARG for null buffers, a bad `which`, `seq` or `ctx`, or a misaligned
 * device_status. */
pod_attn_status pod_attn_gather_kv(pod_attn_handle* h, const void* cache, int which,
                                   const int32_t* block_tables, int seq, int ctx,
                                   const pod_attn_batch* batch, void* out_contig,
                                   int32_t* device_status, void* stream);

/* Debug/test: synchronise `stream` and read the workspace status word written by the last run
 * (bit POD_ATTN_DEVICE_ERR_BAD_PAGE), the per-CU claim totals of each kind (every run counts
 * them; up to cu_cap entries each, indexed by the cu_slot of pod_attn_read_trace; may be NULL)
 * and, if the handle has POD_ATTN_FLAG_DEBUG_CLAIMS, the per-item claim counts (claims[i] for
 * prefill items first, then decode items; up to claims_cap entries).  Returns the number of
 * items in *n_items. */
#define POD_ATTN_DEVICE_ERR_BAD_PAGE 1
pod_attn_status pod_attn_read_device_status(pod_attn_handle* h, const void* workspace,
                                            void* stream, int32_t* status_word,
                                            int32_t* claims, int claims_cap, int* n_items,
                                            int32_t* prefill_claims_per_cu,
                                            int32_t* decode_claims_per_cu, int cu_cap);

/* Run diagnostics ([POD] "Predictable latency and diagnostics": the runtime should expose the
 * virtual-CTA ratio, occupancy and memory throughput of the fused kernel).  Synchronises
 * `stream`, then reads what the last run on this handle left in `workspace` (which must be the
 * workspace of that run): every run counts, per compute unit, the work items of each kind the
 * CU's workgroups claimed, so the balance of the two kinds on each CU is known without a debug
 * flag.  Shares are prefill items / all items of a CU, over the CUs that ran any item.  The
 * kernel time and achieved rates are those of the last run (the same figures pod_attn_get_stats
 * gives once the run has completed). */
typedef struct pod_attn_run_diag {
  int status_word;              /* device status bits of the run (POD_ATTN_DEVICE_ERR_*)       */
  int planned_prefill_items, planned_decode_items;
  int prefill_items, decode_items;   /* items claimed, summed over the CUs (equal to the planned counts) */
  int cus_any;                  /* CUs that ran any item                                      */
  int cus_prefill, cus_decode;  /* CUs that ran at least one item of the kind                 */
  int cus_both;                 /* CUs that ran both kinds in this run                        */
  int max_prefill_per_cu, max_decode_per_cu;
  double prefill_decode_ratio;  /* prefill items / decode items (0 when there is no decode)  */
  double mean_prefill_share, min_prefill_share, max_prefill_share;
  uint64_t run, timed_run;      /* the last run's number and the run the timing belongs to    */
  double kernel_us, achieved_gbps, achieved_tflops;
} pod_attn_run_diag;
pod_attn_status pod_attn_read_run_diagnostics(pod_attn_handle* h, const void* workspace,
                                              void* stream, pod_attn_run_diag* out);

/* Debug/profiling: synchronise `stream` and copy the per-item timeline of the last run, for a
 * handle created with POD_ATTN_FLAG_TRACE (else POD_ATTN_ERR_INVALID_ARG).  One record of 4
 * uint32 per work item, prefill items first then decode items (the order of
 * pod_attn_plan_inspect): {start, end, cu_slot, kind}, start/end being the low 32 bits of the
 * device's 100 MHz constant clock when the item began and ended, cu_slot = XCC_ID*128 +
 * SE*32 + SH*16 + CU of the compute unit that ran it, kind 0 prefill / 1 decode.  At most cap
 * records are written; *n_items receives the item count.  The workspace must be the one
 * passed to that run; tracing adds one 16-byte store per item. */
pod_attn_status pod_attn_read_trace(pod_attn_handle* h, const void* workspace, void* stream,
                                    uint32_t* records, int cap, int* n_items);

/* Host-only (no GPU needed): plan a batch for a device with num_cus compute units and
 * wgs_per_cu persistent workgroups, and return the work items as 16 int32 each
 * {seq, q_row, n_q, q_pos, kv_head, kv_begin, kv_end, group, split, partial_slot, kind
 * (0 prefill, 1 decode), queue, 0...}, prefill items first, in the order the kernels index
 * them.  queue is the per-XCD claim queue (0..7) of a prefill item and -1 for decode.
 * *n_items receives the count; at most items_cap items are written.  stats (may be NULL)
 * receives the planning diagnostics. */
pod_attn_status pod_attn_plan_inspect(const pod_attn_config* cfg, const pod_attn_batch* batch,
                                      int num_cus, int wgs_per_cu, int32_t* items,
                                      int items_cap, int* n_items, pod_attn_stats* stats);

/* Scheduler signals for one batch, host-only (no GPU): what an outer scheduler needs to bucket
 * prefill chunks and decode groups by their resource use ([POD] "Resource characteristics as
 * scheduling inputs": work units, shared memory, arithmetic intensity and bytes read), as this library would
 * plan the batch on a device of num_cus CUs with wgs_per_cu persistent workgroups each.  The
 * "prefill share" is the chunks planned as tiles; the "decode share" is the decodes plus the
 * small-q extends.  FLOPs count 4*D per visible (query head, key) pair; bytes count K and V once
 * per KV head per context token of the share's sequences, q read and out written once, and per
 * page its block-table entry (and, for an FP8 cache, its K and V scales of every KV head).
 * roofline_us = max(total FLOPs / peak_tflops, total bytes / peak_gbps) for the given peaks
 * (<= 0 selects MI355X's: 8000 GB/s; 2500 TFLOP/s bf16, 157.3 fp32). */
typedef struct pod_attn_signals {
  int prefill_items;          /* prefill work items (tile x KV head x split)                    */
  int decode_items;           /* decode-path work items (sequence or extend x KV head x split)  */
  int combine_groups;         /* split groups merged by log-sum-exp                             */
  int small_extends;          /* prefill chunks planned on the decode path                      */
  int grid_wgs;               /* persistent workgroups of the fused launch                      */
  int lds_bytes_per_wg;       /* LDS each fused workgroup holds                                 */
  int fallback_reason;        /* what a FUSED run reports: NONE, NO_PREFILL or NO_DECODE         */
  size_t workspace_bytes;
  double prefill_flops, decode_flops;
  double prefill_bytes, decode_bytes;
  double intensity;           /* total FLOPs / total bytes                                      */
  double roofline_us;
} pod_attn_signals;
pod_attn_status pod_attn_batch_signals(const pod_attn_config* cfg, const pod_attn_batch* batch,
                                       int num_cus, int wgs_per_cu, double peak_gbps,
                                       double peak_tflops, pod_attn_signals* out);

/* Profiling hook: when ev_start / ev_end (hipEvent_t, may be NULL) are set, the next
 * pod_attn_run (or pod_attn_run_append) records ev_start on the launch stream right after the
 * plan upload, before the first attention kernel, and ev_end after the last one (FUSED mode:
 * the fused kernel alone; SEPARATE mode: the append kernel if any, then prefill, decode and
 * combine kernels; STREAMS mode: from the append kernel if any to after the join), so that the
 * kernels' own duration can be read with hipEventElapsedTime.
 * The hook is consumed by that run (one-shot); the events stay owned by the caller. */
pod_attn_status pod_attn_set_kernel_events(pod_attn_handle* h, void* ev_start, void* ev_end);

/* Measurement probes: the peaks that achieved rates can be compared with on the machine at hand,
 * beside the vendor figures.  No handle; asynchronous on `stream`.
 *
 * pod_attn_probe_hbm_read: one streaming read of `bytes` bytes at `buf` (device, 16-byte aligned,
 * bytes a positive multiple of 16), 4096 workgroups of 256 threads; wave v of the grid reads the
 * 16 KiB blocks v, v + 16384, ... (16-byte chunks, consecutive lanes on consecutive chunks) with
 * two blocks in flight.  sink (device, 4096 uint32) receives per workgroup the XOR of
 * the 32-bit words it read, so the XOR of all of sink equals the XOR of the buffer's words.
 *
 * pod_attn_probe_mfma: dense bf16 32x32x16 MFMA work, 4096 workgroups of 4 waves, each wave
 * running 8 independent accumulation chains for `iters` rounds (1 <= iters <= 2^20) on operands
 * whose products add exactly 1.0 per round; sink (device, 4 * 4096 floats) receives 8 * iters per
 * wave.  *flops (may be NULL) receives the FLOPs performed (2*32*32*16 per MFMA).
 *
 * Errors: POD_ATTN_ERR_INVALID_ARG for null or misaligned arguments and out-of-range sizes;
 * POD_ATTN_ERR_HIP if the launch fails. */
pod_attn_status pod_attn_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
pod_attn_status pod_attn_probe_mfma(int iters, float* sink, double* flops, void* stream);

/* Thread-local message for the last non-OK status returned on this thread. */
const char* pod_attn_last_error(void);

/* Release the handle (internal streams and events included).  NULL is ignored. */
void pod_attn_destroy(pod_attn_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* POD_ATTN_H */
