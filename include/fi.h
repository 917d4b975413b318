/*
 * fi.h -- C ABI of the MI355X (gfx950) paged-KV attention library (libfi.so).
 *
 * What the library computes: exact softmax attention of query rows over K/V
 * gathered through a per-request block table (a block-sparse row format over a
 * pool of fixed-size pages), with grouped-query heads, the KV range of each
 * request split into load-balanced chunks by a host-side plan, and the chunks'
 * fp32 partial states (o, lse) merged in a fixed order. Sources:
 *   - Ye et al. catalogue record of the FlashInfer paper, fields "summary"
 *     (block-sparse KV representations; load-balanced scheduling that stays
 *     valid under static graph capture) and "boundary" (exact attention and
 *     paged KV storage are inherited, not changed);
 *   - research note "flashinfer-backend-selection", section "Arithmetic
 *     intensity" (decode reads K/V through a gathered block table; cascade
 *     reads a shared prefix once for all requests that share it);
 *   - FlashInfer PR #4038, section "What it does" (split partials kept in fp32
 *     and reduced in a fixed order, so results repeat bit for bit).
 *
 * Conventions shared by every call
 * --------------------------------
 * Layouts (row-major, element types as named):
 *   q        bf16 [T][Hq][D]      T = batch for decode/cascade, sum(qo) for append
 *   o        bf16 [T][Hq][D]      lse  fp32 [T][Hq] (natural log; may be NULL)
 *   k_cache, v_cache  bf16 [num_pages][Hkv][page_size][D]
 *   kv_indices int32 page ids; request r's pages are
 *            kv_indices[kv_indptr[r] .. kv_indptr[r+1]), token t of the request
 *            in page kv_indices[kv_indptr[r] + t / page_size], slot t % page_size.
 *   q head h reads kv head h / (Hq / Hkv).
 * Ownership: every pointer passed to a run call is caller-owned device memory
 *   and must stay valid until the stream work finishes. The library allocates
 *   no device memory: the plan lives in a caller-owned device workspace and a
 *   caller-owned pinned host staging buffer (sizes from fi_workspace_size).
 *   The fi_plan_t handle itself is library-owned host memory.
 * Streams: `stream` is a hipStream_t (NULL = default stream). Run calls only
 *   enqueue work and return; device faults surface at the caller's next
 *   synchronisation. Run calls neither allocate nor synchronise, so they may be
 *   captured in a HIP graph. A captured call replays its plan; with a
 *   graph-stable plan (fi_plan_desc.cap_batch > 0) it also serves every later
 *   plan of the same description built into the same workspace (Ye et al.
 *   record, "summary": load-balanced scheduling that stays valid under static
 *   graph capture).
 * Errors: every call returns FI_OK (0) or an error code and launches nothing
 *   on error; fi_last_error() gives a thread-local message. Device-side arrays
 *   (kv_indices) are trusted to agree with the host arrays given to fi_plan.
 * Threads: distinct plans are independent; one plan must not be used on two
 *   streams at once, and a re-plan of a workspace must not overlap its use.
 */
#ifndef FI_H
#define FI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fi_status {
  FI_OK = 0,
  FI_ERR_INVALID_ARG = 1,   /* null pointer, bad size, inconsistent host arrays */
  FI_ERR_UNSUPPORTED = 2,   /* head_dim not 64/128, page size, head grouping    */
  FI_ERR_WORKSPACE = 3,     /* a workspace is smaller than the plan needs       */
  FI_ERR_PLAN_MISMATCH = 4, /* plan of another kind used, or no plan            */
  FI_ERR_HIP = 5            /* HIP runtime error (message has its text)         */
} fi_status;

typedef enum fi_kind {
  FI_KIND_DECODE = 0,   /* one query token per request                      */
  FI_KIND_APPEND = 1,   /* qo_r query tokens per request, optional causal   */
  FI_KIND_CASCADE = 2,  /* decode over (shared prefix) || (own suffix)      */
  FI_KIND_BLOCK_SPARSE = 3  /* one sequence, a block mask per kv head (below) */
} fi_kind;

typedef enum fi_dtype { FI_DTYPE_BF16 = 0, FI_DTYPE_F32 = 1 } fi_dtype;

/* Which units run the decode-style levels (decode, and the per-request suffix
 * level of cascade). Both give the same result within the stated tolerance;
 * the choice is a measured speed question (the research note's "Arithmetic
 * intensity" places decode in the memory-bound regime, where either unit can
 * keep up with HBM). */
typedef enum fi_engine {
  FI_ENGINE_DEFAULT = 0, /* the engine measured faster on gfx950 (see fi_plan)   */
  FI_ENGINE_MFMA = 1,    /* bf16 matrix cores, v_mfma_f32_16x16x32_bf16           */
  FI_ENGINE_VALU = 2     /* vector ALU only, v_dot2_f32_bf16; head group <= 8     */
} fi_engine;

/* How a plan with two kinds of rows is launched: append plans (multi-query
 * requests and requests of a few query tokens) and cascade plans (shared
 * prefixes and per-request suffixes). POD attention (research note,
 * "Arithmetic intensity": prefill and decode rows of one batch in one
 * kernel) runs both kinds in one launch whose workgroups share every CU. */
typedef enum fi_launch {
  FI_LAUNCH_DEFAULT = 0,  /* POD, except with the VALU decode engine          */
  FI_LAUNCH_POD = 1,      /* one fused launch (matrix-core engine only)       */
  FI_LAUNCH_SEPARATE = 2  /* one launch per kind of rows                      */
} fi_launch;

/* KV cache format that a decode plan's run calls will read. It only picks
 * the default launch shape (workers_per_cu): results do not depend on it,
 * and any decode plan may be run with any of the decode calls. */
typedef enum fi_kv_format {
  FI_KV_BF16 = 0,   /* fi_paged_decode: 4 workers per CU (one wave per SIMD)  */
  FI_KV_FP8 = 1,    /* fi_paged_decode_fp8: 8 (two waves per SIMD)            */
  FI_KV_MXFP4 = 2   /* fi_paged_decode_mxfp4: 12 (three waves per SIMD; that
                       kernel is bound by ALU work and latency, not by HBM)   */
} fi_kv_format;

/* Where a decode plan's split units are merged (PR #4038, "What it does":
 * fp32 partials reduced in a fixed order). By default a merge kernel runs
 * after the attention kernel. FI_MERGE_FUSED (decode plans on the matrix-core
 * engine) folds them inside the attention kernel instead: when a wave's items
 * are done, each partial item counts in at its unit's merge record (a vector
 * atomic at agent scope, once its partial rows, stored with agent-scope
 * stores, have completed), and the wave whose count completes the record
 * folds it in part order with the merge kernel's arithmetic, so the bits are
 * the same. It saves the merge launch but measured slower on MI355X on full
 * batches: agent-scope stores write through the XCD's L2, which costs more
 * than the merge launch (Llama-like batch: 98 against 90 us per call). Other
 * plans ignore the field. */
typedef enum fi_merge_mode {
  FI_MERGE_DEFAULT = 0,   /* a merge launch after the attention kernel          */
  FI_MERGE_FUSED = 1,     /* folded in the decode kernels (decode plans, matrix
                             cores; the VALU engine uses the merge launch)     */
  FI_MERGE_SEPARATE = 2   /* a merge launch (the default)                       */
} fi_merge_mode;

/* Layout of the K/V a block-sparse plan reads (research note, "Arithmetic
 * intensity": paged and ragged KV-cache layouts). PAGED: pools
 * [num_pages][Hkv][page_size][D] and a page table. RAGGED: one contiguous
 * tensor [tokens][Hkv][D] per K and V, sequence s holding tokens
 * kv_indptr[s] .. kv_indptr[s+1]-1. Plans of other kinds read paged pools. */
typedef enum fi_kv_layout {
  FI_KV_LAYOUT_PAGED = 0,
  FI_KV_LAYOUT_RAGGED = 1
} fi_kv_layout;

/* Plan description. Zero in an optional field selects its default. */
typedef struct fi_plan_desc {
  int32_t kind;              /* fi_kind                                        */
  int32_t batch;             /* number of requests B (>= 0)                    */
  int32_t num_qo_heads;      /* Hq                                             */
  int32_t num_kv_heads;      /* Hkv, divides Hq                                */
  int32_t head_dim;          /* D: 64 or 128                                   */
  int32_t page_size;         /* tokens per page: power of two in [8, 256]      */
  int32_t causal;            /* append: 1 = bottom-right causal mask           */
  int32_t deterministic;     /* 1 = chunk boundaries depend on the request only */
  int32_t det_chunk_pages;   /* deterministic chunk size in pages (default 48)
                                on wide levels; decode-style levels of a bf16
                                cache cut a unit into chunks of half that, at
                                most 16 */
  int32_t min_chunk_pages;   /* balanced mode lower bound on chunk pages (default 8) */
  int32_t num_cus;           /* compute units to plan for (0 = current device) */
  int32_t workers_per_cu;    /* persistent wavefront workers per CU (default 4;
                                8 for a decode plan of format FI_KV_FP8, 12 for
                                FI_KV_MXFP4) */
  int32_t num_prefix_groups; /* cascade: number of shared prefixes             */
  int32_t decode_engine;     /* fi_engine for decode-style levels (default 0)  */
  int32_t max_prefix_depth;  /* cascade: longest chain of nested shared prefixes
                                a request may have (default 1; bounds the
                                workspace and is checked by fi_plan)          */
  int32_t launch;            /* fi_launch, append and cascade (default 0)      */
  int32_t pod_wide_blocks;   /* POD launch: workgroups of the wide role (0 =
                                sized by the plan's cost model)              */
  /* Graph-stable plan (cap_batch > 0; not for block-sparse plans): the
   * workspace is laid out for at most cap_batch requests and these totals
   * (the same bound fi_workspace_size gives for them, with batch =
   * cap_batch), every launch is made and sized from these capacities, and the
   * kernels read this batch's counts from the workspace. A run call captured
   * in a HIP graph then serves any later plan with the same description (the
   * batch and the number of prefix groups may change; max_prefix_depth is
   * part of the capacity) built into the same workspace. fi_workspace_size on
   * such a description returns that layout's size (its max_* arguments are
   * not used). fi_plan fails with FI_ERR_INVALID_ARG if the batch exceeds a
   * capacity. 0 = a plan laid out for its own batch. */
  int32_t cap_batch;
  int32_t cap_kv_pages;      /* sum of the requests' pages (suffix pages)     */
  int32_t cap_qo_tokens;     /* append: sum of query tokens                   */
  int32_t cap_prefix_pages;  /* cascade: sum of the groups' prefix pages      */
  int32_t kv_format;         /* decode: fi_kv_format (default FI_KV_BF16)     */
  int32_t merge_mode;        /* fi_merge_mode (default 0)                     */
  int32_t kv_layout;         /* fi_kv_layout: block-sparse plans (default 0)  */
} fi_plan_desc;

typedef struct fi_plan fi_plan_t;

/* Introspection of a plan's host-side arrays (for tests and tools). The
 * pointers stay valid until fi_plan_destroy. Item and merge records are
 * FI_ITEM_INTS / FI_MERGE_INTS int32 each, field order as in fi_internal.h. */
#define FI_ITEM_INTS 12
#define FI_MERGE_INTS 6
typedef struct fi_plan_info {
  int32_t kind;
  int32_t num_levels;            /* 2 for cascade (prefix, suffix), else 1 */
  int32_t num_workers[2];        /* per level: wavefronts (16-row levels) or
                                    4-wave workgroups (128-row levels) */
  int32_t min_chunk_pages[2];
  int32_t rows_per_block[2];
  int32_t chunk_pages[2];
  int32_t num_items[2];
  const int32_t* items[2];       /* grouped by worker                      */
  const int32_t* worker_indptr[2];
  int32_t num_merges;
  const int32_t* merges;
  int32_t num_parts;
  const int32_t* parts;
  int32_t num_qlist;
  const int32_t* qlist;
  int32_t num_part_rows;
  int32_t num_scatter;
  size_t dev_bytes_used;
  size_t host_bytes_used;
  int32_t pod_wide_blocks;       /* POD plans: workgroups of the wide role (the
                                    rest run the decode role), else 0 */
  int32_t num_plist;             /* block-sparse plans: the page lists the plan */
  const int32_t* plist;          /* built (items' page offsets index it)        */
  int32_t fused_merge;           /* 1: split units are folded in the kernel    */
  const int32_t* item_rec;       /* fused: per level-0 item, its merge record
                                    (-1 for an item writing final rows)        */
  int32_t num_empty_recs;        /* fused: records of units with no keys, which */
  const int32_t* empty_recs;     /* the kernel's workers write at start        */
  int32_t wg_fold;               /* fused tiny batch: unit u on the four waves of
                                    workgroup u (workers 4u..4u+3), folded
                                    after a workgroup barrier                   */
} fi_plan_info;

/* Upper bound on the device and pinned-host workspace bytes of any plan with
 * this description and at most the given totals (all requests' KV pages, all
 * query tokens, all prefix pages). Allocate once at these sizes to keep
 * addresses fixed across plans (graph capture). Pure host computation.
 * Errors: FI_ERR_INVALID_ARG (null/negative), FI_ERR_UNSUPPORTED (shape). */
fi_status fi_workspace_size(const fi_plan_desc* desc, int64_t max_kv_pages,
                            int64_t max_qo_tokens, int64_t max_prefix_pages,
                            size_t* dev_bytes, size_t* host_bytes);

/* Build the work plan (Ye et al. record, "summary": load-balanced scheduling
 * compatible with static graphs). Host arrays (all int32, host memory):
 *   kv_indptr_h [B+1] page offsets (kv_indptr_h[0] == 0, non-decreasing),
 *   kv_len_h [B] tokens, with kv_indptr_h[r+1]-kv_indptr_h[r] ==
 *     ceil(kv_len_h[r] / page_size) (cascade: the per-request suffixes);
 *   qo_indptr_h [B+1] (append only, else NULL): query-token offsets,
 *     qo_r <= kv_len_h[r]; kv_len counts the new tokens;
 *   prefix_indptr_h [NG+1], prefix_len_h [NG], req_prefix_group_h [B]
 *     (cascade only, else NULL): each group's prefix pages and tokens, and the
 *     group of each request (-1 = none);
 *   prefix_parent_h [NG] (cascade, optional): the group whose prefix comes
 *     before this group's (-1 = none), with parent index < group index. A
 *     request of group g then attends to the prefixes of g's chain, root
 *     first, then its own suffix: a tree of shared prefixes (research note,
 *     "Arithmetic intensity": every shared prefix is read once for all the
 *     requests under it). NULL: every group is a root.
 * The plan splits each request's KV range into chunks (deterministic mode:
 * about det_chunk_pages each, half that on bf16 decode-style levels, the same for a
 * request in any batch; balanced: about equal total work per worker), places
 * chunks on num_cus*workers_per_cu persistent workers (longest first), and
 * uploads the result into ws_dev with one hipMemcpyAsync on `stream` from the
 * pinned ws_host. ws_dev == NULL builds the plan on the host only (no HIP
 * call; run calls then refuse it) -- used for CPU tests with num_cus > 0.
 * Before overwriting ws_host the call waits for this workspace's previous
 * upload. On success *out receives a new handle (free with fi_plan_destroy).
 * Errors: FI_ERR_INVALID_ARG, FI_ERR_UNSUPPORTED, FI_ERR_WORKSPACE, FI_ERR_HIP. */
fi_status fi_plan(const fi_plan_desc* desc, const int32_t* kv_indptr_h,
                  const int32_t* kv_len_h, const int32_t* qo_indptr_h,
                  const int32_t* prefix_indptr_h, const int32_t* prefix_len_h,
                  const int32_t* req_prefix_group_h, const int32_t* prefix_parent_h,
                  void* ws_dev, size_t ws_dev_bytes, void* ws_host, size_t ws_host_bytes,
                  void* stream, fi_plan_t** out);

void fi_plan_destroy(fi_plan_t* plan);

fi_status fi_plan_get_info(const fi_plan_t* plan, fi_plan_info* info);

/* Common to the three run calls: the logits are sm_scale * q.k, and sm_scale
 * must be finite and > 0 (FI_ERR_INVALID_ARG otherwise, checked first); the
 * call enqueues its kernels on `stream`, never allocates and never
 * synchronises; a plan of another kind, or a host-only plan, gives
 * FI_ERR_PLAN_MISMATCH. */

/* Decode attention over the paged cache (research note "flashinfer-backend-
 * selection", "Arithmetic intensity": decode through a gathered block table).
 * Plan kind FI_KIND_DECODE. q [B][Hq][D] bf16 -> o [B][Hq][D] bf16 and lse
 * [B][Hq] fp32 (NULL to skip). Split requests are merged in chunk order.
 * A request with kv_len 0 gets o = 0, lse = -inf. */
fi_status fi_paged_decode(const fi_plan_t* plan, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* kv_indices,
                          float sm_scale, void* o, float* lse, void* stream);

/* Decode attention over an FP8 KV cache (v0.7.4 article, TL;DR: decoding
 * from a low-precision KV cache). Plan kind FI_KIND_DECODE on the matrix-core
 * engine (FI_ERR_UNSUPPORTED on the VALU engine). k_cache and v_cache hold
 * FP8 E4M3 codes (OCP 8-bit floating point: bias 7, no infinities, 0x7F and
 * 0xFF are NaN) in the bf16 layout [pages][Hkv][page_size][D], one byte per
 * element; k_scale and v_scale are fp32 [pages][Hkv], device memory, and the
 * element of page p, kv head g is decode(code) * scale[p][g]. Scales must be
 * finite (they are not checked). q, o, lse as in fi_paged_decode. The kernel
 * stages K and V through LDS and is bound by ALU work and latency as much as
 * by HBM: a plan of kv_format FI_KV_FP8 (default workers_per_cu 8, two waves
 * per SIMD) runs it faster than a bf16 plan (4). */
fi_status fi_paged_decode_fp8(const fi_plan_t* plan, const void* q, const void* k_cache,
                              const void* v_cache, const float* k_scale, const float* v_scale,
                              const int32_t* kv_indices, float sm_scale, void* o, float* lse,
                              void* stream);

/* Decode attention over an MXFP4 KV cache (v0.7.4 article, TL;DR: decoding
 * from a 4-bit KV cache), gfx950's native 4-bit format: OCP microscaling FP4,
 * E2M1 elements (0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives; sign in bit 3)
 * with one E8M0 scale (2^(code - 127); 255 = NaN) per 32 consecutive
 * elements of a token row. Plan kind FI_KIND_DECODE on the matrix-core
 * engine. k_codes, v_codes: uint8 [pages][Hkv][page_size][D/2], element 2i
 * in the low nibble of byte i; k_scales, v_scales: uint8
 * [pages][Hkv][page_size][D/32], device memory; D = 64 or 128. The element
 * is value(code) * 2^(scale - 127). q, o, lse as in fi_paged_decode.
 * This kernel is bound by ALU work and latency more than by HBM: a plan of
 * kv_format FI_KV_MXFP4 (default workers_per_cu 12, three waves per SIMD)
 * runs it about 1.2x faster than a bf16 plan (4, one wave per SIMD); any
 * decode plan gives the same results up to rounding. */
fi_status fi_paged_decode_mxfp4(const fi_plan_t* plan, const void* q, const void* k_codes,
                                const void* v_codes, const void* k_scales,
                                const void* v_scales, const int32_t* kv_indices,
                                float sm_scale, void* o, float* lse, void* stream);

/* Bytes of the library's static device scratch (per GPU), which
 * fi_paged_decode_noalloc uses in place of a plan workspace. */
#define FI_NOALLOC_SCRATCH_BYTES (16u << 20)

/* Decode attention that allocates nothing and needs no caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). Same computation,
 * kernels and results, bit for bit, as fi_paged_decode on a plan of the same
 * description and batch. `plan` must be a host-only decode plan (fi_plan with
 * ws_dev = NULL and num_cus > 0, normally the device's CU count): the call
 * uploads the plan's arrays with one hipMemcpyAsync on `stream` from the
 * plan's own host memory into a static device array of the library, of
 * FI_NOALLOC_SCRATCH_BYTES per GPU, which also holds the split partial states;
 * then it launches the attention and merge kernels on `stream`. It calls no
 * allocator. The array is shared by every call on a GPU and keeps the last
 * call's contents: calls that overlap on one GPU (other streams, other
 * threads) race on it and must be serialised by the caller. The plan handle
 * must stay alive until the call returns (the upload reads its host memory).
 * Errors: FI_ERR_PLAN_MISMATCH (not a host-only decode plan), FI_ERR_WORKSPACE
 * (the plan needs more than FI_NOALLOC_SCRATCH_BYTES of workspace, as
 * fi_plan_info.dev_bytes_used reports), FI_ERR_INVALID_ARG and FI_ERR_HIP as
 * fi_paged_decode; nothing is launched on error. */
fi_status fi_paged_decode_noalloc(const fi_plan_t* plan, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* kv_indices,
                                  float sm_scale, void* o, float* lse, void* stream);

/* Debug check of the device page tables that a run call with this plan
 * will read. The run calls trust them (the ABI conventions above); this call
 * lets a caller verify them while debugging. Counts the page ids outside
 * [0, num_pages) among the first kv_indptr[B] entries of kv_indices (the
 * entries the plan's host table covers) and, if prefix_indices is not NULL
 * (cascade plans), among the first prefix_indptr[num_prefix_groups] entries of
 * prefix_indices, and writes the count to *bad_count (one int32 in device
 * memory, overwritten; the write is ordered on `stream`, so read it after the
 * stream). Decode, append and cascade plans (FI_ERR_INVALID_ARG for a
 * block-sparse plan, whose page lists are copied from the host at plan
 * time); num_pages >= 1. */
fi_status fi_check_page_tables(const fi_plan_t* plan, const int32_t* kv_indices,
                               const int32_t* prefix_indices, int32_t num_pages,
                               int32_t* bad_count, void* stream);

/* Append / prefill attention for a mixed batch (research note, "Arithmetic
 * intensity": prefill and decode rows of one batch). Plan kind
 * FI_KIND_APPEND. If k_new and v_new ([sum qo][Hkv][D] bf16) are non-NULL,
 * first writes them into the cache slots of the new tokens (positions
 * kv_len-qo .. kv_len-1 of each request); then query i of request r (global
 * row qo_indptr[r]+i) attends to keys 0..kv_len-qo+i (causal plan) or to all
 * kv_len keys. Both or neither of k_new/v_new.
 * POD launch (the default): a request whose query rows (qo * Hq/Hkv) fit one
 * 16-row block runs in the decode role (one wavefront per worker, K/V
 * streamed through registers), every other request in the wide role (a
 * workgroup sharing K/V through LDS); one launch of
 * num_cus * max(1, workers_per_cu / 2) workgroups (two per CU by default, so
 * both roles share every CU) covers both, the plan giving pod_wide_blocks of
 * them to the wide role by estimated cost. FI_LAUNCH_SEPARATE runs every
 * request on the wide kernel instead. Same results either way, up to
 * rounding. */
fi_status fi_paged_append(const fi_plan_t* plan, const void* q, const void* k_new,
                          const void* v_new, void* k_cache, void* v_cache,
                          const int32_t* kv_indices, float sm_scale, void* o,
                          float* lse, void* stream);

/* Variable block-sparse attention over one sequence (research note,
 * "Arithmetic intensity": block-sparse and variable block-sparse plans; Ye et
 * al. record, "summary": composable block-sparse KV representations). For kv
 * head g, the qo_len query tokens are cut into num_row_blocks row blocks of
 * sizes row_block_sz[g][a] (host int32 [Hkv][num_row_blocks], each row sums
 * to qo_len) and the kv_len keys into num_col_blocks column blocks of sizes
 * col_block_sz[g][b] (host int32 [Hkv][num_col_blocks], each row sums to
 * kv_len, every non-empty block starting on a page boundary, so only the
 * sequence's last block may end inside a page); block_mask (host uint8 [Hkv][num_row_blocks]
 * [num_col_blocks], nonzero = attend) says which column blocks the rows of a
 * row block see. Query i of q head h (kv head g = h / (Hq/Hkv)) attends to
 * the keys of the selected column blocks of its row block, no causal mask; a
 * row with no selected key gets o = 0, lse = -inf. Block sizes may differ per
 * kv head and per block; zero-size blocks are allowed. The sequence's keys
 * are token t in page seq_pages_h[t / page_size] (host int32,
 * ceil(kv_len / page_size) page ids), slot t % page_size, of the usual pools.
 * Plan kind FI_KIND_BLOCK_SPARSE (desc.batch is ignored, desc.causal must be
 * 0): every (kv head, row block) becomes a unit over the page list of its
 * selected column blocks, stored in the plan's workspace, and is planned and
 * launched like an append batch (POD launch by default). Workspace bound from
 * fi_workspace_size_block_sparse. Errors as fi_plan, FI_ERR_INVALID_ARG for
 * sizes that do not add up or blocks off page boundaries. */
fi_status fi_workspace_size_block_sparse(const fi_plan_desc* desc, int32_t qo_len,
                                         int32_t kv_len, int32_t num_row_blocks,
                                         int32_t num_col_blocks, size_t* dev_bytes,
                                         size_t* host_bytes);
fi_status fi_plan_block_sparse(const fi_plan_desc* desc, int32_t qo_len, int32_t kv_len,
                               int32_t num_row_blocks, const int32_t* row_block_sz_h,
                               int32_t num_col_blocks, const int32_t* col_block_sz_h,
                               const uint8_t* block_mask_h, const int32_t* seq_pages_h,
                               void* ws_dev, size_t ws_dev_bytes, void* ws_host,
                               size_t ws_host_bytes, void* stream, fi_plan_t** out);
/* Variable block-sparse attention over a batch of sequences in one plan
 * (research note, "Arithmetic intensity": block-sparse and variable
 * block-sparse plans over paged and ragged KV layouts; Ye et al. record,
 * "summary": composable block-sparse KV representations). Sequence s has
 * qo_len_h[s] queries, q rows sum(qo_len_h[0..s-1]) onward, and kv_len_h[s]
 * keys; per kv head it is cut into num_row_blocks_h[s] row blocks and
 * num_col_blocks_h[s] column blocks with a block mask, exactly as for
 * fi_plan_block_sparse, its arrays concatenated over the sequences:
 * row_block_sz_h holds each sequence's [Hkv][num_row_blocks_h[s]] in turn,
 * col_block_sz_h each [Hkv][num_col_blocks_h[s]], block_mask_h each
 * [Hkv][num_row_blocks_h[s]][num_col_blocks_h[s]] (host memory). Keys:
 * desc.kv_layout PAGED: token t of sequence s in page
 * kv_indices_h[kv_indptr_h[s] + t / page_size] (kv_indptr_h[s+1] -
 * kv_indptr_h[s] == ceil(kv_len_h[s] / page_size)) of the usual pools;
 * RAGGED: token t of sequence s is row kv_indptr_h[s] + t of the [tokens][Hkv][D]
 * tensors (kv_indptr_h[s+1] - kv_indptr_h[s] == kv_len_h[s]; kv_indices_h is
 * not read), with page_size the granule of the key walk (column blocks start
 * on multiples of it, as in the paged layout); the kernels read whole
 * page_size-token runs, so the tensors must hold at least
 * kv_indptr_h[num_seqs] + page_size - 1 rows (rows past a sequence's end are
 * read and ignored). No query attends across sequences. Errors as
 * fi_plan_block_sparse. */
fi_status fi_workspace_size_block_sparse_batch(const fi_plan_desc* desc, int32_t num_seqs,
                                               const int32_t* qo_len_h, const int32_t* kv_len_h,
                                               const int32_t* num_row_blocks_h,
                                               const int32_t* num_col_blocks_h,
                                               size_t* dev_bytes, size_t* host_bytes);
fi_status fi_plan_block_sparse_batch(const fi_plan_desc* desc, int32_t num_seqs,
                                     const int32_t* qo_len_h, const int32_t* kv_len_h,
                                     const int32_t* num_row_blocks_h,
                                     const int32_t* row_block_sz_h,
                                     const int32_t* num_col_blocks_h,
                                     const int32_t* col_block_sz_h, const uint8_t* block_mask_h,
                                     const int32_t* kv_indptr_h, const int32_t* kv_indices_h,
                                     void* ws_dev, size_t ws_dev_bytes, void* ws_host,
                                     size_t ws_host_bytes, void* stream, fi_plan_t** out);
/* Run a block-sparse plan: q [T][Hq][D] bf16 -> o [T][Hq][D] bf16, lse
 * [T][Hq] fp32 (NULL to skip), T the plan's query rows; k_cache, v_cache the
 * pools the plan's page ids index (paged), or the [tokens][Hkv][D] tensors
 * (ragged). The page lists come from the plan's workspace. */
fi_status fi_block_sparse_attention(const fi_plan_t* plan, const void* q, const void* k_cache,
                                    const void* v_cache, float sm_scale, void* o, float* lse,
                                    void* stream);

/* Cascade decode (research note, "Arithmetic intensity": a shared prefix's KV
 * is read once and reused by every request that shares it). Plan kind
 * FI_KIND_CASCADE. Level 0 attends all member queries of a group to the
 * group's prefix pages (prefix_indices), level 1 each request to its own
 * suffix (kv_indices); the two states are merged prefix first. The result is
 * attention over prefix || suffix. By default (FI_LAUNCH_POD) both levels run
 * in one launch, the prefix level as the wide role and the suffix level as
 * the decode role, so the prefix's matrix work and the suffixes' HBM reads
 * overlap on every CU; FI_LAUNCH_SEPARATE runs them one after the other. */
fi_status fi_cascade(const fi_plan_t* plan, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* prefix_indices,
                     const int32_t* kv_indices, float sm_scale, void* o, float* lse,
                     void* stream);

/* Merge S attention states per row in fixed order, index 0 first (PR #4038,
 * "What it does": fp32 partials reduced in a fixed order). v [N][S][H][D] of
 * v_dtype, s [N][S][H] fp32 natural-log LSE -> v_out [N][H][D] of out_dtype,
 * s_out [N][H] (NULL to skip). States with s = -inf contribute nothing; if all
 * are -inf the row is 0 with s_out -inf. D in [1, 1024], a multiple of 4. */
fi_status fi_merge_states(const void* v, int32_t v_dtype, const float* s, int32_t N,
                          int32_t S, int32_t H, int32_t D, void* v_out,
                          int32_t out_dtype, float* s_out, void* stream);

/* Thread-local text of the last error returned on this thread ("" if none). */
const char* fi_last_error(void);

/* Kernel timer for measurement: while enabled, every run call records a HIP
 * event pair on its stream around its attention kernel(s) (not the merge or
 * scatter). fi_timer_begin(capacity) starts a fresh window of up to capacity
 * calls; fi_timer_end synchronises on the recorded events and returns the
 * summed milliseconds and the number of calls recorded, then disables it. */
fi_status fi_timer_begin(int32_t capacity);
fi_status fi_timer_end(double* total_ms, int32_t* calls);

#ifdef __cplusplus
}
#endif

#endif /* FI_H */
