// fi_internal.h -- shared definitions of the plan records and kernel launchers.
//
// Work item record (FI_ITEM_INTS = 12 int32), one per (unit, chunk):
//   0 q_base   first query token of the request (contiguous rows), or offset in
//              the member list of the item's group (FLAG_LIST_Q)
//   1 row0     first query row of the item within its unit's rows;
//              row rho -> query (rho / G), head kv_head*G + rho % G
//   2 n_rows   rows in the item (<= rows per block of its level)
//   3 kv_head
//   4 page_off start of the sequence's page list in its index array
//   5 flags    FLAG_* below
//   6 t_begin  first token (page aligned)
//   7 t_end    one past the last token
//   8 q_pos0   causal: sequence position of query 0 (kv_len - qo)
//   9 dst      first fp32 partial row (FLAG_PARTIAL), else -1
//  10 unit     request (or prefix group) id, informational
//  11 chunk    chunk index within the unit, informational
// Merge record (FI_MERGE_INTS = 6): q_base, row0, n_rows, kv_head, parts_off,
// n_parts; row k < n_rows (at most MERGE_ROWS) is rho = row0 + k of a unit,
// query token q_base + rho / G, head kv_head*G + rho % G, and folds partial
// rows parts[parts_off+j]+k, j in order. Scatter record (2 int32 per new token): index into kv_indices of the
// token's page, slot within the page.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fi {

// Kernel timer (fi_timer_begin): while a run call is timed, its attention
// launches record the timer's events in their own dispatch (the start event
// on the first launch, the stop event on each), so the interval is the
// kernels' execution, as a profiler's kernel trace measures it.
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchTiming& launch_timing();   // this thread's

// Launch an attention kernel with `lds` bytes of dynamic LDS (errors are
// left for hipGetLastError).
template <typename K, typename... Args>
inline void launch_timed_lds(K kernel, dim3 grid, dim3 block, unsigned lds, hipStream_t s,
                             Args... args) {
  LaunchTiming& t = launch_timing();
  if (t.stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, t.start, t.stop, 0, args...);
    t.start = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
}
template <typename K, typename... Args>
inline void launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  launch_timed_lds(kernel, grid, block, 0u, s, args...);
}

enum ItemField {
  F_Q_BASE = 0, F_ROW0, F_NROWS, F_KVHEAD, F_PAGEOFF, F_FLAGS,
  F_TBEGIN, F_TEND, F_QPOS0, F_DST, F_UNIT, F_CHUNK, ITEM_INTS
};
enum MergeField { M_QBASE = 0, M_ROW0, M_NROWS, M_KVHEAD, M_OFF, M_N, MERGE_INTS };
enum ItemFlag { FLAG_LIST_Q = 1, FLAG_PARTIAL = 2, FLAG_CAUSAL = 4, FLAG_PREFIX = 8 };

// Query rows per work item. Decode-style levels (decode, cascade suffix): one
// 16-row MFMA block per wavefront worker. Wide levels (append, cascade
// prefix): 128 rows per 4-wave workgroup worker sharing K/V through LDS.
constexpr int ROWS_DECODE = 16;
constexpr int ROWS_WIDE = 128;
constexpr int WAVES_PER_BLOCK = 4;
// Rows of a merge record at most (a unit's rows are cut into records of this
// many).
constexpr int MERGE_ROWS = 16;
// Plan counts the kernels read from device memory (the plan's meta section),
// so that a launch captured in a graph follows a later plan into the same
// workspace: the POD split, the merge records, their most rows, and the new
// tokens to scatter.
enum MetaField {
  META_POD_WIDE = 0, META_MERGES, META_MERGE_ROWS, META_SCATTER, META_EMPTY, META_INTS
};
// A wide level plans num_cus * max(1, workers_per_cu / 2) workgroups and
// chunks of at least WIDE_CHUNK_FACTOR * min_chunk_pages pages.
constexpr int WIDE_CHUNK_FACTOR = 2;

struct AttnArgs {
  const int32_t* items;
  const int32_t* worker_indptr;
  int32_t num_workers;
  const int32_t* qlist;
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* kv_indices;
  const int32_t* prefix_indices;
  uint16_t* o;
  float* lse;
  float* part_o;
  float* part_lse;
  const float* k_scale;    // FP8 cache only: [pages][Hkv] fp32 scale of each K tile
  const float* v_scale;    // FP8 cache only: the same for V
  const uint8_t* k_bscale; // MXFP4 cache only: E8M0 scale per 32 elements of a K row
  const uint8_t* v_bscale; // MXFP4 cache only: the same for V
  // Fused merge (decode plans; item_rec == NULL: the merge kernel runs after).
  // When a wave's stream of items ends, each of its partial items counts in at
  // its merge record, and the wave that brings a record's count to its part
  // count folds the record's rows in part order (the merge kernel's
  // arithmetic); it then resets the count to 0 for the next call. Records of
  // units with no keys are written (o = 0, lse = -inf) by the workers at start.
  const int32_t* item_rec; // per item of the level: its merge record, or -1
  int32_t* counters;       // per merge record: the level's chunks counted in
  const int32_t* merges;
  const int32_t* parts;
  const int32_t* empty_recs;
  const int32_t* meta;     // META_EMPTY: the number of empty_recs
  // 1: every split unit's chunks are the items of one workgroup's four waves
  // (a tiny batch); the wave with chunk 0 folds the unit after a workgroup
  // barrier instead of the counts above
  int32_t wg_fold;
  float scale_log2;        // sm_scale * log2(e): logits are kept in base 2
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t group;           // Hq / Hkv
  int32_t page_size;
  int32_t page_shift;      // log2(page_size)
};

struct MergeArgs {
  const int32_t* merges;
  int32_t num_merges;
  const int32_t* parts;
  const float* part_o;
  const float* part_lse;
  uint16_t* o;
  float* lse;
  int32_t num_qo_heads;
  int32_t head_dim;
  int32_t group;             // q heads per kv head
  int32_t rows_per_record;   // launch sizing: the most rows of a record (<= MERGE_ROWS)
  const int32_t* counts;     // device meta: the record count and most rows per record
};

struct ScatterArgs {
  const int32_t* scatter;   // 2 int32 per new token
  int32_t num_tokens;       // launch sizing (the count itself is read from counts)
  const int32_t* counts;    // device meta
  const int32_t* kv_indices;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t head_dim;
};

struct MergeStatesArgs {
  const void* v;
  int32_t v_f32;
  const float* s;
  int32_t N, S, H, D;
  void* v_out;
  int32_t out_f32;
  float* s_out;
};

// Decode-style level: one wavefront per worker (a.num_workers waves).
hipError_t launch_decode(const AttnArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_decode_valu(const AttnArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_decode_fp8(const AttnArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_decode_mxfp4(const AttnArgs& a, int head_dim, hipStream_t stream);
// Wide level: one 4-wave workgroup per worker (a.num_workers workgroups);
// list_q: query rows come through the member list (cascade prefix).
// ragged: keys in a [tokens][Hkv][D] layout (block-sparse plans), the page
// lists holding the first token of each page_size-token run.
hipError_t launch_wide(const AttnArgs& a, int head_dim, bool list_q, bool ragged,
                       hipStream_t stream);
// Fused launch: wa.num_workers workgroups; workgroup b < meta[0] is wide
// worker b, the others hold decode workers 4 (b - meta[0]) .. +3 of da;
// list_q as for launch_wide.
hipError_t launch_pod(const AttnArgs& wa, const AttnArgs& da, const int32_t* meta, int head_dim,
                      bool list_q, bool ragged, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_scatter(const ScatterArgs& a, hipStream_t stream);
hipError_t launch_merge_states(const MergeStatesArgs& a, hipStream_t stream);

}  // namespace fi
