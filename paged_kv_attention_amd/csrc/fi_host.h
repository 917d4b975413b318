// fi_host.h -- host-side plan state and error reporting shared by the C ABI
// translation units.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "fi.h"
#include "fi_internal.h"

namespace fi {

fi_status set_error(fi_status st, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));
void clear_error();

struct Level {
  int32_t rows_per_block = 0;
  int32_t num_workers = 0;      // waves (decode-style) or workgroups (wide)
  int32_t min_chunk_pages = 0;
  int32_t chunk_pages = 0;
  std::vector<int32_t> items;          // ITEM_INTS per item, grouped by worker
  std::vector<int32_t> worker_indptr;  // num_workers + 1
  std::vector<int32_t> item_unit;      // per item (in items' order): its unit's index
  int32_t num_items() const { return (int32_t)(items.size() / ITEM_INTS); }
};

struct HostPlan {
  fi_plan_desc desc{};     // defaults filled in
  int32_t num_levels = 0;
  Level level[2];
  std::vector<int32_t> merges;   // MERGE_INTS per entry
  std::vector<int32_t> parts;
  std::vector<int32_t> qlist;
  std::vector<int32_t> scatter;  // 2 per new token (append)
  int32_t num_part_rows = 0;
  // fused mixed batch: level 0 (wide role) runs on workgroups
  // [0, pod_wide_blocks) of one launch, level 1 (decode role) on the rest
  bool pod = false;
  int32_t pod_wide_blocks = 0;
  std::vector<int32_t> plist;    // block-sparse: the units' page lists
  int32_t merge_rows = 0;        // the most rows of any merge record
  // fused merge (decode plans on the matrix cores): per level-0 item its
  // merge record (-1: final rows), and the records of units with no keys
  bool fused = false;
  std::vector<int32_t> item_rec, empty_recs;
  // fused tiny decode plan with every unit on the four waves of one
  // workgroup (workers 4u..4u+3): the fold follows a workgroup barrier
  bool wg_fold = false;
  // graph-stable plan (capacity given in the description): a fixed layout,
  // every launch made whatever the batch, sized by these capacities
  bool stable = false;
  int64_t cap_merges = 0, cap_scatter = 0;
  // entries of the device page tables the run calls read (kv_indptr[B] and,
  // for cascade, prefix_indptr[num_prefix_groups]; 0 for block-sparse plans)
  int64_t kv_entries = 0, prefix_entries = 0;
};

// Byte offsets of each section inside the workspace blob.
struct Layout {
  size_t items[2] = {0, 0}, windptr[2] = {0, 0};
  size_t merges = 0, parts = 0, qlist = 0, scatter = 0;
  size_t meta = 0;           // int32 [META_INTS]: counts the kernels read
  size_t plist = 0;          // block-sparse page lists
  size_t item_rec = 0, counters = 0, empty_recs = 0;   // fused merge
  size_t blob_bytes = 0;     // int32 sections (host staging size)
  size_t part_o = 0, part_lse = 0;
  size_t dev_bytes = 0;      // blob + fp32 partial states
};

Layout layout_for(const int32_t num_workers[2], const size_t n_items[2], size_t n_merges,
                  size_t n_parts, size_t n_qlist, size_t n_scatter, size_t n_part_rows,
                  int32_t head_dim, size_t n_plist = 0, bool fused = false);

// Debug check of device page tables (fi_check.hip): zeroes *count, then adds
// the number of ids outside [0, num_pages) in each non-NULL table.
hipError_t launch_check_page_ids(const int32_t* kv_ids, int64_t n_kv, const int32_t* prefix_ids,
                                 int64_t n_prefix, int32_t num_pages, int32_t* count,
                                 hipStream_t stream);

}  // namespace fi

struct fi_plan {
  fi::HostPlan hp;
  fi::Layout lay;
  bool on_device = false;
  char* dev_base = nullptr;   // caller's device workspace
  std::vector<char> host_blob;   // host-only plans: the int32 sections as laid out
};

namespace fi {

// Kernel arguments of level `level` of plan p, whose workspace sits at device
// address `base` (the caller's workspace, or the library's static scratch).
AttnArgs plan_attn_args(const fi_plan_t* p, const char* base, int level, const void* q,
                        const void* k, const void* v, const int32_t* kv_indices,
                        const int32_t* prefix_indices, float sm_scale, void* o, float* lse);
// The attention launch of a single-level plan (decode engines or wide kernel).
hipError_t plan_launch_level(const fi_plan_t* p, int level, const AttnArgs& a, hipStream_t s);
// The merge launch of plan p with its workspace at `base`.
hipError_t plan_launch_merge(const fi_plan_t* p, const char* base, void* o, float* lse,
                             hipStream_t s);

// Kernel timer hooks (no-ops unless fi_timer_begin enabled them).
struct TimerScope {
  hipStream_t s;
  hipEvent_t stop = nullptr;
  explicit TimerScope(hipStream_t st);
  ~TimerScope() { done(); }
  void done();
};

}  // namespace fi
