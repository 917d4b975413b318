// fi_api.cpp -- run entry points of the C ABI: argument checks, carving the
// plan's arrays out of the caller's workspace, kernel launches, and the
// optional kernel timer used by measurement tools.

#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "fi_host.h"

using namespace fi;

namespace {

// ---------------------------------------------------------------- timer

std::mutex g_timer_mu;
bool g_timer_on = false;
int32_t g_timer_used = 0;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_timer_events;

template <typename T>
T* at(const fi_plan_t* p, size_t off) {
  return (T*)(p->dev_base + off);
}

fi_status check_plan(const fi_plan_t* p, int32_t kind, const char* who) {
  if (!p) return set_error(FI_ERR_PLAN_MISMATCH, "%s: plan is NULL", who);
  if (p->hp.desc.kind != kind)
    return set_error(FI_ERR_PLAN_MISMATCH, "%s: plan was built for kind %d", who, p->hp.desc.kind);
  if (!p->on_device)
    return set_error(FI_ERR_PLAN_MISMATCH, "%s: host-only plan (built without a device workspace)",
                     who);
  return FI_OK;
}

fi_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FI_OK;
  return set_error(FI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

AttnArgs attn_args(const fi_plan_t* p, int level, const void* q, const void* k, const void* v,
                   const int32_t* kv_indices, const int32_t* prefix_indices, float sm_scale,
                   void* o, float* lse) {
  return plan_attn_args(p, p->dev_base, level, q, k, v, kv_indices, prefix_indices, sm_scale,
                        o, lse);
}

hipError_t launch_level(const fi_plan_t* p, int level, const AttnArgs& a, hipStream_t s) {
  return plan_launch_level(p, level, a, s);
}

}  // namespace

namespace fi {

LaunchTiming& launch_timing() {
  static thread_local LaunchTiming t;
  return t;
}

// The scope hands its event pair to the launches in it (launch_timed); if it
// launched nothing, the pair is recorded around nothing, so that every pair
// the timer hands out has been recorded.
TimerScope::TimerScope(hipStream_t st) : s(st) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  if (g_timer_on && g_timer_used < (int32_t)g_timer_events.size()) {
    auto& pr = g_timer_events[g_timer_used++];
    stop = pr.second;
    launch_timing() = LaunchTiming{pr.first, pr.second};
  }
}

void TimerScope::done() {
  if (!stop) return;
  LaunchTiming& t = launch_timing();
  if (t.start) {   // no kernel took the events
    (void)hipEventRecord(t.start, s);
    (void)hipEventRecord(stop, s);
  }
  t = LaunchTiming{};
  stop = nullptr;
}

AttnArgs plan_attn_args(const fi_plan_t* p, const char* base, int level, const void* q,
                        const void* k, const void* v, const int32_t* kv_indices,
                        const int32_t* prefix_indices, float sm_scale, void* o, float* lse) {
  const fi_plan_desc& d = p->hp.desc;
  auto at = [&](size_t off) { return (const int32_t*)(base + off); };
  AttnArgs a;
  a.items = at(p->lay.items[level]);
  a.worker_indptr = at(p->lay.windptr[level]);
  // a graph-stable plan launches every level whatever this batch holds, and
  // a fused-merge plan whenever it has records to write (units with no keys)
  const bool fused = p->hp.fused && level == 0;
  a.num_workers = (p->hp.stable || p->hp.level[level].num_items() > 0 ||
                   (fused && !p->hp.empty_recs.empty()))
                      ? p->hp.level[level].num_workers : 0;
  a.qlist = at(p->lay.qlist);
  a.q = (const uint16_t*)q;
  a.k_cache = (const uint16_t*)k;
  a.v_cache = (const uint16_t*)v;
  a.kv_indices = kv_indices;
  a.prefix_indices = prefix_indices;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.part_o = (float*)(base + p->lay.part_o);
  a.part_lse = (float*)(base + p->lay.part_lse);
  a.k_scale = nullptr;
  a.v_scale = nullptr;
  a.k_bscale = nullptr;
  a.v_bscale = nullptr;
  a.item_rec = fused ? at(p->lay.item_rec) : nullptr;
  a.counters = fused ? (int32_t*)(base + p->lay.counters) : nullptr;
  a.merges = at(p->lay.merges);
  a.parts = at(p->lay.parts);
  a.empty_recs = at(p->lay.empty_recs);
  a.meta = at(p->lay.meta);
  a.wg_fold = (fused && p->hp.wg_fold) ? 1 : 0;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.num_qo_heads = d.num_qo_heads;
  a.num_kv_heads = d.num_kv_heads;
  a.group = d.num_qo_heads / d.num_kv_heads;
  a.page_size = d.page_size;
  a.page_shift = __builtin_ctz((unsigned)d.page_size);
  return a;
}

hipError_t plan_launch_level(const fi_plan_t* p, int level, const AttnArgs& a, hipStream_t s) {
  const int D = p->hp.desc.head_dim;
  if (p->hp.level[level].rows_per_block == ROWS_WIDE)
    return launch_wide(a, D, p->hp.desc.kind == FI_KIND_CASCADE && level == 0,
                       p->hp.desc.kv_layout == FI_KV_LAYOUT_RAGGED, s);
  if (p->hp.desc.decode_engine == FI_ENGINE_VALU) return launch_decode_valu(a, D, s);
  return launch_decode(a, D, s);
}

hipError_t plan_launch_merge(const fi_plan_t* p, const char* base, void* o, float* lse,
                             hipStream_t s) {
  MergeArgs m;
  m.merges = (const int32_t*)(base + p->lay.merges);
  // launch sizing: the plan's records, or a graph-stable plan's capacity
  m.num_merges = p->hp.stable ? (int32_t)p->hp.cap_merges
                              : (int32_t)(p->hp.merges.size() / MERGE_INTS);
  m.parts = (const int32_t*)(base + p->lay.parts);
  m.part_o = (const float*)(base + p->lay.part_o);
  m.part_lse = (const float*)(base + p->lay.part_lse);
  m.o = (uint16_t*)o;
  m.lse = lse;
  m.num_qo_heads = p->hp.desc.num_qo_heads;
  m.head_dim = p->hp.desc.head_dim;
  m.group = p->hp.desc.num_qo_heads / p->hp.desc.num_kv_heads;
  m.rows_per_record = p->hp.stable ? MERGE_ROWS : p->hp.merge_rows;
  m.counts = (const int32_t*)(base + p->lay.meta);
  return launch_merge(m, s);
}

}  // namespace fi

namespace {

// A pod plan's two levels in one launch of a fixed shape: every worker slot of
// both roles, whatever this batch's split.
hipError_t launch_fused(const fi_plan_t* p, const void* q, const void* k, const void* v,
                        const int32_t* kv_indices, const int32_t* prefix_indices,
                        float sm_scale, void* o, float* lse, hipStream_t s) {
  AttnArgs wa = attn_args(p, 0, q, k, v, kv_indices, prefix_indices, sm_scale, o, lse);
  AttnArgs da = attn_args(p, 1, q, k, v, kv_indices, prefix_indices, sm_scale, o, lse);
  wa.num_workers = p->hp.level[0].num_workers;
  da.num_workers = p->hp.level[1].num_workers;
  return launch_pod(wa, da, at<int32_t>(p, p->lay.meta), p->hp.desc.head_dim,
                    p->hp.desc.kind == FI_KIND_CASCADE,
                    p->hp.desc.kv_layout == FI_KV_LAYOUT_RAGGED, s);
}

fi_status run_merge(const fi_plan_t* p, void* o, float* lse, hipStream_t s) {
  if (p->hp.fused) return FI_OK;   // the attention kernel folded its split units
  return hip_status(plan_launch_merge(p, p->dev_base, o, lse, s), "merge launch");
}

}  // namespace

extern "C" fi_status fi_paged_decode(const fi_plan_t* p, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* kv_indices,
                                     float sm_scale, void* o, float* lse, void* stream) {
  clear_error();
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return set_error(FI_ERR_INVALID_ARG, "fi_paged_decode: sm_scale must be finite and > 0, got %g", (double)sm_scale);
  fi_status st = check_plan(p, FI_KIND_DECODE, "fi_paged_decode");
  if (st != FI_OK) return st;
  if (p->hp.desc.batch > 0 && (!q || !k_cache || !v_cache || !kv_indices || !o))
    return set_error(FI_ERR_INVALID_ARG, "fi_paged_decode: NULL tensor pointer");
  hipStream_t s = (hipStream_t)stream;
  const AttnArgs a =
      attn_args(p, 0, q, k_cache, v_cache, kv_indices, nullptr, sm_scale, o, lse);
  TimerScope t(s);
  st = hip_status(launch_level(p, 0, a, s), "attention launch");
  t.done();
  if (st != FI_OK) return st;
  return run_merge(p, o, lse, s);
}

extern "C" fi_status fi_paged_decode_fp8(const fi_plan_t* p, const void* q, const void* k_cache,
                                         const void* v_cache, const float* k_scale,
                                         const float* v_scale, const int32_t* kv_indices,
                                         float sm_scale, void* o, float* lse, void* stream) {
  clear_error();
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return set_error(FI_ERR_INVALID_ARG, "fi_paged_decode_fp8: sm_scale must be finite and > 0, got %g",
                     (double)sm_scale);
  fi_status st = check_plan(p, FI_KIND_DECODE, "fi_paged_decode_fp8");
  if (st != FI_OK) return st;
  if (p->hp.desc.decode_engine != FI_ENGINE_MFMA)
    return set_error(FI_ERR_UNSUPPORTED, "fi_paged_decode_fp8 runs on the matrix-core engine");
  if (p->hp.desc.batch > 0 &&
      (!q || !k_cache || !v_cache || !k_scale || !v_scale || !kv_indices || !o))
    return set_error(FI_ERR_INVALID_ARG, "fi_paged_decode_fp8: NULL tensor pointer");
  hipStream_t s = (hipStream_t)stream;
  AttnArgs a = attn_args(p, 0, q, k_cache, v_cache, kv_indices, nullptr, sm_scale, o, lse);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  TimerScope t(s);
  st = hip_status(launch_decode_fp8(a, p->hp.desc.head_dim, s), "attention launch");
  t.done();
  if (st != FI_OK) return st;
  return run_merge(p, o, lse, s);
}

extern "C" fi_status fi_paged_decode_mxfp4(const fi_plan_t* p, const void* q, const void* k_codes,
                                           const void* v_codes, const void* k_scales,
                                           const void* v_scales, const int32_t* kv_indices,
                                           float sm_scale, void* o, float* lse, void* stream) {
  clear_error();
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return set_error(FI_ERR_INVALID_ARG,
                     "fi_paged_decode_mxfp4: sm_scale must be finite and > 0, got %g",
                     (double)sm_scale);
  fi_status st = check_plan(p, FI_KIND_DECODE, "fi_paged_decode_mxfp4");
  if (st != FI_OK) return st;
  if (p->hp.desc.decode_engine != FI_ENGINE_MFMA)
    return set_error(FI_ERR_UNSUPPORTED, "fi_paged_decode_mxfp4 runs on the matrix-core engine");
  if (p->hp.desc.batch > 0 &&
      (!q || !k_codes || !v_codes || !k_scales || !v_scales || !kv_indices || !o))
    return set_error(FI_ERR_INVALID_ARG, "fi_paged_decode_mxfp4: NULL tensor pointer");
  hipStream_t s = (hipStream_t)stream;
  AttnArgs a = attn_args(p, 0, q, k_codes, v_codes, kv_indices, nullptr, sm_scale, o, lse);
  a.k_bscale = (const uint8_t*)k_scales;
  a.v_bscale = (const uint8_t*)v_scales;
  TimerScope t(s);
  st = hip_status(launch_decode_mxfp4(a, p->hp.desc.head_dim, s), "attention launch");
  t.done();
  if (st != FI_OK) return st;
  return run_merge(p, o, lse, s);
}

extern "C" fi_status fi_check_page_tables(const fi_plan_t* p, const int32_t* kv_indices,
                                          const int32_t* prefix_indices, int32_t num_pages,
                                          int32_t* bad_count, void* stream) {
  clear_error();
  if (!p) return set_error(FI_ERR_PLAN_MISMATCH, "fi_check_page_tables: plan is NULL");
  if (!p->on_device)
    return set_error(FI_ERR_PLAN_MISMATCH,
                     "fi_check_page_tables: host-only plan (built without a device workspace)");
  if (p->hp.desc.kind == FI_KIND_BLOCK_SPARSE)
    return set_error(FI_ERR_INVALID_ARG,
                     "fi_check_page_tables: a block-sparse plan reads no caller page table");
  if (num_pages < 1)
    return set_error(FI_ERR_INVALID_ARG, "fi_check_page_tables: num_pages %d < 1", num_pages);
  if (!bad_count) return set_error(FI_ERR_INVALID_ARG, "fi_check_page_tables: bad_count is NULL");
  if (p->hp.kv_entries > 0 && !kv_indices)
    return set_error(FI_ERR_INVALID_ARG, "fi_check_page_tables: kv_indices is NULL");
  return hip_status(launch_check_page_ids(kv_indices, p->hp.kv_entries, prefix_indices,
                                          prefix_indices ? p->hp.prefix_entries : 0, num_pages,
                                          bad_count, (hipStream_t)stream),
                    "page table check launch");
}

extern "C" fi_status fi_paged_append(const fi_plan_t* p, const void* q, const void* k_new,
                                     const void* v_new, void* k_cache, void* v_cache,
                                     const int32_t* kv_indices, float sm_scale, void* o,
                                     float* lse, void* stream) {
  clear_error();
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return set_error(FI_ERR_INVALID_ARG, "fi_paged_append: sm_scale must be finite and > 0, got %g", (double)sm_scale);
  fi_status st = check_plan(p, FI_KIND_APPEND, "fi_paged_append");
  if (st != FI_OK) return st;
  if ((k_new == nullptr) != (v_new == nullptr))
    return set_error(FI_ERR_INVALID_ARG, "fi_paged_append: give both k_new and v_new or neither");
  if (p->hp.desc.batch > 0 && (!q || !k_cache || !v_cache || !kv_indices || !o))
    return set_error(FI_ERR_INVALID_ARG, "fi_paged_append: NULL tensor pointer");
  hipStream_t s = (hipStream_t)stream;
  const fi_plan_desc& d = p->hp.desc;
  if (k_new) {
    ScatterArgs sa;
    sa.scatter = at<int32_t>(p, p->lay.scatter);
    sa.num_tokens = p->hp.stable ? (int32_t)p->hp.cap_scatter
                                 : (int32_t)(p->hp.scatter.size() / 2);
    sa.counts = at<int32_t>(p, p->lay.meta);
    sa.kv_indices = kv_indices;
    sa.k_new = (const uint16_t*)k_new;
    sa.v_new = (const uint16_t*)v_new;
    sa.k_cache = (uint16_t*)k_cache;
    sa.v_cache = (uint16_t*)v_cache;
    sa.num_kv_heads = d.num_kv_heads;
    sa.page_size = d.page_size;
    sa.head_dim = d.head_dim;
    st = hip_status(launch_scatter(sa, s), "scatter launch");
    if (st != FI_OK) return st;
  }
  TimerScope t(s);
  if (p->hp.pod) {
    st = hip_status(launch_fused(p, q, k_cache, v_cache, kv_indices, nullptr, sm_scale, o, lse, s),
                    "attention launch");
  } else {
    const AttnArgs a =
        attn_args(p, 0, q, k_cache, v_cache, kv_indices, nullptr, sm_scale, o, lse);
    st = hip_status(launch_level(p, 0, a, s), "attention launch");
  }
  t.done();
  if (st != FI_OK) return st;
  return run_merge(p, o, lse, s);
}

extern "C" fi_status fi_block_sparse_attention(const fi_plan_t* p, const void* q,
                                               const void* k_cache, const void* v_cache,
                                               float sm_scale, void* o, float* lse,
                                               void* stream) {
  clear_error();
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return set_error(FI_ERR_INVALID_ARG,
                     "fi_block_sparse_attention: sm_scale must be finite and > 0, got %g",
                     (double)sm_scale);
  fi_status st = check_plan(p, FI_KIND_BLOCK_SPARSE, "fi_block_sparse_attention");
  if (st != FI_OK) return st;
  if (!p->hp.merges.empty() || p->hp.level[0].num_items() > 0 || p->hp.level[1].num_items() > 0)
    if (!q || !k_cache || !v_cache || !o)
      return set_error(FI_ERR_INVALID_ARG, "fi_block_sparse_attention: NULL tensor pointer");
  hipStream_t s = (hipStream_t)stream;
  const int32_t* plist = at<int32_t>(p, p->lay.plist);   // the plan's own page lists
  TimerScope t(s);
  if (p->hp.pod) {
    st = hip_status(launch_fused(p, q, k_cache, v_cache, plist, nullptr, sm_scale, o, lse, s),
                    "attention launch");
  } else {
    const AttnArgs a = attn_args(p, 0, q, k_cache, v_cache, plist, nullptr, sm_scale, o, lse);
    st = hip_status(launch_level(p, 0, a, s), "attention launch");
  }
  t.done();
  if (st != FI_OK) return st;
  return run_merge(p, o, lse, s);
}

extern "C" fi_status fi_cascade(const fi_plan_t* p, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* prefix_indices,
                                const int32_t* kv_indices, float sm_scale, void* o, float* lse,
                                void* stream) {
  clear_error();
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return set_error(FI_ERR_INVALID_ARG, "fi_cascade: sm_scale must be finite and > 0, got %g", (double)sm_scale);
  fi_status st = check_plan(p, FI_KIND_CASCADE, "fi_cascade");
  if (st != FI_OK) return st;
  if (p->hp.desc.batch > 0 && (!q || !k_cache || !v_cache || !kv_indices || !o))
    return set_error(FI_ERR_INVALID_ARG, "fi_cascade: NULL tensor pointer");
  if (p->hp.level[0].num_items() > 0 && !prefix_indices)
    return set_error(FI_ERR_INVALID_ARG, "fi_cascade: NULL prefix_indices");
  hipStream_t s = (hipStream_t)stream;
  TimerScope t(s);
  if (p->hp.pod) {
    st = hip_status(launch_fused(p, q, k_cache, v_cache, kv_indices, prefix_indices, sm_scale,
                                 o, lse, s),
                    "attention launch");
    if (st != FI_OK) return st;
  }
  for (int l = 0; l < 2 && !p->hp.pod; ++l) {
    const AttnArgs a =
        attn_args(p, l, q, k_cache, v_cache, kv_indices, prefix_indices, sm_scale, o, lse);
    st = hip_status(launch_level(p, l, a, s), "attention launch");
    if (st != FI_OK) return st;
  }
  t.done();
  return run_merge(p, o, lse, s);
}

extern "C" fi_status fi_merge_states(const void* v, int32_t v_dtype, const float* s, int32_t N,
                                     int32_t S, int32_t H, int32_t D, void* v_out,
                                     int32_t out_dtype, float* s_out, void* stream) {
  clear_error();
  if (N < 0 || S < 0 || H < 0) return set_error(FI_ERR_INVALID_ARG, "negative size");
  if (D < 4 || D > 1024 || D % 4)
    return set_error(FI_ERR_UNSUPPORTED, "D = %d (need a multiple of 4 in [4, 1024])", D);
  if ((v_dtype != FI_DTYPE_BF16 && v_dtype != FI_DTYPE_F32) ||
      (out_dtype != FI_DTYPE_BF16 && out_dtype != FI_DTYPE_F32))
    return set_error(FI_ERR_INVALID_ARG, "unknown dtype");
  if ((int64_t)N * H == 0) return FI_OK;
  if (!v_out || (S > 0 && (!v || !s)))
    return set_error(FI_ERR_INVALID_ARG, "fi_merge_states: NULL tensor pointer");
  MergeStatesArgs a;
  a.v = v;
  a.v_f32 = v_dtype == FI_DTYPE_F32;
  a.s = s;
  a.N = N;
  a.S = S;
  a.H = H;
  a.D = D;
  a.v_out = v_out;
  a.out_f32 = out_dtype == FI_DTYPE_F32;
  a.s_out = s_out;
  return hip_status(launch_merge_states(a, (hipStream_t)stream), "merge_states launch");
}

extern "C" fi_status fi_timer_begin(int32_t capacity) {
  clear_error();
  if (capacity < 1) return set_error(FI_ERR_INVALID_ARG, "capacity %d < 1", capacity);
  std::lock_guard<std::mutex> lk(g_timer_mu);
  while ((int32_t)g_timer_events.size() < capacity) {
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    if (e != hipSuccess) return hip_status(e, "event create");
    g_timer_events.emplace_back(a, b);
  }
  g_timer_used = 0;
  g_timer_on = true;
  return FI_OK;
}

extern "C" fi_status fi_timer_end(double* total_ms, int32_t* calls) {
  clear_error();
  if (!total_ms || !calls) return set_error(FI_ERR_INVALID_ARG, "NULL output");
  std::lock_guard<std::mutex> lk(g_timer_mu);
  double sum = 0.0;
  for (int32_t i = 0; i < g_timer_used; ++i) {
    hipError_t e = hipEventSynchronize(g_timer_events[i].second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_timer_events[i].first, g_timer_events[i].second);
    if (e != hipSuccess) {
      g_timer_on = false;
      return hip_status(e, "event timing");
    }
    sum += ms;
  }
  *total_ms = sum;
  *calls = g_timer_used;
  g_timer_on = false;
  g_timer_used = 0;
  return FI_OK;
}
