// fi_plan.cpp -- the host-side work plan: validation, load-balanced chunking,
// longest-first placement on persistent workers, merge lists, and the upload
// of the plan into the caller's device workspace.
//
// The pages state the goal (Ye et al. record, "summary": KV ranges split into
// load-balanced chunks, scheduled so that a statically captured graph stays
// valid; PR #4038, "What it does": fp32 partials reduced in a fixed order) but
// give no algorithm. The rule implemented here:
//   units   : (request, row block, kv head); cascade prefix: (group, row block,
//             kv head) over the member requests' rows, a group's members being
//             the requests whose chain of groups (own, parent, ...) passes
//             through it; groups in index order, so a request's prefix parts
//             come root first
//   key range of a unit: [0, t_lim), t_lim = kv_len, or min(kv_len,
//             kv_len - qo + i_last + 1) under the bottom-right causal mask
//   balanced: the level's units, counted in 32-token steps of gp =
//             max(1, 32 / page_size) pages, laid end to end (W steps), are cut
//             into quotas of c = max(1, ceil(min_chunk_pages / gp), ceil(W / S))
//             steps, S = num_cus * workers_per_cu; quota w is worker w's, so
//             every worker runs the same number of steps (even split)
//             small batches: with no more units than workers and the longest
//             unit under kNoSplitSteps steps longer than c, every unit stays
//             whole on worker = its index (a split would save fewer steps
//             than its merge launch costs)
//   deterministic: c = det_chunk_pages; a unit of n pages has k = ceil(n/c)
//             chunks on a wide level, k = min(ceil(n/(c/2)), kDetMaxChunks)
//             on a decode-style one, chunk j [floor(jn/k), floor((j+1)n/k)),
//             boundaries depending on the request alone, placed by Graham's
//             longest-processing-time
//             rule (cost = pages + 1, ties to the lower enumeration index and
//             the lower worker index)
//   outputs : one chunk -> final rows, else fp32 partial rows + merge
//             (cascade: all partial, merged prefix first)
// The grid is always S workers, whatever the batch, so a captured graph is
// re-pointed at a new batch by re-planning into the same workspace.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <map>
#include <mutex>
#include <numeric>
#include <queue>
#include <utility>

#include "fi_host.h"

namespace fi {

// ---------------------------------------------------------------- errors

static thread_local std::string g_last_error;

fi_status set_error(fi_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

// ---------------------------------------------------------------- layout

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Layout layout_for(const int32_t num_workers[2], const size_t n_items[2], size_t n_merges,
                  size_t n_parts, size_t n_qlist, size_t n_scatter, size_t n_part_rows,
                  int32_t head_dim, size_t n_plist, bool fused) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t n_int32) {
    size_t at = off;
    off = align_up(off + n_int32 * 4, 256);
    return at;
  };
  for (int l = 0; l < 2; ++l) {
    L.items[l] = take(n_items[l] * ITEM_INTS);
    L.windptr[l] = take((size_t)num_workers[l] + 1);
  }
  L.merges = take(n_merges * MERGE_INTS);
  L.parts = take(n_parts);
  L.qlist = take(n_qlist);
  L.scatter = take(n_scatter * 2);
  L.meta = take(META_INTS);
  L.plist = take(n_plist);
  // fused merge: per level-0 item its record, a count per record, and the
  // list of records of units with no keys (at most one per record)
  L.item_rec = take(fused ? n_items[0] : 0);
  L.counters = take(fused ? n_merges : 0);
  L.empty_recs = take(fused ? n_merges : 0);
  L.blob_bytes = off;
  L.part_o = off;
  off = align_up(off + n_part_rows * (size_t)head_dim * 4, 256);
  L.part_lse = off;
  off = align_up(off + n_part_rows * 4, 256);
  L.dev_bytes = off;
  return L;
}

// ---------------------------------------------------------------- planning

namespace {

struct Unit {
  int32_t unit, q_base, row0, n_rows, g, page_off, t_lim, n_pages, q_pos0, flags;
};

struct ItemRec {
  int32_t f[ITEM_INTS];
  int32_t pages;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Units of a level whose rows are request query tokens (decode, append,
// cascade suffix). Enumeration order: request, row block, kv head.
// take: if given, only the requests r with take[r] != 0.
void request_units(std::vector<Unit>& out, int32_t B, int32_t G, int32_t Hkv, int32_t ps,
                   int32_t rpb, const int32_t* kv_indptr, const int32_t* kv_len,
                   const int32_t* qo_indptr, bool causal, const uint8_t* take = nullptr) {
  for (int32_t r = 0; r < B; ++r) {
    if (take && !take[r]) continue;
    const int32_t nq = qo_indptr ? qo_indptr[r + 1] - qo_indptr[r] : 1;
    const int32_t qtok = qo_indptr ? qo_indptr[r] : r;
    const int32_t L = kv_len[r];
    const int64_t rows = (int64_t)nq * G;
    const int64_t nblk = ceil_div(rows, rpb);
    for (int64_t b = 0; b < nblk; ++b) {
      const int32_t r0 = (int32_t)(b * rpb);
      const int32_t r1 = (int32_t)std::min<int64_t>(rows, (b + 1) * rpb);
      const int32_t i_last = (r1 - 1) / G;
      const int32_t t_lim = causal ? std::min(L, L - nq + i_last + 1) : L;
      for (int32_t g = 0; g < Hkv; ++g) {
        Unit u;
        u.unit = r;
        u.q_base = qtok;
        u.row0 = r0;
        u.n_rows = r1 - r0;
        u.g = g;
        u.page_off = kv_indptr[r];
        u.t_lim = t_lim;
        u.n_pages = (int32_t)ceil_div(t_lim, ps);
        u.q_pos0 = causal ? L - nq : 0;
        u.flags = causal ? FLAG_CAUSAL : 0;
        out.push_back(u);
      }
    }
  }
}

struct LevelBuild {
  std::vector<ItemRec> items;                // enumeration order
  std::vector<std::pair<int32_t, std::vector<int32_t>>> chunks;  // per unit: k, partial dsts
};

// Balanced mode keeps every unit whole when a split would save fewer steps.
constexpr int64_t kNoSplitSteps = 12;
// Deterministic chunking depends on a unit alone (so a row's bits do not
// depend on its batch). A wide level (128-row units, an item costing about
// four steps to start and end) cuts a unit of n pages into ceil(n / c)
// chunks, c = det_chunk_pages; a decode-style level (16-row units, items
// nearly free) of a bf16 cache into min(ceil(n / (c / 2)), kDetMaxChunks):
// half-size chunks place evenly on the workers, and the cap keeps very long
// requests from merging scores of parts.
constexpr int64_t kDetMaxChunks = 16;
int64_t det_chunks(int64_t n, int64_t c, bool decode_style) {
  if (n <= 0) return 0;
  c = std::max<int64_t>(1, c);
  if (!decode_style) return ceil_div(n, c);
  return std::min<int64_t>(ceil_div(n, std::max<int64_t>(1, c / 2)), kDetMaxChunks);
}
// Fused launch: relative time of a wide-role workgroup step (up to 128 rows
// through MFMA) and of a decode-role wavefront step, with the two roles
// sharing the chip and the KV coming from HBM (a decode workgroup runs four
// wavefronts side by side), and the start and end of a wide item in wide
// steps (the query load, the pipeline fill, the output rows and the closing
// barrier of an item took about four to five steps' time in the fused
// launch, timed inside the kernel on the shared-prefix cascade batch).
constexpr int64_t kPodWideStep = 4;
constexpr int64_t kPodDecodeStep = 9;
constexpr int64_t kPodWideItemSteps = 4;

// tiny: a decode level with fewer steps than workers whose split units are
// folded in the kernel (no merge launch to amortise): chunks of
// max(1, ceil(W / S)) steps and no whole-unit exception, so a short unit's
// steps run on several idle waves side by side. wg (tiny, with at most S/4
// units): unit u runs on the four waves of workgroup u (workers 4u..4u+3),
// chunk c being its steps [c k, (c+1) k), k = ceil(steps / 4), so that the
// chunks are folded after a workgroup barrier.
void build_level(const std::vector<Unit>& units, const fi_plan_desc& d, bool all_partial,
                 int32_t& next_row, LevelBuild& lb, Level& lv, bool tiny = false,
                 bool wg = false) {
  const int32_t ps = d.page_size;
  const int32_t S = lv.num_workers;
  // Per unit: its pieces (page range and, in balanced mode, the worker).
  struct Piece { int64_t p0, p1; int32_t worker; };
  std::vector<std::vector<Piece>> pieces(units.size());
  int64_t c;
  if (d.deterministic) {
    // (the FP8 and MXFP4 decode kernels, with more workers per CU and a
    // costlier item start, keep whole-size chunks)
    const bool decode_style = lv.rows_per_block == ROWS_DECODE && d.kv_format == FI_KV_BF16;
    c = std::max(1, d.det_chunk_pages);
    if (decode_style) c = std::max<int64_t>(1, c / 2);
    for (size_t ui = 0; ui < units.size(); ++ui) {
      const int64_t n = units[ui].n_pages;
      const int64_t k = det_chunks(n, d.det_chunk_pages, decode_style);
      for (int64_t j = 0; j < k; ++j) pieces[ui].push_back({(j * n) / k, ((j + 1) * n) / k, -1});
    }
  } else {
    // Quotas are counted in 32-token steps of gp pages, the granule the
    // kernels walk a unit in, so that no chunk boundary falls inside a step.
    const int64_t gp = std::max(1, 32 / ps);
    int64_t W = 0;
    for (const Unit& u : units) W += ceil_div(u.n_pages, gp);
    const int64_t cs = tiny ? std::max<int64_t>(1, ceil_div(W, S))
                            : std::max<int64_t>({1, ceil_div(lv.min_chunk_pages, gp), ceil_div(W, S)});
    c = cs * gp;
    int64_t longest = 0;
    for (const Unit& u : units) longest = std::max<int64_t>(longest, ceil_div(u.n_pages, gp));
    const bool whole = !tiny && (int64_t)units.size() <= S && longest - cs < kNoSplitSteps;
    if (whole) c = std::max<int64_t>(1, longest) * gp;
    if (wg) c = std::max<int64_t>(1, ceil_div(longest, 4)) * gp;
    for (size_t ui = 0; wg && ui < units.size(); ++ui) {
      const int64_t n = units[ui].n_pages, ns = ceil_div(n, gp), k = ceil_div(ns, 4);
      for (int64_t j = 0; j < 4; ++j) {
        const int64_t s0 = j * k, s1 = std::min(ns, (j + 1) * k);
        if (s0 < s1) pieces[ui].push_back({s0 * gp, std::min(n, s1 * gp), (int32_t)(4 * ui + j)});
      }
    }
    int64_t g = 0;   // global step offset of the unit
    for (size_t ui = 0; whole && ui < units.size(); ++ui)
      if (units[ui].n_pages > 0) pieces[ui].push_back({0, units[ui].n_pages, (int32_t)ui});
    for (size_t ui = 0; !whole && !wg && ui < units.size(); ++ui) {
      const int64_t n = units[ui].n_pages, ns = ceil_div(n, gp);
      for (int64_t p = 0; p < ns;) {
        const int64_t w = (g + p) / cs;
        const int64_t e = std::min(ns, (w + 1) * cs - g);
        pieces[ui].push_back({p * gp, std::min(n, e * gp), (int32_t)w});
        p = e;
      }
      g += ns;
    }
  }
  lv.chunk_pages = (int32_t)c;
  lb.items.clear();
  lb.chunks.clear();
  std::vector<int32_t> item_worker, item_unit;
  for (size_t ui = 0; ui < units.size(); ++ui) {
    const Unit& u = units[ui];
    const int32_t k = (int32_t)pieces[ui].size();
    const bool partial = all_partial || k > 1;
    std::vector<int32_t> dsts;
    for (int32_t j = 0; j < k; ++j) {
      const Piece& pc = pieces[ui][j];
      int32_t dst = -1;
      if (partial) {
        dst = next_row;
        next_row += u.n_rows;
        dsts.push_back(dst);
      }
      ItemRec it;
      it.f[F_Q_BASE] = u.q_base;
      it.f[F_ROW0] = u.row0;
      it.f[F_NROWS] = u.n_rows;
      it.f[F_KVHEAD] = u.g;
      it.f[F_PAGEOFF] = u.page_off;
      it.f[F_FLAGS] = u.flags | (partial ? FLAG_PARTIAL : 0);
      it.f[F_TBEGIN] = (int32_t)(pc.p0 * ps);
      it.f[F_TEND] = (int32_t)std::min<int64_t>(pc.p1 * ps, u.t_lim);
      it.f[F_QPOS0] = u.q_pos0;
      it.f[F_DST] = dst;
      it.f[F_UNIT] = u.unit;
      it.f[F_CHUNK] = j;
      it.pages = (int32_t)(pc.p1 - pc.p0);
      lb.items.push_back(it);
      item_worker.push_back(pc.worker);
      item_unit.push_back((int32_t)ui);
    }
    lb.chunks.emplace_back(k, std::move(dsts));
  }
  const size_t n = lb.items.size();
  std::vector<std::vector<int32_t>> per(S);
  if (d.deterministic) {
    // Longest processing time first: stable sort keeps enumeration order on ties.
    std::vector<int32_t> order(n);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      return lb.items[a].pages > lb.items[b].pages;
    });
    typedef std::pair<int64_t, int32_t> LoadW;
    std::priority_queue<LoadW, std::vector<LoadW>, std::greater<LoadW>> heap;
    for (int32_t w = 0; w < S; ++w) heap.push(LoadW(0, w));
    for (int32_t i : order) {
      LoadW top = heap.top();
      heap.pop();
      per[top.second].push_back(i);
      heap.push(LoadW(top.first + lb.items[i].pages + 1, top.second));
    }
  } else {
    for (size_t i = 0; i < n; ++i) per[item_worker[i]].push_back((int32_t)i);
  }
  lv.items.clear();
  lv.items.reserve(n * ITEM_INTS);
  lv.item_unit.clear();
  lv.item_unit.reserve(n);
  lv.worker_indptr.assign(1, 0);
  for (int32_t w = 0; w < S; ++w) {
    for (int32_t i : per[w]) {
      lv.items.insert(lv.items.end(), lb.items[i].f, lb.items[i].f + ITEM_INTS);
      lv.item_unit.push_back(item_unit[i]);
    }
    lv.worker_indptr.push_back((int32_t)(lv.items.size() / ITEM_INTS));
  }
}

// Fused launch (pod plans): the launch's P workgroups are split between the
// wide role (level 0, one workgroup per worker) and the decode role (level 1,
// four wavefront workers per workgroup) by estimated cost; each level is
// planned over its share, then its worker list is padded with empty workers
// to the whole launch (P and 4P), so the launch shape does not depend on the
// batch.
fi_status pod_levels(const fi_plan_desc& d, const std::vector<Unit> (&units)[2],
                     bool all_partial, int32_t& next_row, LevelBuild (&lb)[2], HostPlan& hp) {
  const int32_t P = d.num_cus * std::max(1, d.workers_per_cu / 2);
  const int64_t gp = std::max(1, 32 / d.page_size);
  int64_t steps[2] = {0, 0};
  for (int l = 0; l < 2; ++l)
    for (const Unit& u : units[l]) steps[l] += ceil_div(u.n_pages, gp);
  if (P < 2 && steps[0] > 0 && steps[1] > 0)
    return set_error(FI_ERR_INVALID_ARG, "a fused launch needs at least 2 workgroups");
  int32_t nw;
  if (steps[1] == 0) {
    nw = P;
  } else if (steps[0] == 0) {
    nw = 0;
  } else if (d.pod_wide_blocks > 0) {
    nw = std::min(d.pod_wide_blocks, P - 1);
  } else {
    // The split whose slower role finishes first. A role's time is its step
    // cost times its quota c of steps (as build_level cuts it), plus for the
    // wide role kPodWideItemSteps per item of its busiest quota (a unit
    // boundary inside a quota adds an item). Ties go to the faster wide
    // role, then to fewer wide workgroups.
    const int64_t cmin[2] = {std::max<int64_t>(1, ceil_div(hp.level[0].min_chunk_pages, gp)),
                             std::max<int64_t>(1, ceil_div(hp.level[1].min_chunk_pages, gp))};
    std::vector<int64_t> bounds;   // wide unit ends on the steps laid end to end
    for (const Unit& u : units[0]) {
      const int64_t ns = ceil_div(u.n_pages, gp);
      if (ns > 0) bounds.push_back((bounds.empty() ? 0 : bounds.back()) + ns);
    }
    std::map<int64_t, int64_t> items_at;   // quota c -> items of the busiest quota
    auto max_items = [&](int64_t c) {
      auto f = items_at.find(c);
      if (f != items_at.end()) return f->second;
      int64_t best = 1, run = 1, q = -1;
      for (size_t i = 0; i + 1 < bounds.size(); ++i) {
        if (bounds[i] % c == 0) continue;
        const int64_t qi = bounds[i] / c;
        run = (qi == q) ? run + 1 : 2;
        q = qi;
        best = std::max(best, run);
      }
      items_at[c] = best;
      return best;
    };
    // Deterministic plans cut each unit into chunks of at most c_det pages
    // and place them longest first: a role's time is then its chunks per
    // worker (rounded up) times its longest chunk, or its steps per worker
    // if larger, the wide role paying kPodWideItemSteps per chunk.
    int64_t nch[2] = {0, 0}, longest[2] = {0, 0};
    if (d.deterministic) {
      for (int l = 0; l < 2; ++l)
        for (const Unit& u : units[l]) {
          if (u.n_pages <= 0) continue;
          const int64_t k = det_chunks(u.n_pages, d.det_chunk_pages, l == 1);
          nch[l] += k;
          longest[l] = std::max(longest[l], ceil_div(ceil_div(u.n_pages, k), gp));
        }
    }
    int64_t best_t = -1, best_w = 0;
    nw = 1;
    for (int32_t n = 1; n < P; ++n) {
      const int64_t waves = (int64_t)WAVES_PER_BLOCK * (P - n);
      int64_t tw, td;
      if (d.deterministic) {
        tw = kPodWideStep * ceil_div(nch[0], n) * (longest[0] + kPodWideItemSteps);
        td = kPodDecodeStep * std::max(longest[1], ceil_div(steps[1], waves));
      } else {
        const int64_t cw = std::max(cmin[0], ceil_div(steps[0], n));
        tw = kPodWideStep * (cw + kPodWideItemSteps * max_items(cw));
        td = kPodDecodeStep * std::max(cmin[1], ceil_div(steps[1], waves));
      }
      const int64_t t = std::max(tw, td);
      if (best_t < 0 || t < best_t || (t == best_t && tw < best_w)) {
        best_t = t;
        best_w = tw;
        nw = n;
      }
    }
  }
  hp.pod = true;
  hp.pod_wide_blocks = nw;
  hp.level[0].num_workers = nw;
  hp.level[1].num_workers = WAVES_PER_BLOCK * (P - nw);
  for (int l = 0; l < 2; ++l) {
    if (hp.level[l].num_workers > 0) {
      build_level(units[l], d, all_partial, next_row, lb[l], hp.level[l]);
    } else {   // a role with no workgroups has no steps: every unit is empty
      lb[l].items.clear();
      lb[l].chunks.assign(units[l].size(), {0, {}});
      hp.level[l].items.clear();
      hp.level[l].item_unit.clear();
      hp.level[l].chunk_pages = 0;
      hp.level[l].worker_indptr.assign(1, 0);
    }
  }
  hp.level[0].worker_indptr.resize((size_t)P + 1, hp.level[0].worker_indptr.back());
  hp.level[1].worker_indptr.resize((size_t)WAVES_PER_BLOCK * P + 1,
                                   hp.level[1].worker_indptr.back());
  hp.level[0].num_workers = P;
  hp.level[1].num_workers = WAVES_PER_BLOCK * P;
  return FI_OK;
}

// Merge records of a level whose units write final rows unless split: the
// rows of a unit of k != 1 chunks are cut into records of MERGE_ROWS rows,
// each over its chunks' partial rows in chunk order (k = 0, no keys: empty
// records, which write o = 0 and lse = -inf).
std::vector<int32_t> unit_merges(const std::vector<Unit>& units, const LevelBuild& lb,
                                 HostPlan& hp) {
  std::vector<int32_t> first_rec(units.size(), -1);   // per unit: its first record
  for (size_t ui = 0; ui < units.size(); ++ui) {
    const Unit& u = units[ui];
    const int32_t k = lb.chunks[ui].first;
    if (k == 1) continue;
    first_rec[ui] = (int32_t)(hp.merges.size() / MERGE_INTS);
    const std::vector<int32_t>& dsts = lb.chunks[ui].second;
    for (int32_t k0 = 0; k0 < u.n_rows; k0 += MERGE_ROWS) {
      const int32_t rec[MERGE_INTS] = {u.q_base, u.row0 + k0, std::min(MERGE_ROWS, u.n_rows - k0),
                                       u.g, (int32_t)hp.parts.size(), (int32_t)dsts.size()};
      hp.merges.insert(hp.merges.end(), rec, rec + MERGE_INTS);
      for (int32_t dd : dsts) hp.parts.push_back(dd + k0);
    }
  }
  return first_rec;
}

}  // namespace

// Engine for decode-style levels when the caller leaves the choice open: the
// one that measured faster for decode on MI355X.
static constexpr int32_t kDefaultEngine = FI_ENGINE_MFMA;

static fi_status fill_defaults(const fi_plan_desc* din, fi_plan_desc& d) {
  if (!din) return set_error(FI_ERR_INVALID_ARG, "desc is NULL");
  d = *din;
  if (d.kind < FI_KIND_DECODE || d.kind > FI_KIND_BLOCK_SPARSE)
    return set_error(FI_ERR_INVALID_ARG, "unknown plan kind %d", d.kind);
  if (d.kind == FI_KIND_BLOCK_SPARSE) {
    if (d.causal) return set_error(FI_ERR_INVALID_ARG, "a block-sparse plan takes no causal mask");
    d.batch = 1;
  }
  if (d.kv_layout != FI_KV_LAYOUT_PAGED && d.kv_layout != FI_KV_LAYOUT_RAGGED)
    return set_error(FI_ERR_INVALID_ARG, "kv_layout %d", d.kv_layout);
  if (d.kv_layout == FI_KV_LAYOUT_RAGGED && d.kind != FI_KIND_BLOCK_SPARSE)
    return set_error(FI_ERR_UNSUPPORTED, "a ragged KV layout is read by block-sparse plans only");
  if (d.batch < 0) return set_error(FI_ERR_INVALID_ARG, "batch %d < 0", d.batch);
  if (d.num_qo_heads < 1 || d.num_kv_heads < 1)
    return set_error(FI_ERR_INVALID_ARG, "head counts must be >= 1");
  if (d.num_qo_heads % d.num_kv_heads)
    return set_error(FI_ERR_INVALID_ARG, "num_qo_heads %d not a multiple of num_kv_heads %d",
                     d.num_qo_heads, d.num_kv_heads);
  if (d.head_dim != 64 && d.head_dim != 128)
    return set_error(FI_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", d.head_dim);
  if (d.page_size < 8 || d.page_size > 256 || (d.page_size & (d.page_size - 1)))
    return set_error(FI_ERR_UNSUPPORTED, "page_size %d (supported: powers of two 8..256)",
                     d.page_size);
  const int32_t G = d.num_qo_heads / d.num_kv_heads;
  if (d.kind == FI_KIND_CASCADE && (G > ROWS_DECODE || ROWS_WIDE % G))
    return set_error(FI_ERR_UNSUPPORTED, "cascade needs a head group size dividing 16, got %d",
                     G);
  if (d.det_chunk_pages < 0 || d.min_chunk_pages < 0 || d.workers_per_cu < 0 ||
      d.num_cus < 0 || d.num_prefix_groups < 0)
    return set_error(FI_ERR_INVALID_ARG, "negative tuning field in desc");
  if (d.decode_engine < FI_ENGINE_DEFAULT || d.decode_engine > FI_ENGINE_VALU)
    return set_error(FI_ERR_INVALID_ARG, "decode_engine %d", d.decode_engine);
  if (d.decode_engine == FI_ENGINE_DEFAULT) d.decode_engine = kDefaultEngine;
  if (d.decode_engine == FI_ENGINE_VALU && G > 8)
    return set_error(FI_ERR_UNSUPPORTED, "the VALU decode engine takes head groups <= 8, got %d",
                     G);
  if (d.max_prefix_depth < 0) return set_error(FI_ERR_INVALID_ARG, "negative max_prefix_depth");
  if (d.max_prefix_depth == 0) d.max_prefix_depth = 1;
  if (d.pod_wide_blocks < 0) return set_error(FI_ERR_INVALID_ARG, "negative pod_wide_blocks");
  if (d.cap_batch < 0 || d.cap_kv_pages < 0 || d.cap_qo_tokens < 0 || d.cap_prefix_pages < 0)
    return set_error(FI_ERR_INVALID_ARG, "negative capacity");
  if (d.kind == FI_KIND_BLOCK_SPARSE) d.cap_batch = 0;
  if (d.launch < FI_LAUNCH_DEFAULT || d.launch > FI_LAUNCH_SEPARATE)
    return set_error(FI_ERR_INVALID_ARG, "launch %d", d.launch);
  if (d.kind == FI_KIND_DECODE) {
    d.launch = FI_LAUNCH_SEPARATE;
  } else if (d.decode_engine == FI_ENGINE_VALU) {
    if (d.launch == FI_LAUNCH_POD)
      return set_error(FI_ERR_UNSUPPORTED, "a POD launch runs its decode role on the matrix cores");
    d.launch = FI_LAUNCH_SEPARATE;
  } else if (d.launch == FI_LAUNCH_DEFAULT) {
    d.launch = FI_LAUNCH_POD;   // measured faster on the cascade and mixed batches
  }
  if (d.launch != FI_LAUNCH_POD) d.pod_wide_blocks = 0;
  if (d.det_chunk_pages == 0) d.det_chunk_pages = 48;   // fastest of 8..64 on the five batches
  if (d.min_chunk_pages == 0) d.min_chunk_pages = 8;
  if (d.kv_format < FI_KV_BF16 || d.kv_format > FI_KV_MXFP4)
    return set_error(FI_ERR_INVALID_ARG, "kv_format %d", d.kv_format);
  if (d.merge_mode < FI_MERGE_DEFAULT || d.merge_mode > FI_MERGE_SEPARATE)
    return set_error(FI_ERR_INVALID_ARG, "merge_mode %d", d.merge_mode);
  if (d.kind != FI_KIND_DECODE) d.kv_format = FI_KV_BF16;
  // one wave per SIMD for the register-ring decode kernel; two and three
  // for the FP8 and MXFP4 kernels, which staging through LDS leaves ALU- and
  // latency-bound
  if (d.workers_per_cu == 0)
    d.workers_per_cu = d.kv_format == FI_KV_MXFP4 ? 12 : d.kv_format == FI_KV_FP8 ? 8 : 4;
  d.causal = d.causal ? 1 : 0;
  d.deterministic = d.deterministic ? 1 : 0;
  if (d.kind != FI_KIND_APPEND) d.causal = 0;   // (block-sparse: refused above if set)
  if (d.kind != FI_KIND_CASCADE) d.num_prefix_groups = 0;
  return FI_OK;
}

// FI_MERGE_FUSED decode plans on the matrix cores fold their split units at
// the end of the attention kernel (its decode kernels count chunks in and the
// last folds); so do default-mode ones with fewer 32-token steps than
// workers (tiny batches: few partial rows, and the plan then spreads each
// unit's steps over idle waves), except graph-stable plans, whose layout is
// fixed by the description. Every other plan launches the merge kernel after
// the attention kernel: on MI355X the fused fold's agent-scope partial stores,
// which write through the XCD's L2, cost more than the merge launch on full
// batches (Llama-like batch: 98 against 90 us per call).
static bool fused_merge(const fi_plan_desc& d) {
  return d.kind == FI_KIND_DECODE && d.decode_engine == FI_ENGINE_MFMA &&
         d.merge_mode == FI_MERGE_FUSED;
}

static bool fused_tiny(const fi_plan_desc& d, int64_t steps, int64_t workers) {
  return d.kind == FI_KIND_DECODE && d.decode_engine == FI_ENGINE_MFMA &&
         d.merge_mode == FI_MERGE_DEFAULT && d.cap_batch == 0 && steps <= workers;
}

static fi_status validate_table(const char* what, int32_t n, const int32_t* indptr,
                                const int32_t* len, int32_t ps) {
  if (n == 0) return FI_OK;
  if (!indptr || !len) return set_error(FI_ERR_INVALID_ARG, "%s arrays are NULL", what);
  if (indptr[0] != 0) return set_error(FI_ERR_INVALID_ARG, "%s indptr[0] = %d", what, indptr[0]);
  for (int32_t r = 0; r < n; ++r) {
    if (len[r] < 0) return set_error(FI_ERR_INVALID_ARG, "%s len[%d] = %d", what, r, len[r]);
    const int64_t pages = (int64_t)indptr[r + 1] - indptr[r];
    if (pages != ceil_div(len[r], ps))
      return set_error(FI_ERR_INVALID_ARG,
                       "%s entry %d: %lld pages for %d tokens at page size %d", what, r,
                       (long long)pages, len[r], ps);
  }
  return FI_OK;
}

static fi_status build(const fi_plan_desc& d, const int32_t* kv_indptr, const int32_t* kv_len,
                       const int32_t* qo_indptr, const int32_t* prefix_indptr,
                       const int32_t* prefix_len, const int32_t* req_group,
                       const int32_t* prefix_parent, HostPlan& hp) {
  const int32_t B = d.batch, Hkv = d.num_kv_heads, G = d.num_qo_heads / d.num_kv_heads;
  const int32_t ps = d.page_size;
  hp.fused = fused_merge(d);
  fi_status st = validate_table("kv", B, kv_indptr, kv_len, ps);
  if (st != FI_OK) return st;
  if (d.kind == FI_KIND_APPEND && B > 0) {
    if (!qo_indptr) return set_error(FI_ERR_INVALID_ARG, "append plan needs qo_indptr");
    if (qo_indptr[0] != 0) return set_error(FI_ERR_INVALID_ARG, "qo_indptr[0] != 0");
    for (int32_t r = 0; r < B; ++r) {
      const int32_t nq = qo_indptr[r + 1] - qo_indptr[r];
      if (nq < 0 || nq > kv_len[r])
        return set_error(FI_ERR_INVALID_ARG, "request %d: qo %d not in [0, kv_len %d]", r, nq,
                         kv_len[r]);
    }
  }
  const int32_t NG = d.num_prefix_groups;
  if (d.kind == FI_KIND_CASCADE) {
    st = validate_table("prefix", NG, prefix_indptr, prefix_len, ps);
    if (st != FI_OK) return st;
    if (B > 0 && !req_group)
      return set_error(FI_ERR_INVALID_ARG, "cascade plan needs req_prefix_group");
    for (int32_t r = 0; r < B; ++r)
      if (req_group[r] < -1 || req_group[r] >= NG)
        return set_error(FI_ERR_INVALID_ARG, "request %d: prefix group %d of %d", r,
                         req_group[r], NG);
    for (int32_t grp = 0; prefix_parent && grp < NG; ++grp)
      if (prefix_parent[grp] < -1 || prefix_parent[grp] >= grp)
        return set_error(FI_ERR_INVALID_ARG,
                         "prefix group %d: parent %d (need -1 or a lower group index)", grp,
                         prefix_parent[grp]);
  }
  int32_t next_row = 0;
  auto decode_level = [&](Level& lv) {
    lv.rows_per_block = ROWS_DECODE;
    lv.num_workers = d.num_cus * d.workers_per_cu;
    lv.min_chunk_pages = d.min_chunk_pages;
  };
  auto wide_level = [&](Level& lv) {
    lv.rows_per_block = ROWS_WIDE;
    lv.num_workers = d.num_cus * std::max(1, d.workers_per_cu / 2);
    lv.min_chunk_pages = WIDE_CHUNK_FACTOR * d.min_chunk_pages;
  };
  if (d.kind == FI_KIND_CASCADE) {
    hp.num_levels = 2;
    wide_level(hp.level[0]);
    decode_level(hp.level[1]);
    std::vector<Unit> pu;
    // members of a group: the requests whose chain (own group, its parent,
    // ...) passes through it, in request order
    std::vector<std::vector<int32_t>> in_group(NG);
    for (int32_t r = 0; r < B; ++r) {
      int32_t depth = 0;
      for (int32_t h = req_group[r]; h >= 0; h = prefix_parent ? prefix_parent[h] : -1) {
        in_group[h].push_back(r);
        ++depth;
      }
      if (depth > d.max_prefix_depth)
        return set_error(FI_ERR_INVALID_ARG, "request %d has %d nested prefixes, max_prefix_depth %d",
                         r, depth, d.max_prefix_depth);
    }
    for (int32_t grp = 0; grp < NG; ++grp) {
      const std::vector<int32_t>& members = in_group[grp];
      if (members.empty() || prefix_len[grp] == 0) continue;
      const int32_t off = (int32_t)hp.qlist.size();
      hp.qlist.insert(hp.qlist.end(), members.begin(), members.end());
      const int64_t rows = (int64_t)members.size() * G;
      for (int64_t b = 0; b < ceil_div(rows, ROWS_WIDE); ++b) {
        const int32_t r0 = (int32_t)(b * ROWS_WIDE);
        const int32_t r1 = (int32_t)std::min<int64_t>(rows, (b + 1) * ROWS_WIDE);
        for (int32_t g = 0; g < Hkv; ++g) {
          Unit u;
          u.unit = grp;
          u.q_base = off;
          u.row0 = r0;
          u.n_rows = r1 - r0;
          u.g = g;
          u.page_off = prefix_indptr[grp];
          u.t_lim = prefix_len[grp];
          u.n_pages = (int32_t)ceil_div(prefix_len[grp], ps);
          u.q_pos0 = 0;
          u.flags = FLAG_LIST_Q | FLAG_PREFIX;
          pu.push_back(u);
        }
      }
    }
    std::vector<Unit> su;
    request_units(su, B, G, Hkv, ps, ROWS_DECODE, kv_indptr, kv_len, nullptr, false);
    LevelBuild lbs2[2];
    LevelBuild& lbp = lbs2[0];
    LevelBuild& lbs = lbs2[1];
    if (d.launch == FI_LAUNCH_POD) {
      const std::vector<Unit> both[2] = {pu, su};
      st = pod_levels(d, both, true, next_row, lbs2, hp);
      if (st != FI_OK) return st;
    } else {
      build_level(pu, d, true, next_row, lbp, hp.level[0]);
      build_level(su, d, true, next_row, lbs, hp.level[1]);
    }
    // prefix partial rows of (request, kv head)
    std::vector<std::vector<int32_t>> pref((size_t)B * Hkv);
    for (size_t ui = 0; ui < pu.size(); ++ui) {
      const Unit& u = pu[ui];
      const std::vector<int32_t>& dsts = lbp.chunks[ui].second;
      for (int32_t local = 0; local < u.n_rows; local += G) {
        const int32_t r = hp.qlist[u.q_base + (u.row0 + local) / G];
        std::vector<int32_t>& v = pref[(size_t)r * Hkv + u.g];
        for (int32_t dd : dsts) v.push_back(dd + local);
      }
    }
    for (size_t ui = 0; ui < su.size(); ++ui) {
      const Unit& u = su[ui];
      const std::vector<int32_t>& pl = pref[(size_t)u.unit * Hkv + u.g];
      const std::vector<int32_t>& dsts = lbs.chunks[ui].second;
      const int32_t n = (int32_t)(pl.size() + dsts.size());
      const int32_t rec[MERGE_INTS] = {u.unit, 0, G, u.g, (int32_t)hp.parts.size(), n};
      hp.merges.insert(hp.merges.end(), rec, rec + MERGE_INTS);
      hp.parts.insert(hp.parts.end(), pl.begin(), pl.end());
      hp.parts.insert(hp.parts.end(), dsts.begin(), dsts.end());
    }
  } else {
    const bool append = d.kind == FI_KIND_APPEND;
    const bool causal = append && d.causal;
    std::vector<Unit> units[2];
    LevelBuild lb[2];
    if (append && d.launch == FI_LAUNCH_POD) {
      // Fused mixed batch: requests whose query rows fit one decode row block
      // go to the decode role (level 1), the others to the wide role (level
      // 0); the launch's P workgroups (as many as a wide level has) are split
      // between the roles by cost.
      hp.num_levels = 2;
      wide_level(hp.level[0]);
      decode_level(hp.level[1]);
      std::vector<uint8_t> small(B), big(B);
      for (int32_t r = 0; r < B; ++r) {
        small[r] = (int64_t)(qo_indptr[r + 1] - qo_indptr[r]) * G <= ROWS_DECODE;
        big[r] = !small[r];
      }
      request_units(units[0], B, G, Hkv, ps, ROWS_WIDE, kv_indptr, kv_len, qo_indptr, causal,
                    big.data());
      request_units(units[1], B, G, Hkv, ps, ROWS_DECODE, kv_indptr, kv_len, qo_indptr, causal,
                    small.data());
      st = pod_levels(d, units, false, next_row, lb, hp);
      if (st != FI_OK) return st;
    } else {
      hp.num_levels = 1;
      if (append) wide_level(hp.level[0]); else decode_level(hp.level[0]);
      request_units(units[0], B, G, Hkv, ps, hp.level[0].rows_per_block, kv_indptr, kv_len,
                    append ? qo_indptr : nullptr, causal);
      bool tiny = false;
      if (!append) {
        const int64_t gp = std::max(1, 32 / ps);
        int64_t steps = 0;
        for (const Unit& u : units[0]) steps += ceil_div(u.n_pages, gp);
        tiny = fused_tiny(d, steps, hp.level[0].num_workers);
        hp.fused = hp.fused || tiny;
      }
      const int32_t S0 = hp.level[0].num_workers;
      hp.wg_fold = tiny && !d.deterministic && S0 % 4 == 0 &&
                   (int64_t)units[0].size() * 4 <= S0;
      build_level(units[0], d, false, next_row, lb[0], hp.level[0], tiny && !d.deterministic,
                  hp.wg_fold);
    }
    std::vector<int32_t> first_rec[2];
    for (int l = 0; l < hp.num_levels; ++l) first_rec[l] = unit_merges(units[l], lb[l], hp);
    if (!append && hp.fused) {
      // decode units have at most MERGE_ROWS rows: one record each
      const Level& lv = hp.level[0];
      hp.item_rec.resize(lv.item_unit.size());
      for (size_t i = 0; i < lv.item_unit.size(); ++i) hp.item_rec[i] = first_rec[0][lv.item_unit[i]];
      for (size_t e = 0; e < hp.merges.size() / MERGE_INTS; ++e)
        if (hp.merges[e * MERGE_INTS + M_N] == 0) hp.empty_recs.push_back((int32_t)e);
    }
    if (append) {
      for (int32_t r = 0; r < B; ++r) {
        const int32_t nq = qo_indptr[r + 1] - qo_indptr[r];
        for (int32_t i = 0; i < nq; ++i) {
          const int32_t pos = kv_len[r] - nq + i;
          hp.scatter.push_back(kv_indptr[r] + pos / ps);
          hp.scatter.push_back(pos % ps);
        }
      }
    }
  }
  hp.num_part_rows = next_row;
  return FI_OK;
}

// A batch of block-sparse sequences, as the host arrays describe it: per
// sequence s its query and key counts, its row and column block counts, and
// offsets of its blocks and mask in the concatenated size and mask arrays.
struct BsBatch {
  int32_t S = 0;
  const int32_t *qo_len = nullptr, *kv_len = nullptr, *nrb = nullptr, *ncb = nullptr;
  const int32_t *row_sz = nullptr, *col_sz = nullptr;
  const uint8_t* mask = nullptr;
  const int32_t *kv_indptr = nullptr, *kv_indices = nullptr;   // kv_indices NULL: ragged
  std::vector<int64_t> row_off, col_off, mask_off;              // per sequence
};

// Check the batch and compute the per-sequence offsets.
static fi_status check_bs_batch(const fi_plan_desc& d, BsBatch& bb) {
  const int32_t Hkv = d.num_kv_heads, ps = d.page_size, S = bb.S;
  const bool ragged = d.kv_layout == FI_KV_LAYOUT_RAGGED;
  if (S < 0) return set_error(FI_ERR_INVALID_ARG, "negative number of sequences");
  if (S > 0 && (!bb.qo_len || !bb.kv_len || !bb.nrb || !bb.ncb || !bb.kv_indptr))
    return set_error(FI_ERR_INVALID_ARG, "block-sparse arrays are NULL");
  if (!ragged && S > 0 && !bb.kv_indices)
    return set_error(FI_ERR_INVALID_ARG, "a paged block-sparse plan needs kv_indices");
  if (S > 0 && bb.kv_indptr[0] != 0)
    return set_error(FI_ERR_INVALID_ARG, "kv_indptr[0] = %d", bb.kv_indptr[0]);
  bb.row_off.assign(S + 1, 0);
  bb.col_off.assign(S + 1, 0);
  bb.mask_off.assign(S + 1, 0);
  for (int32_t q = 0; q < S; ++q) {
    const int32_t qo = bb.qo_len[q], L = bb.kv_len[q], MB = bb.nrb[q], NB = bb.ncb[q];
    if (qo < 0 || L < 0 || MB < 0 || NB < 0)
      return set_error(FI_ERR_INVALID_ARG, "sequence %d: negative block-sparse size", q);
    const int64_t span = (int64_t)bb.kv_indptr[q + 1] - bb.kv_indptr[q];
    const int64_t want = ragged ? L : ceil_div(L, ps);
    if (span != want)
      return set_error(FI_ERR_INVALID_ARG,
                       "sequence %d: kv_indptr spans %lld %s for %d keys", q, (long long)span,
                       ragged ? "tokens" : "pages", L);
    bb.row_off[q + 1] = bb.row_off[q] + (int64_t)Hkv * MB;
    bb.col_off[q + 1] = bb.col_off[q] + (int64_t)Hkv * NB;
    bb.mask_off[q + 1] = bb.mask_off[q] + (int64_t)Hkv * MB * NB;
  }
  if ((bb.row_off[S] > 0 && !bb.row_sz) || (bb.col_off[S] > 0 && !bb.col_sz) ||
      (bb.mask_off[S] > 0 && !bb.mask))
    return set_error(FI_ERR_INVALID_ARG, "block-sparse arrays are NULL");
  for (int32_t q = 0; q < S; ++q) {
    const int32_t MB = bb.nrb[q], NB = bb.ncb[q];
    const int32_t* rsz = bb.row_sz + bb.row_off[q];
    const int32_t* csz = bb.col_sz + bb.col_off[q];
    for (int32_t g = 0; g < Hkv; ++g) {
      int64_t rs = 0, cs = 0;
      for (int32_t a = 0; a < MB; ++a) {
        if (rsz[g * MB + a] < 0) return set_error(FI_ERR_INVALID_ARG, "negative row block size");
        rs += rsz[g * MB + a];
      }
      for (int32_t b = 0; b < NB; ++b) {
        const int32_t c = csz[g * NB + b];
        if (c < 0) return set_error(FI_ERR_INVALID_ARG, "negative column block size");
        if (c > 0 && cs % ps)
          return set_error(FI_ERR_INVALID_ARG,
                           "sequence %d, kv head %d: column block %d starts at key %lld, not a "
                           "page boundary", q, g, b, (long long)cs);
        cs += c;
      }
      if (rs != bb.qo_len[q] || cs != bb.kv_len[q])
        return set_error(FI_ERR_INVALID_ARG,
                         "sequence %d, kv head %d: row blocks sum to %lld (qo_len %d), column "
                         "blocks to %lld (kv_len %d)", q, g, (long long)rs, bb.qo_len[q],
                         (long long)cs, bb.kv_len[q]);
    }
  }
  return FI_OK;
}

// Variable block-sparse over a batch of sequences: every (sequence, kv head
// g, row block a) is a unit set over the page list of a's selected column
// blocks (in column order), appended to hp.plist; units in the order
// sequence, g, a, 128-row (or, in the decode role, 16-row) block. Rows of a
// fit one 16-row block -> decode role of a POD launch. A paged batch lists
// the pool's page ids (kv_indices); a ragged one (keys k[kv_indptr[s] + t]
// of a [tokens][Hkv][D] tensor) lists the first token of each page_size-token
// run, which the kernels address in the ragged layout.
static fi_status build_block_sparse(const fi_plan_desc& d, const BsBatch& bb, HostPlan& hp) {
  const int32_t Hkv = d.num_kv_heads, G = d.num_qo_heads / d.num_kv_heads, ps = d.page_size;
  const bool ragged = d.kv_layout == FI_KV_LAYOUT_RAGGED;
  const bool pod = d.launch == FI_LAUNCH_POD;
  std::vector<Unit> units[2];
  int32_t q_seq = 0, unit_id = 0;   // first query row of the sequence; row-block counter
  for (int32_t q = 0; q < bb.S; ++q) {
    const int32_t MB = bb.nrb[q], NB = bb.ncb[q];
    const int32_t* rsz = bb.row_sz + bb.row_off[q];
    const int32_t* csz = bb.col_sz + bb.col_off[q];
    const uint8_t* msk = bb.mask + bb.mask_off[q];
    const int32_t base = bb.kv_indptr[q];
    for (int32_t g = 0; g < Hkv; ++g) {
      int32_t q0 = q_seq;
      for (int32_t a = 0; a < MB; ++a) {
        const int32_t nq = rsz[g * MB + a];
        const int32_t off = (int32_t)hp.plist.size();
        int32_t t_lim = 0, c0 = 0;
        for (int32_t b = 0; b < NB; ++b) {
          const int32_t c = csz[g * NB + b];
          if (c > 0 && msk[((int64_t)g * MB + a) * NB + b]) {
            for (int32_t pg = c0 / ps; pg < (int32_t)ceil_div(c0 + c, ps); ++pg)
              hp.plist.push_back(ragged ? base + pg * ps : bb.kv_indices[base + pg]);
            t_lim += c;
          }
          c0 += c;
        }
        const int64_t rows = (int64_t)nq * G;
        const int lvl = (pod && rows <= ROWS_DECODE) ? 1 : 0;
        const int32_t rpb = lvl ? ROWS_DECODE : ROWS_WIDE;
        for (int64_t blk = 0; blk < ceil_div(rows, rpb); ++blk) {
          Unit u;
          u.unit = unit_id;
          u.q_base = q0;
          u.row0 = (int32_t)(blk * rpb);
          u.n_rows = (int32_t)std::min<int64_t>(rows - blk * rpb, rpb);
          u.g = g;
          u.page_off = off;
          u.t_lim = t_lim;
          u.n_pages = (int32_t)ceil_div(t_lim, ps);
          u.q_pos0 = 0;
          u.flags = 0;
          units[lvl].push_back(u);
        }
        q0 += nq;
        ++unit_id;
      }
    }
    q_seq += bb.qo_len[q];
  }
  int32_t next_row = 0;
  LevelBuild lb[2];
  Level& l0 = hp.level[0];
  l0.rows_per_block = ROWS_WIDE;
  l0.num_workers = d.num_cus * std::max(1, d.workers_per_cu / 2);
  l0.min_chunk_pages = WIDE_CHUNK_FACTOR * d.min_chunk_pages;
  if (pod) {
    Level& l1 = hp.level[1];
    l1.rows_per_block = ROWS_DECODE;
    l1.num_workers = d.num_cus * d.workers_per_cu;
    l1.min_chunk_pages = d.min_chunk_pages;
    hp.num_levels = 2;
    fi_status st = pod_levels(d, units, false, next_row, lb, hp);
    if (st != FI_OK) return st;
  } else {
    hp.num_levels = 1;
    build_level(units[0], d, false, next_row, lb[0], l0);
  }
  for (int l = 0; l < hp.num_levels; ++l) unit_merges(units[l], lb[l], hp);
  hp.num_part_rows = next_row;
  return FI_OK;
}

// ---------------------------------------------------------------- upload sync

// One event per pinned staging buffer: the next plan into the same buffer
// waits for the previous upload to have read it.
static std::mutex g_upload_mu;
static std::map<void*, hipEvent_t> g_upload_events;

}  // namespace fi

using namespace fi;

// Defaults, and the device's CU count when the caller leaves it open.
static fi_status begin_plan(const fi_plan_desc* desc, void* ws_dev, void* ws_host,
                            fi_plan_desc& d) {
  fi_status st = fill_defaults(desc, d);
  if (st != FI_OK) return st;
  if (ws_dev && !ws_host)
    return set_error(FI_ERR_INVALID_ARG, "a device plan needs a pinned host staging buffer");
  if (d.num_cus == 0) {
    if (!ws_dev)
      return set_error(FI_ERR_INVALID_ARG, "a host-only plan needs num_cus > 0");
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return set_error(FI_ERR_HIP, "device query: %s", hipGetErrorString(e));
    d.num_cus = cus;
  }
  return FI_OK;
}

// The plan's int32 sections at their layout offsets (L.blob_bytes bytes at h;
// the bytes between sections are left as they are).
static void fill_blob(const HostPlan& hp, const Layout& L, char* h) {
  for (int l = 0; l < 2; ++l) {
    if (!hp.level[l].items.empty())
      memcpy(h + L.items[l], hp.level[l].items.data(), hp.level[l].items.size() * 4);
    if (!hp.level[l].worker_indptr.empty())
      memcpy(h + L.windptr[l], hp.level[l].worker_indptr.data(),
             hp.level[l].worker_indptr.size() * 4);
  }
  if (!hp.merges.empty()) memcpy(h + L.merges, hp.merges.data(), hp.merges.size() * 4);
  if (!hp.parts.empty()) memcpy(h + L.parts, hp.parts.data(), hp.parts.size() * 4);
  if (!hp.qlist.empty()) memcpy(h + L.qlist, hp.qlist.data(), hp.qlist.size() * 4);
  if (!hp.scatter.empty()) memcpy(h + L.scatter, hp.scatter.data(), hp.scatter.size() * 4);
  const int32_t meta[META_INTS] = {hp.pod_wide_blocks,
                                   (int32_t)(hp.merges.size() / MERGE_INTS), hp.merge_rows,
                                   (int32_t)(hp.scatter.size() / 2),
                                   (int32_t)hp.empty_recs.size()};
  memcpy(h + L.meta, meta, sizeof(meta));
  if (!hp.plist.empty()) memcpy(h + L.plist, hp.plist.data(), hp.plist.size() * 4);
  if (hp.fused) {
    if (!hp.item_rec.empty()) memcpy(h + L.item_rec, hp.item_rec.data(), hp.item_rec.size() * 4);
    // every count starts at 0; the kernel's last arrival resets its own
    memset(h + L.counters, 0, hp.merges.size() / MERGE_INTS * 4);
    if (!hp.empty_recs.empty())
      memcpy(h + L.empty_recs, hp.empty_recs.data(), hp.empty_recs.size() * 4);
  }
}

// Lay the built plan out, check the caller's workspace, and upload (the
// pinned staging buffer is reused only after its previous upload was read).
struct Caps;
static Layout caps_layout(const Caps& c, int32_t head_dim);
static fi_status check_caps(const HostPlan& hp, const Caps& c);
static fi_status finish_plan(fi_plan_t* p, const Caps* caps, void* ws_dev, size_t ws_dev_bytes,
                             void* ws_host, size_t ws_host_bytes, void* stream,
                             fi_plan_t** out) {
  HostPlan& hp = p->hp;
  const fi_plan_desc& d = hp.desc;
  for (size_t i = M_NROWS; i < hp.merges.size(); i += MERGE_INTS)
    hp.merge_rows = std::max(hp.merge_rows, hp.merges[i]);
  size_t n_items[2] = {(size_t)hp.level[0].num_items(), (size_t)hp.level[1].num_items()};
  const int32_t workers[2] = {hp.level[0].num_workers, hp.level[1].num_workers};
  if (caps) {
    const fi_status st = check_caps(hp, *caps);
    if (st != FI_OK) {
      delete p;
      return st;
    }
    p->lay = caps_layout(*caps, d.head_dim);
  } else {
    p->lay = layout_for(workers, n_items, hp.merges.size() / MERGE_INTS, hp.parts.size(),
                        hp.qlist.size(), hp.scatter.size() / 2, (size_t)hp.num_part_rows,
                        d.head_dim, hp.plist.size(), hp.fused);
  }
  const Layout& L = p->lay;
  if (ws_dev) {
    if (ws_dev_bytes < L.dev_bytes || ws_host_bytes < L.blob_bytes) {
      delete p;
      return set_error(FI_ERR_WORKSPACE,
                       "workspace too small: need %zu device / %zu host bytes, got %zu / %zu",
                       L.dev_bytes, L.blob_bytes, ws_dev_bytes, ws_host_bytes);
    }
    hipStream_t s = (hipStream_t)stream;
    hipEvent_t ev = nullptr;
    {
      std::lock_guard<std::mutex> lk(g_upload_mu);
      auto itv = g_upload_events.find(ws_host);
      if (itv != g_upload_events.end()) ev = itv->second;
    }
    hipError_t e = hipSuccess;
    if (ev) e = hipEventSynchronize(ev);
    if (e != hipSuccess) {
      delete p;
      return set_error(FI_ERR_HIP, "waiting for the previous upload: %s", hipGetErrorString(e));
    }
    fill_blob(hp, L, (char*)ws_host);
    e = hipMemcpyAsync(ws_dev, ws_host, L.blob_bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) {
      if (!ev) {
        e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e == hipSuccess) {
          std::lock_guard<std::mutex> lk(g_upload_mu);
          g_upload_events[ws_host] = ev;
        }
      }
      if (e == hipSuccess) e = hipEventRecord(ev, s);
    }
    if (e != hipSuccess) {
      delete p;
      return set_error(FI_ERR_HIP, "plan upload: %s", hipGetErrorString(e));
    }
    p->on_device = true;
    p->dev_base = (char*)ws_dev;
  } else {
    // a host-only plan keeps its int32 sections laid out as on the device, so
    // that a run call can upload them itself (fi_paged_decode_noalloc)
    p->host_blob.assign(L.blob_bytes, 0);
    fill_blob(hp, L, p->host_blob.data());
  }
  *out = p;
  return FI_OK;
}



// Per-section capacities of any plan with this (defaults-filled) description,
// at most d.batch requests and the given totals.
struct Caps {
  int32_t workers[2] = {0, 0};
  size_t items[2] = {0, 0};
  size_t merges = 0, parts = 0, qlist = 0, scatter = 0, part_rows = 0;
  bool fused = false;
};

static void bound_counts(const fi_plan_desc& d, int32_t num_cus, int64_t max_kv_pages,
                         int64_t max_qo_tokens, int64_t max_prefix_pages, Caps& c) {
  const int64_t S_dec = (int64_t)num_cus * d.workers_per_cu;
  const int64_t S_wide = (int64_t)num_cus * std::max(1, d.workers_per_cu / 2);
  const int64_t B = d.batch, Hkv = d.num_kv_heads, G = d.num_qo_heads / d.num_kv_heads;
  const int64_t c_det = std::max(1, d.det_chunk_pages);
  int64_t part_rows = 0, merges = 0;
  // balanced: items <= S + units (every piece boundary is a quota or a unit
  // boundary); deterministic: items <= pages / c + units
  auto level_bound = [&](int64_t S, int64_t units, int64_t pages_sum, int64_t rpb) {
    const int64_t cl = rpb == ROWS_DECODE ? std::max<int64_t>(1, c_det / 2) : c_det;
    const int64_t items = d.deterministic ? pages_sum / cl + units : S + units;
    part_rows += items * rpb;
    return items;
  };
  if (d.kind == FI_KIND_CASCADE) {
    // groups with members: at most NG, and at most B * depth (each request
    // is a member of at most depth groups; groups without members plan nothing)
    const int64_t NG = std::min<int64_t>(d.num_prefix_groups, B * d.max_prefix_depth);
    const int64_t blocks = ceil_div(B * G * d.max_prefix_depth, ROWS_WIDE) + NG;
    c.items[0] = (size_t)level_bound(S_wide, blocks * Hkv, blocks * Hkv * max_prefix_pages, ROWS_WIDE);
    // a fused launch has 4 decode wavefronts on each of its S_wide workgroups
    const int64_t S1 = d.launch == FI_LAUNCH_POD ? WAVES_PER_BLOCK * S_wide : S_dec;
    c.items[1] = (size_t)level_bound(S1, B * Hkv, Hkv * max_kv_pages, ROWS_DECODE);
    c.workers[0] = (int32_t)S_wide;
    c.workers[1] = (int32_t)S1;
    merges = B * Hkv;
  } else if (d.kind == FI_KIND_APPEND && d.launch == FI_LAUNCH_POD) {
    // wide role: at most P workgroups; decode role: at most 4P wavefronts
    const int64_t P = S_wide;
    const int64_t blocks = ceil_div(max_qo_tokens * G, ROWS_WIDE) + B;
    const int64_t per_req_blocks = ceil_div(max_qo_tokens * G, ROWS_WIDE) + 1;
    c.items[0] = (size_t)level_bound(P, blocks * Hkv, Hkv * per_req_blocks * max_kv_pages,
                                     ROWS_WIDE);
    c.items[1] = (size_t)level_bound(WAVES_PER_BLOCK * P, B * Hkv, Hkv * max_kv_pages,
                                     ROWS_DECODE);
    c.workers[0] = (int32_t)P;
    c.workers[1] = (int32_t)(WAVES_PER_BLOCK * P);
    merges = part_rows + (blocks + B) * Hkv * 2;
  } else if (d.kind == FI_KIND_APPEND) {
    const int64_t blocks = ceil_div(max_qo_tokens * G, ROWS_WIDE) + B;
    const int64_t per_req_blocks = ceil_div(max_qo_tokens * G, ROWS_WIDE) + 1;
    c.items[0] = (size_t)level_bound(S_wide, blocks * Hkv, Hkv * per_req_blocks * max_kv_pages,
                                     ROWS_WIDE);
    c.workers[0] = (int32_t)S_wide;
    merges = part_rows + blocks * Hkv * 2;
  } else {
    const int64_t blocks = B * ceil_div(G, ROWS_DECODE);
    c.items[0] = (size_t)level_bound(S_dec, blocks * Hkv,
                                     Hkv * ceil_div(G, ROWS_DECODE) * max_kv_pages, ROWS_DECODE);
    c.workers[0] = (int32_t)S_dec;
    merges = part_rows + blocks * Hkv * 2;
  }
  c.merges = (size_t)merges;
  c.parts = (size_t)part_rows;
  c.part_rows = (size_t)part_rows;
  c.scatter = d.kind == FI_KIND_APPEND ? (size_t)max_qo_tokens : 0;
  c.qlist = (size_t)B * (d.kind == FI_KIND_CASCADE ? d.max_prefix_depth : 1);
  c.fused = fused_merge(d);
}

// The capacities a graph-stable description (cap_batch > 0) lays its
// workspace out for: cap_batch requests, the capped totals, and at most
// cap_batch * max_prefix_depth prefix groups with members.
static void stable_caps(const fi_plan_desc& d, int32_t num_cus, Caps& c) {
  fi_plan_desc dc = d;
  dc.batch = d.cap_batch;
  dc.num_prefix_groups = d.cap_batch * d.max_prefix_depth;
  bound_counts(dc, num_cus, d.cap_kv_pages, d.cap_qo_tokens, d.cap_prefix_pages, c);
}

static Layout caps_layout(const Caps& c, int32_t head_dim) {
  return layout_for(c.workers, c.items, c.merges, c.parts, c.qlist, c.scatter, c.part_rows,
                    head_dim, 0, c.fused);
}

// A built plan against the capacities of its graph-stable layout (a bound
// that holds by construction; checked so that a broken bound is an error,
// not an overrun).
static fi_status check_caps(const HostPlan& hp, const Caps& c) {
  for (int l = 0; l < 2; ++l)
    if ((size_t)hp.level[l].num_items() > c.items[l] || hp.level[l].num_workers > c.workers[l])
      return set_error(FI_ERR_WORKSPACE, "level %d exceeds its capacity", l);
  if (hp.merges.size() / MERGE_INTS > c.merges || hp.parts.size() > c.parts ||
      hp.qlist.size() > c.qlist || hp.scatter.size() / 2 > c.scatter ||
      (size_t)hp.num_part_rows > c.part_rows)
    return set_error(FI_ERR_WORKSPACE, "plan exceeds its capacity");
  return FI_OK;
}

static fi_status device_cus(int32_t& num_cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return set_error(FI_ERR_HIP, "could not query the device's compute units");
  return FI_OK;
}

extern "C" fi_status fi_workspace_size(const fi_plan_desc* desc, int64_t max_kv_pages,
                                       int64_t max_qo_tokens, int64_t max_prefix_pages,
                                       size_t* dev_bytes, size_t* host_bytes) {
  clear_error();
  fi_plan_desc d;
  fi_status st = fill_defaults(desc, d);
  if (st != FI_OK) return st;
  if (!dev_bytes || !host_bytes) return set_error(FI_ERR_INVALID_ARG, "NULL output pointer");
  if (d.kind == FI_KIND_BLOCK_SPARSE)
    return set_error(FI_ERR_INVALID_ARG, "block-sparse plans: fi_workspace_size_block_sparse");
  if (max_kv_pages < 0 || max_qo_tokens < 0 || max_prefix_pages < 0)
    return set_error(FI_ERR_INVALID_ARG, "negative size bound");
  int32_t num_cus = d.num_cus;
  if (num_cus == 0 && (st = device_cus(num_cus)) != FI_OK) return st;
  Caps c;
  if (d.cap_batch > 0)   // graph-stable: the layout its plans use, whatever the arguments
    stable_caps(d, num_cus, c);
  else
    bound_counts(d, num_cus, max_kv_pages, max_qo_tokens, max_prefix_pages, c);
  const Layout L = caps_layout(c, d.head_dim);
  *dev_bytes = L.dev_bytes;
  *host_bytes = L.blob_bytes;
  return FI_OK;
}

// Workspace bound of a block-sparse batch (the checked batch bb).
static void bs_layout_bound(const fi_plan_desc& d, int32_t num_cus, const BsBatch& bb,
                            size_t* dev_bytes, size_t* host_bytes) {
  const int64_t Hkv = d.num_kv_heads, G = d.num_qo_heads / d.num_kv_heads;
  const int64_t P = (int64_t)num_cus * std::max(1, d.workers_per_cu / 2);
  const int64_t S1 = d.launch == FI_LAUNCH_POD ? WAVES_PER_BLOCK * P : 0;
  const int64_t c_det = std::max(1, d.det_chunk_pages);
  // units: every (sequence, kv head, row block) in blocks of at least 16 rows;
  // pages: each unit's list is at most its sequence's pages
  int64_t units = 0, unit_pages = 0, q_rows = 0, plist = 0;
  for (int32_t q = 0; q < bb.S; ++q) {
    const int64_t seq_pages = ceil_div(bb.kv_len[q], d.page_size);
    const int64_t u = Hkv * (ceil_div((int64_t)bb.qo_len[q] * G, ROWS_DECODE) + bb.nrb[q]);
    units += u;
    unit_pages += u * seq_pages;
    q_rows += bb.qo_len[q];
    plist += Hkv * bb.nrb[q] * seq_pages;
  }
  auto items_of = [&](int64_t S, int64_t c) {
    return d.deterministic ? unit_pages / c + units : S + units;
  };
  size_t n_items[2] = {(size_t)items_of(P, c_det),
                       S1 ? (size_t)items_of(S1, std::max<int64_t>(1, c_det / 2)) : 0};
  const int32_t workers[2] = {(int32_t)P, (int32_t)S1};
  const int64_t part_rows = ((int64_t)n_items[0] + (int64_t)n_items[1]) * ROWS_WIDE;
  const int64_t merges = Hkv * q_rows + 2 * units;
  Layout L = layout_for(workers, n_items, (size_t)merges, (size_t)part_rows, 0, 0,
                        (size_t)part_rows, d.head_dim, (size_t)plist);
  *dev_bytes = L.dev_bytes;
  *host_bytes = L.blob_bytes;
}

static fi_status bs_begin(const fi_plan_desc* desc, fi_plan_desc& d) {
  fi_status st = fill_defaults(desc, d);
  if (st != FI_OK) return st;
  if (d.kind != FI_KIND_BLOCK_SPARSE)
    return set_error(FI_ERR_INVALID_ARG, "block-sparse calls need kind FI_KIND_BLOCK_SPARSE");
  return FI_OK;
}

extern "C" fi_status fi_workspace_size_block_sparse_batch(
    const fi_plan_desc* desc, int32_t num_seqs, const int32_t* qo_len_h, const int32_t* kv_len_h,
    const int32_t* num_row_blocks_h, const int32_t* num_col_blocks_h, size_t* dev_bytes,
    size_t* host_bytes) {
  clear_error();
  fi_plan_desc d;
  fi_status st = bs_begin(desc, d);
  if (st != FI_OK) return st;
  if (!dev_bytes || !host_bytes) return set_error(FI_ERR_INVALID_ARG, "NULL output pointer");
  if (num_seqs < 0) return set_error(FI_ERR_INVALID_ARG, "negative number of sequences");
  if (num_seqs > 0 && (!qo_len_h || !kv_len_h || !num_row_blocks_h || !num_col_blocks_h))
    return set_error(FI_ERR_INVALID_ARG, "block-sparse arrays are NULL");
  BsBatch bb;
  bb.S = num_seqs;
  bb.qo_len = qo_len_h;
  bb.kv_len = kv_len_h;
  bb.nrb = num_row_blocks_h;
  bb.ncb = num_col_blocks_h;
  for (int32_t q = 0; q < num_seqs; ++q)
    if (qo_len_h[q] < 0 || kv_len_h[q] < 0 || num_row_blocks_h[q] < 0 || num_col_blocks_h[q] < 0)
      return set_error(FI_ERR_INVALID_ARG, "negative size bound");
  int32_t num_cus = d.num_cus;
  if (num_cus == 0 && (st = device_cus(num_cus)) != FI_OK) return st;
  bs_layout_bound(d, num_cus, bb, dev_bytes, host_bytes);
  return FI_OK;
}

extern "C" fi_status fi_workspace_size_block_sparse(const fi_plan_desc* desc, int32_t qo_len,
                                                    int32_t kv_len, int32_t num_row_blocks,
                                                    int32_t num_col_blocks, size_t* dev_bytes,
                                                    size_t* host_bytes) {
  return fi_workspace_size_block_sparse_batch(desc, 1, &qo_len, &kv_len, &num_row_blocks,
                                              &num_col_blocks, dev_bytes, host_bytes);
}

extern "C" fi_status fi_plan(const fi_plan_desc* desc, const int32_t* kv_indptr_h,
                             const int32_t* kv_len_h, const int32_t* qo_indptr_h,
                             const int32_t* prefix_indptr_h, const int32_t* prefix_len_h,
                             const int32_t* req_prefix_group_h,
                             const int32_t* prefix_parent_h, void* ws_dev,
                             size_t ws_dev_bytes, void* ws_host, size_t ws_host_bytes,
                             void* stream, fi_plan_t** out) {
  clear_error();
  if (!out) return set_error(FI_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  fi_plan_desc d;
  fi_status st = begin_plan(desc, ws_dev, ws_host, d);
  if (st != FI_OK) return st;
  if (d.kind == FI_KIND_BLOCK_SPARSE)
    return set_error(FI_ERR_INVALID_ARG, "block-sparse plans are built by fi_plan_block_sparse");
  const bool stable = d.cap_batch > 0;
  Caps caps;
  if (stable) {
    // the batch must fit the capacity the workspace is laid out for
    const int32_t B = d.batch;
    const int64_t pages = B > 0 && kv_indptr_h ? kv_indptr_h[B] : 0;
    const int64_t qo = d.kind == FI_KIND_APPEND && B > 0 && qo_indptr_h ? qo_indptr_h[B] : 0;
    const int64_t ppages = d.kind == FI_KIND_CASCADE && d.num_prefix_groups > 0 && prefix_indptr_h
                               ? prefix_indptr_h[d.num_prefix_groups] : 0;
    if (B > d.cap_batch || pages > d.cap_kv_pages || qo > d.cap_qo_tokens ||
        ppages > d.cap_prefix_pages)
      return set_error(FI_ERR_INVALID_ARG,
                       "batch exceeds the plan's capacity: %d requests / %lld pages / %lld "
                       "query tokens / %lld prefix pages against %d / %d / %d / %d",
                       B, (long long)pages, (long long)qo, (long long)ppages, d.cap_batch,
                       d.cap_kv_pages, d.cap_qo_tokens, d.cap_prefix_pages);
    stable_caps(d, d.num_cus, caps);
  }
  fi_plan_t* p = new fi_plan_t();
  p->hp.desc = d;
  st = build(d, kv_indptr_h, kv_len_h, qo_indptr_h, prefix_indptr_h, prefix_len_h,
             req_prefix_group_h, d.kind == FI_KIND_CASCADE ? prefix_parent_h : nullptr, p->hp);
  if (st != FI_OK) {
    delete p;
    return st;
  }
  if (stable) {
    p->hp.stable = true;
    p->hp.cap_merges = (int64_t)caps.merges;
    p->hp.cap_scatter = (int64_t)caps.scatter;
  }
  p->hp.kv_entries = d.batch > 0 ? kv_indptr_h[d.batch] : 0;
  p->hp.prefix_entries = d.kind == FI_KIND_CASCADE && d.num_prefix_groups > 0
                             ? prefix_indptr_h[d.num_prefix_groups] : 0;
  return finish_plan(p, stable ? &caps : nullptr, ws_dev, ws_dev_bytes, ws_host, ws_host_bytes,
                     stream, out);
}

extern "C" fi_status fi_plan_block_sparse_batch(
    const fi_plan_desc* desc, int32_t num_seqs, const int32_t* qo_len_h, const int32_t* kv_len_h,
    const int32_t* num_row_blocks_h, const int32_t* row_block_sz_h,
    const int32_t* num_col_blocks_h, const int32_t* col_block_sz_h, const uint8_t* block_mask_h,
    const int32_t* kv_indptr_h, const int32_t* kv_indices_h, void* ws_dev, size_t ws_dev_bytes,
    void* ws_host, size_t ws_host_bytes, void* stream, fi_plan_t** out) {
  clear_error();
  if (!out) return set_error(FI_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  fi_plan_desc d;
  fi_status st = begin_plan(desc, ws_dev, ws_host, d);
  if (st != FI_OK) return st;
  if (d.kind != FI_KIND_BLOCK_SPARSE)
    return set_error(FI_ERR_INVALID_ARG, "fi_plan_block_sparse needs kind FI_KIND_BLOCK_SPARSE");
  BsBatch bb;
  bb.S = num_seqs;
  bb.qo_len = qo_len_h;
  bb.kv_len = kv_len_h;
  bb.nrb = num_row_blocks_h;
  bb.ncb = num_col_blocks_h;
  bb.row_sz = row_block_sz_h;
  bb.col_sz = col_block_sz_h;
  bb.mask = block_mask_h;
  bb.kv_indptr = kv_indptr_h;
  bb.kv_indices = d.kv_layout == FI_KV_LAYOUT_RAGGED ? nullptr : kv_indices_h;
  st = check_bs_batch(d, bb);
  if (st != FI_OK) return st;
  fi_plan_t* p = new fi_plan_t();
  p->hp.desc = d;
  st = build_block_sparse(d, bb, p->hp);
  if (st != FI_OK) {
    delete p;
    return st;
  }
  return finish_plan(p, nullptr, ws_dev, ws_dev_bytes, ws_host, ws_host_bytes, stream, out);
}

extern "C" fi_status fi_plan_block_sparse(const fi_plan_desc* desc, int32_t qo_len,
                                          int32_t kv_len, int32_t num_row_blocks,
                                          const int32_t* row_block_sz_h, int32_t num_col_blocks,
                                          const int32_t* col_block_sz_h,
                                          const uint8_t* block_mask_h,
                                          const int32_t* seq_pages_h, void* ws_dev,
                                          size_t ws_dev_bytes, void* ws_host,
                                          size_t ws_host_bytes, void* stream, fi_plan_t** out) {
  clear_error();
  if (desc && desc->kv_layout != FI_KV_LAYOUT_PAGED)
    return set_error(FI_ERR_INVALID_ARG,
                     "fi_plan_block_sparse reads a paged sequence (ragged: the batch call)");
  if (kv_len < 0 || qo_len < 0)
    return set_error(FI_ERR_INVALID_ARG, "negative block-sparse size");
  const int32_t ps = desc ? desc->page_size : 0;
  const int32_t indptr[2] = {0, ps > 0 ? (kv_len + ps - 1) / ps : 0};
  return fi_plan_block_sparse_batch(desc, 1, &qo_len, &kv_len, &num_row_blocks, row_block_sz_h,
                                    &num_col_blocks, col_block_sz_h, block_mask_h, indptr,
                                    seq_pages_h, ws_dev, ws_dev_bytes, ws_host, ws_host_bytes,
                                    stream, out);
}

extern "C" void fi_plan_destroy(fi_plan_t* plan) { delete plan; }

extern "C" fi_status fi_plan_get_info(const fi_plan_t* p, fi_plan_info* info) {
  clear_error();
  if (!p || !info) return set_error(FI_ERR_INVALID_ARG, "NULL plan or info");
  memset(info, 0, sizeof(*info));
  const HostPlan& hp = p->hp;
  info->kind = hp.desc.kind;
  info->num_levels = hp.num_levels;
  for (int l = 0; l < 2; ++l) {
    info->num_workers[l] = hp.level[l].num_workers;
    info->min_chunk_pages[l] = hp.level[l].min_chunk_pages;
    info->rows_per_block[l] = hp.level[l].rows_per_block;
    info->chunk_pages[l] = hp.level[l].chunk_pages;
    info->num_items[l] = hp.level[l].num_items();
    info->items[l] = hp.level[l].items.data();
    info->worker_indptr[l] = hp.level[l].worker_indptr.data();
  }
  info->num_merges = (int32_t)(hp.merges.size() / MERGE_INTS);
  info->merges = hp.merges.data();
  info->num_parts = (int32_t)hp.parts.size();
  info->parts = hp.parts.data();
  info->num_qlist = (int32_t)hp.qlist.size();
  info->qlist = hp.qlist.data();
  info->num_part_rows = hp.num_part_rows;
  info->num_scatter = (int32_t)(hp.scatter.size() / 2);
  info->dev_bytes_used = p->lay.dev_bytes;
  info->host_bytes_used = p->lay.blob_bytes;
  info->pod_wide_blocks = hp.pod ? hp.pod_wide_blocks : 0;
  info->num_plist = (int32_t)hp.plist.size();
  info->plist = hp.plist.data();
  info->fused_merge = hp.fused ? 1 : 0;
  info->wg_fold = hp.wg_fold ? 1 : 0;
  info->item_rec = hp.item_rec.data();
  info->num_empty_recs = (int32_t)hp.empty_recs.size();
  info->empty_recs = hp.empty_recs.data();
  return FI_OK;
}

extern "C" const char* fi_last_error(void) { return fi::g_last_error.c_str(); }
