// fi_device.h -- device helpers shared by the attention kernels: plan-record
// reads, bf16 packing, the gfx950 bf16 MFMA, and per-head-dim constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_internal.h"

namespace fi {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309417f;
// The base m that P is taken against only moves when a row's max exceeds it by
// more than this (log2 units): p <= 2^8 stays exact enough in fp32 and bf16,
// and O and l, both relative to the same m, then need no rescale.
constexpr float kRescaleSlack = 8.f;

template <int W> struct RowVec;
template <> struct RowVec<4> { typedef u32x4 T; };
template <> struct RowVec<2> { typedef u32x2 T; };

template <int D>
struct Cfg {
  static constexpr int KJ = D / 32;    // 32-dim k-slices of the q.K contraction
  static constexpr int DPL = D / 16;   // V dims per lane = P.V MFMAs per step
  static constexpr int CH = D / 8;     // 16-byte chunks per K/V row
  typedef typename RowVec<DPL / 2>::T vrow_t;
};

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Two fp32 -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Plan records and page tables are never written while a kernel runs; reading
// them through the constant address space lets wave-uniform reads become
// scalar loads, which do not queue behind in-flight vector loads.
typedef const __attribute__((address_space(4))) int32_t* const_i32p;
__device__ __forceinline__ int ld_uniform(const int32_t* p, int64_t i) {
  return uniform(((const_i32p)p)[i]);
}

// Partial rows that the fused merge folds in another workgroup, which may run
// on another XCD (each XCD has its own L2), are stored and loaded with
// agent-scope atomic accesses. Those are coherent at that scope by themselves
// (gfx950 marks them sc1), so announcing them needs only this wave's own
// stores to have completed -- not a write-back of the whole L2, which an
// agent-scope release fence performs -- and the folding wave needs no L2
// invalidate before it reads them.
__device__ __forceinline__ void st_agent(float* p, f32x4 v) {
  __hip_atomic_store((uint64_t*)p, __builtin_bit_cast(uint64_t, f32x2{v[0], v[1]}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store((uint64_t*)p + 1, __builtin_bit_cast(uint64_t, f32x2{v[2], v[3]}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 ld_agent2(const float* p) {
  return __builtin_bit_cast(f32x2, __hip_atomic_load((uint64_t*)const_cast<float*>(p),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Work item fields, all wave-uniform.
struct Item {
  int q_base, row0, n_rows, g, flags, t_begin, t_end, q_pos0, dst, nsteps;
  const int32_t* plist;
};

__device__ __forceinline__ Item load_item(const AttnArgs& a, int i) {
  const int32_t* it = a.items + (int64_t)i * ITEM_INTS;
  Item r;
  r.q_base = ld_uniform(it, F_Q_BASE);
  r.row0 = ld_uniform(it, F_ROW0);
  r.n_rows = ld_uniform(it, F_NROWS);
  r.g = ld_uniform(it, F_KVHEAD);
  r.flags = ld_uniform(it, F_FLAGS);
  r.t_begin = ld_uniform(it, F_TBEGIN);
  r.t_end = ld_uniform(it, F_TEND);
  r.q_pos0 = ld_uniform(it, F_QPOS0);
  r.dst = ld_uniform(it, F_DST);
  r.nsteps = (r.t_end - r.t_begin + 31) >> 5;
  r.plist = ((r.flags & FLAG_PREFIX) ? a.prefix_indices : a.kv_indices) +
            ld_uniform(it, F_PAGEOFF);
  return r;
}

// Online-softmax state of MB 16-row blocks: O^T accumulators (query row in
// lane%16), running base m and per-lane partial row sums l.
template <int D, int MB>
struct State {
  f32x4 acc[MB][Cfg<D>::DPL];
  float m[MB], l[MB];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      m[mb] = neg_inf();
      l[mb] = 0.f;
#pragma unroll
      for (int d = 0; d < Cfg<D>::DPL; ++d) acc[mb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// Max over the four 16-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_across_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

// Softmax update and P.V for one 16-row block and one 32-token step, given
// its S^T accumulators s0 (tokens 0..15) and s1 (16..31) and the V^T operands.
// scale_log2 = sm_scale * log2(e) must be > 0 (the run calls check sm_scale);
// p = 2^(s * scale_log2 - m) is one fma and one exp per logit.
// T0: first token of the step; lim: last token visible to this lane's row
// (only read when `masked`).
template <int D, int MB>
__device__ __forceinline__ void softmax_pv(State<D, MB>& st, int mb, f32x4 s0, f32x4 s1,
                                           const u32x4 (&vt)[Cfg<D>::DPL], float scale_log2,
                                           bool masked, int T0, int lim, int grp) {
  constexpr int DPL = Cfg<D>::DPL;
  // raw logits; scale_log2 > 0, so their max is the max of the scaled ones
  float x[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = s0[r];
    x[4 + r] = s1[r];
  }
  if (masked) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t0 = T0 + 4 * grp + r;
      if (t0 > lim) x[r] = neg_inf();
      if (t0 + 16 > lim) x[4 + r] = neg_inf();
    }
  }
  // The base m (equal in the four lane groups of a row) only moves when some
  // logit of the row exceeds it by more than the slack. A wave-wide vote on
  // the lane-local max gates the cross-lane exchange, so the common step
  // needs none; inside, each row decides from its own max alone, so a row's
  // base -- and with it the rounding of its p, l and O -- never depends on
  // the other rows of the block (which may belong to other requests, as on a
  // shared prefix).
  const float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))) * scale_log2;
  if (__any(mx > st.m[mb] + kRescaleSlack)) {
    const float rmax = max_across_groups(mx);
    if (rmax > st.m[mb] + kRescaleSlack) {
      const float m_new = rmax;   // > m, finite or +inf only if a logit is
      const float alpha = (st.m[mb] == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(st.m[mb] - m_new);
      st.l[mb] *= alpha;
#pragma unroll
      for (int m = 0; m < DPL; ++m) st.acc[mb][m] *= alpha;
      st.m[mb] = m_new;
    }
  }
  const float nbase = (st.m[mb] == neg_inf()) ? 0.f : -st.m[mb];
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], scale_log2, nbase));
  st.l[mb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  const u32x4 pb = {pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7])};
#pragma unroll
  for (int m = 0; m < DPL; ++m) st.acc[mb][m] = mfma_bf16(vt[m], pb, st.acc[mb][m]);
}

// V^T operands from 8 V rows (the lane's tokens 4g..4g+3, 16+4g..16+4g+3):
// for MFMA m, the lane supplies dim DPL*col+m of its 8 tokens.
template <int D>
__device__ __forceinline__ void transpose_v(const typename Cfg<D>::vrow_t (&vv)[8],
                                            u32x4 (&vt)[Cfg<D>::DPL]) {
#pragma unroll
  for (int m = 0; m < Cfg<D>::DPL; ++m) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t lo = vv[2 * jj][m >> 1], hi = vv[2 * jj + 1][m >> 1];
      vt[m][jj] = __builtin_amdgcn_perm(hi, lo, (m & 1) ? 0x07060302u : 0x05040100u);
    }
  }
}

// Partial states of a workgroup-folded unit (a tiny batch's plan: unit u on
// the four waves of workgroup u, chunk j on wave j) can stay in LDS: wave j
// writes its 16 rows to slot j, rows padded by eight floats against bank
// conflicts (and 32-byte aligned for the fold's row reads), then the lse of
// the four slots. The launch sizes the dynamic LDS with BYTES.
template <int D>
struct FoldLds {
  static constexpr int ROW = D + 8;                 // floats per row
  static constexpr int LSE = WAVES_PER_BLOCK * 16 * ROW;   // float offset of the lse
  static constexpr int BYTES = (LSE + WAVES_PER_BLOCK * 16) * 4;
};

// o = acc / l and lse = (m + log2 l) ln 2 for MB row blocks, to the final
// output or to fp32 partial rows (in LDS slot `wave` when fold is given and
// the plan folds in the workgroup). Rows at or past n_rows are not written.
template <int D, int MB, bool LQ>
__device__ __forceinline__ void finalize_rows(const AttnArgs& a, const Item& it,
                                              const State<D, MB>& st, int rl0, int col,
                                              int grp, float* fold = nullptr) {
  constexpr int DPL = Cfg<D>::DPL;
  typedef typename Cfg<D>::vrow_t vrow_t;
  const int G = a.group;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float lt = st.l[mb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int rl = rl0 + mb * 16 + col;
    if (rl >= it.n_rows) continue;
    const bool live = lt > 0.f;
    const float inv = live ? 1.f / lt : 0.f;
    const float lse_v = live ? (st.m[mb] + log2f(lt)) * kLn2 : neg_inf();
    if ((it.flags & FLAG_PARTIAL) && fold && a.wg_fold) {
      const int slot = uniform(threadIdx.x >> 6) * 16 + rl;
      float* op = fold + slot * FoldLds<D>::ROW;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* d0 = op + DPL * (4 * grp + r);
#pragma unroll
        for (int m = 0; m < DPL; m += 4)
          *(f32x4*)(d0 + m) = f32x4{st.acc[mb][m][r] * inv, st.acc[mb][m + 1][r] * inv,
                                    st.acc[mb][m + 2][r] * inv, st.acc[mb][m + 3][r] * inv};
      }
      if (grp == 0) fold[FoldLds<D>::LSE + slot] = lse_v;
    } else if (it.flags & FLAG_PARTIAL) {
      float* op = a.part_o + (int64_t)(it.dst + rl) * D;
      // rows folded by the fused merge across workgroups: agent-scope stores
      const bool scoped = a.item_rec != nullptr && !a.wg_fold;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* d0 = op + DPL * (4 * grp + r);
#pragma unroll
        for (int m = 0; m < DPL; m += 4) {
          f32x4 v = {st.acc[mb][m][r] * inv, st.acc[mb][m + 1][r] * inv,
                     st.acc[mb][m + 2][r] * inv, st.acc[mb][m + 3][r] * inv};
          if (scoped) st_agent(d0 + m, v);
          else *(f32x4*)(d0 + m) = v;
        }
      }
      if (grp == 0) {
        if (scoped) st_agent(a.part_lse + it.dst + rl, lse_v);
        else a.part_lse[it.dst + rl] = lse_v;
      }
    } else {
      const int rho = it.row0 + rl;
      const int qi = rho / G, h = rho - qi * G;
      const int tok = LQ ? a.qlist[it.q_base + qi] : it.q_base + qi;
      const int64_t orow = (int64_t)tok * a.num_qo_heads + it.g * G + h;
      uint16_t* op = a.o + orow * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vrow_t v;
#pragma unroll
        for (int m = 0; m < DPL; m += 2)
          v[m >> 1] = pack2(st.acc[mb][m][r] * inv, st.acc[mb][m + 1][r] * inv);
        *(vrow_t*)(op + DPL * (4 * grp + r)) = v;
      }
      if (grp == 0 && a.lse) a.lse[orow] = lse_v;
    }
  }
}

// Q rows rl0 + 16*mb + col of an item (B operand of the q.K MFMAs). Rows past
// n_rows (tile padding) read the item's first row: their results are never
// stored and MFMA rows do not mix.
template <int D, int MB, bool LQ>
__device__ __forceinline__ void load_q_rows(const AttnArgs& a, const Item& it, int rl0,
                                            u32x4 (&qf)[MB][Cfg<D>::KJ], int col, int grp) {
  const int G = a.group;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int rl = rl0 + mb * 16 + col < it.n_rows ? rl0 + mb * 16 + col : 0;
    const int rho = it.row0 + rl;
    const int qi = rho / G, h = rho - qi * G;
    const int tok = LQ ? a.qlist[it.q_base + qi] : it.q_base + qi;
    const uint16_t* qp = a.q + ((int64_t)tok * a.num_qo_heads + it.g * G + h) * D + grp * 8;
#pragma unroll
    for (int j = 0; j < Cfg<D>::KJ; ++j) qf[mb][j] = *(const u32x4*)(qp + 32 * j);
  }
}

// ---------------------------------------------------------------- fused merge

// Per element of a merge: acc = fma(w, v, acc), z = z + w, in part order;
// o = acc * (1 / z), lse = M + ln z (M the parts' max lse). The merge kernel
// (fi_merge.hip) and the fused fold below run exactly these operations, so a
// row's bits do not depend on which of them merged it.

template <bool SCOPED>
__device__ __forceinline__ float lse_at(const AttnArgs& a, int64_t i) {
  return SCOPED ? ld_agent(a.part_lse + i) : a.part_lse[i];
}

// FPL = D / 16 consecutive floats of row k of LDS slot j (FoldLds), from
// column col.
template <int D>
__device__ __forceinline__ auto lds_row(const float* fold, int j, int k, int col) {
  constexpr int FPL = D / 16;
  typedef float vec __attribute__((ext_vector_type(FPL)));
  return *(const vec*)(fold + (j * 16 + k) * FoldLds<D>::ROW + col);
}

// FPL = D / 16 consecutive floats of partial row pr, from column col.
template <int D, bool SCOPED>
__device__ __forceinline__ auto part_row(const AttnArgs& a, int pr, int col) {
  constexpr int FPL = D / 16;
  typedef float vec __attribute__((ext_vector_type(FPL)));
  const float* src = a.part_o + (int64_t)pr * D + col;
  vec v;
  if (SCOPED) {
#pragma unroll
    for (int i = 0; i < FPL; i += 2) {
      const f32x2 x = ld_agent2(src + i);
      v[i] = x[0];
      v[i + 1] = x[1];
    }
  } else {
    v = *(const vec*)src;
  }
  return v;
}

// Fold merge record e into the final rows (16 lanes per row, four rows per
// pass): row k < n_rows of the record is unit row row0 + k, query q_base +
// (row0 + k) / G, head kv_head * G + (row0 + k) % G; its parts are partial
// rows parts[off + j] + k, j = 0..n-1 -- or, with fold given, row k of LDS
// slot j (a workgroup-folded unit: part j is chunk j, on wave j). With n = 0
// the rows get o = 0, lse = -inf.
template <int D, bool SCOPED>
__device__ __forceinline__ void fold_record(const AttnArgs& a, int e, int lane,
                                            const float* fold = nullptr) {
  constexpr int FPL = D / 16;   // outputs per lane
  constexpr int kBatch = 4;     // parts loaded together
  typedef float vec __attribute__((ext_vector_type(FPL)));
  typedef uint32_t packed __attribute__((ext_vector_type(FPL / 2)));
  const int32_t* m = a.merges + (int64_t)e * MERGE_INTS;
  const int q_base = ld_uniform(m, M_QBASE), row0 = ld_uniform(m, M_ROW0);
  const int nh = ld_uniform(m, M_NROWS), kv_head = ld_uniform(m, M_KVHEAD);
  const int off = ld_uniform(m, M_OFF), n = ld_uniform(m, M_N);
  const int G = a.group;
  const int col = (lane & 15) * FPL;
  for (int h0 = 0; h0 < nh; h0 += 4) {
    const int row = h0 + (lane >> 4);
    const int rowc = row < nh ? row : h0;     // lanes past the rows load a real row
    float M = neg_inf();
    float z = 0.f;
    vec acc = vec{};
    if (n <= 2 * kBatch) {
      // every part in one round of loads (the common case; a fold at the end
      // of the attention kernel sits on its critical path): the same max and
      // the same multiply-adds, in the same order, as the two passes below
      float l[2 * kBatch];
      vec v[2 * kBatch];
#pragma unroll
      for (int u = 0; u < 2 * kBatch; ++u) {
        l[u] = neg_inf();
        if (u < n && fold) {
          if (u < WAVES_PER_BLOCK) {   // (one slot per wave; a folded unit has at most four parts)
            l[u] = fold[FoldLds<D>::LSE + u * 16 + rowc];
            v[u] = lds_row<D>(fold, u, rowc, col);
          }
        } else if (u < n) {
          const int pr = ld_uniform(a.parts, off + u) + rowc;
          l[u] = lse_at<SCOPED>(a, pr);
          v[u] = part_row<D, SCOPED>(a, pr, col);
        }
      }
#pragma unroll
      for (int u = 0; u < 2 * kBatch; ++u) M = fmaxf(M, l[u]);
#pragma unroll
      for (int u = 0; u < 2 * kBatch; ++u) {
        if (u < n) {
          const float w = (l[u] == neg_inf()) ? 0.f : expf(l[u] - M);
          z += w;
#pragma unroll
          for (int i = 0; i < FPL; ++i) acc[i] = __builtin_fmaf(w, v[u][i], acc[i]);
        }
      }
    }
    for (int j0 = 0; j0 < n && n > 2 * kBatch; j0 += 2 * kBatch) {
      float l[2 * kBatch];
#pragma unroll
      for (int u = 0; u < 2 * kBatch; ++u)
        l[u] = j0 + u < n ? lse_at<SCOPED>(a, ld_uniform(a.parts, off + j0 + u) + rowc) : neg_inf();
#pragma unroll
      for (int u = 0; u < 2 * kBatch; ++u) M = fmaxf(M, l[u]);
    }
    for (int j0 = 0; j0 < n && n > 2 * kBatch; j0 += kBatch) {
      float l[kBatch];
      vec v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j0 + u < n) {
          const int pr = ld_uniform(a.parts, off + j0 + u) + rowc;
          l[u] = lse_at<SCOPED>(a, pr);
          v[u] = part_row<D, SCOPED>(a, pr, col);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j0 + u < n) {
          const float w = (l[u] == neg_inf()) ? 0.f : expf(l[u] - M);
          z += w;
#pragma unroll
          for (int i = 0; i < FPL; ++i) acc[i] = __builtin_fmaf(w, v[u][i], acc[i]);
        }
      }
    }
    if (row >= nh) continue;
    const float inv = z > 0.f ? 1.f / z : 0.f;
    const int rho = row0 + row;
    const int64_t orow = (int64_t)(q_base + rho / G) * a.num_qo_heads + kv_head * G + rho % G;
    packed pk;
#pragma unroll
    for (int i = 0; i < FPL / 2; ++i) pk[i] = pack2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
    *(packed*)(a.o + orow * D + col) = pk;
    if ((lane & 15) == 0 && a.lse) a.lse[orow] = z > 0.f ? M + logf(z) : neg_inf();
  }
}

// At a worker's start: write the records of units with no keys (n_empty of
// them, the plan's META_EMPTY), spread over the workers.
template <int D>
__device__ __forceinline__ void fused_merge_start(const AttnArgs& a, int w, int lane,
                                                  int n_empty) {
  if (!a.item_rec) return;
  for (int k = w; k < n_empty; k += a.num_workers) fold_record<D, false>(a, ld_uniform(a.empty_recs, k), lane);
}
template <int D>
__device__ __forceinline__ void fused_merge_start(const AttnArgs& a, int w, int lane) {
  if (!a.item_rec) return;
  fused_merge_start<D>(a, w, lane, ld_uniform(a.meta, META_EMPTY));
}

// At the end of a worker's stream (so that the wait below, for every load and
// store of the wave, drains no prefetch): count in each of its
// partial items at the item's record -- one lane per item, all at once -- and
// fold every record this wave completed.
//
// A tiny batch's plan (wg_fold) puts each unit on the four waves of one
// workgroup, one chunk per wave: every wave of the workgroup comes here once
// (those with no item too), its partial rows (in LDS when fold is given,
// else in the workspace) become visible to the workgroup, and after the
// barrier the wave holding chunk 0 folds the unit's record (at most four
// parts) -- no agent-scope fence and no count.
template <int D>
__device__ __forceinline__ void fused_merge_end(const AttnArgs& a, int i_begin, int i_end,
                                                int lane, const float* fold = nullptr) {
  if (!a.item_rec) return;
  if (a.wg_fold) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (i_begin < i_end) {
      const int rec = ld_uniform(a.item_rec, i_begin);
      if (rec >= 0 && ld_uniform(a.items, (int64_t)i_begin * ITEM_INTS + F_CHUNK) == 0)
        fold_record<D, false>(a, rec, lane, fold);
    }
    return;
  }
  // waves whose items all wrote final rows have nothing to announce (and
  // skip the wait)
  bool any = false;
  for (int i0 = i_begin; i0 < i_end && !any; i0 += 64)
    any = __ballot(i0 + lane < i_end && a.item_rec[i0 + lane] >= 0) != 0;
  if (!any) return;
  // the partial rows written by this wave (agent-scope stores) have completed,
  // so they are visible at agent scope -- to a folding wave on another XCD --
  // before any count that announces them
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0), expcnt and lgkmcnt untouched
  asm volatile("" ::: "memory");
  for (int i0 = i_begin; i0 < i_end; i0 += 64) {
    const int i = i0 + lane;
    int rec = -1;
    bool last = false;
    if (i < i_end) {
      rec = a.item_rec[i];
      if (rec >= 0) {
        const int n = a.merges[(int64_t)rec * MERGE_INTS + M_N];
        const int before =
            __hip_atomic_fetch_add(a.counters + rec, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = before == n - 1;
        // every chunk of the record has counted in: reset for the next call
        if (last) __hip_atomic_store(a.counters + rec, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    uint64_t done = __ballot(last);
    if (done) {
      // the other chunks' partial rows completed before their counts, and the
      // fold reads them with agent-scope loads, issued after the counts came
      // back
      asm volatile("" ::: "memory");
      while (done) {
        const int l = __builtin_ctzll(done);
        done &= done - 1;
        fold_record<D, true>(a, __builtin_amdgcn_readlane(rec, l), lane);
      }
    }
  }
}

}  // namespace dev
}  // namespace fi
