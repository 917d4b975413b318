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
  // logit exceeds it by more than the slack; the lane-local max decides that,
  // and only then is the row max taken across the groups, so the common step
  // needs no cross-lane exchange.
  const float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))) * scale_log2;
  if (__any(mx > st.m[mb] + kRescaleSlack)) {
    const float m_new = fmaxf(st.m[mb], max_across_groups(mx));
    const float alpha = (m_new == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(st.m[mb] - m_new);
    st.l[mb] *= alpha;
#pragma unroll
    for (int m = 0; m < DPL; ++m) st.acc[mb][m] *= alpha;
    st.m[mb] = m_new;
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

// o = acc / l and lse = (m + log2 l) ln 2 for MB row blocks, to the final
// output or to fp32 partial rows. Rows at or past n_rows are not written.
template <int D, int MB, bool LQ>
__device__ __forceinline__ void finalize_rows(const AttnArgs& a, const Item& it,
                                              const State<D, MB>& st, int rl0, int col,
                                              int grp) {
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
    if (it.flags & FLAG_PARTIAL) {
      float* op = a.part_o + (int64_t)(it.dst + rl) * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* d0 = op + DPL * (4 * grp + r);
#pragma unroll
        for (int m = 0; m < DPL; m += 4) {
          f32x4 v = {st.acc[mb][m][r] * inv, st.acc[mb][m + 1][r] * inv,
                     st.acc[mb][m + 2][r] * inv, st.acc[mb][m + 3][r] * inv};
          *(f32x4*)(d0 + m) = v;
        }
      }
      if (grp == 0) a.part_lse[it.dst + rl] = lse_v;
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

}  // namespace dev
}  // namespace fi
