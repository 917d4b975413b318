// fi_attention.hip -- paged attention work-item kernel for gfx950 (CDNA4).
//
// Computes, for each planned work item, exact softmax attention of up to
// 16*MB query rows (query token i, q head h of kv head g) over the item's
// token range of one sequence, reading K/V through the block table (research
// note "flashinfer-backend-selection", "Arithmetic intensity": decode reads a
// gathered block table instead of a dense cache). Each wavefront is one
// persistent worker that runs the items the plan gave it, in order, as one
// continuous stream of 32-token steps: the loads of step n+1 (possibly the
// first step of the next item) are in flight while step n is computed.
//
// Tiling. Both contractions run on the bf16 MFMA v_mfma_f32_16x16x32_bf16 with
// fp32 accumulation:
//   S^T[token][row] = K[token][:] . Q[row][:]    A = K tile, B = Q^T
//   O^T[d][row]    += V^T[d][token] . P^T[token][row]
// With both outputs transposed, the query row sits in lane%16 of every
// accumulator, so the softmax statistics and the rescale of O stay in-lane;
// only the row max and the final row sum cross the four 16-lane groups.
// Lane l loads K of token 16*blk + l%16 (4 lanes read 64 contiguous bytes of a
// row) and V of 8 tokens (16 lanes read a full 256-byte row per instruction).
// The V rows are transposed in registers with v_perm_b32 into the MFMA A
// layout; the token order inside a lane group (4g..4g+3, 16+4g..16+4g+3) is the
// one the S^T accumulator hands to P, so P needs no shuffle.
//
// Pages. NP = pages one 32-token step touches (4 for page size 8, 2 for 16, 1
// for >= 32). The step's page ids are wave-uniform scalars; which of them a
// lane's token uses is fixed at compile time up to one lane bit, so every
// load is a uniform 64-bit page-tile base plus a 32-bit lane offset. Pages
// past the item's last page are clamped to it, so every address is valid and
// the loads are unconditional; V of tokens past the end is zeroed by a
// select, and their logits are masked to -inf.
//
// Softmax is online (running max m, running sum l, O rescaled by
// exp2(m_old - m_new)) with logits pre-scaled by sm_scale*log2(e); the LSE is
// returned in natural log. P is rounded to bf16 for the P.V MFMA; l sums the
// fp32 P. Under the causal mask a key after a query's position gets -inf.

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "fi_internal.h"

namespace fi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kRescaleSlack = 8.f;

template <int W> struct RowVec;
template <> struct RowVec<4> { typedef u32x4 T; };
template <> struct RowVec<2> { typedef u32x2 T; };

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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
// scalar loads, which do not queue behind the in-flight K/V vector loads.
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
  r.plist = ((r.flags & FLAG_PREFIX) ? a.prefix_indices : a.kv_indices) + ld_uniform(it, F_PAGEOFF);
  return r;
}

template <int D>
struct Cfg {
  static constexpr int KJ = D / 32;    // 32-dim k-slices of the q.K contraction
  static constexpr int DPL = D / 16;   // V dims per lane = P.V MFMAs per step
  typedef typename RowVec<DPL / 2>::T vrow_t;
};

// One step's registers: K and V of 32 tokens, and (first step of an item
// only) the item's Q.
template <int D, int MB>
struct Tile {
  u32x4 k[2][Cfg<D>::KJ];
  typename Cfg<D>::vrow_t v[8];
  u32x4 q[MB][Cfg<D>::KJ];
};

// Issue the loads of step s of item it into T.
template <int D, int MB, int NP>
__device__ __forceinline__ void issue_step(const AttnArgs& a, const Item& it, int s,
                                           Tile<D, MB>& T, int col, int grp) {
  constexpr int KJ = Cfg<D>::KJ, DPL = Cfg<D>::DPL;
  typedef typename Cfg<D>::vrow_t vrow_t;
  const int sh = a.page_shift;
  const int T0 = it.t_begin + 32 * s;
  const int pb = T0 >> sh;
  const int plast = (it.t_end - 1) >> sh;
  const int64_t tile_elems = (int64_t)a.page_size * D;
  const char* kb[NP];
  const char* vb[NP];
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    const int pid = ld_uniform(it.plist, min(pb + n, plast));
    const int64_t off = ((int64_t)pid * a.num_kv_heads + it.g) * tile_elems * 2;
    kb[n] = (const char*)a.k_cache + off;
    vb[n] = (const char*)a.v_cache + off;
  }
  const int slot0 = (NP == 1) ? (T0 & (a.page_size - 1)) : 0;
  // K: token 16*blk + col
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const char* base;
    int slot;
    if (NP == 1) {
      base = kb[0];
      slot = slot0 + 16 * blk + col;
    } else if (NP == 2) {
      base = kb[blk];
      slot = col;
    } else {
      base = (col >> 3) ? kb[2 * blk + 1] : kb[2 * blk];
      slot = col & 7;
    }
    const uint32_t off = (uint32_t)(slot * D + grp * 8) * 2u;
#pragma unroll
    for (int j = 0; j < KJ; ++j) T.k[blk][j] = *(const u32x4*)(base + off + 64u * j);
  }
  // V: tokens 4*grp + i (i < 4) and 16 + 4*grp + (i - 4) (i >= 4)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tl = (i < 4) ? 4 * grp + i : 16 + 4 * grp + (i - 4);
    const char* base;
    int slot;
    if (NP == 1) {
      base = vb[0];
      slot = slot0 + tl;
    } else if (NP == 2) {
      base = vb[i >> 2];
      slot = tl & 15;
    } else {
      base = (grp >> 1) ? vb[2 * (i >> 2) + 1] : vb[2 * (i >> 2)];
      slot = tl & 7;
    }
    const uint32_t off = (uint32_t)(slot * D + DPL * col) * 2u;
    T.v[i] = *(const vrow_t*)(base + off);
  }
}

template <int D, int MB, bool LQ>
__device__ __forceinline__ void load_q(const AttnArgs& a, const Item& it, u32x4 (&qf)[MB][Cfg<D>::KJ],
                                       int col, int grp) {
  const int G = a.group;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    // Rows past n_rows (tile padding) read the item's first row: their
    // results are never stored and MFMA rows do not mix.
    const int rl = mb * 16 + col < it.n_rows ? mb * 16 + col : 0;
    const int rho = it.row0 + rl;
    const int qi = rho / G, h = rho - qi * G;
    const int tok = LQ ? a.qlist[it.q_base + qi] : it.q_base + qi;
    const uint16_t* qp = a.q + ((int64_t)tok * a.num_qo_heads + it.g * G + h) * D + grp * 8;
#pragma unroll
    for (int j = 0; j < Cfg<D>::KJ; ++j) qf[mb][j] = *(const u32x4*)(qp + 32 * j);
  }
}

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

template <int D, int MB>
__device__ __forceinline__ void compute_step(const AttnArgs& a, const Item& it, int s,
                                             const Tile<D, MB>& T,
                                             const u32x4 (&qf)[MB][Cfg<D>::KJ],
                                             State<D, MB>& st, int col, int grp) {
  constexpr int KJ = Cfg<D>::KJ, DPL = Cfg<D>::DPL;
  typedef typename Cfg<D>::vrow_t vrow_t;
  const int T0 = it.t_begin + 32 * s;
  const bool causal = (it.flags & FLAG_CAUSAL) != 0;
  // V rows of tokens past the item's end hold whatever the clamped page has
  // there (even NaN): zero them so that p = 0 cancels them exactly.
  vrow_t vv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) vv[i] = T.v[i];
  if (T0 + 32 > it.t_end) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tl = (i < 4) ? 4 * grp + i : 16 + 4 * grp + (i - 4);
      if (T0 + tl >= it.t_end) vv[i] = vrow_t{};
    }
  }
  // V^T operands: for MFMA m, the lane supplies dim DPL*col+m of its 8 tokens.
  u32x4 vt[DPL];
#pragma unroll
  for (int m = 0; m < DPL; ++m) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t lo = vv[2 * jj][m >> 1], hi = vv[2 * jj + 1][m >> 1];
      vt[m][jj] = __builtin_amdgcn_perm(hi, lo, (m & 1) ? 0x07060302u : 0x05040100u);
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      s0 = mfma_bf16(T.k[0][j], qf[mb][j], s0);
      s1 = mfma_bf16(T.k[1][j], qf[mb][j], s1);
    }
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = s0[r] * a.scale_log2;
      x[4 + r] = s1[r] * a.scale_log2;
    }
    if (T0 + 32 > it.t_end || causal) {
      // last visible token for this lane's row
      int lim = it.t_end - 1;
      if (causal) lim = min(lim, it.q_pos0 + (it.row0 + mb * 16 + col) / a.group);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t0 = T0 + 4 * grp + r;
        if (t0 > lim) x[r] = neg_inf();
        if (t0 + 16 > lim) x[4 + r] = neg_inf();
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // The base m that P is taken against only moves when a row's max exceeds
    // it by more than kRescaleSlack (log2 units): until then p <= 2^slack,
    // which fp32 and bf16 hold exactly as well, and O and l (both relative to
    // the same m) need no rescale. The result is the same exact quotient.
    if (__any(mx > st.m[mb] + kRescaleSlack)) {
      const float m_new = fmaxf(st.m[mb], mx);
      const float alpha =
          (m_new == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(st.m[mb] - m_new);
      st.l[mb] *= alpha;
#pragma unroll
      for (int m = 0; m < DPL; ++m) st.acc[mb][m] *= alpha;
      st.m[mb] = m_new;
    }
    const float base = (st.m[mb] == neg_inf()) ? 0.f : st.m[mb];
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - base);
    st.l[mb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    const u32x4 pb = {pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7])};
#pragma unroll
    for (int m = 0; m < DPL; ++m) st.acc[mb][m] = mfma_bf16(vt[m], pb, st.acc[mb][m]);
  }
}

template <int D, int MB, bool LQ>
__device__ __forceinline__ void finalize(const AttnArgs& a, const Item& it, const State<D, MB>& st,
                                         int col, int grp) {
  constexpr int DPL = Cfg<D>::DPL;
  typedef typename Cfg<D>::vrow_t vrow_t;
  const int G = a.group;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float lt = st.l[mb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int rl = mb * 16 + col;
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

// Tiles in the ring: R-1 steps are in flight while one is computed.
template <int MB> struct Ring { static constexpr int R = MB == 1 ? 4 : 2; };

// LQ: query rows come through the member list (cascade prefix level only).
template <int D, int MB, int NP, bool LQ>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs a) {
  constexpr int KJ = Cfg<D>::KJ;
  constexpr int R = Ring<MB>::R;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int w = blockIdx.x * WAVES_PER_BLOCK + uniform(threadIdx.x >> 6);
  if (w >= a.num_workers) return;
  const int i_end = ld_uniform(a.worker_indptr, w + 1);
  const int i_begin = ld_uniform(a.worker_indptr, w);
  if (i_begin >= i_end) return;

  // Two cursors over the worker's stream of steps: the issue cursor (ii, is)
  // runs R-1 steps ahead of the compute cursor (ci, cs), across item
  // boundaries. Tiles are filled and consumed in the same order.
  int ci = i_begin, cs = 0;
  Item citem = load_item(a, ci);
  int ii = i_begin, is = 0;
  Item iitem = citem;
  Tile<D, MB> T[R];
  u32x4 q_cur[MB][KJ];
  State<D, MB> st;
  st.reset();

  auto issue = [&](Tile<D, MB>& Y) {
    const bool valid = ii < i_end;
    if (valid && is == 0) load_q<D, MB, LQ>(a, iitem, Y.q, col, grp);
    // past the end of the stream: an in-bounds re-load of the current step
    issue_step<D, MB, NP>(a, valid ? iitem : citem, valid ? is : cs, Y, col, grp);
    if (valid && ++is >= iitem.nsteps) {
      ++ii;
      is = 0;
      if (ii < i_end) iitem = load_item(a, ii);
    }
  };

  // Refill Y (the tile computed last), then compute X.
  auto advance = [&](Tile<D, MB>& X, Tile<D, MB>& Y) -> bool {
    issue(Y);
    if (cs == 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < KJ; ++j) q_cur[mb][j] = X.q[mb][j];
    }
    compute_step<D, MB>(a, citem, cs, X, q_cur, st, col, grp);
    if (cs + 1 >= citem.nsteps) {
      finalize<D, MB, LQ>(a, citem, st, col, grp);
      st.reset();
      if (++ci >= i_end) return false;
      cs = 0;
      citem = load_item(a, ci);
    } else {
      ++cs;
    }
    return true;
  };

#pragma unroll
  for (int r = 0; r < R - 1; ++r) issue(T[r]);
  while (true) {
    if (!advance(T[0], T[R - 1])) break;
#pragma unroll
    for (int r = 1; r < R; ++r)
      if (!advance(T[r], T[r - 1])) goto done;
  }
done:;
}

template <int D, int MB, bool LQ>
hipError_t launch_np(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.page_size == 8) {
    hipLaunchKernelGGL((attention_kernel<D, MB, 4, LQ>), grid, dim3(256), 0, s, a);
  } else if (a.page_size == 16) {
    hipLaunchKernelGGL((attention_kernel<D, MB, 2, LQ>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((attention_kernel<D, MB, 1, LQ>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, int rows_per_block, bool list_q, dim3 grid,
                    hipStream_t s) {
  if (list_q) {
    if (rows_per_block == 64) return launch_np<D, 4, true>(a, grid, s);
    return hipErrorInvalidValue;
  }
  switch (rows_per_block) {
    case 16: return launch_np<D, 1, false>(a, grid, s);
    case 32: return launch_np<D, 2, false>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int head_dim, int rows_per_block, bool list_q,
                            hipStream_t stream) {
  const int blocks = (a.num_workers + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  if (blocks == 0) return hipSuccess;
  const dim3 grid(blocks);
  if (head_dim == 128) return launch_d<128>(a, rows_per_block, list_q, grid, stream);
  if (head_dim == 64) return launch_d<64>(a, rows_per_block, list_q, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace fi
