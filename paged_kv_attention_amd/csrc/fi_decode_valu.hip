// fi_decode_valu.hip -- paged decode attention on the vector ALU only.
//
// The same work items, block-table gather, online softmax and partial-state
// output as the matrix-core decode kernel, with both contractions on VALU:
// the decode q.K and P.V are matrix-vector products (a handful of query rows
// per kv head), which is the shape the research note "flashinfer-backend-
// selection", "Arithmetic intensity", calls memory-bound, so the vector units
// are the plain choice and the matrix cores are an option to be measured.
//
// Lanes. Each K/V row (D bf16) is read by LPT = D/8 lanes, 16 bytes each, so
// one load instruction covers TPI = 64/LPT consecutive tokens (1 KiB of one
// page for D = 128). Lane group grp = lane / LPT takes tokens grp, grp + TPI,
// ... of every 32-token step and keeps its own online-softmax state over
// them; the TPI states are merged in registers when the item ends, by the
// same log-sum-exp rule as the merge kernel.
//   q.K: v_dot2_f32_bf16 over the lane's 8 dims, then a sum over the LPT lanes
//        of the token with DPP (quad_perm, row_half_mirror, row_mirror).
//   P.V: v_dot2_f32_bf16 over pairs of tokens: p is rounded to bf16 and V of
//        two tokens is paired per dim with v_perm_b32.
// Pages and prefetch are as in the matrix-core kernel: compile-time page
// selection per instruction, clamped page ids, unconditional loads, and a
// ring of register tiles fed across item boundaries.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_device.h"

namespace fi {
namespace {

using namespace dev;

constexpr int kRingV = 3;

template <int D>
struct VCfg {
  static constexpr int LPT = D / 8;      // lanes per token row
  static constexpr int TPI = 64 / LPT;   // tokens per load instruction
  static constexpr int NI = 32 / TPI;    // tokens per lane per 32-token step
};

// One step's registers (K and V of the lane's NI tokens) and, on an item's
// first step, its query rows.
template <int D, int GM>
struct VTile {
  u32x4 k[VCfg<D>::NI];
  u32x4 v[VCfg<D>::NI];
  u32x4 q[GM];
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPT lanes of a token (aligned groups of 8 or 16 lanes).
template <int LPT>
__device__ __forceinline__ float token_sum(float s) {
  s += dpp<0xB1>(s);    // quad_perm [1,0,3,2]
  s += dpp<0x4E>(s);    // quad_perm [2,3,0,1]
  s += dpp<0x141>(s);   // row_half_mirror: the other quad of the 8
  if constexpr (LPT == 16) s += dpp<0x140>(s);   // row_mirror: the other 8 of the 16
  return s;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

template <int D, int NP, int GM>
__device__ __forceinline__ void issue_step_v(const AttnArgs& a, const Item& it, int s,
                                             VTile<D, GM>& T, int c, int grp) {
  constexpr int TPI = VCfg<D>::TPI, NI = VCfg<D>::NI;
  const int sh = a.page_shift;
  const int T0 = it.t_begin + 32 * s;
  const int pb = T0 >> sh;
  const int plast = (it.t_end - 1) >> sh;
  const int64_t tile_bytes = (int64_t)a.page_size * D * 2;
  const char* kb[NP];
  const char* vb[NP];
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    const int pid = ld_uniform(it.plist, min(pb + n, plast));
    const int64_t off = ((int64_t)pid * a.num_kv_heads + it.g) * tile_bytes;
    kb[n] = (const char*)a.k_cache + off;
    vb[n] = (const char*)a.v_cache + off;
  }
  const int slot0 = (NP == 1) ? (T0 & (a.page_size - 1)) : 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    // tokens TPI*i .. TPI*i + TPI-1 of the step lie in one page
    constexpr int kPS = 32 / NP;   // page size when NP > 1
    const int n = (NP == 1) ? 0 : (TPI * i) / kPS;
    const int slot = slot0 + ((NP == 1) ? TPI * i : (TPI * i) % kPS) + grp;
    const uint32_t off = (uint32_t)(slot * D + 8 * c) * 2u;
    T.k[i] = __builtin_nontemporal_load((const u32x4*)(kb[n] + off));   // read once: nontemporal
    T.v[i] = __builtin_nontemporal_load((const u32x4*)(vb[n] + off));
  }
}

template <int D, int GM>
__device__ __forceinline__ void load_q_v(const AttnArgs& a, const Item& it, u32x4 (&q)[GM],
                                         int c) {
  const int G = a.group;
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    const int rl = h < it.n_rows ? h : 0;
    const int rho = it.row0 + rl;
    const int qi = rho / G, hh = rho - qi * G;
    const uint16_t* qp =
        a.q + ((int64_t)(it.q_base + qi) * a.num_qo_heads + it.g * G + hh) * D + 8 * c;
    q[h] = *(const u32x4*)qp;
  }
}

// Online-softmax state of one lane group: base m, partial sum l (fp32 p) and
// the lane's 8 output dims, per query row.
template <int GM>
struct VState {
  float m[GM], l[GM];
  float acc[GM][8];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      m[h] = neg_inf();
      l[h] = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;
    }
  }
};

template <int D, int GM>
__device__ __forceinline__ void compute_step_v(const AttnArgs& a, const Item& it, int s,
                                               const VTile<D, GM>& T, const u32x4 (&q)[GM],
                                               VState<GM>& st, int grp) {
  constexpr int TPI = VCfg<D>::TPI, NI = VCfg<D>::NI, LPT = VCfg<D>::LPT;
  const int T0 = it.t_begin + 32 * s;
  const bool tail = T0 + 32 > it.t_end;
  float x[NI][GM];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      float sacc = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) sacc = dot2(T.k[i][k], q[h][k], sacc);
      x[i][h] = token_sum<LPT>(sacc) * a.scale_log2;
    }
  }
  // tokens past the item's end: logit -inf, and V zeroed so p = 0 cancels it
  u32x4 vv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const bool ok = T0 + TPI * i + grp < it.t_end;
    vv[i] = ok ? T.v[i] : u32x4{0u, 0u, 0u, 0u};
    if (tail && !ok) {
#pragma unroll
      for (int h = 0; h < GM; ++h) x[i][h] = neg_inf();
    }
  }
  float mx[GM];
  bool grow = false;
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    mx[h] = x[0][h];
#pragma unroll
    for (int i = 1; i < NI; ++i) mx[h] = fmaxf(mx[h], x[i][h]);
    grow = grow || (mx[h] > st.m[h] + kRescaleSlack);
  }
  // The base only moves when some row's max exceeds it by more than the
  // slack (p <= 2^slack is exact enough); every group rescales together.
  if (__any(grow)) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const float m_new = fmaxf(st.m[h], mx[h]);
      const float alpha = (m_new == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(st.m[h] - m_new);
      st.l[h] *= alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) st.acc[h][d] *= alpha;
      st.m[h] = m_new;
    }
  }
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    const float base = (st.m[h] == neg_inf()) ? 0.f : st.m[h];
    float p[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) p[i] = __builtin_amdgcn_exp2f(x[i][h] - base);
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) ls += p[i];
    st.l[h] += ls;
#pragma unroll
    for (int j = 0; j < NI / 2; ++j) {
      const uint32_t pp = pack2(p[2 * j], p[2 * j + 1]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = __builtin_amdgcn_perm(vv[2 * j + 1][k], vv[2 * j][k], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(vv[2 * j + 1][k], vv[2 * j][k], 0x07060302u);
        st.acc[h][2 * k] = dot2(lo, pp, st.acc[h][2 * k]);
        st.acc[h][2 * k + 1] = dot2(hi, pp, st.acc[h][2 * k + 1]);
      }
    }
  }
}

// Merge the TPI lane groups' states (lanes c, c + LPT, ...) and write row h
// from lane group h % TPI: o = acc / l, lse = (m + log2 l) ln 2.
template <int D, int GM>
__device__ __forceinline__ void finalize_v(const AttnArgs& a, const Item& it, VState<GM>& st,
                                           int c, int grp) {
  constexpr int TPI = VCfg<D>::TPI, LPT = VCfg<D>::LPT;
  const int G = a.group;
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    float M = st.m[h];
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float sc = (st.m[h] == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(st.m[h] - M);
    float L = st.l[h] * sc;
    float v[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) v[d] = st.acc[h][d] * sc;
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1) {
      L += __shfl_xor(L, o);
#pragma unroll
      for (int d = 0; d < 8; ++d) v[d] += __shfl_xor(v[d], o);
    }
    if (h >= it.n_rows || grp != h % TPI) continue;
    const bool live = L > 0.f;
    const float inv = live ? 1.f / L : 0.f;
    const float lse_v = live ? (M + log2f(L)) * kLn2 : neg_inf();
    if (it.flags & FLAG_PARTIAL) {
      float* op = a.part_o + (int64_t)(it.dst + h) * D + 8 * c;
      *(f32x4*)op = f32x4{v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
      *(f32x4*)(op + 4) = f32x4{v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv};
      if (c == 0) a.part_lse[it.dst + h] = lse_v;
    } else {
      const int rho = it.row0 + h;
      const int qi = rho / G, hh = rho - qi * G;
      const int64_t orow = (int64_t)(it.q_base + qi) * a.num_qo_heads + it.g * G + hh;
      const u32x4 pk = {pack2(v[0] * inv, v[1] * inv), pack2(v[2] * inv, v[3] * inv),
                        pack2(v[4] * inv, v[5] * inv), pack2(v[6] * inv, v[7] * inv)};
      *(u32x4*)(a.o + orow * D + 8 * c) = pk;
      if (c == 0 && a.lse) a.lse[orow] = lse_v;
    }
  }
}

// GM: query rows per item rounded up to a power of two (the item's n_rows
// <= GM; padding rows read row 0 and are never stored).
template <int D, int NP, int GM>
__global__ __launch_bounds__(256) void decode_valu_kernel(AttnArgs a) {
  constexpr int LPT = VCfg<D>::LPT;
  const int lane = threadIdx.x & 63;
  const int c = lane % LPT, grp = lane / LPT;
  const int w = blockIdx.x * WAVES_PER_BLOCK + uniform(threadIdx.x >> 6);
  if (w >= a.num_workers) return;
  const int i_end = ld_uniform(a.worker_indptr, w + 1);
  const int i_begin = ld_uniform(a.worker_indptr, w);
  if (i_begin >= i_end) return;

  int ci = i_begin, cs = 0;
  Item citem = load_item(a, ci);
  int ii = i_begin, is = 0;
  Item iitem = citem;
  VTile<D, GM> TA, TB, TC;   // the ring (kRingV = 3), named so it stays in registers
  u32x4 q_cur[GM];
  VState<GM> st;
  st.reset();

  auto issue = [&](VTile<D, GM>& Y) {
    const bool valid = ii < i_end;
    if (valid && is == 0) load_q_v<D, GM>(a, iitem, Y.q, c);
    // past the end of the stream: an in-bounds re-load of the current step,
    // every lane at lane 0's addresses (next to no HBM traffic)
    issue_step_v<D, NP, GM>(a, valid ? iitem : citem, valid ? is : cs, Y, valid ? c : 0,
                            valid ? grp : 0);
    if (valid && ++is >= iitem.nsteps) {
      ++ii;
      is = 0;
      if (ii < i_end) iitem = load_item(a, ii);
    }
  };

  // Refill Y (the tile computed last), then compute X.
  auto advance = [&](VTile<D, GM>& X, VTile<D, GM>& Y) -> bool {
    issue(Y);
    if (cs == 0) {
#pragma unroll
      for (int h = 0; h < GM; ++h) q_cur[h] = X.q[h];
    }
    compute_step_v<D, GM>(a, citem, cs, X, q_cur, st, grp);
    if (cs + 1 >= citem.nsteps) {
      finalize_v<D, GM>(a, citem, st, c, grp);
      st.reset();
      if (++ci >= i_end) return false;
      cs = 0;
      citem = load_item(a, ci);
    } else {
      ++cs;
    }
    return true;
  };

  static_assert(kRingV == 3, "the loop below is unrolled for a ring of three tiles");
  issue(TA);
  issue(TB);
  while (advance(TA, TC) && advance(TB, TA) && advance(TC, TB)) {
  }
}

template <int D, int GM>
hipError_t launch_v(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.page_size == 8) {
    launch_timed((decode_valu_kernel<D, 4, GM>), grid, dim3(256), s, a);
  } else if (a.page_size == 16) {
    launch_timed((decode_valu_kernel<D, 2, GM>), grid, dim3(256), s, a);
  } else {
    launch_timed((decode_valu_kernel<D, 1, GM>), grid, dim3(256), s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_vd(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.group <= 1) return launch_v<D, 1>(a, grid, s);
  if (a.group <= 2) return launch_v<D, 2>(a, grid, s);
  if (a.group <= 4) return launch_v<D, 4>(a, grid, s);
  if (a.group <= 8) return launch_v<D, 8>(a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_valu(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const int blocks = (a.num_workers + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  if (blocks == 0) return hipSuccess;
  if (head_dim == 128) return launch_vd<128>(a, dim3(blocks), stream);
  if (head_dim == 64) return launch_vd<64>(a, dim3(blocks), stream);
  return hipErrorInvalidValue;
}

}  // namespace fi
