// fi_attention.hip -- paged attention work-item kernel for gfx950 (CDNA4).
//
// Computes, for each planned work item, exact softmax attention of up to
// 16*MB query rows (query token i, q head h of kv head g) over the item's
// token range of one sequence, reading K/V through the block table (research
// note "flashinfer-backend-selection", "Arithmetic intensity": decode reads a
// gathered block table instead of a dense cache). Each wavefront is one
// persistent worker that runs the items the plan gave it, in order.
//
// Tiling. One step covers 32 tokens. Both contractions run on the bf16 MFMA
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation:
//   S^T[token][row] = K[token][:] . Q[row][:]    A = K tile, B = Q^T
//   O^T[d][row]    += V^T[d][token] . P^T[token][row]
// With both outputs transposed, the query row sits in lane%16 of every
// accumulator, so the softmax statistics and the rescale of O stay in-lane;
// only the row max and the final row sum cross the four 16-lane groups.
// Lane l loads K of token 16*blk + l%16 (64 contiguous bytes per 4 lanes) and
// V of 8 tokens (a full 16-lane row of 256 B per instruction). The V rows are
// transposed in registers with v_perm_b32 into the MFMA A layout; the token
// order inside a lane group (4g..4g+3, 16+4g..16+4g+3) is the same one the
// S^T accumulator hands to P, so P needs no shuffle at all.
//
// Softmax is online (running max m, running sum l, O rescaled by
// exp2(m_old - m_new)) with logits pre-scaled by sm_scale*log2(e); the LSE is
// returned in natural log. P is rounded to bf16 for the P.V MFMA; l sums the
// fp32 P. Keys past the item's end (tail slots of the last page) and, under
// the causal mask, keys after a query's position are masked to -inf and their
// K/V are never loaded.

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

template <int W> struct RowVec;
template <> struct RowVec<4> { typedef u32x4 T; };
template <> struct RowVec<2> { typedef u32x2 T; };

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int D, int MB>
__device__ __forceinline__ void run_item(const AttnArgs& a, const int32_t* __restrict__ it,
                                         const int lane) {
  constexpr int KJ = D / 32;    // 32-dim k-slices of the q.K contraction
  constexpr int DPL = D / 16;   // V dims per lane = P.V MFMAs per step
  typedef typename RowVec<DPL / 2>::T vrow_t;

  const int q_base = it[F_Q_BASE], row0 = it[F_ROW0], n_rows = it[F_NROWS];
  const int g = it[F_KVHEAD], page_off = it[F_PAGEOFF], flags = it[F_FLAGS];
  const int t_begin = it[F_TBEGIN], t_end = it[F_TEND], q_pos0 = it[F_QPOS0];
  const int dst = it[F_DST];

  const int G = a.group, Hq = a.num_qo_heads, Hkv = a.num_kv_heads;
  const int sh = a.page_shift, ps = a.page_size;
  const int col = lane & 15;   // query row within a 16-row block
  const int grp = lane >> 4;   // 16-lane group
  const bool causal = (flags & FLAG_CAUSAL) != 0;
  const int32_t* __restrict__ plist =
      ((flags & FLAG_PREFIX) ? a.prefix_indices : a.kv_indices) + page_off;

  // ---- query rows of this item (B operand of the q.K MFMAs)
  u32x4 qf[MB][KJ];
  int qlim[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int rl = mb * 16 + col;
    const int rho = row0 + rl;
    const int qi = rho / G, h = rho - qi * G;
    const bool ok = rl < n_rows;
    int tok = 0;
    if (ok) tok = (flags & FLAG_LIST_Q) ? a.qlist[q_base + qi] : q_base + qi;
    const uint16_t* qp = a.q + ((int64_t)tok * Hq + g * G + h) * D + grp * 8;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *(const u32x4*)(qp + 32 * j);
      qf[mb][j] = v;
    }
    qlim[mb] = causal ? q_pos0 + qi : INT_MAX;
  }

  f32x4 acc[MB][DPL];
  float m_run[MB], l_run[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    m_run[mb] = neg_inf();
    l_run[mb] = 0.f;
#pragma unroll
    for (int m = 0; m < DPL; ++m) acc[mb][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int np = (32 >> sh) > 1 ? (32 >> sh) : 1;   // pages touched by one step
  const int plast = (t_end - 1) >> sh;

  auto load_step = [&](int s, u32x4 (&kf)[2][KJ], vrow_t (&vf)[8]) {
    const int T0 = t_begin + 32 * s;
    const int pbase = T0 >> sh;
    int pid[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      pid[n] = 0;
      if (n < np) pid[n] = plist[min(pbase + n, plast)];
    }
    auto page_of = [&](int t) {
      const int rel = (t >> sh) - pbase;
      return rel == 0 ? pid[0] : rel == 1 ? pid[1] : rel == 2 ? pid[2] : pid[3];
    };
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int t = T0 + 16 * blk + col;
      const int64_t tile = ((int64_t)page_of(t) * Hkv + g) * ps + (t & (ps - 1));
      const uint16_t* kp = a.k_cache + tile * D + grp * 8;
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (t < t_end) v = *(const u32x4*)(kp + 32 * j);
        kf[blk][j] = v;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = T0 + (i < 4 ? 4 * grp + i : 16 + 4 * grp + (i - 4));
      const int64_t tile = ((int64_t)page_of(t) * Hkv + g) * ps + (t & (ps - 1));
      vrow_t v = {};
      if (t < t_end) v = *(const vrow_t*)(a.v_cache + tile * D + DPL * col);
      vf[i] = v;
    }
  };

  auto compute = [&](int s, const u32x4 (&kf)[2][KJ], const vrow_t (&vf)[8]) {
    const int T0 = t_begin + 32 * s;
    // V^T operands: for MFMA m, lane supplies dim DPL*col+m of its 8 tokens.
    u32x4 vt[DPL];
#pragma unroll
    for (int m = 0; m < DPL; ++m) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t lo = vf[2 * jj][m >> 1], hi = vf[2 * jj + 1][m >> 1];
        vt[m][jj] = __builtin_amdgcn_perm(hi, lo, (m & 1) ? 0x07060302u : 0x05040100u);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
        s0 = mfma_bf16(kf[0][j], qf[mb][j], s0);
        s1 = mfma_bf16(kf[1][j], qf[mb][j], s1);
      }
      float x[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t0 = T0 + 4 * grp + r, t1 = t0 + 16;
        x[r] = (t0 < t_end && t0 <= qlim[mb]) ? s0[r] * a.scale_log2 : neg_inf();
        x[4 + r] = (t1 < t_end && t1 <= qlim[mb]) ? s1[r] * a.scale_log2 : neg_inf();
      }
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[mb], mx);
      const float base = (m_new == neg_inf()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[mb] - base);
      float p[8], psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = __builtin_amdgcn_exp2f(x[i] - base);
        psum += p[i];
      }
      l_run[mb] = l_run[mb] * alpha + psum;
      m_run[mb] = m_new;
      const u32x4 pb = {pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]),
                        pack2(p[6], p[7])};
#pragma unroll
      for (int m = 0; m < DPL; ++m) acc[mb][m] = mfma_bf16(vt[m], pb, acc[mb][m] * alpha);
    }
  };

  const int nsteps = (t_end - t_begin + 31) >> 5;
  u32x4 kA[2][KJ], kB[2][KJ];
  vrow_t vA[8], vB[8];
  if (nsteps > 0) load_step(0, kA, vA);
  for (int s = 0; s < nsteps; s += 2) {
    if (s + 1 < nsteps) load_step(s + 1, kB, vB);
    compute(s, kA, vA);
    if (s + 1 < nsteps) {
      if (s + 2 < nsteps) load_step(s + 2, kA, vA);
      compute(s + 1, kB, vB);
    }
  }

  // ---- finalize: o = acc / l, lse = (m + log2 l) * ln 2
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float lt = l_run[mb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int rl = mb * 16 + col;
    if (rl >= n_rows) continue;
    const bool live = lt > 0.f;
    const float inv = live ? 1.f / lt : 0.f;
    const float lse_v = live ? (m_run[mb] + log2f(lt)) * kLn2 : neg_inf();
    if (flags & FLAG_PARTIAL) {
      float* op = a.part_o + (int64_t)(dst + rl) * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* d0 = op + DPL * (4 * grp + r);
#pragma unroll
        for (int m = 0; m < DPL; m += 4) {
          f32x4 v = {acc[mb][m][r] * inv, acc[mb][m + 1][r] * inv, acc[mb][m + 2][r] * inv,
                     acc[mb][m + 3][r] * inv};
          *(f32x4*)(d0 + m) = v;
        }
      }
      if (grp == 0) a.part_lse[dst + rl] = lse_v;
    } else {
      const int rho = row0 + rl;
      const int qi = rho / G, h = rho - qi * G;
      const int tok = (flags & FLAG_LIST_Q) ? a.qlist[q_base + qi] : q_base + qi;
      const int64_t orow = (int64_t)tok * Hq + g * G + h;
      uint16_t* op = a.o + orow * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vrow_t v;
#pragma unroll
        for (int m = 0; m < DPL; m += 2) v[m >> 1] = pack2(acc[mb][m][r] * inv, acc[mb][m + 1][r] * inv);
        *(vrow_t*)(op + DPL * (4 * grp + r)) = v;
      }
      if (grp == 0 && a.lse) a.lse[orow] = lse_v;
    }
  }
}

template <int D, int MB>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * WAVES_PER_BLOCK + wave;
  if (w >= a.num_workers) return;
  const int i0 = a.worker_indptr[w], i1 = a.worker_indptr[w + 1];
  for (int i = i0; i < i1; ++i) run_item<D, MB>(a, a.items + (int64_t)i * ITEM_INTS, lane);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, int rows_per_block, dim3 grid, hipStream_t s) {
  switch (rows_per_block) {
    case 16: hipLaunchKernelGGL((attention_kernel<D, 1>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((attention_kernel<D, 2>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((attention_kernel<D, 4>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int head_dim, int rows_per_block,
                            hipStream_t stream) {
  const int blocks = (a.num_workers + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  if (blocks == 0) return hipSuccess;
  const dim3 grid(blocks);
  if (head_dim == 128) return launch_d<128>(a, rows_per_block, grid, stream);
  if (head_dim == 64) return launch_d<64>(a, rows_per_block, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace fi
