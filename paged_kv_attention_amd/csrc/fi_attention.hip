// fi_attention.hip -- paged decode attention kernel for gfx950 (CDNA4).
//
// Computes, for each planned work item, exact softmax attention of up to 16
// query rows (the G q heads of one decode query, row = head within the kv
// head's group) over the item's token range of one sequence, reading K/V
// through the block table (research note "flashinfer-backend-selection",
// "Arithmetic intensity": decode reads a gathered block table instead of a
// dense cache). Used for decode and for the per-request suffix level of
// cascade. Each wavefront is one persistent worker that runs the items the
// plan gave it as one continuous stream of 32-token steps.
//
// Tiling. Both contractions run on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation:
//   S^T[token][row] = K[token][:] . Q[row][:]    A = K tile, B = Q^T
//   O^T[d][row]    += V^T[d][token] . P^T[token][row]
// With both outputs transposed, the query row sits in lane%16 of every
// accumulator, so the softmax statistics and the rescale of O stay in-lane;
// only the row max and the final row sum cross the four 16-lane groups. Lane l
// loads K of token 16*blk + l%16 (4 lanes read 64 contiguous bytes of a row)
// and V of 8 tokens (16 lanes read a full 256-byte row per instruction); the V
// rows are transposed in registers with v_perm_b32 into the MFMA A layout, in
// the token order the S^T accumulator hands to P, so P needs no shuffle.
//
// Pages. NP = pages one 32-token step touches (4 for page size 8, 2 for 16, 1
// for >= 32). The step's page ids are wave-uniform scalar loads; which of them
// a lane's token uses is fixed at compile time up to one lane bit, so each
// load is a uniform page-tile base plus a 32-bit lane offset. Pages past the
// item's last page are clamped to it, so every address is valid and every
// load is unconditional; V of tokens past the end is zeroed at use and their
// logits are -inf.
//
// Prefetch. A ring of kRing = 4 register tiles is fed by an issue cursor that
// runs kRing-1 steps ahead of the compute cursor, across item boundaries;
// every iteration issues exactly one step of loads, so the wait for the tile
// being computed never drains the steps behind it. An item's Q travels with
// its first step's tile.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_device.h"

namespace fi {
namespace {

using namespace dev;

constexpr int kRing = 4;

// One step's registers: K and V of 32 tokens, and (first step of an item
// only) the item's Q.
template <int D>
struct Tile {
  u32x4 k[2][Cfg<D>::KJ];
  typename Cfg<D>::vrow_t v[8];
  u32x4 q[1][Cfg<D>::KJ];
};

// Issue the loads of step s of item it into T.
template <int D, int NP>
__device__ __forceinline__ void issue_step(const AttnArgs& a, const Item& it, int s, Tile<D>& T,
                                           int col, int grp) {
  constexpr int KJ = Cfg<D>::KJ, DPL = Cfg<D>::DPL;
  typedef typename Cfg<D>::vrow_t vrow_t;
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
  for (int blk = 0; blk < 2; ++blk) {   // K: token 16*blk + col
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
#pragma unroll
  for (int i = 0; i < 8; ++i) {   // V: tokens 4*grp + i and 16 + 4*grp + (i - 4)
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
    T.v[i] = *(const vrow_t*)(base + (uint32_t)(slot * D + DPL * col) * 2u);
  }
}

template <int D>
__device__ __forceinline__ void compute_step(const AttnArgs& a, const Item& it, int s,
                                             const Tile<D>& T, const u32x4 (&qf)[1][Cfg<D>::KJ],
                                             State<D, 1>& st, int col, int grp) {
  constexpr int KJ = Cfg<D>::KJ, DPL = Cfg<D>::DPL;
  typedef typename Cfg<D>::vrow_t vrow_t;
  const int T0 = it.t_begin + 32 * s;
  const bool tail = T0 + 32 > it.t_end;
  // V rows of tokens past the item's end hold whatever the clamped page has
  // there (even NaN): zero them so that p = 0 cancels them exactly. (A select
  // on every step, not a branch on the tail: the branch keeps the tiles out
  // of registers.)
  vrow_t vv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tl = (i < 4) ? 4 * grp + i : 16 + 4 * grp + (i - 4);
    vv[i] = (T0 + tl >= it.t_end) ? vrow_t{} : T.v[i];
  }
  u32x4 vt[DPL];
  transpose_v<D>(vv, vt);
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    s0 = mfma_bf16(T.k[0][j], qf[0][j], s0);
    s1 = mfma_bf16(T.k[1][j], qf[0][j], s1);
  }
  softmax_pv<D, 1>(st, 0, s0, s1, vt, a.scale_log2, tail, T0, it.t_end - 1, grp);
}

template <int D, int NP>
__global__ __launch_bounds__(256) void decode_kernel(AttnArgs a) {
  constexpr int KJ = Cfg<D>::KJ;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int w = blockIdx.x * WAVES_PER_BLOCK + uniform(threadIdx.x >> 6);
  if (w >= a.num_workers) return;
  const int i_end = ld_uniform(a.worker_indptr, w + 1);
  const int i_begin = ld_uniform(a.worker_indptr, w);
  if (i_begin >= i_end) return;

  // Two cursors over the worker's stream of steps: the issue cursor (ii, is)
  // runs kRing-1 steps ahead of the compute cursor (ci, cs), across item
  // boundaries. Tiles are filled and consumed in the same order.
  int ci = i_begin, cs = 0;
  Item citem = load_item(a, ci);
  int ii = i_begin, is = 0;
  Item iitem = citem;
  Tile<D> TA, TB, TC, TD;   // the ring (kRing = 4), named so it stays in registers
  u32x4 q_cur[1][KJ];
  State<D, 1> st;
  st.reset();

  auto issue = [&](Tile<D>& Y) {
    const bool valid = ii < i_end;
    if (valid && is == 0) load_q_rows<D, 1, false>(a, iitem, 0, Y.q, col, grp);
    // past the end of the stream: an in-bounds re-load of the current step
    issue_step<D, NP>(a, valid ? iitem : citem, valid ? is : cs, Y, col, grp);
    if (valid && ++is >= iitem.nsteps) {
      ++ii;
      is = 0;
      if (ii < i_end) iitem = load_item(a, ii);
    }
  };

  // Refill Y (the tile computed last), then compute X.
  auto advance = [&](Tile<D>& X, Tile<D>& Y) -> bool {
    issue(Y);
    if (cs == 0) {
#pragma unroll
      for (int j = 0; j < KJ; ++j) q_cur[0][j] = X.q[0][j];
    }
    compute_step<D>(a, citem, cs, X, q_cur, st, col, grp);
    if (cs + 1 >= citem.nsteps) {
      finalize_rows<D, 1, false>(a, citem, st, 0, col, grp);
      st.reset();
      if (++ci >= i_end) return false;
      cs = 0;
      citem = load_item(a, ci);
    } else {
      ++cs;
    }
    return true;
  };

  static_assert(kRing == 4, "the loop below is unrolled for a ring of four tiles");
  issue(TA);
  issue(TB);
  issue(TC);
  while (advance(TA, TD) && advance(TB, TA) && advance(TC, TB) && advance(TD, TC)) {
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.page_size == 8) {
    hipLaunchKernelGGL((decode_kernel<D, 4>), grid, dim3(256), 0, s, a);
  } else if (a.page_size == 16) {
    hipLaunchKernelGGL((decode_kernel<D, 2>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<D, 1>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const int blocks = (a.num_workers + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  if (blocks == 0) return hipSuccess;
  if (head_dim == 128) return launch_d<128>(a, dim3(blocks), stream);
  if (head_dim == 64) return launch_d<64>(a, dim3(blocks), stream);
  return hipErrorInvalidValue;
}

}  // namespace fi
