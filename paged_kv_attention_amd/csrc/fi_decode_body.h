// fi_decode_body.h -- the decode worker (one wavefront's stream of work items)
// shared by the decode kernel and the fused mixed-batch kernel. See
// fi_attention.hip for the design.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_device.h"

namespace fi {
namespace dec {

using namespace dev;

constexpr int kRing = 4;

// One step's registers: K and V of 32 tokens, and (QT: first step of an item
// only) the item's Q.
template <int D, bool QT>
struct Tile {
  u32x4 k[2][Cfg<D>::KJ];
  typename Cfg<D>::vrow_t v[8];
  u32x4 q[QT ? 1 : 0][Cfg<D>::KJ];
};

// Issue the loads of step s of item it into T. K and V are read once per call,
// so the loads are nontemporal (on MI355X they stream from HBM ~13% faster
// than default-policy loads). Paged layout: page id pid, kv head g at tile
// (pid * Hkv + g) of ps tokens of D elements. RAGGED layout ([tokens][Hkv][D]):
// the page list holds the first token of each ps-token run, token stride
// Hkv * D elements.
template <int D, int NP, bool QT, bool RAGGED = false>
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const Item& it, int s,
                                           Tile<D, QT>& T, int col, int grp) {
  constexpr int KJ = Cfg<D>::KJ, DPL = Cfg<D>::DPL;
  typedef typename Cfg<D>::vrow_t vrow_t;
  const int sh = a.page_shift;
  const int T0 = it.t_begin + 32 * s;
  const int pb = T0 >> sh;
  const int plast = (it.t_end - 1) >> sh;
  const int64_t tile_bytes = RAGGED ? (int64_t)D * 2 : (int64_t)a.page_size * D * 2;
  const uint32_t tok = RAGGED ? (uint32_t)(a.num_kv_heads * D * 2) : (uint32_t)(D * 2);
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
    const uint32_t off = RAGGED ? (uint32_t)slot * tok + (uint32_t)(grp * 16)
                                : (uint32_t)(slot * D + grp * 8) * 2u;
#pragma unroll
    for (int j = 0; j < KJ; ++j)
      T.k[blk][j] = __builtin_nontemporal_load((const u32x4*)(base + off + 64u * j));
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
    const uint32_t voff = RAGGED ? (uint32_t)slot * tok + (uint32_t)(DPL * col * 2)
                                 : (uint32_t)(slot * D + DPL * col) * 2u;
    T.v[i] = __builtin_nontemporal_load((const vrow_t*)(base + voff));
  }
}

// CAUSAL: items may carry FLAG_CAUSAL (append requests of a few query tokens,
// all in one row block); row rho then sees tokens up to q_pos0 + rho / G.
template <int D, bool CAUSAL, bool QT>
__device__ __forceinline__ void compute_step(const AttnArgs& a, const Item& it, int s,
                                             const Tile<D, QT>& T, const u32x4 (&qf)[1][Cfg<D>::KJ],
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
  int lim = it.t_end - 1;
  bool masked = tail;
  if (CAUSAL && (it.flags & FLAG_CAUSAL)) {
    masked = masked || T0 + 31 > it.q_pos0 + it.row0 / a.group;
    lim = min(lim, it.q_pos0 + (it.row0 + col) / a.group);
  }
  softmax_pv<D, 1>(st, 0, s0, s1, vt, a.scale_log2, masked, T0, lim, grp);
}

// The stream of worker w (one wavefront): its items' 32-token steps. RING
// register tiles: 4 when the wavefront has a SIMD's registers to itself, 2 when
// it shares them with a second wavefront (two workgroups per CU); a ring of 2
// keeps the query out of the tiles and loads it when an item's first step is
// computed, ahead of the next step's loads.
// FOLD: the launch is a workgroup-folded plan's, and lds is the workgroup's
// LDS for the partial states (FoldLds); otherwise they go to the workspace
// (and the stream's code has no LDS path).
template <int D, int NP, bool CAUSAL = false, int RING = kRing, bool RAGGED = false,
          bool FOLD = false>
__device__ __forceinline__ void decode_worker(const AttnArgs& a, int w, float* lds = nullptr) {
  float* const fold = FOLD ? lds : nullptr;
  static_assert(RING == 2 || RING == 4, "rings of two or four tiles");
  constexpr int KJ = Cfg<D>::KJ;
  constexpr bool QT = RING == 4;   // the query travels in the tiles
  typedef Tile<D, QT> TileT;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  // the first loads of every wave in one round trip: its stream's bounds
  // (waves past the last worker read the table's end, then leave) and the
  // plan's count of units with no keys (the meta section is always there)
  const int nw = a.num_workers;
  const int i_begin = ld_uniform(a.worker_indptr, min(w, nw));
  const int i_end = ld_uniform(a.worker_indptr, min(w + 1, nw));
  const int n_empty = ld_uniform(a.meta, META_EMPTY);
  if (w >= nw) return;
  fused_merge_start<D>(a, w, lane, n_empty);
  if (i_begin >= i_end) {   // (a workgroup-folded plan's barrier needs every wave)
    fused_merge_end<D>(a, i_begin, i_end, lane, fold);
    return;
  }

  // Two cursors over the worker's stream of steps: the issue cursor (ii, is)
  // runs RING-1 steps ahead of the compute cursor (ci, cs), across item
  // boundaries. Tiles are filled and consumed in the same order.
  int ci = i_begin, cs = 0;
  Item citem = load_item(a, ci);
  int ii = i_begin, is = 0;
  Item iitem = citem;
  u32x4 q_cur[1][KJ];
  State<D, 1> st;
  st.reset();

  auto issue = [&](TileT& Y) {
    const bool valid = ii < i_end;
    if constexpr (QT) {
      if (valid && is == 0) load_q_rows<D, 1, false>(a, iitem, 0, Y.q, col, grp);
    }
    // past the end of the stream: an in-bounds re-load of the current step,
    // every lane at lane 0's addresses (one line per load, so the extra
    // loads of the ring's last steps add next to no HBM traffic)
    issue_tile<D, NP, QT, RAGGED>(a, valid ? iitem : citem, valid ? is : cs, Y, valid ? col : 0,
                                  valid ? grp : 0);
    if (valid && ++is >= iitem.nsteps) {
      ++ii;
      is = 0;
      if (ii < i_end) iitem = load_item(a, ii);
    }
  };

  // Refill Y (the tile computed last), then compute X.
  auto advance = [&](TileT& X, TileT& Y) -> bool {
    if constexpr (!QT) {
      if (cs == 0) load_q_rows<D, 1, false>(a, citem, 0, q_cur, col, grp);
    }
    issue(Y);
    if constexpr (QT) {
      if (cs == 0) {
#pragma unroll
        for (int j = 0; j < KJ; ++j) q_cur[0][j] = X.q[0][j];
      }
    }
    compute_step<D, CAUSAL, QT>(a, citem, cs, X, q_cur, st, col, grp);
    if (cs + 1 >= citem.nsteps) {
      finalize_rows<D, 1, false>(a, citem, st, 0, col, grp, fold);
      st.reset();
      if (++ci >= i_end) return false;
      cs = 0;
      citem = load_item(a, ci);
    } else {
      ++cs;
    }
    return true;
  };

  // the ring, unrolled and named so that it stays in registers
  if constexpr (RING == 4) {
    TileT TA, TB, TC, TD;
    issue(TA);
    issue(TB);
    issue(TC);
    while (advance(TA, TD) && advance(TB, TA) && advance(TC, TB) && advance(TD, TC)) {
    }
  } else {
    TileT TA, TB;
    issue(TA);
    while (advance(TA, TB) && advance(TB, TA)) {
    }
  }
  fused_merge_end<D>(a, i_begin, i_end, lane, fold);
}

}  // namespace dec
}  // namespace fi
