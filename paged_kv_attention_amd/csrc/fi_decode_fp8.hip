// fi_decode_fp8.hip -- paged decode attention over an FP8 KV cache (gfx950).
//
// The v0.7.4 article ("FlashInfer v0.7.4 Adds Rubin MoE Kernels and a
// Batch-Invariant Mode", TL;DR and "FlashInfer v0.7.4 ships Rubin kernels and
// bit-exact GEMMs") lists decoding from a low-precision (NVFP4) KV cache; on a
// bandwidth-bound path the point is fewer bytes per token. This kernel reads K
// and V stored as FP8 E4M3 codes (the OCP 8-bit floating-point format, the
// one gfx950 converts natively) with one fp32 scale per (page, kv head) for K
// and one for V: value = decode(code) * scale. Half the bytes of bf16.
//
// Every E4M3 value is exact in bf16, so the codes are widened to bf16 with
// v_cvt_scalef32_pk_bf16_fp8 (unit scale) and the bf16 MFMA tiling of the
// bf16 decode kernel is reused. The scales are folded in fp32: the K scale of
// a token's page into its logit's scale, the V scale into its p (the row sum
// l uses the unscaled p); p * v_scale enters P.V as two bf16 parts.
//
// Lanes. K: the contraction order over the head dim is free, so lane group g
// takes dims [g*D/4, (g+1)*D/4) of its token, D/4 contiguous bytes (two 16-byte
// loads at D = 128), and MFMA j of q.K uses bytes 8j..8j+7 of that run; q is
// loaded in the same dim order. V: lane col takes dims D/16*col .. +D/16 of
// the lane group's 8 tokens (the S^T token order), widened to bf16 and
// transposed in registers as in the bf16 kernel.
//
// Pages, clamping, the item stream and the prefetch ring follow the bf16
// decode kernel; with half the bytes per step the ring is six tiles deep so
// the bytes in flight per wave stay about the same.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_device.h"

namespace fi {
namespace {

using namespace dev;

constexpr int kRing8 = 6;

template <int W> struct Words;
template <> struct Words<2> { typedef u32x2 T; };
template <> struct Words<1> { typedef uint32_t T; };

template <int D>
struct C8 {
  static constexpr int KJ = D / 32;          // q.K MFMAs per 16-token block
  static constexpr int KV4 = D / 64;         // 16-byte K loads per lane and token
  static constexpr int DPL = D / 16;         // V dims per lane = P.V MFMAs
  typedef typename Words<DPL / 4>::T vraw_t; // DPL codes of one V row
};

template <int D>
struct Tile8 {
  u32x4 k[2][C8<D>::KV4];
  typename C8<D>::vraw_t v[8];
  float ks[2], vs[2];     // scales of this lane's two token halves
  u32x4 q[C8<D>::KJ];     // the item's q, on its first step only
};

// Two E4M3 codes (the low or high 16 bits of w) -> two bf16 in one dword. The
// result is only ever used as a whole dword.
template <bool HI>
__device__ __forceinline__ uint32_t widen2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ float ld_uniform_f(const float* p, int64_t i) {
  return __builtin_bit_cast(float, ld_uniform((const int32_t*)p, i));
}

template <int D, int NP>
__device__ __forceinline__ void issue_step8(const AttnArgs& a, const Item& it, int s,
                                            Tile8<D>& T, int col, int grp) {
  constexpr int KV4 = C8<D>::KV4, DPL = C8<D>::DPL;
  typedef typename C8<D>::vraw_t vraw_t;
  const int sh = a.page_shift;
  const int T0 = it.t_begin + 32 * s;
  const int pb = T0 >> sh;
  const int plast = (it.t_end - 1) >> sh;
  const int64_t tile_bytes = (int64_t)a.page_size * D;
  const char* kb[NP];
  const char* vb[NP];
  float ks[NP], vs[NP];
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    const int pid = ld_uniform(it.plist, min(pb + n, plast));
    const int64_t ph = (int64_t)pid * a.num_kv_heads + it.g;
    kb[n] = (const char*)a.k_cache + ph * tile_bytes;
    vb[n] = (const char*)a.v_cache + ph * tile_bytes;
    ks[n] = ld_uniform_f(a.k_scale, ph);
    vs[n] = ld_uniform_f(a.v_scale, ph);
  }
  // pages of this lane's tokens 4g..4g+3 and 16+4g..16+4g+3
  if constexpr (NP == 1) {
    T.ks[0] = T.ks[1] = ks[0];
    T.vs[0] = T.vs[1] = vs[0];
  } else if constexpr (NP == 2) {
    T.ks[0] = ks[0];
    T.ks[1] = ks[1];
    T.vs[0] = vs[0];
    T.vs[1] = vs[1];
  } else {
    T.ks[0] = (grp >> 1) ? ks[1] : ks[0];
    T.ks[1] = (grp >> 1) ? ks[NP - 1] : ks[NP - 2];
    T.vs[0] = (grp >> 1) ? vs[1] : vs[0];
    T.vs[1] = (grp >> 1) ? vs[NP - 1] : vs[NP - 2];
  }
  const int slot0 = (NP == 1) ? (T0 & (a.page_size - 1)) : 0;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {   // K: token 16*blk + col, bytes [grp*D/4, +D/4)
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
    const uint32_t off = (uint32_t)(slot * D + grp * (D / 4));
#pragma unroll
    for (int i = 0; i < KV4; ++i)   // K and V are read once: nontemporal loads
      T.k[blk][i] = __builtin_nontemporal_load((const u32x4*)(base + off + 16u * i));
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
    T.v[i] = __builtin_nontemporal_load((const vraw_t*)(base + (uint32_t)(slot * D + DPL * col)));
  }
}

template <int D>
__device__ __forceinline__ void load_q8(const AttnArgs& a, const Item& it, u32x4 (&q)[C8<D>::KJ],
                                        int col, int grp) {
  // row col of the item (rows past n_rows read row 0; never stored)
  const int G = a.group;
  const int rl = col < it.n_rows ? col : 0;
  const int rho = it.row0 + rl;
  const int qi = rho / G, h = rho - qi * G;
  const uint16_t* qp =
      a.q + ((int64_t)(it.q_base + qi) * a.num_qo_heads + it.g * G + h) * D + grp * (D / 4);
#pragma unroll
  for (int j = 0; j < C8<D>::KJ; ++j) q[j] = *(const u32x4*)(qp + 8 * j);
}

template <int D>
__device__ __forceinline__ void compute_step8(const AttnArgs& a, const Item& it, int s,
                                              const Tile8<D>& T, const u32x4 (&qf)[C8<D>::KJ],
                                              State<D, 1>& st, int grp) {
  constexpr int KJ = C8<D>::KJ, DPL = C8<D>::DPL;
  typedef typename Cfg<D>::vrow_t vrow_t;
  const int T0 = it.t_begin + 32 * s;
  const bool tail = T0 + 32 > it.t_end;
  // q.K on the widened K codes
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int w0 = 2 * j, w1 = 2 * j + 1;   // words of this MFMA's 8 codes
    u32x4 ka, kb;
    ka[0] = widen2<false>(T.k[0][w0 >> 2][w0 & 3]);
    ka[1] = widen2<true>(T.k[0][w0 >> 2][w0 & 3]);
    ka[2] = widen2<false>(T.k[0][w1 >> 2][w1 & 3]);
    ka[3] = widen2<true>(T.k[0][w1 >> 2][w1 & 3]);
    kb[0] = widen2<false>(T.k[1][w0 >> 2][w0 & 3]);
    kb[1] = widen2<true>(T.k[1][w0 >> 2][w0 & 3]);
    kb[2] = widen2<false>(T.k[1][w1 >> 2][w1 & 3]);
    kb[3] = widen2<true>(T.k[1][w1 >> 2][w1 & 3]);
    s0 = mfma_bf16(ka, qf[j], s0);
    s1 = mfma_bf16(kb, qf[j], s1);
  }
  // V rows: tokens past the item's end are zeroed as codes (0 is +0), the
  // rest widened to bf16 rows, then transposed to the V^T operand
  // (only tail steps hold such tokens: the selects are made there alone)
  typename C8<D>::vraw_t vraw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) vraw[i] = T.v[i];
  if (tail) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tl = (i < 4) ? 4 * grp + i : 16 + 4 * grp + (i - 4);
      if (T0 + tl >= it.t_end) vraw[i] = typename C8<D>::vraw_t{};
    }
  }
  vrow_t vv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (DPL == 8) {
      const u32x2 raw = vraw[i];
      vv[i] = vrow_t{widen2<false>(raw[0]), widen2<true>(raw[0]), widen2<false>(raw[1]),
                     widen2<true>(raw[1])};
    } else {
      const uint32_t raw = vraw[i];
      vv[i] = vrow_t{widen2<false>(raw), widen2<true>(raw)};
    }
  }
  u32x4 vt[DPL];
  transpose_v<D>(vv, vt);
  // softmax with per-half scales: logit = s * sm_scale * log2(e) * k_scale
  const float xs0 = a.scale_log2 * T.ks[0], xs1 = a.scale_log2 * T.ks[1];
  float x[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = s0[r] * xs0;
    x[4 + r] = s1[r] * xs1;
  }
  if (tail) {
    const int lim = it.t_end - 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t0 = T0 + 4 * grp + r;
      if (t0 > lim) x[r] = neg_inf();
      if (t0 + 16 > lim) x[4 + r] = neg_inf();
    }
  }
  const float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  // lazy rescale: a wave-wide vote on the lane-local max gates it, and each
  // row (the base is equal across a row's lane groups) moves its base only on
  // its own max, so a row's bits never depend on the block's other rows
  if (__any(mx > st.m[0] + kRescaleSlack)) {
    const float rmax = max_across_groups(mx);
    if (rmax > st.m[0] + kRescaleSlack) {
      const float alpha = (st.m[0] == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(st.m[0] - rmax);
      st.l[0] *= alpha;
#pragma unroll
      for (int m = 0; m < DPL; ++m) st.acc[0][m] *= alpha;
      st.m[0] = rmax;
    }
  }
  const float base = (st.m[0] == neg_inf()) ? 0.f : st.m[0];
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - base);
  st.l[0] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  // p * v_scale as a bf16 pair hi + lo (pv - hi is exact in fp32), so that
  // folding an arbitrary fp32 scale into p adds no rounding of its own: P.V
  // runs once on each part (the matrix cores have room to spare in decode)
  float pv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pv[i] = p[i] * (i < 4 ? T.vs[0] : T.vs[1]);
  u32x4 ph, pl;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ph[k] = pack2(pv[2 * k], pv[2 * k + 1]);
    const float h0 = __builtin_bit_cast(float, ph[k] << 16);
    const float h1 = __builtin_bit_cast(float, ph[k] & 0xffff0000u);
    pl[k] = pack2(pv[2 * k] - h0, pv[2 * k + 1] - h1);
  }
#pragma unroll
  for (int m = 0; m < DPL; ++m) {
    st.acc[0][m] = mfma_bf16(vt[m], ph, st.acc[0][m]);
    st.acc[0][m] = mfma_bf16(vt[m], pl, st.acc[0][m]);
  }
}

template <int D, int NP>
__global__ __launch_bounds__(256) void decode_fp8_kernel(AttnArgs a) {
  constexpr int KJ = C8<D>::KJ;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int w = blockIdx.x * WAVES_PER_BLOCK + uniform(threadIdx.x >> 6);
  if (w >= a.num_workers) return;
  fused_merge_start<D>(a, w, lane);
  const int i_end = ld_uniform(a.worker_indptr, w + 1);
  const int i_begin = ld_uniform(a.worker_indptr, w);
  if (i_begin >= i_end) return;

  // Issue cursor (ii, is) kRing8-1 steps ahead of the compute cursor (ci, cs)
  // across item boundaries; tiles are filled and consumed in the same order.
  int ci = i_begin, cs = 0;
  Item citem = load_item(a, ci);
  int ii = i_begin, is = 0;
  Item iitem = citem;
  Tile8<D> TA, TB, TC, TD, TE, TF;   // the ring, named so it stays in registers
  u32x4 q_cur[KJ];
  State<D, 1> st;
  st.reset();

  auto issue = [&](Tile8<D>& Y) {
    const bool valid = ii < i_end;
    if (valid && is == 0) load_q8<D>(a, iitem, Y.q, col, grp);
    // past the end of the stream: an in-bounds re-load of the current step,
    // every lane at lane 0's addresses (next to no HBM traffic)
    issue_step8<D, NP>(a, valid ? iitem : citem, valid ? is : cs, Y, valid ? col : 0,
                       valid ? grp : 0);
    if (valid && ++is >= iitem.nsteps) {
      ++ii;
      is = 0;
      if (ii < i_end) iitem = load_item(a, ii);
    }
  };

  // Refill Y (the tile computed last), then compute X.
  auto advance = [&](Tile8<D>& X, Tile8<D>& Y) -> bool {
    issue(Y);
    if (cs == 0) {
#pragma unroll
      for (int j = 0; j < KJ; ++j) q_cur[j] = X.q[j];
    }
    compute_step8<D>(a, citem, cs, X, q_cur, st, grp);
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

  static_assert(kRing8 == 6, "the loop below is unrolled for a ring of six tiles");
  issue(TA);
  issue(TB);
  issue(TC);
  issue(TD);
  issue(TE);
  while (advance(TA, TF) && advance(TB, TA) && advance(TC, TB) && advance(TD, TC) &&
         advance(TE, TD) && advance(TF, TE)) {
  }
  fused_merge_end<D>(a, i_begin, i_end, lane);
}

template <int D>
hipError_t launch_f8(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.page_size == 8) {
    launch_timed((decode_fp8_kernel<D, 4>), grid, dim3(256), s, a);
  } else if (a.page_size == 16) {
    launch_timed((decode_fp8_kernel<D, 2>), grid, dim3(256), s, a);
  } else {
    launch_timed((decode_fp8_kernel<D, 1>), grid, dim3(256), s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_fp8(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const int blocks = (a.num_workers + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  if (blocks == 0) return hipSuccess;
  if (head_dim == 128) return launch_f8<128>(a, dim3(blocks), stream);
  if (head_dim == 64) return launch_f8<64>(a, dim3(blocks), stream);
  return hipErrorInvalidValue;
}

}  // namespace fi
