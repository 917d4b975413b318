// fi_decode_fp4.hip -- paged decode attention over an MXFP4 KV cache (gfx950).
//
// The v0.7.4 article ("FlashInfer v0.7.4 Adds Rubin MoE Kernels and a
// Batch-Invariant Mode", TL;DR) lists decoding from a 4-bit (NVFP4) KV cache;
// gfx950's native 4-bit format is MXFP4 (OCP microscaling): FP4 E2M1 elements
// (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives), two per byte, low
// nibble first, and one E8M0 scale (2^(code - 127); code 255 is NaN) per 32
// consecutive elements of a token row. K and V of a (page, kv head) tile are
// codes [page_size][D/2] bytes and scales [page_size][D/32] bytes: 68 bytes
// per token and head at D = 128 against 256 for bf16.
//
// Every element value (an E2M1 value times a power of two) is exact in bf16,
// so codes are widened to bf16 with v_cvt_scalef32_pk_bf16_fp4, the scale
// applied by the instruction (measured on the box for every byte, selector
// and scale code: exact, bf16 overflow to infinity, scale 255 -> NaN), and the
// bf16 MFMA tiling of the bf16 decode kernel is reused unchanged: no scale is
// folded into the softmax.
//
// Lanes. K: lane group g takes dims [g*D/4, (g+1)*D/4) of its token (D/8
// contiguous bytes, inside one scale block at D = 128, half of one at 64), and
// MFMA j of q.K uses code bytes 4j..4j+3 of that run; q is loaded in the same
// dim order. V: lane col takes dims D/16*col .. +D/16 of the lane group's 8
// tokens (inside one scale block), widened and transposed in registers as in
// the bf16 kernel. A token's scales are read as one word (D/32 bytes).
//
// Pages, clamping, the item stream and the prefetch ring follow the bf16
// decode kernel; with about a quarter of the bytes per step the ring is eight
// tiles deep.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_device.h"

namespace fi {
namespace {

using namespace dev;

constexpr int kRing4 = 8;

template <int D>
struct C4 {
  static constexpr int KJ = D / 32;          // q.K MFMAs per 16-token block
  static constexpr int KW = D / 32;          // 4-byte code words per lane and K token
  static constexpr int DPL = D / 16;         // V dims per lane = P.V MFMAs
};

template <int N> struct Vec32;
template <> struct Vec32<4> { typedef u32x4 T; };
template <> struct Vec32<2> { typedef u32x2 T; };

template <int D>
struct Tile4 {
  typename Vec32<C4<D>::KW>::T k[2];   // K codes of tokens 16*blk + col
  uint32_t ks[2];                      // their scale words
  uint32_t v[8];                       // V codes of the lane group's 8 tokens (DPL nibbles)
  uint32_t vs[8];                      // their scale words
  u32x4 q[C4<D>::KJ];                  // the item's q, on its first step only
};

// Four E2M1 codes of byte SEL of w -> ... two bf16 of one byte, scaled by
// 2^(e - 127) (e: an E8M0 code); used as whole dwords only.
template <int SEL>
__device__ __forceinline__ uint32_t widen2(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}

// The fp32 whose exponent field is e: the instruction applies only a scale's
// exponent, which is what an E8M0 scale is.
__device__ __forceinline__ float e8m0(uint32_t e) { return __builtin_bit_cast(float, e << 23); }

template <int D, int NP>
__device__ __forceinline__ void issue_step4(const AttnArgs& a, const Item& it, int s,
                                            Tile4<D>& T, int col, int grp) {
  constexpr int KW = C4<D>::KW, DPL = C4<D>::DPL, CB = D / 2, SB = D / 32;
  typedef typename Vec32<KW>::T kraw_t;
  const int sh = a.page_shift;
  const int T0 = it.t_begin + 32 * s;
  const int pb = T0 >> sh;
  const int plast = (it.t_end - 1) >> sh;
  const char* kb[NP];
  const char* vb[NP];
  const uint8_t* kbs[NP];
  const uint8_t* vbs[NP];
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    const int pid = ld_uniform(it.plist, min(pb + n, plast));
    const int64_t ph = ((int64_t)pid * a.num_kv_heads + it.g) * a.page_size;   // first token row
    kb[n] = (const char*)a.k_cache + ph * CB;
    vb[n] = (const char*)a.v_cache + ph * CB;
    kbs[n] = a.k_bscale + ph * SB;
    vbs[n] = a.v_bscale + ph * SB;
  }
  const int slot0 = (NP == 1) ? (T0 & (a.page_size - 1)) : 0;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {   // K: token 16*blk + col, code bytes [grp*D/8, +D/8)
    int n, slot;
    if (NP == 1) {
      n = 0;
      slot = slot0 + 16 * blk + col;
    } else if (NP == 2) {
      n = blk;
      slot = col;
    } else {
      n = 2 * blk + (col >> 3);
      slot = col & 7;
    }
    const char* base = NP == 4 ? ((col >> 3) ? kb[2 * blk + 1] : kb[2 * blk]) : kb[n];
    const uint8_t* sbase = NP == 4 ? ((col >> 3) ? kbs[2 * blk + 1] : kbs[2 * blk]) : kbs[n];
    T.k[blk] = __builtin_nontemporal_load((const kraw_t*)(base + slot * CB + grp * (D / 8)));
    T.ks[blk] = SB == 4 ? __builtin_nontemporal_load((const uint32_t*)(sbase + slot * SB))
                        : (uint32_t)__builtin_nontemporal_load((const uint16_t*)(sbase + slot * SB));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {   // V: tokens 4*grp + i and 16 + 4*grp + (i - 4)
    const int tl = (i < 4) ? 4 * grp + i : 16 + 4 * grp + (i - 4);
    const char* base;
    const uint8_t* sbase;
    int slot;
    if (NP == 1) {
      base = vb[0];
      sbase = vbs[0];
      slot = slot0 + tl;
    } else if (NP == 2) {
      base = vb[i >> 2];
      sbase = vbs[i >> 2];
      slot = tl & 15;
    } else {
      base = (grp >> 1) ? vb[2 * (i >> 2) + 1] : vb[2 * (i >> 2)];
      sbase = (grp >> 1) ? vbs[2 * (i >> 2) + 1] : vbs[2 * (i >> 2)];
      slot = tl & 7;
    }
    const char* vp = base + slot * CB + (DPL / 2) * col;
    T.v[i] = DPL == 8 ? __builtin_nontemporal_load((const uint32_t*)vp)
                      : (uint32_t)__builtin_nontemporal_load((const uint16_t*)vp);
    T.vs[i] = SB == 4 ? __builtin_nontemporal_load((const uint32_t*)(sbase + slot * SB))
                      : (uint32_t)__builtin_nontemporal_load((const uint16_t*)(sbase + slot * SB));
  }
}

template <int D>
__device__ __forceinline__ void load_q4(const AttnArgs& a, const Item& it, u32x4 (&q)[C4<D>::KJ],
                                        int col, int grp) {
  // row col of the item (rows past n_rows read row 0; never stored); dims
  // grp*D/4 + 8j .. +7 feed MFMA j
  const int G = a.group;
  const int rl = col < it.n_rows ? col : 0;
  const int rho = it.row0 + rl;
  const int qi = rho / G, h = rho - qi * G;
  const uint16_t* qp =
      a.q + ((int64_t)(it.q_base + qi) * a.num_qo_heads + it.g * G + h) * D + grp * (D / 4);
#pragma unroll
  for (int j = 0; j < C4<D>::KJ; ++j) q[j] = *(const u32x4*)(qp + 8 * j);
}

template <int D>
__device__ __forceinline__ void compute_step4(const AttnArgs& a, const Item& it, int s,
                                              const Tile4<D>& T, const u32x4 (&qf)[C4<D>::KJ],
                                              State<D, 1>& st, int col, int grp) {
  constexpr int KJ = C4<D>::KJ, DPL = C4<D>::DPL;
  typedef typename Cfg<D>::vrow_t vrow_t;
  const int T0 = it.t_begin + 32 * s;
  const bool tail = T0 + 32 > it.t_end;
  // q.K: the lane's K dims lie in scale block grp (D = 128) or grp / 2 (D = 64)
  const int kshift = 8 * (D == 128 ? grp : grp >> 1);
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const float sc = e8m0((T.ks[blk] >> kshift) & 0xffu);
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const uint32_t w = T.k[blk][j];
      const u32x4 kw = {widen2<0>(w, sc), widen2<1>(w, sc), widen2<2>(w, sc), widen2<3>(w, sc)};
      if (blk == 0) s0 = mfma_bf16(kw, qf[j], s0);
      else s1 = mfma_bf16(kw, qf[j], s1);
    }
  }
  // V rows: the lane's dims lie in scale block DPL*col/32; tokens past the
  // item's end are zeroed after widening (their codes and scales may be NaN)
  const int vshift = 8 * ((DPL * col) >> 5);
  vrow_t vv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tl = (i < 4) ? 4 * grp + i : 16 + 4 * grp + (i - 4);
    const float sc = e8m0((T.vs[i] >> vshift) & 0xffu);
    vrow_t row;
    if constexpr (DPL == 8) {
      row = vrow_t{widen2<0>(T.v[i], sc), widen2<1>(T.v[i], sc), widen2<2>(T.v[i], sc),
                   widen2<3>(T.v[i], sc)};
    } else {
      row = vrow_t{widen2<0>(T.v[i], sc), widen2<1>(T.v[i], sc)};
    }
    vv[i] = (T0 + tl < it.t_end) ? row : vrow_t{};
  }
  u32x4 vt[DPL];
  transpose_v<D>(vv, vt);
  softmax_pv<D, 1>(st, 0, s0, s1, vt, a.scale_log2, tail, T0, it.t_end - 1, grp);
}

template <int D, int NP>
__global__ __launch_bounds__(256) void decode_mxfp4_kernel(AttnArgs a) {
  constexpr int KJ = C4<D>::KJ;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int w = blockIdx.x * WAVES_PER_BLOCK + uniform(threadIdx.x >> 6);
  if (w >= a.num_workers) return;
  const int i_end = ld_uniform(a.worker_indptr, w + 1);
  const int i_begin = ld_uniform(a.worker_indptr, w);
  if (i_begin >= i_end) return;

  // Issue cursor (ii, is) kRing4-1 steps ahead of the compute cursor (ci, cs)
  // across item boundaries; tiles are filled and consumed in the same order.
  int ci = i_begin, cs = 0;
  Item citem = load_item(a, ci);
  int ii = i_begin, is = 0;
  Item iitem = citem;
  Tile4<D> TA, TB, TC, TD, TE, TF, TG, TH;   // the ring, named so it stays in registers
  u32x4 q_cur[KJ];
  State<D, 1> st;
  st.reset();

  auto issue = [&](Tile4<D>& Y) {
    const bool valid = ii < i_end;
    if (valid && is == 0) load_q4<D>(a, iitem, Y.q, col, grp);
    // past the end of the stream: an in-bounds re-load of the current step,
    // every lane at lane 0's addresses (next to no HBM traffic)
    issue_step4<D, NP>(a, valid ? iitem : citem, valid ? is : cs, Y, valid ? col : 0,
                       valid ? grp : 0);
    if (valid && ++is >= iitem.nsteps) {
      ++ii;
      is = 0;
      if (ii < i_end) iitem = load_item(a, ii);
    }
  };

  // Refill Y (the tile computed last), then compute X.
  auto advance = [&](Tile4<D>& X, Tile4<D>& Y) -> bool {
    issue(Y);
    if (cs == 0) {
#pragma unroll
      for (int j = 0; j < KJ; ++j) q_cur[j] = X.q[j];
    }
    compute_step4<D>(a, citem, cs, X, q_cur, st, col, grp);
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

  static_assert(kRing4 == 8, "the loop below is unrolled for a ring of eight tiles");
  issue(TA);
  issue(TB);
  issue(TC);
  issue(TD);
  issue(TE);
  issue(TF);
  issue(TG);
  while (advance(TA, TH) && advance(TB, TA) && advance(TC, TB) && advance(TD, TC) &&
         advance(TE, TD) && advance(TF, TE) && advance(TG, TF) && advance(TH, TG)) {
  }
}

template <int D>
hipError_t launch_f4(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.page_size == 8) {
    hipLaunchKernelGGL((decode_mxfp4_kernel<D, 4>), grid, dim3(256), 0, s, a);
  } else if (a.page_size == 16) {
    hipLaunchKernelGGL((decode_mxfp4_kernel<D, 2>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((decode_mxfp4_kernel<D, 1>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mxfp4(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const int blocks = (a.num_workers + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  if (blocks == 0) return hipSuccess;
  if (head_dim == 128) return launch_f4<128>(a, dim3(blocks), stream);
  if (head_dim == 64) return launch_f4<64>(a, dim3(blocks), stream);
  return hipErrorInvalidValue;
}

}  // namespace fi
