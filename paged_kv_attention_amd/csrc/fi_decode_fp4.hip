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
// applied by the instruction (measured on MI355X for every byte, selector
// and scale code: exact, bf16 overflow to infinity, scale 255 -> NaN), and the
// bf16 MFMA tiling of the bf16 decode kernel is reused unchanged: no scale is
// folded into the softmax.
//
// Staging. A 32-token step is 4.3 KB here against 16 KB in bf16, and the
// operand layout wants 4 bytes of V per lane and token, so loading straight
// into registers takes 16 small loads per step. Instead each wave stages its
// steps in its own LDS ring (no sharing and no barriers between waves) with
// direct global->LDS copies: per step two 1-KiB copies of K codes (one at
// D = 64), two of V codes and one of the K and V scale words, each lane
// fetching 16 (scales: 4) bytes of its own address. The wait for a step is
// an explicit vmcnt count of the copies issued after it. K rows keep their
// 16-byte chunks XOR-swizzled by the token and V rows are placed rotated
// within groups of four tokens, so the operand reads (16 lanes on one chunk
// of 16 tokens; 4 lane groups on 4 different tokens) spread over the banks.
//
// Occupancy. The widening, the V transpose and the softmax make this kernel
// bound by VALU issue and latency rather than by HBM, so it gains from more
// than one wave per SIMD: the ring is 8 stages deep when the plan has up to 7
// workers per CU (one wave per SIMD), 4 with 8 to 11 (two workgroups of 68 KiB
// per CU) and 3 with 12 or more (three of 51 KiB). The MFMA accumulators stay
// in VGPRs (this file is compiled with the VGPR form of MFMA): in AGPRs the
// compiler moved all of them between the register files on every step.
//
// Lanes. K: lane group g takes dims [g*D/4, (g+1)*D/4) of its token (D/8
// contiguous bytes, inside one scale block at D = 128, half of one at 64), and
// MFMA j of q.K uses code bytes 4j..4j+3 of that run; q is loaded in the same
// dim order. V: lane col takes dims D/16*col .. +D/16 of the lane group's 8
// tokens (inside one scale block), widened and transposed in registers as in
// the bf16 kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_device.h"

namespace fi {
namespace {

using namespace dev;

typedef __attribute__((address_space(3))) void* lds_vptr;
typedef const __attribute__((address_space(1))) void* global_vptr;

constexpr int kWaves4 = WAVES_PER_BLOCK;

template <int D>
struct F4 {
  static constexpr int CB = D / 2;           // code bytes per token row
  static constexpr int SB = D / 32;          // scale bytes per token row
  static constexpr int NCH = CB / 16;        // 16-byte chunks per row (4 or 2)
  static constexpr int TPC = 64 / NCH;       // tokens per 1-KiB copy (16 or 32)
  static constexpr int NKC = 32 / TPC;       // copies per step of K (or V) codes
  static constexpr int NCOPY = 2 * NKC + 1;  // copies per step in all
  static constexpr int AREA = 32 * CB;       // K (or V) codes of a step
  static constexpr int SCALES = 2 * AREA;    // offset of the scale words: K, then V
  static constexpr int STAGE = 2 * AREA + 256;
  static constexpr int KJ = D / 32;          // q.K MFMAs per 16-token block
  static constexpr int DPL = D / 16;         // V dims per lane = P.V MFMAs
};

// LDS row of token t (0..31) in a V area: rotated within its group of four,
// so that the four tokens 4g + i (g = 0..3) of one operand read fall in four
// different quarters of the bank space; and its inverse.
__device__ __forceinline__ int v_row_of(int t) { return (t & ~3) | ((t + (t >> 2)) & 3); }
__device__ __forceinline__ int v_token_of(int r) { return (r & ~3) | (((r & 3) - (r >> 2)) & 3); }

// s_waitcnt vmcnt(n) with no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// This lane's part of every copy of a step, fixed for the kernel: the page of
// the step (0..NP-1) its bytes come from and their offset in that page's
// tile, in token rows of the tile (slot) and bytes within the row.
template <int D, int NP>
struct Lanes4 {
  static constexpr int NKC = F4<D>::NKC, NCH = F4<D>::NCH, CB = F4<D>::CB, SB = F4<D>::SB;
  static constexpr int TPP = 32 / NP;          // tokens of the step per page
  int kn[NKC], vn[NKC], sn;
  uint32_t koff[NKC], voff[NKC], soff;          // byte offsets in the code / scale tile
  bool s_is_v;
  __device__ __forceinline__ Lanes4(int lane) {
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      const int p = c * 64 + lane;               // 16-byte slot of the area
      const int r = p / NCH, cs = p % NCH;       // LDS row and chunk slot
      const int tk = r, chk = cs ^ (tk % NCH);   // K: row = token, chunk swizzled
      const int tv = v_token_of(r);              // V: rotated rows, chunks in order
      kn[c] = tk / TPP;
      vn[c] = tv / TPP;
      koff[c] = (uint32_t)((tk % TPP) * CB + chk * 16);
      voff[c] = (uint32_t)((tv % TPP) * CB + cs * 16);
    }
    // scale words: D = 128, one 4-byte word per token (lanes 0..31 K, 32..63
    // V); D = 64, the 2-byte scales of tokens 2j, 2j+1 (lanes 0..15 K, 16..31
    // V, 32..63 repeat 0..31 into spare bytes)
    const int sl = SB == 4 ? lane : (lane & 31);
    const int half = SB == 4 ? 32 : 16;
    s_is_v = sl >= half;
    const int ts = SB == 4 ? (sl & 31) : 2 * (sl & 15);
    sn = ts / TPP;
    soff = (uint32_t)((ts % TPP) * SB);
  }
};

// The first token row of page n (0..NP-1) of the step, selected per lane
// from the step's (wave-uniform) page rows r0..r3 by the bits of n; written
// as selects so that no indexed array (which the compiler may move to LDS) is
// formed.
template <int NP>
__device__ __forceinline__ int64_t pick(int64_t r0, int64_t r1, int64_t r2, int64_t r3, int n) {
  if (NP == 1) return r0;
  if (NP == 2) return (n & 1) ? r1 : r0;
  const int64_t lo = (n & 1) ? r1 : r0, hi = (n & 1) ? r3 : r2;
  return (n & 2) ? hi : lo;
}

// Copy step s of item it into LDS stage `st`. valid = false (past the end of
// the stream): the same number of copies, every lane at the step's first
// bytes (in bounds, next to no HBM traffic), into a stage never read again.
template <int D, int NP>
__device__ __forceinline__ void issue_copies(const AttnArgs& a, const Item& it, int s, char* st,
                                             const Lanes4<D, NP>& ln, bool valid) {
  constexpr int NKC = F4<D>::NKC, CB = F4<D>::CB, SB = F4<D>::SB, AREA = F4<D>::AREA;
  const int sh = a.page_shift;
  const int T0 = it.t_begin + 32 * s;
  const int pb = T0 >> sh;
  const int plast = (it.t_end - 1) >> sh;
  // first token row of each page tile of the step
  auto page_row = [&](int n) -> int64_t {
    if (n >= NP) return 0;
    const int pid = ld_uniform(it.plist, min(pb + n, plast));
    return ((int64_t)pid * a.num_kv_heads + it.g) * a.page_size;
  };
  int64_t r0 = page_row(0);
  const int64_t r1 = page_row(1), r2 = page_row(2), r3 = page_row(3);
  if (NP == 1) r0 += T0 & (a.page_size - 1);
  const char* kc = (const char*)a.k_cache;
  const char* vc = (const char*)a.v_cache;
#pragma unroll
  for (int c = 0; c < NKC; ++c) {
    const char* kp = kc + pick<NP>(r0, r1, r2, r3, valid ? ln.kn[c] : 0) * CB + (valid ? ln.koff[c] : 0u);
    __builtin_amdgcn_global_load_lds((global_vptr)kp, (lds_vptr)(st + c * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < NKC; ++c) {
    const char* vp = vc + pick<NP>(r0, r1, r2, r3, valid ? ln.vn[c] : 0) * CB + (valid ? ln.voff[c] : 0u);
    __builtin_amdgcn_global_load_lds((global_vptr)vp, (lds_vptr)(st + AREA + c * 1024), 16, 0, 0);
  }
  const uint8_t* sbase = ln.s_is_v ? a.v_bscale : a.k_bscale;
  const uint8_t* sp = sbase + pick<NP>(r0, r1, r2, r3, valid ? ln.sn : 0) * SB + (valid ? ln.soff : 0u);
  __builtin_amdgcn_global_load_lds((global_vptr)sp, (lds_vptr)(st + F4<D>::SCALES), 4, 0, 0);
}

template <int D>
__device__ __forceinline__ void load_q4(const AttnArgs& a, const Item& it, u32x4 (&q)[F4<D>::KJ],
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
  for (int j = 0; j < F4<D>::KJ; ++j) q[j] = *(const u32x4*)(qp + 8 * j);
}

// Two E2M1 codes of byte SEL of w -> two bf16 (a dword), scaled by the E8M0
// scale whose exponent field `scale` carries; used as whole dwords only.
template <int SEL>
__device__ __forceinline__ uint32_t widen2(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}

// The fp32 whose exponent field is byte `b` of w: the instruction applies
// only a scale's exponent, which is what an E8M0 scale is.
__device__ __forceinline__ float e8m0(uint32_t w, uint32_t shift) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ubfe(w, shift, 8) << 23);
}

template <int N> struct KRaw;
template <> struct KRaw<4> { typedef u32x4 T; };
template <> struct KRaw<2> { typedef u32x2 T; };

template <int D>
__device__ __forceinline__ void compute_step4(const AttnArgs& a, const Item& it, int s,
                                              const char* st, const u32x4 (&qf)[F4<D>::KJ],
                                              State<D, 1>& st_, int col, int grp) {
  constexpr int KJ = F4<D>::KJ, DPL = F4<D>::DPL, CB = F4<D>::CB, NCH = F4<D>::NCH;
  constexpr int AREA = F4<D>::AREA;
  typedef typename KRaw<KJ>::T kraw_t;
  typedef typename Cfg<D>::vrow_t vrow_t;
  const int T0 = it.t_begin + 32 * s;
  const bool tail = T0 + 32 > it.t_end;
  const uint32_t* sw = (const uint32_t*)(st + F4<D>::SCALES);
  // q.K: the lane's K dims lie in scale block grp (D = 128) or grp / 2 (D = 64)
  const int ch = D == 128 ? grp : grp >> 1;       // 16-byte chunk of the row
  const int sub = D == 128 ? 0 : 8 * (grp & 1);   // byte within it (D = 64)
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int t = 16 * blk + col;
    const kraw_t kw = *(const kraw_t*)(st + t * CB + 16 * (ch ^ (t % NCH)) + sub);
    const float sc = D == 128 ? e8m0(sw[t], 8 * grp)
                              : e8m0(sw[t >> 1], 16 * (t & 1) + 8 * (grp >> 1));
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const uint32_t w = kw[j];
      const u32x4 k4 = {widen2<0>(w, sc), widen2<1>(w, sc), widen2<2>(w, sc), widen2<3>(w, sc)};
      if (blk == 0) s0 = mfma_bf16(k4, qf[j], s0);
      else s1 = mfma_bf16(k4, qf[j], s1);
    }
  }
  // V rows: tokens 4*grp + i (i < 4) and 16 + 4*grp + (i - 4); the lane's
  // dims lie in scale block DPL*col/32. Tokens past the item's end (their
  // scales may be anything, even NaN) are widened at scale 1, so that their
  // values are finite (E2M1 codes are) and p = 0 cancels them.
  const char* vst = st + AREA;
  const uint32_t* vsw = sw + (D == 128 ? 32 : 16);
  const int vshift = 8 * ((DPL * col) >> 5);
  uint32_t vsc[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int tb = 16 * h + 4 * grp;
    if constexpr (D == 128) {
      const u32x4 w4 = *(const u32x4*)(vsw + tb);
#pragma unroll
      for (int i = 0; i < 4; ++i) vsc[4 * h + i] = w4[i];
    } else {
      const u32x2 w2 = *(const u32x2*)(vsw + (tb >> 1));
#pragma unroll
      for (int i = 0; i < 4; ++i) vsc[4 * h + i] = w2[i >> 1] >> (16 * (i & 1));
    }
  }
  if (tail) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tl = (i < 4) ? 4 * grp + i : 16 + 4 * grp + (i - 4);
      if (T0 + tl >= it.t_end) vsc[i] = 0x7f7f7f7fu;   // 127 in every byte: 2^0
    }
  }
  vrow_t vv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tl = (i < 4) ? 4 * grp + i : 16 + 4 * grp + (i - 4);
    const char* vp = vst + v_row_of(tl) * CB + (DPL / 2) * col;
    const uint32_t w = DPL == 8 ? *(const uint32_t*)vp : (uint32_t)(*(const uint16_t*)vp);
    const float sc = e8m0(vsc[i], vshift);
    vrow_t row;
    if constexpr (DPL == 8) {
      row = vrow_t{widen2<0>(w, sc), widen2<1>(w, sc), widen2<2>(w, sc), widen2<3>(w, sc)};
    } else {
      row = vrow_t{widen2<0>(w, sc), widen2<1>(w, sc)};
    }
    vv[i] = row;
  }
  u32x4 vt[DPL];
  transpose_v<D>(vv, vt);
  softmax_pv<D, 1>(st_, 0, s0, s1, vt, a.scale_log2, tail, T0, it.t_end - 1, grp);
}

// R: LDS stages per wave. 8 with one wave per SIMD (136 KiB per workgroup
// at D = 128); 4 when plans give eight workers per CU, so that two
// workgroups, two waves per SIMD, share a CU.
template <int D, int NP, int R>
__global__ __launch_bounds__(256) void decode_mxfp4_kernel(AttnArgs a) {
  constexpr int KJ = F4<D>::KJ, STAGE = F4<D>::STAGE, kRing4 = R;
  __shared__ __attribute__((aligned(1024))) char lds[kWaves4 * kRing4 * STAGE];
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int wave = uniform(threadIdx.x >> 6);
  const int w = blockIdx.x * kWaves4 + wave;
  // first loads in one round trip (as in the bf16 decode worker)
  const int nw = a.num_workers;
  const int i_begin = ld_uniform(a.worker_indptr, min(w, nw));
  const int i_end = ld_uniform(a.worker_indptr, min(w + 1, nw));
  const int n_empty = ld_uniform(a.meta, META_EMPTY);
  if (w >= nw) return;
  fused_merge_start<D>(a, w, lane, n_empty);
  if (i_begin >= i_end) {   // (a workgroup-folded plan's barrier needs every wave)
    fused_merge_end<D>(a, i_begin, i_end, lane);
    return;
  }
  char* ring = lds + wave * (kRing4 * STAGE);
  const Lanes4<D, NP> ln(lane);

  // Issue cursor (ii, is) kRing4-1 steps ahead of the compute cursor (ci, cs)
  // across item boundaries; stages are filled and consumed in the same order.
  int ci = i_begin, cs = 0;
  Item citem = load_item(a, ci);
  int ii = i_begin, is = 0;
  Item iitem = citem;
  u32x4 q_cur[KJ];
  State<D, 1> st;
  st.reset();

  auto issue = [&](int y) {
    const bool valid = ii < i_end;
    issue_copies<D, NP>(a, valid ? iitem : citem, valid ? is : cs, ring + y * STAGE, ln, valid);
    if (valid && ++is >= iitem.nsteps) {
      ++ii;
      is = 0;
      if (ii < i_end) iitem = load_item(a, ii);
    }
  };

  // Compute stage x once its copies have landed (at least kRing4-2 steps'
  // copies were issued after them, maybe also the stores of finished items,
  // which only make the wait stricter), then refill stage y, the one computed
  // before x. An item's q is loaded when its first step is computed: with
  // copies to LDS in flight, the compiler's wait for a register load waits
  // for every outstanding load, so the ring drains once per item either way,
  // and q held per stage would cost the registers that keep the accumulators
  // out of the AGPRs.
  constexpr int kPerStep = F4<D>::NCOPY;
  static_assert((kRing4 - 2) * kPerStep < 64, "vmcnt range");
  auto advance = [&](int x, int y) -> bool {
    wait_vmcnt<(kRing4 - 2) * kPerStep>();
    if (cs == 0) {
      load_q4<D>(a, citem, q_cur, col, grp);
      // take the wait for q here, on this path only, rather than at its use
      // after the paths join (where it would drain the ring on every step)
#pragma unroll
      for (int j = 0; j < KJ; ++j) asm volatile("" : "+v"(q_cur[j]));
    }
    compute_step4<D>(a, citem, cs, ring + x * STAGE, q_cur, st, col, grp);
    bool more = true;
    if (cs + 1 >= citem.nsteps) {
      finalize_rows<D, 1, false>(a, citem, st, 0, col, grp);
      st.reset();
      if (++ci >= i_end) more = false;
      else {
        cs = 0;
        citem = load_item(a, ci);
      }
    } else {
      ++cs;
    }
    if (more) issue(y);
    return more;
  };

  for (int k = 0; k < kRing4 - 1; ++k) issue(k);
  // unrolled so that every stage offset is a constant
  if constexpr (kRing4 == 8) {
    while (advance(0, 7) && advance(1, 0) && advance(2, 1) && advance(3, 2) && advance(4, 3) &&
           advance(5, 4) && advance(6, 5) && advance(7, 6)) {
    }
  } else if constexpr (kRing4 == 4) {
    while (advance(0, 3) && advance(1, 0) && advance(2, 1) && advance(3, 2)) {
    }
  } else {
    static_assert(kRing4 == 3, "rings of three, four or eight stages");
    while (advance(0, 2) && advance(1, 0) && advance(2, 1)) {
    }
  }
  // drain this wave's copies before it exits (the stages are its own)
  wait_vmcnt<0>();
  fused_merge_end<D>(a, i_begin, i_end, lane);
}

template <int D, int R>
hipError_t launch_f4(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.page_size == 8) {
    launch_timed((decode_mxfp4_kernel<D, 4, R>), grid, dim3(256), s, a);
  } else if (a.page_size == 16) {
    launch_timed((decode_mxfp4_kernel<D, 2, R>), grid, dim3(256), s, a);
  } else {
    launch_timed((decode_mxfp4_kernel<D, 1, R>), grid, dim3(256), s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mxfp4(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const int blocks = (a.num_workers + kWaves4 - 1) / kWaves4;
  if (blocks == 0) return hipSuccess;
  // workers per CU of the plan, against this device's CU count
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int per_cu = cus > 0 ? a.num_workers / cus : 0;
  if (head_dim == 128)
    return per_cu >= 12 ? launch_f4<128, 3>(a, dim3(blocks), stream)
         : per_cu >= 8  ? launch_f4<128, 4>(a, dim3(blocks), stream)
                        : launch_f4<128, 8>(a, dim3(blocks), stream);
  if (head_dim == 64)
    return per_cu >= 12 ? launch_f4<64, 3>(a, dim3(blocks), stream)
         : per_cu >= 8  ? launch_f4<64, 4>(a, dim3(blocks), stream)
                        : launch_f4<64, 8>(a, dim3(blocks), stream);
  return hipErrorInvalidValue;
}

}  // namespace fi
