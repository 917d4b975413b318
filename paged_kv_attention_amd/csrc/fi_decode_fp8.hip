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
// Staging. Each wave streams its steps through its own ring of LDS stages
// (no sharing, no barriers between waves) with direct global->LDS copies: per
// step the K codes (four 1-KiB copies at D = 128, two at 64), the V codes
// (the same) and one copy of the step's page scales, each lane fetching 16
// (scales: 4) bytes at an address of its own. The wait for a step is an
// explicit vmcnt count of the copies issued after it. (Staged in registers
// instead, the widening needs the codes in VGPRs while the ring overflows
// into AGPRs, and the compiler's copies between the two files wait for loads
// issued one step earlier: the ring drains every step.) K rows keep their
// 16-byte chunks XOR-swizzled by the token and V rows are placed rotated
// within groups of four tokens, so that the operand reads (16 lanes on one
// chunk of 16 tokens; 4 lane groups on 4 different tokens) spread over the
// banks. The page ids of a step are loaded one issue ahead, so that their
// scalar round trip is not in front of the step's copies.
//
// Lanes. K: the contraction order over the head dim is free, so lane group g
// takes dims [g*D/4, (g+1)*D/4) of its token, D/4 contiguous bytes (two
// 16-byte chunks at D = 128), and MFMA j of q.K uses bytes 8j..8j+7 of that
// run; q is loaded in the same dim order. V: lane col takes dims
// D/16*col .. +D/16 of the lane group's 8 tokens (the S^T token order),
// widened to bf16 and transposed in registers as in the bf16 kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_device.h"

namespace fi {
namespace {

using namespace dev;

typedef __attribute__((address_space(3))) void* lds_vptr;
typedef const __attribute__((address_space(1))) void* global_vptr;

template <int W> struct Words;
template <> struct Words<2> { typedef u32x2 T; };
template <> struct Words<1> { typedef uint32_t T; };

template <int D>
struct C8 {
  static constexpr int KJ = D / 32;          // q.K MFMAs per 16-token block
  static constexpr int KV4 = D / 64;         // 16-byte K chunks per lane and token
  static constexpr int DPL = D / 16;         // V dims per lane = P.V MFMAs
  static constexpr int ROW = D;              // bytes per K (or V) row
  static constexpr int NCH = D / 16;         // 16-byte chunks per row
  static constexpr int RPW = 256 / D;        // rows per 256-byte span of the banks
  static constexpr int TPC = 1024 / D;       // rows per 1-KiB copy
  static constexpr int NKC = 32 / TPC;       // copies per step of K (or V) codes
  static constexpr int NCOPY = 2 * NKC + 1;  // copies per step in all
  static constexpr int AREA = 32 * ROW;      // K (or V) codes of a step
  static constexpr int SCALES = 2 * AREA;    // the step's scales: K of its pages, then V
  static constexpr int STAGE = 2 * AREA + 256;
  typedef typename Words<DPL / 4>::T vraw_t;
};

// One step's operands as read from its stage.
template <int D>
struct Frag8 {
  u32x4 k[2][C8<D>::KV4];
  typename C8<D>::vraw_t v[8];
  float ks[2], vs[2];     // scales of this lane's two token halves
};

// K: chunk c of token t sits at chunk slot c ^ k_swz(t) of row t; the 16
// tokens read together then cover the 256-byte bank span once.
template <int D>
__device__ __forceinline__ int k_swz(int t) {
  return (t / C8<D>::RPW) % C8<D>::NCH;
}

// V: row of token t (0..31), rotated within its group of four so that the
// tokens 4g + i (g = 0..3) of one operand read fall in different parts of the
// bank span; and its inverse.
__device__ __forceinline__ int v_row_of(int t) { return (t & ~3) | ((t + (t >> 2)) & 3); }
__device__ __forceinline__ int v_token_of(int r) { return (r & ~3) | (((r & 3) - (r >> 2)) & 3); }

// Two E4M3 codes (the low or high 16 bits of w) -> two bf16 in one dword. The
// result is only ever used as a whole dword.
template <bool HI>
__device__ __forceinline__ uint32_t widen2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// s_waitcnt vmcnt(n) with no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// This lane's part of every copy of a step, fixed for the kernel: the page of
// the step (0..NP-1) its bytes come from and their offset in that page's tile.
template <int D, int NP>
struct Lanes8 {
  static constexpr int NKC = C8<D>::NKC, NCH = C8<D>::NCH, ROW = C8<D>::ROW;
  static constexpr int TPP = 32 / NP;          // tokens of the step per page
  int kn[NKC], vn[NKC], sn;
  uint32_t koff[NKC], voff[NKC];
  bool s_is_v;
  __device__ __forceinline__ Lanes8(int lane) {
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      const int p = c * 64 + lane;               // 16-byte slot of the area
      const int r = p / NCH, cs = p % NCH;       // LDS row and chunk slot
      const int tk = r, chk = cs ^ k_swz<D>(tk); // K: row = token, chunks swizzled
      const int tv = v_token_of(r);              // V: rotated rows, chunks in order
      kn[c] = tk / TPP;
      vn[c] = tv / TPP;
      koff[c] = (uint32_t)((tk % TPP) * ROW + chk * 16);
      voff[c] = (uint32_t)((tv % TPP) * ROW + cs * 16);
    }
    // scales: lanes 0..NP-1 the K scale of page lane, NP..2NP-1 the V scale
    // of page lane - NP, the rest repeat lane 0's
    s_is_v = lane >= NP && lane < 2 * NP;
    sn = lane < 2 * NP ? lane % NP : 0;
  }
};

// Row sel (0..NP-1) of r0..r3, selected per lane; written as selects so that
// no indexed array (which the compiler may move to scratch) is formed.
template <int NP>
__device__ __forceinline__ int64_t pick(int64_t r0, int64_t r1, int64_t r2, int64_t r3, int n) {
  if (NP == 1) return r0;
  if (NP == 2) return (n & 1) ? r1 : r0;
  const int64_t lo = (n & 1) ? r1 : r0, hi = (n & 1) ? r3 : r2;
  return (n & 2) ? hi : lo;
}

// Page ids of step s of item it (clamped to the item's last page).
template <int NP>
__device__ __forceinline__ void load_pids(const AttnArgs& a, const Item& it, int s,
                                          int (&pid)[NP]) {
  const int sh = a.page_shift;
  const int pb = (it.t_begin + 32 * s) >> sh;
  const int plast = (it.t_end - 1) >> sh;
#pragma unroll
  for (int n = 0; n < NP; ++n) pid[n] = ld_uniform(it.plist, min(pb + n, plast));
}

// Copy step s of item it (page ids pid) into LDS stage `st`. valid = false
// (past the end of the stream): the same number of copies, every lane at the
// step's first bytes (in bounds, next to no HBM traffic), into a stage never
// read again.
template <int D, int NP>
__device__ __forceinline__ void issue_copies8(const AttnArgs& a, const Item& it, int s,
                                              const int (&pid)[NP], char* st,
                                              const Lanes8<D, NP>& ln, bool valid) {
  constexpr int NKC = C8<D>::NKC, ROW = C8<D>::ROW, AREA = C8<D>::AREA;
  const int T0 = it.t_begin + 32 * s;
  // (page, kv head) tile of each page of the step, and its first token row
  auto tile = [&](int n) -> int64_t {
    return n < NP ? (int64_t)pid[n] * a.num_kv_heads + it.g : 0;
  };
  const int64_t h0 = tile(0), h1 = tile(1), h2 = tile(2), h3 = tile(3);
  int64_t r0 = h0 * a.page_size;
  const int64_t r1 = h1 * a.page_size, r2 = h2 * a.page_size, r3 = h3 * a.page_size;
  if (NP == 1) r0 += T0 & (a.page_size - 1);
  const char* kc = (const char*)a.k_cache;
  const char* vc = (const char*)a.v_cache;
#pragma unroll
  for (int c = 0; c < NKC; ++c) {
    const char* kp = kc + pick<NP>(r0, r1, r2, r3, valid ? ln.kn[c] : 0) * ROW +
                     (valid ? ln.koff[c] : 0u);
    __builtin_amdgcn_global_load_lds((global_vptr)kp, (lds_vptr)(st + c * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < NKC; ++c) {
    const char* vp = vc + pick<NP>(r0, r1, r2, r3, valid ? ln.vn[c] : 0) * ROW +
                     (valid ? ln.voff[c] : 0u);
    __builtin_amdgcn_global_load_lds((global_vptr)vp, (lds_vptr)(st + AREA + c * 1024), 16, 0, 0);
  }
  const float* sbase = ln.s_is_v ? a.v_scale : a.k_scale;
  const float* sp = sbase + pick<NP>(h0, h1, h2, h3, valid ? ln.sn : 0);
  __builtin_amdgcn_global_load_lds((global_vptr)sp, (lds_vptr)(st + C8<D>::SCALES), 4, 0, 0);
}

// The operands of this lane from stage st.
template <int D, int NP>
__device__ __forceinline__ void read_frags(const char* st, Frag8<D>& T, int col, int grp) {
  constexpr int KV4 = C8<D>::KV4, ROW = C8<D>::ROW, DPL = C8<D>::DPL, AREA = C8<D>::AREA;
  typedef typename C8<D>::vraw_t vraw_t;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {   // K: token 16*blk + col, chunks KV4*grp ..
    const int t = 16 * blk + col;
#pragma unroll
    for (int h = 0; h < KV4; ++h)
      T.k[blk][h] = *(const u32x4*)(st + t * ROW + 16 * ((KV4 * grp + h) ^ k_swz<D>(t)));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {   // V: tokens 4*grp + i and 16 + 4*grp + (i - 4)
    const int tl = (i < 4) ? 4 * grp + i : 16 + 4 * grp + (i - 4);
    T.v[i] = *(const vraw_t*)(st + AREA + v_row_of(tl) * ROW + DPL * col);
  }
  // pages of this lane's tokens 4g..4g+3 and 16+4g..16+4g+3
  constexpr int TPP = 32 / NP;
  const int n0 = (4 * grp) / TPP, n1 = (16 + 4 * grp) / TPP;
  const float* sc = (const float*)(st + C8<D>::SCALES);
  T.ks[0] = sc[n0];
  T.ks[1] = sc[n1];
  T.vs[0] = sc[NP + n0];
  T.vs[1] = sc[NP + n1];
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
                                              const Frag8<D>& T, const u32x4 (&qf)[C8<D>::KJ],
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

// R: LDS stages per wave. 4 at D = 128 (8.25 KiB a stage, 132 KiB per
// workgroup) and 8 at D = 64 with one wave per SIMD; half that when the plan
// gives eight or more workers per CU (two workgroups per CU).
template <int D, int NP, int R>
__global__ __launch_bounds__(256) void decode_fp8_kernel(AttnArgs a) {
  constexpr int KJ = C8<D>::KJ, STAGE = C8<D>::STAGE, NCOPY = C8<D>::NCOPY;
  __shared__ __attribute__((aligned(1024))) char lds[WAVES_PER_BLOCK * R * STAGE];
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int wave = uniform(threadIdx.x >> 6);
  const int w = blockIdx.x * WAVES_PER_BLOCK + wave;
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
  char* ring = lds + wave * (R * STAGE);
  const Lanes8<D, NP> ln(lane);

  // Issue cursor (ii, is) R-1 steps ahead of the compute cursor (ci, cs)
  // across item boundaries; stages are filled and consumed in the same order.
  // npid: the page ids of the issue cursor's step, loaded one issue ahead.
  int ci = i_begin, cs = 0;
  Item citem = load_item(a, ci);
  int ii = i_begin, is = 0;
  Item iitem = citem;
  int npid[NP];
  load_pids<NP>(a, iitem, 0, npid);
  u32x4 q_cur[KJ];
  State<D, 1> st;
  st.reset();

  auto issue = [&](int y) {
    const bool valid = ii < i_end;
    // past the end: iitem and npid still hold the stream's last step
    issue_copies8<D, NP>(a, iitem, valid ? is : iitem.nsteps - 1, npid, ring + y * STAGE, ln,
                         valid);
    if (valid) {
      if (++is >= iitem.nsteps) {
        ++ii;
        is = 0;
        if (ii < i_end) iitem = load_item(a, ii);
      }
      if (ii < i_end) load_pids<NP>(a, iitem, is, npid);
    }
  };

  // Refill stage y (computed in the previous call), then compute stage x
  // once its copies have landed: R-1 steps' copies were issued after them
  // (maybe also the stores of finished items, which only make the wait
  // stricter). An item's q is loaded when its first step is computed, its
  // wait taken on that path only (at the use after the paths join it would
  // drain the ring on every step).
  static_assert((R - 1) * NCOPY < 64, "vmcnt range");
  auto advance = [&](int x, int y) -> bool {
    asm volatile("" ::: "memory");   // stage y's reads stay before its refill
    issue(y);
    if (cs == 0) {
      load_q8<D>(a, citem, q_cur, col, grp);
#pragma unroll
      for (int j = 0; j < KJ; ++j) asm volatile("" : "+v"(q_cur[j]));
    }
    wait_vmcnt<(R - 1) * NCOPY>();
    Frag8<D> F;
    read_frags<D, NP>(ring + x * STAGE, F, col, grp);
    compute_step8<D>(a, citem, cs, F, q_cur, st, grp);
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

  for (int k = 0; k < R - 1; ++k) issue(k);
  // unrolled so that every stage offset is a constant
  if constexpr (R == 8) {
    while (advance(0, 7) && advance(1, 0) && advance(2, 1) && advance(3, 2) && advance(4, 3) &&
           advance(5, 4) && advance(6, 5) && advance(7, 6)) {
    }
  } else if constexpr (R == 4) {
    while (advance(0, 3) && advance(1, 0) && advance(2, 1) && advance(3, 2)) {
    }
  } else {
    static_assert(R == 2, "rings of two, four or eight stages");
    while (advance(0, 1) && advance(1, 0)) {
    }
  }
  // drain this wave's copies before it exits (the stages are its own)
  wait_vmcnt<0>();
  fused_merge_end<D>(a, i_begin, i_end, lane);
}

template <int D, int R>
hipError_t launch_f8(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.page_size == 8) {
    launch_timed((decode_fp8_kernel<D, 4, R>), grid, dim3(256), s, a);
  } else if (a.page_size == 16) {
    launch_timed((decode_fp8_kernel<D, 2, R>), grid, dim3(256), s, a);
  } else {
    launch_timed((decode_fp8_kernel<D, 1, R>), grid, dim3(256), s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_fp8(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const int blocks = (a.num_workers + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  if (blocks == 0) return hipSuccess;
  // workers per CU of the plan, against this device's CU count
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int per_cu = cus > 0 ? a.num_workers / cus : 0;
  if (head_dim == 128)
    return per_cu >= 8 ? launch_f8<128, 2>(a, dim3(blocks), stream)
                       : launch_f8<128, 4>(a, dim3(blocks), stream);
  if (head_dim == 64)
    return per_cu >= 8 ? launch_f8<64, 4>(a, dim3(blocks), stream)
                       : launch_f8<64, 8>(a, dim3(blocks), stream);
  return hipErrorInvalidValue;
}

}  // namespace fi
