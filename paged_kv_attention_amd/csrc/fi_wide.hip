// fi_wide.hip -- multi-row paged attention for gfx950: append (prefill and
// mixed batches, optionally causal) and the shared-prefix level of cascade.
//
// A work item is (up to 128 query rows, kv head g, token range of one
// sequence). One 4-wave workgroup runs an item: every 32-token step of K and V
// is copied once into LDS and consumed by all 128 rows (32 per wave), so the
// bytes read from HBM per query row drop by the row count (backend-selection
// note, "Arithmetic intensity": cascade reads a shared prefix once and reuses
// it across requests; a prefill tile does the same within one request).
//
// Staging. Three LDS stages of (K, V) per step; the loads are global->LDS
// direct copies (global_load_lds_dwordx4: each lane's 16 bytes land at
// base + 16*lane), so staging costs no VGPRs and two further steps stay in
// flight while one is computed. The wait for a step is an explicit vmcnt
// count of this wave's own copies issued after it, followed by a bare
// s_barrier (no fence, which would drain every outstanding load). K rows are
// stored with their 16-byte chunks XOR-swizzled by the token (chunk c of
// token t at slot c ^ (t mod D/8)), so the MFMA operand reads -- 16 lanes
// reading the same chunk of 16 different tokens -- hit distinct banks. V rows
// are stored as they are: the operand reads already cover whole rows.
//
// Compute per wave and step: the same transposed-output MFMA tiling as the
// decode kernel (S^T = K.Q^T, O^T += V^T.P^T on v_mfma_f32_16x16x32_bf16) for
// two 16-row blocks. Masks (sequence tail, bottom-right causal) are applied
// only on steps that need them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_decode_body.h"
#include "fi_device.h"

namespace fi {
namespace {

using namespace dev;

constexpr int kStages = 3;
// Cache policy of the K/V copies: the default. (Nontemporal copies, the nt
// bit, measured 20-30% slower on the append, cascade and mixed batches: the
// row blocks of one unit re-read its tiles through L2.)
constexpr int kCopyPolicy = 0;
constexpr int kAhead = kStages - 1;   // steps in flight ahead of the computed one
constexpr int kRowsPerWave = 32;   // two 16-row MFMA blocks

typedef __attribute__((address_space(3))) void* lds_vptr;
typedef const __attribute__((address_space(1))) void* global_vptr;

// s_waitcnt vmcnt(n) with no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most k steps' copies (NKS per step) of this wave are
// outstanding, k in [0, kAhead - 1].
template <int NKS>
__device__ __forceinline__ void wait_steps(int k) {
  static_assert(kAhead <= 4, "wait_steps covers up to three outstanding steps");
  if (k >= 3) wait_vmcnt<3 * NKS>();
  else if (k == 2) wait_vmcnt<2 * NKS>();
  else if (k == 1) wait_vmcnt<NKS>();
  else wait_vmcnt<0>();
}

template <int D>
struct Lds {
  static constexpr int ROW = D * 2;           // bytes per K/V row
  static constexpr int AREA = 32 * ROW;       // K (or V) of one step
  static constexpr int STAGE = 2 * AREA;
  static constexpr int NK = (32 * Cfg<D>::CH) / 256;   // copies per wave per area
};

// V rows: chunk c of token t is stored at chunk slot c ^ v_swizzle(t). The
// XOR is even, so each 32-byte run of 16 dims (chunks 2m, 2m+1) stays
// contiguous, and the runs of the tokens read together by one transposed
// read (below) fall on distinct banks: for D = 128 a row is one 256-byte bank
// line and tokens t mod 8 pick distinct runs; for D = 64 two rows share a line
// and (t mod 2, (t / 2) mod 4) pick distinct runs.
template <int D>
__device__ __forceinline__ int v_swizzle(int t) {
  constexpr int RP = 256 / (2 * D);       // rows per 256-byte bank line
  constexpr int RUNS = D / 16;            // 32-byte runs per row
  return 2 * ((t / RP) % RUNS);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4p;

// ds_read_b64_tr_b16: within each 16-lane block, result lane j element r is
// source lane 4r + j/4, element j % 4 (measured on gfx950). With source lane
// L pointing at dims 16m + 4(L % 4) .. +3 of token L / 4 of a 4-token group,
// lane j receives dim 16m + j of the group's 4 tokens, in token order: a
// column of V, which is the V^T MFMA operand's k-slots.
__device__ __forceinline__ u32x2 lds_read_tr(const char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4p)p));
}

// This lane's byte offsets, within a page tile, of the 16-byte slots it copies:
// copy k of the wave (1-KiB block blk = wave*NK + k of the step's K, or V,
// area) holds tokens blk*TPC .. +TPC-1 of the step, which share one page
// (TPC divides a page), so a copy's page base is one scalar and the lane's
// part (token slot in the page and swizzled chunk) is fixed for the kernel.
// tok: bytes from one token of a page to the next in global memory (D * 2 in
// the paged layout, Hkv * D * 2 in the ragged one).
template <int D, int NP>
struct CopyLanes {
  static constexpr int CH = Cfg<D>::CH, NK = Lds<D>::NK, ROW = Lds<D>::ROW;
  static constexpr int TPC = 64 / CH;         // tokens per copy
  static constexpr int TPP = 32 / NP;         // tokens of the step per page (NP > 1)
  uint32_t k[NK], v[NK];
  __device__ __forceinline__ CopyLanes(int wave, int lane, uint32_t tok) {
#pragma unroll
    for (int c = 0; c < NK; ++c) {
      const int p = (wave * NK + c) * 64 + lane;    // 16-byte slot in the area
      const int t = p / CH, cs = p % CH;            // token of the step, stored chunk slot
      const int slot = t % TPP;                     // (NP = 1: plus the step's first slot)
      k[c] = (uint32_t)slot * tok + (uint32_t)((cs ^ (t % CH)) * 16);   // K: swizzled chunk
      v[c] = (uint32_t)slot * tok + (uint32_t)((cs ^ v_swizzle<D>(t)) * 16);
    }
  }
};

// Copy step s of item it into LDS stage st (this wave's share: NK 1-KiB
// copies for K and NK for V). Paged layout: page id pid, kv head g at tile
// (pid * Hkv + g) of ps rows; RAGGED ([tokens][Hkv][D]): the page list holds
// the first token of each ps-token run, row (token) stride Hkv * D elements.
template <int D, int NP, bool RAGGED>
__device__ __forceinline__ void issue_step(const AttnArgs& a, const Item& it, int s, char* stage,
                                           int wave, const CopyLanes<D, NP>& cl) {
  constexpr int NK = Lds<D>::NK, ROW = Lds<D>::ROW, TPC = CopyLanes<D, NP>::TPC;
  const int sh = a.page_shift;
  const int T0 = it.t_begin + 32 * s;
  const int pb = T0 >> sh;
  const int plast = (it.t_end - 1) >> sh;
  const int64_t tile_bytes = RAGGED ? (int64_t)ROW : (int64_t)a.page_size * ROW;
  const int64_t tok = RAGGED ? (int64_t)a.num_kv_heads * ROW : (int64_t)ROW;
  int pids[NP];   // the step's page ids, loaded together
#pragma unroll
  for (int n = 0; n < NP; ++n) pids[n] = ld_uniform(it.plist, min(pb + n, plast));
#pragma unroll
  for (int c = 0; c < NK; ++c) {
    const int blk = wave * NK + c;                       // 1-KiB block of the area
    const int n = NP == 1 ? 0 : (blk * TPC) / (32 / NP);  // its page within the step
    int pid = pids[0];
#pragma unroll
    for (int j = 1; j < NP; ++j) pid = (n == j) ? pids[j] : pid;
    int64_t base = ((int64_t)pid * a.num_kv_heads + it.g) * tile_bytes;
    if (NP == 1) base += (int64_t)(T0 & (a.page_size - 1)) * tok;
    __builtin_amdgcn_global_load_lds((global_vptr)((const char*)a.k_cache + base + cl.k[c]),
                                     (lds_vptr)(stage + blk * 1024), 16, 0, kCopyPolicy);
    __builtin_amdgcn_global_load_lds((global_vptr)((const char*)a.v_cache + base + cl.v[c]),
                                     (lds_vptr)(stage + Lds<D>::AREA + blk * 1024), 16, 0,
                                     kCopyPolicy);
  }
}

// One step of a workgroup item: copy step s+kAhead into `next` (if any), then, for
// s >= 0, read step s's K/V fragments from `cur` and compute. Every copy of the
// item goes through this one call site and the two stage pointers are
// __restrict__: the compiler then knows the copies into `next` cannot alias
// the reads from `cur` and adds no wait of its own; the ordering across steps
// is the explicit vmcnt wait plus barrier in the caller.
template <int D, int NP, bool RAGGED>
__device__ __forceinline__ void wide_step(const AttnArgs& a, const Item& it, int s, bool issue,
                                          char* __restrict__ next, const char* __restrict__ cur,
                                          const u32x4 (&qf)[2][Cfg<D>::KJ], State<D, 2>& st,
                                          int rl0, int wave, int lane,
                                          const CopyLanes<D, NP>& cl) {
  constexpr int KJ = Cfg<D>::KJ, DPL = Cfg<D>::DPL, CH = Cfg<D>::CH, ROW = Lds<D>::ROW;
  const int col = lane & 15, grp = lane >> 4;
  if (issue) issue_step<D, NP, RAGGED>(a, it, s + kAhead, next, wave, cl);
  // row blocks of this wave that hold real rows (0, 1 or 2): a wave or block
  // of padding rows only takes part in the copies and barriers
  const int nmb = min(2, max(0, (it.n_rows - rl0 + 15) >> 4));
  if (s < 0 || nmb == 0) return;
  const char* vst = cur + Lds<D>::AREA;
  const int T0 = it.t_begin + 32 * s;
  const bool tail = T0 + 32 > it.t_end;
  u32x4 kf[2][KJ];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int t = 16 * blk + col;
#pragma unroll
    for (int j = 0; j < KJ; ++j)
      kf[blk][j] = *(const u32x4*)(cur + t * ROW + ((4 * j + grp) ^ (t % CH)) * 16);
  }
  // V^T operand of MFMA m: dims 16m + col, the lane group's tokens 4g..4g+3
  // and 16+4g..16+4g+3 (the token order of the S^T accumulator), read
  // transposed from LDS. Tokens past the item's end are zeroed (they may hold
  // anything, even NaN) so that p = 0 cancels them.
  const int tk = col >> 2, dq = col & 3;   // the token and dim quad this lane points at
  const int t0 = 4 * grp + tk, t1 = 16 + 4 * grp + tk;
  u32x4 vt[DPL];
#pragma unroll
  for (int m = 0; m < DPL; ++m) {
    const u32x2 lo = lds_read_tr(vst + t0 * ROW + 32 * (m ^ (v_swizzle<D>(t0) >> 1)) + 8 * dq);
    const u32x2 hi = lds_read_tr(vst + t1 * ROW + 32 * (m ^ (v_swizzle<D>(t1) >> 1)) + 8 * dq);
    vt[m] = u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
  if (tail) {
    uint32_t keep[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int tb = (h < 2 ? 4 * grp : 16 + 4 * grp) + 2 * (h & 1);   // tokens tb, tb+1
      keep[h] = (T0 + tb < it.t_end ? 0x0000ffffu : 0u) | (T0 + tb + 1 < it.t_end ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int m = 0; m < DPL; ++m)
#pragma unroll
      for (int h = 0; h < 4; ++h) vt[m][h] &= keep[h];
  }
  const bool causal = (it.flags & FLAG_CAUSAL) != 0;
  // both row blocks' logits first: the second block's MFMAs then run under
  // the first block's softmax
  f32x4 sa[2][2];
  // the matrix phase at raised priority, so that the SIMD's other wave (in
  // its softmax) fills the vector unit meanwhile rather than competing
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    sa[mb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    sa[mb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (mb >= nmb) continue;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      sa[mb][0] = mfma_bf16(kf[0][j], qf[mb][j], sa[mb][0]);
      sa[mb][1] = mfma_bf16(kf[1][j], qf[mb][j], sa[mb][1]);
    }
  }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if (mb >= nmb) continue;
    const f32x4 s0 = sa[mb][0], s1 = sa[mb][1];
    const int row_first = it.row0 + rl0 + mb * 16;
    int lim = it.t_end - 1;
    bool masked = tail;
    if (causal) {
      masked = masked || T0 + 31 > it.q_pos0 + row_first / a.group;
      lim = min(lim, it.q_pos0 + (row_first + col) / a.group);
    }
    softmax_pv<D, 2>(st, mb, s0, s1, vt, a.scale_log2, masked, T0, lim, grp);
  }
}

// o = acc / l and lse for the wave's two 16-row blocks. Accumulator m holds
// dims 16m + 4*grp + r (r = 0..3) of row col: four consecutive dims per m.
template <int D, bool LQ>
__device__ __forceinline__ void finalize_wide(const AttnArgs& a, const Item& it,
                                              const State<D, 2>& st, int rl0, int col, int grp) {
  constexpr int DPL = Cfg<D>::DPL;
  const int G = a.group;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    float lt = st.l[mb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int rl = rl0 + mb * 16 + col;
    if (rl >= it.n_rows) continue;
    const bool live = lt > 0.f;
    const float inv = live ? 1.f / lt : 0.f;
    const float lse_v = live ? (st.m[mb] + log2f(lt)) * kLn2 : neg_inf();
    if (it.flags & FLAG_PARTIAL) {
      float* op = a.part_o + (int64_t)(it.dst + rl) * D + 4 * grp;
#pragma unroll
      for (int m = 0; m < DPL; ++m) *(f32x4*)(op + 16 * m) = st.acc[mb][m] * inv;
      if (grp == 0) a.part_lse[it.dst + rl] = lse_v;
    } else {
      const int rho = it.row0 + rl;
      const int qi = rho / G, h = rho - qi * G;
      const int tok = LQ ? a.qlist[it.q_base + qi] : it.q_base + qi;
      const int64_t orow = (int64_t)tok * a.num_qo_heads + it.g * G + h;
      uint16_t* op = a.o + orow * D + 4 * grp;
#pragma unroll
      for (int m = 0; m < DPL; ++m) {
        const f32x4 v = st.acc[mb][m] * inv;
        *(u32x2*)(op + 16 * m) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
      }
      if (grp == 0 && a.lse) a.lse[orow] = lse_v;
    }
  }
}

// The items of workgroup worker wg (the whole 4-wave block).
template <int D, int NP, bool LQ, bool RAGGED>
__device__ __forceinline__ void wide_worker(const AttnArgs& a, int wg) {
  constexpr int KJ = Cfg<D>::KJ, NK = Lds<D>::NK;
  __shared__ __attribute__((aligned(1024))) char lds[kStages * Lds<D>::STAGE];

  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int wave = uniform(threadIdx.x >> 6);
  if (wg >= a.num_workers) return;
  const int i_end = ld_uniform(a.worker_indptr, wg + 1);
  const int rl0 = wave * kRowsPerWave;
  const CopyLanes<D, NP> cl(wave, lane,
                           RAGGED ? (uint32_t)(a.num_kv_heads * Lds<D>::ROW) : (uint32_t)Lds<D>::ROW);

  for (int i = ld_uniform(a.worker_indptr, wg); i < i_end; ++i) {
    const Item it = load_item(a, i);
    u32x4 qf[2][KJ];
    load_q_rows<D, 2, LQ>(a, it, rl0, qf, col, grp);
    State<D, 2> st;
    st.reset();
    const int n = it.nsteps;
    // Step s lives in stage s mod kStages; the loop is unrolled by the stages
    // so every stage address is a compile-time offset of `lds`.
    auto body = [&](int s, char* next, const char* cur) -> bool {
      if (s >= n) return false;
      if (s >= 0) {
        // this wave's copies of step s are done when at most those of the
        // steps after it are outstanding; the barrier then publishes every
        // wave's copies, and tells every wave that step s-1's stage (which
        // step s+kAhead reuses) has been read by all
        wait_steps<2 * NK>(min(kAhead - 1, n - 1 - s));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      wide_step<D, NP, RAGGED>(a, it, s, s + kAhead < n, next, cur, qf, st, rl0, wave, lane, cl);
      return true;
    };
    constexpr int SB = Lds<D>::STAGE;
    // from s = -kAhead (= 1 mod kStages), body j computes stage (1+j) mod
    // kStages and fills stage j
    bool more = true;
    for (int s = -kAhead; more; s += kStages) {
#pragma unroll
      for (int j = 0; j < kStages; ++j) {
        if (more) more = body(s + j, lds + j * SB, lds + ((1 + j) % kStages) * SB);
      }
    }
    finalize_wide<D, LQ>(a, it, st, rl0, col, grp);
    __builtin_amdgcn_s_barrier();   // every wave is done with the stages
    asm volatile("" ::: "memory");
  }
}

template <int D, int NP, bool LQ, bool RAGGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void wide_kernel(AttnArgs a) {
  wide_worker<D, NP, LQ, RAGGED>(a, blockIdx.x);
}

// Mixed batch in one launch (POD attention: prefill and decode rows of one
// batch in one kernel). Workgroups [0, n_wide) run the wide items (one
// workgroup worker each), the others the decode items (four wavefront workers
// each); n_wide comes from the plan in device memory, so the launch shape
// does not depend on the batch. The decode role keeps a ring of two register
// tiles, so a wavefront of either role needs at most half a SIMD's registers
// and two workgroups share a CU: a CU holding one of each overlaps the matrix
// work of the wide role with the HBM streaming of the decode role.
template <int D, int NP, bool LQ, bool RAGGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void pod_kernel(
    AttnArgs wa, AttnArgs da, const int32_t* __restrict__ meta) {
  const int n_wide = ld_uniform(meta, 0);
  if ((int)blockIdx.x < n_wide) {
    wide_worker<D, NP, LQ, RAGGED>(wa, blockIdx.x);
  } else {
    dec::decode_worker<D, NP, true, 2, RAGGED>(da, ((int)blockIdx.x - n_wide) * WAVES_PER_BLOCK +
                                              uniform(threadIdx.x >> 6));
  }
}

template <int D, bool LQ, bool RAGGED>
hipError_t launch_np(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.page_size == 8) {
    launch_timed((wide_kernel<D, 4, LQ, RAGGED>), grid, dim3(256), s, a);
  } else if (a.page_size == 16) {
    launch_timed((wide_kernel<D, 2, LQ, RAGGED>), grid, dim3(256), s, a);
  } else {
    launch_timed((wide_kernel<D, 1, LQ, RAGGED>), grid, dim3(256), s, a);
  }
  return hipGetLastError();
}

template <int D, bool LQ, bool RAGGED>
hipError_t launch_pod_d(const AttnArgs& wa, const AttnArgs& da, const int32_t* meta, dim3 grid,
                        hipStream_t s) {
  if (wa.page_size == 8) {
    launch_timed((pod_kernel<D, 4, LQ, RAGGED>), grid, dim3(256), s, wa, da, meta);
  } else if (wa.page_size == 16) {
    launch_timed((pod_kernel<D, 2, LQ, RAGGED>), grid, dim3(256), s, wa, da, meta);
  } else {
    launch_timed((pod_kernel<D, 1, LQ, RAGGED>), grid, dim3(256), s, wa, da, meta);
  }
  return hipGetLastError();
}

// list_q (cascade prefix level: rows through the member list) and ragged
// (block-sparse plans over a [tokens][Hkv][D] layout) never come together.
template <int D>
hipError_t launch_pod_kind(const AttnArgs& wa, const AttnArgs& da, const int32_t* meta, dim3 grid,
                           bool list_q, bool ragged, hipStream_t s) {
  if (list_q) return launch_pod_d<D, true, false>(wa, da, meta, grid, s);
  if (ragged) return launch_pod_d<D, false, true>(wa, da, meta, grid, s);
  return launch_pod_d<D, false, false>(wa, da, meta, grid, s);
}

template <int D>
hipError_t launch_wide_kind(const AttnArgs& a, dim3 grid, bool list_q, bool ragged,
                            hipStream_t s) {
  if (list_q) return launch_np<D, true, false>(a, grid, s);
  if (ragged) return launch_np<D, false, true>(a, grid, s);
  return launch_np<D, false, false>(a, grid, s);
}

}  // namespace

hipError_t launch_pod(const AttnArgs& wa, const AttnArgs& da, const int32_t* meta, int head_dim,
                      bool list_q, bool ragged, hipStream_t stream) {
  if (wa.num_workers == 0) return hipSuccess;
  if (list_q && ragged) return hipErrorInvalidValue;
  const dim3 grid(wa.num_workers);
  if (head_dim == 128) return launch_pod_kind<128>(wa, da, meta, grid, list_q, ragged, stream);
  if (head_dim == 64) return launch_pod_kind<64>(wa, da, meta, grid, list_q, ragged, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_wide(const AttnArgs& a, int head_dim, bool list_q, bool ragged,
                       hipStream_t stream) {
  if (a.num_workers == 0) return hipSuccess;
  if (list_q && ragged) return hipErrorInvalidValue;
  const dim3 grid(a.num_workers);
  if (head_dim == 128) return launch_wide_kind<128>(a, grid, list_q, ragged, stream);
  if (head_dim == 64) return launch_wide_kind<64>(a, grid, list_q, ragged, stream);
  return hipErrorInvalidValue;
}

}  // namespace fi
