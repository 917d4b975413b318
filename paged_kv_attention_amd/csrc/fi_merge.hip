// fi_merge.hip -- fixed-order merge of fp32 attention states, the public
// n-way state merge, and the scatter of new tokens' K/V into their pages.
//
// Merge (PR #4038, "What it does": split partials are kept in fp32 and folded
// in a fixed order so the result repeats bit for bit). For states (o_j, lse_j),
// j = 0..n-1 in plan order:  M = max_j lse_j;  w_j = exp(lse_j - M);
// z = sum_j w_j (summed j = 0, 1, ...);  o = (sum_j w_j o_j) / z;
// lse = M + ln z.  This is the log-sum-exp identity for attention over the
// union of the states' disjoint key sets; states with lse = -inf add nothing,
// and if every state is empty the row is (0, -inf). The order of every fp32
// operation depends only on the plan's part list, never on timing.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "fi_internal.h"

namespace fi {
namespace {

// Grid-stride kernels here launch at most this many workgroups (eight per CU
// of a 256-CU chip); larger counts loop.
constexpr int64_t kMaxLaunchBlocks = 2048;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Part lists are never written while a kernel runs: reading them through the
// constant address space makes the wave-uniform reads scalar loads.
typedef const __attribute__((address_space(4))) int32_t* const_i32p;
__device__ __forceinline__ int ld_uniform(const int32_t* p, int i) {
  return __builtin_amdgcn_readfirstlane(((const_i32p)p)[i]);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

template <int N> struct FVec { typedef float T __attribute__((ext_vector_type(N))); };
template <> struct FVec<1> { typedef float T; };

// Per element: acc = fma(w_j, v_j, acc) and z = z + w_j for j = 0, 1, ...;
// o = acc * (1 / z); lse = M + ln z -- the same operations, in the same order,
// as the fused fold at the end of the decode kernel (fold_record), so a row's
// bits do not depend on which of the two merged it.
//
// One wavefront per RPW rows of a merge record (RPW = 1, 2 or 4: fewer,
// fuller waves when there are many records). Lane j holds part j's row index
// and the lse of each of the wave's rows (64 parts per pass), the wave
// reduces each row's max, and each lane folds FPL consecutive outputs of one
// row over the parts, its weight broadcast by readlane. Loads of up to kFold
// parts (32 floats a lane) are in flight together (only parts that exist are loaded); the fold
// itself runs j = 0, 1, ... in order (z and acc each a plain left fold), so no
// rounding depends on the batching or on which wave runs it.
template <int D, int RPW>
__device__ __forceinline__ void merge_rows(const MergeArgs& a, int e, int h0, int lane) {
  constexpr int LPR = 64 / RPW;   // lanes per row
  constexpr int FPL = D / LPR;    // outputs per lane
  constexpr int kFold = FPL >= 8 ? 4 : FPL == 4 ? 8 : 16;   // parts in flight (32 floats)
  typedef typename FVec<FPL>::T vec;
  const int32_t* m = a.merges + (int64_t)e * MERGE_INTS;
  const int nh = ld_uniform(m, M_NROWS);
  if (h0 >= nh) return;
  const int rows = min(RPW, nh - h0);
  const int q_base = ld_uniform(m, M_QBASE), row0 = ld_uniform(m, M_ROW0);
  const int kv_head = ld_uniform(m, M_KVHEAD);
  const int off = ld_uniform(m, M_OFF), n = ld_uniform(m, M_N);
  const int32_t* parts = a.parts + off;
  const int rl = lane / LPR;                 // this lane's row within the wave
  const int rlc = min(rl, rows - 1);         // clamped to a real row for loads
  const int col = (lane % LPR) * FPL;

  // parts 0..63 stay in registers; longer lists are re-read per pass
  int prow0 = 0;
  float l0[RPW];
  if (lane < n) prow0 = parts[lane] + h0;
#pragma unroll
  for (int r = 0; r < RPW; ++r) l0[r] = (lane < n && r < rows) ? a.part_lse[prow0 + r] : neg_inf();
  float M[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) M[r] = l0[r];
  for (int j0 = 64; j0 < n; j0 += 64) {
    if (j0 + lane < n) {
      const int pr = parts[j0 + lane] + h0;
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        if (r < rows) M[r] = fmaxf(M[r], a.part_lse[pr + r]);
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) M[r] = wave_max(M[r]);

  vec acc = vec{};
  float z = 0.f;
  for (int j0 = 0; j0 < n; j0 += 64) {
    int prow = prow0;
    float l[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) l[r] = l0[r];
    if (j0 > 0) {
      prow = 0;
      if (j0 + lane < n) prow = parts[j0 + lane] + h0;
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        l[r] = (j0 + lane < n && r < rows) ? a.part_lse[prow + r] : neg_inf();
    }
    float w[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) w[r] = (l[r] == neg_inf()) ? 0.f : expf(l[r] - M[r]);
    const int cnt = min(64, n - j0);
    for (int b = 0; b < cnt; b += kFold) {
      vec v[kFold];
      float wb[kFold];
#pragma unroll
      for (int u = 0; u < kFold; ++u) {
        if (b + u < cnt) {
          const int r0 = __builtin_amdgcn_readlane(prow, b + u);
          float ws = readlane_f(w[0], b + u);
#pragma unroll
          for (int r = 1; r < RPW; ++r) {
            const float wr = readlane_f(w[r], b + u);
            ws = (rl == r) ? wr : ws;
          }
          wb[u] = ws;
          v[u] = *(const vec*)(a.part_o + (int64_t)(r0 + rlc) * D + col);
        }
      }
#pragma unroll
      for (int u = 0; u < kFold; ++u) {
        if (b + u < cnt) {
          z += wb[u];
          if constexpr (FPL == 1) {
            acc = __builtin_fmaf(wb[u], v[u], acc);
          } else {
#pragma unroll
            for (int i = 0; i < FPL; ++i) acc[i] = __builtin_fmaf(wb[u], v[u][i], acc[i]);
          }
        }
      }
    }
  }
  if (rl >= rows) return;
  float mr = M[0];
#pragma unroll
  for (int r = 1; r < RPW; ++r) mr = (rl == r) ? M[r] : mr;
  const float inv = z > 0.f ? 1.f / z : 0.f;
  const int rho = row0 + h0 + rl;   // the unit row: query token and head
  const int64_t orow = (int64_t)(q_base + rho / a.group) * a.num_qo_heads +
                       kv_head * a.group + rho % a.group;
  uint16_t* op = a.o + orow * D + col;
  if constexpr (FPL == 1) {
    *op = (uint16_t)(pack2(acc * inv, 0.f) & 0xffffu);
  } else {
    typedef uint32_t packed_t __attribute__((ext_vector_type(FPL / 2)));
    packed_t pk;
#pragma unroll
    for (int i = 0; i < FPL / 2; ++i) pk[i] = pack2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
    *(packed_t*)op = pk;
  }
  if (col == 0 && a.lse) a.lse[orow] = z > 0.f ? mr + logf(z) : neg_inf();
}

// Waves take (record, first row) pairs in turn, the record count and the most
// rows of a record read from the plan in device memory; the grid is sized by
// the host (from the plan, or its capacity).
template <int D, int RPW>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int num_merges = ld_uniform(a.counts, META_MERGES);
  const int groups = (ld_uniform(a.counts, META_MERGE_ROWS) + RPW - 1) / RPW;
  const int64_t total = (int64_t)num_merges * groups;
  const int64_t nw = (int64_t)gridDim.x * WAVES_PER_BLOCK;
  for (int64_t wv = blockIdx.x * WAVES_PER_BLOCK + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
       wv < total; wv += nw) {
    const int e = (int)(wv / groups);
    merge_rows<D, RPW>(a, e, (int)(wv - (int64_t)e * groups) * RPW, lane);
  }
}

// One wavefront per (n, h) row of fi_merge_states.
__global__ __launch_bounds__(256) void merge_states_kernel(MergeStatesArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * WAVES_PER_BLOCK + (threadIdx.x >> 6);
  if (row >= (int64_t)a.N * a.H) return;
  const int64_t n = row / a.H, h = row - n * a.H;
  const int S = a.S, H = a.H, D = a.D;
  float M = neg_inf();
  for (int j = 0; j < S; ++j) M = fmaxf(M, a.s[(n * S + j) * H + h]);
  for (int d = lane * 4; d < D; d += 256) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float z = 0.f;
    if (M != neg_inf()) {
      for (int j = 0; j < S; ++j) {
        const float lj = a.s[(n * S + j) * H + h];
        const float w = (lj == neg_inf()) ? 0.f : expf(lj - M);
        z += w;
        const int64_t base = ((n * S + j) * H + h) * D + d;
        f32x4 v;
        if (a.v_f32) {
          v = *(const f32x4*)((const float*)a.v + base);
        } else {
          const u32x2 raw = *(const u32x2*)((const uint16_t*)a.v + base);
          v = f32x4{bf16_to_f32(raw[0] & 0xffffu), bf16_to_f32(raw[0] >> 16),
                    bf16_to_f32(raw[1] & 0xffffu), bf16_to_f32(raw[1] >> 16)};
        }
        acc += w * v;
      }
    }
    const float inv = z > 0.f ? 1.f / z : 0.f;
    const f32x4 o = acc * inv;
    const int64_t obase = (n * H + h) * D + d;
    if (a.out_f32) {
      *(f32x4*)((float*)a.v_out + obase) = o;
    } else {
      u32x2 packed = {pack2(o[0], o[1]), pack2(o[2], o[3])};
      *(u32x2*)((uint16_t*)a.v_out + obase) = packed;
    }
    if (d == 0 && a.s_out) a.s_out[n * H + h] = z > 0.f ? M + logf(z) : neg_inf();
  }
}

// One thread per 16 bytes of a new token's K (and the same bytes of V), in a
// grid-stride loop over the token count read from the plan.
__global__ __launch_bounds__(256) void scatter_kernel(ScatterArgs a) {
  const int cpr = a.head_dim / 8;                 // 16-byte chunks per head row
  const int cpt = a.num_kv_heads * cpr;           // per token
  const int64_t n = (int64_t)ld_uniform(a.counts, META_SCATTER) * cpt;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * 256) {
    const int tok = (int)(idx / cpt);
    const int c = (int)(idx - (int64_t)tok * cpt);
    const int g = c / cpr, dc = c - g * cpr;
    const int page = a.kv_indices[a.scatter[2 * tok]];
    const int slot = a.scatter[2 * tok + 1];
    const int64_t dst =
        (((int64_t)page * a.num_kv_heads + g) * a.page_size + slot) * a.head_dim + dc * 8;
    const int64_t src = ((int64_t)tok * a.num_kv_heads + g) * a.head_dim + dc * 8;
    *(u32x4*)(a.k_cache + dst) = *(const u32x4*)(a.k_new + src);
    *(u32x4*)(a.v_cache + dst) = *(const u32x4*)(a.v_new + src);
  }
}

template <int D>
hipError_t launch_merge_d(const MergeArgs& a, hipStream_t stream) {
  // Rows per wave: one while that keeps the wave count within about four per
  // SIMD of a 256-CU chip, else 2 or 4 (each wave's time is mostly load
  // latency, so fewer, fuller waves win once there are many records).
  const int64_t rows = (int64_t)a.num_merges * a.rows_per_record;
  const int rpw = rows <= 4096 ? 1 : rows <= 8192 ? 2 : 4;
  const int64_t waves = (int64_t)a.num_merges * ((a.rows_per_record + rpw - 1) / rpw);
  const dim3 grid((unsigned)std::min<int64_t>(kMaxLaunchBlocks,
                                              (waves + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK));
  if (rpw == 1) {
    hipLaunchKernelGGL((merge_kernel<D, 1>), grid, dim3(256), 0, stream, a);
  } else if (rpw == 2) {
    hipLaunchKernelGGL((merge_kernel<D, 2>), grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((merge_kernel<D, 4>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.num_merges == 0 || a.rows_per_record == 0) return hipSuccess;
  if (a.head_dim == 128) return launch_merge_d<128>(a, stream);
  if (a.head_dim == 64) return launch_merge_d<64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_merge_states(const MergeStatesArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.N * a.H;
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  hipLaunchKernelGGL(merge_states_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.num_tokens * a.num_kv_heads * (a.head_dim / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)std::min<int64_t>(kMaxLaunchBlocks, (n + 255) / 256)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fi
