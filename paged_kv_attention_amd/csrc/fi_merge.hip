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

#include "fi_internal.h"

namespace fi {
namespace {

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

constexpr int kBatch = 8;   // partial states whose loads are in flight together

// One wavefront per merge record; each lane owns 4 consecutive outputs. The
// loads of kBatch partial states are issued together; the fold itself runs
// j = 0, 1, ... in order, so batching does not change any rounding.
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * WAVES_PER_BLOCK + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (e >= a.num_merges) return;
  const int32_t* m = a.merges + (int64_t)e * MERGE_INTS;
  const int q_tok = ld_uniform(m, M_QTOK), head0 = ld_uniform(m, M_HEAD0);
  const int nh = ld_uniform(m, M_NHEADS), off = ld_uniform(m, M_OFF), n = ld_uniform(m, M_N);
  const int32_t* parts = a.parts + off;
  const int D = a.head_dim;
  const int total = nh * D;
  for (int e0 = lane * 4; e0 < total; e0 += 256) {
    const int h = e0 / D, d = e0 - h * D;
    float M = neg_inf();
    for (int j0 = 0; j0 < n; j0 += kBatch) {
      float l[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) l[u] = a.part_lse[ld_uniform(parts, min(j0 + u, n - 1)) + h];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) M = fmaxf(M, l[u]);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float z = 0.f;
    if (M != neg_inf()) {
      for (int j0 = 0; j0 < n; j0 += kBatch) {
        float l[kBatch];
        f32x4 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int row = ld_uniform(parts, min(j0 + u, n - 1)) + h;
          l[u] = a.part_lse[row];
          v[u] = *(const f32x4*)(a.part_o + (int64_t)row * D + d);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (j0 + u < n) {
            const float w = (l[u] == neg_inf()) ? 0.f : expf(l[u] - M);
            z += w;
            acc += w * v[u];
          }
        }
      }
    }
    const float inv = z > 0.f ? 1.f / z : 0.f;
    const int64_t orow = (int64_t)q_tok * a.num_qo_heads + head0 + h;
    u32x2 packed = {pack2(acc[0] * inv, acc[1] * inv), pack2(acc[2] * inv, acc[3] * inv)};
    *(u32x2*)(a.o + orow * D + d) = packed;
    if (d == 0 && a.lse) a.lse[orow] = z > 0.f ? M + logf(z) : neg_inf();
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

// One thread per 16 bytes of a new token's K (and the same bytes of V).
__global__ __launch_bounds__(256) void scatter_kernel(ScatterArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = a.head_dim / 8;                 // 16-byte chunks per head row
  const int cpt = a.num_kv_heads * cpr;           // per token
  if (idx >= (int64_t)a.num_tokens * cpt) return;
  const int tok = (int)(idx / cpt);
  const int c = (int)(idx - (int64_t)tok * cpt);
  const int g = c / cpr, dc = c - g * cpr;
  const int page = a.kv_indices[a.scatter[2 * tok]];
  const int slot = a.scatter[2 * tok + 1];
  const int64_t dst = (((int64_t)page * a.num_kv_heads + g) * a.page_size + slot) * a.head_dim + dc * 8;
  const int64_t src = ((int64_t)tok * a.num_kv_heads + g) * a.head_dim + dc * 8;
  *(u32x4*)(a.k_cache + dst) = *(const u32x4*)(a.k_new + src);
  *(u32x4*)(a.v_cache + dst) = *(const u32x4*)(a.v_new + src);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.num_merges == 0) return hipSuccess;
  const int blocks = (a.num_merges + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  hipLaunchKernelGGL(merge_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
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
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fi
