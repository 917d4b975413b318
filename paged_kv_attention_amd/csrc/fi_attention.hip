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

#include "fi_decode_body.h"

namespace fi {
namespace {

// FOLD: a workgroup-folded plan's launch, whose partial states stay in the
// dynamic LDS (FoldLds<D>::BYTES of it).
template <int D, int NP, bool FOLD>
__global__ __launch_bounds__(256) void decode_kernel(AttnArgs a) {
  extern __shared__ float fold_lds[];
  dec::decode_worker<D, NP, false, dec::kRing, false, FOLD>(
      a, blockIdx.x * WAVES_PER_BLOCK + dev::uniform(threadIdx.x >> 6), fold_lds);
}

template <int D, bool FOLD>
hipError_t launch_d(const AttnArgs& a, dim3 grid, hipStream_t s) {
  const unsigned lds = FOLD ? dev::FoldLds<D>::BYTES : 0;
  if (a.page_size == 8) {
    launch_timed_lds((decode_kernel<D, 4, FOLD>), grid, dim3(256), lds, s, a);
  } else if (a.page_size == 16) {
    launch_timed_lds((decode_kernel<D, 2, FOLD>), grid, dim3(256), lds, s, a);
  } else {
    launch_timed_lds((decode_kernel<D, 1, FOLD>), grid, dim3(256), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const int blocks = (a.num_workers + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  if (blocks == 0) return hipSuccess;
  if (head_dim == 128)
    return a.wg_fold ? launch_d<128, true>(a, dim3(blocks), stream)
                     : launch_d<128, false>(a, dim3(blocks), stream);
  if (head_dim == 64)
    return a.wg_fold ? launch_d<64, true>(a, dim3(blocks), stream)
                     : launch_d<64, false>(a, dim3(blocks), stream);
  return hipErrorInvalidValue;
}

}  // namespace fi
