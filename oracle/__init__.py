"""fp64 CPU oracle for paged-KV attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The library (``paged_kv_attention_amd``) never does, and this
package imports nothing from it: the two share no code, headers, tables or
helpers. Inputs reach both sides from the seeded generators in ``workloads``.

Sources (the pages this follows; cited by title and section):

* Ye et al., "customizable load-balanced attention kernels for serving"
  (catalogue record of the FlashInfer paper), fields *summary* and *boundary*:
  the engine computes exact attention over block-sparse / paged KV storage and
  schedules it in load-balanced chunks; exact attention itself is inherited.
* "flashinfer-backend-selection" research note, section *Arithmetic
  intensity*: decode reads K/V through a gathered block table (same FLOPs as a
  dense cache); cascade attention reads a shared prefix once for all requests.
* FlashInfer PR #4038 "split-K, occupancy, and m=1 stream-GEMV decode
  tactics", section *What it does*: split partials kept in fp32 and reduced in
  a fixed order so results are deterministic.
* "FlashInfer v0.7.4 Adds Rubin MoE Kernels and a Batch-Invariant Mode",
  *TL;DR*: decoding from a low-precision KV cache. The FP8 format itself is the
  OCP 8-bit floating-point E4M3 definition, and the 4-bit one the OCP
  microscaling (MX) FP4 E2M1 element with an E8M0 scale per 32 elements
  (published standards, not among the pages).

Parity status of each function is stated in its docstring ("pinned by" lists
the tests in ``tests/test_oracle.py`` that tie it to something other than
itself). The pages print no worked attention example, so every pin is a
closed form, an invariant, brute force, or an independent library routine.
"""

from .attention import (  # noqa: F401
    NEG_INF,
    attend,
    gather_tokens,
    paged_decode,
    paged_decode_fp8,
    e4m3_values,
    e2m1_values,
    e8m0_values,
    mxfp4_dequantize,
    paged_decode_mxfp4,
    paged_append,
    block_sparse,
    block_sparse_batch,
    gather_ragged,
    scatter_new_kv,
    merge_states,
    merge_two,
    cascade_flat,
    cascade_two_level,
)
from .plan_ref import plan_ref  # noqa: F401
