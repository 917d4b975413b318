"""GPU: the allocation-free decode entry point against fi_paged_decode.

fi_paged_decode_noalloc runs the same plan and kernels as fi_paged_decode,
with the plan's workspace in the library's static device scratch. Two calls
in a row on the same GPU, the second on a smaller batch (the scratch keeps the
first call's contents), must each give fi_paged_decode's bits, and both are
held to the oracle. A plan larger than the scratch is refused before any
launch.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_amd as fi
from tests.helpers import compare, gpu_decode, oracle_decode
from workloads import make_config, make_decode

pytestmark = pytest.mark.gpu


def _host_plan(w, dev, **kw):
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    return fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                   w.page_size, device=None, num_cus=cus, **kw)


def _noalloc(w, dev, **kw):
    p = _host_plan(w, dev, **kw)
    g = w.to(dev)
    out = torch.full((w.batch, w.num_qo_heads, w.head_dim), 7.0, dtype=torch.bfloat16,
                     device=dev)
    lse = torch.full((w.batch, w.num_qo_heads), 7.0, dtype=torch.float32, device=dev)
    fi.paged_decode_noalloc(p, g.q, g.k_cache, g.v_cache, g.kv_indices, w.sm_scale, out, lse)
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_decode_matches_paged_decode(gpu):
    dev = gpu
    big = make_config(1, poison=True)                       # 64 requests, split
    rng = np.random.default_rng(5)
    small = make_decode([int(x) for x in rng.integers(1, 3000, 9)], 32, 8, 128, 16, seed=6,
                        poison="nan")
    for w, kw in ((big, {}), (small, dict(deterministic=True, det_chunk_pages=4))):
        print(f"noalloc: B={w.batch} {kw}", flush=True)
        o_ref_gpu, l_ref_gpu, _ = gpu_decode(w, dev, **kw)
        o, lse = _noalloc(w, dev, **kw)
        assert torch.equal(o, o_ref_gpu) and torch.equal(lse, l_ref_gpu), f"B={w.batch}"
        reqs = list(range(min(w.batch, 12)))
        o_ref, l_ref, a_ref = oracle_decode(w, requests=reqs)
        compare(o, lse, o_ref, l_ref, a_ref, rows=np.asarray(reqs), what=f"noalloc B={w.batch}")


def test_noalloc_refuses_oversized_plans(gpu):
    """A plan whose workspace exceeds the scratch is refused before any
    launch (the tensors only need the shapes the call checks), and a plan
    with a device workspace is not taken."""
    dev = gpu
    B, ps = 128, 16   # (deterministic chunks of a unit are capped at 16: many units)
    lens = torch.full((B,), 32768, dtype=torch.int32)
    indptr = torch.arange(B + 1, dtype=torch.int32) * (32768 // ps)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    p = fi.Plan("decode", indptr, lens, 32, 8, 128, ps, device=None, num_cus=cus,
                deterministic=True, det_chunk_pages=4)
    assert p.info()["dev_bytes_used"] > 16 << 20
    q = torch.zeros(B, 32, 128, dtype=torch.bfloat16, device=dev)
    kv = torch.zeros(1, 8, ps, 128, dtype=torch.bfloat16, device=dev)
    idx = torch.zeros(int(indptr[-1]), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    with pytest.raises(fi.FIError, match="static scratch"):
        fi.paged_decode_noalloc(p, q, kv, kv, idx, 0.088, out)
    dp = fi.Plan("decode", indptr[:2], lens[:1], 32, 8, 128, ps, device=dev)
    with pytest.raises(ValueError, match="host-only"):
        fi.paged_decode_noalloc(dp, q[:1], kv, kv, idx, 0.088, out[:1])
