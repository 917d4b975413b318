"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Full-size configurations are compared on sampled requests (the oracle computes
each request independently); small cases are compared in full. Every case is
seeded; inputs are poisoned (NaN in unused pages, 1e4 in tail slots, NaN in
not-yet-written append slots) so that a stray read shows up in the output; the
small sweeps put NaN in the tail slots as well, so a tail V row that reaches
the P.V product unzeroed turns the output into NaN.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_amd as fi
from tests.helpers import (compare, gpu_decode, np_pools, oracle_decode, request_rows,
                           sample_requests)
from workloads import (cascade_flat_tables, make_append, make_block_sparse,
                       make_block_sparse_batch, make_cascade, make_config, make_decode,
                       make_pod_mix, make_sparse_video, to_fp8_cache, to_mxfp4_cache, to_ragged)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev(gpu):
    return gpu


@pytest.fixture(scope="module")
def cfg1():
    return make_config(1, poison=True)


# ---------------------------------------------------------------- configs


def test_tiny_decode_config(dev):
    w = make_config(0, poison=True)
    o, lse, _ = gpu_decode(w, dev)
    o_ref, l_ref, a_ref = oracle_decode(w)
    compare(o, lse, o_ref, l_ref, a_ref, what="tiny_decode")


@pytest.mark.parametrize("det", [False, True])
def test_llama_decode_config_sampled(dev, cfg1, det):
    w = cfg1
    o, lse, p = gpu_decode(w, dev, deterministic=det)
    rng = np.random.default_rng(1)
    reqs = sample_requests(w.batch, 10, rng, must=[int(torch.argmax(w.kv_len))])
    o_ref, l_ref, a_ref = oracle_decode(w, requests=reqs)
    compare(o, lse, o_ref, l_ref, a_ref, rows=request_rows(reqs), what=f"llama_decode det={det}")


@pytest.mark.parametrize("det", [False, True])
def test_skewed_decode_config_sampled(dev, det):
    w = make_config(2, poison=True)
    o, lse, p = gpu_decode(w, dev, deterministic=det)
    long = [int(i) for i in torch.nonzero(w.kv_len == 32768).flatten()]
    assert len(long) >= 4
    rng = np.random.default_rng(2)
    reqs = sample_requests(w.batch, 6, rng, must=long + [int(torch.argmin(w.kv_len))])
    o_ref, l_ref, a_ref = oracle_decode(w, requests=reqs)
    compare(o, lse, o_ref, l_ref, a_ref, rows=request_rows(reqs), what=f"skewed_decode det={det}")
    assert max(p.info()["levels"][0]["items"][:, 11]) > 0, "long requests were not split"


def _cascade_run(w, dev, **kw):
    p = fi.Plan("cascade", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                w.page_size, prefix_indptr=w.prefix_indptr, prefix_len=w.prefix_len,
                req_prefix_group=w.req_prefix_group, prefix_parent=w.prefix_parent, device=dev,
                **kw)
    g = w.to(dev)
    o, lse = fi.cascade(p, g.q, g.k_cache, g.v_cache, g.prefix_indices, g.kv_indices, w.sm_scale)
    torch.cuda.synchronize()
    return o, lse


def _oracle_cascade(w, reqs):
    kp, vp = np_pools(w)
    q = w.q.double().numpy()
    tabs = (w.prefix_indptr.numpy(), w.prefix_indices.numpy(), w.prefix_len.numpy(),
            w.req_prefix_group.numpy(), w.kv_indptr.numpy(), w.kv_indices.numpy(),
            w.kv_len.numpy(), w.page_size, w.sm_scale)
    par = None if w.prefix_parent is None else w.prefix_parent.numpy()
    o, lse = oracle.cascade_flat(q, kp, vp, *tabs, requests=reqs, prefix_parent=par)
    a, _ = oracle.cascade_flat(q, kp, np.abs(vp), *tabs, requests=reqs, prefix_parent=par)
    return o, lse, a


@pytest.mark.parametrize("det", [False, True])
@pytest.mark.parametrize("launch", ["pod", "separate"])
def test_cascade_config_sampled(dev, launch, det):
    """The cascade batch, every one of its 64 requests against the oracle."""
    w = make_config(3, poison=True)
    o, lse = _cascade_run(w, dev, launch=launch, deterministic=det)
    reqs = list(range(w.batch))
    o_ref, l_ref, a_ref = _oracle_cascade(w, reqs)
    compare(o, lse, o_ref, l_ref, a_ref, rows=request_rows(reqs),
            what=f"cascade {launch} det={det}")
    # cascade equals flat decode over the concatenated table (both on the GPU)
    ip, ix, ln = cascade_flat_tables(w)
    p = fi.Plan("decode", ip, ln, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                device=dev)
    g = w.to(dev)
    of, lf = fi.paged_decode(p, g.q, g.k_cache, g.v_cache, ix.to(dev), w.sm_scale)
    compare(of, lf, o_ref, l_ref, a_ref, rows=request_rows(reqs),
            what="flat decode of cascade input")


@pytest.mark.parametrize("det", [False, True])
@pytest.mark.parametrize("launch", ["pod", "separate"])
def test_append_config_sampled(dev, launch, det):
    """The mixed append batch: the scatter bit for bit, and all 16 requests'
    query rows against the oracle."""
    w = make_config(4, poison=True)
    p = fi.Plan("append", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                w.page_size, qo_indptr=w.qo_indptr, causal=True, device=dev, launch=launch,
                deterministic=det)
    g = w.to(dev)
    o, lse = fi.paged_append(p, g.q, g.k_cache, g.v_cache, g.kv_indices, w.sm_scale,
                             k_new=g.k_new, v_new=g.v_new)
    torch.cuda.synchronize()
    kp, vp = np_pools(w)
    kp2, vp2 = oracle.scatter_new_kv(kp, vp, w.k_new.float().numpy(), w.v_new.float().numpy(),
                                     w.qo_indptr.numpy(), w.kv_indptr.numpy(),
                                     w.kv_indices.numpy(), w.kv_len.numpy(), w.page_size)
    # scatter is a bit-exact copy; every other pool byte is unchanged
    assert np.array_equal(g.k_cache.float().cpu().numpy(), kp2, equal_nan=True)
    assert np.array_equal(g.v_cache.float().cpu().numpy(), vp2, equal_nan=True)
    o_ref, l_ref, a_ref = _oracle_append(w, kp2, vp2, True)
    compare(o, lse, o_ref, l_ref, a_ref, what=f"append {launch} det={det}")


def _oracle_append(w, kp2, vp2, causal, reqs=None):
    q = w.q.double().numpy()
    tabs = (w.kv_indptr.numpy(), w.kv_indices.numpy(), w.kv_len.numpy(), w.page_size,
            w.sm_scale)
    o, lse = oracle.paged_append(q, w.qo_indptr.numpy(), kp2, vp2, *tabs, causal=causal,
                                 requests=reqs)
    a, _ = oracle.paged_append(q, w.qo_indptr.numpy(), kp2, np.abs(vp2), *tabs, causal=causal,
                               requests=reqs)
    return o, lse, a


# ---------------------------------------------------------------- small sweeps

SMALL_LENS = [0, 1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 100, 517, 1000]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("ps", [8, 16, 32, 64, 256])
@pytest.mark.parametrize("G", [1, 4, 8, 24])
def test_decode_small_sweep(dev, D, ps, G):
    Hkv = 2
    w = make_decode(SMALL_LENS, G * Hkv, Hkv, D, ps, seed=100 + D + ps + G, poison="nan")
    o_ref, l_ref, a_ref = oracle_decode(w)
    plans = [dict(), dict(deterministic=True, det_chunk_pages=1),
             dict(deterministic=True, det_chunk_pages=3), dict(min_chunk_pages=1)]
    for kw in plans:
        o, lse, _ = gpu_decode(w, dev, **kw)
        compare(o, lse, o_ref, l_ref, a_ref, what=f"decode D={D} ps={ps} G={G} {kw}")


@pytest.mark.parametrize("B,D,rows_min,rows_max", [(150, 128, 4097, 8192), (300, 64, 8193, None),
                                                   (300, 128, 8193, None)])
def test_decode_many_merge_records(dev, B, D, rows_min, rows_max):
    """One-page chunks split every request, so the merge runs with many
    records: two and four rows per merge wave."""
    Hkv, G, ps = 8, 4, 16
    lens = torch.randint(17, 121, (B,), generator=torch.Generator().manual_seed(B + D)).tolist()
    w = make_decode(lens, G * Hkv, Hkv, D, ps, seed=300 + B + D)
    o, lse, p = gpu_decode(w, dev, deterministic=True, det_chunk_pages=1)
    rows = int(p.info()["merges"][:, 2].sum())
    assert rows >= rows_min and (rows_max is None or rows <= rows_max), rows
    o_ref, l_ref, a_ref = oracle_decode(w)
    compare(o, lse, o_ref, l_ref, a_ref, what=f"decode many merges B={B} D={D}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D,ps,G", [(128, 16, 4), (64, 8, 2), (128, 32, 8), (64, 16, 24),
                                    (128, 256, 4)])
def test_append_small_sweep(dev, causal, D, ps, G):
    prefix = [0, 5, 16, 40, 300, 1]
    qo = [1, 3, 17, 40, 70, 33]
    Hkv = 2
    w = make_append(prefix, qo, G * Hkv, Hkv, D, ps, seed=200 + D + ps + G, causal=causal,
                    poison="nan")
    kp, vp = np_pools(w)
    kp2, vp2 = oracle.scatter_new_kv(kp, vp, w.k_new.float().numpy(), w.v_new.float().numpy(),
                                     w.qo_indptr.numpy(), w.kv_indptr.numpy(),
                                     w.kv_indices.numpy(), w.kv_len.numpy(), ps)
    o_ref, l_ref, a_ref = _oracle_append(w, kp2, vp2, causal)
    for kw in [dict(), dict(deterministic=True, det_chunk_pages=1), dict(min_chunk_pages=1),
               dict(launch="separate"),
               dict(launch="separate", deterministic=True, det_chunk_pages=1)]:
        g = w.to(dev)
        p = fi.Plan("append", w.kv_indptr, w.kv_len, w.num_qo_heads, Hkv, D, ps,
                    qo_indptr=w.qo_indptr, causal=causal, device=dev, **kw)
        o, lse = fi.paged_append(p, g.q, g.k_cache, g.v_cache, g.kv_indices, w.sm_scale,
                                 k_new=g.k_new, v_new=g.v_new)
        torch.cuda.synchronize()
        compare(o, lse, o_ref, l_ref, a_ref,
                what=f"append causal={causal} D={D} ps={ps} G={G} {kw}")


def test_cascade_small_multi_group(dev):
    ps = 16
    w = make_cascade([64, 40, 0], [0, 1, 1, -1, 2, 0, 1, 0], [5, 0, 40, 33, 16, 1, 300, 17],
                     32, 8, 128, ps, seed=300, poison="nan")
    o_ref, l_ref, a_ref = _oracle_cascade(w, None)
    for kw in [dict(), dict(deterministic=True, det_chunk_pages=1), dict(min_chunk_pages=1),
               dict(launch="separate"),
               dict(launch="separate", deterministic=True, det_chunk_pages=1),
               dict(pod_wide_blocks=1), dict(num_cus=2)]:
        o, lse = _cascade_run(w, dev, **kw)
        compare(o, lse, o_ref, l_ref, a_ref, what=f"cascade groups {kw}")


# ---------------------------------------------------------------- invariants


def test_pool_permutation_is_bit_identical(dev):
    w = make_decode([700, 33, 2048, 5, 1500], 32, 8, 128, 16, seed=400)
    o1, l1, _ = gpu_decode(w, dev, min_chunk_pages=2)
    P = w.num_pages
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(5))
    k2 = torch.empty_like(w.k_cache)
    v2 = torch.empty_like(w.v_cache)
    k2[perm] = w.k_cache
    v2[perm] = w.v_cache
    w2 = make_decode([1], 32, 8, 128, 16, seed=1)   # container, fields replaced below
    w2.kv_len, w2.kv_indptr, w2.q = w.kv_len, w.kv_indptr, w.q
    w2.kv_indices = perm[w.kv_indices.long()].to(torch.int32)
    w2.k_cache, w2.v_cache = k2, v2
    o2, l2, _ = gpu_decode(w2, dev, min_chunk_pages=2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("cfg", [1, 2])
def test_fused_merge_bits_equal_merge_kernel(dev, cfg):
    """merge="fused" decode plans fold their split units inside the attention
    kernel; the bits equal those of the merge kernel (the default launch), on
    every decode kernel, in both modes, and stay the same over repeated calls
    on one plan (the arrival counts reset themselves)."""
    w = make_config(cfg, poison=True)
    if cfg == 1:
        w = to_mxfp4_cache(to_fp8_cache(w, poison=True), poison=True)
    g = w.to(dev)
    kernels = ["bf16"] + (["fp8", "mxfp4"] if cfg == 1 else [])
    for det in (False, True):
        for kern in kernels:
            outs = []
            for merge in ("fused", "default"):
                p = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads,
                            w.head_dim, w.page_size, device=dev, deterministic=det, merge=merge)
                assert p.info()["fused_merge"] == (merge == "fused")
                for rep in range(3 if merge == "fused" else 1):
                    if kern == "bf16":
                        o, lse = fi.paged_decode(p, g.q, g.k_cache, g.v_cache, g.kv_indices,
                                                 w.sm_scale)
                    elif kern == "fp8":
                        o, lse = fi.paged_decode_fp8(p, g.q, g.k_fp8, g.v_fp8, g.k_scale,
                                                     g.v_scale, g.kv_indices, w.sm_scale)
                    else:
                        o, lse = fi.paged_decode_mxfp4(p, g.q, g.k_fp4, g.v_fp4, g.k_bscale,
                                                       g.v_bscale, g.kv_indices, w.sm_scale)
                    torch.cuda.synchronize()
                    outs.append((o, lse))
            for o, lse in outs[1:]:
                assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1]), (kern, det)


@pytest.mark.parametrize("D,ps,hq,hkv", [(64, 8, 8, 2), (128, 32, 32, 8), (64, 64, 16, 2),
                                         (128, 16, 16, 1)])
def test_workgroup_fold_lds_shapes(dev, D, ps, hq, hkv):
    """The bf16 kernel of a workgroup-folded plan keeps the four partial
    states in LDS (its own instantiation per head size and pages per step):
    every head size, page size and group size (up to 16 rows) matches the
    oracle and repeats its bits over calls."""
    lens = [37, 300, 5, 0, 129, 64]
    w = make_decode(lens, hq, hkv, D, ps, seed=91, poison=True)
    g = w.to(dev)
    p = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                w.page_size, device=dev)
    assert p.info()["wg_fold"]
    outs = []
    for rep in range(3):
        outs.append(fi.paged_decode(p, g.q, g.k_cache, g.v_cache, g.kv_indices, w.sm_scale))
        torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])
    o_ref, l_ref, a_ref = oracle_decode(w)
    compare(outs[0][0], outs[0][1], o_ref, l_ref, a_ref, what=f"lds fold D={D} ps={ps} G={hq // hkv}")


@pytest.mark.parametrize("lens", [[37, 300, 120, 5, 0, 64], [1, 2, 33, 64, 65, 400]])
def test_workgroup_fold_tiny_decode(dev, lens):
    """A tiny decode batch (no more steps than workers, at most a quarter as
    many units) runs each unit on the four waves of one workgroup and folds
    it after a workgroup barrier: the plan says so, the bf16 result matches
    the oracle, and every decode kernel repeats its bits over calls."""
    w = to_mxfp4_cache(to_fp8_cache(make_decode(lens, 8, 2, 128, 16, seed=77, poison=True),
                                    poison=True), poison=True)
    g = w.to(dev)
    p = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                w.page_size, device=dev)
    assert p.info()["wg_fold"] and p.info()["fused_merge"]
    o_ref, l_ref, a_ref = oracle_decode(w)
    for kern in ("bf16", "fp8", "mxfp4"):
        outs = []
        for rep in range(3):
            if kern == "bf16":
                o, lse = fi.paged_decode(p, g.q, g.k_cache, g.v_cache, g.kv_indices, w.sm_scale)
            elif kern == "fp8":
                o, lse = fi.paged_decode_fp8(p, g.q, g.k_fp8, g.v_fp8, g.k_scale, g.v_scale,
                                             g.kv_indices, w.sm_scale)
            else:
                o, lse = fi.paged_decode_mxfp4(p, g.q, g.k_fp4, g.v_fp4, g.k_bscale,
                                               g.v_bscale, g.kv_indices, w.sm_scale)
            torch.cuda.synchronize()
            outs.append((o, lse))
        for o, lse in outs[1:]:
            assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1]), kern
        if kern == "bf16":
            compare(outs[0][0], outs[0][1], o_ref, l_ref, a_ref, what=f"wg fold {lens}")


def test_repeat_runs_are_bit_identical(dev, cfg1):
    for det in (False, True):
        o1, l1, _ = gpu_decode(cfg1, dev, deterministic=det)
        o2, l2, _ = gpu_decode(cfg1, dev, deterministic=det)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), det


def _sub_batch(w, reqs):
    """Decode workload with the requests ``reqs`` of ``w`` (same pool)."""
    ptr, idx = [0], []
    for r in reqs:
        a, b = int(w.kv_indptr[r]), int(w.kv_indptr[r + 1])
        idx.append(w.kv_indices[a:b])
        ptr.append(ptr[-1] + (b - a))
    sub = make_decode([1], w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, seed=1)
    sub.kv_len = w.kv_len[list(reqs)].clone()
    sub.kv_indptr = torch.tensor(ptr, dtype=torch.int32)
    sub.kv_indices = torch.cat(idx).to(torch.int32)
    sub.q = w.q[list(reqs)].clone()
    sub.k_cache, sub.v_cache = w.k_cache, w.v_cache
    return sub


def test_deterministic_mode_is_batch_invariant(dev):
    rng = np.random.default_rng(6)
    lens = [5000] + list(rng.integers(1, 9000, 63))
    w = make_decode(lens, 32, 8, 128, 16, seed=500, poison=False)
    target = 0
    outs = []
    for reqs in ([target], [3, target, 9, 4], [9, 5, target],
                 list(rng.permutation(64))):
        sub = _sub_batch(w, [int(r) for r in reqs])
        pos = [int(r) for r in reqs].index(target)
        o, lse, _ = gpu_decode(sub, dev, deterministic=True, det_chunk_pages=16)
        outs.append((o[pos].clone(), lse[pos].clone()))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    o_ref, l_ref, a_ref = oracle_decode(w, requests=[target])
    compare(outs[0][0][None], outs[0][1][None], o_ref[[target]], l_ref[[target]],
            a_ref[[target]], what="batch-invariant target vs oracle")


@pytest.mark.parametrize("ps", [8, 16, 32])
def test_needle_keys_are_gathered_exactly(dev, ps):
    lens = [100, 37, 16, 300, 64]
    w = make_decode(lens, 8, 2, 128, ps, seed=600 + ps)
    needles = [0, 36, 15, 257, 32]        # positions across page boundaries
    q = torch.zeros_like(w.q)
    q[:, :, 0] = 8.0
    w.q = q
    for r, t in enumerate(needles):
        page = int(w.kv_indices[int(w.kv_indptr[r]) + t // ps])
        w.k_cache[page, :, t % ps, 0] = 100.0
    o, lse, _ = gpu_decode(w, dev, min_chunk_pages=1)
    o = o.cpu()
    for r, t in enumerate(needles):
        page = int(w.kv_indices[int(w.kv_indptr[r]) + t // ps])
        for h in range(8):
            assert torch.equal(o[r, h], w.v_cache[page, h // 4, t % ps]), (r, h)


def test_append_single_query_matches_decode(dev):
    w = make_decode([3, 40, 77, 1000, 2500], 32, 8, 128, 16, seed=700)
    od, ld, _ = gpu_decode(w, dev)
    p = fi.Plan("append", w.kv_indptr, w.kv_len, 32, 8, 128, 16,
                qo_indptr=torch.arange(6, dtype=torch.int32), causal=True, device=dev)
    g = w.to(dev)
    oa, la = fi.paged_append(p, g.q, g.k_cache, g.v_cache, g.kv_indices, w.sm_scale)
    torch.cuda.synchronize()
    o_ref, l_ref, a_ref = oracle_decode(w)
    compare(od, ld, o_ref, l_ref, a_ref, what="decode")
    compare(oa, la, o_ref, l_ref, a_ref, what="append with one query per request")


def test_empty_batch_and_empty_requests(dev):
    w = make_decode([0, 0, 5, 0], 8, 2, 64, 16, seed=800)
    o, lse, _ = gpu_decode(w, dev)
    assert torch.all(o[[0, 1, 3]] == 0) and torch.all(torch.isneginf(lse[[0, 1, 3]]))
    p = fi.Plan("decode", [0], [], 8, 2, 64, 16, device=dev)
    q = torch.empty(0, 8, 64, dtype=torch.bfloat16, device=dev)
    o, lse = fi.paged_decode(p, q, w.k_cache.to(dev), w.v_cache.to(dev),
                             torch.zeros(1, dtype=torch.int32, device=dev), w.sm_scale)
    torch.cuda.synchronize()
    assert o.numel() == 0


def test_page_table_check_counts_out_of_range_ids(dev):
    """fi_check_page_tables counts the ids outside [0, num_pages) among the
    entries the plan covers (planted in a copy of the table), not beyond
    them, and checks a cascade plan's prefix table when given."""
    w = make_decode([100, 37, 300, 16], 8, 2, 64, 16, seed=77)
    p = fi.Plan("decode", w.kv_indptr, w.kv_len, 8, 2, 64, 16, device=dev)
    P = w.num_pages
    n = int(w.kv_indptr[-1])
    idx = torch.cat([w.kv_indices, torch.tensor([-5, P + 9], dtype=torch.int32)]).to(dev)
    assert fi.check_page_tables(p, idx, P) == 0          # entries past kv_indptr[B] ignored
    bad = idx.clone()
    bad[0], bad[7], bad[n - 1] = -1, P, 2 ** 30
    assert fi.check_page_tables(p, bad, P) == 3
    assert fi.check_page_tables(p, idx, int(idx[:n].max())) == 1   # the largest id is now out
    c = make_cascade([64, 32], [0, 1, -1], [40, 7, 100], 8, 2, 64, 16, seed=78)
    pc = fi.Plan("cascade", c.kv_indptr, c.kv_len, 8, 2, 64, 16, prefix_indptr=c.prefix_indptr,
                 prefix_len=c.prefix_len, req_prefix_group=c.req_prefix_group, device=dev)
    gi, gp = c.kv_indices.to(dev), c.prefix_indices.to(dev).clone()
    assert fi.check_page_tables(pc, gi, c.num_pages, gp) == 0
    gp[1] = -3
    assert fi.check_page_tables(pc, gi, c.num_pages, gp) == 1
    assert fi.check_page_tables(pc, gi, c.num_pages) == 0     # prefix table not given
    with pytest.raises(fi.FIError):
        fi.check_page_tables(p, idx, 0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_merge_states_api(dev, dtype):
    g = torch.Generator().manual_seed(9)
    N, S, H, D = 6, 7, 3, 128
    v = torch.randn(N, S, H, D, generator=g).to(dtype)
    s = torch.randn(N, S, H, generator=g) * 4
    s[0, :, 1] = -float("inf")        # all states empty for one row
    s[1, 2:5, 0] = -float("inf")      # some empty
    vo, so = fi.merge_states(v.to(dev), s.to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge_states(v.double().numpy(), s.double().numpy())
    assert np.allclose(vo.cpu().numpy(), o_ref, atol=2e-6, rtol=2e-6)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(so.cpu().numpy()), ~fin)
    assert np.allclose(so.cpu().numpy()[fin], l_ref[fin], atol=1e-5, rtol=1e-6)
    assert torch.all(vo[0, 1] == 0)


# ---------------------------------------------------------------- VALU engine


def test_valu_engine_configs(dev, cfg1):
    w = make_config(0, poison=True)
    o, lse, _ = gpu_decode(w, dev, engine="valu")
    o_ref, l_ref, a_ref = oracle_decode(w)
    compare(o, lse, o_ref, l_ref, a_ref, what="tiny_decode valu")
    w = cfg1
    rng = np.random.default_rng(11)
    reqs = sample_requests(w.batch, 10, rng, must=[int(torch.argmax(w.kv_len))])
    o_ref, l_ref, a_ref = oracle_decode(w, requests=reqs)
    for det in (False, True):
        o, lse, _ = gpu_decode(w, dev, engine="valu", deterministic=det)
        compare(o, lse, o_ref, l_ref, a_ref, rows=request_rows(reqs),
                what=f"llama_decode valu det={det}")
    o2, lse2, _ = gpu_decode(w, dev, engine="valu", deterministic=True)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "VALU runs differ"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("ps", [8, 16, 32, 64, 256])
@pytest.mark.parametrize("G", [1, 3, 4, 8])
def test_valu_decode_small_sweep(dev, D, ps, G):
    Hkv = 2
    w = make_decode(SMALL_LENS, G * Hkv, Hkv, D, ps, seed=400 + D + ps + G, poison="nan")
    o_ref, l_ref, a_ref = oracle_decode(w)
    for kw in [dict(), dict(deterministic=True, det_chunk_pages=1), dict(min_chunk_pages=1)]:
        o, lse, _ = gpu_decode(w, dev, engine="valu", **kw)
        compare(o, lse, o_ref, l_ref, a_ref, what=f"valu decode D={D} ps={ps} G={G} {kw}")


def test_valu_engine_cascade(dev):
    w = make_config(3, poison=True)
    o, lse = _cascade_run(w, dev, engine="valu")
    rng = np.random.default_rng(13)
    reqs = sample_requests(w.batch, 6, rng)
    o_ref, l_ref, a_ref = _oracle_cascade(w, reqs)
    compare(o, lse, o_ref, l_ref, a_ref, rows=request_rows(reqs), what="cascade valu")


# ---------------------------------------------------------------- fused mixed batch


def _append_run(w, dev, causal=True, **kw):
    p = fi.Plan("append", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                w.page_size, qo_indptr=w.qo_indptr, causal=causal, device=dev, **kw)
    g = w.to(dev)
    o, lse = fi.paged_append(p, g.q, g.k_cache, g.v_cache, g.kv_indices, w.sm_scale,
                             k_new=g.k_new, v_new=g.v_new)
    torch.cuda.synchronize()
    return o, lse, p


def _scattered_pools(w):
    kp, vp = np_pools(w)
    return oracle.scatter_new_kv(kp, vp, w.k_new.float().numpy(), w.v_new.float().numpy(),
                                 w.qo_indptr.numpy(), w.kv_indptr.numpy(), w.kv_indices.numpy(),
                                 w.kv_len.numpy(), w.page_size)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D,ps,G", [(128, 16, 4), (64, 8, 2), (128, 32, 8), (64, 16, 1),
                                    (128, 64, 16), (64, 256, 4)])
def test_pod_small_sweep(dev, causal, D, ps, G):
    """Mixed batches in one fused launch: requests whose rows fit 16 run in the
    decode role (with the causal mask over their few query tokens), the rest
    in the wide role; every plan variant against the oracle."""
    prefix = [0, 5, 16, 40, 300, 1, 700, 33, 1000, 2, 7]
    qo = [1, 3, 17, 1, 70, 2, 1, 4, 1, 40, 0]
    Hkv = 2
    w = make_append(prefix, qo, G * Hkv, Hkv, D, ps, seed=600 + D + ps + G, causal=causal,
                    poison="nan")
    kp2, vp2 = _scattered_pools(w)
    o_ref, l_ref, a_ref = _oracle_append(w, kp2, vp2, causal)
    for kw in [dict(), dict(deterministic=True, det_chunk_pages=1), dict(min_chunk_pages=1),
               dict(pod_wide_blocks=1), dict(num_cus=3)]:
        o, lse, p = _append_run(w, dev, causal, launch="pod", **kw)
        info = p.info()
        assert len(info["levels"][1]["items"]) > 0
        compare(o, lse, o_ref, l_ref, a_ref,
                what=f"pod causal={causal} D={D} ps={ps} G={G} {kw} n_w={info['pod_wide_blocks']}")


@pytest.mark.parametrize("det", [False, True])
def test_pod_mixed_sampled(dev, det):
    """The chunked-prefill serving step (64 decode requests beside two
    512-token prefill chunks) through the fused launch: sampled requests of
    both roles against the oracle, and the whole batch against the unfused
    plan."""
    w = make_pod_mix(poison=True)
    o, lse, p = _append_run(w, dev, launch="pod", deterministic=det)
    info = p.info()
    assert 1 <= info["pod_wide_blocks"] < info["levels"][0]["num_workers"]
    qo = w.qo_indptr.diff()
    pre = [int(i) for i in torch.nonzero(qo > 1).flatten()]
    rng = np.random.default_rng(31)
    dec = [int(i) for i in rng.choice(torch.nonzero(qo == 1).flatten().numpy(), 6, replace=False)]
    reqs = sorted(pre[:1] + dec)
    kp2, vp2 = _scattered_pools(w)
    o_ref, l_ref, a_ref = _oracle_append(w, kp2, vp2, True, reqs)
    rows = np.concatenate([np.arange(int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])) for r in reqs])
    compare(o, lse, o_ref, l_ref, a_ref, rows=rows, what=f"pod mixed det={det}")
    o2, lse2, _ = _append_run(w, dev, launch="separate", deterministic=det)
    assert float((o2.float() - o.float()).abs().max()) <= 2e-2
    assert float(((lse2 - lse).abs() / lse.abs().clamp(min=1)).max()) <= 2e-3


def test_pod_deterministic_bits_independent_of_split(dev):
    """Deterministic mode: a request's bits do not depend on how the launch
    is split between the roles."""
    w = make_pod_mix(poison=False, n_decode=24, n_prefill=1, prefill_q=200)
    outs = [_append_run(w, dev, launch="pod", deterministic=True, det_chunk_pages=8,
                        pod_wide_blocks=nw)[:2] for nw in (0, 3, 100)]
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


# ---------------------------------------------------------------- variable block-sparse


def _bs_run(w, dev, **kw):
    p = fi.BlockSparsePlan(w.q.shape[0], int(w.kv_len[0]), w.row_block_sz, w.col_block_sz,
                           w.block_mask, w.kv_indices, w.num_qo_heads, w.num_kv_heads,
                           w.head_dim, w.page_size, device=dev, **kw)
    g = w.to(dev)
    o, lse = fi.block_sparse_attention(p, g.q, g.k_cache, g.v_cache, w.sm_scale)
    torch.cuda.synchronize()
    return o, lse, p


def _bs_oracle(w, rows=None):
    kp, vp = np_pools(w)
    args = (w.kv_indices.numpy(), int(w.kv_len[0]), w.page_size, w.row_block_sz.numpy(),
            w.col_block_sz.numpy(), w.block_mask.numpy(), w.sm_scale)
    q = w.q.double().numpy()
    o, lse = oracle.block_sparse(q, kp, vp, *args, rows=rows)
    a, _ = oracle.block_sparse(q, kp, np.abs(vp), *args, rows=rows)
    return o, lse, a


@pytest.mark.parametrize("D,ps,G", [(128, 16, 4), (64, 8, 1), (128, 32, 8), (64, 16, 2),
                                    (128, 64, 16), (128, 256, 4)])
def test_block_sparse_small_sweep(dev, D, ps, G):
    """Variable blocks per kv head (some empty), random masks with a row block
    that sees nothing, every plan variant, against the oracle in full."""
    Hkv = 2
    w = make_block_sparse(90, 700, G * Hkv, Hkv, D, ps, 6, 9, 0.45, seed=900 + D + ps + G,
                          poison="nan")
    w.block_mask[1, 2, :] = False          # kv head 1, row block 2: no keys
    o_ref, l_ref, a_ref = _bs_oracle(w)
    for kw in [dict(), dict(launch="separate"), dict(deterministic=True, det_chunk_pages=1),
               dict(launch="separate", deterministic=True, det_chunk_pages=2),
               dict(min_chunk_pages=1), dict(pod_wide_blocks=1), dict(num_cus=3)]:
        o, lse, p = _bs_run(w, dev, **kw)
        compare(o, lse, o_ref, l_ref, a_ref, what=f"block sparse D={D} ps={ps} G={G} {kw}")


def test_block_sparse_full_mask_equals_append(dev):
    """One row block and one column block, fully selected: the same attention
    as a non-causal append of the whole sequence (GPU against GPU and the
    oracle)."""
    T, Lk, Hq, Hkv = 200, 1500, 32, 8
    w = make_block_sparse(T, Lk, Hq, Hkv, 128, 16, 1, 1, 1.0, seed=950)
    o, lse, _ = _bs_run(w, dev)
    o_ref, l_ref, a_ref = _bs_oracle(w)
    compare(o, lse, o_ref, l_ref, a_ref, what="block sparse full mask")
    pa = fi.Plan("append", w.kv_indptr, w.kv_len, Hq, Hkv, 128, 16,
                 qo_indptr=torch.tensor([0, T], dtype=torch.int32), causal=False, device=dev)
    g = w.to(dev)
    oa, la = fi.paged_append(pa, g.q, g.k_cache, g.v_cache, g.kv_indices, w.sm_scale)
    torch.cuda.synchronize()
    compare(oa, la, o_ref, l_ref, a_ref, what="append over the same sequence")


@pytest.mark.parametrize("launch", ["default", "separate"])
def test_sparse_video_sampled(dev, launch):
    """The video-shaped sparse self-attention batch (8192 tokens, 16 heads,
    64 variable blocks per head): sampled query rows against the oracle."""
    w = make_sparse_video(poison=True)
    o, lse, p = _bs_run(w, dev, launch=launch)
    rng = np.random.default_rng(41)
    rows = sorted(set(rng.choice(w.q.shape[0], 48, replace=False).tolist()) | {0, 8191})
    o_ref, l_ref, a_ref = _bs_oracle(w, rows=rows)
    compare(o, lse, o_ref, l_ref, a_ref, rows=np.asarray(rows), what=f"sparse video {launch}")


# ---------------------------------------------------------------- HIP graphs


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


@pytest.mark.parametrize("cfg", [0, 1, 3, 4, "pod", "cascade_pod", "fp8", "mxfp4", "fused"])
def test_graph_replay_matches_eager(dev, cfg):
    """A captured run call (no allocation, no memset inside) replays to the
    eager bits, replay after replay, with other eager work in between. The
    tiny batch (folded after a workgroup barrier) and merge="fused" (folded
    by arrival counts, which each call's last arrival resets) are included:
    a count left over from a call would leave rows unfolded."""
    w = (make_pod_mix(poison=False) if cfg == "pod" else
         make_config(3 if cfg == "cascade_pod" else 1 if cfg in ("fp8", "mxfp4", "fused") else cfg,
                     poison=False))
    if cfg == "fp8":
        w = to_fp8_cache(w, poison=False)
    elif cfg == "mxfp4":
        w = to_mxfp4_cache(w, poison=False)
    g = w.to(dev)
    T = g.q.shape[0]
    out = torch.empty_like(g.q)
    lse = torch.empty(T, w.num_qo_heads, dtype=torch.float32, device=dev)
    if cfg in ("fp8", "mxfp4"):
        p = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                    w.page_size, device=dev, kv_format=cfg)
        if cfg == "fp8":
            call = lambda o, l: fi.paged_decode_fp8(p, g.q, g.k_fp8, g.v_fp8, g.k_scale,  # noqa
                                                    g.v_scale, g.kv_indices, w.sm_scale,
                                                    out=o, lse=l)
        else:
            call = lambda o, l: fi.paged_decode_mxfp4(p, g.q, g.k_fp4, g.v_fp4,  # noqa
                                                      g.k_bscale, g.v_bscale, g.kv_indices,
                                                      w.sm_scale, out=o, lse=l)
    elif w.kind == "decode":
        p = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                    w.page_size, device=dev, merge="fused" if cfg == "fused" else "default")
        if cfg in (0, "fused"):
            assert p.info()["fused_merge"]
        call = lambda o, l: fi.paged_decode(p, g.q, g.k_cache, g.v_cache, g.kv_indices,  # noqa
                                            w.sm_scale, out=o, lse=l)
    elif w.kind == "cascade":
        p = fi.Plan("cascade", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads,
                    w.head_dim, w.page_size, prefix_indptr=w.prefix_indptr,
                    prefix_len=w.prefix_len, req_prefix_group=w.req_prefix_group, device=dev,
                    launch="pod" if cfg == "cascade_pod" else "separate")
        call = lambda o, l: fi.cascade(p, g.q, g.k_cache, g.v_cache, g.prefix_indices,  # noqa
                                       g.kv_indices, w.sm_scale, out=o, lse=l)
    else:
        p = fi.Plan("append", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                    w.page_size, qo_indptr=w.qo_indptr, causal=True, device=dev,
                    launch="pod" if cfg == "pod" else "separate")
        call = lambda o, l: fi.paged_append(p, g.q, g.k_cache, g.v_cache, g.kv_indices,  # noqa
                                            w.sm_scale, k_new=g.k_new, v_new=g.v_new, out=o,
                                            lse=l)
    ref_o, ref_l = torch.empty_like(out), torch.empty_like(lse)
    call(ref_o, ref_l)
    torch.cuda.synchronize()
    graph = _capture(lambda: call(out, lse))
    for rep in range(3):
        out.fill_(7.0)
        lse.fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"config {cfg} replay {rep}"
        other_o, other_l = torch.empty_like(out), torch.empty_like(lse)
        call(other_o, other_l)          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other_o, ref_o)


def _stage(buf, t):
    """Copy t into the leading rows of a fixed buffer; return that view."""
    v = buf[: t.shape[0]]
    v.copy_(t)
    return v


@pytest.mark.parametrize("kind", ["decode", "append", "cascade"])
def test_graph_follows_replan_into_stable_workspace(dev, kind):
    """A run call captured once serves later batches: each batch is re-planned
    into the same graph-stable workspace and its inputs copied into the same
    buffers, and every replay equals the eager call on that batch, bit for
    bit, whatever its size, split or POD role mix."""
    Hq, Hkv, D, ps = 32, 8, 128, 16
    if kind == "decode":
        ws = [make_decode(L, Hq, Hkv, D, ps, seed=1000 + i, poison=False)
              for i, L in enumerate([[700, 33, 2048, 5], [100] * 9 + [3000], [9]])]
        cap = (10, 400, 0, 0)
    elif kind == "append":
        ws = [make_append(P, Q, Hq, Hkv, D, ps, seed=1100 + i, poison=False, causal=True)
              for i, (P, Q) in enumerate([([900, 40, 2000], [1, 130, 2]),
                                          ([50] * 6, [1] * 6),
                                          ([3000, 10], [300, 64])])]
        cap = (8, 400, 400, 0)
    else:
        ws = [make_cascade(P, grp, suf, Hq, Hkv, D, ps, seed=1200 + i, poison=False)
              for i, (P, grp, suf) in enumerate([([1024], [0, 0, 0, -1], [100, 5, 300, 40]),
                                                  ([2048, 64], [1, 0, 1, 0, 1, 0], [7] * 6),
                                                  ([16], [0], [999])])]
        cap = (8, 200, 0, 200)
    maxP = max(w.num_pages for w in ws)
    bufs = dict(q=torch.zeros(cap[0] * 64, Hq, D, dtype=torch.bfloat16, device=dev),
                k=torch.zeros(maxP, Hkv, ps, D, dtype=torch.bfloat16, device=dev),
                v=torch.zeros(maxP, Hkv, ps, D, dtype=torch.bfloat16, device=dev),
                idx=torch.zeros(512, dtype=torch.int32, device=dev),
                kn=torch.zeros(cap[0] * 64, Hkv, D, dtype=torch.bfloat16, device=dev),
                vn=torch.zeros(cap[0] * 64, Hkv, D, dtype=torch.bfloat16, device=dev),
                pidx=torch.zeros(512, dtype=torch.int32, device=dev),
                o=torch.zeros(cap[0] * 64, Hq, D, dtype=torch.bfloat16, device=dev),
                lse=torch.zeros(cap[0] * 64, Hq, dtype=torch.float32, device=dev))

    def plan_of(w, workspace=None):
        kw = dict(capacity=cap, device=dev, workspace=workspace)
        if kind == "append":
            kw.update(qo_indptr=w.qo_indptr, causal=True)
        if kind == "cascade":
            kw.update(prefix_indptr=w.prefix_indptr, prefix_len=w.prefix_len,
                      req_prefix_group=w.req_prefix_group)
        return fi.Plan(kind, w.kv_indptr, w.kv_len, Hq, Hkv, D, ps, **kw)

    def stage(w):
        g = w.to(dev)
        q = _stage(bufs["q"], g.q)
        bufs["k"][: w.num_pages].copy_(g.k_cache)
        bufs["v"][: w.num_pages].copy_(g.v_cache)
        idx = _stage(bufs["idx"], g.kv_indices)
        pidx = _stage(bufs["pidx"], g.prefix_indices) if kind == "cascade" else None
        new = None
        if kind == "append":      # the new tokens' K/V, scattered by the call
            new = (_stage(bufs["kn"], g.k_new), _stage(bufs["vn"], g.v_new))
        return q, idx, pidx, new

    def run(plan, q, idx, pidx, new):
        T = q.shape[0]
        o, lse = bufs["o"][:T], bufs["lse"][:T]
        if kind == "decode":
            fi.paged_decode(plan, q, bufs["k"], bufs["v"], idx, ws[0].sm_scale, out=o, lse=lse)
        elif kind == "append":
            fi.paged_append(plan, q, bufs["k"], bufs["v"], idx, ws[0].sm_scale, k_new=new[0],
                            v_new=new[1], out=o, lse=lse)
        else:
            fi.cascade(plan, q, bufs["k"], bufs["v"], pidx, idx, ws[0].sm_scale, out=o, lse=lse)

    p0 = plan_of(ws[0])
    args0 = stage(ws[0])
    graph = _capture(lambda: run(p0, *args0))
    for rep, w in enumerate(ws[1:] + ws[:1]):
        p = plan_of(w, workspace=p0.workspace)
        args = stage(w)
        T = args[0].shape[0]
        run(p, *args)                                  # eager, on this batch
        torch.cuda.synchronize()
        ref_o, ref_l = bufs["o"][:T].clone(), bufs["lse"][:T].clone()
        bufs["o"].fill_(7.0)
        bufs["lse"].fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["o"][:T], ref_o), f"{kind} batch {rep}: outputs differ"
        assert torch.equal(bufs["lse"][:T], ref_l), f"{kind} batch {rep}: lse differs"
        o_ref, l_ref, a_ref = _stable_oracle(kind, w)
        compare(bufs["o"][:T], bufs["lse"][:T], o_ref, l_ref, a_ref,
                what=f"graph replay after re-plan, {kind} batch {rep}")


def _stable_oracle(kind, w):
    if kind == "decode":
        return oracle_decode(w)
    if kind == "append":
        kp2, vp2 = _scattered_pools(w)
        return _oracle_append(w, kp2, vp2, True)
    return _oracle_cascade(w, None)


# ---------------------------------------------------------------- FP8 cache


def _fp8_oracle(w, requests=None):
    args = (w.kv_indptr.numpy(), w.kv_indices.numpy(), w.kv_len.numpy(), w.page_size,
            w.sm_scale)
    q = w.q.double().numpy()
    kc, vc = w.k_fp8.numpy(), w.v_fp8.numpy()
    ks, vs = w.k_scale.numpy(), w.v_scale.numpy()
    o, lse = oracle.paged_decode_fp8(q, kc, vc, ks, vs, *args, requests=requests)
    a, _ = oracle.paged_decode_fp8(q, kc, vc & 0x7F, ks, vs, *args, requests=requests)   # |V|
    return o, lse, a


def _fp8_run(w, dev, **kw):
    p = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                w.page_size, device=dev, **kw)
    g = w.to(dev)
    o, lse = fi.paged_decode_fp8(p, g.q, g.k_fp8, g.v_fp8, g.k_scale, g.v_scale, g.kv_indices,
                                 w.sm_scale)
    torch.cuda.synchronize()
    return o, lse


def test_fp8_llama_decode_sampled(dev):
    w = to_fp8_cache(make_config(1, poison=False), poison=True)
    rng = np.random.default_rng(21)
    reqs = sample_requests(w.batch, 8, rng, must=[int(torch.argmax(w.kv_len))])
    o_ref, l_ref, a_ref = _fp8_oracle(w, reqs)
    # an FP8 plan (two waves per SIMD, two LDS stages per wave) and a bf16
    # one (one wave, four stages)
    for kw in (dict(), dict(kv_format="fp8"), dict(deterministic=True),
               dict(deterministic=True, kv_format="fp8")):
        o, lse = _fp8_run(w, dev, **kw)
        compare(o, lse, o_ref, l_ref, a_ref, rows=request_rows(reqs), what=f"fp8 llama {kw}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("ps", [8, 16, 32, 64, 256])
@pytest.mark.parametrize("G", [1, 4, 8, 16, 24])
def test_fp8_decode_small_sweep(dev, D, ps, G):
    Hkv = 2
    w = to_fp8_cache(make_decode(SMALL_LENS, G * Hkv, Hkv, D, ps, seed=500 + D + ps + G,
                                 poison=False), poison=True)
    o_ref, l_ref, a_ref = _fp8_oracle(w)
    for kw in [dict(), dict(deterministic=True, det_chunk_pages=1), dict(min_chunk_pages=1),
               dict(kv_format="fp8", min_chunk_pages=1)]:
        o, lse = _fp8_run(w, dev, **kw)
        compare(o, lse, o_ref, l_ref, a_ref, what=f"fp8 decode D={D} ps={ps} G={G} {kw}")


def test_fp8_decode_refuses_the_valu_engine(dev):
    w = to_fp8_cache(make_decode([40, 7], 8, 2, 64, 16, seed=9, poison=False), poison=True)
    with pytest.raises(fi.FIError, match="matrix-core"):
        _fp8_run(w, dev, engine="valu")


# ---------------------------------------------------------------- MXFP4 cache


def _fp4_oracle(w, requests=None):
    args = (w.kv_indptr.numpy(), w.kv_indices.numpy(), w.kv_len.numpy(), w.page_size,
            w.sm_scale)
    q = w.q.double().numpy()
    kc, vc = w.k_fp4.numpy(), w.v_fp4.numpy()
    ks, vs = w.k_bscale.numpy(), w.v_bscale.numpy()
    o, lse = oracle.paged_decode_mxfp4(q, kc, vc, ks, vs, *args, requests=requests)
    a, _ = oracle.paged_decode_mxfp4(q, kc, vc & 0x77, ks, vs, *args, requests=requests)  # |V|
    return o, lse, a


def _fp4_run(w, dev, **kw):
    p = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                w.page_size, device=dev, **kw)
    g = w.to(dev)
    o, lse = fi.paged_decode_mxfp4(p, g.q, g.k_fp4, g.v_fp4, g.k_bscale, g.v_bscale,
                                   g.kv_indices, w.sm_scale)
    torch.cuda.synchronize()
    return o, lse


def test_mxfp4_llama_decode_sampled(dev):
    w = to_mxfp4_cache(make_config(1, poison=False), poison=True)
    rng = np.random.default_rng(22)
    reqs = sample_requests(w.batch, 8, rng, must=[int(torch.argmax(w.kv_len))])
    o_ref, l_ref, a_ref = _fp4_oracle(w, reqs)
    for kw in (dict(), dict(deterministic=True), dict(workers_per_cu=8),
               dict(kv_format="mxfp4"), dict(kv_format="mxfp4", deterministic=True)):
        o, lse = _fp4_run(w, dev, **kw)
        compare(o, lse, o_ref, l_ref, a_ref, rows=request_rows(reqs),
                what=f"mxfp4 llama {kw}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("ps", [8, 16, 32, 64, 256])
@pytest.mark.parametrize("G", [1, 4, 8, 16, 24])
def test_mxfp4_decode_small_sweep(dev, D, ps, G):
    Hkv = 2
    w = to_mxfp4_cache(make_decode(SMALL_LENS, G * Hkv, Hkv, D, ps, seed=600 + D + ps + G,
                                   poison=False), poison=True)
    o_ref, l_ref, a_ref = _fp4_oracle(w)
    for kw in [dict(), dict(deterministic=True, det_chunk_pages=1), dict(min_chunk_pages=1),
               dict(workers_per_cu=8, min_chunk_pages=1), dict(workers_per_cu=12)]:
        o, lse = _fp4_run(w, dev, **kw)
        compare(o, lse, o_ref, l_ref, a_ref, what=f"mxfp4 decode D={D} ps={ps} G={G} {kw}")


def test_mxfp4_decode_extreme_scales(dev):
    """Block scales spread far from 1 and different in every 32-element block
    of a row (K 2^-9 .. 2^0, V 2^-27 .. 2^23): each block's elements must take
    their own scale, exactly. Outputs are compared after division by one
    power of two (exact on both sides) so the absolute bar stays meaningful."""
    w = to_mxfp4_cache(make_decode([70, 33, 5], 8, 2, 128, 16, seed=61, poison=False),
                       poison=True)
    gen = torch.Generator().manual_seed(62)
    kb = torch.randint(118, 128, w.k_bscale.shape, generator=gen, dtype=torch.int32)
    vb = torch.randint(100, 151, w.v_bscale.shape, generator=gen, dtype=torch.int32)
    w.k_bscale = torch.where(w.k_bscale != 255, kb.to(torch.uint8), w.k_bscale)
    w.v_bscale = torch.where(w.v_bscale != 255, vb.to(torch.uint8), w.v_bscale)
    o_ref, l_ref, a_ref = _fp4_oracle(w)
    o, lse = _fp4_run(w, dev)
    c = 2.0 ** math.ceil(math.log2(np.abs(a_ref).max()))
    compare(o.double() / c, lse, o_ref / c, l_ref, a_ref / c, what="mxfp4 extreme scales")


def test_mxfp4_deterministic_mode_is_batch_invariant(dev):
    """Deterministic MXFP4 decode: a request's output bits do not depend on
    the rest of the batch nor on the plan's workers per CU (which picks the
    kernel's LDS ring depth: 8, 4 or 3 stages)."""
    rng = np.random.default_rng(16)
    lens = [4100] + list(rng.integers(1, 6000, 31))
    w = to_mxfp4_cache(make_decode(lens, 32, 8, 128, 16, seed=520, poison=False), poison=True)
    target = 0
    outs = []
    for reqs, wpc in (([target], 0), ([3, target, 9, 4], 4), ([9, 5, target], 8),
                      (list(rng.permutation(32)), 12)):
        sub = _sub_batch(w, [int(r) for r in reqs])
        for f in ("k_fp4", "v_fp4", "k_bscale", "v_bscale"):
            setattr(sub, f, getattr(w, f))
        pos = [int(r) for r in reqs].index(target)
        o, lse = _fp4_run(sub, dev, deterministic=True, det_chunk_pages=16, workers_per_cu=wpc)
        outs.append((o[pos].clone(), lse[pos].clone()))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    o_ref, l_ref, a_ref = _fp4_oracle(w, requests=[target])
    compare(outs[0][0][None], outs[0][1][None], o_ref[[target]], l_ref[[target]],
            a_ref[[target]], what="mxfp4 batch-invariant target vs oracle")


def test_mxfp4_decode_refuses_the_valu_engine(dev):
    w = to_mxfp4_cache(make_decode([40, 7], 8, 2, 64, 16, seed=9, poison=False), poison=True)
    with pytest.raises(fi.FIError, match="matrix-core"):
        _fp4_run(w, dev, engine="valu")


# ---------------------------------------------------------------- prefix trees


@pytest.mark.parametrize("det", [False, True])
def test_cascade_tree(dev, det):
    """Nested shared prefixes: 0 (root) <- 1 <- 3, 0 <- 2, and a second root 4;
    requests on every node and on none. Each prefix is read once for every
    request under it; the result is attention over the chain || suffix."""
    parent = [-1, 0, 0, 1, -1]
    pref = [2048, 512, 256, 128, 1008]
    rng = np.random.default_rng(31)
    B = 40
    groups = [int(x) for x in rng.integers(-1, 5, B)]
    suf = [int(x) for x in rng.integers(0, 700, B)]
    w = make_cascade(pref, groups, suf, 32, 8, 128, 16, seed=32, poison=True,
                     prefix_parent=parent)
    o_ref, l_ref, a_ref = _oracle_cascade(w, None)
    for pod in (False, True):
        o, lse = _cascade_run(w, dev, deterministic=det,
                              launch="pod" if pod else "separate")
        compare(o, lse, o_ref, l_ref, a_ref, what=f"cascade tree det={det} pod={pod}")
    # the same batch as plain decode over the flattened tables (GPU vs GPU)
    ip, ix, ln = cascade_flat_tables(w)
    p = fi.Plan("decode", ip, ln, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                device=dev)
    g = w.to(dev)
    of, lf = fi.paged_decode(p, g.q, g.k_cache, g.v_cache, ix.to(dev), w.sm_scale)
    torch.cuda.synchronize()
    compare(of, lf, o_ref, l_ref, a_ref, what="flat decode of the tree")


# ---------------------------------------------------------------- block-sparse batches


BSB_SEQS = [(90, 700, 6, 9), (3, 64, 1, 2), (0, 100, 0, 2), (40, 333, 3, 4), (1, 17, 1, 1),
            (130, 1000, 4, 6)]


def _bsb_run(w, dev, layout="paged", **kw):
    """A block-sparse batch through one plan: the paged pool, or the ragged
    copy of the same keys."""
    g = w.to(dev)
    if layout == "paged":
        p = fi.BlockSparsePlan(w.qo_lens, [int(x) for x in w.kv_len], w.row_block_szs,
                               w.col_block_szs, w.block_masks, None, w.num_qo_heads,
                               w.num_kv_heads, w.head_dim, w.page_size, kv_indptr=w.kv_indptr,
                               kv_indices=w.kv_indices, device=dev, **kw)
        k, v = g.k_cache, g.v_cache
    else:
        p = fi.BlockSparsePlan(w.qo_lens, [int(x) for x in w.kv_len], w.row_block_szs,
                               w.col_block_szs, w.block_masks, None, w.num_qo_heads,
                               w.num_kv_heads, w.head_dim, w.page_size,
                               kv_indptr=w.ragged_indptr, layout="ragged", device=dev, **kw)
        k, v = g.k_ragged, g.v_ragged
    o, lse = fi.block_sparse_attention(p, g.q, k, v, w.sm_scale)
    torch.cuda.synchronize()
    return o, lse, p


def _bsb_oracle(w, rows=None):
    kp, vp = np_pools(w)
    args = (w.qo_lens, [int(x) for x in w.kv_len], [r.numpy() for r in w.row_block_szs],
            [c.numpy() for c in w.col_block_szs], [m.numpy() for m in w.block_masks],
            w.sm_scale, w.kv_indptr.numpy())
    q = w.q.double().numpy()
    kw = dict(kv_indices=w.kv_indices.numpy(), page_size=w.page_size, rows=rows)
    o, lse = oracle.block_sparse_batch(q, kp, vp, *args, **kw)
    a, _ = oracle.block_sparse_batch(q, kp, np.abs(vp), *args, **kw)
    return o, lse, a


@pytest.mark.parametrize("D,ps,G", [(128, 16, 4), (64, 8, 1), (128, 32, 8), (64, 16, 2),
                                    (128, 64, 16), (128, 256, 4)])
def test_block_sparse_batch_small_sweep(dev, D, ps, G):
    """Several sequences in one block-sparse plan, each with its own variable
    blocks and mask (one without queries, one of a single key), through the
    paged pool and through a ragged copy of the same keys: every plan
    variant against the oracle, and the ragged bits equal the paged ones."""
    Hkv = 2
    w = to_ragged(make_block_sparse_batch(BSB_SEQS, G * Hkv, Hkv, D, ps, seed=960 + D + ps + G,
                                          poison="nan"), poison=True)
    o_ref, l_ref, a_ref = _bsb_oracle(w)
    for kw in [dict(), dict(launch="separate"), dict(deterministic=True, det_chunk_pages=1),
               dict(launch="separate", deterministic=True, det_chunk_pages=2),
               dict(min_chunk_pages=1), dict(pod_wide_blocks=1), dict(num_cus=3)]:
        o, lse, _ = _bsb_run(w, dev, "paged", **kw)
        compare(o, lse, o_ref, l_ref, a_ref, what=f"bs batch paged D={D} ps={ps} G={G} {kw}")
        o2, lse2, _ = _bsb_run(w, dev, "ragged", **kw)
        assert torch.equal(o2, o) and torch.equal(lse2, lse), f"ragged != paged {kw}"


@pytest.mark.parametrize("layout", ["paged", "ragged"])
def test_block_sparse_batch_deterministic_is_batch_invariant(dev, layout):
    """Deterministic mode: a sequence's rows keep their bits alone and in
    batches of other sequences, at any position."""
    Hq, Hkv, D, ps = 16, 4, 128, 16
    seqs = [(120, 900, 5, 8), (7, 300, 2, 3), (60, 500, 3, 5), (1, 40, 1, 2)]
    base = make_block_sparse_batch(seqs, Hq, Hkv, D, ps, seed=981, poison=True)
    target = 0
    outs = []
    for order in ([0], [2, 0, 3], [1, 3, 0, 2], [3, 2, 1, 0]):
        sub = _bsb_subset(base, order)
        o, lse, _ = _bsb_run(to_ragged(sub) if layout == "ragged" else sub, dev, layout,
                             deterministic=True, det_chunk_pages=4)
        q0 = sum(sub.qo_lens[:order.index(target)])
        outs.append((o[q0:q0 + seqs[target][0]].clone(), lse[q0:q0 + seqs[target][0]].clone()))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    o_ref, l_ref, a_ref = _bsb_oracle(base, rows=list(range(seqs[target][0])))
    r = np.arange(seqs[target][0])
    compare(outs[0][0], outs[0][1], o_ref[r], l_ref[r], a_ref[r],
            what=f"bs batch target {layout} vs oracle")


def _bsb_subset(w, order):
    """The block-sparse batch of sequences ``order`` of ``w`` (same pool)."""
    ptr, idx, qs = [0], [], []
    q_off = np.concatenate([[0], np.cumsum(w.qo_lens)])
    for s in order:
        a, b = int(w.kv_indptr[s]), int(w.kv_indptr[s + 1])
        idx.append(w.kv_indices[a:b])
        ptr.append(ptr[-1] + (b - a))
        qs.append(w.q[int(q_off[s]):int(q_off[s + 1])])
    kw = {f: getattr(w, f) for f in ("name", "kind", "num_qo_heads", "num_kv_heads", "head_dim",
                                      "page_size", "sm_scale", "seed", "k_cache", "v_cache")}
    from workloads import Workload
    return Workload(kv_len=w.kv_len[list(order)].clone(),
                    kv_indptr=torch.tensor(ptr, dtype=torch.int32),
                    kv_indices=torch.cat(idx).to(torch.int32), q=torch.cat(qs),
                    qo_lens=[w.qo_lens[s] for s in order],
                    row_block_szs=[w.row_block_szs[s] for s in order],
                    col_block_szs=[w.col_block_szs[s] for s in order],
                    block_masks=[w.block_masks[s] for s in order], **kw)
