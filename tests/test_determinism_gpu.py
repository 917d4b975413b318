"""GPU: deterministic mode is batch-invariant on every plan kind.

The contract (v0.7.4 article, *TL;DR* and *Three things to check before you
upgrade*): in deterministic mode the bits of a request's output rows do not
depend on the batch it runs in -- its size, its other requests, the request's
position in it. Each test runs one target request (or row block) inside
batches of different sizes and compositions, with the same pools, and asserts
that the target's o and lse are bit-identical in all of them; the first run is
also held to the oracle. The runs cover the cascade prefix level, where one
16-row MFMA block holds the rows of several requests (a request's row position
in the block moves with the member list), append in both launch shapes (the
POD launch's decode and wide roles), variable block-sparse plans (row blocks
of other heads and masks beside the target), and the FP8 and VALU decode
kernels.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_amd as fi
from tests.helpers import compare, np_pools, oracle_decode
from workloads import make_append, make_block_sparse, make_cascade, make_decode, to_fp8_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev(gpu):
    return gpu


def _assert_all_equal(outs, what):
    o0, l0 = outs[0]
    for i, (o, l) in enumerate(outs[1:], 1):
        assert torch.equal(o, o0), f"{what}: o bits differ in batch {i}"
        assert torch.equal(l, l0), f"{what}: lse bits differ in batch {i}"


def _tables(indptr, indices, lens, reqs):
    ptr, idx = [0], []
    for r in reqs:
        a, b = int(indptr[r]), int(indptr[r + 1])
        idx.append(indices[a:b])
        ptr.append(ptr[-1] + (b - a))
    return (torch.tensor(ptr, dtype=torch.int32),
            torch.cat(idx).to(torch.int32) if idx else torch.zeros(0, dtype=torch.int32),
            lens[list(reqs)].clone().to(torch.int32))


# ---------------------------------------------------------------- cascade


def _sub_cascade(w, reqs, q=None):
    """The cascade batch of requests ``reqs`` of ``w`` (same pool, same shared
    prefix, every request in group 0); ``q`` overrides the base queries."""
    ip, ix, ln = _tables(w.kv_indptr, w.kv_indices, w.kv_len, reqs)
    qq = (w.q if q is None else q)[list(reqs)].clone()
    return ip, ix, ln, qq


@pytest.mark.parametrize("launch", ["pod", "separate"])
def test_cascade_deterministic_is_batch_invariant(dev, launch):
    """Cascade: the target's bits are the same whether its prefix group holds
    1, 4, 33 or 64 members, wherever it sits in the member list (so in any row
    of a 16-row block of the prefix level), and beside a member whose scaled
    query moves its running max at other steps than the target's."""
    B, Hq, Hkv, D, ps = 64, 32, 8, 128, 16
    rng = np.random.default_rng(70)
    suf = [int(x) for x in rng.integers(0, 700, B)]
    w = make_cascade([3000], [0] * B, suf, Hq, Hkv, D, ps, seed=71, poison=True)
    q_hot = w.q.clone()
    q_hot[5] = (w.q[5].float() * 6.0).to(torch.bfloat16)   # a co-member with 6x logits
    target = 0
    batches = [([target], None), ([3, target, 9, 4], None), ([9, 5, target, 2], q_hot),
               ([5, target], q_hot), ([int(r) for r in rng.permutation(33)] + [target], None),
               ([int(r) for r in rng.permutation(B)], q_hot)]
    g = w.to(dev)
    outs = []
    for reqs, q in batches:
        reqs = list(dict.fromkeys(reqs))          # target once, order kept
        ip, ix, ln, qq = _sub_cascade(w, reqs, q)
        p = fi.Plan("cascade", ip, ln, Hq, Hkv, D, ps, prefix_indptr=w.prefix_indptr,
                    prefix_len=w.prefix_len,
                    req_prefix_group=torch.zeros(len(reqs), dtype=torch.int32), device=dev,
                    deterministic=True, det_chunk_pages=16, launch=launch)
        o, lse = fi.cascade(p, qq.to(dev), g.k_cache, g.v_cache, g.prefix_indices, ix.to(dev),
                            w.sm_scale)
        torch.cuda.synchronize()
        pos = reqs.index(target)
        outs.append((o[pos].clone(), lse[pos].clone()))
    _assert_all_equal(outs, f"cascade {launch}")
    kp, vp = np_pools(w)
    tabs = (w.prefix_indptr.numpy(), w.prefix_indices.numpy(), w.prefix_len.numpy(),
            w.req_prefix_group.numpy(), w.kv_indptr.numpy(), w.kv_indices.numpy(),
            w.kv_len.numpy(), w.page_size, w.sm_scale)
    qd = w.q.double().numpy()
    o_ref, l_ref = oracle.cascade_flat(qd, kp, vp, *tabs, requests=[target])
    a_ref, _ = oracle.cascade_flat(qd, kp, np.abs(vp), *tabs, requests=[target])
    compare(outs[0][0][None], outs[0][1][None], o_ref[[target]], l_ref[[target]],
            a_ref[[target]], what=f"cascade target {launch} vs oracle")


# ---------------------------------------------------------------- append


def _sub_append(w, reqs):
    """The append batch of requests ``reqs`` of ``w``: tables, query rows and
    new K/V rows of those requests, in that order."""
    ip, ix, ln = _tables(w.kv_indptr, w.kv_indices, w.kv_len, reqs)
    qo = [0]
    qs, kn, vn = [], [], []
    for r in reqs:
        a, b = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        qs.append(w.q[a:b])
        kn.append(w.k_new[a:b])
        vn.append(w.v_new[a:b])
        qo.append(qo[-1] + (b - a))
    return ip, ix, ln, torch.tensor(qo, dtype=torch.int32), torch.cat(qs), torch.cat(kn), \
        torch.cat(vn)


@pytest.mark.parametrize("launch", ["pod", "separate"])
def test_append_deterministic_is_batch_invariant(dev, launch):
    """Append (causal): two targets -- one of 50 query tokens (wide role), one
    of 3 (decode role under the POD launch) -- alone and in mixed batches of
    other sizes and orders; their rows' bits never change."""
    Hq, Hkv, D, ps = 32, 8, 128, 16
    rng = np.random.default_rng(80)
    B = 24
    prefix = [2000, 1500] + [int(x) for x in rng.integers(0, 3000, B - 2)]
    qo = [50, 3] + [int(x) for x in rng.choice([1, 1, 2, 7, 40, 130], B - 2)]
    w = make_append(prefix, qo, Hq, Hkv, D, ps, seed=81, poison=True, causal=True)
    targets = [0, 1]
    batches = [[0, 1], [1, 0], [4, 0, 9, 1, 2], [int(r) for r in rng.permutation(B)],
               [7, 1, 11, 0, 3, 5, 13]]
    outs = {t: [] for t in targets}
    for reqs in batches:
        ip, ix, ln, qo_ip, q, kn, vn = _sub_append(w, reqs)
        p = fi.Plan("append", ip, ln, Hq, Hkv, D, ps, qo_indptr=qo_ip, causal=True,
                    device=dev, deterministic=True, det_chunk_pages=8, launch=launch)
        kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)     # fresh pools: the call scatters
        o, lse = fi.paged_append(p, q.to(dev), kc, vc, ix.to(dev), w.sm_scale,
                                 k_new=kn.to(dev), v_new=vn.to(dev))
        torch.cuda.synchronize()
        for t in targets:
            j = reqs.index(t)
            a, b = int(qo_ip[j]), int(qo_ip[j + 1])
            outs[t].append((o[a:b].clone(), lse[a:b].clone()))
    for t in targets:
        _assert_all_equal(outs[t], f"append {launch} target {t}")
    kp, vp = np_pools(w)
    kp2, vp2 = oracle.scatter_new_kv(kp, vp, w.k_new.float().numpy(), w.v_new.float().numpy(),
                                     w.qo_indptr.numpy(), w.kv_indptr.numpy(),
                                     w.kv_indices.numpy(), w.kv_len.numpy(), ps)
    tabs = (w.kv_indptr.numpy(), w.kv_indices.numpy(), w.kv_len.numpy(), ps, w.sm_scale)
    qd = w.q.double().numpy()
    o_ref, l_ref = oracle.paged_append(qd, w.qo_indptr.numpy(), kp2, vp2, *tabs, causal=True,
                                       requests=targets)
    a_ref, _ = oracle.paged_append(qd, w.qo_indptr.numpy(), kp2, np.abs(vp2), *tabs,
                                   causal=True, requests=targets)
    for t in targets:
        a, b = int(w.qo_indptr[t]), int(w.qo_indptr[t + 1])
        compare(outs[t][0][0], outs[t][0][1], o_ref[a:b], l_ref[a:b], a_ref[a:b],
                what=f"append target {t} {launch} vs oracle")


# ---------------------------------------------------------------- block-sparse


@pytest.mark.parametrize("launch", ["default", "separate"])
def test_block_sparse_deterministic_is_invariant_to_other_blocks(dev, launch):
    """Block-sparse: the rows of a (kv head, row block) keep their bits when
    every other row block's selection, and the other kv head's, change (so
    the plan around it -- units, chunk placement, POD split -- changes). Two
    targets: a row block of 3 queries (12 rows: the decode role of a POD
    launch) and one of 60 (the wide role)."""
    Hq, Hkv, D, ps = 8, 2, 128, 16
    T, Lk = 300, 2000
    rows_sz = torch.tensor([[100, 3, 60, 90, 47], [32, 51, 170, 39, 8]], dtype=torch.int32)
    base = make_block_sparse(T, Lk, Hq, Hkv, D, ps, 5, 12, 0.5, seed=90, poison=True,
                             row_block_sz=rows_sz)
    G = Hq // Hkv
    targets = [(0, 1), (0, 2)]
    for g_t, a_t in targets:
        base.block_mask[g_t, a_t, 1::2] = True      # some keys for each target
    gen = torch.Generator().manual_seed(91)
    masks = [base.block_mask.clone()]
    for dens in (0.0, 0.9, 0.3):
        m = torch.rand(base.block_mask.shape, generator=gen) < dens
        for g_t, a_t in targets:
            m[g_t, a_t] = base.block_mask[g_t, a_t]
        masks.append(m)
    spans = []
    for g_t, a_t in targets:
        r = rows_sz[g_t].tolist()
        spans.append((sum(r[:a_t]), sum(r[:a_t + 1]), slice(g_t * G, (g_t + 1) * G)))
    g = base.to(dev)
    outs = [[] for _ in targets]
    for m in masks:
        p = fi.BlockSparsePlan(T, Lk, base.row_block_sz, base.col_block_sz, m, base.kv_indices,
                               Hq, Hkv, D, ps, device=dev, deterministic=True,
                               det_chunk_pages=4, launch=launch)
        o, lse = fi.block_sparse_attention(p, g.q, g.k_cache, g.v_cache, base.sm_scale)
        torch.cuda.synchronize()
        for i, (r0, r1, heads) in enumerate(spans):
            outs[i].append((o[r0:r1, heads].clone(), lse[r0:r1, heads].clone()))
    kp, vp = np_pools(base)
    args = (base.kv_indices.numpy(), Lk, ps, base.row_block_sz.numpy(),
            base.col_block_sz.numpy(), base.block_mask.numpy(), base.sm_scale)
    qd = base.q.double().numpy()
    for i, (r0, r1, heads) in enumerate(spans):
        _assert_all_equal(outs[i], f"block sparse {launch} target {targets[i]}")
        rr = list(range(r0, r1))
        o_ref, l_ref = oracle.block_sparse(qd, kp, vp, *args, rows=rr)
        a_ref, _ = oracle.block_sparse(qd, kp, np.abs(vp), *args, rows=rr)
        compare(outs[i][0][0], outs[i][0][1], o_ref[r0:r1, heads], l_ref[r0:r1, heads],
                a_ref[r0:r1, heads], what=f"block sparse target {targets[i]} {launch} vs oracle")


# ---------------------------------------------------------------- decode kernels


def _sub_decode(w, reqs):
    ip, ix, ln = _tables(w.kv_indptr, w.kv_indices, w.kv_len, reqs)
    return ip, ix, ln, w.q[list(reqs)].clone()


@pytest.mark.parametrize("kernel", ["fp8", "valu"])
def test_decode_kernels_deterministic_are_batch_invariant(dev, kernel):
    """The FP8 decode kernel and the VALU decode engine: a request's bits in
    deterministic mode do not depend on its batch."""
    rng = np.random.default_rng(100)
    lens = [4500] + [int(x) for x in rng.integers(1, 7000, 47)]
    w = make_decode(lens, 32, 8, 128, 16, seed=101, poison=kernel != "fp8")
    if kernel == "fp8":
        w = to_fp8_cache(w, poison=True)
    g = w.to(dev)
    target = 0
    outs = []
    for reqs in ([target], [3, target, 9, 4], [9, 5, target], [int(r) for r in rng.permutation(48)]):
        ip, ix, ln, q = _sub_decode(w, reqs)
        kw = dict(engine="valu") if kernel == "valu" else {}
        p = fi.Plan("decode", ip, ln, 32, 8, 128, 16, device=dev, deterministic=True,
                    det_chunk_pages=16, **kw)
        if kernel == "fp8":
            o, lse = fi.paged_decode_fp8(p, q.to(dev), g.k_fp8, g.v_fp8, g.k_scale, g.v_scale,
                                         ix.to(dev), w.sm_scale)
        else:
            o, lse = fi.paged_decode(p, q.to(dev), g.k_cache, g.v_cache, ix.to(dev), w.sm_scale)
        torch.cuda.synchronize()
        pos = reqs.index(target)
        outs.append((o[pos].clone(), lse[pos].clone()))
    _assert_all_equal(outs, f"decode {kernel}")
    if kernel == "valu":
        o_ref, l_ref, a_ref = oracle_decode(w, requests=[target])
        compare(outs[0][0][None], outs[0][1][None], o_ref[[target]], l_ref[[target]],
                a_ref[[target]], what="valu target vs oracle")
