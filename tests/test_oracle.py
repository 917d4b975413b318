"""Pins for the fp64 oracle: each check ties it to something other than itself.

* torch's scaled_dot_product_attention (float64, CPU) on dense K/V that the
  test itself scatters into a randomly permuted page pool (pins the gather,
  the head grouping, the scale, the softmax and the causal alignment);
* closed forms (one key, equal logits, two keys, constant V, needle);
* invariants (pool permutation, page size, split + merge, cascade == flat,
  append with one query == decode);
* mutation checks: mistakes planted in the oracle (on the CPU) must fail at
  least one pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A

RNG = np.random.default_rng(20241203)


# ---------------------------------------------------------------------------
# helpers that build paged inputs from dense ones (independent of the oracle)


def paginate(dense_list, page_size, rng, slack_pages=3, fill=np.nan):
    """dense_list[r] is [Hkv, L_r, D]; returns (pool, indptr, indices, lens)
    with pages placed at random pool slots and unused slots set to ``fill``."""
    Hkv, D = dense_list[0].shape[0], dense_list[0].shape[2]
    counts = [-(-d.shape[1] // page_size) for d in dense_list]
    total = sum(counts)
    P = total + slack_pages
    perm = rng.permutation(P)
    pool = np.full((P, Hkv, page_size, D), fill)
    indptr = np.zeros(len(dense_list) + 1, dtype=np.int64)
    indices = np.zeros(total, dtype=np.int64)
    pos = 0
    for r, d in enumerate(dense_list):
        L = d.shape[1]
        for p in range(counts[r]):
            page = perm[pos]
            indices[pos] = page
            for s in range(page_size):
                t = p * page_size + s
                if t < L:
                    pool[page, :, s, :] = d[:, t, :]
            pos += 1
        indptr[r + 1] = pos
    return pool, indptr, indices, np.array([d.shape[1] for d in dense_list])


def sdpa(q, k, v, scale, mask=None):
    """torch SDPA on float64 CPU tensors: q [n, D], k/v [L, D]."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, None]
    kt = torch.from_numpy(np.ascontiguousarray(k))[None, None]
    vt = torch.from_numpy(np.ascontiguousarray(v))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return out[0, 0].numpy()


def decode_case(B, Hq, Hkv, D, ps, lens, rng):
    dense_k = [rng.standard_normal((Hkv, L, D)) for L in lens]
    dense_v = [rng.standard_normal((Hkv, L, D)) for L in lens]
    kp, indptr, indices, L = paginate(dense_k, ps, rng)
    vp = np.full_like(kp, np.nan)
    # same page placement for V: copy through the same table
    for r, dv in enumerate(dense_v):
        for t in range(dv.shape[1]):
            vp[indices[indptr[r] + t // ps], :, t % ps, :] = dv[:, t, :]
    q = rng.standard_normal((B, Hq, D))
    return q, dense_k, dense_v, kp, vp, indptr, indices, L


# ---------------------------------------------------------------------------
# pins against torch SDPA


def check_decode_vs_sdpa(ps, D, Hq=8, Hkv=2, lens=(1, 7, 33, 40), seed=1):
    rng = np.random.default_rng(seed)
    B = len(lens)
    q, dk, dv, kp, vp, indptr, indices, L = decode_case(B, Hq, Hkv, D, ps, lens, rng)
    scale = 1.0 / math.sqrt(D)
    o, lse = A.paged_decode(q, kp, vp, indptr, indices, L, ps, scale)
    G = Hq // Hkv
    for r in range(B):
        for h in range(Hq):
            ref = sdpa(q[r, h][None], dk[r][h // G], dv[r][h // G], scale)[0]
            np.testing.assert_allclose(o[r, h], ref, rtol=0, atol=1e-12)
            # lse: log of the SDPA normaliser, via scipy's logsumexp on the dense logits
            from scipy.special import logsumexp
            s = scale * dk[r][h // G] @ q[r, h]
            assert abs(lse[r, h] - logsumexp(s)) <= 1e-12 * max(1.0, abs(lse[r, h]))


@pytest.mark.parametrize("ps", [1, 16, 64])
@pytest.mark.parametrize("D", [4, 64])
def test_decode_matches_sdpa(ps, D):
    check_decode_vs_sdpa(ps, D)


def check_append_vs_sdpa(ps=16, D=8, Hq=4, Hkv=2, prefixes=(5, 30), qos=(3, 17), seed=2):
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    lens = [p + n for p, n in zip(prefixes, qos)]
    _, dk, dv, kp, vp, indptr, indices, L = decode_case(len(lens), Hq, Hkv, D, ps, lens, rng)
    qo_indptr = np.concatenate([[0], np.cumsum(qos)])
    q = rng.standard_normal((int(qo_indptr[-1]), Hq, D))
    scale = 0.3
    o, lse = A.paged_append(q, qo_indptr, kp, vp, indptr, indices, L, ps, scale, causal=True)
    for r, (P, n) in enumerate(zip(prefixes, qos)):
        Lr = P + n
        mask = np.arange(Lr)[None, :] <= (P + np.arange(n))[:, None]   # bottom-right
        for h in range(Hq):
            ref = sdpa(q[qo_indptr[r]:qo_indptr[r + 1], h], dk[r][h // G], dv[r][h // G],
                       scale, mask)
            np.testing.assert_allclose(o[qo_indptr[r]:qo_indptr[r + 1], h], ref,
                                       rtol=0, atol=1e-12)


def test_append_matches_sdpa_bottom_right_causal():
    check_append_vs_sdpa()


# ---------------------------------------------------------------------------
# closed forms


def test_single_key():
    q = RNG.standard_normal((3, 16))
    k = RNG.standard_normal((1, 16))
    v = RNG.standard_normal((1, 16))
    o, lse = A.attend(q, k, v, 0.25)
    np.testing.assert_array_equal(o, np.repeat(v, 3, axis=0))
    np.testing.assert_allclose(lse, 0.25 * (q @ k[0]), rtol=0, atol=1e-15)


def test_equal_logits_mean_and_log_count():
    L = 37
    k = np.tile(RNG.standard_normal((1, 8)), (L, 1))
    v = RNG.standard_normal((L, 8))
    q = RNG.standard_normal((2, 8))
    o, lse = A.attend(q, k, v, 0.5)
    np.testing.assert_allclose(o, np.repeat(v.mean(0, keepdims=True), 2, 0), atol=1e-14)
    np.testing.assert_allclose(lse, 0.5 * (q @ k[0]) + math.log(L), atol=1e-13)
    o0, lse0 = A.attend(np.zeros((1, 8)), RNG.standard_normal((L, 8)), v, 1.0)
    np.testing.assert_allclose(lse0, [math.log(L)], atol=1e-14)


def test_constant_values():
    v = np.full((50, 4), 2.5)
    o, _ = A.attend(RNG.standard_normal((3, 4)), RNG.standard_normal((50, 4)), v, 1.0)
    np.testing.assert_allclose(o, 2.5, atol=1e-14)


def test_two_keys_closed_form():
    q = np.array([[1.0, -2.0]])
    k = np.array([[0.5, 1.0], [2.0, 0.25]])
    v = np.array([[1.0, 3.0], [-4.0, 0.5]])
    sc = 0.7
    s0 = sc * (1.0 * 0.5 + -2.0 * 1.0)
    s1 = sc * (1.0 * 2.0 + -2.0 * 0.25)
    lse = math.log(math.exp(s0) + math.exp(s1))
    a = 1.0 / (1.0 + math.exp(s1 - s0))   # sigma(s0 - s1)
    o_ref = [a * 1.0 + (1 - a) * -4.0, a * 3.0 + (1 - a) * 0.5]
    o, l = A.attend(q, k, v, sc)
    assert abs(l[0] - lse) < 1e-15
    np.testing.assert_allclose(o[0], o_ref, atol=1e-15)


@pytest.mark.parametrize("t_star", [0, 15, 16, 17, 63, 64, 99])
def test_needle_across_page_boundaries(t_star):
    """One key with a logit 60+ above all others: o is that key's value row."""
    ps, D, L = 16, 32, 100
    rng = np.random.default_rng(t_star)
    k = rng.standard_normal((1, L, D)) * 0.01
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    k[0, t_star, 0] = 100.0
    v = rng.standard_normal((1, L, D))
    kp, indptr, indices, Ls = paginate([k], ps, np.random.default_rng(t_star + 1))
    vp, _, _, _ = paginate([v], ps, np.random.default_rng(t_star + 1))  # same seed -> same perm
    assert np.array_equal(np.isnan(kp), np.isnan(vp))
    o, lse = A.paged_decode(q, kp, vp, indptr, indices, Ls, ps, 1.0)
    np.testing.assert_allclose(o[0, 0], v[0, t_star], rtol=1e-20, atol=1e-20)
    assert abs(lse[0, 0] - 100.0) < 1e-20 + 1e-15 * 100


def test_empty_sequence_is_zero_and_neg_inf():
    o, lse = A.attend(np.ones((2, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    vis = np.zeros((2, 3), dtype=bool)
    o, lse = A.attend(np.ones((2, 4)), np.ones((3, 4)), np.ones((3, 4)), 1.0, vis)
    assert np.all(o == 0) and np.all(lse == -np.inf)


# ---------------------------------------------------------------------------
# invariants


def test_pool_permutation_is_bit_identical():
    rng = np.random.default_rng(5)
    q, dk, dv, kp, vp, indptr, indices, L = decode_case(3, 4, 2, 16, 8, [9, 40, 23], rng)
    o1, l1 = A.paged_decode(q, kp, vp, indptr, indices, L, 8, 0.25)
    P = kp.shape[0]
    perm = rng.permutation(P)            # page p moves to slot perm[p]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    o2, l2 = A.paged_decode(q, kp2, vp2, indptr, perm[indices], L, 8, 0.25)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_page_size_is_bit_identical():
    rng = np.random.default_rng(6)
    lens = [1, 16, 65, 200]
    dk = [rng.standard_normal((2, L, 16)) for L in lens]
    dv = [rng.standard_normal((2, L, 16)) for L in lens]
    q = rng.standard_normal((4, 8, 16))
    outs = []
    for ps in (1, 16, 64):
        kp, ip, ix, L = paginate(dk, ps, np.random.default_rng(ps))
        vp, _, _, _ = paginate(dv, ps, np.random.default_rng(ps))
        outs.append(A.paged_decode(q, kp, vp, ip, ix, L, ps, 0.25))
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])


@pytest.mark.parametrize("cuts", [[5], [1, 2, 3], [10, 11, 50, 90], [0, 0, 40]])
def test_split_and_merge_equals_whole(cuts):
    rng = np.random.default_rng(len(cuts))
    L = 100
    q = rng.standard_normal((4, 32))
    k = rng.standard_normal((L, 32))
    v = rng.standard_normal((L, 32))
    o_full, l_full = A.attend(q, k, v, 0.2)
    bounds = [0] + sorted(cuts) + [L]
    states = [A.attend(q, k[a:b], v[a:b], 0.2) for a, b in zip(bounds[:-1], bounds[1:])]
    vs = np.stack([s[0] for s in states], axis=1)[:, :, None, :]     # [N=4, S, H=1, D]
    ss = np.stack([s[1] for s in states], axis=1)[:, :, None]
    o, l = A.merge_states(vs, ss)
    np.testing.assert_allclose(o[:, 0], o_full, atol=1e-12)
    np.testing.assert_allclose(l[:, 0], l_full, atol=1e-12)


def test_merge_algebra():
    rng = np.random.default_rng(7)
    o = rng.standard_normal((3, 5, 8))
    lse = rng.standard_normal((3, 5)) * 3
    a, b, c = [(o[i], lse[i]) for i in range(3)]
    ab = A.merge_two(*a, *b)
    ba = A.merge_two(*b, *a)
    np.testing.assert_allclose(ab[0], ba[0], atol=1e-14)
    np.testing.assert_allclose(ab[1], ba[1], atol=1e-14)
    l_ = A.merge_two(*A.merge_two(*a, *b), *c)
    r_ = A.merge_two(*a, *A.merge_two(*b, *c))
    np.testing.assert_allclose(l_[0], r_[0], atol=1e-13)
    np.testing.assert_allclose(l_[1], r_[1], atol=1e-13)
    empty = (np.zeros_like(o[0]), np.full(5, -np.inf))
    ident = A.merge_two(*a, *empty)
    np.testing.assert_array_equal(ident[1], a[1])
    np.testing.assert_allclose(ident[0], a[0], atol=1e-15)
    both = A.merge_two(*empty, *empty)
    assert np.all(both[0] == 0) and np.all(both[1] == -np.inf)


def test_cascade_flat_equals_two_level_and_flat_decode():
    rng = np.random.default_rng(8)
    ps, Hq, Hkv, D = 8, 4, 2, 16
    pref_lens = [32, 24]
    suf_lens = [5, 0, 17, 9, 30]
    groups = [0, 0, 1, -1, 0]
    dense_pref_k = [rng.standard_normal((Hkv, L, D)) for L in pref_lens]
    dense_pref_v = [rng.standard_normal((Hkv, L, D)) for L in pref_lens]
    dense_suf_k = [rng.standard_normal((Hkv, L, D)) for L in suf_lens]
    dense_suf_v = [rng.standard_normal((Hkv, L, D)) for L in suf_lens]
    allk = dense_pref_k + dense_suf_k
    allv = dense_pref_v + dense_suf_v
    kp, ip, ix, _ = paginate(allk, ps, np.random.default_rng(1))
    vp, _, _, _ = paginate(allv, ps, np.random.default_rng(1))
    npf = len(pref_lens)
    prefix_indptr = ip[:npf + 1]
    prefix_indices = ix
    kv_indptr = ip[npf:] - 0
    q = rng.standard_normal((len(suf_lens), Hq, D))
    args = (q, kp, vp, prefix_indptr, prefix_indices, np.array(pref_lens), np.array(groups),
            kv_indptr, ix, np.array(suf_lens), ps, 0.25)
    of, lf = A.cascade_flat(*args)
    o2, l2 = A.cascade_two_level(*args)
    np.testing.assert_allclose(of, o2, atol=1e-12)
    np.testing.assert_allclose(lf, l2, atol=1e-12)
    # flat page tables (prefixes are page aligned) through plain decode
    fl_indptr, fl_idx, fl_len = [0], [], []
    for r, g in enumerate(groups):
        pages = []
        L = suf_lens[r]
        if g >= 0:
            pages += list(ix[prefix_indptr[g]:prefix_indptr[g + 1]])
            L += pref_lens[g]
        pages += list(ix[kv_indptr[r]:kv_indptr[r + 1]])
        fl_idx += pages
        fl_indptr.append(len(fl_idx))
        fl_len.append(L)
    od, ld = A.paged_decode(q, kp, vp, np.array(fl_indptr), np.array(fl_idx), np.array(fl_len),
                            ps, 0.25)
    assert np.array_equal(od, of) and np.array_equal(ld, lf)


def check_cascade_tree():
    """Tree of prefixes 0 <- 1 <- 3 and 0 <- 2: flat definition == level by
    level == plain decode over the flat table built here by walking parents."""
    rng = np.random.default_rng(18)
    ps, Hq, Hkv, D = 8, 4, 2, 16
    pref_lens = [32, 24, 16, 8]
    parent = [-1, 0, 0, 1]
    suf_lens = [5, 0, 17, 9, 30, 3, 11]
    groups = [0, 1, 2, -1, 3, 3, 1]
    dk = [rng.standard_normal((Hkv, L, D)) for L in pref_lens + suf_lens]
    dv = [rng.standard_normal((Hkv, L, D)) for L in pref_lens + suf_lens]
    kp, ip, ix, _ = paginate(dk, ps, np.random.default_rng(2))
    vp, _, _, _ = paginate(dv, ps, np.random.default_rng(2))
    npf = len(pref_lens)
    prefix_indptr, kv_indptr = ip[:npf + 1], ip[npf:]
    q = rng.standard_normal((len(suf_lens), Hq, D))
    args = (q, kp, vp, prefix_indptr, ix, np.array(pref_lens), np.array(groups), kv_indptr, ix,
            np.array(suf_lens), ps, 0.25)
    of, lf = A.cascade_flat(*args, prefix_parent=np.array(parent))
    o2, l2 = A.cascade_two_level(*args, prefix_parent=np.array(parent))
    np.testing.assert_allclose(of, o2, atol=1e-12)
    np.testing.assert_allclose(lf, l2, atol=1e-12)
    fl_indptr, fl_idx, fl_len = [0], [], []
    for r, g in enumerate(groups):
        chain = []
        while g >= 0:
            chain.insert(0, g)
            g = parent[g]
        pages, L = [], suf_lens[r]
        for h in chain:
            pages += list(ix[prefix_indptr[h]:prefix_indptr[h + 1]])
            L += pref_lens[h]
        pages += list(ix[kv_indptr[r]:kv_indptr[r + 1]])
        fl_idx += pages
        fl_indptr.append(len(fl_idx))
        fl_len.append(L)
    od, ld = A.paged_decode(q, kp, vp, np.array(fl_indptr), np.array(fl_idx), np.array(fl_len),
                            ps, 0.25)
    np.testing.assert_allclose(od, of, atol=1e-12)
    np.testing.assert_allclose(ld, lf, atol=1e-12)


def test_cascade_tree_flat_equals_levels_and_flat_decode():
    check_cascade_tree()


def test_append_single_query_equals_decode():
    rng = np.random.default_rng(9)
    q, dk, dv, kp, vp, indptr, indices, L = decode_case(3, 8, 2, 16, 16, [3, 40, 77], rng)
    od, ld = A.paged_decode(q, kp, vp, indptr, indices, L, 16, 0.25)
    oa, la = A.paged_append(q, np.arange(4), kp, vp, indptr, indices, L, 16, 0.25, causal=True)
    np.testing.assert_allclose(oa, od, atol=1e-15)
    np.testing.assert_allclose(la, ld, atol=1e-15)


def test_causal_horizon_needle():
    """A dominant key at position p is seen by exactly the queries whose
    position is >= p (bottom-right alignment)."""
    ps, D = 4, 8
    P, n = 10, 6
    L = P + n
    rng = np.random.default_rng(10)
    for p_needle in (P - 1, P, P + 2, L - 1):
        k = rng.standard_normal((1, L, D)) * 0.01
        k[0, p_needle, 0] = 80.0
        v = rng.standard_normal((1, L, D))
        kp, ip, ix, Ls = paginate([k], ps, np.random.default_rng(3))
        vp, _, _, _ = paginate([v], ps, np.random.default_rng(3))
        q = np.zeros((n, 1, D))
        q[:, 0, 0] = 1.0
        o, _ = A.paged_append(q, np.array([0, n]), kp, vp, ip, ix, Ls, ps, 1.0, causal=True)
        for i in range(n):
            sees = P + i >= p_needle
            hit = np.allclose(o[i, 0], v[0, p_needle], atol=1e-20)
            assert hit == sees, (p_needle, i)


def test_scatter_writes_only_new_slots():
    rng = np.random.default_rng(11)
    ps, Hkv, D = 4, 2, 8
    lens = np.array([7, 12])
    qo = np.array([3, 5])
    indptr = np.array([0, 2, 5])
    indices = np.array([4, 0, 2, 6, 1])
    pool = rng.standard_normal((8, Hkv, ps, D))
    pool_v = rng.standard_normal((8, Hkv, ps, D))
    qo_indptr = np.array([0, 3, 8])
    k_new = rng.standard_normal((8, Hkv, D))
    v_new = rng.standard_normal((8, Hkv, D))
    k2, v2 = A.scatter_new_kv(pool, pool_v, k_new, v_new, qo_indptr, indptr, indices, lens, ps)
    touched = np.zeros((8, ps), dtype=bool)
    # request 0: positions 4,5,6 -> page indices[0 + 1] = 0, slots 0,1,2
    for pos, tok in zip([4, 5, 6], [0, 1, 2]):
        pg = indices[0 + pos // ps]
        np.testing.assert_array_equal(k2[pg, :, pos % ps], k_new[tok])
        np.testing.assert_array_equal(v2[pg, :, pos % ps], v_new[tok])
        touched[pg, pos % ps] = True
    # request 1: positions 7..11 -> pages indices[2 + pos//4]
    for pos, tok in zip(range(7, 12), range(3, 8)):
        pg = indices[2 + pos // ps]
        np.testing.assert_array_equal(k2[pg, :, pos % ps], k_new[tok])
        touched[pg, pos % ps] = True
    keep = ~touched
    np.testing.assert_array_equal(k2.transpose(0, 2, 1, 3)[keep], pool.transpose(0, 2, 1, 3)[keep])
    np.testing.assert_array_equal(v2.transpose(0, 2, 1, 3)[keep], pool_v.transpose(0, 2, 1, 3)[keep])


# ---------------------------------------------------------------------------
# mutation checks: plausible mistakes planted in the oracle must fail a pin


def _mut_gather_reverse_pages(pool, indices, start, length, page_size, kv_head):
    d = pool.shape[-1]
    if length <= 0:
        return np.zeros((0, d))
    n = -(-length // page_size)
    pages = np.asarray(indices[start:start + n])[::-1]
    return np.asarray(pool[pages, kv_head], np.float64).reshape(-1, d)[:length]


def _mut_gather_wrong_head(pool, indices, start, length, page_size, kv_head):
    return _ORIG["gather_tokens"](pool, indices, start, length, page_size,
                                  (kv_head + 1) % pool.shape[1])


def _mut_attend_no_scale(q, k, v, sm_scale, visible=None):
    return _ORIG["attend"](q, k, v, 1.0, visible)


def _mut_attend_log2(q, k, v, sm_scale, visible=None):
    o, l = _ORIG["attend"](q, k, v, sm_scale, visible)
    return o, l / math.log(2.0)


def _mut_attend_transposed_v(q, k, v, sm_scale, visible=None):
    o, l = _ORIG["attend"](q, k, v[::-1], sm_scale, visible)
    return o, l


def _mut_merge_sign(o1, l1, o2, l2):
    o, l = _ORIG["merge_two"](o1, l1, o2, -np.asarray(l2))
    return o, l


_ORIG = {n: getattr(A, n) for n in ("gather_tokens", "attend", "merge_two", "paged_append",
                                    "paged_decode_fp8", "e4m3_values", "_chain", "block_sparse",
                                    "gather_ragged")}


def _mut_append_top_left(q, qo_indptr, k_pool, v_pool, kv_indptr, kv_indices, kv_len,
                         page_size, sm_scale, causal=True, requests=None):
    # top-left alignment: query i sees keys 0..i (a classic mistake)
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    o = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    for r in range(len(kv_len)):
        q0, q1 = int(qo_indptr[r]), int(qo_indptr[r + 1])
        for g in range(Hkv):
            K = A.gather_tokens(k_pool, kv_indices, int(kv_indptr[r]), int(kv_len[r]), page_size, g)
            V = A.gather_tokens(v_pool, kv_indices, int(kv_indptr[r]), int(kv_len[r]), page_size, g)
            for i in range(q1 - q0):
                hs = slice(g * G, (g + 1) * G)
                o[q0 + i, hs], lse[q0 + i, hs] = A.attend(q[q0 + i, hs], K[:i + 1], V[:i + 1],
                                                          sm_scale)
    return o, lse


# ---------------------------------------------------------------------------
# FP8 (E4M3) cache


def test_e4m3_values_match_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = A.e4m3_values()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))   # -0 at 0x80


def test_e4m3_closed_forms():
    v = A.e4m3_values()
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0xC0] == -2.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0            # largest finite
    assert v[0x08] == 2.0 ** -6                                # smallest normal
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9    # subnormals
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2


def fp8_case(seed=3, ps=16, D=64, Hq=8, Hkv=2, lens=(1, 17, 40, 100)):
    rng = np.random.default_rng(seed)
    B = len(lens)
    n = [-(-L // ps) for L in lens]
    P = sum(n) + 3
    perm = rng.permutation(P)
    indptr = np.concatenate([[0], np.cumsum(n)])
    indices = perm[:sum(n)]
    kc = rng.integers(0, 256, (P, Hkv, ps, D), dtype=np.uint8)
    vc = rng.integers(0, 256, (P, Hkv, ps, D), dtype=np.uint8)
    for c in (kc, vc):                      # no NaN codes in used slots
        c[(c & 0x7F) == 0x7F] = 0x3C
    ks = rng.uniform(0.01, 0.1, (P, Hkv)).astype(np.float32)
    vs = rng.uniform(0.1, 2.0, (P, Hkv)).astype(np.float32)
    q = rng.standard_normal((B, Hq, D))
    return q, kc, vc, ks, vs, indptr, indices, np.array(lens), ps


def test_fp8_decode_equals_decode_of_torch_dequantized_pools():
    q, kc, vc, ks, vs, indptr, indices, L, ps = fp8_case()
    deq = lambda c, s: (torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()  # noqa
                        * s.astype(np.float64)[:, :, None, None])
    kp, vp = deq(kc, ks), deq(vc, vs)
    scale = 0.125
    o_ref, l_ref = A.paged_decode(q, kp, vp, indptr, indices, L, ps, scale)
    o, lse = A.paged_decode_fp8(q, kc, vc, ks, vs, indptr, indices, L, ps, scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, l_ref, rtol=1e-14, atol=0)
    # a subset of requests decodes only their pages and leaves the rest NaN
    o2, l2 = A.paged_decode_fp8(q, kc, vc, ks, vs, indptr, indices, L, ps, scale, requests=[1, 3])
    np.testing.assert_array_equal(o2[[1, 3]], o[[1, 3]])
    assert np.isnan(o2[[0, 2]]).all()


# ---------------------------------------------------------------------------
# MXFP4 (E2M1 elements, E8M0 block scales) cache


def test_e2m1_closed_forms():
    """The eight FP4 E2M1 magnitudes of the OCP microscaling format, in code
    order, then the same with the sign bit (bit 3) set; no NaN or infinity."""
    v = A.e2m1_values()
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(v[:8]) == mags
    assert list(v[8:]) == [-m for m in mags]
    assert np.signbit(v[8]) and not np.signbit(v[0])
    assert np.isfinite(v).all()


def test_e8m0_values_match_torch_for_every_code():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = A.e8m0_values()
    assert np.isnan(got[255]) and np.isnan(ref[255]) and np.isnan(got).sum() == 1
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[128] == 2.0 and got[0] == 2.0 ** -127
    assert got[254] == 2.0 ** 127


def test_mxfp4_dequantize_nibble_order_and_scale_blocks():
    # byte 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0x21
    codes[0, 17] = 0xF7          # element 34 = code 7 (6), element 35 = code 15 (-6)
    scales = np.array([[127, 130]], dtype=np.uint8)     # 1 for dims 0..31, 8 for 32..63
    d = A.mxfp4_dequantize(codes, scales)
    assert d.shape == (1, 64)
    want = np.zeros(64)
    want[0], want[1], want[34], want[35] = 0.5, 1.0, 48.0, -48.0
    assert np.array_equal(d[0], want)
    # the scale of element i is block i // 32 (not i % n_blocks)
    codes[0, :] = 0x22           # every element 1.0
    d = A.mxfp4_dequantize(codes, scales)
    assert np.array_equal(d[0, :32], np.ones(32)) and np.array_equal(d[0, 32:], np.full(32, 8.0))
    # a NaN scale poisons exactly its 32 elements
    d = A.mxfp4_dequantize(codes, np.array([[255, 127]], dtype=np.uint8))
    assert np.isnan(d[0, :32]).all() and np.array_equal(d[0, 32:], np.ones(32))


def mxfp4_case(seed=4, ps=16, D=64, Hq=8, Hkv=2, lens=(1, 17, 40, 100)):
    rng = np.random.default_rng(seed)
    B = len(lens)
    n = [-(-L // ps) for L in lens]
    P = sum(n) + 3
    indptr = np.concatenate([[0], np.cumsum(n)])
    indices = rng.permutation(P)[:sum(n)]
    kc = rng.integers(0, 256, (P, Hkv, ps, D // 2), dtype=np.uint8)
    vc = rng.integers(0, 256, (P, Hkv, ps, D // 2), dtype=np.uint8)
    ks = rng.integers(120, 128, (P, Hkv, ps, D // 32), dtype=np.uint8)
    vs = rng.integers(124, 134, (P, Hkv, ps, D // 32), dtype=np.uint8)
    q = rng.standard_normal((B, Hq, D))
    return q, kc, vc, ks, vs, indptr, indices, np.array(lens), ps


def _dequantize_by_fields(codes, scales):
    """Element by element from the integer bit fields of each code: sign bit 3,
    exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is m * 2^-1."""
    P, H, ps, nb = codes.shape
    D = 2 * nb
    out = np.empty((P, H, ps, D))
    for idx in np.ndindex(P, H, ps):
        for i in range(D):
            c = (int(codes[idx][i // 2]) >> (4 * (i % 2))) & 0xF
            e, m = (c >> 1) & 3, c & 1
            mag = m * 0.5 if e == 0 else (2 + m) * 2.0 ** (e - 2)
            out[idx][i] = (-mag if c & 8 else mag) * math.ldexp(1.0, int(scales[idx][i // 32]) - 127)
    return out


def test_mxfp4_decode_equals_decode_of_field_dequantized_pools():
    q, kc, vc, ks, vs, indptr, indices, L, ps = mxfp4_case()
    kp, vp = _dequantize_by_fields(kc, ks), _dequantize_by_fields(vc, vs)
    scale = 0.125
    o_ref, l_ref = A.paged_decode(q, kp, vp, indptr, indices, L, ps, scale)
    o, lse = A.paged_decode_mxfp4(q, kc, vc, ks, vs, indptr, indices, L, ps, scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, l_ref, rtol=1e-14, atol=0)
    o2, l2 = A.paged_decode_mxfp4(q, kc, vc, ks, vs, indptr, indices, L, ps, scale,
                                  requests=[0, 2])
    np.testing.assert_array_equal(o2[[0, 2]], o[[0, 2]])
    assert np.isnan(o2[[1, 3]]).all()


def test_mxfp4_planted_mistakes_fail_the_pins():
    """A nibble swap or an off-by-one scale bias in the dequantization is seen
    by the field-by-field route."""
    q, kc, vc, ks, vs, indptr, indices, L, ps = mxfp4_case(seed=6)
    kp = _dequantize_by_fields(kc, ks)
    swapped = ((kc & 0xF) << 4) | (kc >> 4)
    assert not np.array_equal(A.mxfp4_dequantize(swapped, ks), kp)
    assert not np.array_equal(A.mxfp4_dequantize(kc, ks + 1), kp)
    assert np.array_equal(A.mxfp4_dequantize(kc, ks), kp)


# ---------------------------------------------------------------------------
# variable block-sparse attention


def _cuts(rng, total, n, align=1):
    """n consecutive block sizes summing to total, every non-empty block
    starting at a multiple of align (the last may end anywhere)."""
    units = -(-total // align)
    edges = np.sort(rng.integers(0, units + 1, n - 1)) * align
    edges = np.concatenate([[0], np.minimum(edges, total), [total]])
    return np.diff(edges).astype(np.int64)


def block_sparse_case(seed, T=9, Lk=23, Hkv=2, G=2, D=4, ps=4, MB=3, NB=4, p_mask=0.5):
    rng = np.random.default_rng(seed)
    dk = rng.standard_normal((Hkv, Lk, D))
    dv = rng.standard_normal((Hkv, Lk, D))
    kp, indptr, indices, _ = paginate([dk], ps, rng)
    vp = np.full_like(kp, np.nan)
    for t in range(Lk):
        vp[indices[t // ps], :, t % ps, :] = dv[:, t, :]
    q = rng.standard_normal((T, Hkv * G, D))
    row = np.stack([_cuts(rng, T, MB) for _ in range(Hkv)])
    col = np.stack([_cuts(rng, Lk, NB, ps) for _ in range(Hkv)])
    mask = rng.random((Hkv, MB, NB)) < p_mask
    return q, dk, dv, kp, vp, indices, Lk, ps, row, col, mask


def brute_block_sparse(q, dk, dv, row, col, mask, scale):
    """Pure-Python loops: each row's visible keys listed one by one."""
    T, Hq, D = q.shape
    Hkv = dk.shape[0]
    G = Hq // Hkv
    o = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -math.inf)
    for h in range(Hq):
        g = h // G
        for i in range(T):
            a, acc = 0, 0
            while acc + row[g][a] <= i:
                acc += row[g][a]
                a += 1
            keys = []
            start = 0
            for b, c in enumerate(col[g]):
                if mask[g][a][b]:
                    keys.extend(range(start, start + c))
                start += c
            if not keys:
                continue
            s = [scale * sum(q[i, h, d] * dk[g, t, d] for d in range(D)) for t in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            lse[i, h] = m + math.log(z)
            for d in range(D):
                o[i, h, d] = sum(wj * dv[g, t, d] for wj, t in zip(w, keys)) / z
    return o, lse


def check_block_sparse_brute(seed=5):
    q, dk, dv, kp, vp, idx, Lk, ps, row, col, mask = block_sparse_case(seed, MB=3, NB=3)
    mask[:, 0, 1] = True
    mask[:, 1, 0] = False             # asymmetric, so a transposed lookup differs
    scale = 0.37
    o, lse = A.block_sparse(q, kp, vp, idx, Lk, ps, row, col, mask, scale)
    o_ref, l_ref = brute_block_sparse(q, dk, dv, row, col, mask, scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(l_ref))
    fin = np.isfinite(l_ref)
    np.testing.assert_allclose(lse[fin], l_ref[fin], rtol=1e-13, atol=0)


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_block_sparse_brute_force(seed):
    check_block_sparse_brute(seed)


def test_block_sparse_full_mask_is_plain_attention():
    q, dk, dv, kp, vp, idx, Lk, ps, row, col, mask = block_sparse_case(8, T=12, Lk=40, ps=8)
    mask[:] = True
    o, lse = A.block_sparse(q, kp, vp, idx, Lk, ps, row, col, mask, 0.5)
    G = q.shape[1] // dk.shape[0]
    for h in range(q.shape[1]):
        ref = sdpa(q[:, h], dk[h // G], dv[h // G], 0.5)
        np.testing.assert_allclose(o[:, h], ref, rtol=0, atol=1e-12)


def test_block_sparse_block_diagonal_is_per_block_attention():
    rng = np.random.default_rng(9)
    q, dk, dv, kp, vp, idx, Lk, ps, _, _, _ = block_sparse_case(9, T=10, Lk=32, ps=8)
    row = np.array([[3, 7, 0, 0], [5, 5, 0, 0]])
    col = np.array([[8, 24, 0, 0], [16, 16, 0, 0]])
    mask = np.zeros((2, 4, 4), dtype=bool)
    mask[:, 0, 0] = mask[:, 1, 1] = True
    o, lse = A.block_sparse(q, kp, vp, idx, Lk, ps, row, col, mask, 0.25)
    G = 2
    for h in range(q.shape[1]):
        g = h // G
        r0, c0 = 0, 0
        for a in range(2):
            r1, c1 = r0 + row[g][a], c0 + col[g][a]
            ref = sdpa(q[r0:r1, h], dk[g, c0:c1], dv[g, c0:c1], 0.25)
            np.testing.assert_allclose(o[r0:r1, h], ref, rtol=0, atol=1e-12)
            r0, c0 = r1, c1


def test_block_sparse_row_without_keys_is_zero_and_neg_inf():
    q, dk, dv, kp, vp, idx, Lk, ps, row, col, mask = block_sparse_case(10)
    mask[0, 1, :] = False                 # kv head 0, row block 1 sees nothing
    o, lse = A.block_sparse(q, kp, vp, idx, Lk, ps, row, col, mask, 1.0)
    r0, r1 = row[0][0], row[0][0] + row[0][1]
    assert np.all(o[r0:r1, 0:2] == 0) and np.all(np.isneginf(lse[r0:r1, 0:2]))


def block_sparse_batch_case(seed, seqs=((9, 23, 3, 4), (5, 8, 2, 1), (0, 12, 0, 2), (7, 1, 1, 1)),
                            Hkv=2, G=2, D=4, ps=4, p_mask=0.5):
    """A tiny batch: per sequence (queries, keys, row blocks, column blocks);
    dense per-sequence keys, a ragged [tokens, Hkv, D] copy (sequences at
    seeded gaps in the tensor: kv_indptr is not the running sum) and a paged
    copy in a random pool."""
    rng = np.random.default_rng(seed)
    dks, dvs, rows, cols, masks, qo, kl = [], [], [], [], [], [], []
    for (T, Lk, MB, NB) in seqs:
        dks.append(rng.standard_normal((Hkv, Lk, D)))
        dvs.append(rng.standard_normal((Hkv, Lk, D)))
        rows.append(np.stack([_cuts(rng, T, MB) if MB else np.zeros(0, np.int64)
                              for _ in range(Hkv)]).reshape(Hkv, MB))
        cols.append(np.stack([_cuts(rng, Lk, NB, ps) for _ in range(Hkv)]))
        masks.append(rng.random((Hkv, MB, NB)) < p_mask)
        qo.append(T)
        kl.append(Lk)
    gaps = rng.integers(0, 5, len(seqs))
    starts = np.cumsum(np.concatenate([[0], np.asarray(kl[:-1]) + gaps[:-1]])) + gaps[0]
    N = int(starts[-1] + kl[-1] + 3)
    kr = np.full((N, Hkv, D), np.nan)
    vr = np.full((N, Hkv, D), np.nan)
    for s, a0 in enumerate(starts):
        kr[a0:a0 + kl[s]] = dks[s].transpose(1, 0, 2)
        vr[a0:a0 + kl[s]] = dvs[s].transpose(1, 0, 2)
    # paged copy: every sequence's pages at random places of one pool
    n = [-(-L // ps) for L in kl]
    P = sum(n) + 2
    perm = rng.permutation(P)
    kp = np.full((P, Hkv, ps, D), np.nan)
    vp = np.full((P, Hkv, ps, D), np.nan)
    pindptr = np.concatenate([[0], np.cumsum(n)])
    pidx = perm[:sum(n)]
    for s in range(len(seqs)):
        for t in range(kl[s]):
            pg = pidx[pindptr[s] + t // ps]
            kp[pg, :, t % ps] = dks[s][:, t]
            vp[pg, :, t % ps] = dvs[s][:, t]
    q = rng.standard_normal((sum(qo), Hkv * G, D))
    return dict(q=q, dks=dks, dvs=dvs, rows=rows, cols=cols, masks=masks, qo=qo, kl=kl,
                kr=kr, vr=vr, r_indptr=np.append(starts, 0)[:-1], kp=kp, vp=vp,
                p_indptr=pindptr, p_idx=pidx, ps=ps)


def check_block_sparse_batch_brute(seed=11):
    c = block_sparse_batch_case(seed)
    for m in c["masks"]:
        if m.shape[1] > 1 and m.shape[2] > 1:
            m[:, 0, 1] = True
            m[:, 1, 0] = False
    scale = 0.41
    o, lse = A.block_sparse_batch(c["q"], c["kr"], c["vr"], c["qo"], c["kl"], c["rows"],
                                  c["cols"], c["masks"], scale, c["r_indptr"])
    q0 = 0
    for s, T in enumerate(c["qo"]):
        if T:
            o_ref, l_ref = brute_block_sparse(c["q"][q0:q0 + T], c["dks"][s], c["dvs"][s],
                                              c["rows"][s], c["cols"][s], c["masks"][s], scale)
            np.testing.assert_allclose(o[q0:q0 + T], o_ref, rtol=0, atol=1e-12)
            np.testing.assert_array_equal(np.isinf(lse[q0:q0 + T]), np.isinf(l_ref))
            fin = np.isfinite(l_ref)
            np.testing.assert_allclose(lse[q0:q0 + T][fin], l_ref[fin], rtol=1e-13, atol=0)
        q0 += T


@pytest.mark.parametrize("seed", [11, 12])
def test_block_sparse_batch_brute_force(seed):
    """A ragged batch (sequences at gaps in the tensor, one without queries,
    one of a single key) against pure-Python loops per sequence."""
    check_block_sparse_batch_brute(seed)


def test_block_sparse_batch_paged_equals_ragged_and_per_sequence():
    """The same keys laid out paged (a permuted pool) and ragged give the same
    result, and each sequence's rows equal block_sparse on that sequence
    alone with its own page list."""
    c = block_sparse_batch_case(13)
    scale = 0.3
    args = (c["q"], c["qo"], c["kl"], c["rows"], c["cols"], c["masks"], scale)
    o_r, l_r = A.block_sparse_batch(c["q"], c["kr"], c["vr"], *args[1:], c["r_indptr"])
    o_p, l_p = A.block_sparse_batch(c["q"], c["kp"], c["vp"], *args[1:], c["p_indptr"],
                                    kv_indices=c["p_idx"], page_size=c["ps"])
    np.testing.assert_allclose(o_p, o_r, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(l_p, l_r)
    q0 = 0
    for s, T in enumerate(c["qo"]):
        pages = c["p_idx"][c["p_indptr"][s]:c["p_indptr"][s + 1]]
        o1, l1 = A.block_sparse(c["q"][q0:q0 + T], c["kp"], c["vp"], pages, c["kl"][s], c["ps"],
                                c["rows"][s], c["cols"][s], c["masks"][s], scale)
        np.testing.assert_array_equal(o1, o_p[q0:q0 + T])
        np.testing.assert_array_equal(l1, l_p[q0:q0 + T])
        q0 += T


def _mut_ragged_from_zero(kv, start, length, kv_head):
    return _ORIG["gather_ragged"](kv, 0, length, kv_head)


def _mut_block_sparse_mask_transposed(q, kp, vp, idx, Lk, ps, row, col, mask, scale):
    return _ORIG["block_sparse"](q, kp, vp, idx, Lk, ps, row, col,
                                 np.transpose(np.asarray(mask), (0, 2, 1)), scale)


def _mut_chain_own_group_only(req_group, prefix_parent, r):
    return _ORIG["_chain"](req_group, None, r)


def _mut_fp8_swap_scales(q, kc, vc, ks, vs, *rest, **kw):
    return _ORIG["paged_decode_fp8"](q, kc, vc, vs, ks, *rest, **kw)


def _mut_e4m3_bias8():
    return _ORIG["e4m3_values"]() / 2.0


MUTATIONS = {
    "gather_reverse_pages": ("gather_tokens", _mut_gather_reverse_pages,
                             lambda: check_decode_vs_sdpa(16, 4)),
    "gather_wrong_head": ("gather_tokens", _mut_gather_wrong_head,
                          lambda: check_decode_vs_sdpa(16, 4)),
    "attend_no_scale": ("attend", _mut_attend_no_scale, lambda: check_decode_vs_sdpa(16, 4)),
    "attend_lse_log2": ("attend", _mut_attend_log2, test_two_keys_closed_form),
    "attend_transposed_v": ("attend", _mut_attend_transposed_v, test_two_keys_closed_form),
    "merge_sign": ("merge_two", _mut_merge_sign, lambda: test_split_and_merge_equals_whole([5])),
    "append_top_left": ("paged_append", _mut_append_top_left, check_append_vs_sdpa),
    "fp8_scales_swapped": ("paged_decode_fp8", _mut_fp8_swap_scales,
                           test_fp8_decode_equals_decode_of_torch_dequantized_pools),
    "e4m3_bias_8": ("e4m3_values", _mut_e4m3_bias8, test_e4m3_values_match_torch_for_every_code),
    "cascade_no_parents": ("_chain", _mut_chain_own_group_only, check_cascade_tree),
    "block_sparse_mask_transposed": ("block_sparse", _mut_block_sparse_mask_transposed,
                                     check_block_sparse_brute),
    "ragged_from_zero": ("gather_ragged", _mut_ragged_from_zero, check_block_sparse_batch_brute),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn, pin = MUTATIONS[name]
    pin()                                   # passes on the real oracle
    monkeypatch.setattr(A, attr, fn)
    with pytest.raises(AssertionError):
        pin()


def test_oracle_exports():
    for n in ("attend", "paged_decode", "paged_append", "merge_states", "cascade_flat",
              "plan_ref", "paged_decode_fp8", "e4m3_values", "block_sparse"):
        assert hasattr(oracle, n)
