"""Properties of the reference plan rule (CPU, no library needed).

These pin ``oracle.plan_ref`` to what any correct split-KV schedule must
satisfy: chunks partition each unit's key range in order, no chunk is empty or
larger than the chunk size, every output row is produced exactly once (by a
final write or by one merge entry), partial rows never overlap, and in
deterministic mode a request's chunk boundaries do not depend on its batch.
"""

import numpy as np
import pytest

from oracle.plan_ref import (FLAG_CAUSAL, FLAG_LIST_Q, FLAG_PARTIAL, ITEM_FIELDS, plan_ref)

F = {n: i for i, n in enumerate(ITEM_FIELDS)}


def _decode_inputs(lens, ps):
    n = [-(-L // ps) for L in lens]
    return np.concatenate([[0], np.cumsum(n)]).astype(int), np.array(lens)


def _all_items(plan):
    out = []
    for lv in plan["levels"]:
        out.extend(lv["items"])
    return out


def check_partition(plan, ps):
    units = {}
    for it in _all_items(plan):
        key = (it[F["flags"]] & FLAG_LIST_Q, it[F["unit"]], it[F["row0"]], it[F["kv_head"]])
        units.setdefault(key, []).append(it)
    for key, its in units.items():
        its.sort(key=lambda x: x[F["chunk"]])
        assert [x[F["chunk"]] for x in its] == list(range(len(its)))
        assert its[0][F["t_begin"]] == 0
        for a, b in zip(its[:-1], its[1:]):
            assert a[F["t_end"]] == b[F["t_begin"]]
            assert a[F["t_end"]] % ps == 0
        for x in its:
            assert x[F["t_end"]] > x[F["t_begin"]]
    return units


def check_outputs_once(plan, G, Hq, n_tokens):
    covered = np.zeros((n_tokens, Hq), dtype=int)
    rows_used = np.zeros(plan["n_part_rows"], dtype=int)
    for it in _all_items(plan):
        if it[F["flags"]] & FLAG_PARTIAL:
            rows_used[it[F["dst"]]:it[F["dst"]] + it[F["n_rows"]]] += 1
            continue
        assert not (it[F["flags"]] & FLAG_LIST_Q)
        for rho in range(it[F["row0"]], it[F["row0"]] + it[F["n_rows"]]):
            covered[it[F["q_base"]] + rho // G, it[F["kv_head"]] * G + rho % G] += 1
    assert np.all(rows_used == 1)
    for (qb, row0, nr, g, off, n) in plan["merges"]:
        for rho in range(row0, row0 + nr):
            covered[qb + rho // G, g * G + rho % G] += 1
        for p in plan["parts"][off:off + n]:
            assert 0 <= p and p + nr <= plan["n_part_rows"]
    return covered


@pytest.mark.parametrize("det", [False, True])
@pytest.mark.parametrize("ps", [8, 16])
def test_decode_plan_properties(det, ps):
    rng = np.random.default_rng(ps)
    lens = list(rng.integers(0, 700, 23)) + [0, 1, ps, ps + 1]
    indptr, L = _decode_inputs(lens, ps)
    S = 37
    p = plan_ref("decode", 32, 8, ps, indptr, L, S, [16], deterministic=det, det_chunk_pages=5,
                 min_chunk_pages=2)
    units = check_partition(p, ps)
    cov = check_outputs_once(p, 4, 32, len(lens))
    assert np.all(cov == 1)
    lv = p["levels"][0]
    assert lv["worker_indptr"][0] == 0 and lv["worker_indptr"][-1] == len(lv["items"])
    assert len(lv["worker_indptr"]) == S + 1
    if det:
        # rule 4 on a decode-style level: chunks of at most c // 2 pages, or
        # a 16th of the unit when that cap binds; equal within a page
        for its in units.values():
            n = -(-its[-1][F["t_end"]] // ps)
            k = min(-(-n // 2), 16)
            assert len(its) == k
            sizes = [-(-(x[F["t_end"]] - x[F["t_begin"]]) // ps) for x in its]
            assert max(sizes) <= max(2, -(-n // 16)) and max(sizes) - min(sizes) <= 1
    else:
        c = max(2, -(-8 * sum(-(-x // ps) for x in lens) // S))
        for it in lv["items"]:
            assert -(-(it[F["t_end"]] - it[F["t_begin"]]) // ps) <= c


def test_append_plan_properties():
    rng = np.random.default_rng(3)
    prefix = rng.integers(0, 300, 9)
    qo = rng.integers(0, 70, 9)
    qo[2] = 0
    L = prefix + qo
    ps = 16
    indptr, _ = _decode_inputs(list(L), ps)
    qo_indptr = np.concatenate([[0], np.cumsum(qo)])
    p = plan_ref("append", 32, 8, ps, indptr, L, 50, [32], qo_indptr=qo_indptr, causal=True)
    units = check_partition(p, ps)
    cov = check_outputs_once(p, 4, 32, int(qo_indptr[-1]))
    assert np.all(cov == 1)
    for its in units.values():
        it = its[-1]
        assert it[F["flags"]] & FLAG_CAUSAL
        r = it[F["unit"]]
        i_last = (it[F["row0"]] + it[F["n_rows"]] - 1) // 4
        assert it[F["t_end"]] == min(L[r], L[r] - qo[r] + i_last + 1)


def test_cascade_plan_properties():
    ps = 16
    suf = [5, 0, 40, 33, 16]
    groups = [0, 0, 1, -1, 0]
    pref = [64, 100]
    indptr, L = _decode_inputs(suf, ps)
    pindptr, PL = _decode_inputs(pref, ps)
    p = plan_ref("cascade", 8, 2, ps, indptr, L, 13, [8, 16], prefix_indptr=pindptr,
                 prefix_len=PL, req_group=groups)
    check_partition(p, ps)
    cov = check_outputs_once(p, 4, 8, len(suf))
    assert np.all(cov == 1)
    assert all(it[F["flags"]] & FLAG_PARTIAL for it in _all_items(p))
    assert p["qlist"] == [0, 1, 4, 2]


def test_deterministic_chunks_independent_of_batch():
    ps = 16
    target = 1234
    others = [17, 5000, 300, 0, 64, 9999]

    def chunks_of(lens, pos):
        indptr, L = _decode_inputs(lens, ps)
        p = plan_ref("decode", 32, 8, ps, indptr, L, 64, [16], deterministic=True,
                     det_chunk_pages=8)
        got = sorted((it[F["kv_head"]], it[F["chunk"]], it[F["t_begin"]], it[F["t_end"]])
                     for it in p["levels"][0]["items"] if it[F["unit"]] == pos)
        return got

    alone = chunks_of([target], 0)
    for k in range(1, len(others) + 1):
        for pos in (0, k // 2, k):
            lens = others[:k]
            lens = lens[:pos] + [target] + lens[pos:]
            assert chunks_of(lens, pos) == alone


def _worker_pages(lv, S, ps):
    out = []
    for w in range(S):
        its = lv["items"][lv["worker_indptr"][w]:lv["worker_indptr"][w + 1]]
        out.append(sum(-(-(x[F["t_end"]] - x[F["t_begin"]]) // ps) for x in its))
    return np.array(out)


@pytest.mark.parametrize("lens", [[32768] * 4 + [1024] * 124, list(range(500, 4600, 64)),
                                  [1, 2, 3, 17, 0, 5000]])
def test_balanced_mode_splits_steps_evenly(lens):
    """Every used worker runs exactly c 32-token steps, except the last used
    one; chunk boundaries fall on step boundaries (the kernels' granule)."""
    for ps in (8, 16, 64):
        gp = max(1, 32 // ps)
        indptr, L = _decode_inputs(lens, ps)
        S = 97
        p = plan_ref("decode", 32, 8, ps, indptr, L, S, [16], min_chunk_pages=2)
        lv = p["levels"][0]
        c = lv["chunk_pages"] // gp
        W = 8 * sum(-(-(-(-x // ps)) // gp) for x in lens)
        steps = np.zeros(S, dtype=np.int64)
        for w in range(S):
            for it in lv["items"][lv["worker_indptr"][w]:lv["worker_indptr"][w + 1]]:
                assert it[F["t_begin"]] % (gp * ps) == 0
                steps[w] += -(-(it[F["t_end"]] - it[F["t_begin"]]) // (gp * ps))
        used = -(-W // c)
        assert steps.sum() == W
        assert np.all(steps[:used - 1] == c) and 0 < steps[used - 1] <= c
        assert np.all(steps[used:] == 0)


def test_lpt_balances_deterministic_chunks():
    ps = 16
    lens = [32768] * 4 + [1024] * 124
    indptr, L = _decode_inputs(lens, ps)
    S = 2048
    p = plan_ref("decode", 32, 8, ps, indptr, L, S, [16], deterministic=True, det_chunk_pages=16)
    lv = p["levels"][0]
    loads = []
    for w in range(S):
        its = lv["items"][lv["worker_indptr"][w]:lv["worker_indptr"][w + 1]]
        loads.append(sum(-(-(x[F["t_end"]] - x[F["t_begin"]]) // ps) + 1 for x in its))
    total = sum(loads)
    # Graham's LPT bound: max load <= mean + largest item
    largest = max(-(-(x[F["t_end"]] - x[F["t_begin"]]) // ps) + 1 for x in lv["items"])
    assert max(loads) <= total / S + largest


def test_small_batch_keeps_units_whole():
    """Balanced mode: when splitting would save fewer than NO_SPLIT_STEPS steps,
    each unit is one item on worker = its enumeration index, and nothing merges."""
    ps, S = 16, 1024
    lens = [37, 300, 120, 5, 0]
    indptr, L = _decode_inputs(lens, ps)
    p = plan_ref("decode", 8, 2, ps, indptr, L, S, [16], fold_tiny=False)
    lv = p["levels"][0]
    # only the empty request's zero-part records (they write o = 0, lse = -inf)
    assert all(m[5] == 0 for m in p["merges"]) and len(p["merges"]) == 2
    units = [(r, g) for r in range(len(lens)) for g in range(2)]
    for i, (r, g) in enumerate(units):
        its = lv["items"][lv["worker_indptr"][i]:lv["worker_indptr"][i + 1]]
        if lens[r] == 0:
            assert len(its) == 0
            continue
        assert len(its) == 1 and its[0][F["t_begin"]] == 0 and its[0][F["t_end"]] == lens[r]
    # one long request: a split saves many steps, so it still happens
    lens2 = [37, 300, 4096]
    indptr2, L2 = _decode_inputs(lens2, ps)
    p2 = plan_ref("decode", 8, 2, ps, indptr2, L2, S, [16], fold_tiny=False)
    assert any(m[5] > 1 for m in p2["merges"])


# ---------------------------------------------------------------- rule 6 (fused launch)


def _append_inputs(prefix, qo, ps):
    L = np.asarray(prefix) + np.asarray(qo)
    indptr, _ = _decode_inputs(list(L), ps)
    return indptr, L, np.concatenate([[0], np.cumsum(qo)]).astype(int)


@pytest.mark.parametrize("det", [False, True])
def test_pod_roles_rows_and_padding(det):
    """Rule 6: a request whose rows (qo * G) fit 16 has all its items in the
    decode role (level 1) and none in the wide role, every other request the
    reverse; every query row is written exactly once across both roles; the
    worker lists are padded to P and 4P, with the padding workers empty."""
    ps, G, Hq, Hkv, P = 16, 4, 32, 8, 40
    rng = np.random.default_rng(60)
    qo = [int(x) for x in rng.choice([1, 2, 3, 4, 5, 17, 60, 200, 0], 30)]
    prefix = [int(x) for x in rng.integers(0, 2500, 30)]
    indptr, L, qo_indptr = _append_inputs(prefix, qo, ps)
    p = plan_ref("append", Hq, Hkv, ps, indptr, L, None, [128, 16], deterministic=det,
                 det_chunk_pages=6, min_chunk_pages=[4, 2], qo_indptr=qo_indptr, causal=True,
                 pod_blocks=P)
    n_w = p["pod_wide_blocks"]
    assert 1 <= n_w <= P - 1
    small = [q * G <= 16 for q in qo]
    for lev, role_small in ((0, False), (1, True)):
        for it in p["levels"][lev]["items"]:
            assert small[it[F["unit"]]] == role_small
            assert it[F["n_rows"]] <= (16 if role_small else 128)
    cov = check_outputs_once(p, G, Hq, int(qo_indptr[-1]))
    assert np.all(cov == 1)
    w0, w1 = p["levels"][0]["worker_indptr"], p["levels"][1]["worker_indptr"]
    assert len(w0) == P + 1 and len(w1) == 4 * P + 1
    assert w0[-1] == len(p["levels"][0]["items"]) and w1[-1] == len(p["levels"][1]["items"])
    assert all(w0[w] == w0[w + 1] for w in range(n_w, P))
    assert all(w1[w] == w1[w + 1] for w in range(4 * (P - n_w), 4 * P))


def test_pod_split_follows_the_work():
    """Rule 6's split: only wide work gives every workgroup to the wide role,
    only decode work none; an override is capped at P - 1; and as the decode
    role's work grows against fixed wide work, the wide role's share never
    grows."""
    ps, G, P = 16, 4, 64
    prefill = ([3000, 2000], [300, 129])

    def n_w(prefix, qo, **kw):
        indptr, L, qo_indptr = _append_inputs(prefix, qo, ps)
        return plan_ref("append", 32, 8, ps, indptr, L, None, [128, 16], qo_indptr=qo_indptr,
                        causal=True, min_chunk_pages=[16, 8], pod_blocks=P, **kw)["pod_wide_blocks"]

    assert n_w(*prefill) == P
    assert n_w([500] * 10, [1] * 10) == 0
    assert n_w(prefill[0] + [500], prefill[1] + [1], pod_wide_blocks=10 ** 6) == P - 1
    shares = []
    for n_dec in (1, 8, 32, 128, 512):
        shares.append(n_w(prefill[0] + [4000] * n_dec, prefill[1] + [1] * n_dec))
    assert all(a >= b for a, b in zip(shares, shares[1:])), shares
    assert shares[0] > shares[-1]


# ---------------------------------------------------------------- rule 7 (block-sparse)


@pytest.mark.parametrize("pod", [None, 24])
def test_block_sparse_units_address_the_selected_keys(pod):
    """Rule 7: token t of a (kv head, row block) unit must be the t-th key of
    its selected set, in key order. For every unit, the plan's page list at
    the unit's offset, read the way the kernels read it (page t // ps of the
    list, slot t % ps), addresses the same pool slot as that key does through
    the sequence's own page table; the unit's key count is the selected
    count, and its rows are the row block's."""
    rng = np.random.default_rng(70)
    ps, Hq, Hkv = 16, 8, 2
    G = Hq // Hkv
    T, Lk, MB, NB = 120, 900, 5, 7
    row_sz = np.array([[30, 2, 0, 50, 38], [1, 60, 59, 0, 0]])
    col_sz = []
    for g in range(Hkv):
        cuts = np.sort(rng.choice(np.arange(1, -(-Lk // ps)), NB - 1, replace=False)) * ps
        col_sz.append(np.diff(np.concatenate([[0], np.minimum(cuts, Lk), [Lk]])))
    col_sz = np.array(col_sz)
    col_sz[1, 2] = 0                                   # an empty column block
    mask = rng.random((Hkv, MB, NB)) < 0.5
    mask[0, 1, :] = False                               # a row block with no keys
    seq_pages = rng.permutation(200)[:-(-Lk // ps)]
    p = plan_ref("block_sparse", Hq, Hkv, ps, [0], [0], 31 if pod is None else None,
                 [128] if pod is None else [128, 16], min_chunk_pages=1,
                 block_sparse=(T, row_sz, col_sz, mask, seq_pages), pod_blocks=pod)
    plist = p["plist"]
    seen = {}
    for lv in p["levels"]:
        for it in lv["items"]:
            g, unit = it[F["kv_head"]], it[F["unit"]]
            a = unit - g * MB
            assert 0 <= a < MB
            keys = [c0 + t for b, (c0, c) in enumerate(zip(np.cumsum(col_sz[g]) - col_sz[g],
                                                           col_sz[g]))
                    if mask[g, a, b] for t in range(c)]
            assert it[F["q_base"]] == int(row_sz[g, :a].sum())
            assert it[F["row0"]] + it[F["n_rows"]] <= row_sz[g, a] * G
            for t in range(it[F["t_begin"]], it[F["t_end"]]):
                k = keys[t]
                assert plist[it[F["page_off"]] + t // ps] == seq_pages[k // ps]
                assert t % ps == k % ps
            seen.setdefault((g, a, it[F["row0"]]), []).append((it[F["t_begin"]], it[F["t_end"]]))
            assert it[F["t_end"]] <= len(keys)
    for g in range(Hkv):
        for a in range(MB):
            nsel = sum(int(c) for b, c in enumerate(col_sz[g]) if mask[g, a, b])
            for r0 in range(0, int(row_sz[g, a]) * G,
                            16 if pod and row_sz[g, a] * G <= 16 else 128):
                spans = sorted(seen.get((g, a, r0), []))
                covered = sum(e - b for b, e in spans)
                assert covered == nsel, (g, a, r0, covered, nsel)
    cov = check_outputs_once(p, G, Hq, T)
    assert np.all(cov == 1)


# ---------------------------------------------------------------- prefix trees


@pytest.mark.parametrize("det", [False, True])
def test_prefix_tree_parts_fold_root_first(det):
    """Rule 1 and 5 for a tree of prefixes: a request's merge folds the
    prefix parts of its chain in chain order from the root down, each
    prefix's chunks in chunk order, then its own suffix chunks in order; a
    group's units are over exactly the requests whose chain passes through
    it."""
    ps, Hq, Hkv = 16, 8, 2
    G = Hq // Hkv
    parent = [-1, 0, 1, 0, -1]
    pref = [300, 160, 96, 500, 64]
    groups = [2, 1, 0, 3, -1, 4, 2, 0, 1]
    suf = [40, 0, 700, 17, 33, 5, 90, 300, 1]
    indptr, L = _decode_inputs(suf, ps)
    pindptr, PL = _decode_inputs(pref, ps)
    p = plan_ref("cascade", Hq, Hkv, ps, indptr, L, [5, 11], [128, 16], deterministic=det,
                 det_chunk_pages=3, min_chunk_pages=1, prefix_indptr=pindptr, prefix_len=PL,
                 req_group=groups, prefix_parent=parent)

    def chain_root_first(r):
        c, h = [], groups[r]
        while h >= 0:
            c.append(h)
            h = parent[h]
        return c[::-1]

    # who wrote each partial row: (level, group or request, chunk), row offset
    owner = {}
    for lev, lv in enumerate(p["levels"]):
        for it in lv["items"]:
            for k in range(it[F["n_rows"]]):
                owner[it[F["dst"]] + k] = (lev, it[F["unit"]], it[F["chunk"]], it[F["kv_head"]],
                                          it[F["q_base"]], it[F["row0"]] + k)
    qlist = p["qlist"]
    assert len(p["merges"]) == len(suf) * Hkv
    for (r, row0, nr, g, off, n) in p["merges"]:
        assert row0 == 0 and nr == G
        seq = [owner[x] for x in p["parts"][off:off + n]]
        for lev, unit, chunk, kvh, qb, rho in seq:
            assert kvh == g
            if lev == 0:       # a prefix part: its row is this request's first head
                assert qlist[qb + rho // G] == r and rho % G == 0
            else:
                assert unit == r and rho == 0
        got = [(lev, unit, chunk) for lev, unit, chunk, *_ in seq]
        want = []
        for grp in chain_root_first(r):
            its = [it for it in p["levels"][0]["items"]
                   if it[F["unit"]] == grp and it[F["kv_head"]] == g]
            m = qlist.index(r, its[0][F["q_base"]]) - its[0][F["q_base"]]   # member index
            k = sum(1 for it in its if it[F["row0"]] <= m * G < it[F["row0"]] + it[F["n_rows"]])
            want.extend((0, grp, j) for j in range(k))
        ks = sum(1 for it in p["levels"][1]["items"]
                 if it[F["unit"]] == r and it[F["kv_head"]] == g)
        want.extend((1, r, j) for j in range(ks))
        assert got == want, (r, g, got, want)
    for grp in range(len(pref)):
        members = sorted(r for r in range(len(suf)) if grp in chain_root_first(r))
        its = [it for it in p["levels"][0]["items"] if it[F["unit"]] == grp]
        if not members:
            assert not its
            continue
        qb = its[0][F["q_base"]]
        assert qlist[qb:qb + len(members)] == members


def test_tiny_decode_spreads_steps_over_idle_workers():
    """Rule 3b: a decode batch with no more 32-token steps than workers, its
    split units folded in the kernel, runs one step per worker (W <= S):
    every unit of n steps is n one-step chunks on n distinct workers, in
    order, and every output row is still written exactly once. (Twelve
    units on 40 workers: more than S/4, so rule 3c does not apply.)"""
    ps, S = 16, 40
    lens = [37, 300, 120, 5, 0, 64]
    indptr, L = _decode_inputs(lens, ps)
    p = plan_ref("decode", 8, 2, ps, indptr, L, S, [16])
    check_partition(p, ps)
    assert np.all(check_outputs_once(p, 4, 8, len(lens)) == 1)
    lv = p["levels"][0]
    per_worker = np.diff(lv["worker_indptr"])
    assert per_worker.max() == 1                     # one step each
    W = sum(2 * -(-x // 32) for x in lens)           # 2 kv heads
    assert per_worker.sum() == W
    for it in lv["items"]:
        assert it[F["t_end"]] - it[F["t_begin"]] <= 32
    # with more steps than workers the rule does not apply
    assert (plan_ref("decode", 8, 2, ps, indptr, L, 8, [16], min_chunk_pages=8)
            == plan_ref("decode", 8, 2, ps, indptr, L, 8, [16], min_chunk_pages=8,
                        fold_tiny=False))


def test_tiny_decode_units_on_one_workgroup_each():
    """Rule 3c: with at most S/4 units, unit u's chunks are the items of
    workers 4u..4u+3 (one workgroup), chunk j covering steps [j k, (j+1) k)
    with k = ceil(steps / 4); every output row is written exactly once."""
    ps, S = 16, 1024
    lens = [37, 300, 120, 5, 0, 64]
    indptr, L = _decode_inputs(lens, ps)
    p = plan_ref("decode", 8, 2, ps, indptr, L, S, [16])
    check_partition(p, ps)
    assert np.all(check_outputs_once(p, 4, 8, len(lens)) == 1)
    lv = p["levels"][0]
    wi = np.asarray(lv["worker_indptr"])
    assert np.diff(wi).max() == 1
    by_worker = {w: lv["items"][wi[w]] for w in range(S) if wi[w + 1] > wi[w]}
    u = 0
    for r, n_tok in enumerate(lens):
        for g in range(2):           # units: requests x kv heads, in order
            ns = -(-n_tok // 32)
            k = -(-ns // 4)
            got = [(w % 4, it[F["t_begin"]], it[F["t_end"]]) for w, it in by_worker.items()
                   if w // 4 == u]
            want = [(j, 32 * j * k, min(n_tok, 32 * (j + 1) * k)) for j in range(4)
                    if j * k < min(ns, (j + 1) * k)]
            assert sorted(got) == want, (r, g, got, want)
            u += 1
    assert lv["chunk_pages"] == -(-(-(-300 // 32)) // 4) * 2
