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
    check_partition(p, ps)
    cov = check_outputs_once(p, 4, 32, len(lens))
    assert np.all(cov == 1)
    lv = p["levels"][0]
    assert lv["worker_indptr"][0] == 0 and lv["worker_indptr"][-1] == len(lv["items"])
    assert len(lv["worker_indptr"]) == S + 1
    c = 5 if det else max(2, -(-8 * sum(-(-x // ps) for x in lens) // S))
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
    p = plan_ref("decode", 8, 2, ps, indptr, L, S, [16])
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
    p2 = plan_ref("decode", 8, 2, ps, indptr2, L2, S, [16])
    assert any(m[5] > 1 for m in p2["merges"])
