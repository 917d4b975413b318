"""CPU tests of the C ABI: the library loads and exports every declared symbol,
the C++ planner equals the reference plan rule element for element, the
workspace bound covers every plan, and host-detectable errors are reported
with their codes before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_attention_amd as fi
from paged_kv_attention_amd import _lib as L
from oracle.plan_ref import plan_ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fi.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fi_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = fi.load()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"libfi.so does not export {n}"
    assert set(names) == set(L.SIGNATURES), "binding and header disagree"


def _indptr(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _decode_host(lens, ps):
    return _indptr([-(-int(x) // ps) for x in lens]), np.asarray(lens, dtype=np.int32)


def host_plan(kind, indptr, lens, Hq, Hkv, D, ps, **kw):
    return fi.Plan(kind, indptr, lens, Hq, Hkv, D, ps, device=None, **kw)


def level_params(info):
    """Per-level workers, rows per block and minimum chunk, as plan_ref takes them."""
    lv = info["levels"]
    return dict(num_workers=[x["num_workers"] for x in lv],
                rows_per_block=[x["rows_per_block"] for x in lv],
                min_chunk_pages=[x["min_chunk_pages"] for x in lv])


def compare(info, ref):
    assert len(info["levels"]) == len(ref["levels"])
    for lv, rl in zip(info["levels"], ref["levels"]):
        items = np.array(rl["items"], dtype=np.int32).reshape(-1, L.FI_ITEM_INTS)
        assert np.array_equal(lv["items"], items)
        assert np.array_equal(lv["worker_indptr"], np.array(rl["worker_indptr"], dtype=np.int32))
    assert np.array_equal(info["merges"],
                          np.array(ref["merges"], dtype=np.int32).reshape(-1, L.FI_MERGE_INTS))
    assert np.array_equal(info["parts"], np.array(ref["parts"], dtype=np.int32))
    assert np.array_equal(info["qlist"], np.array(ref["qlist"], dtype=np.int32))
    assert info["num_part_rows"] == ref["n_part_rows"]


@pytest.mark.parametrize("det", [False, True])
@pytest.mark.parametrize("ps,Hq,Hkv", [(16, 32, 8), (8, 8, 2), (32, 4, 4), (16, 40, 2)])
def test_decode_plan_matches_reference(det, ps, Hq, Hkv):
    rng = np.random.default_rng(ps * 100 + Hq)
    lens = list(rng.integers(0, 3000, 40)) + [0, 1, ps, 32768]
    indptr, L_ = _decode_host(lens, ps)
    kw = dict(deterministic=det, det_chunk_pages=16, min_chunk_pages=4, num_cus=7,
              workers_per_cu=5)
    p = host_plan("decode", indptr, L_, Hq, Hkv, 128, ps, **kw)
    info = p.info()
    assert info["levels"][0]["num_workers"] == 35
    ref = plan_ref("decode", Hq, Hkv, ps, indptr, L_, **level_params(info),
                   deterministic=det, det_chunk_pages=16)
    compare(info, ref)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("det", [False, True])
def test_append_plan_matches_reference(causal, det):
    rng = np.random.default_rng(7)
    ps = 16
    prefix = rng.integers(0, 2000, 12)
    qo = rng.integers(0, 130, 12)
    qo[3] = 0
    lens = prefix + qo
    indptr, L_ = _decode_host(lens, ps)
    qo_indptr = _indptr(qo)
    p = host_plan("append", indptr, L_, 32, 8, 128, ps, qo_indptr=qo_indptr, causal=causal,
                  deterministic=det, det_chunk_pages=8, num_cus=4, workers_per_cu=8,
                  launch="separate")
    info = p.info()
    assert info["levels"][0]["rows_per_block"] == 128 and info["levels"][0]["num_workers"] == 16
    ref = plan_ref("append", 32, 8, ps, indptr, L_, **level_params(info),
                   deterministic=det, det_chunk_pages=8, qo_indptr=qo_indptr, causal=causal)
    compare(info, ref)
    assert info["num_scatter"] == int(qo.sum())


def _pod_batch(rng, n_small, n_big, ps, G):
    """Requests of a few query tokens (rows fit one 16-row block) mixed with
    prefill chunks; kv lengths include the new tokens."""
    small_q = rng.integers(0, 16 // G + 1, n_small)
    big_q = rng.integers(16 // G + 1, 300, n_big)
    qo = np.concatenate([small_q, big_q])
    rng.shuffle(qo)
    lens = rng.integers(0, 3000, qo.size) + qo
    indptr, L_ = _decode_host(lens, ps)
    return indptr, L_, _indptr(qo), qo


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("det", [False, True])
@pytest.mark.parametrize("mix,force", [((20, 4), 0), ((30, 0), 0), ((0, 6), 0), ((12, 3), 5),
                                       ((12, 3), 40)])
def test_pod_plan_matches_reference(causal, det, mix, force):
    rng = np.random.default_rng(17 + mix[0] + force)
    ps, Hq, Hkv = 16, 32, 8
    indptr, L_, qo_indptr, qo = _pod_batch(rng, mix[0], mix[1], ps, Hq // Hkv)
    p = host_plan("append", indptr, L_, Hq, Hkv, 128, ps, qo_indptr=qo_indptr, causal=causal,
                  deterministic=det, det_chunk_pages=8, num_cus=6, workers_per_cu=8, launch="pod",
                  pod_wide_blocks=force)
    info = p.info()
    P = 6 * (8 // 2)     # two workgroups per CU per two workers
    lv = info["levels"]
    assert [x["num_workers"] for x in lv] == [P, 4 * P]
    assert [x["rows_per_block"] for x in lv] == [128, 16]
    ref = plan_ref("append", Hq, Hkv, ps, indptr, L_, **level_params(info), deterministic=det,
                   det_chunk_pages=8, qo_indptr=qo_indptr, causal=causal, pod_blocks=P,
                   pod_wide_blocks=force)
    compare(info, ref)
    n_w = info["pod_wide_blocks"]
    assert n_w == ref["pod_wide_blocks"]
    if mix[1] == 0:
        assert n_w == 0
    elif mix[0] == 0:
        assert n_w == P
    else:
        assert 1 <= n_w <= P - 1
        if force:
            assert n_w == min(force, P - 1)
    # the decode role holds exactly the requests whose rows fit 16, each row
    # block whole: a request's items sit in one role
    G = Hq // Hkv
    for role, items in ((0, lv[0]["items"]), (1, lv[1]["items"])):
        for q_base in np.unique(items[:, 0]) if len(items) else []:
            r = int(np.searchsorted(qo_indptr, q_base, side="right")) - 1
            assert (qo[r] * G <= 16) == (role == 1)
    # wide workers past n_w and decode workers past 4 (P - n_w) are empty
    wi, di = lv[0]["worker_indptr"], lv[1]["worker_indptr"]
    assert np.all(wi[n_w:] == wi[-1]) and np.all(di[4 * (P - n_w):] == di[-1])
    assert info["num_scatter"] == int(qo.sum())


def test_launch_defaults():
    """POD by default for append and cascade; decode plans ignore the field;
    the VALU decode engine runs separate launches."""
    rng = np.random.default_rng(3)
    indptr, L_, qo_indptr, qo = _pod_batch(rng, 8, 2, 16, 4)
    kw = dict(qo_indptr=qo_indptr, num_cus=4)
    p = host_plan("append", indptr, L_, 32, 8, 128, 16, **kw)
    q = host_plan("append", indptr, L_, 32, 8, 128, 16, launch="pod", **kw)
    compare(p.info(), dict(levels=[dict(items=x["items"], worker_indptr=x["worker_indptr"])
                                   for x in q.info()["levels"]],
                           merges=q.info()["merges"], parts=q.info()["parts"],
                           qlist=q.info()["qlist"], n_part_rows=q.info()["num_part_rows"]))
    assert p.info()["pod_wide_blocks"] == q.info()["pod_wide_blocks"] > 0
    p = host_plan("append", indptr, L_, 32, 8, 128, 16, launch="separate", **kw)
    assert len(p.info()["levels"]) == 1 and p.info()["pod_wide_blocks"] == 0
    p = host_plan("append", indptr, L_, 32, 8, 128, 16, engine="valu", **kw)
    assert len(p.info()["levels"]) == 1 and p.info()["pod_wide_blocks"] == 0
    d_indptr, d_len = _decode_host([100, 200], 16)
    p = host_plan("decode", d_indptr, d_len, 32, 8, 128, 16, num_cus=4, launch="pod")
    assert len(p.info()["levels"]) == 1 and p.info()["pod_wide_blocks"] == 0
    with pytest.raises(fi.FIError):
        host_plan("append", indptr, L_, 32, 8, 128, 16, qo_indptr=qo_indptr, num_cus=4,
                  launch="pod", pod_wide_blocks=-1)


def test_page_table_check_refuses_bad_plans_before_any_launch():
    lib = fi.load()
    cnt = ctypes.c_int32(0)
    assert lib.fi_check_page_tables(None, None, None, 10, ctypes.byref(cnt), None) == \
        L.FI_ERR_PLAN_MISMATCH
    d_indptr, d_len = _decode_host([100, 20], 16)
    p = host_plan("decode", d_indptr, d_len, 8, 2, 64, 16, num_cus=4)
    assert lib.fi_check_page_tables(p.handle, None, None, 10, ctypes.byref(cnt), None) == \
        L.FI_ERR_PLAN_MISMATCH                        # host-only plan
    assert b"host-only" in lib.fi_last_error()


def test_kv_format_picks_the_default_worker_count():
    """A decode plan for an MXFP4 cache defaults to 12 workers per CU, FP8 to
    8 and bf16 to 4; an explicit count wins; other plan kinds ignore the
    field; an unknown format is refused."""
    d_indptr, d_len = _decode_host([100, 2000, 37], 16)
    for fmt, wpc in (("bf16", 4), ("fp8", 8), ("mxfp4", 12)):
        p = host_plan("decode", d_indptr, d_len, 32, 8, 128, 16, num_cus=5, kv_format=fmt)
        assert p.info()["levels"][0]["num_workers"] == 5 * wpc
    p = host_plan("decode", d_indptr, d_len, 32, 8, 128, 16, num_cus=5, kv_format="mxfp4",
                  workers_per_cu=6)
    assert p.info()["levels"][0]["num_workers"] == 30
    rng = np.random.default_rng(4)
    indptr, L_, qo_indptr, qo = _pod_batch(rng, 8, 2, 16, 4)
    a = host_plan("append", indptr, L_, 32, 8, 128, 16, qo_indptr=qo_indptr, num_cus=4,
                  kv_format="mxfp4")
    b = host_plan("append", indptr, L_, 32, 8, 128, 16, qo_indptr=qo_indptr, num_cus=4)
    assert [lv["num_workers"] for lv in a.info()["levels"]] == \
        [lv["num_workers"] for lv in b.info()["levels"]]
    d = L.PlanDesc(kind=0, batch=3, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                   page_size=16, num_cus=5, kv_format=3)
    h = ctypes.c_void_p()
    ind = np.asarray(d_indptr, dtype=np.int32)
    ln = np.asarray(d_len, dtype=np.int32)
    st = fi.load().fi_plan(ctypes.byref(d), ind.ctypes.data_as(L.I32P), ln.ctypes.data_as(L.I32P),
                           None, None, None, None, None,   # qo, prefixes, groups, parents
                           None, 0, None, 0, None, ctypes.byref(h))
    assert st == L.FI_ERR_INVALID_ARG
    assert b"kv_format" in fi.load().fi_last_error()


@pytest.mark.parametrize("pod", [False, True])
@pytest.mark.parametrize("det", [False, True])
def test_cascade_plan_matches_reference(det, pod):
    rng = np.random.default_rng(11)
    ps = 16
    suf = list(rng.integers(0, 900, 30)) + [0]
    groups = list(rng.integers(-1, 3, 31))
    pref = [8192, 100, 0]
    indptr, L_ = _decode_host(suf, ps)
    pindptr, PL = _decode_host(pref, ps)
    p = host_plan("cascade", indptr, L_, 32, 8, 128, ps, prefix_indptr=pindptr, prefix_len=PL,
                  req_prefix_group=groups, deterministic=det, num_cus=16, workers_per_cu=4,
                  launch="pod" if pod else "separate")
    info = p.info()
    ref = plan_ref("cascade", 32, 8, ps, indptr, L_, **level_params(info), deterministic=det,
                   det_chunk_pages=48, prefix_indptr=pindptr, prefix_len=PL, req_group=groups,
                   pod_blocks=32 if pod else None)
    compare(info, ref)
    if pod:
        assert [x["num_workers"] for x in info["levels"]] == [32, 128]
        assert info["pod_wide_blocks"] == ref["pod_wide_blocks"] and \
            1 <= info["pod_wide_blocks"] <= 31


def test_fused_cascade_edge_splits():
    """Fused cascade plans where one role has nothing to do: all suffixes
    empty (the wide role takes the whole launch) and no prefixes."""
    ps = 16
    pindptr, PL = _decode_host([700], ps)
    for suf, groups in (([0, 0, 0], [0, 0, 0]), ([100, 30, 0], [-1, -1, -1])):
        indptr, L_ = _decode_host(suf, ps)
        p = host_plan("cascade", indptr, L_, 32, 8, 128, ps, prefix_indptr=pindptr,
                      prefix_len=PL, req_prefix_group=groups, num_cus=4, launch="pod")
        info = p.info()
        ref = plan_ref("cascade", 32, 8, ps, indptr, L_, **level_params(info),
                       prefix_indptr=pindptr, prefix_len=PL, req_group=groups, pod_blocks=8)
        compare(info, ref)
        assert info["pod_wide_blocks"] == (8 if sum(suf) == 0 else 0)
    with pytest.raises(fi.FIError):
        host_plan("cascade", indptr, L_, 32, 8, 128, ps, prefix_indptr=pindptr, prefix_len=PL,
                  req_prefix_group=groups, num_cus=4, launch="pod", engine="valu")


@pytest.mark.parametrize("det", [False, True])
def test_cascade_tree_plan_matches_reference(det):
    """A tree of shared prefixes: 0 is the root, 1 and 2 extend it, 3 extends 1,
    4 is a second root; requests hang off any node or none."""
    rng = np.random.default_rng(12)
    ps = 16
    suf = list(rng.integers(0, 900, 40)) + [0]
    groups = list(rng.integers(-1, 5, 41))
    pref = [4096, 512, 0, 1000, 300]
    parent = [-1, 0, 0, 1, -1]
    indptr, L_ = _decode_host(suf, ps)
    pindptr, PL = _decode_host(pref, ps)
    p = host_plan("cascade", indptr, L_, 32, 8, 128, ps, prefix_indptr=pindptr, prefix_len=PL,
                  req_prefix_group=groups, prefix_parent=parent, deterministic=det, num_cus=16,
                  workers_per_cu=4, launch="separate")
    info = p.info()
    ref = plan_ref("cascade", 32, 8, ps, indptr, L_, **level_params(info), deterministic=det,
                   det_chunk_pages=48, prefix_indptr=pindptr, prefix_len=PL, req_group=groups,
                   prefix_parent=parent)
    compare(info, ref)
    # a request of group 3 merges the prefixes of 0, 1, 3 (root first), then its suffix
    r = groups.index(3)
    m = [x for x in info["merges"] if x[0] == r][0]
    assert m[5] >= 3


def test_cascade_tree_errors():
    d = _desc(kind=2, num_prefix_groups=2)
    kw = dict(pindptr=[0, 2, 3], plen=[32, 10], grp=[1, 0])
    st, msg = _raw_plan(d, GOOD_INDPTR, GOOD_LENS, par=[-1, 1], **kw)      # own index
    assert st == L.FI_ERR_INVALID_ARG and "parent" in msg, msg
    st, msg = _raw_plan(d, GOOD_INDPTR, GOOD_LENS, par=[1, -1], **kw)      # forward
    assert st == L.FI_ERR_INVALID_ARG and "parent" in msg, msg
    st, msg = _raw_plan(d, GOOD_INDPTR, GOOD_LENS, par=[-1, 0], **kw)      # depth 2 > 1
    assert st == L.FI_ERR_INVALID_ARG and "max_prefix_depth" in msg, msg
    d2 = _desc(kind=2, num_prefix_groups=2, max_prefix_depth=2)
    st, msg = _raw_plan(d2, GOOD_INDPTR, GOOD_LENS, par=[-1, 0], **kw)
    assert st == L.FI_OK, msg


def test_workspace_bound_covers_plans():
    rng = np.random.default_rng(3)
    for trial in range(30):
        ps = int(rng.choice([8, 16, 32]))
        B = int(rng.integers(1, 60))
        kind = ["decode", "append", "cascade"][trial % 3]
        det = bool(trial % 2)
        pod = kind != "decode" and trial % 4 in (1, 2)
        lens = rng.integers(0, 5000, B)
        qo = np.minimum(lens, rng.integers(0, 100, B))
        if pod:   # mostly requests of one to four query tokens
            qo = np.minimum(lens, np.where(rng.random(B) < 0.8, rng.integers(1, 5, B), qo))
        indptr, L_ = _decode_host(lens, ps)
        kw = dict(deterministic=det, det_chunk_pages=int(rng.integers(1, 80)), num_cus=9,
                  workers_per_cu=3)
        n_q = 0
        n_p = 0
        if kind == "append":
            kw.update(qo_indptr=_indptr(qo), causal=True, launch="pod" if pod else "separate")
            n_q = int(qo.sum())
        depth = 1
        if kind == "cascade":
            pref = [int(x) for x in rng.integers(0, 4000, 2)]
            pi, pl = _decode_host(pref, ps)
            kw.update(prefix_indptr=pi, prefix_len=pl,
                      req_prefix_group=rng.integers(-1, 2, B))
            if trial % 4 == 2:
                kw.update(prefix_parent=[-1, 0])
                depth = 2
            kw.update(launch="pod" if pod else "separate")
            n_p = int(pi[-1])
        p = host_plan(kind, indptr, L_, 32, 8, 128, ps, **kw)
        info = p.info()
        desc = L.PlanDesc(kind={"decode": 0, "append": 1, "cascade": 2}[kind], batch=B,
                          num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=ps,
                          causal=1, deterministic=int(det), det_chunk_pages=kw["det_chunk_pages"],
                          num_cus=9, workers_per_cu=3,
                          num_prefix_groups=2 if kind == "cascade" else 0,
                          max_prefix_depth=depth, launch=1 if pod else 2)
        assert len(info["levels"]) == (2 if pod or kind == "cascade" else 1)
        dev, host = fi.Workspace.bound(desc, int(indptr[-1]), n_q, n_p)
        assert dev >= info["dev_bytes_used"], (trial, kind)
        assert host >= info["host_bytes_used"], (trial, kind)


# ---------------------------------------------------------------------------
# host-detectable errors


def _raw_plan(desc, indptr, lens, qo=None, pindptr=None, plen=None, grp=None, par=None):
    lib = fi.load()
    h = ctypes.c_void_p()
    arr = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.int32)  # noqa: E731
    keep = [arr(x) for x in (indptr, lens, qo, pindptr, plen, grp)]
    ptrs = [None if a is None else a.ctypes.data_as(L.I32P) for a in keep]
    par_arr = arr(par)
    parent = None if par_arr is None else par_arr.ctypes.data_as(L.I32P)
    st = lib.fi_plan(ctypes.byref(desc), *ptrs, parent, None, 0, None, 0, None, ctypes.byref(h))
    if st == 0:
        lib.fi_plan_destroy(h)
    return st, lib.fi_last_error().decode()


def _desc(**kw):
    base = dict(kind=0, batch=2, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                num_cus=4)
    base.update(kw)
    return L.PlanDesc(**base)


GOOD_INDPTR = [0, 1, 3]
GOOD_LENS = [10, 20]


@pytest.mark.parametrize("desc_kw,code", [
    (dict(head_dim=96), L.FI_ERR_UNSUPPORTED),
    (dict(page_size=12), L.FI_ERR_UNSUPPORTED),
    (dict(page_size=4), L.FI_ERR_UNSUPPORTED),
    (dict(num_qo_heads=6, num_kv_heads=4), L.FI_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), L.FI_ERR_INVALID_ARG),
    (dict(kind=7), L.FI_ERR_INVALID_ARG),
    (dict(batch=-1), L.FI_ERR_INVALID_ARG),
    (dict(num_cus=0), L.FI_ERR_INVALID_ARG),       # host-only plan needs num_cus
    (dict(det_chunk_pages=-2), L.FI_ERR_INVALID_ARG),
])
def test_plan_rejects_bad_desc(desc_kw, code):
    st, msg = _raw_plan(_desc(**desc_kw), GOOD_INDPTR, GOOD_LENS)
    assert st == code, msg
    assert msg


@pytest.mark.parametrize("indptr,lens", [
    ([1, 2, 4], [10, 20]),        # indptr[0] != 0
    ([0, 1, 2], [10, 20]),        # 20 tokens need 2 pages
    ([0, 2, 4], [10, 20]),        # 10 tokens need 1 page
    ([0, 1, 3], [10, -1]),        # negative length
])
def test_plan_rejects_inconsistent_tables(indptr, lens):
    st, msg = _raw_plan(_desc(), indptr, lens)
    assert st == L.FI_ERR_INVALID_ARG, msg


def test_append_rejects_qo_longer_than_kv():
    st, msg = _raw_plan(_desc(kind=1), GOOD_INDPTR, GOOD_LENS, qo=[0, 11, 32])
    assert st == L.FI_ERR_INVALID_ARG and "qo" in msg
    st, _ = _raw_plan(_desc(kind=1), GOOD_INDPTR, GOOD_LENS, qo=None)
    assert st == L.FI_ERR_INVALID_ARG


def test_cascade_rejects_bad_group_and_grouping():
    d = _desc(kind=2, num_prefix_groups=1)
    st, msg = _raw_plan(d, GOOD_INDPTR, GOOD_LENS, pindptr=[0, 2], plen=[32], grp=[0, 1])
    assert st == L.FI_ERR_INVALID_ARG, msg
    st, msg = _raw_plan(d, GOOD_INDPTR, GOOD_LENS, pindptr=[0, 2], plen=[32], grp=[0, -1])
    assert st == L.FI_OK, msg
    d = _desc(kind=2, num_prefix_groups=1, num_qo_heads=24, num_kv_heads=1)   # G = 24
    st, msg = _raw_plan(d, GOOD_INDPTR, GOOD_LENS, pindptr=[0, 2], plen=[32], grp=[0, -1])
    assert st == L.FI_ERR_UNSUPPORTED, msg


def test_decode_engine_field():
    d = _desc(decode_engine=L.FI_ENGINE_VALU)                       # G = 4
    st, msg = _raw_plan(d, GOOD_INDPTR, GOOD_LENS)
    assert st == L.FI_OK, msg
    d = _desc(decode_engine=L.FI_ENGINE_VALU, num_qo_heads=32, num_kv_heads=2)   # G = 16
    st, msg = _raw_plan(d, GOOD_INDPTR, GOOD_LENS)
    assert st == L.FI_ERR_UNSUPPORTED and "VALU" in msg, msg
    d = _desc(decode_engine=L.FI_ENGINE_MFMA, num_qo_heads=32, num_kv_heads=2)
    st, msg = _raw_plan(d, GOOD_INDPTR, GOOD_LENS)
    assert st == L.FI_OK, msg
    for bad in (-1, 3):
        st, msg = _raw_plan(_desc(decode_engine=bad), GOOD_INDPTR, GOOD_LENS)
        assert st == L.FI_ERR_INVALID_ARG, msg


def test_run_calls_reject_non_positive_scale():
    lib = fi.load()
    for bad in (0.0, -0.125, float("nan"), float("inf")):
        assert lib.fi_paged_decode(None, None, None, None, None, bad, None, None, None) == \
            L.FI_ERR_INVALID_ARG
        assert lib.fi_cascade(None, None, None, None, None, None, bad, None, None, None) == \
            L.FI_ERR_INVALID_ARG
        assert lib.fi_paged_append(None, None, None, None, None, None, None, bad, None, None,
                                   None) == L.FI_ERR_INVALID_ARG
        assert "sm_scale" in lib.fi_last_error().decode()


def test_run_calls_refuse_without_device_plan():
    lib = fi.load()
    assert lib.fi_paged_decode(None, None, None, None, None, 1.0, None, None, None) == \
        L.FI_ERR_PLAN_MISMATCH
    p = host_plan("decode", GOOD_INDPTR, GOOD_LENS, 8, 2, 128, 16, num_cus=2)
    st = lib.fi_paged_decode(p.handle, None, None, None, None, 1.0, None, None, None)
    assert st == L.FI_ERR_PLAN_MISMATCH and "host-only" in lib.fi_last_error().decode()
    st = lib.fi_cascade(p.handle, None, None, None, None, None, 1.0, None, None, None)
    assert st == L.FI_ERR_PLAN_MISMATCH


def test_merge_states_rejects_bad_shapes():
    lib = fi.load()
    assert lib.fi_merge_states(None, 0, None, 1, 1, 1, 6, None, 0, None, None) == \
        L.FI_ERR_UNSUPPORTED
    assert lib.fi_merge_states(None, 3, None, 1, 1, 1, 8, None, 0, None, None) == \
        L.FI_ERR_INVALID_ARG
    assert lib.fi_merge_states(None, 0, None, -1, 1, 1, 8, None, 0, None, None) == \
        L.FI_ERR_INVALID_ARG
    # empty problem is a no-op, no launch
    assert lib.fi_merge_states(None, 0, None, 0, 3, 4, 8, None, 0, None, None) == L.FI_OK


def test_workspace_size_rejects_bad_input():
    lib = fi.load()
    dev, host = ctypes.c_size_t(), ctypes.c_size_t()
    d = _desc()
    assert lib.fi_workspace_size(ctypes.byref(d), -1, 0, 0, ctypes.byref(dev),
                                 ctypes.byref(host)) == L.FI_ERR_INVALID_ARG
    assert lib.fi_workspace_size(None, 1, 0, 0, ctypes.byref(dev), ctypes.byref(host)) == \
        L.FI_ERR_INVALID_ARG
    d = _desc(head_dim=256)
    assert lib.fi_workspace_size(ctypes.byref(d), 1, 0, 0, ctypes.byref(dev),
                                 ctypes.byref(host)) == L.FI_ERR_UNSUPPORTED


# ---------------------------------------------------------------- block-sparse plans


def _bs_spec(rng, Hkv, T, Lk, ps, MB, NB, p_mask=0.5):
    def cuts(total, n, align):
        units = -(-total // align)
        e = np.sort(rng.integers(0, units + 1, n - 1)) * align
        return np.diff(np.concatenate([[0], np.minimum(e, total), [total]])).astype(np.int32)
    row = np.stack([cuts(T, MB, 1) for _ in range(Hkv)])
    col = np.stack([cuts(Lk, NB, ps) for _ in range(Hkv)])
    mask = (rng.random((Hkv, MB, NB)) < p_mask).astype(np.uint8)
    pages = rng.permutation(-(-Lk // ps) + 5)[: -(-Lk // ps)].astype(np.int32)
    return row, col, mask, pages


@pytest.mark.parametrize("launch", ["pod", "separate"])
@pytest.mark.parametrize("det", [False, True])
@pytest.mark.parametrize("Hq,Hkv,ps,T,Lk,MB,NB", [(8, 2, 16, 300, 1000, 5, 7),
                                                   (32, 8, 8, 40, 333, 3, 4),
                                                   (4, 4, 32, 17, 64, 17, 2),
                                                   (16, 2, 16, 1, 5000, 1, 9)])
def test_block_sparse_plan_matches_reference(launch, det, Hq, Hkv, ps, T, Lk, MB, NB):
    rng = np.random.default_rng(T + Lk + MB)
    row, col, mask, pages = _bs_spec(rng, Hkv, T, Lk, ps, MB, NB)
    p = fi.BlockSparsePlan(T, Lk, row, col, mask, pages, Hq, Hkv, 128, ps, device=None,
                           num_cus=5, workers_per_cu=4, deterministic=det, det_chunk_pages=6,
                           launch=launch)
    info = p.info()
    P = 5 * 2
    ref = plan_ref("block_sparse", Hq, Hkv, ps, [0], [], **level_params(info),
                   deterministic=det, det_chunk_pages=6,
                   pod_blocks=P if launch == "pod" else None,
                   block_sparse=(T, row, col, mask, pages))
    compare(info, ref)
    assert np.array_equal(info["plist"], np.array(ref["plist"], dtype=np.int32))
    if launch == "pod":
        assert info["pod_wide_blocks"] == ref["pod_wide_blocks"]
    # every (kv head, query token) row is covered exactly once: by one item
    # whose unit is unsplit, or by merge records
    G = Hq // Hkv
    seen = np.zeros((T, Hq), dtype=np.int64)
    for lv in info["levels"]:
        for it in lv["items"]:
            if it[5] & 2:       # partial rows: covered by the merges below
                continue
            for rho in range(it[1], it[1] + it[2]):
                seen[it[0] + rho // G, it[3] * G + rho % G] += 1
    for m in info["merges"]:
        for rho in range(m[1], m[1] + m[2]):
            seen[m[0] + rho // G, m[3] * G + rho % G] += 1
    assert np.all(seen == 1)
    # the plan fits its workspace bound
    d = L.PlanDesc(kind=L.FI_KIND_BLOCK_SPARSE, batch=1, num_qo_heads=Hq, num_kv_heads=Hkv,
                   head_dim=128, page_size=ps, deterministic=int(det), det_chunk_pages=6,
                   num_cus=5, workers_per_cu=4,
                   launch=L.FI_LAUNCH_POD if launch == "pod" else L.FI_LAUNCH_SEPARATE)
    db, hb = ctypes.c_size_t(), ctypes.c_size_t()
    assert fi.load().fi_workspace_size_block_sparse(ctypes.byref(d), T, Lk, MB, NB,
                                                    ctypes.byref(db), ctypes.byref(hb)) == 0
    assert db.value >= info["dev_bytes_used"] and hb.value >= info["host_bytes_used"]


def test_block_sparse_plan_errors():
    rng = np.random.default_rng(1)
    row, col, mask, pages = _bs_spec(rng, 2, 20, 100, 16, 2, 3)
    kw = dict(device=None, num_cus=4)
    bad_col = col.copy()
    bad_col[0, 0] += 1
    bad_col[0, 1] -= 1                      # second block starts off a page boundary
    if bad_col[0, 0] > 0 and bad_col[0, 1] >= 0 and bad_col[0, 1] + bad_col[0, 2] > 0:
        with pytest.raises(fi.FIError, match="page boundary"):
            fi.BlockSparsePlan(20, 100, row, bad_col, mask, pages, 8, 2, 64, 16, **kw)
    bad_row = row.copy()
    bad_row[1, 0] += 1                      # rows no longer sum to qo_len
    with pytest.raises(fi.FIError, match="sum"):
        fi.BlockSparsePlan(20, 100, bad_row, col, mask, pages, 8, 2, 64, 16, **kw)
    # fi_plan and fi_workspace_size refuse the block-sparse kind
    d = L.PlanDesc(kind=L.FI_KIND_BLOCK_SPARSE, batch=1, num_qo_heads=8, num_kv_heads=2,
                   head_dim=64, page_size=16, num_cus=4)
    h = ctypes.c_void_p()
    lib = fi.load()
    assert lib.fi_plan(ctypes.byref(d), None, None, None, None, None, None, None, None, 0, None,
                       0, None, ctypes.byref(h)) == L.FI_ERR_INVALID_ARG
    db, hb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.fi_workspace_size(ctypes.byref(d), 10, 0, 0, ctypes.byref(db),
                                 ctypes.byref(hb)) == L.FI_ERR_INVALID_ARG
    d.causal = 1
    assert lib.fi_plan_block_sparse(ctypes.byref(d), 20, 100, 2, None, 3, None, None, None, None,
                                    0, None, 0, None, ctypes.byref(h)) == L.FI_ERR_INVALID_ARG


# ---------------------------------------------------------------- graph-stable plans


@pytest.mark.parametrize("kind", ["decode", "append", "cascade"])
def test_stable_plans_share_one_layout(kind):
    """Plans of different batches under one capacity lay the workspace out
    identically (the size fi_workspace_size reports for the description), so a
    launch captured on one serves the others; a batch over a capacity is
    refused."""
    rng = np.random.default_rng(5)
    ps, cap = 16, (12, 500, 600, 300)
    sizes = set()
    for trial in range(6):
        B = int(rng.integers(1, 13))
        lens = rng.integers(1, 600, B)
        kw = dict(num_cus=6, capacity=cap)
        if kind == "append":
            qo = np.minimum(lens, rng.integers(1, 50, B))
            kw.update(qo_indptr=_indptr(qo), causal=True)
        if kind == "cascade":
            ng = int(rng.integers(1, 4))
            pi, pl = _decode_host([int(x) for x in rng.integers(0, 1200, ng)], ps)
            kw.update(prefix_indptr=pi, prefix_len=pl, req_prefix_group=rng.integers(-1, ng, B))
        indptr, L_ = _decode_host(lens, ps)
        info = host_plan(kind, indptr, L_, 32, 8, 128, ps, **kw).info()
        sizes.add((info["dev_bytes_used"], info["host_bytes_used"]))
    assert len(sizes) == 1
    d = L.PlanDesc(kind={"decode": 0, "append": 1, "cascade": 2}[kind], batch=1,
                   num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=ps, num_cus=6,
                   causal=int(kind == "append"), num_prefix_groups=2 if kind == "cascade" else 0,
                   cap_batch=cap[0], cap_kv_pages=cap[1], cap_qo_tokens=cap[2],
                   cap_prefix_pages=cap[3])
    for args in ((0, 0, 0), (10, 20, 30)):     # the bound ignores its arguments
        dev, host = fi.Workspace.bound(d, *args)
        assert (dev, host) == sizes.pop() if args == (0, 0, 0) else (dev, host) == (dev0, host0)
        dev0, host0 = dev, host
    indptr, L_ = _decode_host([16 * 600], ps)                 # 600 pages > 500
    kw = dict(num_cus=6, capacity=cap)
    if kind == "append":
        kw.update(qo_indptr=_indptr([1]))
    if kind == "cascade":
        pi, pl = _decode_host([16], ps)
        kw.update(prefix_indptr=pi, prefix_len=pl, req_prefix_group=[0])
    with pytest.raises(fi.FIError, match="capacity"):
        host_plan(kind, indptr, L_, 32, 8, 128, ps, **kw)


@pytest.mark.parametrize("det", [False, True])
def test_fused_merge_records(det):
    """A merge="fused" decode plan on the matrix cores folds its split units
    in the kernel:
    each item that writes partial rows points at the merge record whose part
    list holds its rows (the record of its own unit: same query and kv head),
    items writing final rows point nowhere, every split record is pointed at
    by exactly its part count of items, and the records of units with no keys
    are listed for the kernel to write. The VALU engine, merge="separate" and
    default plans launch the merge kernel instead."""
    ps = 16
    rng = np.random.default_rng(31)
    lens = list(rng.integers(0, 5000, 37)) + [0, 1, 0, 32768]
    indptr, L_ = _decode_host(lens, ps)
    p = host_plan("decode", indptr, L_, 32, 8, 128, ps, deterministic=det, det_chunk_pages=16,
                  num_cus=5, workers_per_cu=4, merge="fused")
    info = p.info()
    assert info["fused_merge"]
    items = info["levels"][0]["items"]
    rec = info["item_rec"]
    assert rec.shape == (len(items),)
    hits = np.zeros(len(info["merges"]), dtype=int)
    for it, e in zip(items, rec):
        partial = bool(it[5] & 2)
        assert (e >= 0) == partial
        if not partial:
            continue
        q_base, row0, n_rows, g, off, n = info["merges"][e]
        assert (q_base, g, row0, n_rows) == (it[0], it[3], it[1], it[2])
        assert it[9] in info["parts"][off:off + n]
        hits[e] += 1
    assert np.array_equal(hits, info["merges"][:, 5])
    assert list(info["empty_recs"]) == [e for e in range(len(info["merges"]))
                                       if info["merges"][e, 5] == 0]
    assert len(info["empty_recs"]) == 8 * 2          # two empty requests, 8 kv heads
    for kw in (dict(engine="valu", merge="fused"), dict(merge="separate"), dict()):
        q = host_plan("decode", indptr, L_, 32, 8, 128, ps, deterministic=det,
                      det_chunk_pages=16, num_cus=5, workers_per_cu=4, **kw).info()
        assert not q["fused_merge"] and len(q["item_rec"]) == 0


def _bs_batch_spec(rng, Hkv, ps, seqs, layout):
    """Per sequence (queries, keys, row blocks, column blocks): sizes, masks,
    and the key table of a paged pool (page ids) or a ragged tensor (token
    offsets with gaps between sequences)."""
    def cuts(total, n, align):
        if n == 0:
            return np.zeros(0, np.int32)
        units = -(-total // align)
        e = np.sort(rng.integers(0, units + 1, n - 1)) * align
        return np.diff(np.concatenate([[0], np.minimum(e, total), [total]])).astype(np.int32)
    rows, cols, masks = [], [], []
    for (T, Lk, MB, NB) in seqs:
        rows.append(np.stack([cuts(T, MB, 1) for _ in range(Hkv)]).reshape(Hkv, MB))
        cols.append(np.stack([cuts(Lk, NB, ps) for _ in range(Hkv)]).reshape(Hkv, NB))
        masks.append((rng.random((Hkv, MB, NB)) < 0.5).astype(np.uint8))
    if layout == "paged":
        n = [-(-Lk // ps) for (_, Lk, _, _) in seqs]
        indptr = _indptr(n)
        indices = rng.permutation(int(indptr[-1]) + 7)[: int(indptr[-1])].astype(np.int32)
    else:
        lens = [Lk for (_, Lk, _, _) in seqs]
        indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        indices = None
    return rows, cols, masks, indptr, indices


@pytest.mark.parametrize("layout", ["paged", "ragged"])
@pytest.mark.parametrize("launch", ["pod", "separate"])
@pytest.mark.parametrize("det", [False, True])
def test_block_sparse_batch_plan_matches_reference(layout, launch, det):
    """A batch of block-sparse sequences, paged or ragged: the C++ plan equals
    plan_ref rule 7 element for element, page lists included, every query
    row of every sequence is written exactly once, and the plan fits the
    batch workspace bound."""
    rng = np.random.default_rng(71 + det)
    Hq, Hkv, ps = 16, 4, 16
    seqs = [(300, 1000, 5, 7), (3, 64, 1, 2), (0, 200, 0, 3), (40, 333, 3, 4), (1, 17, 1, 1)]
    rows, cols, masks, indptr, indices = _bs_batch_spec(rng, Hkv, ps, seqs, layout)
    qo = [s[0] for s in seqs]
    kl = [s[1] for s in seqs]
    p = fi.BlockSparsePlan(qo, kl, rows, cols, masks, None, Hq, Hkv, 128, ps, kv_indptr=indptr,
                           kv_indices=indices, layout=layout, device=None, num_cus=5,
                           workers_per_cu=4, deterministic=det, det_chunk_pages=6,
                           launch=launch)
    info = p.info()
    P = 5 * 2
    ref = plan_ref("block_sparse", Hq, Hkv, ps, [0], [], **level_params(info),
                   deterministic=det, det_chunk_pages=6,
                   pod_blocks=P if launch == "pod" else None,
                   block_sparse_batch=(qo, rows, cols, masks, indptr, indices))
    compare(info, ref)
    assert np.array_equal(info["plist"], np.array(ref["plist"], dtype=np.int32))
    G = Hq // Hkv
    T = sum(qo)
    seen = np.zeros((T, Hq), dtype=np.int64)
    for lv in info["levels"]:
        for it in lv["items"]:
            if it[5] & 2:
                continue
            for rho in range(it[1], it[1] + it[2]):
                seen[it[0] + rho // G, it[3] * G + rho % G] += 1
    for m in info["merges"]:
        for rho in range(m[1], m[1] + m[2]):
            seen[m[0] + rho // G, m[3] * G + rho % G] += 1
    assert np.all(seen == 1)
    d = L.PlanDesc(kind=L.FI_KIND_BLOCK_SPARSE, batch=1, num_qo_heads=Hq, num_kv_heads=Hkv,
                   head_dim=128, page_size=ps, deterministic=int(det), det_chunk_pages=6,
                   num_cus=5, workers_per_cu=4,
                   launch=L.FI_LAUNCH_POD if launch == "pod" else L.FI_LAUNCH_SEPARATE,
                   kv_layout=L.FI_KV_LAYOUT_RAGGED if layout == "ragged" else 0)
    db, hb = ctypes.c_size_t(), ctypes.c_size_t()
    a = p._ha
    assert fi.load().fi_workspace_size_block_sparse_batch(
        ctypes.byref(d), len(seqs), a["qo_len"].ctypes.data_as(L.I32P),
        a["kv_len"].ctypes.data_as(L.I32P), a["nrb"].ctypes.data_as(L.I32P),
        a["ncb"].ctypes.data_as(L.I32P), ctypes.byref(db), ctypes.byref(hb)) == 0
    assert db.value >= info["dev_bytes_used"] and hb.value >= info["host_bytes_used"]


def test_block_sparse_batch_errors():
    rng = np.random.default_rng(3)
    Hkv, ps = 2, 16
    seqs = [(20, 100, 2, 3), (5, 40, 1, 2)]
    rows, cols, masks, indptr, indices = _bs_batch_spec(rng, Hkv, ps, seqs, "ragged")
    kw = dict(device=None, num_cus=4, layout="ragged")
    bad = indptr.copy()
    bad[2] += 1                             # ragged span != kv_len
    with pytest.raises(fi.FIError, match="spans"):
        fi.BlockSparsePlan([20, 5], [100, 40], rows, cols, masks, None, 8, 2, 64, ps,
                           kv_indptr=bad, **kw)
    with pytest.raises(fi.FIError, match="spans"):   # paged: spans are pages
        fi.BlockSparsePlan([20, 5], [100, 40], rows, cols, masks, None, 8, 2, 64, ps,
                           kv_indptr=indptr, kv_indices=np.arange(200, dtype=np.int32),
                           device=None, num_cus=4)
    # a ragged layout is for block-sparse plans only
    d = L.PlanDesc(kind=L.FI_KIND_DECODE, batch=1, num_qo_heads=8, num_kv_heads=2, head_dim=64,
                   page_size=16, num_cus=4, kv_layout=L.FI_KV_LAYOUT_RAGGED)
    h = ctypes.c_void_p()
    ip = np.array([0, 1], np.int32)
    ln = np.array([5], np.int32)
    assert fi.load().fi_plan(ctypes.byref(d), ip.ctypes.data_as(L.I32P),
                             ln.ctypes.data_as(L.I32P), None, None, None, None, None, None, 0,
                             None, 0, None, ctypes.byref(h)) == L.FI_ERR_UNSUPPORTED


@pytest.mark.parametrize("det", [False, True])
def test_tiny_decode_plan_folds_in_kernel(det):
    """A decode batch with fewer steps than workers: the default plan folds
    its split units in the kernel and (balanced) spreads each unit's steps
    over idle workers, equal to plan_ref rule 3b; merge="separate" keeps the
    plain rule and the merge launch."""
    ps = 16
    lens = [37, 300, 120, 5, 0, 64]
    indptr, L_ = _decode_host(lens, ps)
    kw = dict(deterministic=det, det_chunk_pages=4, num_cus=256)
    p = host_plan("decode", indptr, L_, 8, 2, 64, ps, **kw)
    info = p.info()
    assert info["fused_merge"]
    ref = plan_ref("decode", 8, 2, ps, indptr, L_, **level_params(info), deterministic=det,
                   det_chunk_pages=4)
    compare(info, ref)
    q = host_plan("decode", indptr, L_, 8, 2, 64, ps, merge="separate", **kw).info()
    assert not q["fused_merge"]
    compare(q, plan_ref("decode", 8, 2, ps, indptr, L_, **level_params(q), deterministic=det,
                        det_chunk_pages=4, fold_tiny=False))


def test_binding_tensor_checks_name_the_failure():
    # the binding's one-expression fast path must not let through what the
    # detailed checks refuse; on the CPU every call takes the detailed path
    import torch
    from paged_kv_attention_amd import api
    cpu = torch.device("cpu")
    t = torch.zeros(4, 3, 8, dtype=torch.bfloat16)
    api._check_tensor(t, "q", torch.bfloat16, cpu, (4, 3, 8))
    api._check_tensor(t, "q", torch.bfloat16, cpu, t.shape)
    with pytest.raises(TypeError, match="q must be torch.bfloat16"):
        api._check_tensor(t.float(), "q", torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="q has shape"):
        api._check_tensor(t, "q", torch.bfloat16, cpu, (4, 3, 9))
    with pytest.raises(ValueError, match="contiguous"):
        api._check_tensor(t.transpose(0, 1), "q", torch.bfloat16, cpu)
    with pytest.raises(TypeError, match="torch.Tensor"):
        api._check_tensor([1, 2], "q", torch.bfloat16, cpu)
    assert api._device(None) is None
    assert api._device("cpu") == cpu
    assert api._ptr(None) is None and api._ptr(t) == t.data_ptr()


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_deterministic_decode_chunks_by_kv_format(fmt):
    """Deterministic decode plans: a bf16 cache's units are cut into
    half-size chunks (at most 16 a unit), FP8 and MXFP4 ones into whole-size
    chunks; the C++ planner equals the reference rule either way."""
    rng = np.random.default_rng(51)
    lens = list(rng.integers(0, 5000, 30)) + [0, 1, 40000]
    indptr, L_ = _decode_host(lens, 16)
    p = host_plan("decode", indptr, L_, 32, 8, 128, 16, deterministic=True, det_chunk_pages=48,
                  num_cus=6, kv_format=fmt)
    info = p.info()
    ref = plan_ref("decode", 32, 8, 16, indptr, L_, **level_params(info), deterministic=True,
                   det_chunk_pages=48, det_half=fmt == "bf16")
    compare(info, ref)
    it = info["levels"][0]["items"]
    longest_unit = [x for x in it if x[10] == 32]   # the 40000-token request's chunks
    assert len(longest_unit) == 8 * (16 if fmt == "bf16" else -(-2500 // 48))
