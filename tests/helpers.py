"""Shared helpers for the parity tests: run a workload through the HIP library
and through the oracle, and compare them with the stated tolerances."""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import paged_kv_attention_amd as fi
from workloads import Workload

# Bars the method is held to (bf16 outputs, fp32 LSE):
O_ABS_BAR = 1e-2          # max |o_gpu - o_oracle|
LSE_REL_BAR = 1e-3        # |lse_gpu - lse_oracle| / max(1, |lse_oracle|)
# Tighter internal bars, derived from the kernel arithmetic:
# * o: the P.V contraction takes P rounded to bf16 (unit roundoff u = 2^-8) and
#   the output is rounded to bf16 once, so |o_gpu - o| <= u * (A + |o|) up to
#   fp32 accumulation noise, where A = sum_t p_t |v_t| / sum_t p_t is the
#   oracle's attention over |V| (``a_ref``);
# * lse: fp32 logits and sums give ~1e-7 relative; the bar is 1e-5. A dropped
#   or doubled page at these lengths moves lse by ~1e-3 and fails it by 100x.
U_BF16 = 2.0 ** -8
LSE_TIGHT = 1e-5


def compare(o_gpu, lse_gpu, o_ref, lse_ref, a_ref=None, rows=None, what=""):
    """Assert the graded bars, and the derived tight bars when ``a_ref`` (the
    oracle's attention over |V|) is given; returns the error summary."""
    og = o_gpu.float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.cpu().numpy().astype(np.float64)
    if rows is not None:
        og, lg, o_ref, lse_ref = og[rows], lg[rows], o_ref[rows], lse_ref[rows]
        if a_ref is not None:
            a_ref = a_ref[rows]
    assert np.all(np.isfinite(og)), f"{what}: non-finite output"
    d_o = np.abs(og - o_ref)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), empty), f"{what}: empty rows differ"
    rel = np.abs(lg[~empty] - lse_ref[~empty]) / np.maximum(1.0, np.abs(lse_ref[~empty]))
    summary = dict(max_abs_o=float(d_o.max(initial=0.0)),
                   max_rel_lse=float(rel.max(initial=0.0)))
    if a_ref is not None:
        tight_o = U_BF16 * (np.abs(a_ref) + np.abs(o_ref)) * (1 + 1e-3) + 1e-6
        summary["max_bound_frac"] = float((d_o / tight_o).max(initial=0.0))
    print(f"[{what}] {summary}", flush=True)
    assert summary["max_abs_o"] <= O_ABS_BAR, (what, summary)
    assert summary["max_rel_lse"] <= LSE_REL_BAR, (what, summary)
    if a_ref is not None:
        assert summary["max_bound_frac"] <= 1.0, (what, summary)
    assert summary["max_rel_lse"] <= LSE_TIGHT, (what, summary)
    return summary


def np_pools(w: Workload):
    return w.k_cache.float().numpy(), w.v_cache.float().numpy()


def oracle_decode(w: Workload, requests=None, k_pool=None, v_pool=None):
    """(o, lse, a): the oracle's decode and its attention over |V|."""
    if k_pool is None:
        k_pool, v_pool = np_pools(w)
    args = (w.kv_indptr.numpy(), w.kv_indices.numpy(), w.kv_len.numpy(), w.page_size, w.sm_scale)
    q = w.q.double().numpy()
    o, lse = oracle.paged_decode(q, k_pool, v_pool, *args, requests=requests)
    a, _ = oracle.paged_decode(q, k_pool, np.abs(v_pool), *args, requests=requests)
    return o, lse, a


def gpu_decode(w: Workload, dev, **plan_kw):
    p = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                w.page_size, device=dev, **plan_kw)
    g = w.to(dev) if w.q.device != dev else w
    o, lse = fi.paged_decode(p, g.q, g.k_cache, g.v_cache, g.kv_indices, w.sm_scale)
    torch.cuda.synchronize()
    return o, lse, p


def request_rows(requests):
    return np.asarray(sorted(requests), dtype=np.int64)


def sample_requests(B, n, rng, must=()):
    pick = set(int(x) for x in must)
    pick.update(int(x) for x in rng.choice(B, size=min(n, B), replace=False))
    return sorted(pick)
