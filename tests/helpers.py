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
# Tighter internal bars (derived from the kernel arithmetic): o within two bf16
# ulps of the oracle plus 1e-4 (P is rounded to bf16 for the P.V contraction),
# lse within 1e-5 relative (fp32 logits, fp32 sums). A dropped or doubled page
# at these lengths moves lse by ~1e-3 and fails the LSE bar by 100x.
O_ULPS = 2.0
O_FLOOR = 1e-4
LSE_TIGHT = 1e-5


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1e-30)))
    return np.where(ax > 0, np.exp2(e - 7), 2.0 ** -133)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, rows=None, what=""):
    """Assert graded and tight bars; returns the error summary."""
    og = o_gpu.float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.cpu().numpy().astype(np.float64)
    if rows is not None:
        og, lg, o_ref, lse_ref = og[rows], lg[rows], o_ref[rows], lse_ref[rows]
    assert np.all(np.isfinite(og)), f"{what}: non-finite output"
    d_o = np.abs(og - o_ref)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), empty), f"{what}: empty rows differ"
    rel = np.abs(lg[~empty] - lse_ref[~empty]) / np.maximum(1.0, np.abs(lse_ref[~empty]))
    tight_o = O_ULPS * bf16_ulp(o_ref) + O_FLOOR
    summary = dict(max_abs_o=float(d_o.max(initial=0.0)),
                   max_ulp_excess=float((d_o / tight_o).max(initial=0.0)),
                   max_rel_lse=float(rel.max(initial=0.0)))
    print(f"[{what}] {summary}", flush=True)
    assert summary["max_abs_o"] <= O_ABS_BAR, (what, summary)
    assert summary["max_rel_lse"] <= LSE_REL_BAR, (what, summary)
    assert np.all(d_o <= tight_o), (what, summary)
    assert summary["max_rel_lse"] <= LSE_TIGHT, (what, summary)
    return summary


def np_pools(w: Workload):
    return w.k_cache.float().numpy(), w.v_cache.float().numpy()


def oracle_decode(w: Workload, requests=None, k_pool=None, v_pool=None):
    if k_pool is None:
        k_pool, v_pool = np_pools(w)
    return oracle.paged_decode(w.q.double().numpy(), k_pool, v_pool, w.kv_indptr.numpy(),
                               w.kv_indices.numpy(), w.kv_len.numpy(), w.page_size, w.sm_scale,
                               requests=requests)


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
