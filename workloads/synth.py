"""Seeded synthetic paged-KV workloads.

Every tensor is drawn from a CPU ``torch.Generator`` so that the same seed gives
the same bits on any machine. Draw order is fixed: lengths, forced positions,
page permutation, q, K pool, V pool, k_new, v_new.

Layouts (the ones the library's C ABI takes):

* ``q``            bf16 ``[T, Hq, D]``   (decode and cascade: T = batch)
* ``k_cache``      bf16 ``[P, Hkv, ps, D]`` ("HND": one (page, kv head) tile is
  contiguous); ``v_cache`` the same
* ``kv_indptr``    int32 ``[B+1]``  page offsets into ``kv_indices``
* ``kv_indices``   int32 ``[nnz]``  page ids into the pool
* ``kv_len``       int32 ``[B]``    tokens per request
* ``qo_indptr``    int32 ``[B+1]``  (append) query-token offsets into ``q``
* ``k_new/v_new``  bf16 ``[sum(qo), Hkv, D]`` (append) keys/values of the new tokens
* cascade: ``prefix_indptr [G+1]``, ``prefix_indices``, ``prefix_len [G]``,
  ``req_prefix_group [B]`` (-1 = no shared prefix); ``kv_*`` then describe the
  per-request suffixes.

Token ``t`` of a sequence sits in page ``indices[indptr[r] + t // ps]`` at slot
``t % ps``. With ``poison=True`` the pages no request uses are NaN, the slots
past a request's length in its last page hold 1e4, and (append) the slots the
new tokens will occupy hold NaN until the kernel scatters them: a kernel that
reads a byte it should not shows up in the output. ``poison="nan"`` puts NaN
in the tail slots too, so that a tail V row reaching the P.V product with
p = 0 (rather than being zeroed first) turns the output into NaN.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, fields
from typing import Optional, Sequence

import torch

BASE_SEED = 1234
POOL_SLACK = 0.125        # pool holds 12.5% more pages than the batch uses
TAIL_POISON = 1.0e4       # finite poison for slots past a sequence's end
_GEN_CHUNK_PAGES = 2048   # pool pages drawn per randn call (bounds host memory)

CONFIG_NAMES = (
    "tiny_decode",            # B=4, 8/2 heads, D=64, ps=16, L~U[37,300]
    "llama3_8b_decode",       # B=64, 32/8 heads, D=128, ps=16, L~U[512,4096]
    "skewed_decode",          # B=128, lognormal(median 1024, sigma 1) + 4 x 32768
    "cascade_shared_prefix",  # 64 x (8192 shared + U[256,1024] own)
    "mixed_append",           # 16 x (U[1024,8192] prefix + U[1,128] new, causal)
)


def fp32_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) rounded to fp32, returned as the exact Python float."""
    return float(torch.tensor(1.0 / math.sqrt(head_dim), dtype=torch.float32).item())


@dataclass
class Workload:
    name: str
    kind: str                      # "decode" | "append" | "cascade" | "block_sparse"
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    sm_scale: float
    seed: int
    kv_len: torch.Tensor
    kv_indptr: torch.Tensor
    kv_indices: torch.Tensor
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    causal: bool = False
    qo_indptr: Optional[torch.Tensor] = None
    k_new: Optional[torch.Tensor] = None
    v_new: Optional[torch.Tensor] = None
    prefix_indptr: Optional[torch.Tensor] = None
    prefix_indices: Optional[torch.Tensor] = None
    prefix_len: Optional[torch.Tensor] = None
    req_prefix_group: Optional[torch.Tensor] = None
    prefix_parent: Optional[torch.Tensor] = None   # cascade tree: parent group (-1 = root)
    k_fp8: Optional[torch.Tensor] = None      # FP8 E4M3 codes, uint8, pool layout
    v_fp8: Optional[torch.Tensor] = None
    k_scale: Optional[torch.Tensor] = None    # fp32 [P, Hkv]
    v_scale: Optional[torch.Tensor] = None
    k_fp4: Optional[torch.Tensor] = None      # MXFP4 E2M1 codes, uint8 [P, Hkv, ps, D/2]
    v_fp4: Optional[torch.Tensor] = None
    k_bscale: Optional[torch.Tensor] = None   # E8M0 block scales, uint8 [P, Hkv, ps, D/32]
    v_bscale: Optional[torch.Tensor] = None
    row_block_sz: Optional[torch.Tensor] = None   # block_sparse: int32 [Hkv, MB]
    col_block_sz: Optional[torch.Tensor] = None   # int32 [Hkv, NB]
    block_mask: Optional[torch.Tensor] = None     # bool [Hkv, MB, NB]
    # block-sparse batch: per sequence its queries and [Hkv, MB_s], [Hkv, NB_s],
    # [Hkv, MB_s, NB_s] arrays (kv_len / kv_indptr / kv_indices as for decode)
    qo_lens: Optional[list] = None
    row_block_szs: Optional[list] = None
    col_block_szs: Optional[list] = None
    block_masks: Optional[list] = None
    # ragged copy of the keys and values: [tokens, Hkv, D], sequence s in rows
    # ragged_indptr[s] .. ragged_indptr[s+1]-1, followed by page_size - 1 (or
    # more) rows no sequence owns
    k_ragged: Optional[torch.Tensor] = None
    v_ragged: Optional[torch.Tensor] = None
    ragged_indptr: Optional[torch.Tensor] = None

    @property
    def batch(self) -> int:
        return int(self.kv_len.numel())

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    def to(self, device) -> "Workload":
        """Copy with every tensor moved to ``device`` (the per-sequence block
        lists stay on the host: they feed the plan)."""
        kw = {}
        for f in fields(self):
            v = getattr(self, f.name)
            if isinstance(v, torch.Tensor):
                v = v.to(device)
            kw[f.name] = v
        return Workload(**kw)

    def kv_bytes_fp8(self) -> int:
        """K+V bytes of one pass over the FP8 cache (one byte per element)."""
        return self.kv_bytes() // 2

    def kv_bytes_mxfp4(self) -> int:
        """K+V bytes of one pass over the MXFP4 cache: D/2 code bytes and
        D/32 scale bytes per token row, i.e. 17/64 of the bf16 bytes."""
        return self.kv_bytes() * 17 // 64

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one pass reads: exactly kv_len tokens per
        request per kv head (a shared prefix counted once)."""
        per_tok = self.num_kv_heads * self.head_dim * 2 * 2
        toks = int(self.kv_len.sum())
        if self.prefix_len is not None:
            toks += int(self.prefix_len.sum())
        return toks * per_tok


# --------------------------------------------------------------------------
# building blocks


def _pages_for(lengths: torch.Tensor, ps: int) -> torch.Tensor:
    return (lengths + ps - 1) // ps


def _indptr(counts: torch.Tensor) -> torch.Tensor:
    out = torch.zeros(counts.numel() + 1, dtype=torch.int64)
    out[1:] = torch.cumsum(counts.to(torch.int64), 0)
    return out.to(torch.int32)


def _randn_bf16(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def _randn_pool(gen, n_pages, hkv, ps, d) -> torch.Tensor:
    out = torch.empty((n_pages, hkv, ps, d), dtype=torch.bfloat16)
    for p0 in range(0, n_pages, _GEN_CHUNK_PAGES):
        p1 = min(n_pages, p0 + _GEN_CHUNK_PAGES)
        out[p0:p1] = _randn_bf16(gen, (p1 - p0, hkv, ps, d))
    return out


def _pool_size(used_pages: int) -> int:
    return max(1, int(math.ceil(used_pages * (1.0 + POOL_SLACK))))


def _tail_value(poison) -> float:
    """Value of the slots past a sequence's end under ``poison``: True gives
    the finite TAIL_POISON (a stray read of K or V shows up as a huge logit or
    value), ``"nan"`` gives NaN (a kernel that lets a p = 0 multiply such a V
    row, instead of zeroing it, turns the output into NaN)."""
    return float("nan") if poison == "nan" else TAIL_POISON


def _poison_pool(pool: torch.Tensor, used: torch.Tensor, tables, tail: float = TAIL_POISON) -> None:
    """NaN in unused pages; ``tail`` in slots past each sequence's end.
    ``tables`` is a list of (indices, start, length) for every sequence."""
    ps = pool.shape[2]
    mask = torch.ones(pool.shape[0], dtype=torch.bool)
    mask[used.to(torch.int64)] = False
    pool[mask] = float("nan")
    for indices, start, length in tables:
        if length % ps:
            last = int(indices[start + (length - 1) // ps])
            pool[last, :, length % ps:, :] = tail


def _lengths_uniform(gen, n, lo, hi) -> torch.Tensor:
    return torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int64)


# --------------------------------------------------------------------------
# public constructors


def make_decode(lengths: Sequence[int], num_qo_heads: int, num_kv_heads: int,
                head_dim: int, page_size: int, seed: int, poison: bool = True,
                name: str = "decode", _gen: Optional[torch.Generator] = None) -> Workload:
    """One query token per request, attending to ``lengths[r]`` cached tokens."""
    gen = _gen if _gen is not None else torch.Generator().manual_seed(seed)
    L = torch.as_tensor(list(lengths) if not isinstance(lengths, torch.Tensor) else lengths,
                        dtype=torch.int64)
    n = _pages_for(L, page_size)
    total = int(n.sum())
    pool = _pool_size(total)
    perm = torch.randperm(pool, generator=gen).to(torch.int32)
    indptr = _indptr(n)
    indices = perm[:total].clone()
    B = L.numel()
    q = _randn_bf16(gen, (B, num_qo_heads, head_dim))
    k = _randn_pool(gen, pool, num_kv_heads, page_size, head_dim)
    v = _randn_pool(gen, pool, num_kv_heads, page_size, head_dim)
    if poison:
        tabs = [(indices, int(indptr[r]), int(L[r])) for r in range(B)]
        _poison_pool(k, indices, tabs, _tail_value(poison))
        _poison_pool(v, indices, tabs, _tail_value(poison))
    return Workload(name=name, kind="decode", num_qo_heads=num_qo_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
                    sm_scale=fp32_scale(head_dim), seed=seed,
                    kv_len=L.to(torch.int32), kv_indptr=indptr, kv_indices=indices,
                    q=q, k_cache=k, v_cache=v)


def to_fp8_cache(w: Workload, poison: bool = True) -> Workload:
    """``w`` plus an FP8 copy of its K/V pools: for every (page, kv head) tile,
    scale = max |x| / 448 over the slots the batch uses (448 is the largest
    finite E4M3 value; a tile with no used slot or all zeros gets scale 1), and
    codes = torch's round-to-nearest-even E4M3 (``float8_e4m3fn``) of x / scale.
    ``w`` should be built without poison; with ``poison`` the codes of unused
    pages and of slots past each sequence's end are the NaN code 0x7F."""
    used = _used_slots(w)                            # (page, slot) holds a token

    def quant(pool):
        x = pool.float()
        m = (x.abs() * used[:, None, :, None]).amax(dim=(2, 3))
        scale = torch.where(m > 0, m / 448.0, torch.ones_like(m)).to(torch.float32)
        codes = (x / scale[:, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        if poison:
            codes = torch.where(used[:, None, :, None], codes, torch.full_like(codes, 0x7F))
        return codes.contiguous(), scale.contiguous()

    kc, ksc = quant(w.k_cache)
    vc, vsc = quant(w.v_cache)
    kw = {f.name: getattr(w, f.name) for f in fields(w)}
    kw.update(k_fp8=kc, v_fp8=vc, k_scale=ksc, v_scale=vsc, name=w.name + "_fp8")
    return Workload(**kw)


def _used_slots(w: Workload) -> torch.Tensor:
    """bool [pages, page_size]: the (page, slot) pairs that hold a token of
    some request of ``w``."""
    P, _, ps, _ = w.k_cache.shape
    used = torch.zeros(P, ps, dtype=torch.bool)
    for r in range(w.batch):
        a, L = int(w.kv_indptr[r]), int(w.kv_len[r])
        for j in range(-(-L // ps)):
            page = int(w.kv_indices[a + j])
            used[page, :min(ps, L - j * ps)] = True
    return used


# Midpoints between consecutive E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
_E2M1_CUTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def to_mxfp4_cache(w: Workload, poison: bool = True, pages_per_chunk: int = 4096) -> Workload:
    """``w`` plus an MXFP4 copy of its K/V pools. Each token row of D elements
    is cut into D/32 blocks of 32; a block with max |x| = m > 0 gets the E8M0
    scale code 127 + s with s the smallest integer such that m / 2^s <= 6 (6
    is the largest E2M1 magnitude; code 127, scale 1, for an all-zero block),
    and each element the E2M1 code of the magnitude nearest to |x| / 2^s (ties
    to the smaller one) with the sign of x in bit 3. Codes are packed two per
    byte, element 2i in the low nibble. ``w`` should be built without poison;
    with ``poison`` the scale of every unused slot is 255 (NaN) and its codes
    0xFF."""
    P, Hkv, ps, D = w.k_cache.shape
    used = _used_slots(w)
    cuts = torch.tensor(_E2M1_CUTS, dtype=torch.float32)

    def quant(pool):
        codes = torch.empty(P, Hkv, ps, D // 2, dtype=torch.uint8)
        scales = torch.empty(P, Hkv, ps, D // 32, dtype=torch.uint8)
        for p0 in range(0, P, pages_per_chunk):
            p1 = min(P, p0 + pages_per_chunk)
            x = pool[p0:p1].float().reshape(p1 - p0, Hkv, ps, D // 32, 32)
            m = x.abs().amax(dim=-1).double()
            mant, ex = torch.frexp(m / 6.0)               # m / 6 = mant * 2^ex, mant in [0.5, 1)
            s = torch.where(mant == 0.5, ex - 1, ex).to(torch.int64)
            s = torch.where(m > 0, s, torch.zeros_like(s)).clamp(-127, 127)
            mag = (x.abs() * torch.pow(2.0, -s.to(torch.float32))[..., None]).clamp(max=6.0)
            c = torch.bucketize(mag, cuts).to(torch.uint8) | ((x < 0).to(torch.uint8) << 3)
            c = c.reshape(p1 - p0, Hkv, ps, D)
            cb = c[..., 0::2] | (c[..., 1::2] << 4)
            sc = (s + 127).to(torch.uint8)
            if poison:
                u = used[p0:p1, None, :, None]
                cb = torch.where(u, cb, torch.full_like(cb, 0xFF))
                sc = torch.where(u, sc, torch.full_like(sc, 255))
            codes[p0:p1] = cb
            scales[p0:p1] = sc
        return codes, scales

    kc, ks = quant(w.k_cache)
    vc, vs = quant(w.v_cache)
    kw = {f.name: getattr(w, f.name) for f in fields(w)}
    kw.update(k_fp4=kc, v_fp4=vc, k_bscale=ks, v_bscale=vs, name=w.name + "_mxfp4")
    return Workload(**kw)


def make_append(prefix_lens: Sequence[int], qo_lens: Sequence[int], num_qo_heads: int,
                num_kv_heads: int, head_dim: int, page_size: int, seed: int,
                poison: bool = True, causal: bool = True, with_new_kv: bool = True,
                name: str = "append", _gen: Optional[torch.Generator] = None) -> Workload:
    """``qo_lens[r]`` new query tokens per request appended after ``prefix_lens[r]``
    cached tokens; kv_len = prefix + qo. With ``with_new_kv`` the new tokens' K/V
    come in ``k_new``/``v_new`` (their pool slots start as NaN under poison);
    otherwise they are already in the pool."""
    gen = _gen if _gen is not None else torch.Generator().manual_seed(seed)
    P = torch.as_tensor(list(prefix_lens), dtype=torch.int64)
    Qn = torch.as_tensor(list(qo_lens), dtype=torch.int64)
    L = P + Qn
    n = _pages_for(L, page_size)
    total = int(n.sum())
    pool = _pool_size(total)
    perm = torch.randperm(pool, generator=gen).to(torch.int32)
    indptr = _indptr(n)
    indices = perm[:total].clone()
    qo_indptr = _indptr(Qn)
    T = int(Qn.sum())
    B = L.numel()
    q = _randn_bf16(gen, (T, num_qo_heads, head_dim))
    k = _randn_pool(gen, pool, num_kv_heads, page_size, head_dim)
    v = _randn_pool(gen, pool, num_kv_heads, page_size, head_dim)
    k_new = v_new = None
    if with_new_kv:
        k_new = _randn_bf16(gen, (T, num_kv_heads, head_dim))
        v_new = _randn_bf16(gen, (T, num_kv_heads, head_dim))
    if poison:
        tabs = [(indices, int(indptr[r]), int(L[r])) for r in range(B)]
        _poison_pool(k, indices, tabs, _tail_value(poison))
        _poison_pool(v, indices, tabs, _tail_value(poison))
        if with_new_kv:
            for r in range(B):
                for t in range(int(P[r]), int(L[r])):
                    pg = int(indices[int(indptr[r]) + t // page_size])
                    k[pg, :, t % page_size, :] = float("nan")
                    v[pg, :, t % page_size, :] = float("nan")
    return Workload(name=name, kind="append", num_qo_heads=num_qo_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
                    sm_scale=fp32_scale(head_dim), seed=seed,
                    kv_len=L.to(torch.int32), kv_indptr=indptr, kv_indices=indices,
                    q=q, k_cache=k, v_cache=v, causal=causal,
                    qo_indptr=qo_indptr, k_new=k_new, v_new=v_new)


def make_cascade(prefix_lens: Sequence[int], req_group: Sequence[int],
                 suffix_lens: Sequence[int], num_qo_heads: int, num_kv_heads: int,
                 head_dim: int, page_size: int, seed: int, poison: bool = True,
                 name: str = "cascade", _gen: Optional[torch.Generator] = None,
                 prefix_parent: Optional[Sequence[int]] = None) -> Workload:
    """Decode queries over (shared prefix of group ``req_group[r]``) || (own suffix).
    Each prefix is stored once in the pool; ``req_group[r] = -1`` means no prefix.
    With ``prefix_parent`` (parent index < group index, -1 = root) the groups
    form a tree and a request's prefix is the chain root .. own group."""
    gen = _gen if _gen is not None else torch.Generator().manual_seed(seed)
    PL = torch.as_tensor(list(prefix_lens), dtype=torch.int64)
    S = torch.as_tensor(list(suffix_lens), dtype=torch.int64)
    grp = torch.as_tensor(list(req_group), dtype=torch.int64)
    npf = _pages_for(PL, page_size)
    ns = _pages_for(S, page_size)
    tot_pf, tot_s = int(npf.sum()), int(ns.sum())
    pool = _pool_size(tot_pf + tot_s)
    perm = torch.randperm(pool, generator=gen).to(torch.int32)
    prefix_indptr = _indptr(npf)
    prefix_indices = perm[:tot_pf].clone()
    indptr = _indptr(ns)
    indices = perm[tot_pf:tot_pf + tot_s].clone()
    B = S.numel()
    q = _randn_bf16(gen, (B, num_qo_heads, head_dim))
    k = _randn_pool(gen, pool, num_kv_heads, page_size, head_dim)
    v = _randn_pool(gen, pool, num_kv_heads, page_size, head_dim)
    if poison:
        used = perm[:tot_pf + tot_s]
        tabs = [(prefix_indices, int(prefix_indptr[g]), int(PL[g])) for g in range(PL.numel())]
        tabs += [(indices, int(indptr[r]), int(S[r])) for r in range(B)]
        _poison_pool(k, used, tabs, _tail_value(poison))
        _poison_pool(v, used, tabs, _tail_value(poison))
    return Workload(name=name, kind="cascade", num_qo_heads=num_qo_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
                    sm_scale=fp32_scale(head_dim), seed=seed,
                    kv_len=S.to(torch.int32), kv_indptr=indptr, kv_indices=indices,
                    q=q, k_cache=k, v_cache=v,
                    prefix_indptr=prefix_indptr, prefix_indices=prefix_indices,
                    prefix_len=PL.to(torch.int32), req_prefix_group=grp.to(torch.int32),
                    prefix_parent=None if prefix_parent is None else
                    torch.as_tensor(list(prefix_parent), dtype=torch.int32))


def cascade_flat_tables(w: Workload):
    """(kv_indptr, kv_indices, kv_len) of the flat table (prefixes of the
    request's chain, root first) || suffix per request. Only defined when every
    prefix length is a multiple of the page size, so the flat page list is the
    plain concatenation of the lists."""
    assert w.kind == "cascade"
    ps = w.page_size
    assert all(int(x) % ps == 0 for x in w.prefix_len), "prefix not page aligned"
    idx, counts, lens = [], [], []
    for r in range(w.batch):
        chain, g = [], int(w.req_prefix_group[r])
        while g >= 0:
            chain.append(g)
            g = -1 if w.prefix_parent is None else int(w.prefix_parent[g])
        a, b = int(w.kv_indptr[r]), int(w.kv_indptr[r + 1])
        pages = []
        L = int(w.kv_len[r])
        for g in reversed(chain):
            pa, pb = int(w.prefix_indptr[g]), int(w.prefix_indptr[g + 1])
            pages.append(w.prefix_indices[pa:pb])
            L += int(w.prefix_len[g])
        pages.append(w.kv_indices[a:b])
        cat = torch.cat(pages)
        idx.append(cat)
        counts.append(cat.numel())
        lens.append(L)
    return (_indptr(torch.tensor(counts)), torch.cat(idx).to(torch.int32),
            torch.tensor(lens, dtype=torch.int32))


def _block_cuts(gen, total: int, n: int, align: int) -> torch.Tensor:
    """n consecutive block sizes summing to ``total``, every non-empty block
    starting at a multiple of ``align`` (the last may end anywhere); some
    blocks may be empty."""
    units = -(-total // align)
    e = torch.sort(torch.randint(0, units + 1, (n - 1,), generator=gen)).values * align
    e = torch.clamp(e, max=total)
    edges = torch.cat([torch.zeros(1, dtype=torch.int64), e, torch.tensor([total])])
    return torch.diff(edges).to(torch.int32)


def make_block_sparse(qo_len: int, kv_len: int, num_qo_heads: int, num_kv_heads: int,
                      head_dim: int, page_size: int, num_row_blocks: int, num_col_blocks: int,
                      density: float, seed: int, poison: bool = True,
                      name: str = "block_sparse", row_block_sz=None, col_block_sz=None,
                      block_mask=None, _gen: Optional[torch.Generator] = None) -> Workload:
    """One sequence of ``qo_len`` queries over ``kv_len`` keys with a variable
    block partition and mask per kv head: random cut points (column cuts on
    page boundaries), each (row block, column block) kept with probability
    ``density``; explicit sizes or mask override the random ones. The
    sequence's pages are placed by a seeded permutation of the pool."""
    gen = _gen if _gen is not None else torch.Generator().manual_seed(seed)
    Hkv = num_kv_heads
    if row_block_sz is None:
        row_block_sz = torch.stack([_block_cuts(gen, qo_len, num_row_blocks, 1)
                                    for _ in range(Hkv)])
    if col_block_sz is None:
        col_block_sz = torch.stack([_block_cuts(gen, kv_len, num_col_blocks, page_size)
                                    for _ in range(Hkv)])
    row_block_sz = torch.as_tensor(row_block_sz, dtype=torch.int32).reshape(Hkv, -1)
    col_block_sz = torch.as_tensor(col_block_sz, dtype=torch.int32).reshape(Hkv, -1)
    MB, NB = row_block_sz.shape[1], col_block_sz.shape[1]
    if block_mask is None:
        block_mask = torch.rand((Hkv, MB, NB), generator=gen) < density
    block_mask = torch.as_tensor(block_mask, dtype=torch.bool).reshape(Hkv, MB, NB)
    n = -(-kv_len // page_size)
    pool = _pool_size(n)
    perm = torch.randperm(pool, generator=gen).to(torch.int32)
    indices = perm[:n].clone()
    q = _randn_bf16(gen, (qo_len, num_qo_heads, head_dim))
    k = _randn_pool(gen, pool, Hkv, page_size, head_dim)
    v = _randn_pool(gen, pool, Hkv, page_size, head_dim)
    if poison:
        tabs = [(indices, 0, kv_len)]
        _poison_pool(k, indices, tabs, _tail_value(poison))
        _poison_pool(v, indices, tabs, _tail_value(poison))
    return Workload(name=name, kind="block_sparse", num_qo_heads=num_qo_heads,
                    num_kv_heads=Hkv, head_dim=head_dim, page_size=page_size,
                    sm_scale=fp32_scale(head_dim), seed=seed,
                    kv_len=torch.tensor([kv_len], dtype=torch.int32),
                    kv_indptr=torch.tensor([0, n], dtype=torch.int32), kv_indices=indices,
                    q=q, k_cache=k, v_cache=v, row_block_sz=row_block_sz,
                    col_block_sz=col_block_sz, block_mask=block_mask)


def make_block_sparse_batch(seqs, num_qo_heads: int, num_kv_heads: int, head_dim: int,
                            page_size: int, seed: int, density: float = 0.5,
                            poison=True, name: str = "block_sparse_batch") -> Workload:
    """A batch of block-sparse sequences in one paged pool: ``seqs`` lists
    (queries, keys, row blocks, column blocks) per sequence; each gets its own
    random cut points (column cuts on page boundaries; empty blocks occur)
    and mask (block pairs kept with probability ``density``). Draw order:
    per sequence its cuts and mask, then the page permutation, q, K pool, V
    pool. q rows are the sequences' queries in order."""
    gen = torch.Generator().manual_seed(seed)
    Hkv = num_kv_heads
    rows, cols, masks = [], [], []
    for (T, Lk, MB, NB) in seqs:
        r = [(_block_cuts(gen, T, MB, 1) if MB else torch.zeros(0, dtype=torch.int32))
             for _ in range(Hkv)]
        c = [(_block_cuts(gen, Lk, NB, page_size) if NB else torch.zeros(0, dtype=torch.int32))
             for _ in range(Hkv)]
        rows.append(torch.stack(r).reshape(Hkv, MB).to(torch.int32))
        cols.append(torch.stack(c).reshape(Hkv, NB).to(torch.int32))
        masks.append(torch.rand((Hkv, MB, NB), generator=gen) < density)
    L = torch.tensor([s[1] for s in seqs], dtype=torch.int64)
    n = _pages_for(L, page_size)
    total = int(n.sum())
    pool = _pool_size(total)
    perm = torch.randperm(pool, generator=gen).to(torch.int32)
    indptr = _indptr(n)
    indices = perm[:total].clone()
    T = sum(s[0] for s in seqs)
    q = _randn_bf16(gen, (T, num_qo_heads, head_dim))
    k = _randn_pool(gen, pool, Hkv, page_size, head_dim)
    v = _randn_pool(gen, pool, Hkv, page_size, head_dim)
    if poison:
        tabs = [(indices, int(indptr[r]), int(L[r])) for r in range(len(seqs))]
        _poison_pool(k, indices, tabs, _tail_value(poison))
        _poison_pool(v, indices, tabs, _tail_value(poison))
    return Workload(name=name, kind="block_sparse_batch", num_qo_heads=num_qo_heads,
                    num_kv_heads=Hkv, head_dim=head_dim, page_size=page_size,
                    sm_scale=fp32_scale(head_dim), seed=seed, kv_len=L.to(torch.int32),
                    kv_indptr=indptr, kv_indices=indices, q=q, k_cache=k, v_cache=v,
                    qo_lens=[s[0] for s in seqs], row_block_szs=rows, col_block_szs=cols,
                    block_masks=masks)


def to_ragged(w: Workload, poison: bool = True) -> Workload:
    """``w`` plus a ragged copy of its keys and values: each sequence's
    kv_len tokens gathered from its pages into consecutive rows of
    ``[tokens, Hkv, D]`` tensors (token-major), sequences back to back,
    followed by page_size - 1 rows that belong to no sequence (NaN under
    ``poison``, else zero). Data movement only."""
    ps, Hkv, D = w.page_size, w.num_kv_heads, w.head_dim
    lens = [int(x) for x in w.kv_len]
    N = sum(lens) + ps - 1
    fill = float("nan") if poison else 0.0
    kr = torch.full((N, Hkv, D), fill, dtype=torch.bfloat16)
    vr = torch.full((N, Hkv, D), fill, dtype=torch.bfloat16)
    row = 0
    for r, Lr in enumerate(lens):
        a = int(w.kv_indptr[r])
        for j in range(-(-Lr // ps)):
            t0, t1 = j * ps, min(Lr, (j + 1) * ps)
            page = int(w.kv_indices[a + j])
            kr[row + t0: row + t1] = w.k_cache[page, :, : t1 - t0].transpose(0, 1)
            vr[row + t0: row + t1] = w.v_cache[page, :, : t1 - t0].transpose(0, 1)
        row += Lr
    kw = {f.name: getattr(w, f.name) for f in fields(w)}
    kw.update(k_ragged=kr, v_ragged=vr, ragged_indptr=_indptr(torch.tensor(lens)),
              name=w.name + "_ragged")
    return Workload(**kw)


SPARSE_VIDEO_NAME = "sparse_video_attention"


def make_sparse_video(poison: bool = False, seed: Optional[int] = None) -> Workload:
    """Block-sparse self-attention shaped like a video diffusion transformer's
    sparse attention: 8192 tokens (queries = keys), 16 q / 16 kv heads (MHA),
    D 128, page 16; per head the tokens are cut into 64 blocks of variable size
    (multiples of 16 averaging 128) and a block pair is kept on the diagonal
    band |a - b| <= 1 and with probability 0.15 elsewhere."""
    seed = BASE_SEED + 200 if seed is None else seed
    gen = torch.Generator().manual_seed(seed)
    H, T, nb = 16, 8192, 64
    sizes = []
    for _ in range(H):
        w = torch.randint(4, 13, (nb,), generator=gen).to(torch.float64)   # 64..192 tokens
        edges = torch.round(torch.cumsum(w, 0) / w.sum() * (T // 16)).to(torch.int64)
        edges = torch.cat([torch.zeros(1, dtype=torch.int64), edges])
        sizes.append((torch.diff(edges) * 16).to(torch.int32))
    sz = torch.stack(sizes)
    a = torch.arange(nb)
    band = (a[:, None] - a[None, :]).abs() <= 1
    mask = band[None] | (torch.rand((H, nb, nb), generator=gen) < 0.15)
    return make_block_sparse(T, T, H, H, 128, 16, nb, nb, 0.0, seed, poison,
                             SPARSE_VIDEO_NAME, row_block_sz=sz, col_block_sz=sz,
                             block_mask=mask, _gen=gen)


POD_MIX_NAME = "pod_mixed"


def make_pod_mix(poison: bool = False, seed: Optional[int] = None, n_decode: int = 64,
                 n_prefill: int = 2, prefill_q: int = 512) -> Workload:
    """One step of a chunked-prefill serving batch: ``n_decode`` requests
    decoding one token over kv U[512, 4096] (the Llama-3-8B-like decode
    shape) beside ``n_prefill`` prefill chunks of ``prefill_q`` query tokens
    over cached prefixes U[1024, 4096]; 32 q / 8 kv heads, D 128, page 16,
    causal, new K/V scattered. Decode and prefill requests are interleaved."""
    seed = BASE_SEED + 100 if seed is None else seed
    gen = torch.Generator().manual_seed(seed)
    dec = _lengths_uniform(gen, n_decode, 512, 4096) - 1
    pre = _lengths_uniform(gen, n_prefill, 1024, 4096)
    prefix = torch.cat([dec, pre])
    qo = torch.cat([torch.ones(n_decode, dtype=torch.int64),
                    torch.full((n_prefill,), prefill_q, dtype=torch.int64)])
    order = torch.randperm(prefix.numel(), generator=gen)
    return make_append(prefix[order].tolist(), qo[order].tolist(), 32, 8, 128, 16, seed, poison,
                       True, True, POD_MIX_NAME, _gen=gen)


def make_config(k: int, poison: bool = False, seed: Optional[int] = None) -> Workload:
    """The five benchmark configurations, by 0-based index (see CONFIG_NAMES)."""
    seed = BASE_SEED + k if seed is None else seed
    gen = torch.Generator().manual_seed(seed)
    name = CONFIG_NAMES[k]
    if k == 0:
        L = _lengths_uniform(gen, 4, 37, 300)
        return make_decode(L, 8, 2, 64, 16, seed, poison, name, _gen=gen)
    if k == 1:
        L = _lengths_uniform(gen, 64, 512, 4096)
        return make_decode(L, 32, 8, 128, 16, seed, poison, name, _gen=gen)
    if k == 2:
        z = torch.randn(128, generator=gen, dtype=torch.float64)
        L = torch.round(torch.exp(math.log(1024.0) + 1.0 * z)).clamp(1, 32768).to(torch.int64)
        forced = torch.randperm(128, generator=gen)[:4]
        L[forced] = 32768
        return make_decode(L, 32, 8, 128, 16, seed, poison, name, _gen=gen)
    if k == 3:
        S = _lengths_uniform(gen, 64, 256, 1024)
        return make_cascade([8192], [0] * 64, S, 32, 8, 128, 16, seed, poison, name, _gen=gen)
    if k == 4:
        P = _lengths_uniform(gen, 16, 1024, 8192)
        Qn = _lengths_uniform(gen, 16, 1, 128)
        return make_append(P, Qn, 32, 8, 128, 16, seed, poison, True, True, name, _gen=gen)
    raise ValueError(f"no config {k}")
