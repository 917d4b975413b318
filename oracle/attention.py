"""Exact attention over a paged KV cache, in float64, written from definitions.

TEST INFRASTRUCTURE: see the package docstring for who may import this.

What is computed (Ye et al. record, *boundary*: the engine's result is plain
exact attention; backend-selection note, *Arithmetic intensity*: the paged
layout changes where K/V are read from, not the FLOPs):

    for query row q (one query token, one q head h, kv head g = h // (Hq/Hkv)):
        s_t  = sm_scale * <q, K[t]>              over the visible keys t
        lse  = ln sum_t exp(s_t)                 (natural log)
        o    = sum_t exp(s_t - lse) * V[t]
    no visible key:  o = 0, lse = -inf

Readings where the pages are silent (each also listed in the design notes):
* q head h reads kv head h // (Hq/Hkv) (contiguous groups);
* token t of a sequence is in page ``indices[start + t // ps]``, slot ``t % ps``;
* append: the i-th of qo new queries sits at absolute position L - qo + i and
  sees keys 0..L-qo+i (bottom-right causal alignment);
* the LSE is reported in natural log;
* merging states (o_j, lse_j) is the log-sum-exp identity, folded left in
  index order; merging with (x, -inf) is the identity.

Inputs are NumPy arrays; pools may be float32 (bf16 values are exact in fp32)
and every gathered row is upcast to float64 before any arithmetic.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _heads_of(kv_head: int, group: int) -> slice:
    return slice(kv_head * group, (kv_head + 1) * group)


def gather_tokens(pool, indices, start: int, length: int, page_size: int,
                  kv_head: int) -> np.ndarray:
    """Tokens 0..length-1 of one sequence for one kv head, in token order.

    Block-table gather (backend-selection note, *Arithmetic intensity*; Ye et
    al. record, *summary*: block-sparse KV storage). ``pool`` is
    ``[num_pages, Hkv, page_size, D]``. Pinned by: brute force against a dense
    cache scattered into random pages, pool-permutation and page-size
    invariance, needle keys placed across page boundaries.
    """
    d = pool.shape[-1]
    if length <= 0:
        return np.zeros((0, d), dtype=np.float64)
    n_pages = (length + page_size - 1) // page_size
    pages = np.asarray(indices[start:start + n_pages], dtype=np.int64)
    assert pages.size == n_pages, "block table shorter than the sequence"
    tiles = np.asarray(pool[pages, kv_head], dtype=np.float64)   # [n, ps, D]
    return tiles.reshape(n_pages * page_size, d)[:length]


def attend(q, k, v, sm_scale: float, visible=None):
    """Exact softmax attention of query rows ``q [n, D]`` over ``k, v [L, D]``.

    Returns ``(o [n, D], lse [n])``. ``visible`` is an optional ``[n, L]``
    boolean mask. Rows that see no key get ``o = 0, lse = -inf``. Pinned by:
    torch's scaled_dot_product_attention in float64 (o), closed forms for L=1,
    equal logits, two tokens and a needle (o and lse), constant V.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape[0], v.shape[1] if v.ndim == 2 else q.shape[1]
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.full(n, NEG_INF, dtype=np.float64)
    if k.shape[0] == 0 or n == 0:
        return o, lse
    s = float(sm_scale) * (q @ k.T)
    if visible is not None:
        s = np.where(visible, s, NEG_INF)
    m = s.max(axis=1)
    live = m > NEG_INF
    if not live.any():
        return o, lse
    w = np.exp(s[live] - m[live, None])
    z = w.sum(axis=1)
    lse[live] = m[live] + np.log(z)
    o[live] = (w @ v) / z[:, None]
    return o, lse


def _req_list(batch, requests):
    return range(batch) if requests is None else [int(r) for r in requests]


def paged_decode(q, k_pool, v_pool, kv_indptr, kv_indices, kv_len, page_size: int,
                 sm_scale: float, requests=None):
    """Decode attention: one query token per request over its paged KV.

    ``q [B, Hq, D]``; returns ``o [B, Hq, D]``, ``lse [B, Hq]`` (rows of
    requests not in ``requests`` are NaN). Pinned by: dense brute force via
    torch SDPA, invariants (pool permutation, page size, split + merge),
    needle and poison tests.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    o = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    for r in _req_list(B, requests):
        a, L = int(kv_indptr[r]), int(kv_len[r])
        for g in range(Hkv):
            K = gather_tokens(k_pool, kv_indices, a, L, page_size, g)
            V = gather_tokens(v_pool, kv_indices, a, L, page_size, g)
            hs = _heads_of(g, G)
            o[r, hs], lse[r, hs] = attend(q[r, hs], K, V, sm_scale)
    return o, lse


def e4m3_values():
    """Value of every FP8 E4M3 code (index = code), float64, NaN for the two
    NaN codes. The format is the OCP 8-bit floating-point E4M3 definition:
    sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
    subnormal, m/8 * 2^-6; exponent 15 with mantissa 7 is NaN; there are no
    infinities (largest finite 448). Pinned by: all 256 codes against torch's
    float8_e4m3fn conversion; closed forms (1, 448, 2^-9, 2^-6, signs)."""
    out = np.empty(256)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 0x7
        if e == 15 and m == 7:
            out[c] = np.nan
        elif e == 0:
            out[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            out[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def paged_decode_fp8(q, k_codes, v_codes, k_scale, v_scale, kv_indptr, kv_indices, kv_len,
                     page_size: int, sm_scale: float, requests=None):
    """Decode attention over an FP8 cache (v0.7.4 article, TL;DR: decoding from
    a low-precision KV cache): the element of page p, kv head g is
    e4m3_values()[code] * scale[p, g] in fp64, and the result is exactly
    paged_decode over those values. Only the pages of the selected requests
    are decoded. Pinned by: equality with paged_decode over pools dequantized
    by torch's float8_e4m3fn conversion (an independent route)."""
    B = q.shape[0]
    reqs = _req_list(B, requests)
    pages = np.unique(np.concatenate(
        [np.asarray(kv_indices[int(kv_indptr[r]):int(kv_indptr[r + 1])]) for r in reqs]
        + [np.zeros(0, dtype=np.int64)]).astype(np.int64))
    table = e4m3_values()
    ks = np.asarray(k_scale, dtype=np.float64)[pages][:, :, None, None]
    vs = np.asarray(v_scale, dtype=np.float64)[pages][:, :, None, None]
    kp = table[np.asarray(k_codes)[pages]] * ks
    vp = table[np.asarray(v_codes)[pages]] * vs
    remap = np.zeros(int(np.asarray(k_codes).shape[0]), dtype=np.int64)
    remap[pages] = np.arange(pages.size)
    idx = remap[np.asarray(kv_indices, dtype=np.int64)]
    return paged_decode(q, kp, vp, kv_indptr, idx, kv_len, page_size, sm_scale, requests=reqs)


def e2m1_values():
    """Value of every FP4 E2M1 code (index = code 0..15), float64. The format
    is the OCP microscaling FP4 element: sign bit (bit 3), 2 exponent bits
    (bias 1), 1 mantissa bit; exponent field 0 is subnormal, m/2; no
    infinities or NaN (largest 6). Pinned by: the closed-form table
    {0, 0.5, 1, 1.5, 2, 3, 4, 6} and its negatives."""
    out = np.empty(16)
    for c in range(16):
        sign = -1.0 if c & 0x8 else 1.0
        e, m = (c >> 1) & 0x3, c & 0x1
        out[c] = sign * (m / 2.0 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return out


def e8m0_values():
    """Value of every E8M0 scale code (index = code 0..255): 2^(code - 127),
    NaN for 255 (OCP microscaling shared scale). Pinned by closed forms."""
    out = 2.0 ** (np.arange(256, dtype=np.float64) - 127.0)
    out[255] = np.nan
    return out


def mxfp4_dequantize(codes, scales):
    """Elements of MXFP4 rows: ``codes [..., D/2]`` uint8 (element 2i in the
    low nibble of byte i, 2i+1 in the high nibble), ``scales [..., D/32]``
    uint8 E8M0, one per 32 consecutive elements; returns ``[..., D]`` float64,
    value = e2m1(code) * 2^(scale - 127). Pinned by: bytes built from known
    elements, the nibble order, and a NaN scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo, hi = codes & 0xF, codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    vals = e2m1_values()[nib]
    sc = e8m0_values()[np.asarray(scales, dtype=np.uint8)]
    return vals * np.repeat(sc, 32, axis=-1)


def paged_decode_mxfp4(q, k_codes, v_codes, k_scales, v_scales, kv_indptr, kv_indices, kv_len,
                       page_size: int, sm_scale: float, requests=None):
    """Decode attention over an MXFP4 cache (v0.7.4 article, TL;DR: decoding
    from a 4-bit KV cache): K and V elements are mxfp4_dequantize of the
    pools' codes and scales in fp64, and the result is exactly paged_decode
    over those values. Only the pages of the selected requests are decoded.
    Pinned by: equality with paged_decode over pools dequantized by an
    independent route (integer bit fields of each code), and the element
    layout pins of mxfp4_dequantize."""
    B = q.shape[0]
    reqs = _req_list(B, requests)
    pages = np.unique(np.concatenate(
        [np.asarray(kv_indices[int(kv_indptr[r]):int(kv_indptr[r + 1])]) for r in reqs]
        + [np.zeros(0, dtype=np.int64)]).astype(np.int64))
    kp = mxfp4_dequantize(np.asarray(k_codes)[pages], np.asarray(k_scales)[pages])
    vp = mxfp4_dequantize(np.asarray(v_codes)[pages], np.asarray(v_scales)[pages])
    remap = np.zeros(int(np.asarray(k_codes).shape[0]), dtype=np.int64)
    remap[pages] = np.arange(pages.size)
    idx = remap[np.asarray(kv_indices, dtype=np.int64)]
    return paged_decode(q, kp, vp, kv_indptr, idx, kv_len, page_size, sm_scale, requests=reqs)


def paged_append(q, qo_indptr, k_pool, v_pool, kv_indptr, kv_indices, kv_len,
                 page_size: int, sm_scale: float, causal: bool = True, requests=None):
    """Attention for ``qo`` new query tokens per request over ``kv_len`` keys
    (which already include the new tokens). Causal: query i (0-based among the
    request's qo queries) sees keys ``t <= kv_len - qo + i``.

    ``q [T, Hq, D]`` with request r's queries at rows ``qo_indptr[r]..``.
    Returns ``o [T, Hq, D]``, ``lse [T, Hq]``. Pinned by: torch SDPA with an
    explicit bottom-right mask, append with qo=1 == decode, a needle key
    placed just past a query's horizon.
    """
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    o = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    for r in _req_list(len(kv_len), requests):
        q0, q1 = int(qo_indptr[r]), int(qo_indptr[r + 1])
        nq, L, a = q1 - q0, int(kv_len[r]), int(kv_indptr[r])
        if nq == 0:
            continue
        for g in range(Hkv):
            K = gather_tokens(k_pool, kv_indices, a, L, page_size, g)
            V = gather_tokens(v_pool, kv_indices, a, L, page_size, g)
            hs = _heads_of(g, G)
            rows = np.asarray(q[q0:q1, hs], dtype=np.float64).reshape(nq * G, D)
            vis = None
            if causal:
                qpos = (L - nq) + np.repeat(np.arange(nq), G)        # row -> position
                vis = np.arange(L)[None, :] <= qpos[:, None]
            ob, lb = attend(rows, K, V, sm_scale, vis)
            o[q0:q1, hs] = ob.reshape(nq, G, D)
            lse[q0:q1, hs] = lb.reshape(nq, G)
    return o, lse


def gather_ragged(kv, start: int, length: int, kv_head: int) -> np.ndarray:
    """Tokens ``start .. start+length-1`` of a ragged ``[tokens, Hkv, D]`` K or
    V tensor for one kv head, in token order (research note, *Arithmetic
    intensity*: ragged KV-cache layouts, one contiguous run of tokens per
    sequence). Pinned by: a ragged tensor scattered into a paged pool gathers
    to the same keys, and brute force over explicit key lists."""
    d = kv.shape[-1]
    if length <= 0:
        return np.zeros((0, d), dtype=np.float64)
    return np.asarray(kv[start:start + length, kv_head], dtype=np.float64)


def _block_sparse_seq(q, keys_of, kv_len: int, row_sz, col_sz, mask, sm_scale: float, sel,
                      o, lse):
    """Block-sparse attention of one sequence: ``q [T, Hq, D]`` its queries,
    ``keys_of(g)`` its (K, V) for kv head g, ``sel`` the query indices to
    compute; writes ``o``/``lse`` rows ``sel`` (the definition in
    ``block_sparse``)."""
    T, Hq, D = q.shape
    Hkv = len(row_sz)
    G = Hq // Hkv
    for g in range(Hkv):
        K, V = keys_of(g)
        rs = np.asarray(row_sz[g], dtype=np.int64)
        cs = np.asarray(col_sz[g], dtype=np.int64)
        assert rs.sum() == T and cs.sum() == kv_len, "blocks must cover the sequence"
        row_block = np.repeat(np.arange(rs.size), rs)          # query -> its row block
        col_block = np.repeat(np.arange(cs.size), cs)          # key -> its column block
        m = np.asarray(mask[g], dtype=bool)
        vis_tok = m[row_block[sel][:, None], col_block[None, :]]    # [rows, kv_len]
        hs = _heads_of(g, G)
        qr = np.asarray(q[sel][:, hs], dtype=np.float64).reshape(sel.size * G, D)
        ob, lb = attend(qr, K, V, sm_scale, np.repeat(vis_tok, G, axis=0))
        o[sel, hs] = ob.reshape(sel.size, G, D)
        lse[sel, hs] = lb.reshape(sel.size, G)


def block_sparse(q, k_pool, v_pool, seq_pages, kv_len: int, page_size: int, row_sz, col_sz,
                 mask, sm_scale: float, rows=None):
    """Variable block-sparse attention of one sequence (research note,
    *Arithmetic intensity*: block-sparse and variable block-sparse plans; Ye
    et al. record, *summary*: composable block-sparse KV representations).

    For kv head g the ``qo_len`` queries are cut into consecutive row blocks
    of sizes ``row_sz[g]`` and the ``kv_len`` keys into consecutive column
    blocks of sizes ``col_sz[g]``; query i sees key t iff ``mask[g][a][b]``
    for the row block a holding i and the column block b holding t. Each q
    head h uses the partition and mask of its kv head h // (Hq/Hkv). No causal
    mask; a row that sees no key gets o = 0, lse = -inf. ``q [qo_len, Hq, D]``;
    keys are gathered through ``seq_pages``. Returns ``o [qo_len, Hq, D]``,
    ``lse [qo_len, Hq]``; with ``rows`` (query indices) only those rows are
    computed and the others are NaN. Pinned by: brute force over explicit
    per-row key lists on tiny inputs, the all-ones mask equal to unmasked
    attention, a block-diagonal mask equal to independent attention per
    block (torch SDPA), and rows with no selected block.
    """
    T, Hq, D = q.shape
    sel = np.arange(T) if rows is None else np.asarray(sorted(rows), dtype=np.int64)
    o = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)

    def keys_of(g):
        return (gather_tokens(k_pool, seq_pages, 0, kv_len, page_size, g),
                gather_tokens(v_pool, seq_pages, 0, kv_len, page_size, g))
    _block_sparse_seq(q, keys_of, kv_len, row_sz, col_sz, mask, sm_scale, sel, o, lse)
    return o, lse


def block_sparse_batch(q, k, v, qo_len, kv_len, row_sz, col_sz, mask, sm_scale: float,
                       kv_indptr, kv_indices=None, page_size: int = 0, rows=None):
    """Block-sparse attention over a batch of sequences, each with its own
    partitions and mask (``row_sz[s]``, ``col_sz[s]``, ``mask[s]`` as in
    ``block_sparse``); sequence s's queries are q rows ``sum(qo_len[:s])``
    onward and see only its own keys. Keys, paged (``kv_indices`` given):
    token t of sequence s in page ``kv_indices[kv_indptr[s] + t // page_size]``
    of pools ``k, v [P, Hkv, ps, D]``; ragged (``kv_indices`` None): rows
    ``kv_indptr[s] + t`` of ``k, v [tokens, Hkv, D]``. Returns
    ``o [T, Hq, D]``, ``lse [T, Hq]`` (``rows``: only those global query rows,
    others NaN). Pinned by: brute force over explicit per-row key lists on a
    tiny ragged batch, equality with ``block_sparse`` per sequence, and
    ragged equal to paged for the same keys.
    """
    T, Hq, D = q.shape
    o = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    want = None if rows is None else set(int(r) for r in rows)
    q0 = 0
    for s in range(len(qo_len)):
        nq, L, base = int(qo_len[s]), int(kv_len[s]), int(kv_indptr[s])
        sel = np.array([i for i in range(nq) if want is None or q0 + i in want], dtype=np.int64)
        if sel.size:
            if kv_indices is None:
                def keys_of(g):
                    return gather_ragged(k, base, L, g), gather_ragged(v, base, L, g)
            else:
                def keys_of(g):
                    return (gather_tokens(k, kv_indices, base, L, page_size, g),
                            gather_tokens(v, kv_indices, base, L, page_size, g))
            os_ = np.full((nq, Hq, D), np.nan)
            ls_ = np.full((nq, Hq), np.nan)
            _block_sparse_seq(q[q0:q0 + nq], keys_of, L, row_sz[s], col_sz[s], mask[s],
                              sm_scale, sel, os_, ls_)
            o[q0 + sel] = os_[sel]
            lse[q0 + sel] = ls_[sel]
        q0 += nq
    return o, lse


def scatter_new_kv(k_pool, v_pool, k_new, v_new, qo_indptr, kv_indptr, kv_indices,
                   kv_len, page_size: int):
    """Copies of the pools with the new tokens' K/V written into their slots.

    New token i of request r (of qo) is sequence position ``kv_len - qo + i``.
    Every other pool element is unchanged. Pinned by: direct element checks in
    the tests (written slots equal the inputs, all other bytes untouched).
    """
    k_out, v_out = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    for r in range(len(kv_len)):
        q0, q1 = int(qo_indptr[r]), int(qo_indptr[r + 1])
        L, a = int(kv_len[r]), int(kv_indptr[r])
        for i in range(q1 - q0):
            pos = L - (q1 - q0) + i
            page = int(kv_indices[a + pos // page_size])
            k_out[page, :, pos % page_size, :] = k_new[q0 + i]
            v_out[page, :, pos % page_size, :] = v_new[q0 + i]
    return k_out, v_out


def merge_two(o1, l1, o2, l2):
    """Combine two attention states over disjoint key sets.

    With M = max(l1, l2):  lse = M + ln(e^(l1-M) + e^(l2-M)),
    o = (e^(l1-M) o1 + e^(l2-M) o2) / (e^(l1-M) + e^(l2-M)).  Two empty states
    give (0, -inf). Works elementwise over leading dims (``o`` has a trailing D).
    Pinned by: split-and-merge equals attention over the union (any partition),
    commutativity, associativity, identity element.
    """
    o1 = np.asarray(o1, dtype=np.float64)
    o2 = np.asarray(o2, dtype=np.float64)
    l1 = np.asarray(l1, dtype=np.float64)
    l2 = np.asarray(l2, dtype=np.float64)
    M = np.maximum(l1, l2)
    empty = M == NEG_INF
    Ms = np.where(empty, 0.0, M)
    w1 = np.where(l1 == NEG_INF, 0.0, np.exp(l1 - Ms))
    w2 = np.where(l2 == NEG_INF, 0.0, np.exp(l2 - Ms))
    z = w1 + w2
    zs = np.where(empty, 1.0, z)
    lse = np.where(empty, NEG_INF, Ms + np.log(zs))
    o = (w1[..., None] * o1 + w2[..., None] * o2) / zs[..., None]
    o = np.where(empty[..., None], 0.0, o)
    return o, lse


def merge_states(v, s):
    """Fixed-order fold of ``S`` states per row: ``v [N, S, H, D]``,
    ``s [N, S, H]`` -> ``([N, H, D], [N, H])``, combining index 0 first
    (PR #4038, *What it does*: fp32 partials reduced in a fixed order).
    """
    v = np.asarray(v, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    N, S, H, D = v.shape
    if S == 0:
        return np.zeros((N, H, D)), np.full((N, H), NEG_INF)
    o, l = v[:, 0], s[:, 0]
    for j in range(1, S):
        o, l = merge_two(o, l, v[:, j], s[:, j])
    return o, l


def _chain(req_group, prefix_parent, r):
    """Request r's prefix groups, root first (own group last)."""
    out, h = [], int(req_group[r])
    while h >= 0:
        out.append(h)
        h = -1 if prefix_parent is None else int(prefix_parent[h])
    return out[::-1]


def _cascade_kv(k_pool, v_pool, prefix_indptr, prefix_indices, prefix_len, req_group,
                kv_indptr, kv_indices, kv_len, page_size, r, g, prefix_parent=None):
    parts_k, parts_v = [], []
    for grp in _chain(req_group, prefix_parent, r):
        a, L = int(prefix_indptr[grp]), int(prefix_len[grp])
        parts_k.append(gather_tokens(k_pool, prefix_indices, a, L, page_size, g))
        parts_v.append(gather_tokens(v_pool, prefix_indices, a, L, page_size, g))
    a, L = int(kv_indptr[r]), int(kv_len[r])
    suf_k = gather_tokens(k_pool, kv_indices, a, L, page_size, g)
    suf_v = gather_tokens(v_pool, kv_indices, a, L, page_size, g)
    return parts_k, parts_v, suf_k, suf_v


def cascade_flat(q, k_pool, v_pool, prefix_indptr, prefix_indices, prefix_len, req_group,
                 kv_indptr, kv_indices, kv_len, page_size: int, sm_scale: float,
                 requests=None, prefix_parent=None):
    """The definition of the cascade result: decode attention of each request
    over the concatenation (its groups' shared prefixes, root first) || (its own
    suffix) (backend-selection note, *Arithmetic intensity*: a shared prefix is
    read once and reused across requests; the result is the same attention).
    ``prefix_parent[g]`` (optional) is the group whose prefix precedes g's, so
    the groups form a tree. Pinned by: equality with the level-by-level form,
    and with plain decode over a flat table.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    o = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    for r in _req_list(B, requests):
        for g in range(Hkv):
            pk, pv, sk, sv = _cascade_kv(k_pool, v_pool, prefix_indptr, prefix_indices,
                                         prefix_len, req_group, kv_indptr, kv_indices,
                                         kv_len, page_size, r, g, prefix_parent)
            K = np.concatenate(pk + [sk]) if pk else sk
            V = np.concatenate(pv + [sv]) if pv else sv
            hs = _heads_of(g, G)
            o[r, hs], lse[r, hs] = attend(q[r, hs], K, V, sm_scale)
    return o, lse


def cascade_two_level(q, k_pool, v_pool, prefix_indptr, prefix_indices, prefix_len,
                      req_group, kv_indptr, kv_indices, kv_len, page_size: int,
                      sm_scale: float, requests=None, prefix_parent=None):
    """Level-by-level form: one attention state per prefix of the request's
    chain and one for its suffix, folded root first with ``merge_two``. Must
    equal ``cascade_flat``."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    o = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    for r in _req_list(B, requests):
        for g in range(Hkv):
            pk, pv, sk, sv = _cascade_kv(k_pool, v_pool, prefix_indptr, prefix_indices,
                                         prefix_len, req_group, kv_indptr, kv_indices,
                                         kv_len, page_size, r, g, prefix_parent)
            hs = _heads_of(g, G)
            oc, lc = np.zeros((G, D)), np.full(G, NEG_INF)
            for kk, vv in zip(pk, pv):
                op, lp = attend(q[r, hs], kk, vv, sm_scale)
                oc, lc = merge_two(oc, lc, op, lp)
            os_, ls = attend(q[r, hs], sk, sv, sm_scale)
            o[r, hs], lse[r, hs] = merge_two(oc, lc, os_, ls)
    return o, lse
