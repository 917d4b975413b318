"""Reference statement of the work plan (load-balanced split of KV ranges).

TEST INFRASTRUCTURE: see the package docstring for who may import this.

The pages say the engine splits long KV ranges into load-balanced chunks with a
schedule that stays valid under static graph capture (Ye et al. record,
*summary*), and that split partials are kept in fp32 and reduced in a fixed
order (PR #4038, *What it does*). They give no algorithm, so the rule below is
a reading, restated here in plain Python so that the library's C++ planner can
be compared with it element for element:

1. Work units. Each request's query rows (query token i, head h of kv head g:
   row = i*G + h) are cut into blocks of ``rows_per_block`` rows. A unit is
   (request, block, kv head), enumerated in that nesting order. For the
   cascade prefix level a unit is (group, block, kv head) over the rows of the
   group's member requests (ascending request index); with a tree of prefixes
   (``prefix_parent``, parent index < group index) a group's members are the
   requests whose chain of groups (own group, its parent, ...) passes through
   it, and each request's prefix parts are merged in group index order, root
   first.
2. Key range. A unit sees tokens [0, t_lim): t_lim = kv_len, or under the
   causal mask min(kv_len, kv_len - qo + i_last + 1) with i_last the last
   query token in the block. It spans n = ceil(t_lim / ps) pages.
3. Balanced mode (even split). The kernels walk a unit in 32-token steps,
   so the split is counted in steps: a unit of n pages is s = ceil(n / gp)
   steps, gp = max(1, 32 / ps) pages each. The units' steps are laid end to
   end in enumeration order (W steps in all) and cut into consecutive quotas
   of c = max(1, ceil(min_chunk_pages / gp), ceil(W / S)) steps, S = number of
   persistent workers; quota w goes to worker w. A unit's pieces, in order,
   are its chunks (page ranges: step boundaries times gp, the last clipped to
   n), so each worker runs c steps (the last one fewer) in page order, and no
   chunk boundary falls inside a step. The reported chunk size is c*gp pages.
   Exception for small batches: if there are no more units than workers and
   the longest unit has fewer than NO_SPLIT_STEPS = 12 steps more than c,
   every unit stays whole on worker = its enumeration index (splitting would
   save fewer steps than the merge it needs costs); the reported chunk size
   is then the longest unit's steps times gp.
3b. Tiny decode batches (no more steps W than workers S, on the matrix
   cores, merge mode left to the library, not graph-stable): the split units
   are folded inside the attention kernel, so there is no merge launch to
   amortise: c = max(1, ceil(W / S)) steps and no whole-unit exception, so a
   unit's steps run on several waves side by side. (``fold_tiny=False``
   gives the plans that do not take this rule.)
3c. Tiny batches with at most S/4 units (S a multiple of 4): unit u runs on
   the four waves of workgroup u, workers 4u..4u+3, so that the kernel folds
   it after a workgroup barrier: with ns = ceil(n / gp) steps and
   k = ceil(ns / 4), chunk j covers steps [j k, min(ns, (j+1) k)) (empty
   ones dropped) on worker 4u + j; the reported chunk size is
   max(1, ceil(longest / 4)) * gp pages.
4. Deterministic mode. A unit of n pages has k chunks, chunk j covering
   pages [floor(j*n/k), floor((j+1)*n/k)): k = ceil(n / c) on a wide level
   (128-row units), k = min(ceil(n / max(1, c // 2)), DET_MAX_CHUNKS = 16)
   on a decode-style one (16-row units) of a bf16 cache (``det_half``; FP8
   and MXFP4 decode plans take ceil(n / c) too), c = det_chunk_pages;
   boundaries depend on the request alone. Chunks are
   placed longest-processing-time-first (Graham): sorted by (cost
   descending, enumeration index), cost = pages + 1, each given to the
   worker with the smallest load, ties to the lowest worker index; a worker
   runs its chunks in the order it received them.
5. Outputs. A unit with one chunk writes its final rows directly; otherwise
   each chunk writes fp32 partial rows (allocated in enumeration order) that a
   merge folds in chunk order. Merge records are ``(q_base, row0, n_rows,
   kv_head, parts_off, n_parts)``: rows row0 .. row0+n_rows-1 of a unit (row
   rho is query q_base + rho // G, head kv_head*G + rho % G), a unit's rows cut
   into records of MERGE_ROWS = 16; part j of record row k is partial row
   parts[parts_off + j] + k. Cascade writes partials for everything and
   merges, per (request, kv head), the prefix chunk(s) first, then the suffix
   chunks.
6. Fused mixed batch (append, research note *Arithmetic intensity*: POD
   attention runs a batch's prefill and decode rows in one kernel). A request
   whose query rows (qo * G) fit one 16-row block belongs to the decode role
   (level 1, 16-row units), every other request to the wide role (level 0,
   128-row units). The launch has P workgroups; with W_w and W_d the two
   roles' steps (as in 3), the wide role gets n_w = P if there are no decode
   steps, 0 if there are no wide steps, else the override if one is given
   (capped at P - 1), else the n in [1, P - 1] that minimises, in order,
   max(T_w, T_d), then T_w, then n. With c_w = max(m_w, ceil(W_w / n)) and
   c_d = max(m_d, ceil(W_d / (4 (P - n)))) the two roles' quotas under rule 3
   (m: a role's minimum chunk in steps), T_d = 9 c_d and T_w = 4 (c_w + 4 k),
   k the most items any wide quota holds (1 + the unit ends strictly inside
   it): a decode wavefront step takes about 9/4 of a wide workgroup step when
   the two roles share the chip and the KV comes from HBM, and a wide item
   costs about four steps to start and end. Deterministic plans (rule 4
   chunks): with N_r a role's chunk count and L_r its longest chunk in steps,
   T_w = 4 ceil(N_w / n) (L_w + 4) and T_d = 9 max(L_d, ceil(W_d / (4 (P -
   n)))). Each role is planned as in
   3-4 over its own workers (n_w workgroups; 4 (P - n_w) wavefronts), then
   its worker list is padded with empty workers to P (wide) and 4P (decode).
   Partial rows are allocated wide role first; merges likewise. A cascade
   plan may be fused the same way: its prefix level is the wide role and its
   suffix level the decode role, split by the same rule.
7. Variable block-sparse (research note *Arithmetic intensity*: block-sparse
   and variable block-sparse plans over paged and ragged layouts). For
   sequence s, kv head g and row block a (rows = a's query tokens times G),
   the page list is the pages of a's selected non-empty column blocks in
   column order (a block of c keys starting at key c0 covers pages c0/ps ..
   ceil((c0+c)/ps)-1 of the sequence), appended to ``plist``; a paged
   sequence lists its page ids, a ragged one (keys in rows kv_indptr[s] + t
   of one [tokens][Hkv][D] tensor) the first token kv_indptr[s] + pg*ps of
   each page-sized run. t_lim = the selected keys. Units are enumerated s, g,
   a, row block (128 rows; in a POD plan a row block of at most 16 rows is one
   decode-role unit), with q_base = a's first query row in the batch and
   page_off = the list's offset; no causal mask. Levels, merges (a unit with
   no keys gets empty records: o = 0, lse = -inf) as in 3-6.
"""

from __future__ import annotations

import heapq

NO_SPLIT_STEPS = 12  # balanced mode keeps units whole if splitting saves fewer steps
DET_MAX_CHUNKS = 16  # deterministic chunks of a decode-style unit at most
POD_WIDE_STEP = 4        # fused launch: time of a wide workgroup step ...
POD_DECODE_STEP = 9      # ... and of a decode wavefront step
POD_WIDE_ITEM_STEPS = 4  # starting and ending a wide item, in wide steps
POD_DECODE_ROWS = 16  # query rows of a request that runs in the decode role
MERGE_ROWS = 16       # unit rows per merge record at most
FLAG_LIST_Q = 1     # query rows come from the member list (cascade prefix)
FLAG_PARTIAL = 2    # write fp32 partial rows instead of final rows
FLAG_CAUSAL = 4     # bottom-right causal mask
FLAG_PREFIX = 8     # page list is the shared-prefix table

ITEM_FIELDS = ("q_base", "row0", "n_rows", "kv_head", "page_off", "flags",
               "t_begin", "t_end", "q_pos0", "dst", "unit", "chunk")


def _ceil_div(a, b):
    return -(-a // b)


def _lpt(items, num_workers):
    order = sorted(range(len(items)),
                   key=lambda i: (-(items[i]["t_pages"] + 1), i))
    heap = [(0, w) for w in range(num_workers)]
    per_worker = [[] for _ in range(num_workers)]
    for i in order:
        load, w = heapq.heappop(heap)
        per_worker[w].append(i)
        heapq.heappush(heap, (load + items[i]["t_pages"] + 1, w))
    flat, indptr = [], [0]
    for w in range(num_workers):
        flat.extend(per_worker[w])
        indptr.append(len(flat))
    return flat, indptr


def _det_chunks(n, c, decode_style):
    """Rule 4: the number of deterministic chunks of a unit of n pages."""
    if n <= 0:
        return 0
    c = max(1, int(c))
    if not decode_style:
        return _ceil_div(n, c)
    return min(_ceil_div(n, max(1, c // 2)), DET_MAX_CHUNKS)


def _unit_pieces(units, num_workers, deterministic, det_chunk_pages, min_chunk_pages,
                 page_size, tiny=False, wg=False, decode_style=False):
    """Per unit: list of (p0, p1, worker) page pieces in order; and c in pages.
    ``tiny`` (rule 3b): quotas of max(1, ceil(W / S)) steps and no whole-unit
    exception; ``wg`` (rule 3c): unit u on workers 4u..4u+3."""
    pieces = []
    if deterministic:
        c = max(1, int(det_chunk_pages))
        if decode_style:
            c = max(1, c // 2)
        for u in units:
            n = u["n_pages"]
            k = _det_chunks(n, det_chunk_pages, decode_style)
            pieces.append([((j * n) // k, ((j + 1) * n) // k, None) for j in range(k)])
        return pieces, c
    # balanced: quotas counted in 32-token steps (gp pages each), so that no
    # chunk boundary falls inside a step
    gp = max(1, 32 // page_size)
    steps = [_ceil_div(u["n_pages"], gp) for u in units]
    W = sum(steps)
    c = max(1, _ceil_div(W, num_workers)) if tiny else \
        max(1, _ceil_div(int(min_chunk_pages), gp), _ceil_div(W, num_workers))
    longest = max(steps, default=0)
    if wg:
        out = []
        for ui, (u, ns) in enumerate(zip(units, steps)):
            n, k = u["n_pages"], _ceil_div(ns, 4)
            out.append([(j * k * gp, min(n, min(ns, (j + 1) * k) * gp), 4 * ui + j)
                        for j in range(4) if j * k < min(ns, (j + 1) * k)])
        return out, max(1, _ceil_div(longest, 4)) * gp
    if not tiny and len(units) <= num_workers and longest - c < NO_SPLIT_STEPS:
        # small batch: splitting would save fewer steps than a merge costs
        return [[(0, u["n_pages"], i)] if u["n_pages"] > 0 else []
                for i, u in enumerate(units)], max(1, longest) * gp
    g = 0
    for u, ns in zip(units, steps):
        n = u["n_pages"]
        lst = []
        p = 0
        while p < ns:
            w = (g + p) // c
            e = min(ns, (w + 1) * c - g)
            lst.append((p * gp, min(n, e * gp), w))
            p = e
        pieces.append(lst)
        g += ns
    return pieces, c * gp


def plan_ref(kind, num_qo_heads, num_kv_heads, page_size, kv_indptr, kv_len,
             num_workers, rows_per_block, deterministic=False, det_chunk_pages=48,
             min_chunk_pages=1, qo_indptr=None, causal=False, prefix_indptr=None,
             prefix_len=None, req_group=None, prefix_parent=None, pod_blocks=None,
             pod_wide_blocks=0, block_sparse=None, block_sparse_batch=None, fold_tiny=True,
             det_half=True):
    """Return the plan as plain lists.

    ``kind`` is "decode", "append" or "cascade". ``rows_per_block`` is a list
    with one entry per level (cascade: [prefix, suffix]; otherwise one);
    ``num_workers`` and ``min_chunk_pages`` are a number (all levels) or such a
    list.
    Result: ``{"levels": [{"items": [...12-tuples...], "worker_indptr": [...]}],
    "merges": [(q_tok, head0, n_heads, parts_off, n_parts)], "parts": [...],
    "qlist": [...], "n_part_rows": int}``.
    ``pod_blocks`` (append, cascade, block_sparse): plan one fused launch of
    that many workgroups (rule 6; ``rows_per_block`` and ``min_chunk_pages``
    then name the wide and the decode role); the result also holds
    ``pod_wide_blocks``. ``kind="block_sparse"`` takes ``block_sparse =
    (qo_len, row_sz [Hkv][MB], col_sz [Hkv][NB], mask [Hkv][MB][NB],
    seq_pages)`` (rule 7; ``kv_indptr`` and ``kv_len`` are then unused) and
    the result also holds ``plist``; or ``block_sparse_batch = (qo_lens,
    row_szs, col_szs, masks, kv_indptr, kv_indices)`` for a batch of
    sequences (per-sequence lists; ``kv_indices`` None for a ragged layout,
    ``kv_indptr`` then in tokens).
    """
    nlev = len(rows_per_block)
    workers = list(num_workers) if isinstance(num_workers, (list, tuple)) else [num_workers] * nlev
    min_chunk = (list(min_chunk_pages) if isinstance(min_chunk_pages, (list, tuple))
                 else [min_chunk_pages] * nlev)
    B = len(kv_len)
    G = num_qo_heads // num_kv_heads
    ps = page_size
    kv_len = [int(x) for x in kv_len]
    kv_indptr = [int(x) for x in kv_indptr]

    def request_units(rpb, qo_of, qtok_of, is_causal, take=lambda r: True):
        units = []
        for r in range(B):
            if not take(r):
                continue
            nq, L = qo_of(r), kv_len[r]
            rows = nq * G
            for b in range(_ceil_div(rows, rpb)):
                r0, r1 = b * rpb, min(rows, (b + 1) * rpb)
                i_last = (r1 - 1) // G
                t_lim = min(L, L - nq + i_last + 1) if is_causal else L
                for g in range(num_kv_heads):
                    units.append(dict(unit=r, q_base=qtok_of(r), row0=r0, n_rows=r1 - r0,
                                      g=g, page_off=kv_indptr[r], t_lim=t_lim,
                                      n_pages=_ceil_div(t_lim, ps),
                                      q_pos0=(L - nq) if is_causal else 0,
                                      flags=FLAG_CAUSAL if is_causal else 0, nq=nq))
        return units

    qlist = []
    page_list = []      # block_sparse: the units' page lists
    levels_units = []
    if kind == "cascade":
        NG = len(prefix_len)
        pu = []
        rpb = rows_per_block[0]
        def chain(r):           # request r's groups, own first, then parents
            out, h = [], int(req_group[r])
            while h >= 0:
                out.append(h)
                h = -1 if prefix_parent is None else int(prefix_parent[h])
            return out
        chains = [chain(r) for r in range(B)]
        for grp in range(NG):
            members = [r for r in range(B) if grp in chains[r]]
            PL = int(prefix_len[grp])
            if not members or PL == 0:
                continue
            off = len(qlist)
            qlist.extend(members)
            rows = len(members) * G
            for b in range(_ceil_div(rows, rpb)):
                r0, r1 = b * rpb, min(rows, (b + 1) * rpb)
                for g in range(num_kv_heads):
                    pu.append(dict(unit=grp, q_base=off, row0=r0, n_rows=r1 - r0, g=g,
                                   page_off=int(prefix_indptr[grp]), t_lim=PL,
                                   n_pages=_ceil_div(PL, ps), q_pos0=0,
                                   flags=FLAG_LIST_Q | FLAG_PREFIX, nq=None))
        levels_units.append(pu)
        levels_units.append(request_units(rows_per_block[1], lambda r: 1, lambda r: r, False))
    elif kind == "append":
        qo = [int(qo_indptr[r + 1]) - int(qo_indptr[r]) for r in range(B)]
        if pod_blocks is None:
            levels_units.append(request_units(rows_per_block[0], lambda r: qo[r],
                                              lambda r: int(qo_indptr[r]), bool(causal)))
        else:
            small = [qo[r] * G <= POD_DECODE_ROWS for r in range(B)]
            for lev, role in ((0, False), (1, True)):
                levels_units.append(request_units(
                    rows_per_block[lev], lambda r: qo[r], lambda r: int(qo_indptr[r]),
                    bool(causal), take=lambda r, role=role: small[r] == role))
    elif kind == "block_sparse":
        if block_sparse is not None:      # one paged sequence
            qo_len, row_sz, col_sz, mask, seq_pages = block_sparse
            n = _ceil_div(sum(int(x) for x in col_sz[0]), ps) if len(col_sz) else 0
            seqs = ([qo_len], [row_sz], [col_sz], [mask], [0, n], list(seq_pages))
        else:
            seqs = block_sparse_batch
        qo_lens, rows_s, cols_s, masks_s, kvp, kvi = seqs
        wide, small = [], []
        q_seq, unit_id = 0, 0
        for sq in range(len(qo_lens)):
            row_sz, col_sz, mask = rows_s[sq], cols_s[sq], masks_s[sq]
            base = int(kvp[sq])
            for g in range(num_kv_heads):
                q0 = q_seq
                for a, nq in enumerate(int(x) for x in row_sz[g]):
                    off, t_lim, c0 = len(page_list), 0, 0
                    for b, c in enumerate(int(x) for x in col_sz[g]):
                        if c > 0 and mask[g][a][b]:
                            # paged: the pool's page ids; ragged (kvi None):
                            # the first token of each ps-token run
                            page_list.extend(
                                (base + pg * ps) if kvi is None else int(kvi[base + pg])
                                for pg in range(c0 // ps, _ceil_div(c0 + c, ps)))
                            t_lim += c
                        c0 += c
                    rows = nq * G
                    to_small = pod_blocks is not None and rows <= POD_DECODE_ROWS
                    rpb = rows_per_block[1] if to_small else rows_per_block[0]
                    for blk in range(_ceil_div(rows, rpb)):
                        (small if to_small else wide).append(dict(
                            unit=unit_id, q_base=q0, row0=blk * rpb,
                            n_rows=min(rows - blk * rpb, rpb), g=g, page_off=off, t_lim=t_lim,
                            n_pages=_ceil_div(t_lim, ps), q_pos0=0, flags=0, nq=nq))
                    q0 += nq
                    unit_id += 1
            q_seq += int(qo_lens[sq])
        levels_units.append(wide)
        if pod_blocks is not None:
            levels_units.append(small)
    else:
        levels_units.append(request_units(rows_per_block[0], lambda r: 1, lambda r: r, False))

    if pod_blocks is not None and kind != "decode":
        # rule 6: split the launch's P workgroups between the two roles
        P = int(pod_blocks)
        gp = max(1, 32 // ps)
        w_steps = [sum(_ceil_div(u["n_pages"], gp) for u in lu) for lu in levels_units]
        if w_steps[1] == 0:
            n_w = P
        elif w_steps[0] == 0:
            n_w = 0
        elif pod_wide_blocks > 0:
            n_w = min(int(pod_wide_blocks), P - 1)
        else:
            cmin = [max(1, _ceil_div(int(m), gp)) for m in min_chunk]
            ends, acc = [], 0
            for u in levels_units[0]:
                ns = _ceil_div(u["n_pages"], gp)
                if ns > 0:
                    acc += ns
                    ends.append(acc)

            def busiest(c):
                # items of the quota holding most unit ends strictly inside it
                inside = [e // c for e in ends[:-1] if e % c]
                return 1 + max((inside.count(q) for q in set(inside)), default=0)

            # deterministic chunks (rule 4): per role the chunk count and the
            # longest chunk in steps
            nch, longest = [0, 0], [0, 0]
            for lev_i, lu in enumerate(levels_units):
                for u in lu:
                    if u["n_pages"] > 0:
                        k = _det_chunks(u["n_pages"], det_chunk_pages, lev_i == 1)
                        nch[lev_i] += k
                        longest[lev_i] = max(longest[lev_i],
                                             _ceil_div(_ceil_div(u["n_pages"], k), gp))

            def cost(n):
                if deterministic:
                    tw = POD_WIDE_STEP * _ceil_div(nch[0], n) * (longest[0] + POD_WIDE_ITEM_STEPS)
                    td = POD_DECODE_STEP * max(longest[1], _ceil_div(w_steps[1], 4 * (P - n)))
                    return (max(tw, td), tw, n)
                cw = max(cmin[0], _ceil_div(w_steps[0], n))
                tw = POD_WIDE_STEP * (cw + POD_WIDE_ITEM_STEPS * busiest(cw))
                td = POD_DECODE_STEP * max(cmin[1], _ceil_div(w_steps[1], 4 * (P - n)))
                return (max(tw, td), tw, n)
            n_w = min(range(1, P), key=cost)
        workers = [n_w, 4 * (P - n_w)]

    all_partial = kind == "cascade"
    next_row = 0
    levels = []
    unit_chunks = []    # per level: per unit (k, [partial dst rows])
    for lev, units in enumerate(levels_units):
        S = workers[lev]
        if S == 0:      # a fused role with no workgroups (and no steps)
            assert all(u["n_pages"] == 0 for u in units)
            levels.append(dict(items=[], worker_indptr=[0], chunk_pages=0))
            unit_chunks.append([(0, [])] * len(units))
            continue
        gp = max(1, 32 // ps)
        tiny = (fold_tiny and kind == "decode" and not deterministic
                and sum(_ceil_div(u["n_pages"], gp) for u in units) <= S)
        wg = tiny and S % 4 == 0 and 4 * len(units) <= S
        pieces, c = _unit_pieces(units, S, deterministic, det_chunk_pages, min_chunk[lev],
                                 page_size, tiny, wg,
                                 decode_style=det_half and rows_per_block[lev] == 16)
        items = []
        chunks_of = []
        for u, lst in zip(units, pieces):
            k = len(lst)
            partial = all_partial or k > 1
            dsts = []
            for j, (p0, p1, w) in enumerate(lst):
                dst = -1
                if partial:
                    dst = next_row
                    next_row += u["n_rows"]
                    dsts.append(dst)
                items.append(dict(
                    q_base=u["q_base"], row0=u["row0"], n_rows=u["n_rows"], kv_head=u["g"],
                    page_off=u["page_off"], flags=u["flags"] | (FLAG_PARTIAL if partial else 0),
                    t_begin=p0 * ps, t_end=min(p1 * ps, u["t_lim"]), q_pos0=u["q_pos0"],
                    dst=dst, unit=u["unit"], chunk=j, t_pages=p1 - p0, worker=w))
            chunks_of.append((k, dsts))
        if deterministic:
            order, indptr = _lpt(items, S)
        else:
            per = [[] for _ in range(S)]
            for i, it in enumerate(items):
                per[it["worker"]].append(i)
            order, indptr = [], [0]
            for w in range(S):
                order.extend(per[w])
                indptr.append(len(order))
        levels.append(dict(items=[tuple(items[i][f] for f in ITEM_FIELDS) for i in order],
                           worker_indptr=indptr, chunk_pages=c))
        unit_chunks.append(chunks_of)

    merges, parts = [], []
    if kind == "cascade":
        pu, su = levels_units
        pchunks, schunks = unit_chunks
        # prefix partial row of (request r, kv head g): find r's unit and local row
        pref = {}
        for ui, u in enumerate(pu):
            k, dsts = pchunks[ui]
            members = qlist[u["q_base"]:]
            for local in range(0, u["n_rows"], G):
                r = members[(u["row0"] + local) // G]
                # groups come in index order (parents first): root prefix first
                pref.setdefault((r, u["g"]), []).extend(d + local for d in dsts)
        for ui, u in enumerate(su):
            r, g = u["unit"], u["g"]
            k, dsts = schunks[ui]
            plist = pref.get((r, g), []) + list(dsts)
            merges.append((r, 0, G, g, len(parts), len(plist)))
            parts.extend(plist)
    else:
        for units, chunks_of in zip(levels_units, unit_chunks):
            for ui, u in enumerate(units):
                k, dsts = chunks_of[ui]
                if k == 1:
                    continue
                for k0 in range(0, u["n_rows"], MERGE_ROWS):
                    merges.append((u["q_base"], u["row0"] + k0,
                                   min(MERGE_ROWS, u["n_rows"] - k0), u["g"], len(parts), k))
                    parts.extend(d + k0 for d in dsts)
    out = dict(levels=levels, merges=merges, parts=parts, qlist=qlist, n_part_rows=next_row,
               plist=page_list)
    if kind != "decode" and pod_blocks is not None:
        P = int(pod_blocks)
        for lev, total in ((0, P), (1, 4 * P)):
            ind = levels[lev]["worker_indptr"]
            ind.extend([ind[-1]] * (total + 1 - len(ind)))
        out["pod_wide_blocks"] = workers[0]
    return out
