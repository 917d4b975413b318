"""Python binding over the C ABI: argument marshalling only.

Every step of the computation runs in libfi.so's HIP kernels; this module
checks tensor shapes/dtypes, passes raw pointers and the current torch stream,
and turns error codes into exceptions. PyTorch supplies device memory and
streams.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import _lib as L

_KINDS = {"decode": L.FI_KIND_DECODE, "append": L.FI_KIND_APPEND, "cascade": L.FI_KIND_CASCADE}
_ENGINES = {"default": L.FI_ENGINE_DEFAULT, "mfma": L.FI_ENGINE_MFMA, "valu": L.FI_ENGINE_VALU}
_LAUNCHES = {"default": L.FI_LAUNCH_DEFAULT, "pod": L.FI_LAUNCH_POD,
             "separate": L.FI_LAUNCH_SEPARATE}
_KV_FORMATS = {"bf16": L.FI_KV_BF16, "fp8": L.FI_KV_FP8, "mxfp4": L.FI_KV_MXFP4}
_MERGES = {"default": L.FI_MERGE_DEFAULT, "fused": L.FI_MERGE_FUSED,
           "separate": L.FI_MERGE_SEPARATE}


def _host_i32(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(L.I32P)


def _ptr(t: Optional[torch.Tensor]):
    # the entry points declare these arguments c_void_p, so ctypes converts
    # the integer address (and None) itself
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    """The raw handle of the current torch stream on ``device`` (a CUDA
    torch.device with an index)."""
    return torch._C._cuda_getCurrentRawStream(device.index)


def _device(device) -> Optional[torch.device]:
    """torch.device with the index filled in (``"cuda"`` is the current
    device), so that tensors compare equal to it."""
    if device is None:
        return None
    d = torch.device(device)
    if d.type == "cuda" and d.index is None:
        d = torch.device("cuda", torch.cuda.current_device())
    return d


class Workspace:
    """Caller-owned plan storage: a device buffer and a pinned host staging
    buffer. Reusing one workspace across plans keeps device addresses fixed."""

    def __init__(self, dev_bytes: int, host_bytes: int, device="cuda"):
        self.dev = torch.empty(max(int(dev_bytes), 256), dtype=torch.uint8, device=device)
        self.host = torch.empty(max(int(host_bytes), 256), dtype=torch.uint8, pin_memory=True)

    @staticmethod
    def bound(desc: L.PlanDesc, max_kv_pages: int, max_qo_tokens: int = 0,
              max_prefix_pages: int = 0):
        dev, host = ctypes.c_size_t(), ctypes.c_size_t()
        L.check(L.load().fi_workspace_size(ctypes.byref(desc), int(max_kv_pages),
                                           int(max_qo_tokens), int(max_prefix_pages),
                                           ctypes.byref(dev), ctypes.byref(host)),
                "fi_workspace_size")
        return dev.value, host.value


def _prefix_depth(parent, ng: int) -> int:
    """Longest chain of nested prefix groups (1 without parents). Invalid
    parents are left for fi_plan to report."""
    if parent is None or ng == 0:
        return 1
    depth = [1] * ng
    for g in range(ng):
        p = int(parent[g])
        if 0 <= p < g:
            depth[g] = depth[p] + 1
    return max(depth)


class Plan:
    """A work plan for one batch (fi_plan). ``device=None`` builds it on the
    host only (needs ``num_cus``), which the run calls refuse. ``kv_format``
    ("bf16", "fp8" or "mxfp4") names the cache a decode plan will be run on:
    it only picks the default ``workers_per_cu`` (8 for "fp8", 12 for "mxfp4",
    else 4). ``merge``
    ("default", "fused" or "separate") says where a decode plan's split units
    are merged: by a merge launch after the attention kernel (the default and
    "separate") or inside the decode kernels ("fused", matrix-core engine;
    same bits, measured slower on MI355X). ``capacity =
    (batch, kv_pages, qo_tokens, prefix_pages[, prefix_depth])`` makes it
    graph-stable: laid out for at most those sizes (and nested prefixes at
    most ``prefix_depth`` deep, default 1), so that a run call captured in a
    HIP graph serves every later plan of the same kind and shape built into
    the same ``workspace``."""

    def __init__(self, kind: str, kv_indptr, kv_len, num_qo_heads: int, num_kv_heads: int,
                 head_dim: int, page_size: int, *, qo_indptr=None, causal: bool = False,
                 prefix_indptr=None, prefix_len=None, req_prefix_group=None, prefix_parent=None,
                 deterministic: bool = False, det_chunk_pages: int = 0, min_chunk_pages: int = 0,
                 num_cus: int = 0, workers_per_cu: int = 0, engine: str = "default",
                 launch: str = "default", pod_wide_blocks: int = 0, kv_format: str = "bf16",
                 merge: str = "default", device="cuda", workspace: Optional[Workspace] = None,
                 capacity=None):
        lib = L.load()
        self.kind = kind
        self._ha = dict(kv_indptr=_host_i32(kv_indptr), kv_len=_host_i32(kv_len),
                        qo_indptr=_host_i32(qo_indptr), prefix_indptr=_host_i32(prefix_indptr),
                        prefix_len=_host_i32(prefix_len),
                        req_prefix_group=_host_i32(req_prefix_group),
                        prefix_parent=_host_i32(prefix_parent))
        B = int(self._ha["kv_len"].size)
        ng = 0 if prefix_len is None else int(self._ha["prefix_len"].size)
        self.desc = L.PlanDesc(kind=_KINDS[kind], batch=B, num_qo_heads=num_qo_heads,
                               num_kv_heads=num_kv_heads, head_dim=head_dim,
                               page_size=page_size, causal=int(causal),
                               deterministic=int(deterministic),
                               det_chunk_pages=det_chunk_pages, min_chunk_pages=min_chunk_pages,
                               num_cus=num_cus, workers_per_cu=workers_per_cu,
                               num_prefix_groups=ng, decode_engine=_ENGINES[engine],
                               max_prefix_depth=_prefix_depth(self._ha["prefix_parent"], ng),
                               launch=_LAUNCHES[launch], pod_wide_blocks=pod_wide_blocks,
                               kv_format=_KV_FORMATS[kv_format], merge_mode=_MERGES[merge])
        if capacity is not None:
            cap = [int(x) for x in capacity] + [1] * (5 - len(capacity))
            (self.desc.cap_batch, self.desc.cap_kv_pages, self.desc.cap_qo_tokens,
             self.desc.cap_prefix_pages, self.desc.max_prefix_depth) = cap
        self.num_qo_heads, self.num_kv_heads = num_qo_heads, num_kv_heads
        self.head_dim, self.page_size, self.batch = head_dim, page_size, B
        self.device = _device(device)
        self.workspace = workspace
        ws_dev = ws_host = None
        dev_b = host_b = 0
        if self.device is not None:
            if self.workspace is None:
                n_q = 0 if qo_indptr is None else int(self._ha["qo_indptr"][-1])
                n_p = 0 if prefix_indptr is None else int(self._ha["prefix_indptr"][-1])
                n_kv = int(self._ha["kv_indptr"][-1]) if B else 0
                # (a graph-stable description sizes itself from its capacity)
                db, hb = Workspace.bound(self.desc, n_kv, n_q, n_p)
                self.workspace = Workspace(db, hb, self.device)
            ws_dev, ws_host = _ptr(self.workspace.dev), _ptr(self.workspace.host)
            dev_b, host_b = self.workspace.dev.numel(), self.workspace.host.numel()
            stream = _stream(self.device)
        else:
            stream = None
        h = ctypes.c_void_p()
        a = self._ha
        L.check(lib.fi_plan(ctypes.byref(self.desc), _p(a["kv_indptr"]), _p(a["kv_len"]),
                            _p(a["qo_indptr"]), _p(a["prefix_indptr"]), _p(a["prefix_len"]),
                            _p(a["req_prefix_group"]), _p(a["prefix_parent"]), ws_dev, dev_b,
                            ws_host, host_b, stream,
                            ctypes.byref(h)), "fi_plan")
        self._h = h
        self.num_q_tokens = B if qo_indptr is None else int(self._ha["qo_indptr"][-1])

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                L.load().fi_plan_destroy(h)
            except Exception:
                pass
            self._h = None

    def info(self) -> dict:
        """Copies of the plan's host arrays (items, worker lists, merges...)."""
        inf = L.PlanInfo()
        L.check(L.load().fi_plan_get_info(self._h, ctypes.byref(inf)), "fi_plan_get_info")

        def arr(ptr, n):
            if n == 0:
                return np.zeros(0, dtype=np.int32)
            return np.ctypeslib.as_array(ptr, shape=(n,)).copy()

        levels = []
        for l in range(inf.num_levels):
            levels.append(dict(
                rows_per_block=inf.rows_per_block[l], chunk_pages=inf.chunk_pages[l],
                num_workers=inf.num_workers[l], min_chunk_pages=inf.min_chunk_pages[l],
                items=arr(inf.items[l], inf.num_items[l] * L.FI_ITEM_INTS).reshape(-1, L.FI_ITEM_INTS),
                worker_indptr=arr(inf.worker_indptr[l], inf.num_workers[l] + 1)))
        return dict(kind=inf.kind, levels=levels,
                    merges=arr(inf.merges, inf.num_merges * L.FI_MERGE_INTS).reshape(-1, L.FI_MERGE_INTS),
                    parts=arr(inf.parts, inf.num_parts), qlist=arr(inf.qlist, inf.num_qlist),
                    num_part_rows=inf.num_part_rows, num_scatter=inf.num_scatter,
                    dev_bytes_used=inf.dev_bytes_used, host_bytes_used=inf.host_bytes_used,
                    pod_wide_blocks=inf.pod_wide_blocks, plist=arr(inf.plist, inf.num_plist),
                    fused_merge=bool(inf.fused_merge),
                    item_rec=arr(inf.item_rec, inf.num_items[0] if inf.fused_merge else 0),
                    empty_recs=arr(inf.empty_recs, inf.num_empty_recs),
                    wg_fold=bool(inf.wg_fold))


class BlockSparsePlan(Plan):
    """A variable block-sparse plan over a batch of sequences
    (fi_plan_block_sparse_batch). Sequence s has ``qo_len[s]`` queries (q
    rows in sequence order) and ``kv_len[s]`` keys; ``row_block_sz[s]``
    ``[Hkv, MB_s]`` and ``col_block_sz[s]`` ``[Hkv, NB_s]`` cut them per kv
    head and ``block_mask[s]`` ``[Hkv, MB_s, NB_s]`` selects the block pairs.
    ``layout="paged"``: keys through ``kv_indptr`` (pages) and ``kv_indices``
    into pools ``[P, Hkv, ps, D]``; ``layout="ragged"``: sequence s is rows
    ``kv_indptr[s] ..`` of K/V tensors ``[tokens, Hkv, D]`` (``kv_indices``
    unused), ``page_size`` the granule of the key walk. A single sequence may
    be given without the lists: ``qo_len``/``kv_len`` ints, the size and mask
    arrays of that sequence, and ``seq_pages`` (paged) for its page ids."""

    def __init__(self, qo_len, kv_len, row_block_sz, col_block_sz, block_mask,
                 seq_pages=None, num_qo_heads: int = 0, num_kv_heads: int = 0,
                 head_dim: int = 0, page_size: int = 0, *, kv_indptr=None, kv_indices=None,
                 layout: str = "paged", deterministic: bool = False, det_chunk_pages: int = 0,
                 min_chunk_pages: int = 0, num_cus: int = 0, workers_per_cu: int = 0,
                 launch: str = "default", pod_wide_blocks: int = 0, device="cuda",
                 workspace: Optional[Workspace] = None):
        lib = L.load()
        self.kind = "block_sparse"
        Hkv, ps = num_kv_heads, page_size
        single = np.ndim(qo_len) == 0
        if single:
            qo_len, kv_len = [int(qo_len)], [int(kv_len)]
            row_block_sz, col_block_sz, block_mask = [row_block_sz], [col_block_sz], [block_mask]
            if layout == "paged":
                n = -(-int(kv_len[0]) // ps)
                kv_indptr = [0, n]
                kv_indices = seq_pages if seq_pages is not None else np.zeros(0, np.int32)
        S = len(qo_len)
        rows, cols, masks, nrb, ncb = [], [], [], [], []
        for s in range(S):
            r = _host_i32(row_block_sz[s]).reshape(Hkv, -1)
            c = _host_i32(col_block_sz[s]).reshape(Hkv, -1)
            m = block_mask[s]
            m = m.detach().cpu().numpy() if isinstance(m, torch.Tensor) else np.asarray(m)
            m = m.astype(np.uint8).reshape(Hkv, r.shape[1], c.shape[1])
            rows.append(r.ravel()), cols.append(c.ravel()), masks.append(m.ravel())
            nrb.append(r.shape[1]), ncb.append(c.shape[1])
        cat = lambda xs, dt: np.ascontiguousarray(np.concatenate(xs).astype(dt)) if xs \
            else np.zeros(0, dt)  # noqa: E731
        self._ha = dict(qo_len=_host_i32(qo_len), kv_len=_host_i32(kv_len),
                        nrb=_host_i32(nrb), ncb=_host_i32(ncb), row=cat(rows, np.int32),
                        col=cat(cols, np.int32), mask=cat(masks, np.uint8),
                        kv_indptr=_host_i32(kv_indptr),
                        kv_indices=_host_i32(kv_indices) if layout == "paged" else None)
        if self._ha["kv_indptr"] is None:
            raise ValueError("kv_indptr is required")
        self.layout = layout
        self.desc = L.PlanDesc(kind=L.FI_KIND_BLOCK_SPARSE, batch=1, num_qo_heads=num_qo_heads,
                               num_kv_heads=Hkv, head_dim=head_dim, page_size=ps,
                               deterministic=int(deterministic), det_chunk_pages=det_chunk_pages,
                               min_chunk_pages=min_chunk_pages, num_cus=num_cus,
                               workers_per_cu=workers_per_cu, launch=_LAUNCHES[launch],
                               pod_wide_blocks=pod_wide_blocks,
                               kv_layout=L.FI_KV_LAYOUT_RAGGED if layout == "ragged"
                               else L.FI_KV_LAYOUT_PAGED)
        self.num_qo_heads, self.num_kv_heads = num_qo_heads, Hkv
        self.head_dim, self.page_size, self.batch = head_dim, ps, S
        self.num_q_tokens = int(self._ha["qo_len"].sum()) if S else 0
        # ragged: the kernels read whole page_size-token runs, the last of them
        # up to page_size - 1 rows past the last sequence's end
        self.kv_tokens = int(self._ha["kv_indptr"][-1]) + ps - 1 if layout == "ragged" and S \
            else 0
        self.device = _device(device)
        self.workspace = workspace
        ws_dev = ws_host = None
        dev_b = host_b = 0
        stream = None
        a = self._ha
        if self.device is not None:
            if self.workspace is None:
                db, hb = ctypes.c_size_t(), ctypes.c_size_t()
                L.check(lib.fi_workspace_size_block_sparse_batch(
                    ctypes.byref(self.desc), S, _p(a["qo_len"]), _p(a["kv_len"]), _p(a["nrb"]),
                    _p(a["ncb"]), ctypes.byref(db), ctypes.byref(hb)),
                    "fi_workspace_size_block_sparse_batch")
                self.workspace = Workspace(db.value, hb.value, self.device)
            ws_dev, ws_host = _ptr(self.workspace.dev), _ptr(self.workspace.host)
            dev_b, host_b = self.workspace.dev.numel(), self.workspace.host.numel()
            stream = _stream(self.device)
        h = ctypes.c_void_p()
        L.check(lib.fi_plan_block_sparse_batch(
            ctypes.byref(self.desc), S, _p(a["qo_len"]), _p(a["kv_len"]), _p(a["nrb"]),
            _p(a["row"]), _p(a["ncb"]), _p(a["col"]), a["mask"].ctypes.data_as(ctypes.c_void_p),
            _p(a["kv_indptr"]), _p(a["kv_indices"]), ws_dev, dev_b, ws_host, host_b, stream,
            ctypes.byref(h)), "fi_plan_block_sparse_batch")
        self._h = h


def _check_tensor(t, name, dtype, device, shape=None):
    # the common case in one expression; anything else goes through the
    # checks below, which name what is wrong
    try:
        if (t.dtype is dtype and t.get_device() == device.index and t.is_contiguous()
                and (shape is None or t.shape == shape)):
            return
    except AttributeError:
        pass
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_cache(plan: Plan, k_cache, v_cache):
    dev = plan.device
    _check_tensor(k_cache, "k_cache", torch.bfloat16, dev)
    _check_tensor(v_cache, "v_cache", torch.bfloat16, dev, k_cache.shape)
    if k_cache.dim() != 4 or k_cache.shape[1:] != (plan.num_kv_heads, plan.page_size,
                                                   plan.head_dim):
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match the plan "
                         f"[P, {plan.num_kv_heads}, {plan.page_size}, {plan.head_dim}]")


def _outputs(plan: Plan, q, out, lse):
    T = plan.num_q_tokens
    if out is None:
        out = torch.empty_like(q)
    _check_tensor(out, "out", torch.bfloat16, plan.device, (T, plan.num_qo_heads, plan.head_dim))
    if lse is not None:
        _check_tensor(lse, "lse", torch.float32, plan.device, (T, plan.num_qo_heads))
    return out, lse


def _check_table(plan: Plan, t, name: str, key: str):
    """A device page table must hold at least the entries the plan's host
    table covers (``plan._ha[key][-1]``): the kernels read that many ids
    unchecked, so a shorter table would be read past its end."""
    _check_tensor(t, name, torch.int32, plan.device)
    needs = plan.__dict__.setdefault("_table_need", {})
    need = needs.get(key)
    if need is None:
        ptr = plan._ha.get(key)
        need = needs[key] = int(ptr[-1]) if ptr is not None and ptr.size else 0
    if t.numel() < need:
        raise ValueError(f"{name} has {t.numel()} entries, the plan's table needs {need}")


def _check_run(plan: Plan, kind: str):
    if plan.kind != kind:
        raise ValueError(f"plan kind is {plan.kind}, not {kind}")
    if plan.device is None:
        raise ValueError("host-only plan: build it with a device to run it")


def paged_decode(plan: Plan, q, k_cache, v_cache, kv_indices, sm_scale: float, out=None,
                 lse=None, return_lse: bool = True):
    """fi_paged_decode: q [B, Hq, D] bf16 -> (out [B, Hq, D] bf16, lse [B, Hq] fp32)."""
    _check_run(plan, "decode")
    _check_tensor(q, "q", torch.bfloat16, plan.device,
                  (plan.batch, plan.num_qo_heads, plan.head_dim))
    _check_cache(plan, k_cache, v_cache)
    _check_table(plan, kv_indices, "kv_indices", "kv_indptr")
    if lse is None and return_lse:
        lse = torch.empty(plan.batch, plan.num_qo_heads, dtype=torch.float32, device=plan.device)
    out, lse = _outputs(plan, q, out, lse)
    L.check(L.load().fi_paged_decode(plan.handle, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(kv_indices), float(sm_scale), _ptr(out), _ptr(lse),
                                     _stream(plan.device)), "fi_paged_decode")
    return out, lse


def paged_decode_noalloc(plan: Plan, q, k_cache, v_cache, kv_indices, sm_scale: float, out,
                         lse=None):
    """fi_paged_decode_noalloc: the decode of ``paged_decode`` with the plan's
    workspace in the library's static device scratch, for callers that cannot
    allocate. ``plan`` is a host-only decode plan (``device=None`` and
    ``num_cus`` given); ``out`` (and ``lse``, if given) are caller buffers,
    since this call allocates nothing; tensors on the current device. Calls
    that overlap on one GPU race on the shared scratch."""
    if plan.kind != "decode":
        raise ValueError(f"plan kind is {plan.kind}, not decode")
    if plan.device is not None:
        raise ValueError("fi_paged_decode_noalloc takes a host-only plan (device=None)")
    dev = q.device
    _check_tensor(q, "q", torch.bfloat16, dev, (plan.batch, plan.num_qo_heads, plan.head_dim))
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _check_tensor(t, n, torch.bfloat16, dev)
        if t.dim() != 4 or tuple(t.shape[1:]) != (plan.num_kv_heads, plan.page_size,
                                                  plan.head_dim):
            raise ValueError(f"{n} shape {tuple(t.shape)} does not match the plan")
    _check_tensor(kv_indices, "kv_indices", torch.int32, dev)
    need = int(plan._ha["kv_indptr"][-1]) if plan._ha["kv_indptr"].size else 0
    if kv_indices.numel() < need:
        raise ValueError(f"kv_indices has {kv_indices.numel()} entries, the plan needs {need}")
    _check_tensor(out, "out", torch.bfloat16, dev, (plan.batch, plan.num_qo_heads, plan.head_dim))
    if lse is not None:
        _check_tensor(lse, "lse", torch.float32, dev, (plan.batch, plan.num_qo_heads))
    L.check(L.load().fi_paged_decode_noalloc(plan.handle, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                             _ptr(kv_indices), float(sm_scale), _ptr(out),
                                             _ptr(lse), _stream(dev)), "fi_paged_decode_noalloc")
    return out, lse


def paged_decode_fp8(plan: Plan, q, k_cache, v_cache, k_scale, v_scale, kv_indices,
                     sm_scale: float, out=None, lse=None, return_lse: bool = True):
    """fi_paged_decode_fp8: K/V pools of FP8 E4M3 codes (uint8, same shape as
    the bf16 pools) with fp32 scales [pages, Hkv]; q, out, lse as paged_decode."""
    _check_run(plan, "decode")
    _check_tensor(q, "q", torch.bfloat16, plan.device,
                  (plan.batch, plan.num_qo_heads, plan.head_dim))
    _check_tensor(k_cache, "k_cache", torch.uint8, plan.device)
    _check_tensor(v_cache, "v_cache", torch.uint8, plan.device, k_cache.shape)
    if k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (plan.num_kv_heads, plan.page_size,
                                                          plan.head_dim):
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match the plan "
                         f"[P, {plan.num_kv_heads}, {plan.page_size}, {plan.head_dim}]")
    P = k_cache.shape[0]
    _check_tensor(k_scale, "k_scale", torch.float32, plan.device, (P, plan.num_kv_heads))
    _check_tensor(v_scale, "v_scale", torch.float32, plan.device, (P, plan.num_kv_heads))
    _check_table(plan, kv_indices, "kv_indices", "kv_indptr")
    if lse is None and return_lse:
        lse = torch.empty(plan.batch, plan.num_qo_heads, dtype=torch.float32, device=plan.device)
    out, lse = _outputs(plan, q, out, lse)
    L.check(L.load().fi_paged_decode_fp8(plan.handle, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(k_scale), _ptr(v_scale), _ptr(kv_indices),
                                         float(sm_scale), _ptr(out), _ptr(lse),
                                         _stream(plan.device)), "fi_paged_decode_fp8")
    return out, lse


def paged_decode_mxfp4(plan: Plan, q, k_codes, v_codes, k_scales, v_scales, kv_indices,
                       sm_scale: float, out=None, lse=None, return_lse: bool = True):
    """fi_paged_decode_mxfp4: K/V as MXFP4 codes (uint8 [P, Hkv, ps, D/2], two
    E2M1 elements per byte, low nibble first) with E8M0 scales (uint8
    [P, Hkv, ps, D/32], one per 32 elements); q, out, lse as paged_decode."""
    _check_run(plan, "decode")
    _check_tensor(q, "q", torch.bfloat16, plan.device,
                  (plan.batch, plan.num_qo_heads, plan.head_dim))
    D = plan.head_dim
    _check_tensor(k_codes, "k_codes", torch.uint8, plan.device)
    P = k_codes.shape[0]
    _check_tensor(k_codes, "k_codes", torch.uint8, plan.device,
                  (P, plan.num_kv_heads, plan.page_size, D // 2))
    _check_tensor(v_codes, "v_codes", torch.uint8, plan.device, k_codes.shape)
    sshape = (P, plan.num_kv_heads, plan.page_size, D // 32)
    _check_tensor(k_scales, "k_scales", torch.uint8, plan.device, sshape)
    _check_tensor(v_scales, "v_scales", torch.uint8, plan.device, sshape)
    _check_table(plan, kv_indices, "kv_indices", "kv_indptr")
    if lse is None and return_lse:
        lse = torch.empty(plan.batch, plan.num_qo_heads, dtype=torch.float32, device=plan.device)
    out, lse = _outputs(plan, q, out, lse)
    L.check(L.load().fi_paged_decode_mxfp4(plan.handle, _ptr(q), _ptr(k_codes), _ptr(v_codes),
                                           _ptr(k_scales), _ptr(v_scales), _ptr(kv_indices),
                                           float(sm_scale), _ptr(out), _ptr(lse),
                                           _stream(plan.device)), "fi_paged_decode_mxfp4")
    return out, lse


def check_page_tables(plan: Plan, kv_indices, num_pages: int, prefix_indices=None) -> int:
    """fi_check_page_tables (debugging aid): the number of page ids outside
    [0, num_pages) in the entries of ``kv_indices`` (and ``prefix_indices``)
    that run calls with ``plan`` read. Synchronises the stream to return it."""
    if plan.device is None:
        raise ValueError("host-only plan: the check runs on the plan's device")
    _check_table(plan, kv_indices, "kv_indices", "kv_indptr")
    if prefix_indices is not None:
        _check_table(plan, prefix_indices, "prefix_indices", "prefix_indptr")
    count = torch.empty(1, dtype=torch.int32, device=plan.device)
    L.check(L.load().fi_check_page_tables(plan.handle, _ptr(kv_indices), _ptr(prefix_indices),
                                          int(num_pages), _ptr(count), _stream(plan.device)),
            "fi_check_page_tables")
    return int(count.item())


def paged_append(plan: Plan, q, k_cache, v_cache, kv_indices, sm_scale: float, k_new=None,
                 v_new=None, out=None, lse=None, return_lse: bool = True):
    """fi_paged_append: q [sum qo, Hq, D]; optional k_new/v_new [sum qo, Hkv, D]
    are scattered into the cache first."""
    _check_run(plan, "append")
    T = plan.num_q_tokens
    _check_tensor(q, "q", torch.bfloat16, plan.device, (T, plan.num_qo_heads, plan.head_dim))
    _check_cache(plan, k_cache, v_cache)
    _check_table(plan, kv_indices, "kv_indices", "kv_indptr")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        shp = (T, plan.num_kv_heads, plan.head_dim)
        _check_tensor(k_new, "k_new", torch.bfloat16, plan.device, shp)
        _check_tensor(v_new, "v_new", torch.bfloat16, plan.device, shp)
    if lse is None and return_lse:
        lse = torch.empty(T, plan.num_qo_heads, dtype=torch.float32, device=plan.device)
    out, lse = _outputs(plan, q, out, lse)
    L.check(L.load().fi_paged_append(plan.handle, _ptr(q), _ptr(k_new), _ptr(v_new),
                                     _ptr(k_cache), _ptr(v_cache), _ptr(kv_indices),
                                     float(sm_scale), _ptr(out), _ptr(lse),
                                     _stream(plan.device)), "fi_paged_append")
    return out, lse


def cascade(plan: Plan, q, k_cache, v_cache, prefix_indices, kv_indices, sm_scale: float,
            out=None, lse=None, return_lse: bool = True):
    """fi_cascade: decode over (group prefix) || (own suffix), prefix read once."""
    _check_run(plan, "cascade")
    _check_tensor(q, "q", torch.bfloat16, plan.device,
                  (plan.batch, plan.num_qo_heads, plan.head_dim))
    _check_cache(plan, k_cache, v_cache)
    _check_table(plan, prefix_indices, "prefix_indices", "prefix_indptr")
    _check_table(plan, kv_indices, "kv_indices", "kv_indptr")
    if lse is None and return_lse:
        lse = torch.empty(plan.batch, plan.num_qo_heads, dtype=torch.float32, device=plan.device)
    out, lse = _outputs(plan, q, out, lse)
    L.check(L.load().fi_cascade(plan.handle, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                _ptr(prefix_indices), _ptr(kv_indices), float(sm_scale),
                                _ptr(out), _ptr(lse), _stream(plan.device)), "fi_cascade")
    return out, lse


def block_sparse_attention(plan: BlockSparsePlan, q, k_cache, v_cache, sm_scale: float,
                           out=None, lse=None, return_lse: bool = True):
    """fi_block_sparse_attention: q [T, Hq, D] bf16 -> (out, lse [T, Hq]), T
    the plan's query rows; k_cache/v_cache paged pools, or [tokens, Hkv, D]
    tensors for a ragged plan."""
    _check_run(plan, "block_sparse")
    T = plan.num_q_tokens
    _check_tensor(q, "q", torch.bfloat16, plan.device, (T, plan.num_qo_heads, plan.head_dim))
    if getattr(plan, "layout", "paged") == "ragged":
        _check_tensor(k_cache, "k", torch.bfloat16, plan.device)
        _check_tensor(v_cache, "v", torch.bfloat16, plan.device, k_cache.shape)
        if (k_cache.dim() != 3 or tuple(k_cache.shape[1:]) != (plan.num_kv_heads, plan.head_dim)
                or k_cache.shape[0] < plan.kv_tokens):
            raise ValueError(f"ragged K/V shape {tuple(k_cache.shape)} does not match the plan "
                             f"[>= {plan.kv_tokens}, {plan.num_kv_heads}, {plan.head_dim}]")
    else:
        _check_cache(plan, k_cache, v_cache)
    if lse is None and return_lse:
        lse = torch.empty(T, plan.num_qo_heads, dtype=torch.float32, device=plan.device)
    out, lse = _outputs(plan, q, out, lse)
    L.check(L.load().fi_block_sparse_attention(plan.handle, _ptr(q), _ptr(k_cache),
                                               _ptr(v_cache), float(sm_scale), _ptr(out),
                                               _ptr(lse), _stream(plan.device)),
            "fi_block_sparse_attention")
    return out, lse


def merge_states(v, s, out_dtype=None, return_lse: bool = True):
    """fi_merge_states: v [N, S, H, D] (bf16 or fp32), s [N, S, H] fp32 ->
    (v_out [N, H, D], s_out [N, H]), folding index 0 first."""
    if v.dim() != 4 or s.dim() != 3 or tuple(s.shape) != tuple(v.shape[:3]):
        raise ValueError("expected v [N, S, H, D] and s [N, S, H]")
    if v.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("v must be bf16 or fp32")
    _check_tensor(v, "v", v.dtype, v.device)
    _check_tensor(s, "s", torch.float32, v.device)
    out_dtype = v.dtype if out_dtype is None else out_dtype
    N, S, H, D = v.shape
    v_out = torch.empty(N, H, D, dtype=out_dtype, device=v.device)
    s_out = torch.empty(N, H, dtype=torch.float32, device=v.device) if return_lse else None
    dt = lambda t: L.FI_DTYPE_F32 if t == torch.float32 else L.FI_DTYPE_BF16  # noqa: E731
    L.check(L.load().fi_merge_states(_ptr(v), dt(v.dtype), _ptr(s), N, S, H, D, _ptr(v_out),
                                     dt(out_dtype), _ptr(s_out), _stream(v.device)),
            "fi_merge_states")
    return v_out, s_out


class KernelTimer:
    """Context manager over fi_timer_begin/fi_timer_end: HIP events recorded on
    the launch stream around each run call's attention kernel(s)."""

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.total_ms = None
        self.calls = None

    def __enter__(self):
        L.check(L.load().fi_timer_begin(self.capacity), "fi_timer_begin")
        return self

    def __exit__(self, *exc):
        ms, n = ctypes.c_double(), ctypes.c_int32()
        L.check(L.load().fi_timer_end(ctypes.byref(ms), ctypes.byref(n)), "fi_timer_end")
        self.total_ms, self.calls = ms.value, n.value
        return False
