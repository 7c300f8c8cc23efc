"""Thin Python binding over libdkv's C ABI (argument marshalling only).

PyTorch supplies device memory and the current HIP stream; every step of the
path runs in libdkv's kernels.  Names follow the C functions:

  project_rope_append  -> dkv_project_rope_append
  decode_plan          -> dkv_decode_plan
  decode_attn_split    -> dkv_decode_attn_split
  merge_lse            -> dkv_merge_lse
  prefill_plan / prefill_attn_split -> dkv_prefill_plan / dkv_prefill_attn_split
  host_alloc / HostBuffer -> dkv_host_alloc / dkv_host_free
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib
from ._lib import KvDesc, PagerStats, PlanInfo, Tuning, BwResult, check, lib

DKV_HOST_COHERENT = _lib.DKV_HOST_COHERENT
DKV_HOST_NONCOHERENT = _lib.DKV_HOST_NONCOHERENT


def _stream(stream):
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return C.c_void_p(t.data_ptr())
    if isinstance(t, np.ndarray):
        return C.c_void_p(t.ctypes.data)
    return C.c_void_p(int(t))


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def version() -> int:
    return lib().dkv_version()


def split_point(ratio: float, length: int) -> int:
    out = C.c_int64()
    check(lib().dkv_split_point(float(ratio), int(length), C.byref(out)))
    return out.value


class HostBuffer:
    """Host-pinned block mapped into the GPU's address space (dkv_host_alloc)."""

    def __init__(self, nbytes: int, flags: int = DKV_HOST_COHERENT):
        h, d = C.c_void_p(), C.c_void_p()
        check(lib().dkv_host_alloc(int(nbytes), int(flags), C.byref(h), C.byref(d)))
        self.host_ptr = h.value
        self.dev_ptr = d.value
        self.nbytes = int(nbytes)
        self.flags = flags

    def numpy(self, dtype=np.uint16, shape=None) -> np.ndarray:
        buf = (C.c_uint8 * self.nbytes).from_address(self.host_ptr)
        a = np.frombuffer(buf, dtype=np.uint8).view(dtype)
        return a.reshape(shape) if shape is not None else a

    def free(self):
        if self.host_ptr:
            torch.cuda.synchronize()
            check(lib().dkv_host_free(C.c_void_p(self.host_ptr)))
            self.host_ptr = None
            self.dev_ptr = None

    def __del__(self):
        # hipHostFree waits for the device before releasing pinned memory
        try:
            if self.host_ptr:
                lib().dkv_host_free(C.c_void_p(self.host_ptr))
        except Exception:
            pass


class KVCache:
    """Two tier pools (host-pinned and HBM) plus the placement description.

    Rows are tokens: [num_kv_heads][head_dim] bf16, K and V in separate pools.
    ``page_table`` (paged placement) is an int32 array [batch][max_pages] with
    entries phys << 1 | tier; it is uploaded to the device and kept on the host.
    """

    def __init__(self, num_kv_heads: int, head_dim: int, *, host_rows: int = 0, dev_rows: int = 0,
                 page_size: int = 0, page_table=None, host_stride: int = 0, dev_stride: int = 0,
                 host_flags: int = DKV_HOST_COHERENT, device: str = "cuda"):
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        self.page_size = int(page_size)
        self.host_stride = int(host_stride)
        self.dev_stride = int(dev_stride)
        self.host_rows = int(host_rows)
        self.dev_rows = int(dev_rows)
        row_bytes = self.num_kv_heads * self.head_dim * 2
        self.host_k = HostBuffer(max(1, self.host_rows) * row_bytes, host_flags) if self.host_rows else None
        self.host_v = HostBuffer(max(1, self.host_rows) * row_bytes, host_flags) if self.host_rows else None
        shape = (max(1, self.dev_rows), self.num_kv_heads, self.head_dim)
        self.dev_k = torch.empty(shape, dtype=torch.bfloat16, device=device) if self.dev_rows else None
        self.dev_v = torch.empty(shape, dtype=torch.bfloat16, device=device) if self.dev_rows else None
        self.page_table_host = None
        self.page_table = None
        self.max_pages = 0
        if self.page_size:
            self.set_page_table(page_table)

    def set_page_table(self, page_table):
        """Replace the page table (host copy and device copy).  Work already
        queued may still read the old device table, so the current stream is
        synchronized before the old one is released."""
        pt = np.ascontiguousarray(np.asarray(page_table, dtype=np.int32))
        if pt.ndim != 2:
            raise ValueError("page_table must be [batch][max_pages]")
        if self.page_table is not None:
            torch.cuda.current_stream().synchronize()
        self.page_table_host = pt
        self.max_pages = int(pt.shape[1])
        self.page_table = torch.from_numpy(pt).to("cuda")

    def update_page_table(self, page_table):
        """Overwrite the page table in place (same shape): host copy now, device
        copy by a copy queued on the current stream after earlier work."""
        pt = np.ascontiguousarray(np.asarray(page_table, dtype=np.int32))
        if self.page_table is None or pt.shape != self.page_table_host.shape:
            raise ValueError("update_page_table needs a table of the current shape")
        np.copyto(self.page_table_host, pt)
        self.page_table.copy_(torch.from_numpy(pt))

    def with_page_table(self, page_table) -> "KVCache":
        """A view that shares this cache's pools and has its own page table
        (for a batch made of some of the sequences).  Freeing a view does not
        free the pools."""
        import copy
        v = copy.copy(self)
        v.page_table = None
        v.page_table_host = None
        v.set_page_table(page_table)
        v._is_view = True
        return v

    def host_view(self, which: str) -> np.ndarray:
        """uint16 numpy view [host_rows][Hkv][D] of a host pool ('k' or 'v')."""
        buf = self.host_k if which == "k" else self.host_v
        return buf.numpy(np.uint16, (self.host_rows, self.num_kv_heads, self.head_dim))

    def desc(self) -> KvDesc:
        d = KvDesc()
        d.num_kv_heads = self.num_kv_heads
        d.head_dim = self.head_dim
        d.page_size = self.page_size
        d.max_pages = self.max_pages
        d.host_stride = self.host_stride
        d.dev_stride = self.dev_stride
        d.host_rows = self.host_rows
        d.dev_rows = self.dev_rows
        d.host_k = self.host_k.dev_ptr if self.host_k else None
        d.host_v = self.host_v.dev_ptr if self.host_v else None
        d.dev_k = self.dev_k.data_ptr() if self.dev_k is not None else None
        d.dev_v = self.dev_v.data_ptr() if self.dev_v is not None else None
        d.page_table = self.page_table.data_ptr() if self.page_table is not None else None
        d.page_table_host = self.page_table_host.ctypes.data if self.page_table_host is not None else None
        return d

    def free(self):
        if getattr(self, "_is_view", False):
            return
        for b in (self.host_k, self.host_v):
            if b is not None:
                b.free()


class PagedKVAllocator:
    """Paged KV pools managed by the native allocator (dkv_pager_*).

    ``pools`` is a paged KVCache over all ``max_seqs`` sequence slots: append
    through it with seq_idx = slot.  ``reserve`` / ``release`` change the
    allocator's table and copy it to ``pools``; ``batch(slots)`` is a view
    over the same pools whose page table rows are the given slots, for an
    attention call over those sequences.
    """

    def __init__(self, num_kv_heads: int, head_dim: int, *, n_host_pages: int, n_dev_pages: int,
                 max_seqs: int, max_pages: int, host_fraction: float, page_size: int = 16,
                 host_flags: int = DKV_HOST_COHERENT):
        h = C.c_void_p()
        check(lib().dkv_pager_create(int(n_host_pages), int(n_dev_pages), int(page_size), int(max_seqs),
                                     int(max_pages), float(host_fraction), C.byref(h)))
        self._h = h
        tbl, npg = _lib.PI32(), _lib.PI32()
        check(lib().dkv_pager_table(h, C.byref(tbl), C.byref(npg)))
        self._table = np.ctypeslib.as_array(tbl, shape=(int(max_seqs), int(max_pages)))
        self._npages = np.ctypeslib.as_array(npg, shape=(int(max_seqs),))
        self.page_size = int(page_size)
        self.host_fraction = float(host_fraction)
        self.pools = KVCache(num_kv_heads, head_dim, host_rows=int(n_host_pages) * self.page_size,
                             dev_rows=int(n_dev_pages) * self.page_size, page_size=self.page_size,
                             page_table=self._table.copy(), host_flags=host_flags)

    def reserve(self, seq: int, n_tokens: int, sync: bool = True):
        """Pages for tokens [0, n_tokens) of slot ``seq`` (all or nothing)."""
        check(lib().dkv_pager_reserve(self._h, int(seq), int(n_tokens)))
        if sync:
            self.sync()

    def release(self, seq: int, sync: bool = True):
        check(lib().dkv_pager_release(self._h, int(seq)))
        if sync:
            self.sync()

    def sync(self):
        """Copy the allocator's table into ``pools`` (host and device copies)."""
        self.pools.update_page_table(self._table)

    def table(self) -> np.ndarray:
        return self._table.copy()

    def pages_of(self, seq: int) -> int:
        return int(self._npages[int(seq)])

    def stats(self) -> dict:
        st = PagerStats()
        check(lib().dkv_pager_stats_get(self._h, C.byref(st)))
        return st.as_dict()

    def batch(self, slots) -> KVCache:
        return self.pools.with_page_table(self._table[np.asarray(list(slots), dtype=np.int64)])

    def close(self):
        if self._h is not None:
            check(lib().dkv_pager_destroy(self._h))
            self._h = None
            self._table = self._npages = None
            self.pools.free()


def append_workspace_bytes(n_new: int, hidden: int, kv_dim: int) -> int:
    return int(lib().dkv_append_workspace_bytes(int(n_new), int(hidden), int(kv_dim)))


def project_rope_append(cache: KVCache, batch: int, seq_lens, ratio: float, seq_idx: torch.Tensor,
                        pos: torch.Tensor, *, x=None, wk=None, wv=None, k_new=None, v_new=None,
                        rope_theta: float = 1e4, workspace: torch.Tensor | None = None, stream=None):
    """dkv_project_rope_append.  seq_lens / seq_idx / pos are device int32 tensors."""
    n_new = int(seq_idx.numel())
    hidden = int(x.shape[-1]) if x is not None else 0
    ws_bytes = 0
    if x is not None:
        need = append_workspace_bytes(n_new, hidden, cache.num_kv_heads * cache.head_dim)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    d = cache.desc()
    check(lib().dkv_project_rope_append(
        C.byref(d), int(batch), _ptr(seq_lens), float(ratio), n_new, _ptr(seq_idx), _ptr(pos),
        _ptr(x), hidden, _ptr(wk), _ptr(wv), _ptr(k_new), _ptr(v_new), float(rope_theta),
        _ptr(workspace), ws_bytes, _stream(stream)))


def decode_plan(cache: KVCache, batch: int, num_q_heads: int, seq_lens, ratio: float) -> dict:
    """dkv_decode_plan; ``seq_lens`` (host, or None) adds the items those lengths give."""
    d = cache.desc()
    sl = None if seq_lens is None else _host_i32(seq_lens)
    info = PlanInfo()
    check(lib().dkv_decode_plan(C.byref(d), int(batch), int(num_q_heads), _ptr(sl), float(ratio),
                                C.byref(info)))
    return info.as_dict()


def plan_inspect(cache_or_desc, batch: int, num_q_heads: int, seq_lens, ratio: float, num_cus: int):
    """dkv_plan_inspect: (items [n][5] int64, page_list, split_offsets, info)."""
    d = cache_or_desc.desc() if isinstance(cache_or_desc, KVCache) else cache_or_desc
    sl = _host_i32(seq_lens)
    info = PlanInfo()
    check(lib().dkv_plan_inspect(C.byref(d), int(batch), int(num_q_heads), _ptr(sl), float(ratio),
                                 int(num_cus), None, 0, None, 0, None, C.byref(info)))
    n = info.host_items + info.dev_items
    items = np.zeros((max(n, 1), 5), dtype=np.int64)
    npl = int(sum(int(x) for x in sl)) if d.page_size else 0
    npl = (npl // max(1, d.page_size) + len(sl) + 1) if d.page_size else 1
    plist = np.zeros(npl, dtype=np.int32)
    offs = np.zeros(int(batch) + 1, dtype=np.int32)
    check(lib().dkv_plan_inspect(C.byref(d), int(batch), int(num_q_heads), _ptr(sl), float(ratio),
                                 int(num_cus), _ptr(items), n, _ptr(plist), len(plist), _ptr(offs),
                                 C.byref(info)))
    return items[:n], plist, offs, info.as_dict()


def prefill_plan_inspect(cache_or_desc, batch: int, num_q_heads: int, q_start, q_pos0, seq_lens,
                         ratio: float, num_cus: int, fused: bool = False):
    """dkv_prefill_plan_inspect: dict of items [n][11] int64, page pairs [m][2],
    staging tiles [k][3] int64, split_offsets [T+1] and the plan info."""
    d = cache_or_desc.desc() if isinstance(cache_or_desc, KVCache) else cache_or_desc
    qs, qp, sl = _host_i32(q_start), _host_i32(q_pos0), _host_i32(seq_lens)
    info = PlanInfo()
    args = (C.byref(d), int(batch), int(num_q_heads), _ptr(qs), _ptr(qp), _ptr(sl), float(ratio), int(bool(fused)),
            int(num_cus))
    check(lib().dkv_prefill_plan_inspect(*args, None, 0, None, 0, None, 0, None, 0, C.byref(info)))
    n = info.host_items + info.dev_items
    T = int(qs[-1])
    items = np.zeros((max(n, 1), 11), dtype=np.int64)
    # page pairs: at most (pages of the sequence) per item of a block
    npg = 2 * (n * (int(max(sl)) // max(1, d.page_size) + 2) if d.page_size else 1)
    pages = np.zeros(max(npg, 2), dtype=np.int32)
    ntile = int(sum(int(x) for x in sl)) + len(sl)
    tiles = np.zeros((max(ntile, 1), 3), dtype=np.int64)
    offs = np.zeros(T + 1, dtype=np.int32)
    check(lib().dkv_prefill_plan_inspect(*args, _ptr(items), n, _ptr(pages), len(pages), _ptr(tiles), ntile,
                                         _ptr(offs), T + 1, C.byref(info)))
    return {"items": items[:n], "pages": pages, "tiles": tiles[tiles[:, 2] > 0], "split_offsets": offs,
            "info": info.as_dict()}


def _dev_i32(a, device="cuda"):
    """int32 lengths/positions on the device: a device tensor is passed through
    (it must be int32); a host sequence is copied (convenience for tests)."""
    if isinstance(a, torch.Tensor):
        if a.dtype != torch.int32 or not a.is_cuda:
            raise ValueError("expected a device int32 tensor")
        return a.contiguous()
    return torch.tensor(np.asarray(a, dtype=np.int32), dtype=torch.int32, device=device)


@dataclass
class DecodeBuffers:
    workspace: torch.Tensor
    part_o: torch.Tensor
    part_lse: torch.Tensor
    split_offsets: torch.Tensor
    out_o: torch.Tensor
    out_lse: torch.Tensor
    info: dict


def alloc_decode_buffers(cache: KVCache, batch: int, num_q_heads: int, seq_lens, ratio: float,
                         device="cuda") -> DecodeBuffers:
    """Buffers of the split form for this shape: partials for the split bound of
    the shape (any lengths that fit the pools), a zero-filled workspace.
    ``seq_lens`` (host, optional) only adds the item counts to ``info``."""
    sl = None if seq_lens is None or isinstance(seq_lens, torch.Tensor) else seq_lens
    info = decode_plan(cache, batch, num_q_heads, sl, ratio)
    S = max(1, info["num_splits"])
    D = cache.head_dim
    return DecodeBuffers(
        workspace=torch.zeros(max(256, info["workspace_bytes"]), dtype=torch.uint8, device=device),
        part_o=torch.empty((S, num_q_heads, D), dtype=torch.float32, device=device),
        part_lse=torch.empty((S, num_q_heads), dtype=torch.float32, device=device),
        split_offsets=torch.empty(batch + 1, dtype=torch.int32, device=device),
        out_o=torch.empty((batch, num_q_heads, D), dtype=torch.float32, device=device),
        out_lse=torch.empty((batch, num_q_heads), dtype=torch.float32, device=device),
        info=info,
    )


def decode_attn_split(cache: KVCache, q: torch.Tensor, q_pos: torch.Tensor, seq_lens, ratio: float,
                      scale: float, rope_theta: float, *, bufs: DecodeBuffers | None = None,
                      stream=None) -> DecodeBuffers:
    """dkv_decode_attn_split.  q [B,Hq,D] bf16, q_pos [B] and seq_lens [B] int32
    on the device (a host list of lengths is copied).  Returns the buffers
    holding part_o/part_lse/split_offsets."""
    B, Hq, D = q.shape
    if bufs is None:
        bufs = alloc_decode_buffers(cache, B, Hq, seq_lens, ratio, q.device)
    sl = _dev_i32(seq_lens, q.device)
    d = cache.desc()
    check(lib().dkv_decode_attn_split(
        C.byref(d), int(B), int(Hq), _ptr(q), _ptr(q_pos), _ptr(sl), float(ratio), float(scale),
        float(rope_theta), _ptr(bufs.workspace), bufs.workspace.numel(), _ptr(bufs.part_o),
        _ptr(bufs.part_lse), _ptr(bufs.split_offsets), int(bufs.part_o.shape[0]), _stream(stream)))
    return bufs


def merge_lse(part_o: torch.Tensor, part_lse: torch.Tensor, split_offsets: torch.Tensor, batch: int,
              num_q_heads: int, head_dim: int, *, out_o=None, out_lse=None, stream=None):
    """dkv_merge_lse -> (o [B,Hq,D] fp32, lse [B,Hq] fp32)."""
    dev = part_o.device
    if out_o is None:
        out_o = torch.empty((batch, num_q_heads, head_dim), dtype=torch.float32, device=dev)
    if out_lse is None:
        out_lse = torch.empty((batch, num_q_heads), dtype=torch.float32, device=dev)
    check(lib().dkv_merge_lse(_ptr(part_o), _ptr(part_lse), _ptr(split_offsets), int(batch),
                              int(num_q_heads), int(head_dim), _ptr(out_o), _ptr(out_lse),
                              _stream(stream)))
    return out_o, out_lse


def decode(cache: KVCache, q, q_pos, seq_lens, ratio, scale, rope_theta, *, bufs=None, stream=None):
    """decode_attn_split followed by merge_lse on the same stream."""
    B, Hq, D = q.shape
    bufs = decode_attn_split(cache, q, q_pos, seq_lens, ratio, scale, rope_theta, bufs=bufs,
                             stream=stream)
    merge_lse(bufs.part_o, bufs.part_lse, bufs.split_offsets, B, Hq, D, out_o=bufs.out_o,
              out_lse=bufs.out_lse, stream=stream)
    return bufs.out_o, bufs.out_lse, bufs


def decode_step_plan(cache: KVCache, batch: int, num_q_heads: int, ratio: float, hidden: int = 0) -> dict:
    """dkv_decode_step_plan."""
    d = cache.desc()
    info = PlanInfo()
    check(lib().dkv_decode_step_plan(C.byref(d), int(batch), int(num_q_heads), float(ratio), int(hidden),
                                     C.byref(info)))
    return info.as_dict()


def decode_step_workspace(cache: KVCache, batch: int, num_q_heads: int, ratio: float, hidden: int = 0,
                          device="cuda") -> torch.Tensor:
    """A zero-filled workspace for dkv_decode_step (every call leaves it zeroed)."""
    info = decode_step_plan(cache, batch, num_q_heads, ratio, hidden)
    return torch.zeros(max(256, info["workspace_bytes"]), dtype=torch.uint8, device=device)


def decode_step(cache: KVCache, q: torch.Tensor, q_pos: torch.Tensor, seq_lens: torch.Tensor, ratio: float,
                scale: float, rope_theta: float, *, pos_new=None, k_new=None, v_new=None, x=None, wk=None,
                wv=None, workspace: torch.Tensor | None = None, out_o=None, out_lse=None, stream=None):
    """dkv_decode_step: append each sequence's new token (k_new/v_new [B,Hkv,D]
    bf16, or x [B,hidden] with wk/wv) at pos_new (default seq_lens), attend over
    seq_lens + 1 tokens and merge, in one launch.  Returns (o [B,Hq,D], lse [B,Hq])."""
    B, Hq, D = q.shape
    hidden = int(x.shape[1]) if x is not None else 0
    sl = _dev_i32(seq_lens, q.device)
    if workspace is None:
        workspace = decode_step_workspace(cache, B, Hq, ratio, hidden, q.device)
    if out_o is None:
        out_o = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if out_lse is None:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    d = cache.desc()
    check(lib().dkv_decode_step(
        C.byref(d), int(B), int(Hq), _ptr(q), _ptr(q_pos), _ptr(sl), _ptr(pos_new), _ptr(x), hidden, _ptr(wk),
        _ptr(wv), _ptr(k_new), _ptr(v_new), float(ratio), float(scale), float(rope_theta), _ptr(workspace),
        workspace.numel(), _ptr(out_o), _ptr(out_lse), _stream(stream)))
    return out_o, out_lse


def decode_step_static(cache: KVCache, q: torch.Tensor, q_pos: torch.Tensor, seq_lens: torch.Tensor, ratio: float,
                       scale: float, rope_theta: float, *, out_o: torch.Tensor, out_lse: torch.Tensor | None = None,
                       pos_new=None, k_new=None, v_new=None, x=None, wk=None, wv=None, stream=None):
    """dkv_decode_step_static: decode_step on the library's static scratch (no
    workspace, no allocation: the caller passes the outputs)."""
    B, Hq, D = q.shape
    hidden = int(x.shape[1]) if x is not None else 0
    if not isinstance(seq_lens, torch.Tensor):
        raise ValueError("seq_lens must be a device int32 tensor (this entry point allocates nothing)")
    d = cache.desc()
    check(lib().dkv_decode_step_static(
        C.byref(d), int(B), int(Hq), _ptr(q), _ptr(q_pos), _ptr(seq_lens), _ptr(pos_new), _ptr(x), hidden, _ptr(wk),
        _ptr(wv), _ptr(k_new), _ptr(v_new), float(ratio), float(scale), float(rope_theta), _ptr(out_o),
        _ptr(out_lse), _stream(stream)))
    return out_o, out_lse


def decode_staged_plan(cache: KVCache, num_q_heads: int, seq_len: int, ratio: float, chunk_tokens: int) -> dict:
    """dkv_decode_staged_plan."""
    d = cache.desc()
    info = PlanInfo()
    check(lib().dkv_decode_staged_plan(C.byref(d), int(num_q_heads), int(seq_len), float(ratio), int(chunk_tokens),
                                       C.byref(info)))
    return info.as_dict()


def decode_staged(cache: KVCache, q: torch.Tensor, q_pos: torch.Tensor, seq_len: int, ratio: float, scale: float,
                  rope_theta: float, chunk_tokens: int, *, workspace: torch.Tensor | None = None, out_o=None,
                  out_lse=None, stream=None):
    """dkv_decode_staged (one sequence): the host tier copied chunk by chunk
    into an HBM ring by the DMA engine and attended from there; returns
    (o [Hq, D], lse [Hq])."""
    _, Hq, D = q.shape
    if workspace is None:
        info = decode_staged_plan(cache, Hq, seq_len, ratio, chunk_tokens)
        workspace = torch.zeros(max(256, info["workspace_bytes"]), dtype=torch.uint8, device=q.device)
    if out_o is None:
        out_o = torch.empty((Hq, D), dtype=torch.float32, device=q.device)
    if out_lse is None:
        out_lse = torch.empty((Hq,), dtype=torch.float32, device=q.device)
    d = cache.desc()
    check(lib().dkv_decode_staged(C.byref(d), int(Hq), _ptr(q), _ptr(q_pos), int(seq_len), float(ratio),
                                  float(scale), float(rope_theta), int(chunk_tokens), _ptr(workspace),
                                  workspace.numel(), _ptr(out_o), _ptr(out_lse), _stream(stream)))
    return out_o, out_lse


def decode_errors(cache: KVCache, workspace: torch.Tensor, clear: bool = True) -> int:
    """dkv_decode_errors: layout error flags the decode kernels left in ``workspace``."""
    d = cache.desc()
    f = C.c_int32()
    check(lib().dkv_decode_errors(C.byref(d), _ptr(workspace), int(bool(clear)), C.byref(f)))
    return f.value


def set_tuning(**kw):
    t = Tuning()
    for k, v in kw.items():
        setattr(t, k, v)
    check(lib().dkv_set_tuning(C.byref(t)))


def reset_tuning():
    check(lib().dkv_set_tuning(None))


def get_tuning() -> dict:
    t = Tuning()
    check(lib().dkv_get_tuning(C.byref(t)))
    return {k: getattr(t, k) for k, _ in t._fields_}


def probe_read(src_dev_ptr: int, nbytes: int, nwg: int, nontemporal: bool = True, iters: int = 5,
               dma_dst=None, dma_src_host=None, stream=None, blocked: bool = False, src2_dev_ptr=None,
               segments: bool = False) -> dict:
    """dkv_probe_read: best of ``iters`` passes; ``blocked`` gives each workgroup
    one contiguous slice instead of a grid-stride walk, ``segments`` one 256-byte
    segment of every 2 KiB row of a slice; ``src2_dev_ptr`` adds a second buffer
    of ``nbytes`` read at the same time (the rate counts both)."""
    r = BwResult()
    mode = int(bool(nontemporal)) | (4 if segments else (2 if blocked else 0))
    src2 = C.c_void_p(int(src2_dev_ptr)) if src2_dev_ptr else None
    check(lib().dkv_probe_read(C.c_void_p(int(src_dev_ptr)), src2, int(nbytes), int(nwg), mode,
                               int(iters), _ptr(dma_dst), _ptr(dma_src_host), C.byref(r), _stream(stream)))
    return {"read_gbs": r.read_gbs, "read_ms": r.read_ms, "dma_gbs": r.dma_gbs}


KERNELS = {"attn": _lib.DKV_KERNEL_ATTN, "rope_q": _lib.DKV_KERNEL_ROPE_Q,
           "merge": _lib.DKV_KERNEL_MERGE, "append": _lib.DKV_KERNEL_APPEND,
           "prefill": _lib.DKV_KERNEL_PREFILL, "stage": _lib.DKV_KERNEL_STAGE,
           "linear": _lib.DKV_KERNEL_LINEAR, "tiers": _lib.DKV_KERNEL_TIERS}


def kernel_timing(enable: bool):
    """dkv_kernel_timing: bracket each launch with HIP events on its stream."""
    check(lib().dkv_kernel_timing(int(bool(enable))))


def kernel_timing_read(kernel: str) -> tuple[int, float]:
    """dkv_kernel_timing_read -> (launches timed, summed ms); clears the record."""
    n = C.c_int32()
    ms = C.c_double()
    check(lib().dkv_kernel_timing_read(KERNELS[kernel], C.byref(n), C.byref(ms)))
    return n.value, ms.value


def attn_trace(buffer: torch.Tensor | None):
    """dkv_attn_trace: per-workgroup (start, end, role, units) of later attention
    launches into ``buffer`` (int64 device tensor [n, 4]); None turns it off."""
    if buffer is None:
        check(lib().dkv_attn_trace(None, 0))
    else:
        assert buffer.dtype == torch.int64 and buffer.is_cuda and buffer.dim() == 2 and buffer.shape[1] == 4
        check(lib().dkv_attn_trace(_ptr(buffer), int(buffer.shape[0])))


class StepGraph:
    """A decode step (any sequence of binding calls on the current stream)
    captured once into a HIP graph and replayed.

    ``fn`` is run ``warmup`` times on a side stream first, which also builds
    and caches every plan it needs outside the capture.  Replays reuse the
    buffers ``fn`` wrote during capture; inputs are read from the same device
    addresses on every replay.
    """

    def __init__(self, fn, warmup: int = 2):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            fn()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()


def plan_cache_stats() -> dict:
    """dkv_plan_cache_stats: prefill plans cached, held by captured graphs, pinned bytes."""
    n, k, b = C.c_int32(), C.c_int32(), C.c_int64()
    check(lib().dkv_plan_cache_stats(C.byref(n), C.byref(k), C.byref(b)))
    return {"entries": n.value, "captured": k.value, "pinned_bytes": b.value}


def plan_cache_release_captured():
    """dkv_plan_cache_release_captured: call once every graph that captured a
    prefill call has been destroyed."""
    check(lib().dkv_plan_cache_release_captured())


def prefill_plan(cache: KVCache, batch: int, num_q_heads: int, q_start, q_pos0, seq_lens,
                 ratio: float) -> dict:
    """dkv_prefill_plan (host int32 arrays)."""
    d = cache.desc()
    qs, qp, sl = _host_i32(q_start), _host_i32(q_pos0), _host_i32(seq_lens)
    info = PlanInfo()
    check(lib().dkv_prefill_plan(C.byref(d), int(batch), int(num_q_heads), _ptr(qs), _ptr(qp), _ptr(sl),
                                 float(ratio), C.byref(info)))
    return info.as_dict()


def alloc_prefill_buffers(cache: KVCache, batch: int, num_q_heads: int, q_start, q_pos0, seq_lens,
                          ratio: float, device="cuda") -> DecodeBuffers:
    info = prefill_plan(cache, batch, num_q_heads, q_start, q_pos0, seq_lens, ratio)
    T = int(np.asarray(q_start)[-1])
    S = max(1, info["num_splits"])
    D = cache.head_dim
    return DecodeBuffers(
        workspace=torch.empty(max(256, info["workspace_bytes"]), dtype=torch.uint8, device=device),
        part_o=torch.empty((S, num_q_heads, D), dtype=torch.float32, device=device),
        part_lse=torch.empty((S, num_q_heads), dtype=torch.float32, device=device),
        split_offsets=torch.empty(T + 1, dtype=torch.int32, device=device),
        out_o=torch.empty((max(T, 1), num_q_heads, D), dtype=torch.float32, device=device),
        out_lse=torch.empty((max(T, 1), num_q_heads), dtype=torch.float32, device=device),
        info=info,
    )


def prefill_attn_split(cache: KVCache, q: torch.Tensor, q_start, q_pos0, seq_lens, ratio: float,
                       scale: float, rope_theta: float, *, bufs: DecodeBuffers | None = None,
                       stream=None) -> DecodeBuffers:
    """dkv_prefill_attn_split.  q [T,Hq,D] bf16 on the device; q_start [B+1],
    q_pos0 [B], seq_lens [B] on the host."""
    T, Hq, D = q.shape
    qs, qp, sl = _host_i32(q_start), _host_i32(q_pos0), _host_i32(seq_lens)
    B = len(sl)
    if bufs is None:
        bufs = alloc_prefill_buffers(cache, B, Hq, qs, qp, sl, ratio, q.device)
    d = cache.desc()
    check(lib().dkv_prefill_attn_split(
        C.byref(d), int(B), int(Hq), _ptr(q), _ptr(qs), _ptr(qp), _ptr(sl), float(ratio), float(scale),
        float(rope_theta), _ptr(bufs.workspace), bufs.workspace.numel(), _ptr(bufs.part_o),
        _ptr(bufs.part_lse), _ptr(bufs.split_offsets), int(bufs.part_o.shape[0]), _stream(stream)))
    return bufs


def prefill_fused_plan(cache: KVCache, batch: int, num_q_heads: int, q_start, q_pos0, seq_lens, ratio: float,
                       hidden: int = 0) -> dict:
    """dkv_prefill_fused_plan (host int32 arrays; hidden > 0 with projection)."""
    d = cache.desc()
    qs, qp, sl = _host_i32(q_start), _host_i32(q_pos0), _host_i32(seq_lens)
    info = PlanInfo()
    check(lib().dkv_prefill_fused_plan(C.byref(d), int(batch), int(num_q_heads), _ptr(qs), _ptr(qp), _ptr(sl),
                                       float(ratio), int(hidden), C.byref(info)))
    return info.as_dict()


def prefill_fused(cache: KVCache, q: torch.Tensor, q_start, q_pos0, seq_lens, ratio: float, scale: float,
                  rope_theta: float, *, k_new=None, v_new=None, x=None, wk=None, wv=None, workspace=None,
                  out_o=None, out_lse=None, stream=None):
    """dkv_prefill_fused: append the T new rows (k_new/v_new [T,Hkv,D] bf16, or
    x [T,hidden] with wk/wv) and attend causally; returns (o [T,Hq,D], lse [T,Hq])."""
    T, Hq, D = q.shape
    qs, qp, sl = _host_i32(q_start), _host_i32(q_pos0), _host_i32(seq_lens)
    B = len(qp)
    hidden = int(x.shape[1]) if x is not None else 0
    if T == 0:
        return (torch.empty((0, Hq, D), dtype=torch.float32, device=q.device),
                torch.empty((0, Hq), dtype=torch.float32, device=q.device))
    if workspace is None:
        info = prefill_fused_plan(cache, B, Hq, qs, qp, sl, ratio, hidden)
        workspace = torch.empty(max(256, info["workspace_bytes"]), dtype=torch.uint8, device=q.device)
    if out_o is None:
        out_o = torch.empty((max(T, 1), Hq, D), dtype=torch.float32, device=q.device)
    if out_lse is None:
        out_lse = torch.empty((max(T, 1), Hq), dtype=torch.float32, device=q.device)
    d = cache.desc()
    check(lib().dkv_prefill_fused(C.byref(d), B, int(Hq), _ptr(q), _ptr(qs), _ptr(qp), _ptr(sl), float(ratio),
                                  float(scale), float(rope_theta), _ptr(x), hidden, _ptr(wk), _ptr(wv),
                                  _ptr(k_new), _ptr(v_new), _ptr(workspace), workspace.numel(), _ptr(out_o),
                                  _ptr(out_lse), _stream(stream)))
    return out_o[:T], out_lse[:T]


def prefill(cache: KVCache, q, q_start, q_pos0, seq_lens, ratio, scale, rope_theta, *, bufs=None,
            stream=None):
    """prefill_attn_split followed by merge_lse over the T query rows."""
    T, Hq, D = q.shape
    bufs = prefill_attn_split(cache, q, q_start, q_pos0, seq_lens, ratio, scale, rope_theta, bufs=bufs,
                              stream=stream)
    if T > 0:
        merge_lse(bufs.part_o, bufs.part_lse, bufs.split_offsets, T, Hq, D, out_o=bufs.out_o,
                  out_lse=bufs.out_lse, stream=stream)
    return bufs.out_o[:T], bufs.out_lse[:T], bufs


# ------------------------------------------------------------------ offloaded linear

def linear_plan(m: int, out_features: int, in_features: int, ratio: float) -> dict:
    """dkv_linear_plan."""
    info = PlanInfo()
    check(lib().dkv_linear_plan(int(m), int(out_features), int(in_features), float(ratio), C.byref(info)))
    return info.as_dict()


def linear_plan_inspect(out_features: int, in_features: int, ratio: float, num_cus: int):
    """dkv_linear_plan_inspect: (items [n][6] int32, info)."""
    info = PlanInfo()
    check(lib().dkv_linear_plan_inspect(int(out_features), int(in_features), float(ratio), int(num_cus), None, 0,
                                        C.byref(info)))
    n = info.host_items + info.dev_items
    items = np.zeros((max(n, 1), 6), dtype=np.int32)
    check(lib().dkv_linear_plan_inspect(int(out_features), int(in_features), float(ratio), int(num_cus),
                                        _ptr(items), n, C.byref(info)))
    return items[:n], info.as_dict()


class OffloadedLinear:
    """A linear weight W [N][K] bf16 split by output rows: the first
    floor(r N) rows in mapped host memory, the rest in an HBM tensor."""

    def __init__(self, w_bits: np.ndarray, ratio: float, device="cuda", host_flags: int = DKV_HOST_COHERENT):
        w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
        self.out_features, self.in_features = (int(v) for v in w_bits.shape)
        self.ratio = float(ratio)
        self.n_host = split_point(self.ratio, self.out_features)
        K = self.in_features
        self.host = None
        if self.n_host > 0:
            self.host = HostBuffer(self.n_host * K * 2, host_flags)
            self.host.numpy(np.uint16, (self.n_host, K))[:] = w_bits[: self.n_host]
        nd = self.out_features - self.n_host
        self.dev = torch.from_numpy(w_bits[self.n_host:].view(np.int16).copy()).to(device) if nd > 0 else None
        self._ws = None

    def plan(self, m: int) -> dict:
        return linear_plan(m, self.out_features, self.in_features, self.ratio)

    def workspace(self, m: int, device="cuda") -> torch.Tensor:
        """A zero-filled workspace for calls of up to m tokens (every call
        leaves its counters at zero again)."""
        return torch.zeros(max(256, self.plan(m)["workspace_bytes"]), dtype=torch.uint8, device=device)

    def __call__(self, x: torch.Tensor, y: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
        """y = x W^T for x [m][K] bf16 (int16 bits) on the device; returns y [m][N] fp32."""
        m = int(x.shape[0])
        if y is None:
            y = torch.empty((m, self.out_features), dtype=torch.float32, device=x.device)
        if workspace is None:
            need = max(256, self.plan(m)["workspace_bytes"])
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.zeros(need, dtype=torch.uint8, device=x.device)   # every call leaves it zeroed
            workspace = self._ws
        check(lib().dkv_linear_split(C.c_void_p(self.host.dev_ptr if self.host else 0),
                                     _ptr(self.dev), self.out_features, self.in_features, self.ratio,
                                     _ptr(x), m, _ptr(y), _ptr(workspace), workspace.numel(), _stream(stream)))
        return y

    def free(self):
        if self.host is not None:
            self.host.free()
            self.host = None
        self.dev = None
