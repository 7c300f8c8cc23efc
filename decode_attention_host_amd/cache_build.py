"""Builders that fill tier pools through dkv_project_rope_append (bulk mode).

Raw (unrotated) keys and values are appended in chunks: the append kernel
rotates every key at its own position and writes both tiers, so the cache
content always comes from the GPU path.  Staging of the raw chunk into HBM is
plain torch copying (plumbing), not part of the method.
"""
from __future__ import annotations

import numpy as np
import torch

from .api import DKV_HOST_COHERENT, KVCache, project_rope_append, split_point

CHUNK_TOKENS = 1 << 16


def _append_rows(cache: KVCache, batch: int, b: int, t0: int, k_raw: np.ndarray, v_raw: np.ndarray,
                 seq_lens_dev, ratio: float, theta: float, positions=None):
    n = k_raw.shape[0]
    dev = "cuda"
    for c0 in range(0, n, CHUNK_TOKENS):
        c1 = min(n, c0 + CHUNK_TOKENS)
        k = torch.from_numpy(np.ascontiguousarray(k_raw[c0:c1]).view(np.int16)).to(dev)
        v = torch.from_numpy(np.ascontiguousarray(v_raw[c0:c1]).view(np.int16)).to(dev)
        if positions is None:
            pos = torch.arange(t0 + c0, t0 + c1, dtype=torch.int32, device=dev)
        else:
            pos = torch.as_tensor(np.asarray(positions[c0:c1], dtype=np.int32), device=dev)
        sidx = torch.full((c1 - c0,), b, dtype=torch.int32, device=dev)
        project_rope_append(cache, batch, seq_lens_dev, ratio, sidx, pos, k_new=k, v_new=v,
                            rope_theta=theta)


def contiguous_cache(hkv: int, d: int, lens, ratio: float, k_raw, v_raw, theta: float,
                     host_flags: int = DKV_HOST_COHERENT, host_stride=None, dev_stride=None,
                     upto=None) -> KVCache:
    """Contiguous-split cache: k_raw[b] / v_raw[b] are uint16 [L_b, Hkv, D] (bf16 bits).
    The placement follows the full lengths; tokens [0, upto[b]) are appended
    (default: all of them)."""
    lens = [int(x) for x in lens]
    nh = [split_point(ratio, n) for n in lens]
    hs = max(nh) if host_stride is None else int(host_stride)
    ds = max(n - h for n, h in zip(lens, nh)) if dev_stride is None else int(dev_stride)
    B = len(lens)
    cache = KVCache(hkv, d, host_rows=B * hs if hs else 0, dev_rows=B * ds if ds else 0,
                    host_stride=hs, dev_stride=ds, host_flags=host_flags)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for b in range(B):
        n = lens[b] if upto is None else int(upto[b])
        if n > 0:
            _append_rows(cache, B, b, 0, k_raw[b][:n], v_raw[b][:n], sl, ratio, theta)
    torch.cuda.synchronize()
    return cache


def paged_cache(hkv: int, d: int, lens, page_table: np.ndarray, n_host_pages: int, n_dev_pages: int,
                k_raw, v_raw, theta: float, page: int = 16, host_flags: int = DKV_HOST_COHERENT,
                upto=None) -> KVCache:
    """Paged cache; tokens [0, upto[b]) of each sequence are appended (default: all)."""
    lens = [int(x) for x in lens]
    B = len(lens)
    cache = KVCache(hkv, d, host_rows=n_host_pages * page, dev_rows=n_dev_pages * page,
                    page_size=page, page_table=page_table, host_flags=host_flags)
    for b in range(B):
        n = lens[b] if upto is None else int(upto[b])
        if n > 0:
            _append_rows(cache, B, b, 0, k_raw[b][:n], v_raw[b][:n], None, 0.0, theta)
    torch.cuda.synchronize()
    return cache


class SplitView:
    """Contiguous-split view of one sequence over full host and device copies
    of its cache (both built with every token at row t): tokens [0, n_host)
    are read from the host copy, the rest from the device copy.  Lets one
    pair of copies serve every offload ratio."""

    def __init__(self, host_full: KVCache, dev_full: KVCache, length: int, ratio: float):
        self.host_full, self.dev_full = host_full, dev_full
        self.head_dim = host_full.head_dim
        self.num_kv_heads = host_full.num_kv_heads
        self.length = int(length)
        self.n_host = split_point(ratio, self.length)

    def desc(self):
        d = self.host_full.desc()
        row_bytes = self.num_kv_heads * self.head_dim * 2
        L, nh = self.length, self.n_host
        d.host_stride = L
        d.host_rows = nh
        if nh == 0:
            d.host_k = d.host_v = None
        dd = self.dev_full.desc()
        d.dev_stride = L
        d.dev_rows = L - nh
        if L - nh > 0:
            d.dev_k = dd.dev_k + nh * row_bytes
            d.dev_v = dd.dev_v + nh * row_bytes
        else:
            d.dev_k = d.dev_v = None
        return d
