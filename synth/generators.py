"""Seeded, synthetic inputs shaped like the decode-attention workloads.

The DirectKV README (Artifact Evaluation, Figure 10 / Figure 11 rows) measures
LLaMA-3-8B and OPT-6.7B serving; no weights, prompts or traces are used here.
Instead every tensor is drawn from a seeded normal distribution with the layer
shapes of those models, and ragged batches / page tables are drawn from seeded
integer streams.  The same arrays feed the fp64 oracle and the GPU path.

Recipe (stated once, used everywhere):
  * each tensor has its own stream ``numpy.random.default_rng([seed, id, chunk])``
    where ``id`` is a :class:`TensorId` and ``chunk`` indexes fixed blocks of
    ``CHUNK`` elements (so generation can run on several threads and stays
    bit-identical whatever the thread count);
  * float32 standard normals scaled by ``std`` are rounded to bfloat16 with
    round-to-nearest-even and returned as raw ``uint16`` bit patterns;
  * ragged lengths are ``rng.integers(lo, hi + 1)`` (both bounds inclusive);
  * page tables give each sequence ``ceil(n_tokens / page)`` pages, mark exactly
    ``floor(host_frac * n_pages)`` of them host-resident by a seeded
    permutation, and place pages at seeded-permuted physical slots inside the
    pool of their tier.  Entry encoding: ``phys << 1 | tier`` with tier 1 = host.
"""
from __future__ import annotations

import enum
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22  # elements per independent random stream


class TensorId(enum.IntEnum):
    Q = 1
    K = 2
    V = 3
    X = 4
    WK = 5
    WV = 6
    K_NEW = 7
    V_NEW = 8
    LENS = 9
    PAGES = 10
    EXTRA = 11


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill_chunk(out_flat, seed, tid, c, std):
    lo = c * CHUNK
    hi = min(out_flat.size, lo + CHUNK)
    rng = np.random.default_rng([seed, int(tid), c])
    x = rng.standard_normal(hi - lo, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    out_flat[lo:hi] = bf16_bits_from_f32(x)


def normal_bf16(seed: int, tid: int, shape, std: float = 1.0, out: np.ndarray | None = None,
                threads: int | None = None) -> np.ndarray:
    """bf16 (uint16 bits) array of N(0, std^2) draws; ``out`` may be a pinned buffer view."""
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == n and out.flags.c_contiguous
    flat = out.reshape(-1)
    nchunks = (n + CHUNK - 1) // CHUNK
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if nchunks <= 1 or threads <= 1:
        for c in range(nchunks):
            _fill_chunk(flat, seed, tid, c, std)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda c: _fill_chunk(flat, seed, tid, c, std), range(nchunks)))
    return out


def kv_raw(seed: int, lens, hkv: int, d: int, threads: int | None = None):
    """Raw (unrotated) keys and values per sequence: lists of uint16 [L_b, Hkv, D].
    Sequence b draws from seed ``seed * 1000 + b`` (tensor ids K and V)."""
    ks, vs = [], []
    for b, n in enumerate(lens):
        ks.append(normal_bf16(seed * 1000 + b, TensorId.K, (int(n), hkv, d), threads=threads))
        vs.append(normal_bf16(seed * 1000 + b, TensorId.V, (int(n), hkv, d), threads=threads))
    return ks, vs


def query(seed: int, batch: int, hq: int, d: int) -> np.ndarray:
    """Query bits [B, Hq, D], N(0, 1)."""
    return normal_bf16(seed, TensorId.Q, (batch, hq, d))


def ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Integer lengths uniform on [lo, hi], both inclusive."""
    rng = np.random.default_rng([seed, int(TensorId.LENS)])
    return rng.integers(lo, hi + 1, size=batch).astype(np.int64)


def paged_table(seed: int, n_tokens, page: int, host_frac: float, max_pages: int | None = None):
    """Random page table for sequences holding ``n_tokens[b]`` tokens.

    Returns ``(table[int32 B x max_pages], n_host_pages_total, n_dev_pages_total)``.
    Unused entries are -1.
    """
    rng = np.random.default_rng([seed, int(TensorId.PAGES)])
    n_tokens = [int(n) for n in n_tokens]
    n_pages = [(n + page - 1) // page for n in n_tokens]
    if max_pages is None:
        max_pages = max(n_pages)
    tiers = []
    for npg in n_pages:
        nh = int(math.floor(host_frac * npg))
        t = np.zeros(npg, dtype=np.int64)
        t[rng.permutation(npg)[:nh]] = 1
        tiers.append(t)
    n_host_total = int(sum(int(t.sum()) for t in tiers))
    n_dev_total = int(sum(len(t) - int(t.sum()) for t in tiers))
    host_slots = rng.permutation(n_host_total)
    dev_slots = rng.permutation(n_dev_total)
    table = np.full((len(n_tokens), max_pages), -1, dtype=np.int32)
    ih = idv = 0
    for b, t in enumerate(tiers):
        for j, tier in enumerate(t):
            if tier:
                phys = int(host_slots[ih]); ih += 1
            else:
                phys = int(dev_slots[idv]); idv += 1
            table[b, j] = (phys << 1) | int(tier)
    return table, n_host_total, n_dev_total


# The workloads: shapes of LLaMA-3-8B / OPT-6.7B attention layers (DirectKV
# README, Artifact Evaluation "What is reproduced" table; SplitKernel README,
# Overview and Key Features for the host/device split and offloading ratio),
# a 2048-row prefill of the LLaMA-3-8B layer, and the LLaMA-3-8B MLP
# up-projection as the offloaded-linear workload (SplitKernel README, Key
# Features: offloaded linear).
CONFIGS = {
    "tiny": dict(batch=1, hq=4, hkv=2, d=64, lens=[512], ratio=1.0, theta=1e4,
                 layout="contig"),
    "llama3_8b_32k": dict(batch=1, hq=32, hkv=8, d=128, lens=[32768], ratio=1.0,
                          theta=5e5, layout="contig"),
    "opt_6_7b_b8": dict(batch=8, hq=32, hkv=32, d=128, lens=[8192] * 8, ratio=0.5,
                        theta=1e4, layout="contig"),
    "llama3_8b_1m": dict(batch=1, hq=32, hkv=8, d=128, lens=[1 << 20], ratio=1.0,
                         theta=5e5, layout="contig",
                         ratios=[0.0, 0.25, 0.5, 0.75, 0.9, 1.0]),
    "llama3_8b_prefill_2k": dict(batch=1, hq=32, hkv=8, d=128, lens=[2048], new=[2048], ratio=1.0,
                                 theta=5e5, layout="contig", ratios=[1.0, 0.0]),
    "llama3_8b_mlp_up_linear": dict(out_features=14336, in_features=4096, tokens=[1, 16], w_std=0.02,
                                    layout="linear"),
    "fused_ragged": dict(batch=16, hq=32, hkv=8, d=128, lens_range=(1024, 65536),
                         ratio=0.8, theta=5e5, layout="paged", page=16, hidden=4096,
                         w_std=0.02),
}


def workload(name: str, seed: int = 0, **over):
    """Shape dictionary for a named workload, with ragged lengths drawn if needed."""
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    if "lens_range" in cfg and "lens" not in over:
        lo, hi = cfg["lens_range"]
        cfg["lens"] = [int(x) for x in ragged_lengths(seed, cfg["batch"], lo, hi)]
    cfg["name"] = name
    cfg["seed"] = seed
    return cfg
