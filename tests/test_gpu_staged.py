"""GPU parity of the staged-prefetch comparator (dkv_decode_staged): the host
tier copied by the DMA engine chunk by chunk into an HBM ring and attended
from there must give the oracle's result (max |do|, |dlse| <= 2e-3), like the
zero-copy path on the same cache.  Full size for the LLaMA-3-8B 32k layer
(all heads) and the 1M-token layer (sampled heads), at r = 0.25 and 1, plus
chunkings that do not divide the host tier, and no host tier at all.
"""
import math

import numpy as np
import pytest

import oracle as O
from synth import kv_raw, query, workload

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def dk():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import decode_attention_host_amd as dk
    dk.reset_tuning()
    return dk


def _run(dk, cache, qb, L, r, th, chunk):
    import torch
    hq, d = qb.shape[1], qb.shape[2]
    q = torch.from_numpy(qb.view(np.int16)).cuda()
    qpos = torch.tensor([L - 1], dtype=torch.int32, device="cuda")
    info = dk.decode_staged_plan(cache, hq, L, r, chunk)
    o, lse = dk.decode_staged(cache, q, qpos, L, r, 1 / math.sqrt(d), th, chunk)
    zo, zl, _ = dk.decode(cache, q, qpos, [L], r, 1 / math.sqrt(d), th)
    torch.cuda.synchronize()
    return (o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            zo[0].cpu().numpy().astype(np.float64), zl[0].cpu().numpy().astype(np.float64), info)


def _check(o, lse, ro, rl, what):
    eo = float(np.abs(o - ro).max())
    el = float(np.abs(lse - rl).max())
    print(f"{what}: max|do|={eo:.3g} max|dlse|={el:.3g}", flush=True)
    assert eo <= TOL and el <= TOL, what


@pytest.mark.parametrize("L,r,chunk", [(5000, 0.6, 1024), (3000, 1.0, 64), (777, 0.0, 256), (2049, 0.25, 2048)])
def test_staged_small(dk, L, r, chunk):
    from decode_attention_host_amd.cache_build import contiguous_cache
    hq, hkv, d, th = 16, 4, 128, 1e4
    ks, vs = kv_raw(95, [L], hkv, d)
    qb = query(95, 1, hq, d)
    cache = contiguous_cache(hkv, d, [L], r, ks, vs, th)
    o, lse, zo, zl, info = _run(dk, cache, qb, L, r, th, chunk)
    nh = O.contig_split_point(r, L)
    assert info["host_items"] == -(-nh // chunk) and info["staged_bytes"] == nh * hkv * d * 4
    ro, rl = O.decode_sequence(qb[0], ks[0], vs[0], L - 1, th, 1 / math.sqrt(d))
    _check(o, lse, ro, rl, f"staged L={L} r={r} chunk={chunk}")
    _check(zo, zl, ro, rl, "zero-copy, same cache")
    cache.free()


@pytest.mark.parametrize("r", [0.25, 1.0])
def test_staged_llama3_8b_32k_all_heads(dk, r):
    from decode_attention_host_amd.cache_build import contiguous_cache
    cfg = workload("llama3_8b_32k")
    L, hkv, hq, d, th = cfg["lens"][0], cfg["hkv"], cfg["hq"], cfg["d"], cfg["theta"]
    ks, vs = kv_raw(0, [L], hkv, d)
    qb = query(0, 1, hq, d)
    cache = contiguous_cache(hkv, d, [L], r, ks, vs, th)
    o, lse, zo, zl, _ = _run(dk, cache, qb, L, r, th, 8192)
    ro, rl = O.decode_sequence(qb[0], ks[0], vs[0], L - 1, th, 1 / math.sqrt(d))
    _check(o, lse, ro, rl, f"staged 32k r={r}")
    _check(zo, zl, ro, rl, f"zero-copy 32k r={r}")
    cache.free()


def test_staged_llama3_8b_1m_sampled_heads(dk):
    from decode_attention_host_amd.cache_build import SplitView, contiguous_cache
    cfg = workload("llama3_8b_1m")
    L, hkv, hq, d, th = cfg["lens"][0], cfg["hkv"], cfg["hq"], cfg["d"], cfg["theta"]
    ks, vs = kv_raw(0, [L], hkv, d)
    qb = query(0, 1, hq, d)
    host_full = contiguous_cache(hkv, d, [L], 1.0, ks, vs, th)
    dev_full = contiguous_cache(hkv, d, [L], 0.0, ks, vs, th)
    heads = [0, 13, 31]
    ro, rl = O.decode_sequence(qb[0], ks[0], vs[0], L - 1, th, 1 / math.sqrt(d), heads=heads)
    for r in (0.25, 1.0):
        view = SplitView(host_full, dev_full, L, r)
        o, lse, zo, zl, _ = _run(dk, view, qb, L, r, th, 16384)
        _check(o[heads], lse[heads], ro, rl, f"staged 1M r={r}")
        _check(zo[heads], zl[heads], ro, rl, f"zero-copy 1M r={r}")
    host_full.free()
    dev_full.free()
