"""GPU parity of causal prefill over the split cache against the fp64 oracle.

The new rows' keys and values are appended first (same positions); then each
row attends causally to the cache.  Bar: max |do|, |dlse| <= 2e-3.
"""
import math

import numpy as np
import pytest

import oracle as O
from synth import kv_raw, normal_bf16, paged_table, query

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


def _prefill(dk, cache, qs, q_start, q_pos0, lens, ratio, theta, d):
    import torch
    q = torch.from_numpy(np.concatenate(qs, axis=0).view(np.int16)).cuda()
    o, lse, bufs = dk.prefill(cache, q, q_start, q_pos0, lens, ratio, 1.0 / math.sqrt(d), theta)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), bufs


def _check(o, lse, ro, rl, what):
    eo, el = np.abs(o - ro).max(), np.abs(lse - rl).max()
    print(f"{what}: max|do|={eo:.3g} max|dlse|={el:.3g}", flush=True)
    assert eo <= TOL and el <= TOL, what


CASES = [
    # (lens, new rows per seq, hq, hkv, d, ratio, theta)
    ([64], [64], 4, 2, 64, 1.0, 1e4),                  # all new KV, host tier
    ([377], [77], 32, 8, 128, 0.5, 5e5),               # cached prefix split over both tiers
    ([200, 33, 1000], [200, 1, 130], 8, 8, 128, 0.3, 1e4),  # MHA, ragged, an all-new sequence
    ([300], [40], 16, 2, 64, 0.0, 1e4),                # g = 8, HBM only
    ([130, 65], [65, 64], 8, 4, 128, 1.0, 5e5),        # g = 2, host only
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_contiguous(dk, case):
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, news, hq, hkv, d, r, th = CASES[case]
    ks, vs = kv_raw(70 + case, lens, hkv, d)
    qs = [normal_bf16(70 + case, 1, (n, hq, d)) for n in news]
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th)
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q_pos0 = [L - n for L, n in zip(lens, news)]
    o, lse, _ = _prefill(dk, cache, qs, q_start, q_pos0, lens, r, th, d)
    for b in range(len(lens)):
        ro, rl = O.prefill_sequence(qs[b], ks[b], vs[b], q_pos0[b], th, 1 / math.sqrt(d))
        _check(o[q_start[b]:q_start[b + 1]], lse[q_start[b]:q_start[b + 1]], ro, rl, f"case {case} seq {b}")
    cache.free()


def test_prefill_paged_ragged(dk):
    from decode_attention_host_amd.cache_build import paged_cache
    lens, news, hq, hkv, d, th = [500, 17, 1200], [100, 17, 333], 32, 8, 128, 5e5
    ks, vs = kv_raw(80, lens, hkv, d)
    qs = [normal_bf16(80 + b, 1, (n, hq, d)) for b, n in enumerate(news)]
    pt, nh, nd = paged_table(80, lens, 16, 0.8)
    cache = paged_cache(hkv, d, lens, pt, nh, nd, ks, vs, th)
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q_pos0 = [L - n for L, n in zip(lens, news)]
    o, lse, _ = _prefill(dk, cache, qs, q_start, q_pos0, lens, 0.0, th, d)
    for b in range(3):
        ro, rl = O.prefill_sequence(qs[b], ks[b], vs[b], q_pos0[b], th, 1 / math.sqrt(d))
        _check(o[q_start[b]:q_start[b + 1]], lse[q_start[b]:q_start[b + 1]], ro, rl, f"paged seq {b}")
    cache.free()


def test_prefill_single_row_equals_decode(dk):
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, hq, hkv, d, r, th = [999], 32, 8, 128, 0.5, 5e5
    ks, vs = kv_raw(81, lens, hkv, d)
    qb = query(81, 1, hq, d)
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th)
    o_p, l_p, _ = _prefill(dk, cache, [qb], np.array([0, 1], dtype=np.int32), [lens[0] - 1], lens, r, th, d)
    q = torch.from_numpy(qb.view(np.int16)).cuda()
    qpos = torch.tensor([lens[0] - 1], dtype=torch.int32, device="cuda")
    o_d, l_d, _ = dk.decode(cache, q, qpos, lens, r, 1 / math.sqrt(d), th)
    assert np.abs(o_p - o_d.cpu().numpy()).max() < 1e-5
    assert np.abs(l_p - l_d.cpu().numpy()).max() < 1e-5
    cache.free()


def test_prefill_rows_deep_in_a_long_cache(dk):
    # 48 rows at positions ~70000 over a 70048-token cache split host/HBM
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, n, hq, hkv, d, r, th = [70048], 48, 32, 8, 128, 0.6, 5e5
    ks, vs = kv_raw(83, lens, hkv, d)
    qb = normal_bf16(83, 1, (n, hq, d))
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th)
    q_pos0 = lens[0] - n
    o, lse, _ = _prefill(dk, cache, [qb], np.array([0, n], dtype=np.int32), [q_pos0], lens, r, th, d)
    heads = [0, 5, 18, 31]
    ro, rl = O.prefill_sequence(qb, ks[0], vs[0], q_pos0, th, 1 / math.sqrt(d), heads=heads)
    _check(o[:, heads], lse[:, heads], ro, rl, "deep rows")
    cache.free()


def test_prefill_staged_equals_direct(dk):
    # host rows read by several row blocks: staged copy vs direct host reads
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, news, hq, hkv, d, r, th = [700, 300], [300, 300], 32, 8, 128, 0.8, 5e5
    ks, vs = kv_raw(84, lens, hkv, d)
    qs = [normal_bf16(84 + b, 1, (n, hq, d)) for b, n in enumerate(news)]
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th)
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q_pos0 = [L - n for L, n in zip(lens, news)]
    outs = []
    try:
        for mib in (0, -1):
            dk.set_tuning(stage_max_mib=mib)
            o, lse, bufs = _prefill(dk, cache, qs, q_start, q_pos0, lens, r, th, d)
            print("stage_max_mib", mib, "staged bytes", bufs.info["staged_bytes"], flush=True)
            assert (bufs.info["staged_bytes"] > 0) == (mib == 0)
            outs.append((o, lse))
    finally:
        dk.reset_tuning()
    assert np.abs(outs[0][0] - outs[1][0]).max() < 1e-5
    assert np.abs(outs[0][1] - outs[1][1]).max() < 1e-5
    for b in range(2):
        ro, rl = O.prefill_sequence(qs[b], ks[b], vs[b], q_pos0[b], th, 1 / math.sqrt(d))
        _check(outs[0][0][q_start[b]:q_start[b + 1]], outs[0][1][q_start[b]:q_start[b + 1]], ro, rl,
               f"staged seq {b}")
    cache.free()


@pytest.mark.parametrize("ratio", [1.0, 0.0])
def test_prefill_llama3_2k_full_size(dk, ratio):
    # LLaMA-3-8B layer shape, 2048 new rows over an all-new cache: sampled rows
    from decode_attention_host_amd.cache_build import contiguous_cache
    L, hq, hkv, d, th = 2048, 32, 8, 128, 5e5
    ks, vs = kv_raw(0, [L], hkv, d)
    qb = normal_bf16(0, 1, (L, hq, d))
    cache = contiguous_cache(hkv, d, [L], ratio, ks, vs, th)
    o, lse, bufs = _prefill(dk, cache, [qb], np.array([0, L], dtype=np.int32), [0], [L], ratio, th, d)
    rows = [0, 1, 2, 63, 64, 127, 1000, 2047]
    heads = [0, 3, 17, 31]
    for r in rows:
        ro, rl = O.prefill_sequence(qb[r:r + 1], ks[0][:r + 1], vs[0][:r + 1], r, th, 1 / math.sqrt(d),
                                    heads=heads)
        _check(o[r:r + 1, heads], lse[r:r + 1, heads], ro, rl, f"r={ratio} row {r}")
    cache.free()


def test_prefill_many_small_items(dk):
    # tuned 128-token chunks: every row block is cut into several items per
    # tier (partials merged per row), and the ratio puts the tier boundary
    # inside a tile
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, news, hq, hkv, d, r, th = [3000, 1500], [200, 130], 32, 8, 128, 0.37, 5e5
    ks, vs = kv_raw(85, lens, hkv, d)
    qs = [normal_bf16(85 + b, 1, (n, hq, d)) for b, n in enumerate(news)]
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th)
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q_pos0 = [L - n for L, n in zip(lens, news)]
    try:
        dk.set_tuning(host_chunk=128, dev_chunk=128, stage_max_mib=-1)
        o, lse, bufs = _prefill(dk, cache, qs, q_start, q_pos0, lens, r, th, d)
        print("plan", bufs.info, flush=True)
        assert bufs.info["num_splits"] > 4 * sum(news)
    finally:
        dk.reset_tuning()
    for b in range(2):
        ro, rl = O.prefill_sequence(qs[b], ks[b], vs[b], q_pos0[b], th, 1 / math.sqrt(d))
        _check(o[q_start[b]:q_start[b + 1]], lse[q_start[b]:q_start[b + 1]], ro, rl, f"small items seq {b}")
    cache.free()


@pytest.mark.parametrize("page", [32, 128, 256])
def test_prefill_paged_page_sizes(dk, page):
    # pages smaller than, equal to and larger than a 128-key tile
    from decode_attention_host_amd.cache_build import paged_cache
    lens, news, hq, hkv, d, th = [700, 300], [90, 300], 16, 4, 128, 1e4
    ks, vs = kv_raw(86, lens, hkv, d)
    qs = [normal_bf16(86 + b, 1, (n, hq, d)) for b, n in enumerate(news)]
    pt, nh, nd = paged_table(86, lens, page, 0.6)
    cache = paged_cache(hkv, d, lens, pt, nh, nd, ks, vs, th, page=page)
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q_pos0 = [L - n for L, n in zip(lens, news)]
    o, lse, _ = _prefill(dk, cache, qs, q_start, q_pos0, lens, 0.0, th, d)
    for b in range(2):
        ro, rl = O.prefill_sequence(qs[b], ks[b], vs[b], q_pos0[b], th, 1 / math.sqrt(d))
        _check(o[q_start[b]:q_start[b + 1]], lse[q_start[b]:q_start[b + 1]], ro, rl, f"page {page} seq {b}")
    cache.free()
