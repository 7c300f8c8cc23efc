"""Decode attention over pools managed by the native paged allocator.

Sequences grow page by page through dkv_pager_reserve and the append ABI,
one is released and its slot refilled with another sequence, and every live
sequence's attention matches the fp64 oracle (max |do|, |dlse| <= 2e-3), also
for a batch made of a reordered subset of the slots.
"""
import math

import numpy as np
import pytest

import oracle as O
from synth import normal_bf16

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


def _decode(dk, cache, qbits, lens, theta):
    import torch
    d = qbits.shape[2]
    q = torch.from_numpy(qbits.view(np.int16)).cuda()
    qpos = torch.tensor([n - 1 for n in lens], dtype=torch.int32, device="cuda")
    o, lse, _ = dk.decode(cache, q, qpos, lens, 0.0, 1.0 / math.sqrt(d), theta)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def test_allocator_managed_cache_decode(dk):
    import torch
    from decode_attention_host_amd.cache_build import _append_rows
    hq, hkv, d, th, page, slots = 32, 8, 128, 5e5, 16, 4
    alloc = dk.PagedKVAllocator(hkv, d, n_host_pages=200, n_dev_pages=40, max_seqs=slots, max_pages=64,
                                host_fraction=0.8, page_size=page)
    rng = np.random.default_rng(7)
    dummy_lens = torch.zeros(slots, dtype=torch.int32, device="cuda")
    raw = {}
    lens = [0] * slots

    def admit(s, seed, target):
        raw[s] = (normal_bf16(seed, 2, (target, hkv, d)), normal_bf16(seed, 3, (target, hkv, d)), target)
        lens[s] = 0

    def grow(s, n_add):
        k, v, target = raw[s]
        new = min(target, lens[s] + n_add)
        if new == lens[s]:
            return
        alloc.reserve(s, new)
        _append_rows(alloc.pools, slots, s, lens[s], k[lens[s]:new], v[lens[s]:new], dummy_lens, 0.0, th)
        lens[s] = new

    try:
        for s, (seed, target) in enumerate([(90, 700), (91, 333), (92, 1000), (93, 64)]):
            admit(s, seed, target)
        for rnd in range(12):
            for s in range(slots):
                grow(s, int(rng.integers(1, 160)))
            if rnd == 4:  # slot 1 finishes early; its pages go to a new sequence
                alloc.release(1)
                admit(1, 94, 500)
        for s in range(slots):
            grow(s, 10 ** 6)
        st = alloc.stats()
        print("pager", st, "pages", [alloc.pages_of(s) for s in range(slots)], flush=True)
        assert lens == [raw[s][2] for s in range(slots)]
        host_pages = [int((alloc.table()[s, :alloc.pages_of(s)] & 1).sum()) for s in range(slots)]
        assert host_pages == [math.floor(0.8 * alloc.pages_of(s)) for s in range(slots)]
        torch.cuda.synchronize()

        qb = normal_bf16(95, 1, (slots, hq, d))
        o, lse = _decode(dk, alloc.batch(range(slots)), qb, lens, th)
        for s in range(slots):
            ro, rl = O.decode_sequence(qb[s], raw[s][0], raw[s][1], lens[s] - 1, th, 1.0 / math.sqrt(d))
            eo, el = np.abs(o[s] - ro).max(), np.abs(lse[s] - rl).max()
            print(f"slot {s}: L={lens[s]} max|do|={eo:.3g} max|dlse|={el:.3g}", flush=True)
            assert eo <= TOL and el <= TOL
        # a batch of a reordered subset of the slots
        sub = [2, 0]
        o2, l2 = _decode(dk, alloc.batch(sub), qb[sub], [lens[s] for s in sub], th)
        assert np.abs(o2 - o[sub]).max() < 1e-5 and np.abs(l2 - lse[sub]).max() < 1e-5
    finally:
        alloc.close()
