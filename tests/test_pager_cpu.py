"""The native paged KV allocator (dkv_pager_*) on the CPU: placement rule,
pool accounting, reuse, spill, all-or-nothing failures, and the slots the
page table gives every token (through the oracle's paged placement)."""
import ctypes as C
import math
import os

import numpy as np
import pytest

import oracle as O
from decode_attention_host_amd import _lib as dkv_lib


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dkv_lib.LIB_PATH):
        pytest.fail("libdkv.so is not built (python -m decode_attention_host_amd.build)")
    return dkv_lib.lib()


class Pager:
    def __init__(self, L, nh, nd, page, seqs, maxp, f):
        self.L = L
        self.h = C.c_void_p()
        assert L.dkv_pager_create(nh, nd, page, seqs, maxp, f, C.byref(self.h)) == dkv_lib.DKV_OK
        t, n = dkv_lib.PI32(), dkv_lib.PI32()
        assert L.dkv_pager_table(self.h, C.byref(t), C.byref(n)) == 0
        self.table = np.ctypeslib.as_array(t, shape=(seqs, maxp))
        self.npages = np.ctypeslib.as_array(n, shape=(seqs,))
        self.page, self.nh, self.nd = page, nh, nd

    def reserve(self, s, n):
        return self.L.dkv_pager_reserve(self.h, s, n)

    def release(self, s):
        return self.L.dkv_pager_release(self.h, s)

    def stats(self):
        st = dkv_lib.PagerStats()
        assert self.L.dkv_pager_stats_get(self.h, C.byref(st)) == 0
        return st.as_dict()

    def close(self):
        assert self.L.dkv_pager_destroy(self.h) == 0


def _check_consistent(p):
    """Every held page is in range and held once; counts match the stats."""
    seen = set()
    used = [0, 0]
    for s in range(p.table.shape[0]):
        n = int(p.npages[s])
        row = p.table[s]
        assert (row[n:] == -1).all()
        for e in row[:n]:
            e = int(e)
            assert e >= 0
            tier, phys = e & 1, e >> 1
            assert phys < (p.nh if tier else p.nd)
            assert (tier, phys) not in seen
            seen.add((tier, phys))
            used[tier] += 1
    st = p.stats()
    assert st["used_host_pages"] == used[1] and st["used_dev_pages"] == used[0]
    assert st["free_host_pages"] == p.nh - used[1] and st["free_dev_pages"] == p.nd - used[0]


@pytest.mark.parametrize("f", [0.0, 0.25, 0.5, 0.8, 0.9, 1.0])
def test_host_share_is_floor_of_fraction_at_every_length(L, f):
    p = Pager(L, 400, 400, 16, 2, 64, f)
    try:
        for n_tok in range(0, 64 * 16 + 1, 7):  # grow token by token (strided)
            assert p.reserve(0, n_tok) == 0
            n = int(p.npages[0])
            assert n == -(-n_tok // 16)
            host = int(((p.table[0, :n] & 1) == 1).sum())
            assert host == math.floor(f * n), (n_tok, n, host)
        # the rule is per logical page: page j is host iff floor(f(j+1)) > floor(f j)
        tiers = p.table[0, :64] & 1
        assert list(tiers) == [int(math.floor(f * (j + 1)) > math.floor(f * j)) for j in range(64)]
        assert p.stats()["spilled_pages"] == 0
        _check_consistent(p)
    finally:
        p.close()


def test_interleaved_growth_release_and_reuse(L):
    rng = np.random.default_rng(5)
    p = Pager(L, 300, 200, 32, 6, 40, 0.7)
    try:
        lens = [0] * 6
        for step in range(400):
            s = int(rng.integers(0, 6))
            if rng.random() < 0.08 and lens[s]:
                held = [int(e) for e in p.table[s, :p.npages[s]]]
                assert p.release(s) == 0
                lens[s] = 0
                # the next reserve of another slot takes the released pages
                # back in the same order (LIFO pools)
                other = (s + 1) % 6
                want = lens[other] + 32 * len(held)
                if want <= 40 * 32:
                    before = int(p.npages[other])
                    if p.reserve(other, want) == 0:
                        lens[other] = want
                        got = [int(e) for e in p.table[other, before:p.npages[other]]]
                        # same tier choices as the rule; pages of a tier come back in release order
                        for tier in (0, 1):
                            freed = [e >> 1 for e in held if e & 1 == tier]
                            taken = [e >> 1 for e in got if e & 1 == tier]
                            k = min(len(freed), len(taken))
                            assert taken[:k] == freed[:k]
            else:
                want = min(40 * 32, lens[s] + int(rng.integers(1, 200)))
                st = p.reserve(s, want)
                assert st in (dkv_lib.DKV_OK, dkv_lib.DKV_ERR_NOMEM)
                if st == 0:
                    lens[s] = want
            _check_consistent(p)
            for q in range(6):
                assert int(p.npages[q]) == -(-lens[q] // 32)
    finally:
        p.close()


def test_spill_to_the_other_pool_and_all_or_nothing(L):
    p = Pager(L, 3, 10, 16, 3, 32, 0.5)
    try:
        assert p.reserve(0, 16 * 8) == 0  # wants 4 host + 4 HBM pages; the host pool has 3
        st = p.stats()
        assert st["spilled_pages"] == 1
        assert st["used_host_pages"] == 3 and st["used_dev_pages"] == 5
        _check_consistent(p)
        snap = p.table.copy()
        # 5 free pages left: a request for 6 more fails and changes nothing
        assert p.reserve(1, 16 * 6) == dkv_lib.DKV_ERR_NOMEM
        assert b"free pages" in L.dkv_last_error()
        assert (p.table == snap).all() and p.stats()["used_dev_pages"] == 5
        assert p.reserve(1, 16 * 5) == 0
        assert p.stats()["free_host_pages"] == 0 and p.stats()["free_dev_pages"] == 0
        _check_consistent(p)
        assert p.release(0) == 0 and p.release(0) == 0  # releasing twice is harmless
        assert p.reserve(2, 1) == 0
        _check_consistent(p)
    finally:
        p.close()


def test_reserve_never_shrinks_and_rejects_bad_arguments(L):
    p = Pager(L, 8, 8, 16, 2, 4, 0.5)
    try:
        assert p.reserve(0, 40) == 0 and int(p.npages[0]) == 3
        assert p.reserve(0, 1) == 0 and int(p.npages[0]) == 3
        assert p.reserve(0, 4 * 16 + 1) == dkv_lib.DKV_ERR_INVALID  # beyond max_pages
        assert p.reserve(2, 1) == dkv_lib.DKV_ERR_INVALID  # slot out of range
        assert p.reserve(-1, 1) == dkv_lib.DKV_ERR_INVALID
        assert p.reserve(0, -1) == dkv_lib.DKV_ERR_INVALID
        assert p.release(5) == dkv_lib.DKV_ERR_INVALID
    finally:
        p.close()
    h = C.c_void_p()
    for args in [(-1, 4, 16, 1, 1, 0.5), (4, 4, 12, 1, 1, 0.5), (4, 4, 16, 0, 1, 0.5),
                 (4, 4, 16, 1, 0, 0.5), (4, 4, 16, 1, 1, 1.5), (4, 4, 16, 1, 1, float("nan")),
                 (1 << 30, 4, 1, 1, 1, 0.5), (1 << 27, 4, 32, 1, 1, 0.5)]:
        assert L.dkv_pager_create(*args, C.byref(h)) == dkv_lib.DKV_ERR_INVALID, args
    assert L.dkv_pager_create(4, 4, 16, 1, 1, 0.5, None) == dkv_lib.DKV_ERR_INVALID
    assert L.dkv_pager_reserve(None, 0, 1) == dkv_lib.DKV_ERR_INVALID


def test_token_slots_through_the_oracle_placement(L):
    # every token of every held page maps (oracle paged_slot) to a distinct
    # row inside its pool; the tier of a token is its page's tier
    page = 16
    p = Pager(L, 64, 64, page, 4, 16, 0.8)
    try:
        lens = [1, 37, 200, 256]
        for s, n in enumerate(lens):
            assert p.reserve(s, n) == 0
        rows = {}
        for s, n in enumerate(lens):
            for t in range(n):
                tier, row = O.paged_slot(p.table, s, t, page)
                assert 0 <= row < (p.nh if tier else p.nd) * page
                assert (tier, row) not in rows
                rows[(tier, row)] = (s, t)
                assert tier == int(p.table[s, t // page]) & 1
        assert len(rows) == sum(lens)
    finally:
        p.close()
