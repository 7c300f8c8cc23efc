"""Prefill planner on the CPU (through dkv_prefill_plan_inspect, no HIP call).

Every query row must see each token of [0, its block's last position] exactly
once, at the pool row the placement gives (host, HBM, or the HBM staging copy
of host rows, whose copy list must map back to the right host rows); split
slots must be a bijection onto [0, num_splits) that agrees with the CSR
offsets.  Placement is checked against the oracle's own slot formulas.
"""
import numpy as np
import pytest

import oracle as O
from synth import paged_table

dkv_lib = pytest.importorskip("decode_attention_host_amd._lib")
from decode_attention_host_amd.api import prefill_plan_inspect, reset_tuning, set_tuning  # noqa: E402

FAKE = 1 << 40
QROWS = 128  # query-head rows per row block


@pytest.fixture(scope="module")
def L():
    try:
        return dkv_lib.lib()
    except OSError as e:
        pytest.fail(f"libdkv.so must be built first: {e}")


def desc(hkv, d, page=0, max_pages=0, host_rows=1 << 20, dev_rows=1 << 20, hs=1 << 16, ds=1 << 16, pt=None):
    x = dkv_lib.KvDesc()
    x.num_kv_heads, x.head_dim, x.page_size, x.max_pages = hkv, d, page, max_pages
    x.host_stride, x.dev_stride, x.host_rows, x.dev_rows = hs, ds, host_rows, dev_rows
    x.host_k, x.host_v, x.dev_k, x.dev_v = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    if pt is not None:
        x.page_table = FAKE + (4 << 30)
        x._pt = pt
        x.page_table_host = pt.ctypes.data
    return x


def _check(plan, lens, news, hq, hkv, slot_of, stage_src, fused=False):
    """slot_of(b, t) -> (pool 0/1, row); stage_src: staging row -> host row.
    fused: tokens at or after a sequence's first new row come from pool 3 (the
    new rows, in query-row order)."""
    items, offs, info = plan["items"], plan["split_offsets"], plan["info"]
    G = hq // hkv
    QB = QROWS // G
    q_start = np.concatenate([[0], np.cumsum(news)])
    T = int(q_start[-1])
    assert len(offs) == T + 1 and offs[-1] == info["num_splits"]
    by_block = {}
    for it in items:
        by_block.setdefault((int(it[1]), int(it[2])), []).append(it)
    slots = set()
    for b, (L_b, n) in enumerate(zip(lens, news)):
        p0 = L_b - n
        for r0 in range(0, n, QB):
            row0 = int(q_start[b] + r0)
            blk = by_block.pop((b, row0))
            n_rows = min(QB, n - r0)
            end = p0 + r0 + n_rows
            S_k = len(blk)
            seen = {}
            for it in blk:
                pool, _, _, nr, pos0, ntok, first, tok0, sidx, nspl, base = (int(v) for v in it)
                assert nr == n_rows and pos0 == p0 + r0 and nspl == S_k and 0 <= sidx < S_k
                assert ntok >= 1
                for r in range(n_rows):
                    assert offs[row0 + r] == base + r * S_k
                    s = base + r * S_k + sidx
                    assert s not in slots
                    slots.add(s)
                for k in range(ntok):
                    if pool == 3:
                        t, row = tok0 + k, first + k
                        assert fused and t >= p0 and row == q_start[b] + (t - p0), (b, t)
                        assert t not in seen
                        seen[t] = 1
                        continue
                    if plan["paged"]:
                        P = plan["P"]
                        lp, pp = plan["pages"][2 * (first + k // P)], plan["pages"][2 * (first + k // P) + 1]
                        t, row = int(lp) * P + k % P, int(pp) * P + k % P
                    else:
                        t, row = tok0 + k, first + k
                    assert t not in seen, (b, row0, t)
                    assert not fused or t < p0, (b, t)
                    seen[t] = 1
                    tier, want = slot_of(b, t)
                    if pool == 2:
                        assert tier == 1 and stage_src[row] == want, (b, t)
                    else:
                        assert pool == (0 if tier == 1 else 1) and row == want, (b, t, pool)
            assert sorted(seen) == list(range(end)), (b, row0)
    assert not by_block
    assert slots == set(range(info["num_splits"]))


def _stage_map(plan):
    m = {}
    for src, dst, n in plan["tiles"]:
        for i in range(int(n)):
            assert int(dst) + i not in m
            m[int(dst) + i] = int(src) + i
    return m


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 8, 64), (16, 2, 64), (8, 4, 128)])
@pytest.mark.parametrize("ratio", [0.0, 0.3, 1.0])
@pytest.mark.parametrize("stage", [True, False])
@pytest.mark.parametrize("fused", [False, True])
def test_prefill_plan_contiguous(L, hq, hkv, d, ratio, stage, fused):
    lens, news = [64, 377, 33, 1000, 200], [64, 77, 1, 130, 200]
    hs, ds = 1024, 1001  # unequal: a host/device stride swap moves rows
    x = desc(hkv, d, host_rows=len(lens) * hs, dev_rows=len(lens) * ds, hs=hs, ds=ds)
    try:
        set_tuning(stage_max_mib=0 if stage else -1)
        plan = prefill_plan_inspect(x, len(lens), hq, np.concatenate([[0], np.cumsum(news)]),
                                    [a - n for a, n in zip(lens, news)], lens, ratio, 16, fused=fused)
    finally:
        reset_tuning()
    plan["paged"] = False

    def slot_of(b, t):
        return O.contig_slot(b, t, lens[b], ratio, hs, ds)

    _check(plan, lens, news, hq, hkv, slot_of, _stage_map(plan), fused)
    G = hq // hkv
    nblk = [-(-n // (QROWS // G)) for n in news]
    # staged: host rows below the first new row (fused) or below the last row
    staged_rows = sum(min(O.contig_split_point(ratio, a), a - n if fused else a)
                      for a, n, k in zip(lens, news, nblk) if k >= 2)
    assert plan["info"]["staged_bytes"] == (staged_rows * hkv * d * 4 if stage else 0)
    if stage:
        assert sum(int(t[2]) for t in plan["tiles"]) == staged_rows
    else:
        assert len(plan["tiles"]) == 0


@pytest.mark.parametrize("stage", [True, False])
@pytest.mark.parametrize("fused", [False, True])
def test_prefill_plan_paged(L, stage, fused):
    lens, news, hq, hkv, d = [500, 17, 1200, 40], [100, 17, 333, 1], 32, 8, 128
    pt, nh, nd = paged_table(80, lens, 16, 0.8)
    x = desc(hkv, d, page=16, max_pages=pt.shape[1], host_rows=nh * 16, dev_rows=nd * 16, pt=pt)
    try:
        set_tuning(stage_max_mib=0 if stage else -1)
        plan = prefill_plan_inspect(x, len(lens), hq, np.concatenate([[0], np.cumsum(news)]),
                                    [a - n for a, n in zip(lens, news)], lens, 0.0, 16, fused=fused)
    finally:
        reset_tuning()
    plan["paged"], plan["P"] = True, 16

    def slot_of(b, t):
        return O.paged_slot(pt, b, t, 16)

    _check(plan, lens, news, hq, hkv, slot_of, _stage_map(plan), fused)
    assert (plan["info"]["staged_bytes"] > 0) == stage   # sequences 0 and 2 span several blocks


def test_prefill_plan_staging_budget(L):
    # two sequences of 4096 all-host tokens, 16 heads x 128 dims: 32 MiB of K+V each
    lens, news, hq, hkv, d = [4096, 4096], [4096, 4096], 32, 16, 128
    x = desc(hkv, d, host_rows=2 * 4096, dev_rows=1, hs=4096, ds=0)
    q0 = np.array([0, 4096, 8192])
    try:
        set_tuning(stage_max_mib=40)   # room for one sequence only
        plan = prefill_plan_inspect(x, 2, hq, q0, [0, 0], lens, 1.0, 16)
    finally:
        reset_tuning()
    per = 4096 * hkv * d * 4
    assert plan["info"]["staged_bytes"] == per
    assert {int(it[0]) for it in plan["items"] if it[1] == 0} == {2}
    assert {int(it[0]) for it in plan["items"] if it[1] == 1} == {0}
    assert plan["info"]["workspace_bytes"] >= per


def test_prefill_plan_rejects_bad_rows(L):
    x = desc(8, 128)
    with pytest.raises(dkv_lib.DkvError):
        prefill_plan_inspect(x, 1, 32, [0, 10], [95], [100], 0.5, 16)   # rows past the cache
    with pytest.raises(dkv_lib.DkvError):
        prefill_plan_inspect(x, 1, 32, [1, 10], [0], [100], 0.5, 16)    # q_start[0] != 0
    with pytest.raises(dkv_lib.DkvError):
        prefill_plan_inspect(x, 1, 24, [0, 10], [0], [100], 0.5, 16)    # group size 3
