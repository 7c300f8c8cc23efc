"""CPU tests of the C ABI: exports, argument validation and the split planner.

No GPU work happens here: the planner is reached through dkv_plan_inspect,
which runs without HIP, and every validation failure returns before any HIP
call.  The expected placements come from the oracle's placement functions.
"""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import oracle as O
from synth import paged_table

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

dkv_lib = pytest.importorskip("decode_attention_host_amd._lib")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dkv_lib.LIB_PATH):
        pytest.fail("libdkv.so is not built (python -m decode_attention_host_amd.build)")
    return dkv_lib.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "dkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dkv_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_function_is_exported_and_bound(L):
    names = header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), f"{n} declared in dkv.h but not exported"
        assert n in dkv_lib.SIGNATURES, f"{n} has no ctypes signature"
    assert set(dkv_lib.SIGNATURES) == set(names)


def _c_layout(struct, fields):
    """sizeof and offsetof of a struct of include/dkv.h, from the C compiler."""
    import shutil
    import subprocess
    import tempfile
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler to read the header's layout")
    src = "#include <stddef.h>\n#include <stdio.h>\n#include \"dkv.h\"\nint main(void){\n"
    src += f'printf("%zu\\n", sizeof({struct}));\n'
    for f in fields:
        src += f'printf("%zu\\n", offsetof({struct}, {f}));\n'
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        with open(os.path.join(d, "l.c"), "w") as fh:
            fh.write(src)
        subprocess.run([cc, "-I", os.path.join(ROOT, "include"), os.path.join(d, "l.c"), "-o",
                        os.path.join(d, "l")], check=True)
        out = subprocess.run([os.path.join(d, "l")], check=True, capture_output=True, text=True).stdout
    v = [int(x) for x in out.split()]
    return v[0], v[1:]


@pytest.mark.parametrize("struct,cls", [("dkv_kv_desc", "KvDesc"), ("dkv_plan_info", "PlanInfo"),
                                        ("dkv_tuning", "Tuning"), ("dkv_bw_result", "BwResult"),
                                        ("dkv_pager_stats", "PagerStats")])
def test_struct_layouts_match_header(struct, cls):
    t = getattr(dkv_lib, cls)
    names = [n for n, _ in t._fields_]
    size, offs = _c_layout(struct, names)
    assert C.sizeof(t) == size
    assert [getattr(t, n).offset for n in names] == offs


def test_version_and_last_error(L):
    assert L.dkv_version() >= 10000
    out = C.c_int64()
    assert L.dkv_split_point(1.5, 10, C.byref(out)) == dkv_lib.DKV_ERR_INVALID
    assert b"offload_ratio" in L.dkv_last_error()
    assert L.dkv_split_point(0.5, 10, C.byref(out)) == dkv_lib.DKV_OK
    assert L.dkv_last_error() == b""


def test_split_point_matches_oracle_and_golden(L, golden):
    out = C.c_int64()
    for c in golden["split_point"]["cases"]:
        assert L.dkv_split_point(c["r"], c["L"], C.byref(out)) == 0
        assert out.value == c["n_host"], c["why"]
    rng = np.random.default_rng(0)
    for _ in range(2000):
        r = float(rng.random()); n = int(rng.integers(0, 1 << 22))
        assert L.dkv_split_point(r, n, C.byref(out)) == 0
        assert out.value == O.contig_split_point(r, n)
    assert L.dkv_split_point(float("nan"), 5, C.byref(out)) == dkv_lib.DKV_ERR_INVALID
    assert L.dkv_split_point(-0.1, 5, C.byref(out)) == dkv_lib.DKV_ERR_INVALID
    assert L.dkv_split_point(0.5, -1, C.byref(out)) == dkv_lib.DKV_ERR_INVALID


FAKE = 1 << 40  # aligned stand-in addresses: never dereferenced on the CPU


def desc(hkv=8, d=128, page=0, max_pages=0, host_rows=1 << 20, dev_rows=1 << 20, hs=1 << 16,
         ds=1 << 16, pt=None):
    x = dkv_lib.KvDesc()
    x.num_kv_heads, x.head_dim, x.page_size, x.max_pages = hkv, d, page, max_pages
    x.host_stride, x.dev_stride, x.host_rows, x.dev_rows = hs, ds, host_rows, dev_rows
    x.host_k, x.host_v, x.dev_k, x.dev_v = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    if pt is not None:
        x.page_table = FAKE + (4 << 30)
        x._pt = pt
        x.page_table_host = pt.ctypes.data
    return x


def inspect(L, x, batch, hq, lens, ratio, cus=256):
    from decode_attention_host_amd.api import plan_inspect
    return plan_inspect(x, batch, hq, lens, ratio, cus)


def test_validation_errors_before_any_hip_call(L):
    info = dkv_lib.PlanInfo()
    lens = np.array([100], dtype=np.int32)
    bad = desc(d=96)
    assert L.dkv_decode_plan(C.byref(bad), 1, 8, lens.ctypes.data, 1.0, C.byref(info)) == dkv_lib.DKV_ERR_UNSUPPORTED
    x = desc()
    # group size 3 not built
    assert L.dkv_decode_plan(C.byref(desc(hkv=2)), 1, 6, lens.ctypes.data, 1.0, C.byref(info)) == dkv_lib.DKV_ERR_UNSUPPORTED
    # Hq not a multiple of Hkv
    assert L.dkv_decode_plan(C.byref(x), 1, 12, lens.ctypes.data, 1.0, C.byref(info)) == dkv_lib.DKV_ERR_INVALID
    # ratio outside [0, 1]
    assert L.dkv_decode_plan(C.byref(x), 1, 32, lens.ctypes.data, 1.5, C.byref(info)) == dkv_lib.DKV_ERR_INVALID
    # page size not a power of two
    assert L.dkv_decode_plan(C.byref(desc(page=24, max_pages=4)), 1, 32, lens.ctypes.data, 0.0,
                             C.byref(info)) == dkv_lib.DKV_ERR_INVALID
    # attention call: missing buffers
    assert L.dkv_decode_attn_split(C.byref(x), 1, 32, FAKE, None, lens.ctypes.data, 1.0, 0.1, 1e4,
                                   FAKE, 1 << 20, FAKE, FAKE, FAKE, 10, None) == dkv_lib.DKV_ERR_INVALID
    # unaligned workspace
    assert L.dkv_decode_attn_split(C.byref(x), 1, 32, FAKE, FAKE, lens.ctypes.data, 1.0, 0.1, 1e4,
                                   FAKE + 8, 1 << 20, FAKE, FAKE, FAKE, 10, None) == dkv_lib.DKV_ERR_INVALID
    # theta must be > 0
    assert L.dkv_decode_attn_split(C.byref(x), 1, 32, FAKE, FAKE, lens.ctypes.data, 1.0, 0.1, 0.0,
                                   FAKE, 1 << 20, FAKE, FAKE, FAKE, 10, None) == dkv_lib.DKV_ERR_INVALID
    # merge: head_dim not built, batch < 1
    assert L.dkv_merge_lse(FAKE, FAKE, FAKE, 1, 4, 80, FAKE, None, None) == dkv_lib.DKV_ERR_UNSUPPORTED
    assert L.dkv_merge_lse(FAKE, FAKE, FAKE, 0, 4, 64, FAKE, None, None) == dkv_lib.DKV_ERR_INVALID
    assert L.dkv_merge_lse(None, FAKE, FAKE, 1, 4, 64, FAKE, None, None) == dkv_lib.DKV_ERR_INVALID
    # append: hidden not a multiple of 256, missing k/v, bad ratio
    assert L.dkv_project_rope_append(C.byref(x), 1, FAKE, 0.5, 4, FAKE, FAKE, FAKE, 100, FAKE, FAKE,
                                     None, None, 1e4, FAKE, 1 << 20, None) == dkv_lib.DKV_ERR_UNSUPPORTED
    assert L.dkv_project_rope_append(C.byref(x), 1, FAKE, 0.5, 4, FAKE, FAKE, None, 0, None, None,
                                     None, None, 1e4, None, 0, None) == dkv_lib.DKV_ERR_INVALID
    assert L.dkv_project_rope_append(C.byref(x), 1, FAKE, 2.0, 4, FAKE, FAKE, None, 0, None, None,
                                     FAKE, FAKE, 1e4, None, 0, None) == dkv_lib.DKV_ERR_INVALID
    # projection workspace too small
    assert L.dkv_project_rope_append(C.byref(x), 1, FAKE, 0.5, 16, FAKE, FAKE, FAKE, 4096, FAKE, FAKE,
                                     None, None, 1e4, FAKE, 1024, None) == dkv_lib.DKV_ERR_INVALID
    # n_new == 0 is a no-op success
    assert L.dkv_project_rope_append(C.byref(x), 1, FAKE, 0.5, 0, None, None, None, 0, None, None,
                                     None, None, 1e4, None, 0, None) == dkv_lib.DKV_OK
    # host allocation arguments
    h, d = C.c_void_p(), C.c_void_p()
    assert L.dkv_host_alloc(0, 0, C.byref(h), C.byref(d)) == dkv_lib.DKV_ERR_INVALID
    assert L.dkv_host_alloc(16, 7, C.byref(h), C.byref(d)) == dkv_lib.DKV_ERR_INVALID
    # tuning
    t = dkv_lib.Tuning(); t.host_wgs = -1
    assert L.dkv_set_tuning(C.byref(t)) == dkv_lib.DKV_ERR_INVALID
    t = dkv_lib.Tuning(); t.writer_wgs = -1
    assert L.dkv_set_tuning(C.byref(t)) == dkv_lib.DKV_ERR_INVALID
    t = dkv_lib.Tuning(); t.reserved = 1
    assert L.dkv_set_tuning(C.byref(t)) == dkv_lib.DKV_ERR_INVALID
    t = dkv_lib.Tuning(); t.writer_wgs = 16
    assert L.dkv_set_tuning(C.byref(t)) == dkv_lib.DKV_OK
    got = dkv_lib.Tuning()
    assert L.dkv_get_tuning(C.byref(got)) == dkv_lib.DKV_OK and got.writer_wgs == 16
    assert L.dkv_set_tuning(None) == dkv_lib.DKV_OK


def test_append_workspace_size(L):
    assert L.dkv_append_workspace_bytes(16, 4096, 1024) >= 16 * 2048 * 4 * (4096 // 256 + 1)
    assert L.dkv_append_workspace_bytes(0, 4096, 1024) == 0


def _check_contig_cover(items, offs, lens, ratio, hs, ds):
    # every token of every sequence appears in exactly one item, in the tier
    # and row the placement gives
    seen = {}
    for tier, b, slot, ntok, first in items:
        assert ntok >= 1
        nh = O.contig_split_point(ratio, lens[b])
        t0 = first - b * hs if tier else first - b * ds + nh
        for t in range(t0, t0 + ntok):
            exp_tier, exp_row = O.contig_slot(int(b), int(t), int(lens[b]), ratio, hs, ds)
            assert exp_tier == tier and exp_row == first + (t - t0)
            assert (b, t) not in seen
            seen[(b, t)] = slot
    assert len(seen) == sum(lens)
    slots = sorted(set(int(s) for s in items[:, 2]))
    assert slots == list(range(len(items)))
    for b in range(len(lens)):
        bs = [int(s) for tier, bb, s, _, _ in items if bb == b]
        assert sorted(bs) == list(range(offs[b], offs[b + 1]))


@pytest.mark.parametrize("ratio", [0.0, 0.25, 0.5, 0.9, 1.0])
def test_planner_contiguous_coverage(L, ratio):
    lens = [1, 63, 64, 65, 1000, 4097]
    # unequal strides: a host/device stride swap in the planner moves rows
    hs, ds = 8192, 4099
    x = desc(hkv=2, d=64, host_rows=len(lens) * hs, dev_rows=len(lens) * ds, hs=hs, ds=ds)
    items, _, offs, info = inspect(L, x, len(lens), 8, lens, ratio, cus=8)
    _check_contig_cover(items, offs, lens, ratio, hs, ds)
    assert info["num_splits"] == len(items) == offs[-1]
    n_host = sum(O.contig_split_point(ratio, n) for n in lens)
    assert info["host_bytes"] == n_host * 2 * 64 * 2 * 2
    assert info["dev_bytes"] == (sum(lens) - n_host) * 2 * 64 * 2 * 2
    if ratio == 0.0:
        assert info["host_items"] == 0 and info["host_wgs"] == 0
    if ratio == 1.0:
        assert info["dev_items"] == 0 and info["dev_wgs"] == 0


def test_planner_paged_coverage_and_tiers(L):
    lens = [1, 16, 17, 300, 1025]
    pt, nh, nd = paged_table(1, lens, 16, 0.8)
    x = desc(hkv=8, d=128, page=16, max_pages=pt.shape[1], host_rows=nh * 16, dev_rows=nd * 16, pt=pt)
    items, plist, offs, info = inspect(L, x, len(lens), 32, lens, 0.0, cus=16)
    seen = set()
    for tier, b, slot, ntok, first in items:
        npg = (ntok + 15) // 16
        pages = plist[first:first + npg]
        tot = 0
        for k, j in enumerate(pages):
            e = int(pt[b, j])
            assert (e & 1) == tier
            nt = min(16, lens[b] - 16 * int(j))
            if k < npg - 1:
                assert nt == 16  # only an item's last page may be partial
            tot += nt
            for t in range(16 * int(j), 16 * int(j) + nt):
                assert (b, t) not in seen
                seen.add((b, t))
        assert tot == ntok
    assert len(seen) == sum(lens)
    assert offs[-1] == info["num_splits"]


def test_planner_workgroup_split_follows_bandwidth(L):
    lens = [1 << 16]
    x = desc(hkv=8, d=128)
    from decode_attention_host_amd.api import reset_tuning, set_tuning
    try:
        set_tuning(host_bw_gbs=50.0, dev_bw_gbs=5000.0, host_wgs=8)
        _, _, _, i1 = inspect(L, x, 1, 32, lens, 0.5, cus=256)
        set_tuning(host_bw_gbs=500.0, dev_bw_gbs=5000.0, host_wgs=8)
        _, _, _, i2 = inspect(L, x, 1, 32, lens, 0.5, cus=256)
    finally:
        reset_tuning()
    assert i1["host_wgs"] >= 8 and i2["host_wgs"] > i1["host_wgs"]
    assert i1["dev_wgs"] > i1["host_wgs"]


def test_planner_rejects_layout_overflow(L):
    x = desc(hkv=8, d=128, host_rows=100, dev_rows=100, hs=100, ds=100)
    from decode_attention_host_amd.api import plan_inspect
    with pytest.raises(dkv_lib.DkvError):
        plan_inspect(x, 1, 32, [300], 0.5, 8)   # 150 host rows needed > 100
    pt = np.array([[3 << 1 | 1, -1]], dtype=np.int32)
    xp = desc(hkv=8, d=128, page=16, max_pages=2, host_rows=32, dev_rows=32, pt=pt)
    with pytest.raises(dkv_lib.DkvError):
        plan_inspect(xp, 1, 32, [10], 0.0, 8)   # host page 3 beyond a 2-page pool
    with pytest.raises(dkv_lib.DkvError):
        plan_inspect(xp, 1, 32, [20], 0.0, 8)   # second page unmapped
    with pytest.raises(dkv_lib.DkvError):
        plan_inspect(xp, 1, 32, [40], 0.0, 8)   # 3 pages > max_pages


def _ranges_cover(items, lens, ratio, hs, ds):
    # item token ranges tile [0, L_b) of every sequence exactly once
    per = {b: [] for b in range(len(lens))}
    for tier, b, slot, ntok, first in items:
        nh = O.contig_split_point(ratio, lens[b])
        t0 = first - b * hs if tier else first - b * ds + nh
        per[int(b)].append((int(t0), int(ntok), int(tier)))
    for b, rs in per.items():
        rs.sort()
        t = 0
        nh = O.contig_split_point(ratio, lens[b])
        for t0, n, tier in rs:
            assert t0 == t and n >= 1 and tier == (1 if t0 < nh else 0) and (t0 + n <= nh or t0 >= nh)
            t += n
        assert t == lens[b]


def test_planner_guided_tail_contiguous(L):
    # long HBM ranges: the last part of each sequence is cut into smaller
    # units that come last in the HBM work list; coverage is unchanged
    lens = [1 << 20, 200000]
    hs = ds = 1 << 20
    x = desc(hkv=8, d=128, host_rows=0, dev_rows=2 * ds, hs=hs, ds=ds)
    items, _, offs, info = inspect(L, x, 2, 32, lens, 0.0, cus=256)
    _ranges_cover(items, lens, 0.0, hs, ds)
    assert info["num_splits"] == len(items) == offs[-1]
    for b in range(len(lens)):
        assert sorted(int(s) for _, bb, s, _, _ in items if bb == b) == list(range(offs[b], offs[b + 1]))
    ntok = items[:, 3]
    big = int(info["dev_chunk"])
    small = ntok < big // 2
    assert small.any() and (~small).any()
    first_small = int(np.argmax(small))
    assert small[first_small:].all()                    # the small units come last
    assert int(ntok[small].max()) <= (big // 4 + 63) // 64 * 64
    # about two small units per HBM workgroup
    n_small_units = int(small.sum()) * 8
    assert info["dev_wgs"] <= n_small_units <= 4 * info["dev_wgs"]


def test_planner_guided_tail_paged(L):
    lens = [1 << 20]
    npg = (1 << 20) // 16
    perm = np.random.default_rng(1).permutation(npg).astype(np.int32)
    pt = (perm << 1)[None, :].copy()
    x = desc(hkv=8, d=128, page=16, max_pages=npg, host_rows=16, dev_rows=npg * 16, pt=pt)
    items, plist, offs, info = inspect(L, x, 1, 32, lens, 0.0, cus=256)
    covered = np.zeros(npg, dtype=np.int32)
    for tier, b, slot, ntok, first in items:
        assert tier == 0 and ntok % 16 == 0
        covered[plist[first:first + ntok // 16]] += 1
    assert (covered == 1).all()
    ntok = items[:, 3]
    small = ntok < int(info["dev_chunk"]) // 2
    assert small.any() and small[int(np.argmax(small)):].all()


def test_planner_no_guided_tail_when_units_are_small(L):
    lens = [32768]
    x = desc(hkv=8, d=128, host_rows=0, dev_rows=1 << 15, hs=1 << 15, ds=1 << 15)
    items, _, offs, info = inspect(L, x, 1, 32, lens, 0.0, cus=256)
    assert set(int(n) for n in items[:, 3]) == {int(info["dev_chunk"])}


def test_decode_batch_bound(L):
    # the decode kernel derives items for up to 512 sequences (per-sequence
    # prefixes in LDS): 512 plans, 513 is refused before any HIP call
    x = desc(hkv=2, d=64, host_rows=513 * 1024, dev_rows=513 * 1024, hs=1024, ds=1024)
    lens = np.full(513, 100, dtype=np.int32)
    from decode_attention_host_amd.api import set_tuning, reset_tuning
    try:
        set_tuning(num_cus=256)
        info = dkv_lib.PlanInfo()
        assert L.dkv_decode_plan(C.byref(x), 512, 8, lens.ctypes.data, 0.5, C.byref(info)) == dkv_lib.DKV_OK
        assert info.num_splits >= 512
        assert L.dkv_decode_plan(C.byref(x), 513, 8, lens.ctypes.data, 0.5, C.byref(info)) == \
            dkv_lib.DKV_ERR_UNSUPPORTED
        assert L.dkv_decode_step_plan(C.byref(x), 512, 8, 0.5, 0, C.byref(info)) == dkv_lib.DKV_OK
        assert L.dkv_decode_step_plan(C.byref(x), 513, 8, 0.5, 0, C.byref(info)) == dkv_lib.DKV_ERR_UNSUPPORTED
    finally:
        reset_tuning()


def test_staged_plan_layout_and_validation(L):
    """dkv_decode_staged_plan (host only): chunks of the host tier, bytes
    staged into HBM, a workspace that holds the two-slot ring; paged layouts,
    chunk sizes off the 64-token grid and rows beyond the layout are refused."""
    from decode_attention_host_amd.api import set_tuning, reset_tuning
    hkv, d, hq = 8, 128, 32
    row = hkv * d * 2
    try:
        set_tuning(num_cus=256)
        x = desc(hkv=hkv, d=d, host_rows=1 << 16, dev_rows=1 << 16, hs=1 << 16, ds=1 << 16)
        info = dkv_lib.PlanInfo()
        for L_, r, chunk in [(5000, 0.6, 1024), (3000, 1.0, 64), (777, 0.0, 256), (40000, 0.25, 4096)]:
            assert L.dkv_decode_staged_plan(C.byref(x), hq, L_, r, chunk, C.byref(info)) == dkv_lib.DKV_OK
            nh = O.contig_split_point(r, L_)
            assert info.host_items == -(-nh // chunk)
            assert info.staged_bytes == nh * row * 2
            assert info.host_bytes == nh * row * 2 and info.dev_bytes == (L_ - nh) * row * 2
            assert info.workspace_bytes >= 4 * chunk * row  # two ring slots of K and of V
        assert L.dkv_decode_staged_plan(C.byref(x), hq, 5000, 0.5, 100, C.byref(info)) == dkv_lib.DKV_ERR_INVALID
        assert L.dkv_decode_staged_plan(C.byref(x), hq, 0, 0.5, 1024, C.byref(info)) == dkv_lib.DKV_ERR_INVALID
        assert L.dkv_decode_staged_plan(C.byref(x), hq, 1 << 20, 0.5, 1024, C.byref(info)) == dkv_lib.DKV_ERR_INVALID
        pt = np.zeros((1, 4), dtype=np.int32)
        xp = desc(hkv=hkv, d=d, page=16, max_pages=4, host_rows=64, dev_rows=64, pt=pt)
        assert L.dkv_decode_staged_plan(C.byref(xp), hq, 64, 0.5, 64, C.byref(info)) == dkv_lib.DKV_ERR_UNSUPPORTED
    finally:
        reset_tuning()


def test_plan_cache_stats_and_release_without_a_gpu(L):
    # nothing is captured without a GPU, and releasing captured plans then
    # drops nothing (the cache is within its capacity) and makes no HIP call
    n, k, b = C.c_int32(-1), C.c_int32(-1), C.c_int64(-1)
    assert L.dkv_plan_cache_stats(C.byref(n), C.byref(k), C.byref(b)) == dkv_lib.DKV_OK
    assert k.value == 0 and 0 <= n.value <= 64 and b.value >= 0
    assert L.dkv_plan_cache_release_captured() == dkv_lib.DKV_OK
    assert L.dkv_plan_cache_stats(None, C.byref(k), C.byref(b)) == dkv_lib.DKV_ERR_INVALID
