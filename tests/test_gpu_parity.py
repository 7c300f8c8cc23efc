"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bar (fp32 outputs from bf16 inputs with fp32 accumulation): max |o - o_ref|
<= 2e-3 and max |lse - lse_ref| <= 2e-3; page-table / append indexing
bit-exact; appended K within one bf16 ulp of bf16(RoPE(k)) and V bit-exact.
Shapes span several 64-token tiles plus a ragged tail, both tiers, every
built group size and head dim, and the degenerate cases of the method.
"""
import math

import numpy as np
import pytest

import oracle as O
from synth import normal_bf16, paged_table, ragged_lengths

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


def _raw(seed, lens, hkv, d, tid_k=2, tid_v=3):
    ks, vs = [], []
    for b, n in enumerate(lens):
        ks.append(normal_bf16(seed * 1000 + b, tid_k, (n, hkv, d)))
        vs.append(normal_bf16(seed * 1000 + b, tid_v, (n, hkv, d)))
    return ks, vs


def _q(seed, B, hq, d):
    return normal_bf16(seed, 1, (B, hq, d))


def _run_decode(dk, cache, qbits, lens, ratio, theta, q_pos=None):
    import torch
    B, hq, d = qbits.shape
    q = torch.from_numpy(qbits.view(np.int16)).cuda()
    qp = np.asarray([n - 1 for n in lens] if q_pos is None else q_pos, dtype=np.int32)
    qpos = torch.from_numpy(qp).cuda()
    o, lse, bufs = dk.decode(cache, q, qpos, lens, ratio, 1.0 / math.sqrt(d), theta)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), bufs


def _oracle(qbits, ks, vs, lens, theta, q_pos=None, key_positions=None):
    B, hq, d = qbits.shape
    outs, lses = [], []
    for b in range(B):
        qp = lens[b] - 1 if q_pos is None else q_pos[b]
        o, l = O.decode_sequence(qbits[b], ks[b], vs[b], qp, theta, 1.0 / math.sqrt(d),
                                 key_positions=None if key_positions is None else key_positions[b])
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def _assert_close(o, lse, o_ref, l_ref, tol=TOL):
    eo = np.abs(o - o_ref).max()
    el = np.abs(lse - l_ref).max()
    assert eo <= tol and el <= tol, f"max|do|={eo:.3g} max|dlse|={el:.3g}"
    return eo, el


# ----------------------------------------------------------------------- contiguous

CASES = [
    # (lens, hq, hkv, d, ratio, theta)
    ([512], 4, 2, 64, 1.0, 1e4),                 # the tiny workload
    ([1], 4, 2, 64, 1.0, 1e4),                   # single token
    ([1], 8, 8, 128, 0.0, 1e4),
    ([65], 8, 1, 128, 0.5, 5e5),                 # g = 8, ragged tail
    ([300, 1, 129], 8, 4, 64, 0.3, 1e4),         # g = 2, ragged batch
    ([1000, 777], 32, 8, 128, 0.75, 5e5),        # g = 4
    ([640, 2049], 16, 16, 128, 0.5, 1e4),        # MHA
    ([4096], 32, 8, 128, 0.0, 5e5),              # HBM only
    ([4096], 32, 8, 128, 1.0, 5e5),              # host only
    ([5000, 63, 64], 16, 4, 64, 0.9, 1e4),
    ([3000, 10], 16, 2, 64, 0.4, 1e4),           # g = 8, D = 64
    ([1500], 8, 8, 64, 0.6, 1e4),                # MHA, D = 64
    ([2500, 700], 16, 8, 128, 0.2, 5e5),         # g = 2, D = 128
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_contiguous_parity(dk, case):
    lens, hq, hkv, d, ratio, theta = CASES[case]
    ks, vs = _raw(10 + case, lens, hkv, d)
    qb = _q(10 + case, len(lens), hq, d)
    from decode_attention_host_amd.cache_build import contiguous_cache
    cache = contiguous_cache(hkv, d, lens, ratio, ks, vs, theta)
    o, lse, bufs = _run_decode(dk, cache, qb, lens, ratio, theta)
    o_ref, l_ref = _oracle(qb, ks, vs, lens, theta)
    _assert_close(o, lse, o_ref, l_ref)
    cache.free()


def test_single_token_returns_v0_exactly(dk):
    lens, hq, hkv, d = [1, 1], 8, 2, 128
    ks, vs = _raw(3, lens, hkv, d)
    qb = _q(3, 2, hq, d)
    from decode_attention_host_amd.cache_build import contiguous_cache
    for ratio in (0.0, 1.0):
        cache = contiguous_cache(hkv, d, lens, ratio, ks, vs, 1e4)
        o, lse, _ = _run_decode(dk, cache, qb, lens, ratio, 1e4)
        for b in range(2):
            for h in range(hq):
                assert np.array_equal(o[b, h], O.bf16_to_f64(vs[b][0, h // 4]))
        cache.free()


def test_identical_keys_give_mean_of_values(dk):
    lens, hq, hkv, d = [777], 4, 1, 64
    k1 = normal_bf16(5, 2, (1, hkv, d))
    ks = [np.repeat(k1, lens[0], axis=0)]
    # identical raw keys rotate differently per position, so use q = 0 instead
    vs = [normal_bf16(5, 3, (lens[0], hkv, d))]
    qb = np.zeros((1, hq, d), dtype=np.uint16)
    from decode_attention_host_amd.cache_build import contiguous_cache
    cache = contiguous_cache(hkv, d, lens, 0.5, ks, vs, 1e4)
    o, lse, _ = _run_decode(dk, cache, qb, lens, 0.5, 1e4)
    mean_v = O.bf16_to_f64(vs[0][:, 0, :]).mean(axis=0)
    for h in range(hq):
        assert np.abs(o[0, h] - mean_v).max() < 1e-5
        assert abs(lse[0, h] - math.log(lens[0])) < 1e-5
    cache.free()


def test_split_offsets_and_partials_are_consistent(dk):
    # merge of the partials = the unsplit oracle, and each split's partial is
    # the oracle over that split's tokens
    import torch
    lens, hq, hkv, d, ratio, theta = [1500, 200], 8, 2, 128, 0.6, 1e4
    ks, vs = _raw(7, lens, hkv, d)
    qb = _q(7, 2, hq, d)
    from decode_attention_host_amd.cache_build import contiguous_cache
    cache = contiguous_cache(hkv, d, lens, ratio, ks, vs, theta)
    dk.set_tuning(host_chunk=256, dev_chunk=128, host_wgs=3, dev_wgs=5)
    try:
        o, lse, bufs = _run_decode(dk, cache, qb, lens, ratio, theta)
        offs = bufs.split_offsets.cpu().numpy()
        items, _, offs2, info = dk.plan_inspect(cache, 2, hq, lens, ratio,
                                                torch.cuda.get_device_properties(0).multi_processor_count)
    finally:
        dk.reset_tuning()
    assert np.array_equal(offs, offs2)
    po = bufs.part_o.cpu().numpy().astype(np.float64)
    pl = bufs.part_lse.cpu().numpy().astype(np.float64)
    for tier, b, slot, ntok, first in items:
        nh = O.contig_split_point(ratio, lens[b])
        t0 = first - b * cache.host_stride if tier else first - b * cache.dev_stride + nh
        ref_o, ref_l = O.decode_sequence_split(qb[b], ks[b], vs[b], lens[b] - 1, theta, 1 / math.sqrt(d),
                                               [np.arange(t0, t0 + ntok)])
        assert np.abs(po[slot] - ref_o).max() < TOL and np.abs(pl[slot] - ref_l).max() < TOL
    o_ref, l_ref = _oracle(qb, ks, vs, lens, theta)
    _assert_close(o, lse, o_ref, l_ref)
    cache.free()


# ----------------------------------------------------------------------- merge

@pytest.mark.parametrize("B,hq,d", [(3, 8, 128), (3, 8, 64), (40, 8, 128)])
def test_merge_lse_against_oracle(dk, B, hq, d):
    # fewer than 256 (b, h) pairs: dims sliced over several workgroups per
    # pair; 320 pairs: one workgroup per pair
    import torch
    rng = np.random.default_rng(11)
    counts = [1, 5, 37] + [int(c) for c in rng.integers(1, 90, size=B - 3)]
    S = sum(counts)
    po = rng.standard_normal((S, hq, d)).astype(np.float32)
    pl = (rng.standard_normal((S, hq)) * 5).astype(np.float32)
    pl[2, 3] = -np.inf
    pl[0, :] = -np.inf   # sequence 0: its only split is empty
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    o, lse = dk.merge_lse(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                          torch.from_numpy(offs).cuda(), B, hq, d)
    o = o.cpu().numpy(); lse = lse.cpu().numpy()
    for b in range(B):
        ro, rl = O.merge_lse(po[offs[b]:offs[b + 1]].astype(np.float64), pl[offs[b]:offs[b + 1]].astype(np.float64))
        if b == 0:
            assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
        else:
            assert np.abs(o[b] - ro).max() < 1e-5 and np.abs(lse[b] - rl).max() < 1e-5


@pytest.mark.parametrize("d", [64, 128])
def test_merge_lse_many_pairs(dk, d):
    # >= 2048 (b, h) pairs takes the one-wave-per-pair merge
    import torch
    rng = np.random.default_rng(12)
    B, hq = 300, 8
    counts = rng.integers(0, 4, size=B)
    counts[:4] = [0, 1, 70, 2]
    S = int(counts.sum())
    po = rng.standard_normal((S, hq, d)).astype(np.float32)
    pl = (rng.standard_normal((S, hq)) * 5).astype(np.float32)
    pl[rng.random((S, hq)) < 0.05] = -np.inf
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    o, lse = dk.merge_lse(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                          torch.from_numpy(offs).cuda(), B, hq, d)
    o = o.cpu().numpy(); lse = lse.cpu().numpy()
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    fin = np.isfinite(pl[offs[1]])
    assert np.array_equal(o[1][fin], po[offs[1]][fin])      # one split: returned exactly
    for b in range(1, B):
        ro, rl = O.merge_lse(po[offs[b]:offs[b + 1]].astype(np.float64),
                             pl[offs[b]:offs[b + 1]].astype(np.float64))
        assert np.abs(o[b] - ro).max() < 1e-5, b
        assert np.array_equal(np.isneginf(lse[b]), np.isneginf(rl)), b
        f = np.isfinite(rl)
        assert np.abs(lse[b][f] - rl[f]).max(initial=0) < 1e-5, b


# ----------------------------------------------------------------------- paged

@pytest.mark.parametrize("lens,hq,hkv,d,frac", [
    ([17, 1, 300, 1025], 32, 8, 128, 0.8),
    ([2000, 48], 8, 8, 64, 0.5),
    ([100], 4, 1, 128, 0.0),
    ([100], 4, 1, 128, 1.0),
])
def test_paged_parity_and_equals_contiguous(dk, lens, hq, hkv, d, frac):
    ks, vs = _raw(21, lens, hkv, d)
    qb = _q(21, len(lens), hq, d)
    pt, nh, nd = paged_table(4, lens, 16, frac)
    from decode_attention_host_amd.cache_build import contiguous_cache, paged_cache
    cache = paged_cache(hkv, d, lens, pt, nh, nd, ks, vs, 5e5)
    o, lse, _ = _run_decode(dk, cache, qb, lens, 0.0, 5e5)
    o_ref, l_ref = _oracle(qb, ks, vs, lens, 5e5)
    _assert_close(o, lse, o_ref, l_ref)
    c2 = contiguous_cache(hkv, d, lens, 0.5, ks, vs, 5e5)
    o2, l2, _ = _run_decode(dk, c2, qb, lens, 0.5, 5e5)
    assert np.abs(o2 - o).max() < 1e-4
    cache.free(); c2.free()


@pytest.mark.parametrize("page,d", [(1, 128), (8, 128), (32, 128), (256, 128), (8, 64), (32, 64)])
def test_paged_page_sizes(dk, page, d):
    # pages shorter than a chunk's rows (16 at D = 128, 32 at D = 64: per-lane
    # lookups) and as long or longer (workgroup-uniform scalar lookups),
    # ragged lengths over both tiers
    lens = [1, 255, 700, 1301]
    hq, hkv = 16, 4
    ks, vs = _raw(23, lens, hkv, d)
    qb = _q(23, len(lens), hq, d)
    pt, nh, nd = paged_table(5 + page, lens, page, 0.6)
    from decode_attention_host_amd.cache_build import paged_cache
    cache = paged_cache(hkv, d, lens, pt, nh, nd, ks, vs, 5e5, page=page)
    o, lse, _ = _run_decode(dk, cache, qb, lens, 0.0, 5e5)
    o_ref, l_ref = _oracle(qb, ks, vs, lens, 5e5)
    _assert_close(o, lse, o_ref, l_ref)
    cache.free()


# ----------------------------------------------------------------------- append indexing

def _pool_bits(cache, tier, which):
    if tier == 1:
        return cache.host_view(which).copy()
    t = cache.dev_k if which == "k" else cache.dev_v
    return t.view(__import__("torch").int16).cpu().numpy().view(np.uint16).copy()


def test_append_writes_only_target_rows_paged(dk):
    import torch
    hkv, d, theta = 8, 128, 5e5
    lens = [40, 70]
    pt, nh, nd = paged_table(9, lens, 16, 0.5)
    B = len(lens)
    cache = dk.KVCache(hkv, d, host_rows=nh * 16, dev_rows=nd * 16, page_size=16, page_table=pt)
    # sentinel fill
    cache.host_view("k")[...] = 0x7FA1
    cache.host_view("v")[...] = 0x7FA2
    cache.dev_k.view(torch.int16).fill_(0x7FA3)
    cache.dev_v.view(torch.int16).fill_(0x7FA4)
    torch.cuda.synchronize()
    before = {(t, w): _pool_bits(cache, t, w) for t in (0, 1) for w in ("k", "v")}
    # new tokens: (b, p) pairs spread over both sequences, pages and tiers
    toks = [(0, 0), (0, 17), (0, 39), (1, 5), (1, 16), (1, 69), (1, 33)]
    n = len(toks)
    kn = normal_bf16(77, 7, (n, hkv, d)); vn = normal_bf16(77, 8, (n, hkv, d))
    sidx = torch.tensor([b for b, _ in toks], dtype=torch.int32, device="cuda")
    pos = torch.tensor([p for _, p in toks], dtype=torch.int32, device="cuda")
    dk.project_rope_append(cache, B, None, 0.0, sidx, pos, k_new=torch.from_numpy(kn.view(np.int16)).cuda(),
                           v_new=torch.from_numpy(vn.view(np.int16)).cuda(), rope_theta=theta)
    torch.cuda.synchronize()
    expect = {k: v.copy() for k, v in before.items()}
    for i, (b, p) in enumerate(toks):
        tier, row = O.paged_slot(pt, b, p, 16)
        kr, vr = O.append_expected_rows(kn[i], vn[i], p, theta)
        expect[(tier, "k")][row] = kr
        expect[(tier, "v")][row] = vr
    for key in expect:
        got = _pool_bits(cache, *key)
        if key[1] == "v":
            assert np.array_equal(got, expect[key]), key
        else:
            diff = np.abs(got.astype(np.int32) - expect[key].astype(np.int32))
            assert diff.max() <= 1, key   # at most one bf16 ulp on rotated keys
            changed = np.any(got != before[key], axis=(1, 2))
            want = np.any(expect[key] != before[key], axis=(1, 2))
            assert np.array_equal(changed, want), key
    cache.free()


def test_append_writes_only_target_rows_contiguous(dk):
    import torch
    hkv, d, theta, ratio = 2, 64, 1e4, 0.5
    lens = [10, 7]
    # unequal strides: a host/device stride swap in the slot rule moves rows
    hs, ds = 8, 13
    cache = dk.KVCache(hkv, d, host_rows=2 * hs, dev_rows=2 * ds, host_stride=hs, dev_stride=ds)
    cache.host_view("k")[...] = 0x1111
    cache.host_view("v")[...] = 0x2222
    cache.dev_k.view(torch.int16).fill_(0x3333)
    cache.dev_v.view(torch.int16).fill_(0x4444)
    torch.cuda.synchronize()
    before = {(t, w): _pool_bits(cache, t, w) for t in (0, 1) for w in ("k", "v")}
    toks = [(0, 0), (0, 4), (0, 5), (0, 9), (1, 2), (1, 3), (1, 6)]
    n = len(toks)
    kn = normal_bf16(78, 7, (n, hkv, d)); vn = normal_bf16(78, 8, (n, hkv, d))
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dk.project_rope_append(cache, 2, sl, ratio, torch.tensor([b for b, _ in toks], dtype=torch.int32, device="cuda"),
                           torch.tensor([p for _, p in toks], dtype=torch.int32, device="cuda"),
                           k_new=torch.from_numpy(kn.view(np.int16)).cuda(),
                           v_new=torch.from_numpy(vn.view(np.int16)).cuda(), rope_theta=theta)
    torch.cuda.synchronize()
    expect = {k: v.copy() for k, v in before.items()}
    for i, (b, p) in enumerate(toks):
        tier, row = O.contig_slot(b, p, lens[b], ratio, hs, ds)
        kr, vr = O.append_expected_rows(kn[i], vn[i], p, theta)
        expect[(tier, "k")][row] = kr
        expect[(tier, "v")][row] = vr
    for key in expect:
        got = _pool_bits(cache, *key)
        tol = 1 if key[1] == "k" else 0
        assert np.abs(got.astype(np.int32) - expect[key].astype(np.int32)).max() <= tol, key
    cache.free()


def test_append_skips_tokens_outside_the_layout(dk):
    import torch
    hkv, d = 1, 64
    pt = np.array([[0 << 1 | 1, -1]], dtype=np.int32)
    cache = dk.KVCache(hkv, d, host_rows=16, dev_rows=16, page_size=16, page_table=pt)
    cache.host_view("k")[...] = 0x5555
    cache.dev_k.view(torch.int16).fill_(0x5555)
    torch.cuda.synchronize()
    kn = normal_bf16(1, 7, (4, hkv, d)); vn = normal_bf16(1, 8, (4, hkv, d))
    # page 1 unmapped, page 5 beyond max_pages, sequence 3 beyond batch, negative position
    dk.project_rope_append(cache, 1, None, 0.0, torch.tensor([0, 0, 3, 0], dtype=torch.int32, device="cuda"),
                           torch.tensor([20, 90, 1, -1], dtype=torch.int32, device="cuda"),
                           k_new=torch.from_numpy(kn.view(np.int16)).cuda(),
                           v_new=torch.from_numpy(vn.view(np.int16)).cuda(), rope_theta=1e4)
    torch.cuda.synchronize()
    assert np.all(cache.host_view("k") == 0x5555)
    assert np.all(cache.dev_k.view(torch.int16).cpu().numpy() == 0x5555)
    cache.free()


def test_append_rope_at_large_positions_and_peaked_window(dk):
    # keys rotated at positions near 2^20, query at 2^20 + 7, scores made peaked:
    # the case where fp32 angles would break the tolerance
    import torch
    hkv, hq, d, theta = 8, 32, 128, 5e5
    P0 = 1 << 20
    n = 8
    kraw = normal_bf16(31, 2, (n, hkv, d)); vraw = normal_bf16(31, 3, (n, hkv, d))
    max_pages = P0 // 16 + 1
    pt_w = np.full((1, max_pages), -1, dtype=np.int32)
    pt_w[0, P0 // 16] = (0 << 1) | 1         # writer: logical page of P0 -> host page 0
    cache = dk.KVCache(hkv, d, host_rows=16, dev_rows=16, page_size=16, page_table=pt_w)
    pos = torch.arange(P0, P0 + n, dtype=torch.int32, device="cuda")
    dk.project_rope_append(cache, 1, None, 0.0, torch.zeros(n, dtype=torch.int32, device="cuda"), pos,
                           k_new=torch.from_numpy(kraw.view(np.int16)).cuda(),
                           v_new=torch.from_numpy(vraw.view(np.int16)).cuda(), rope_theta=theta)
    torch.cuda.synchronize()
    kr, _ = O.append_expected_rows(kraw[0], vraw[0], P0, theta)
    assert np.abs(cache.host_view("k")[0].astype(np.int32) - kr.astype(np.int32)).max() <= 1
    # reader: same physical page seen as tokens 0..7
    cache.set_page_table(np.array([[(0 << 1) | 1]], dtype=np.int32))
    qb = normal_bf16(31, 1, (1, hq, d))
    q4 = O.bf16_rne_bits(O.bf16_to_f64(qb) * 4.0)   # sharper softmax
    o, lse, _ = _run_decode(dk, cache, q4, [n], 0.0, theta, q_pos=[P0 + n - 1])
    o_ref, l_ref = _oracle(q4, [kraw], [vraw], [n], theta, q_pos=[P0 + n - 1],
                           key_positions=[np.arange(P0, P0 + n)])
    _assert_close(o, lse, o_ref, l_ref)
    cache.free()


# ----------------------------------------------------------------------- projection

def test_projection_append_matches_oracle(dk):
    import torch
    hkv, d, hidden, theta = 8, 128, 4096, 5e5
    kvd = hkv * d
    n = 16
    x = normal_bf16(41, 4, (n, hidden)); wk = normal_bf16(41, 5, (hidden, kvd), std=0.02)
    wv = normal_bf16(41, 6, (hidden, kvd), std=0.02)
    lens = [1 + 37 * i for i in range(n)]
    pt, nh, nd = paged_table(41, lens, 16, 0.8)
    cache = dk.KVCache(hkv, d, host_rows=nh * 16, dev_rows=nd * 16, page_size=16, page_table=pt)
    pos = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device="cuda")
    dk.project_rope_append(cache, n, None, 0.0, torch.arange(n, dtype=torch.int32, device="cuda"), pos,
                           x=torch.from_numpy(x.view(np.int16)).cuda(),
                           wk=torch.from_numpy(wk.view(np.int16)).cuda(),
                           wv=torch.from_numpy(wv.view(np.int16)).cuda(), rope_theta=theta)
    torch.cuda.synchronize()
    kk = O.project(O.bf16_to_f64(x), O.bf16_to_f64(wk))
    vv = O.project(O.bf16_to_f64(x), O.bf16_to_f64(wv))
    for i, L in enumerate(lens):
        tier, row = O.paged_slot(pt, i, L - 1, 16)
        kr = O.rope_neox(kk[i].reshape(hkv, d), np.full(hkv, L - 1), theta)
        got_k = O.bf16_to_f64(_pool_bits(cache, tier, "k")[row])
        got_v = O.bf16_to_f64(_pool_bits(cache, tier, "v")[row])
        ulp_k = np.ldexp(1.0, np.frexp(kr)[1] - 8)
        ulp_v = np.ldexp(1.0, np.frexp(vv[i].reshape(hkv, d))[1] - 8)
        assert np.all(np.abs(got_k - kr) <= 2 * ulp_k + 1e-3)
        assert np.all(np.abs(got_v - vv[i].reshape(hkv, d)) <= 2 * ulp_v + 1e-3)
    cache.free()


# ----------------------------------------------------------------------- fused ragged step

def test_fused_ragged_step_small(dk):
    """Paged cache of L_b tokens, append of the projected new token at L_b, then
    attention over L_b + 1 tokens (the fused ragged workload at reduced size)."""
    import torch
    hkv, hq, d, hidden, theta = 8, 32, 128, 1024, 5e5
    B = 5
    lens = [int(x) for x in ragged_lengths(3, B, 20, 700)]
    ntok = [L + 1 for L in lens]
    pt, nh, nd = paged_table(3, ntok, 16, 0.8)
    ks, vs = _raw(3, lens, hkv, d)
    from decode_attention_host_amd.cache_build import paged_cache
    cache = paged_cache(hkv, d, ntok, pt, nh, nd, ks, vs, theta, upto=lens)
    x = normal_bf16(3, 4, (B, hidden)); wk = normal_bf16(3, 5, (hidden, hkv * d), std=0.02)
    wv = normal_bf16(3, 6, (hidden, hkv * d), std=0.02)
    dk.project_rope_append(cache, B, None, 0.0, torch.arange(B, dtype=torch.int32, device="cuda"),
                           torch.tensor(lens, dtype=torch.int32, device="cuda"),
                           x=torch.from_numpy(x.view(np.int16)).cuda(), wk=torch.from_numpy(wk.view(np.int16)).cuda(),
                           wv=torch.from_numpy(wv.view(np.int16)).cuda(), rope_theta=theta)
    qb = _q(3, B, hq, d)
    o, lse, _ = _run_decode(dk, cache, qb, ntok, 0.0, theta)
    kk = O.project(O.bf16_to_f64(x), O.bf16_to_f64(wk)).reshape(B, hkv, d)
    vv = O.project(O.bf16_to_f64(x), O.bf16_to_f64(wv)).reshape(B, hkv, d)
    for b in range(B):
        # oracle cache: stored keys of the old tokens + the new token's stored row
        k_new_bits, v_new_bits = O.append_expected_rows(kk[b], vv[b], lens[b], theta, k_is_bits=False)
        kst = O.bf16_to_f64(O.bf16_rne_bits(O.rope_neox(O.bf16_to_f64(ks[b]), np.arange(lens[b])[:, None], theta)))
        kst = np.concatenate([kst, O.bf16_to_f64(k_new_bits)[None]], axis=0)
        vst = np.concatenate([O.bf16_to_f64(vs[b]), O.bf16_to_f64(v_new_bits)[None]], axis=0)
        q_rot = O.rope_neox(O.bf16_to_f64(qb[b]), np.full(hq, lens[b]), theta)
        ro, rl = O.attention(q_rot, kst, vst, 1 / math.sqrt(d))
        _assert_close(o[b], lse[b], ro, rl)
    cache.free()
