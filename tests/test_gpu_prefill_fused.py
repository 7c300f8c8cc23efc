"""GPU parity of the fused prefill step (append of the new rows + causal
attention in one call) against the fp64 oracle, and against the two-call path.

The cache holds only the prefix before the call; the call must leave the new
rows in their slots (K within one bf16 ulp of the oracle's rounding of the
fp64 rotation, V bit-exact) and return o/lse within 2e-3 of the oracle.
"""
import math

import numpy as np
import pytest

import oracle as O
from synth import kv_raw, normal_bf16, paged_table

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


def _check(o, lse, ro, rl, what):
    eo, el = np.abs(o - ro).max(), np.abs(lse - rl).max()
    print(f"{what}: max|do|={eo:.3g} max|dlse|={el:.3g}", flush=True)
    assert eo <= TOL and el <= TOL, what


def _new_rows(ks, vs, lens, news):
    kn = np.concatenate([k[L - n:] for k, L, n in zip(ks, lens, news)])
    vn = np.concatenate([v[L - n:] for v, L, n in zip(vs, lens, news)])
    return kn, vn


def _pool_rows(cache, ratio, lens, b, positions, which):
    """Stored rows of sequence b at the given positions (contiguous layout)."""
    import torch
    nh = O.contig_split_point(ratio, lens[b])
    out = []
    for p in positions:
        tier, row = O.contig_slot(b, p, lens[b], ratio, cache.host_stride, cache.dev_stride)
        if tier == 1:
            out.append(cache.host_view(which)[row].copy())
        else:
            t = cache.dev_k if which == "k" else cache.dev_v
            out.append(t[row].view(torch.int16).cpu().numpy().view(np.uint16))
    return np.stack(out)


CASES = [
    # (lens, new rows, hq, hkv, d, ratio, theta)
    ([2048], [2048], 32, 8, 128, 1.0, 5e5),            # all new KV, host tier (the pages' prefill case)
    ([377, 64], [77, 64], 32, 8, 128, 0.5, 5e5),       # cached prefix + new rows, both tiers
    ([300, 33], [40, 1], 16, 2, 64, 0.0, 1e4),         # g = 8, HBM only, single-row sequence
    ([700], [300], 8, 8, 128, 0.8, 1e4),               # MHA, prefix staged, new rows in both tiers
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fused_contiguous(dk, case):
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, news, hq, hkv, d, r, th = CASES[case]
    ks, vs = kv_raw(100 + case, lens, hkv, d)
    qs = [normal_bf16(100 + case + b, 1, (n, hq, d)) for b, n in enumerate(news)]
    pre = [L - n for L, n in zip(lens, news)]
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th, upto=pre)
    kn, vn = _new_rows(ks, vs, lens, news)
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = torch.from_numpy(np.concatenate(qs).view(np.int16)).cuda()
    o, lse = dk.prefill_fused(cache, q, q_start, pre, lens, r, 1 / math.sqrt(d), th,
                              k_new=torch.from_numpy(kn.view(np.int16)).cuda(),
                              v_new=torch.from_numpy(vn.view(np.int16)).cuda())
    torch.cuda.synchronize()
    o = o.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    for b in range(len(lens)):
        ro, rl = O.prefill_sequence(qs[b], ks[b], vs[b], pre[b], th, 1 / math.sqrt(d))
        _check(o[q_start[b]:q_start[b + 1]], lse[q_start[b]:q_start[b + 1]], ro, rl, f"fused case {case} seq {b}")
        # the new rows are in the cache: V exact, K within one bf16 ulp
        pos = np.arange(pre[b], lens[b])
        rows = [O.append_expected_rows(ks[b][p], vs[b][p], int(p), th) for p in pos]
        kb = np.stack([a for a, _ in rows]); vb = np.stack([v for _, v in rows])
        got_k = _pool_rows(cache, r, lens, b, pos, "k")
        got_v = _pool_rows(cache, r, lens, b, pos, "v")
        assert np.array_equal(got_v, vb), f"V rows of seq {b}"
        assert np.abs(got_k.astype(np.int32) - kb.astype(np.int32)).max() <= 1, f"K rows of seq {b}"
    cache.free()


def test_fused_equals_two_call_path(dk):
    # same cache and rows: fused step vs append + prefill_attn_split + merge
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, news, hq, hkv, d, r, th = [900, 200], [400, 200], 32, 8, 128, 0.6, 5e5
    ks, vs = kv_raw(110, lens, hkv, d)
    qs = [normal_bf16(110 + b, 1, (n, hq, d)) for b, n in enumerate(news)]
    pre = [L - n for L, n in zip(lens, news)]
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = torch.from_numpy(np.concatenate(qs).view(np.int16)).cuda()
    kn, vn = _new_rows(ks, vs, lens, news)
    c1 = contiguous_cache(hkv, d, lens, r, ks, vs, th, upto=pre)
    o1, l1 = dk.prefill_fused(c1, q, q_start, pre, lens, r, 1 / math.sqrt(d), th,
                              k_new=torch.from_numpy(kn.view(np.int16)).cuda(),
                              v_new=torch.from_numpy(vn.view(np.int16)).cuda())
    c2 = contiguous_cache(hkv, d, lens, r, ks, vs, th)   # every row appended beforehand
    o2, l2, _ = dk.prefill(c2, q, q_start, pre, lens, r, 1 / math.sqrt(d), th)
    torch.cuda.synchronize()
    assert np.abs(o1.cpu().numpy() - o2.cpu().numpy()).max() < 1e-5
    assert np.abs(l1.cpu().numpy() - l2.cpu().numpy()).max() < 1e-5
    c1.free(); c2.free()


@pytest.mark.parametrize("host_frac", [0.8, 0.0])
def test_fused_paged_ragged(dk, host_frac):
    # 0.8: some new rows land in host pages (written by the prefill launch's
    # writer workgroups); 0.0: every page is in HBM (the append writes them)
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    lens, news, hq, hkv, d, th = [500, 17, 1200], [100, 17, 333], 32, 8, 128, 5e5
    ks, vs = kv_raw(120, lens, hkv, d)
    qs = [normal_bf16(120 + b, 1, (n, hq, d)) for b, n in enumerate(news)]
    pt, nh, nd = paged_table(120, lens, 16, host_frac)
    pre = [L - n for L, n in zip(lens, news)]
    cache = paged_cache(hkv, d, lens, pt, nh, nd, ks, vs, th, upto=pre)
    kn, vn = _new_rows(ks, vs, lens, news)
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = torch.from_numpy(np.concatenate(qs).view(np.int16)).cuda()
    o, lse = dk.prefill_fused(cache, q, q_start, pre, lens, 0.0, 1 / math.sqrt(d), th,
                              k_new=torch.from_numpy(kn.view(np.int16)).cuda(),
                              v_new=torch.from_numpy(vn.view(np.int16)).cuda())
    torch.cuda.synchronize()
    o = o.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    for b in range(3):
        ro, rl = O.prefill_sequence(qs[b], ks[b], vs[b], pre[b], th, 1 / math.sqrt(d))
        _check(o[q_start[b]:q_start[b + 1]], lse[q_start[b]:q_start[b + 1]], ro, rl, f"fused paged seq {b}")
        # the new rows are in their pages
        for p in range(pre[b], lens[b], 37):
            tier, row = O.paged_slot(pt, b, p, 16)
            pool = cache.host_view("v") if tier == 1 else cache.dev_v.view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(pool[row], vs[b][p])
    cache.free()


def test_fused_with_projection(dk):
    # new rows' K/V projected from x on MFMA, then appended and attended
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    hkv, hq, d, hidden, th, r = 8, 32, 128, 1024, 5e5, 0.5
    lens, news = [300], [96]
    pre = [lens[0] - news[0]]
    ks, vs = kv_raw(130, lens, hkv, d)
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th, upto=pre)
    x = normal_bf16(130, 4, (news[0], hidden))
    wk = normal_bf16(130, 5, (hidden, hkv * d), std=0.02)
    wv = normal_bf16(130, 6, (hidden, hkv * d), std=0.02)
    qb = normal_bf16(130, 1, (news[0], hq, d))
    q_start = np.array([0, news[0]], dtype=np.int32)
    o, lse = dk.prefill_fused(cache, torch.from_numpy(qb.view(np.int16)).cuda(), q_start, pre, lens, r,
                              1 / math.sqrt(d), th, x=torch.from_numpy(x.view(np.int16)).cuda(),
                              wk=torch.from_numpy(wk.view(np.int16)).cuda(),
                              wv=torch.from_numpy(wv.view(np.int16)).cuda())
    torch.cuda.synchronize()
    o = o.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    # oracle: stored keys of the prefix, then the projected rows rotated and rounded once
    kk = O.project(O.bf16_to_f64(x), O.bf16_to_f64(wk)).reshape(news[0], hkv, d)
    vv = O.project(O.bf16_to_f64(x), O.bf16_to_f64(wv)).reshape(news[0], hkv, d)
    pos = np.arange(pre[0], lens[0])
    rows = [O.append_expected_rows(kk[j], vv[j], int(p), th, k_is_bits=False) for j, p in enumerate(pos)]
    kb = np.stack([a for a, _ in rows]); vb = np.stack([v for _, v in rows])
    kst = O.bf16_to_f64(O.bf16_rne_bits(O.rope_neox(O.bf16_to_f64(ks[0][:pre[0]]),
                                                    np.arange(pre[0])[:, None], th)))
    kst = np.concatenate([kst, O.bf16_to_f64(kb)])
    vst = np.concatenate([O.bf16_to_f64(vs[0][:pre[0]]), O.bf16_to_f64(vb)])
    q_rot = O.rope_neox(O.bf16_to_f64(qb), np.repeat(pos[:, None], hq, axis=1), th)
    for j in range(0, news[0], 7):
        ro, rl = O.attention(q_rot[j], kst[:pos[j] + 1], vst[:pos[j] + 1], 1 / math.sqrt(d))
        _check(o[j], lse[j], ro, rl, f"projected row {j}")
    cache.free()


def test_fused_edge_cases(dk):
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    hq, hkv, d, th, r = 8, 2, 64, 1e4, 0.5
    lens = [50, 9]
    ks, vs = kv_raw(140, lens, hkv, d)
    # no query rows at all: nothing to do, no error
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th)
    q0 = torch.empty((0, hq, d), dtype=torch.int16, device="cuda")
    z = torch.empty((0, hkv, d), dtype=torch.int16, device="cuda")
    o, l = dk.prefill_fused(cache, q0, [0, 0, 0], [50, 9], lens, r, 0.125, th, k_new=z, v_new=z)
    assert o.shape[0] == 0
    o2, l2, _ = dk.prefill(cache, q0, [0, 0, 0], [50, 9], lens, r, 0.125, th)
    assert o2.shape[0] == 0
    # one new row in the middle of a cache (rows after it stay invisible), and
    # one row per sequence with the second sequence's row at position 0
    news = [1, 1]
    pre = [20, 0]
    qs = [normal_bf16(141 + b, 1, (1, hq, d)) for b in range(2)]
    q = torch.from_numpy(np.concatenate(qs).view(np.int16)).cuda()
    kn = np.concatenate([ks[b][p:p + 1] for b, p in enumerate(pre)])
    vn = np.concatenate([vs[b][p:p + 1] for b, p in enumerate(pre)])
    o, l = dk.prefill_fused(cache, q, [0, 1, 2], pre, lens, r, 0.125, th,
                            k_new=torch.from_numpy(kn.view(np.int16)).cuda(),
                            v_new=torch.from_numpy(vn.view(np.int16)).cuda())
    torch.cuda.synchronize()
    o = o.cpu().numpy().astype(np.float64)
    l = l.cpu().numpy().astype(np.float64)
    for b in range(2):
        ro, rl = O.prefill_sequence(qs[b], ks[b], vs[b], pre[b], th, 0.125)
        _check(o[b:b + 1], l[b:b + 1], ro, rl, f"edge seq {b}")
    # position 0 sees only itself: every head's o is its KV head's V0 exactly
    g = hq // hkv
    assert np.array_equal(o[1], O.bf16_to_f64(vs[1][0])[np.arange(hq) // g])
    cache.free()
