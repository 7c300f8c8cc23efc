"""GPU parity of the one-launch decode step (dkv_decode_step) and of the
growing decode loop, against the fp64 oracle.

A step appends each sequence's new token (key rotated at its position, one
bf16 rounding) into its slot and attends over the cached tokens plus the new
one, merging the per-tier partials inside the same launch.  Bar: max |do| and
max |dlse| <= 2e-3; the appended rows bit-exact in place (K within one bf16
ulp of bf16(RoPE(k)), V exact), every other row unchanged.

The loop tests run 100 steps with the length growing by one each step, once
eagerly and once as replays of a single captured graph (which also advances
the lengths), and compare steps 1, 50 and 100 with the oracle.
"""
import math

import numpy as np
import pytest

import oracle as O
from synth import TensorId, kv_raw, normal_bf16, paged_table, query

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


def _dev(a):
    import torch
    return torch.tensor(np.asarray(a, dtype=np.int32), dtype=torch.int32, device="cuda")


def _bits(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _pool_bits(cache, tier, which):
    import torch
    if tier == 1:
        return cache.host_view(which).copy()
    t = cache.dev_k if which == "k" else cache.dev_v
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _check(o, lse, ro, rl, what):
    eo = float(np.abs(o - ro).max())
    el = float(np.abs(lse - rl).max())
    print(f"{what}: max|do|={eo:.3g} max|dlse|={el:.3g}", flush=True)
    assert eo <= TOL and el <= TOL, what


def _oracle_step(qb, ks, vs, lens, theta):
    """Each sequence after the append: tokens 0..L_b (the new one at L_b), query at L_b."""
    out, lses = [], []
    for b, L in enumerate(lens):
        o, l = O.decode_sequence(qb[b], ks[b][:L + 1], vs[b][:L + 1], L, theta, 1 / math.sqrt(qb.shape[2]))
        out.append(o)
        lses.append(l)
    return np.stack(out), np.stack(lses)


STEP_CASES = [
    # (cached lens, hq, hkv, d, ratio, theta)
    ([511], 4, 2, 64, 1.0, 1e4),                 # the tiny workload after its append
    ([0], 4, 2, 64, 1.0, 1e4),                   # empty cache: only the new token
    ([0, 5], 8, 8, 128, 0.0, 1e4),
    ([64], 8, 1, 128, 0.5, 5e5),                 # g = 8
    ([299, 0, 128], 8, 4, 64, 0.3, 1e4),         # g = 2, ragged
    ([999, 776], 32, 8, 128, 0.75, 5e5),         # g = 4
    ([639, 2048], 16, 16, 128, 0.5, 1e4),        # MHA
    ([4095], 32, 8, 128, 0.0, 5e5),              # HBM only
    ([4095], 32, 8, 128, 1.0, 5e5),              # host only
    ([2999, 9], 16, 2, 64, 0.4, 1e4),            # g = 8, D = 64
]


@pytest.mark.parametrize("case", range(len(STEP_CASES)))
def test_step_contiguous_parity_and_append(dk, case):
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, hq, hkv, d, ratio, theta = STEP_CASES[case]
    B = len(lens)
    full = [L + 1 for L in lens]
    ks, vs = kv_raw(70 + case, full, hkv, d)
    qb = query(70 + case, B, hq, d)
    # placement of the cache after the append (L + 1 tokens); tokens 0..L-1 present
    cache = contiguous_cache(hkv, d, full, ratio, ks, vs, theta, upto=lens)
    before = {(t, w): _pool_bits(cache, t, w) for t in (0, 1) for w in ("k", "v")
              if (cache.host_rows if t else cache.dev_rows)}
    k_new = _bits(np.stack([k[L] for k, L in zip(ks, lens)]))
    v_new = _bits(np.stack([v[L] for v, L in zip(vs, lens)]))
    sl = _dev(lens)
    o, lse = dk.decode_step(cache, _bits(qb), _dev(lens), sl, ratio, 1 / math.sqrt(d), theta, k_new=k_new,
                            v_new=v_new)
    torch.cuda.synchronize()
    ro, rl = _oracle_step(qb, ks, vs, lens, theta)
    _check(o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl, f"case {case}")
    # appended rows: exactly the target rows changed
    expect = {k: v.copy() for k, v in before.items()}
    for b, L in enumerate(lens):
        tier, row = O.contig_slot(b, L, L + 1, ratio, cache.host_stride, cache.dev_stride)
        kr, vr = O.append_expected_rows(ks[b][L], vs[b][L], L, theta)
        expect[(tier, "k")][row] = kr
        expect[(tier, "v")][row] = vr
    for key in expect:
        got = _pool_bits(cache, *key)
        tol = 1 if key[1] == "k" else 0
        assert np.abs(got.astype(np.int32) - expect[key].astype(np.int32)).max() <= tol, key
        changed = np.any(got != before[key], axis=(1, 2))
        want = np.any(expect[key] != before[key], axis=(1, 2))
        assert np.array_equal(changed, want), key
    cache.free()


@pytest.mark.parametrize("lens,hq,hkv,d,frac", [
    ([16, 0, 300, 1024], 32, 8, 128, 0.8),
    ([1999, 47], 8, 8, 64, 0.5),
    ([99], 4, 1, 128, 0.0),
    ([99], 4, 1, 128, 1.0),
])
def test_step_paged_parity_and_append(dk, lens, hq, hkv, d, frac):
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    theta = 5e5
    B = len(lens)
    full = [L + 1 for L in lens]
    ks, vs = kv_raw(81, full, hkv, d)
    qb = query(81, B, hq, d)
    pt, nh, nd = paged_table(81, full, 16, frac)
    cache = paged_cache(hkv, d, full, pt, nh, nd, ks, vs, theta, upto=lens)
    o, lse = dk.decode_step(cache, _bits(qb), _dev(lens), _dev(lens), 0.0, 1 / math.sqrt(d), theta,
                            k_new=_bits(np.stack([k[L] for k, L in zip(ks, lens)])),
                            v_new=_bits(np.stack([v[L] for v, L in zip(vs, lens)])))
    torch.cuda.synchronize()
    ro, rl = _oracle_step(qb, ks, vs, lens, theta)
    _check(o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl, f"paged {lens}")
    for b, L in enumerate(lens):
        tier, row = O.paged_slot(pt, b, L, 16)
        kr, vr = O.append_expected_rows(ks[b][L], vs[b][L], L, theta)
        gk, gv = _pool_bits(cache, tier, "k")[row], _pool_bits(cache, tier, "v")[row]
        assert np.abs(gk.astype(np.int32) - kr.astype(np.int32)).max() <= 1
        assert np.array_equal(gv, vr)
    cache.free()


def test_max_batch_512_both_forms(dk):
    """The largest batch the decode kernel takes (512 sequences, lengths 0..200
    tokens, some empty, paged with pages split 50/50 between the tiers): the
    fused step appends each new token and attends; then the split form
    attends over the grown cache.  Every sequence against the oracle."""
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    B, hq, hkv, d, theta = 512, 8, 2, 64, 1e4
    lens = [int(x) for x in np.random.default_rng(512).integers(0, 201, B)]
    lens[3] = lens[200] = 0
    full = [L + 1 for L in lens]
    ks, vs = kv_raw(512, full, hkv, d)
    qb = query(512, B, hq, d)
    pt, nh, nd = paged_table(512, full, 16, 0.5)
    cache = paged_cache(hkv, d, full, pt, nh, nd, ks, vs, theta, upto=lens)
    o, lse = dk.decode_step(cache, _bits(qb), _dev(lens), _dev(lens), 0.0, 1 / math.sqrt(d), theta,
                            k_new=_bits(np.stack([k[L] for k, L in zip(ks, lens)])),
                            v_new=_bits(np.stack([v[L] for v, L in zip(vs, lens)])))
    torch.cuda.synchronize()
    ro, rl = _oracle_step(qb, ks, vs, lens, theta)
    _check(o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl, "512 fused step")
    so, sl, _ = dk.decode(cache, _bits(qb), _dev(lens), full, 0.0, 1 / math.sqrt(d), theta)
    torch.cuda.synchronize()
    _check(so.cpu().numpy().astype(np.float64), sl.cpu().numpy().astype(np.float64), ro, rl, "512 split form")
    cache.free()


@pytest.mark.parametrize("ratio", [0.0, 0.5])
def test_step_merge_group_boundaries(dk, ratio):
    """The fused step folds a sequence's partial slots (its new token's, then one
    per item) in groups of 16 and then folds the groups.  With one-tile items
    (64 tokens) the cached lengths below give 1, 2, 16, 17, 18, 33, 34 and 81
    slots: a single slot, one partial group, one full group, a last group of
    one slot (its own result) or of two, and five full groups plus one; at
    r = 0.5 the items of a sequence lie in both tiers.  With and without the
    new token, against the oracle (and, without it, the split form)."""
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, hq, hkv, d, th = [0, 1, 64, 960, 1024, 1025, 2048, 2049, 5120], 8, 2, 64, 1e4
    B = len(lens)
    full = [L + 1 for L in lens]
    ks, vs = kv_raw(95, full, hkv, d)
    qb = query(95, B, hq, d)
    dk.set_tuning(host_chunk=64, dev_chunk=64)
    try:
        cache = contiguous_cache(hkv, d, full, ratio, ks, vs, th, upto=lens)
        k_new = _bits(np.stack([k[L] for k, L in zip(ks, lens)]))
        v_new = _bits(np.stack([v[L] for v, L in zip(vs, lens)]))
        o, lse = dk.decode_step(cache, _bits(qb), _dev(lens), _dev(lens), ratio, 1 / math.sqrt(d), th,
                                k_new=k_new, v_new=v_new)
        torch.cuda.synchronize()
        ro, rl = _oracle_step(qb, ks, vs, lens, th)
        o, lse = o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
        for b, L in enumerate(lens):
            _check(o[b], lse[b], ro[b], rl[b], f"r={ratio} cached {L} + new token")
        cache.free()
        # no new token: the cached tokens only (the first sequence has none)
        cache = contiguous_cache(hkv, d, lens, ratio, ks, vs, th)
        qpos = _dev([max(0, L - 1) for L in lens])
        o, lse = dk.decode_step(cache, _bits(qb), qpos, _dev(lens), ratio, 1 / math.sqrt(d), th)
        o2, l2, _ = dk.decode(cache, _bits(qb), qpos, _dev(lens), ratio, 1 / math.sqrt(d), th)
        torch.cuda.synchronize()
        o, lse, o2, l2 = (t.cpu().numpy().astype(np.float64) for t in (o, lse, o2, l2))
        assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
        assert np.abs(o[1:] - o2[1:]).max() < 1e-5 and np.abs(lse[1:] - l2[1:]).max() < 1e-5
        for b, L in enumerate(lens[1:], start=1):
            rob, rlb = O.decode_sequence(qb[b], ks[b][:L], vs[b][:L], L - 1, th, 1 / math.sqrt(d))
            _check(o[b], lse[b], rob, rlb, f"r={ratio} cached {L}, no new token")
        cache.free()
    finally:
        dk.reset_tuning()


def test_step_merge_folds_groups_in_chunks(dk):
    """A sequence with more group results than the final fold stages at once
    (288 lse values per head at D = 64, G = 8): 300,000 cached tokens in
    one-tile items give 4,689 slots per KV head, so 294 groups, folded in two
    chunks.  Against the oracle over every head."""
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    L, hq, hkv, d, th = 300000, 16, 2, 64, 5e5
    ks, vs = kv_raw(96, [L + 1], hkv, d)
    qb = query(96, 1, hq, d)
    dk.set_tuning(dev_chunk=64)
    try:
        cache = contiguous_cache(hkv, d, [L + 1], 0.0, ks, vs, th, upto=[L])
        o, lse = dk.decode_step(cache, _bits(qb), _dev([L]), _dev([L]), 0.0, 1 / math.sqrt(d), th,
                                k_new=_bits(ks[0][L:L + 1]), v_new=_bits(vs[0][L:L + 1]))
        torch.cuda.synchronize()
        cache.free()
    finally:
        dk.reset_tuning()
    ro, rl = _oracle_step(qb, ks, vs, [L], th)
    _check(o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
           "300k tokens, 294 merge groups")


def test_step_without_new_token_equals_split_form(dk):
    # no new token: the fused launch attends to the cached tokens only and must
    # agree with the split form (attention + merge) and the oracle
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, hq, hkv, d, r, th = [3000, 517, 0], 32, 8, 128, 0.6, 5e5
    ks, vs = kv_raw(83, lens, hkv, d)
    qb = query(83, 3, hq, d)
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th)
    qpos = _dev([max(0, L - 1) for L in lens])
    o, lse = dk.decode_step(cache, _bits(qb), qpos, _dev(lens), r, 1 / math.sqrt(d), th)
    o2, l2, _ = dk.decode(cache, _bits(qb), qpos, _dev(lens), r, 1 / math.sqrt(d), th)
    torch.cuda.synchronize()
    o, lse, o2, l2 = (t.cpu().numpy().astype(np.float64) for t in (o, lse, o2, l2))
    assert np.abs(o - o2).max() < 1e-5 and np.abs(lse[:2] - l2[:2]).max() < 1e-5
    # the empty sequence: o = 0, lse = -inf in both forms
    assert np.all(o[2] == 0) and np.all(np.isneginf(lse[2])) and np.all(np.isneginf(l2[2]))
    for b in range(2):
        ro, rl = O.decode_sequence(qb[b], ks[b], vs[b], lens[b] - 1, th, 1 / math.sqrt(d))
        _check(o[b], lse[b], ro, rl, f"no new token, seq {b}")
    cache.free()


def test_step_with_projection(dk):
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    hkv, hq, d, hid, th, B = 8, 32, 128, 1024, 5e5, 3
    lens = [100, 1500, 40]
    full = [L + 1 for L in lens]
    ks, vs = kv_raw(84, lens, hkv, d)
    pt, nh, nd = paged_table(84, full, 16, 0.8)
    cache = paged_cache(hkv, d, full, pt, nh, nd, ks, vs, th, upto=lens)
    x = normal_bf16(84, TensorId.X, (B, hid))
    wk = normal_bf16(84, TensorId.WK, (hid, hkv * d), std=0.02)
    wv = normal_bf16(84, TensorId.WV, (hid, hkv * d), std=0.02)
    qb = query(84, B, hq, d)
    o, lse = dk.decode_step(cache, _bits(qb), _dev(lens), _dev(lens), 0.0, 1 / math.sqrt(d), th, x=_bits(x),
                            wk=_bits(wk), wv=_bits(wv))
    torch.cuda.synchronize()
    o = o.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    kk = O.project(O.bf16_to_f64(x), O.bf16_to_f64(wk)).reshape(B, hkv, d)
    vv = O.project(O.bf16_to_f64(x), O.bf16_to_f64(wv)).reshape(B, hkv, d)
    for b in range(B):
        kn, vn = O.append_expected_rows(kk[b], vv[b], lens[b], th, k_is_bits=False)
        kst = O.bf16_to_f64(O.bf16_rne_bits(O.rope_neox(O.bf16_to_f64(ks[b]), np.arange(lens[b])[:, None], th)))
        kst = np.concatenate([kst, O.bf16_to_f64(kn)[None]], axis=0)
        vst = np.concatenate([O.bf16_to_f64(vs[b]), O.bf16_to_f64(vn)[None]], axis=0)
        q_rot = O.rope_neox(O.bf16_to_f64(qb[b]), np.full(hq, lens[b]), th)
        ro, rl = O.attention(q_rot, kst, vst, 1 / math.sqrt(d))
        _check(o[b], lse[b], ro, rl, f"projection seq {b}")
        # the stored rows after the projection (2 bf16 ulp + 1e-3, as for the append)
        tier, row = O.paged_slot(pt, b, lens[b], 16)
        gk = O.bf16_to_f64(_pool_bits(cache, tier, "k")[row])
        gv = O.bf16_to_f64(_pool_bits(cache, tier, "v")[row])
        for got, ref in ((gk, O.bf16_to_f64(kn)), (gv, O.bf16_to_f64(vn))):
            assert np.all(np.abs(got - ref) <= 2 * np.abs(ref) * 2.0 ** -8 + 1e-3)
    cache.free()


@pytest.mark.parametrize("queued", [False, True])
def test_workspace_is_left_zeroed_and_clean(dk, queued):
    # Dealt: few units per workgroup, dealt round-robin, no queue counter
    # moves.  Queued: one workgroup per KV head and tier and one-tile items,
    # so both tiers take units from their counters and the last workgroup out
    # resets them; three calls in a row on one workspace stay right.
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    hkv, hq, d, th = 8, 32, 128, 5e5
    lens = [700, 33]
    full = [L + 1 for L in lens]
    ks, vs = kv_raw(85, full, hkv, d)
    pt, nh, nd = paged_table(85, full, 16, 0.5)
    cache = paged_cache(hkv, d, full, pt, nh, nd, ks, vs, th, upto=lens)
    if queued:
        dk.set_tuning(host_wgs=hkv, dev_wgs=hkv, host_chunk=64, dev_chunk=64)
    try:
        ws = dk.decode_step_workspace(cache, 2, hq, 0.0)
        qb = query(85, 2, hq, d)
        for _ in range(3):
            o, lse = dk.decode_step(cache, _bits(qb), _dev(lens), _dev(lens), 0.0, 1 / math.sqrt(d), th,
                                    k_new=_bits(np.stack([k[L] for k, L in zip(ks, lens)])),
                                    v_new=_bits(np.stack([v[L] for v, L in zip(vs, lens)])), workspace=ws)
        torch.cuda.synchronize()
        # queues, exit count, error word and the (sequence, KV head) counters
        head = ws[:512].cpu().numpy()
        assert np.all(head == 0), np.nonzero(head)
        assert dk.decode_errors(cache, ws) == 0
        ro, rl = _oracle_step(qb, ks, vs, lens, th)
        _check(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, f"third call ({'queued' if queued else 'dealt'})")
    finally:
        dk.reset_tuning()
        cache.free()


@pytest.mark.parametrize("queued", [False, True])
def test_split_form_buffers_reused(dk, queued):
    # The split form on one set of buffers, three calls in a row, with its
    # units dealt round-robin or (one workgroup per KV head and tier, one-tile
    # items) taken from the queue counters: the counters are back at zero
    # after every call and each call matches the oracle.
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    hkv, hq, d, th = 8, 32, 128, 5e5
    lens = [700, 33]
    ks, vs = kv_raw(86, lens, hkv, d)
    pt, nh, nd = paged_table(86, lens, 16, 0.5)
    cache = paged_cache(hkv, d, lens, pt, nh, nd, ks, vs, th)
    if queued:
        dk.set_tuning(host_wgs=hkv, dev_wgs=hkv, host_chunk=64, dev_chunk=64)
    try:
        qb = query(86, 2, hq, d)
        bufs = dk.alloc_decode_buffers(cache, 2, hq, lens, 0.0)
        ro, rl = [], []
        for b, L in enumerate(lens):
            o1, l1 = O.decode_sequence(qb[b], ks[b], vs[b], L - 1, th, 1 / math.sqrt(d))
            ro.append(o1)
            rl.append(l1)
        for call in range(3):
            o, lse, _ = dk.decode(cache, _bits(qb), _dev([L - 1 for L in lens]), lens, 0.0, 1 / math.sqrt(d), th,
                                  bufs=bufs)
            torch.cuda.synchronize()
            assert np.all(bufs.workspace[:16].cpu().numpy() == 0), "queue counters left set"
            _check(o.cpu().numpy(), lse.cpu().numpy(), np.stack(ro), np.stack(rl),
                   f"split form call {call} ({'queued' if queued else 'dealt'})")
        assert dk.decode_errors(cache, bufs.workspace) == 0
    finally:
        dk.reset_tuning()
        cache.free()


def test_layout_violation_is_flagged_not_read(dk):
    # a length beyond the contiguous layout: the sequence is skipped and
    # flagged; the others are still right
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, hq, hkv, d, r, th = [200, 100], 8, 2, 64, 0.5, 1e4
    ks, vs = kv_raw(86, lens, hkv, d)
    qb = query(86, 2, hq, d)
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th)
    ws = dk.decode_step_workspace(cache, 2, hq, r)
    bad = [200, 100000]  # sequence 1 far beyond its stride
    o, lse = dk.decode_step(cache, _bits(qb), _dev([199, 99]), _dev(bad), r, 1 / math.sqrt(d), th, workspace=ws)
    torch.cuda.synchronize()
    assert dk.decode_errors(cache, ws) & 1
    assert dk.decode_errors(cache, ws) == 0  # cleared by the previous read
    ro, rl = O.decode_sequence(qb[0], ks[0], vs[0], 199, th, 1 / math.sqrt(d))
    _check(o[0].cpu().numpy().astype(np.float64), lse[0].cpu().numpy().astype(np.float64), ro, rl, "valid seq")
    assert np.all(o[1].cpu().numpy() == 0) and np.all(np.isneginf(lse[1].cpu().numpy()))
    cache.free()


def test_paged_tier_lists_over_several_chunks(dk):
    """A sequence of 20000 one-token pages spans two chunks of the tier-list
    kernel (16384 page entries each): its attention must match the oracle;
    with one page entry of the second chunk unmapped, that token is left out
    (the oracle without it) and the page error is flagged."""
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    lens, hq, hkv, d, th = [20000, 3000], 8, 2, 64, 1e4
    ks, vs = kv_raw(87, lens, hkv, d)
    qb = query(87, 2, hq, d)
    pt, nh, nd = paged_table(87, lens, 1, 0.5)
    cache = paged_cache(hkv, d, lens, pt, nh, nd, ks, vs, th, page=1)
    ws = dk.decode_step_workspace(cache, 2, hq, 0.0)
    qpos = [L - 1 for L in lens]
    o, lse = dk.decode_step(cache, _bits(qb), _dev(qpos), _dev(lens), 0.0, 1 / math.sqrt(d), th, workspace=ws)
    torch.cuda.synchronize()
    assert dk.decode_errors(cache, ws) == 0
    for b in range(2):
        ro, rl = O.decode_sequence(qb[b], ks[b], vs[b], qpos[b], th, 1 / math.sqrt(d))
        _check(o[b].cpu().numpy().astype(np.float64), lse[b].cpu().numpy().astype(np.float64), ro, rl,
               f"paged 1-token pages, seq {b}")
    # unmap token 17000 of sequence 0 (second chunk of its row)
    drop = 17000
    pt_bad = pt.copy()
    pt_bad[0, drop] = -1
    cache.update_page_table(pt_bad)
    o, lse = dk.decode_step(cache, _bits(qb), _dev(qpos), _dev(lens), 0.0, 1 / math.sqrt(d), th, workspace=ws)
    torch.cuda.synchronize()
    assert dk.decode_errors(cache, ws) & 2
    keep = np.ones(lens[0], dtype=bool)
    keep[drop] = False
    kst = O.bf16_to_f64(O.bf16_rne_bits(O.rope_neox(O.bf16_to_f64(ks[0]), np.arange(lens[0])[:, None], th)))
    vst = O.bf16_to_f64(vs[0])
    g = hq // hkv
    q_rot = O.rope_neox(O.bf16_to_f64(qb[0]), np.full(hq, qpos[0]), th)
    for kvh in range(hkv):
        heads = list(range(kvh * g, (kvh + 1) * g))
        ro, rl = O.attention(q_rot[heads], kst[keep][:, kvh:kvh + 1], vst[keep][:, kvh:kvh + 1], 1 / math.sqrt(d))
        _check(o[0, heads].cpu().numpy().astype(np.float64), lse[0, heads].cpu().numpy().astype(np.float64), ro, rl,
               f"token {drop} unmapped, kv head {kvh}")
    cache.free()


# ----------------------------------------------------------------- growing decode loop

CHECK_STEPS = (1, 50, 100)


def _loop(dk, cache, qb, ks, vs, L0, theta, ratio, graph):
    """100 steps: append at L, attend over L + 1, L += 1.  Returns the outputs
    of the steps in CHECK_STEPS (1-based)."""
    import torch
    B, hq, d = qb.shape
    q = _bits(qb)
    sl = _dev(L0)
    pos = _dev(L0)
    k_step = torch.empty((B,) + ks[0].shape[1:], dtype=torch.int16, device="cuda")
    v_step = torch.empty_like(k_step)
    ws = dk.decode_step_workspace(cache, B, hq, ratio)
    out_o = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
    out_l = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    k_all = [_bits(k) for k in ks]
    v_all = [_bits(v) for v in vs]

    def load(s):  # the new token of step s (0-based) into the fixed buffers
        for b in range(B):
            k_step[b].copy_(k_all[b][L0[b] + s])
            v_step[b].copy_(v_all[b][L0[b] + s])

    def step():
        dk.decode_step(cache, q, pos, sl, ratio, 1 / math.sqrt(d), theta, k_new=k_step, v_new=v_step,
                       workspace=ws, out_o=out_o, out_lse=out_l)
        sl.add_(1)
        pos.add_(1)

    got = {}
    g = None
    if graph:
        load(0)
        sl0, pos0 = sl.clone(), pos.clone()
        g = dk.StepGraph(step, warmup=1)   # warm-up and capture advance the lengths: rewind
        sl.copy_(sl0)
        pos.copy_(pos0)
        torch.cuda.synchronize()
    for s in range(100):
        load(s)
        if graph:
            g.replay()
        else:
            step()
        if s + 1 in CHECK_STEPS:
            torch.cuda.synchronize()
            got[s + 1] = (out_o.cpu().numpy().astype(np.float64), out_l.cpu().numpy().astype(np.float64))
            out_o.fill_(float("nan"))
    torch.cuda.synchronize()
    assert np.array_equal(sl.cpu().numpy(), np.asarray(L0) + 100)
    return got


def _check_loop(got, qb, ks, vs, L0, theta, what):
    d = qb.shape[2]
    for s, (o, lse) in got.items():
        for b in range(qb.shape[0]):
            L = L0[b] + s - 1  # cached tokens before step s; the new token sits at L
            ro, rl = O.decode_sequence(qb[b], ks[b][:L + 1], vs[b][:L + 1], L, theta, 1 / math.sqrt(d))
            _check(o[b], lse[b], ro, rl, f"{what} step {s} seq {b}")


@pytest.mark.parametrize("graph", [False, True])
def test_decode_loop_contiguous_host(dk, graph):
    # LLaMA-3-8B heads, all KV in host memory (r = 1: every new token lands in
    # the host pool, so the contiguous layout stays consistent as it grows)
    from decode_attention_host_amd.cache_build import contiguous_cache
    hq, hkv, d, th = 32, 8, 128, 5e5
    L0 = [2000]
    cap = [L0[0] + 100]
    ks, vs = kv_raw(87, cap, hkv, d)
    qb = query(87, 1, hq, d)
    cache = contiguous_cache(hkv, d, cap, 1.0, ks, vs, th, upto=L0)
    got = _loop(dk, cache, qb, ks, vs, L0, th, 1.0, graph)
    _check_loop(got, qb, ks, vs, L0, th, "contiguous r=1" + (" graph" if graph else ""))
    cache.free()


@pytest.mark.parametrize("graph", [False, True])
def test_decode_loop_paged_allocator(dk, graph):
    # three sequences in pages from the native allocator (80% host pages);
    # pages for all 100 steps are reserved up front
    import torch
    from decode_attention_host_amd.cache_build import _append_rows
    hq, hkv, d, th = 32, 8, 128, 5e5
    L0 = [1000, 77, 16]
    cap = [L + 101 for L in L0]
    ks, vs = kv_raw(88, cap, hkv, d)
    qb = query(88, 3, hq, d)
    alloc = dk.PagedKVAllocator(hkv, d, n_host_pages=200, n_dev_pages=200, max_seqs=3, max_pages=128,
                                host_fraction=0.8, page_size=16)
    for b, n in enumerate(cap):
        alloc.reserve(b, n)
    cache = alloc.pools
    for b in range(3):
        _append_rows(cache, 3, b, 0, ks[b][:L0[b]], vs[b][:L0[b]], None, 0.0, th)
    torch.cuda.synchronize()
    got = _loop(dk, cache, qb, ks, vs, L0, th, 0.0, graph)
    _check_loop(got, qb, ks, vs, L0, th, "paged" + (" graph" if graph else ""))
    alloc.close()
