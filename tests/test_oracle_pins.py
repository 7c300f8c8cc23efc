"""Pins for the fp64 oracle: closed forms, invariants and brute force.

Every oracle function is checked here against something other than itself:
hand-derived values in tests/golden/closed_forms.json, identities that the
mathematics fixes (norm preservation, composition, shift invariance, softmax
normalisation, special cases with a known answer) and a pure-Python scalar
twin on tiny inputs.  Each test below names the mistake it would catch.
"""
import math

import numpy as np
import pytest

import oracle as O
from oracle import brute as BR
from synth import bf16_bits_from_f32, normal_bf16, paged_table


def _theta(case, g):
    t = case["theta"]
    return g["rope_neox"]["theta_quarter_turn"] if t == "quarter_turn" else float(t)


# ------------------------------------------------------------------ bf16

def test_bf16_rne_golden(golden):
    for c in golden["bf16_rne"]["cases"]:
        got = int(O.bf16_rne_bits(np.array([c["x"]]))[0])
        assert got == int(c["bits"], 16), c["why"]
        # widening back is exact for representable values
    assert O.bf16_to_f64(np.array([0x3F81], dtype=np.uint16))[0] == 1.0 + 2.0 ** -7


def test_bf16_rne_matches_float32_route_where_no_double_rounding():
    # For float32 inputs the single rounding f64->bf16 must equal the classic
    # float32 bit trick (catches a truncating or round-half-up implementation).
    rng = np.random.default_rng(7)
    x = rng.standard_normal(100000).astype(np.float32)
    assert np.array_equal(O.bf16_rne_bits(x.astype(np.float64)), bf16_bits_from_f32(x))


def test_bf16_rne_is_nearest():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(20000) * 3.0
    r = O.bf16_to_f64(O.bf16_rne_bits(x))
    # neighbours one bf16 ulp away are never closer
    ulp = np.ldexp(1.0, np.frexp(x)[1] - 8)
    assert np.all(np.abs(r - x) <= ulp / 2 + 1e-300)


# ------------------------------------------------------------------ RoPE

def test_rope_inv_freq_golden(golden):
    for c in golden["rope_inv_freq"]["cases"]:
        np.testing.assert_allclose(O.rope_inv_freq(c["D"], c["theta"]), c["f"], rtol=1e-15)


def test_rope_golden(golden):
    for c in golden["rope_neox"]["cases"]:
        y = O.rope_neox(np.array(c["x"], dtype=np.float64), c["pos"], _theta(c, golden))
        np.testing.assert_allclose(y, c["y"], atol=1e-15, err_msg=c["why"])


def test_rope_position_zero_is_identity_exactly():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 128))
    assert np.array_equal(O.rope_neox(x, np.zeros(5), 5e5), x)


@pytest.mark.parametrize("D,theta", [(64, 1e4), (128, 5e5)])
def test_rope_preserves_norm(D, theta):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, D))
    p = rng.integers(0, 1 << 20, size=64)
    y = O.rope_neox(x, p, theta)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)


def test_rope_composition():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 64))
    a, b = 1234, 777
    y1 = O.rope_neox(O.rope_neox(x, np.full(8, a), 1e4), np.full(8, b), 1e4)
    y2 = O.rope_neox(x, np.full(8, a + b), 1e4)
    np.testing.assert_allclose(y1, y2, atol=1e-9)


def test_rope_shift_invariance_of_scores():
    # R(q,a).R(k,b) depends only on a - b: the property attention relies on.
    rng = np.random.default_rng(4)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    ref = O.rope_neox(q, 500, 5e5) @ O.rope_neox(k, 123, 5e5)
    for s in (1, 1000, 65536):
        got = O.rope_neox(q, 500 + s, 5e5) @ O.rope_neox(k, 123 + s, 5e5)
        assert abs(got - ref) < 1e-9


def test_rope_matches_scalar_twin():
    rng = np.random.default_rng(5)
    for D in (2, 4, 8, 64):
        x = rng.standard_normal(D)
        for p in (0, 1, 17, 511):
            y = O.rope_neox(x, p, 1e4)
            yb = BR.rope_neox_py(list(x), p, 1e4)
            np.testing.assert_allclose(y, yb, atol=1e-13)


# ------------------------------------------------------------------ projection

def test_projection_matches_scalar_twin_and_is_linear():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 16))
    w = rng.standard_normal((16, 12))
    y = O.project(x, w)
    for r in range(2):
        np.testing.assert_allclose(y[r], BR.matvec_rows_py(list(x[r]), w.tolist()), atol=1e-12)
    np.testing.assert_allclose(O.project(2 * x[0:1] + x[1:2], w), 2 * y[0:1] + y[1:2], atol=1e-12)
    # column h*D + d layout: projecting a basis vector reads one row of W
    e = np.zeros((1, 16)); e[0, 3] = 1.0
    assert np.array_equal(O.project(e, w)[0], w[3])


# ------------------------------------------------------------------ offloaded linear

def test_linear_matches_scalar_twin():
    # catches a transposed or wrongly indexed weight (N != K here)
    xb = normal_bf16(31, 1, (3, 8))
    wb = normal_bf16(31, 2, (5, 8))
    y = O.linear(xb, wb)
    assert y.shape == (3, 5)
    ref = BR.linear_py(O.bf16_to_f64(xb).tolist(), O.bf16_to_f64(wb).tolist())
    np.testing.assert_allclose(y, ref, atol=1e-12)


def test_linear_closed_forms():
    one = bf16_bits_from_f32(np.ones((1, 6), np.float32))
    # all-ones: every output is the inner dimension
    assert np.array_equal(O.linear(one, bf16_bits_from_f32(np.ones((4, 6), np.float32))), np.full((1, 4), 6.0))
    # identity weight returns x exactly; a basis input reads one column of W
    xb = normal_bf16(32, 1, (2, 6))
    eye = bf16_bits_from_f32(np.eye(6, dtype=np.float32))
    assert np.array_equal(O.linear(xb, eye), O.bf16_to_f64(xb))
    wb = normal_bf16(32, 2, (4, 6))
    e = np.zeros((1, 6), np.float32); e[0, 2] = 1.0
    assert np.array_equal(O.linear(bf16_bits_from_f32(e), wb)[0], O.bf16_to_f64(wb)[:, 2])


def test_linear_split_rows_and_concat(golden):
    for c in golden["split_point"]["cases"]:
        assert O.linear_split_rows(c["r"], c["L"]) == c["n_host"]
    xb = normal_bf16(33, 1, (3, 16))
    wb = normal_bf16(33, 2, (10, 16))
    for r in (0.0, 0.3, 0.7, 1.0):
        nh = O.linear_split_rows(r, 10)
        np.testing.assert_array_equal(O.linear_split(xb, wb[:nh], wb[nh:]), O.linear(xb, wb))
    assert O.linear_split_rows(0.7, 10) == 7 and O.linear_split_rows(1.0, 10) == 10


# ------------------------------------------------------------------ attention

def test_attention_golden(golden):
    for c in golden["attention"]["cases"]:
        o, lse = O.attention(np.array(c["q_rot"]), np.array(c["k"]), np.array(c["v"]), c["scale"])
        np.testing.assert_allclose(o, c["o"], atol=1e-13, err_msg=c["why"])
        np.testing.assert_allclose(lse, c["lse"], atol=1e-13, err_msg=c["why"])


def test_single_token_returns_v0_exactly():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((4, 64)); k = rng.standard_normal((1, 2, 64)); v = rng.standard_normal((1, 2, 64))
    o, lse = O.attention(q, k, v, 0.125)
    for h in range(4):
        assert np.array_equal(o[h], v[0, h // 2])
        assert abs(lse[h] - 0.125 * (q[h] @ k[0, h // 2])) < 1e-14


def test_identical_keys_and_zero_query_give_mean_of_v():
    rng = np.random.default_rng(11)
    N = 37
    k = np.repeat(rng.standard_normal((1, 2, 64)), N, axis=0)
    v = rng.standard_normal((N, 2, 64))
    q = rng.standard_normal((4, 64))
    o, lse = O.attention(q, k, v, 0.125)
    for h in range(4):
        np.testing.assert_allclose(o[h], v[:, h // 2].mean(axis=0), atol=1e-13)
    k2 = rng.standard_normal((N, 2, 64))
    o, lse = O.attention(np.zeros((4, 64)), k2, v, 0.125)
    for h in range(4):
        np.testing.assert_allclose(o[h], v[:, h // 2].mean(axis=0), atol=1e-13)
        assert abs(lse[h] - math.log(N)) < 1e-13


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(12)
    N, D = 50, 64
    q = rng.standard_normal((1, D))
    k = rng.standard_normal((N, 1, D)) * 0.01
    k[17, 0] = q[0] * 100.0
    v = rng.standard_normal((N, 1, D))
    o, _ = O.attention(q, k, v, 1.0)
    np.testing.assert_allclose(o[0], v[17, 0], atol=1e-12)


def test_gqa_head_mapping():
    # query head h must read KV head h // g (consecutive groups)
    N, D = 9, 8
    rng = np.random.default_rng(13)
    k = rng.standard_normal((N, 4, D))
    v = np.zeros((N, 4, D))
    for j in range(4):
        v[:, j, :] = j + 1.0
    o, _ = O.attention(rng.standard_normal((16, D)), k, v, 0.3)
    for h in range(16):
        np.testing.assert_allclose(o[h], h // 4 + 1.0, atol=1e-13)


def test_attention_linear_in_v_and_permutation_invariant():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((2, 16)); k = rng.standard_normal((20, 1, 16))
    v1 = rng.standard_normal((20, 1, 16)); v2 = rng.standard_normal((20, 1, 16))
    o1, _ = O.attention(q, k, v1, 0.25); o2, _ = O.attention(q, k, v2, 0.25)
    o3, _ = O.attention(q, k, 3 * v1 - v2, 0.25)
    np.testing.assert_allclose(o3, 3 * o1 - o2, atol=1e-12)
    perm = rng.permutation(20)
    o4, l4 = O.attention(q, k[perm], v1[perm], 0.25)
    o5, l5 = O.attention(q, k, v1, 0.25)
    np.testing.assert_allclose(o4, o5, atol=1e-13); np.testing.assert_allclose(l4, l5, atol=1e-13)


@pytest.mark.parametrize("N,Hq,Hkv,D", [(1, 2, 1, 4), (5, 4, 2, 8), (8, 3, 3, 6)])
def test_attention_matches_scalar_twin(N, Hq, Hkv, D):
    rng = np.random.default_rng(15 + N)
    q = rng.standard_normal((Hq, D)); k = rng.standard_normal((N, Hkv, D)); v = rng.standard_normal((N, Hkv, D))
    o, lse = O.attention(q, k, v, 1 / math.sqrt(D))
    ob, lb = BR.attention_py(q.tolist(), k.tolist(), v.tolist(), 1 / math.sqrt(D))
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lb, atol=1e-12)


# ------------------------------------------------------------------ merge

def test_merge_golden(golden):
    for c in golden["merge_lse"]["cases"]:
        ls = np.array([[(-np.inf if x == "-inf" else x) for x in row] for row in c["lse"]], dtype=np.float64)
        o, lse = O.merge_lse(np.array(c["o"], dtype=np.float64), ls)
        np.testing.assert_allclose(o, c["o_out"], atol=1e-13, err_msg=c["why"])
        np.testing.assert_allclose(lse, c["lse_out"], atol=1e-13, err_msg=c["why"])


def test_merge_of_only_empty_partitions():
    o, lse = O.merge_lse(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_split_then_merge_equals_unsplit():
    rng = np.random.default_rng(16)
    N, Hq, Hkv, D = 97, 8, 2, 16
    q = rng.standard_normal((Hq, D)); k = rng.standard_normal((N, Hkv, D)); v = rng.standard_normal((N, Hkv, D))
    o_ref, l_ref = O.attention(q, k, v, 0.25)
    for trial in range(5):
        labels = rng.integers(0, 6, size=N)
        parts = [np.nonzero(labels == j)[0] for j in range(7)]  # part 6 is empty
        parts.append(np.array([int(rng.integers(0, N))]))  # a singleton (duplicated token removed below)
        parts[int(labels[parts[-1][0]])] = np.setdiff1d(parts[int(labels[parts[-1][0]])], parts[-1])
        res = [O.attention_subset(q, k, v, p, 0.25) for p in parts]
        o, l = O.merge_lse(np.stack([r[0] for r in res]), np.stack([r[1] for r in res]))
        np.testing.assert_allclose(o, o_ref, atol=1e-12)
        np.testing.assert_allclose(l, l_ref, atol=1e-12)
        # order independence
        perm = rng.permutation(len(res))
        o2, l2 = O.merge_lse(np.stack([res[i][0] for i in perm]), np.stack([res[i][1] for i in perm]))
        np.testing.assert_allclose(o2, o, atol=1e-13)


def test_merge_is_associative_and_matches_scalar_twin():
    rng = np.random.default_rng(17)
    parts = [(rng.standard_normal((3, 5)), rng.standard_normal(3) * 4) for _ in range(4)]
    o_all, l_all = O.merge_lse(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    a = O.merge_lse(np.stack([parts[0][0], parts[1][0]]), np.stack([parts[0][1], parts[1][1]]))
    b = O.merge_lse(np.stack([parts[2][0], parts[3][0]]), np.stack([parts[2][1], parts[3][1]]))
    o2, l2 = O.merge_lse(np.stack([a[0], b[0]]), np.stack([a[1], b[1]]))
    np.testing.assert_allclose(o2, o_all, atol=1e-13); np.testing.assert_allclose(l2, l_all, atol=1e-13)
    ob, lb = BR.merge_py([(p[0].tolist(), p[1].tolist()) for p in parts])
    np.testing.assert_allclose(o_all, ob, atol=1e-13); np.testing.assert_allclose(l_all, lb, atol=1e-13)


# ------------------------------------------------------------------ placement

def test_split_point_golden(golden):
    for c in golden["split_point"]["cases"]:
        assert O.contig_split_point(c["r"], c["L"]) == c["n_host"], c["why"]


def test_paged_slot_golden(golden):
    for c in golden["paged_slot"]["cases"]:
        assert O.paged_slot(c["table"], c["b"], c["t"], c["P"]) == (c["tier"], c["row"]), c["why"]


def test_contig_slots_are_injective_and_cover():
    # unequal strides (host 16, device 21 rows per sequence) so that a swap of
    # the two strides, or of the tiers they belong to, changes the rows
    lens = [5, 1, 9, 16]
    hs, ds = 16, 21
    for r in (0.0, 0.3, 0.5, 1.0):
        seen = set()
        for b, L in enumerate(lens):
            nh = O.contig_split_point(r, L)
            for t in range(L):
                tier, row = O.contig_slot(b, t, L, r, hs, ds)
                # brute-force statement of the layout
                assert tier == (1 if t < nh else 0)
                assert row == (b * hs + t if tier else b * ds + t - nh)
                assert (tier, row) not in seen
                seen.add((tier, row))
        assert len(seen) == sum(lens)


def test_contig_slot_golden_unequal_strides():
    # sequence 2 of a cache with 10 host rows and 7 device rows per sequence,
    # L = 10, r = 0.7 (7 host tokens, see the split-point golden case):
    # token 6 is host row 2*10 + 6 = 26; token 7 is the first device token,
    # device row 2*7 + 0 = 14; token 9 is device row 2*7 + 2 = 16
    assert O.contig_slot(2, 6, 10, 0.7, 10, 7) == (1, 26)
    assert O.contig_slot(2, 7, 10, 0.7, 10, 7) == (0, 14)
    assert O.contig_slot(2, 9, 10, 0.7, 10, 7) == (0, 16)


def test_paged_table_slots_injective_and_ratio():
    lens = [33, 1, 160, 47]
    table, nh, nd = paged_table(3, lens, 16, 0.8)
    seen = set()
    host = 0
    for b, L in enumerate(lens):
        npg = (L + 15) // 16
        host += sum(int(table[b, j]) & 1 for j in range(npg))
        assert sum(int(table[b, j]) & 1 for j in range(npg)) == math.floor(0.8 * npg)
        for t in range(L):
            s = O.paged_slot(table, b, t, 16)
            assert s not in seen
            seen.add(s)
            assert s[1] < 16 * (nh if s[0] else nd)
    assert host == nh


def test_paged_layout_gives_same_attention_as_contiguous():
    # gather rows through a page table and attend: must equal attention over
    # the logical order (the result does not depend on where rows live)
    rng = np.random.default_rng(18)
    L, Hkv, D = 70, 2, 8
    k = rng.standard_normal((L, Hkv, D)); v = rng.standard_normal((L, Hkv, D))
    q = rng.standard_normal((4, D))
    table, nh, nd = paged_table(5, [L], 16, 0.5)
    host_k = np.zeros((nh * 16, Hkv, D)); dev_k = np.zeros((nd * 16, Hkv, D))
    host_v = np.zeros_like(host_k); dev_v = np.zeros_like(dev_k)
    for t in range(L):
        tier, row = O.paged_slot(table, 0, t, 16)
        (host_k if tier else dev_k)[row] = k[t]
        (host_v if tier else dev_v)[row] = v[t]
    kk = np.stack([(host_k if O.paged_slot(table, 0, t, 16)[0] else dev_k)[O.paged_slot(table, 0, t, 16)[1]] for t in range(L)])
    vv = np.stack([(host_v if O.paged_slot(table, 0, t, 16)[0] else dev_v)[O.paged_slot(table, 0, t, 16)[1]] for t in range(L)])
    o1, l1 = O.attention(q, kk, vv, 0.3)
    o2, l2 = O.attention(q, k, v, 0.3)
    np.testing.assert_allclose(o1, o2, atol=1e-14)


# ------------------------------------------------------------------ decode pipeline

def _tiny_inputs(seed, N, Hq, Hkv, D):
    q = normal_bf16(seed, 1, (Hq, D)); k = normal_bf16(seed, 2, (N, Hkv, D)); v = normal_bf16(seed, 3, (N, Hkv, D))
    return q, k, v


def test_decode_sequence_matches_scalar_pipeline():
    # full pipeline re-stated with the scalar twin: rotate keys at their own
    # positions, round to bf16, rotate the query at N-1, attend.
    N, Hq, Hkv, D, theta = 6, 4, 2, 8, 1e4
    q, k, v = _tiny_inputs(21, N, Hq, Hkv, D)
    o, lse = O.decode_sequence(q, k, v, N - 1, theta, 1 / math.sqrt(D))
    kf = O.bf16_to_f64(k); vf = O.bf16_to_f64(v); qf = O.bf16_to_f64(q)
    kr = [[BR.rope_neox_py(list(kf[t, j]), t, theta) for j in range(Hkv)] for t in range(N)]
    kr = [[list(O.bf16_to_f64(O.bf16_rne_bits(np.array(row)))) for row in tok] for tok in kr]
    qr = [BR.rope_neox_py(list(qf[h]), N - 1, theta) for h in range(Hq)]
    ob, lb = BR.attention_py(qr, kr, vf.tolist(), 1 / math.sqrt(D))
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lb, atol=1e-12)


def test_decode_batch_matches_scalar_pipeline_per_sequence():
    # a ragged batch (1, 3 and 6 cached tokens) with each query at its own
    # position: every sequence is re-stated with the scalar twin (keys rotated
    # at their positions and rounded to bf16, query rotated at q_pos[b]); a
    # mix-up of sequences, lengths or positions fails
    Hq, Hkv, D, theta, scale = 4, 2, 8, 1e4, 0.3
    lens = [1, 3, 6]
    qpos = [0, 2, 5]
    qb = normal_bf16(41, 1, (len(lens), Hq, D))
    caches = [(normal_bf16(41 + b, 2, (L, Hkv, D)), normal_bf16(41 + b, 3, (L, Hkv, D)))
              for b, L in enumerate(lens)]
    o, lse = O.decode_batch(qb, caches, qpos, theta, scale)
    assert o.shape == (3, Hq, D) and lse.shape == (3, Hq)
    for b, (kb, vb) in enumerate(caches):
        kf = O.bf16_to_f64(kb); vf = O.bf16_to_f64(vb); qf = O.bf16_to_f64(qb[b])
        kr = [[list(O.bf16_to_f64(O.bf16_rne_bits(np.array(BR.rope_neox_py(list(kf[t, j]), t, theta)))))
               for j in range(Hkv)] for t in range(lens[b])]
        qr = [BR.rope_neox_py(list(qf[h]), qpos[b], theta) for h in range(Hq)]
        ob, lb = BR.attention_py(qr, kr, vf.tolist(), scale)
        np.testing.assert_allclose(o[b], ob, atol=1e-12)
        np.testing.assert_allclose(lse[b], lb, atol=1e-12)
    # the single-token sequence returns its value exactly
    for h in range(Hq):
        assert np.array_equal(o[0, h], O.bf16_to_f64(caches[0][1][0, h // 2]))


def test_decode_shift_invariance_without_rounding():
    # shifting every position (keys and query) leaves the result unchanged
    N, Hq, Hkv, D, theta = 40, 4, 2, 16, 1e4
    q, k, v = _tiny_inputs(22, N, Hq, Hkv, D)
    kf = O.bf16_to_f64(k); vf = O.bf16_to_f64(v); qf = O.bf16_to_f64(q)
    def run(shift):
        kr = O.rope_neox(kf, (np.arange(N) + shift)[:, None], theta)
        qr = O.rope_neox(qf, np.full(Hq, N - 1 + shift), theta)
        return O.attention(qr, kr, vf, 0.25)
    o0, l0 = run(0)
    o1, l1 = run(4096)
    np.testing.assert_allclose(o1, o0, atol=1e-10)
    np.testing.assert_allclose(l1, l0, atol=1e-10)


def test_decode_split_equals_unsplit_and_sampled_heads():
    N, Hq, Hkv, D, theta = 130, 8, 2, 16, 5e5
    q, k, v = _tiny_inputs(23, N, Hq, Hkv, D)
    o, lse = O.decode_sequence(q, k, v, N - 1, theta, 0.25)
    nh = O.contig_split_point(0.3, N)
    o2, l2 = O.decode_sequence_split(q, k, v, N - 1, theta, 0.25,
                                     [np.arange(0, nh), np.arange(nh, N), np.array([], dtype=np.int64)])
    np.testing.assert_allclose(o2, o, atol=1e-12); np.testing.assert_allclose(l2, lse, atol=1e-12)
    o3, l3 = O.decode_sequence(q, k, v, N - 1, theta, 0.25, heads=[5, 1])
    np.testing.assert_allclose(o3, o[[5, 1]], atol=1e-14)


def test_append_expected_rows():
    rng = np.random.default_rng(24)
    kb = bf16_bits_from_f32(rng.standard_normal((2, 8)).astype(np.float32))
    vb = bf16_bits_from_f32(rng.standard_normal((2, 8)).astype(np.float32))
    k_rows, v_rows = O.append_expected_rows(kb, vb, 0, 1e4)
    assert np.array_equal(k_rows, kb) and np.array_equal(v_rows, vb)  # position 0: identity
    k_rows, _ = O.append_expected_rows(kb, vb, 300, 1e4)
    ref = np.array([BR.rope_neox_py(list(O.bf16_to_f64(kb[j])), 300, 1e4) for j in range(2)])
    assert np.array_equal(k_rows, O.bf16_rne_bits(ref))
    # projection mode rounds the projected value once
    x = rng.standard_normal((1, 8)); w = rng.standard_normal((8, 16)) * 0.1
    kv = O.project(x, w)[0].reshape(2, 8)
    k2, v2 = O.append_expected_rows(kv, kv, 0, 1e4, k_is_bits=False)
    assert np.array_equal(k2, O.bf16_rne_bits(kv)) and np.array_equal(v2, O.bf16_rne_bits(kv))


# ------------------------------------------------------------------ prefill

def test_prefill_single_row_equals_decode():
    N, Hq, Hkv, D, th = 50, 8, 2, 16, 1e4
    q, k, v = _tiny_inputs(31, N, Hq, Hkv, D)
    o_d, l_d = O.decode_sequence(q, k, v, N - 1, th, 0.25)
    o_p, l_p = O.prefill_sequence(q[None], k, v, N - 1, th, 0.25)
    np.testing.assert_allclose(o_p[0], o_d, atol=1e-13)
    np.testing.assert_allclose(l_p[0], l_d, atol=1e-13)


def test_prefill_all_new_first_row_is_v0_and_rows_are_causal():
    # all new KV (q_pos0 = 0): row 0 sees only token 0; changing later tokens
    # leaves earlier rows unchanged
    n, Hq, Hkv, D, th = 12, 4, 2, 8, 1e4
    q = normal_bf16(32, 1, (n, Hq, D)); k = normal_bf16(32, 2, (n, Hkv, D)); v = normal_bf16(32, 3, (n, Hkv, D))
    o, lse = O.prefill_sequence(q, k, v, 0, th, 0.35)
    for h in range(Hq):
        assert np.array_equal(o[0, h], O.bf16_to_f64(v[0, h // 2]))
    k2 = k.copy(); v2 = v.copy()
    k2[7:] = normal_bf16(33, 2, (n - 7, Hkv, D)); v2[7:] = normal_bf16(33, 3, (n - 7, Hkv, D))
    o2, l2 = O.prefill_sequence(q, k2, v2, 0, th, 0.35)
    np.testing.assert_array_equal(o2[:7], o[:7])
    assert np.abs(o2[7:] - o[7:]).max() > 1e-3


def test_prefill_matches_scalar_twin_with_cached_prefix():
    N0, n, Hq, Hkv, D, th = 5, 4, 4, 2, 8, 1e4
    N = N0 + n
    q = normal_bf16(34, 1, (n, Hq, D)); k = normal_bf16(34, 2, (N, Hkv, D)); v = normal_bf16(34, 3, (N, Hkv, D))
    o, lse = O.prefill_sequence(q, k, v, N0, th, 0.3)
    kf = O.bf16_to_f64(k); qf = O.bf16_to_f64(q)
    kr = [[list(O.bf16_to_f64(O.bf16_rne_bits(np.array(BR.rope_neox_py(list(kf[t, j]), t, th)))))
           for j in range(Hkv)] for t in range(N)]
    qr = [[BR.rope_neox_py(list(qf[j, h]), N0 + j, th) for h in range(Hq)] for j in range(n)]
    ob, lb = BR.prefill_py(qr, kr, O.bf16_to_f64(v).tolist(), [N0 + j for j in range(n)], 0.3)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lb, atol=1e-12)
