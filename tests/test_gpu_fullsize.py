"""GPU parity at the workloads' full sizes, in the launch configuration the
bench uses (default planner tuning), against the fp64 oracle.

Where the oracle over every head would take too long, sampled query heads or
sequences are compared (each sampled output is the complete oracle over all
its tokens).  Same bar as the small cases: max |do|, |dlse| <= 2e-3.
"""
import math

import numpy as np
import pytest

import oracle as O
from synth import TensorId, kv_raw, normal_bf16, paged_table, query, workload

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


def _decode(dk, cache, qb, lens, ratio, theta, q_pos=None):
    import torch
    B, hq, d = qb.shape
    q = torch.from_numpy(qb.view(np.int16)).cuda()
    qp = torch.tensor([n - 1 for n in lens] if q_pos is None else q_pos, dtype=torch.int32, device="cuda")
    o, lse, _ = dk.decode(cache, q, qp, lens, ratio, 1.0 / math.sqrt(d), theta)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _step(dk, cache, qb, ks, vs, lens, ratio, theta):
    """The one-launch fused step the bench times: each sequence's newest token
    (position L_b - 1, the bits already cached) appended again, then attention
    over all L_b tokens and the merge, in one launch."""
    import torch
    B, hq, d = qb.shape
    q = torch.from_numpy(qb.view(np.int16)).cuda()
    cached = torch.tensor([n - 1 for n in lens], dtype=torch.int32, device="cuda")
    k_new = torch.from_numpy(np.stack([k[-1] for k in ks]).view(np.int16)).cuda()
    v_new = torch.from_numpy(np.stack([v[-1] for v in vs]).view(np.int16)).cuda()
    ws = dk.decode_step_workspace(cache, B, hq, ratio)
    o, lse = dk.decode_step(cache, q, cached.clone(), cached, ratio, 1.0 / math.sqrt(d), theta,
                            k_new=k_new, v_new=v_new, workspace=ws)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(o, lse, ref_o, ref_l, what):
    eo = np.abs(o - ref_o).max()
    el = np.abs(lse - ref_l).max()
    print(f"{what}: max|do|={eo:.3g} max|dlse|={el:.3g}", flush=True)
    assert eo <= TOL and el <= TOL, what


@pytest.mark.parametrize("ratio", [None, 0.25, 0.0079])
def test_llama3_8b_32k_all_heads(dk, ratio):
    """The headline 32k layer at its own ratio (all host), at a quarter offloaded
    and at the 1M layer's best-split share r* (0.79%: 258 host tokens), split
    form and fused step."""
    from decode_attention_host_amd.cache_build import contiguous_cache
    cfg = workload("llama3_8b_32k")
    L, hkv, hq, d, th = cfg["lens"][0], cfg["hkv"], cfg["hq"], cfg["d"], cfg["theta"]
    r = cfg["ratio"] if ratio is None else ratio
    ks, vs = kv_raw(0, [L], hkv, d)
    qb = query(0, 1, hq, d)
    cache = contiguous_cache(hkv, d, [L], r, ks, vs, th)
    ro, rl = O.decode_sequence(qb[0], ks[0], vs[0], L - 1, th, 1 / math.sqrt(d))
    o, lse = _decode(dk, cache, qb, [L], r, th)
    _check(o[0], lse[0], ro, rl, f"llama3_8b_32k r={r} split form")
    o, lse = _step(dk, cache, qb, ks, vs, [L], r, th)
    _check(o[0], lse[0], ro, rl, f"llama3_8b_32k r={r} fused step")
    cache.free()


def test_opt_6_7b_b8_all_heads(dk):
    from decode_attention_host_amd.cache_build import contiguous_cache
    cfg = workload("opt_6_7b_b8")
    lens, hkv, hq, d, th, r = cfg["lens"], cfg["hkv"], cfg["hq"], cfg["d"], cfg["theta"], cfg["ratio"]
    ks, vs = kv_raw(0, lens, hkv, d)
    qb = query(0, cfg["batch"], hq, d)
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th)
    o, lse = _decode(dk, cache, qb, lens, r, th)
    fo, fl = _step(dk, cache, qb, ks, vs, lens, r, th)
    for b in range(cfg["batch"]):
        ro, rl = O.decode_sequence(qb[b], ks[b], vs[b], lens[b] - 1, th, 1 / math.sqrt(d))
        _check(o[b], lse[b], ro, rl, f"opt_6_7b_b8 seq {b} split form")
        _check(fo[b], fl[b], ro, rl, f"opt_6_7b_b8 seq {b} fused step")
    cache.free()


def test_llama3_8b_1m_ratios_sampled_heads(dk):
    from decode_attention_host_amd.cache_build import SplitView, contiguous_cache
    cfg = workload("llama3_8b_1m")
    L, hkv, hq, d, th = cfg["lens"][0], cfg["hkv"], cfg["hq"], cfg["d"], cfg["theta"]
    ks, vs = kv_raw(0, [L], hkv, d)
    qb = query(0, 1, hq, d)
    host_full = contiguous_cache(hkv, d, [L], 1.0, ks, vs, th)
    dev_full = contiguous_cache(hkv, d, [L], 0.0, ks, vs, th)
    heads = [0, 13, 31]  # KV heads 0, 3, 7
    ro, rl = O.decode_sequence(qb[0], ks[0], vs[0], L - 1, th, 1 / math.sqrt(d), heads=heads)
    # r* = BW_h / (BW_h + BW_d) with the measured 57.5 GB/s link and 7.2 TB/s
    # HBM read (0.79%), half of it, and three larger shares; both step forms
    for r in (0.0, 0.0040, 0.0079, 0.75, 1.0):
        view = SplitView(host_full, dev_full, L, r)
        o, lse = _decode(dk, view, qb, [L], r, th)
        _check(o[0, heads], lse[0, heads], ro, rl, f"llama3_8b_1m r={r} split form")
        o, lse = _step(dk, view, qb, ks, vs, [L], r, th)
        _check(o[0, heads], lse[0, heads], ro, rl, f"llama3_8b_1m r={r} fused step")
    host_full.free()
    dev_full.free()
    # the same tokens in permuted 16-token pages, all in HBM: the long HBM
    # range takes the planner's guided tail on the paged path
    from decode_attention_host_amd.cache_build import paged_cache
    pt, nh, nd = paged_table(1, [L], 16, 0.0)
    paged = paged_cache(hkv, d, [L], pt, nh, nd, ks, vs, th)
    o, lse = _decode(dk, paged, qb, [L], 0.0, th)
    _check(o[0, heads], lse[0, heads], ro, rl, "llama3_8b_1m paged, HBM")
    paged.free()


def test_fused_ragged_full_sampled_sequences(dk):
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    cfg = workload("fused_ragged")
    B, hkv, hq, d, th, hid = cfg["batch"], cfg["hkv"], cfg["hq"], cfg["d"], cfg["theta"], cfg["hidden"]
    lens = cfg["lens"]
    ntok = [L + 1 for L in lens]
    ks, vs = kv_raw(0, lens, hkv, d)
    pt, nh, nd = paged_table(0, ntok, cfg["page"], cfg["ratio"])
    cache = paged_cache(hkv, d, ntok, pt, nh, nd, ks, vs, th, page=cfg["page"], upto=lens)
    x = normal_bf16(0, TensorId.X, (B, hid))
    wk = normal_bf16(0, TensorId.WK, (hid, hkv * d), std=cfg["w_std"])
    wv = normal_bf16(0, TensorId.WV, (hid, hkv * d), std=cfg["w_std"])
    dk.project_rope_append(cache, B, None, 0.0, torch.arange(B, dtype=torch.int32, device="cuda"),
                           torch.tensor(lens, dtype=torch.int32, device="cuda"),
                           x=torch.from_numpy(x.view(np.int16)).cuda(), wk=torch.from_numpy(wk.view(np.int16)).cuda(),
                           wv=torch.from_numpy(wv.view(np.int16)).cuda(), rope_theta=th)
    qb = query(0, B, hq, d)
    o, lse = _decode(dk, cache, qb, ntok, 0.0, th)
    # the fused step: projection of the same hidden states, the same slots
    # written again, attention over L_b + 1 tokens and the merge in one launch
    cached = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ws = dk.decode_step_workspace(cache, B, hq, 0.0, hid)
    fo, fl = dk.decode_step(cache, torch.from_numpy(qb.view(np.int16)).cuda(), cached.clone(), cached, 0.0,
                            1.0 / math.sqrt(d), th, x=torch.from_numpy(x.view(np.int16)).cuda(),
                            wk=torch.from_numpy(wk.view(np.int16)).cuda(),
                            wv=torch.from_numpy(wv.view(np.int16)).cuda(), workspace=ws)
    torch.cuda.synchronize()
    fo, fl = fo.cpu().numpy().astype(np.float64), fl.cpu().numpy().astype(np.float64)
    kk = O.project(O.bf16_to_f64(x), O.bf16_to_f64(wk)).reshape(B, hkv, d)
    vv = O.project(O.bf16_to_f64(x), O.bf16_to_f64(wv)).reshape(B, hkv, d)
    order = np.argsort(lens)
    for b in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        kn, vn = O.append_expected_rows(kk[b], vv[b], lens[b], th, k_is_bits=False)
        for kvh in (0, 5):
            heads = list(range(kvh * 4, kvh * 4 + 4))
            kst = O.bf16_to_f64(O.bf16_rne_bits(
                O.rope_neox(O.bf16_to_f64(ks[b][:, kvh]), np.arange(lens[b]), th)))
            kst = np.concatenate([kst, O.bf16_to_f64(kn[kvh])[None]], axis=0)[:, None, :]
            vst = np.concatenate([O.bf16_to_f64(vs[b][:, kvh]), O.bf16_to_f64(vn[kvh])[None]], axis=0)[:, None, :]
            q_rot = O.rope_neox(O.bf16_to_f64(qb[b][heads]), np.full(4, lens[b]), th)
            ro, rl = O.attention(q_rot, kst, vst, 1 / math.sqrt(d))
            _check(o[b, heads], lse[b, heads], ro, rl, f"fused_ragged seq {b} (L={lens[b]}) kv head {kvh}")
            _check(fo[b, heads], fl[b, heads], ro, rl, f"fused_ragged seq {b} kv head {kvh}, fused step")
    cache.free()
