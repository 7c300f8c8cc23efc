"""The decode step captured into a HIP graph: every replay must equal the
eager result bit for bit (same kernels, same inputs; each work unit writes its
own split slot, so the dynamic unit order does not change any value).

Replays are interleaved with eager work and synchronizations, as a serving
loop would run them, and the outputs are cleared before each replay so a
replay that skipped a kernel would be caught.
"""
import math

import numpy as np
import pytest

import oracle as O
from synth import TensorId, kv_raw, normal_bf16, paged_table, query

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dk():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import decode_attention_host_amd as dk
    dk.reset_tuning()
    return dk


def _check_replays(dk, step, bufs, n=4):
    import torch
    step()
    torch.cuda.synchronize()
    ref_o = bufs.out_o.clone()
    ref_l = bufs.out_lse.clone()
    g = dk.StepGraph(step)
    scratch = torch.randn(1 << 20, device="cuda")
    for i in range(n):
        bufs.out_o.fill_(float("nan"))
        bufs.out_lse.fill_(float("nan"))
        scratch.mul_(1.0001).add_(1.0)   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs.out_o, ref_o), f"replay {i}: o differs from the eager step"
        assert torch.equal(bufs.out_lse, ref_l), f"replay {i}: lse differs from the eager step"
    return ref_o, ref_l


def test_graph_replays_contiguous_split(dk):
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, hq, hkv, d, r, th = [3000, 517], 32, 8, 128, 0.6, 5e5
    ks, vs = kv_raw(61, lens, hkv, d)
    qb = query(61, 2, hq, d)
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th)
    q = torch.from_numpy(qb.view(np.int16)).cuda()
    qpos = torch.tensor([n - 1 for n in lens], dtype=torch.int32, device="cuda")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sidx = torch.arange(2, dtype=torch.int32, device="cuda")
    k_new = torch.from_numpy(np.stack([k[-1] for k in ks]).view(np.int16)).cuda()
    v_new = torch.from_numpy(np.stack([v[-1] for v in vs]).view(np.int16)).cuda()
    bufs = dk.alloc_decode_buffers(cache, 2, hq, lens, r)

    def step():
        dk.project_rope_append(cache, 2, sl, r, sidx, qpos, k_new=k_new, v_new=v_new, rope_theta=th)
        dk.decode_attn_split(cache, q, qpos, sl, r, 1 / math.sqrt(d), th, bufs=bufs)
        dk.merge_lse(bufs.part_o, bufs.part_lse, bufs.split_offsets, 2, hq, d, out_o=bufs.out_o,
                     out_lse=bufs.out_lse)

    o, l = _check_replays(dk, step, bufs)
    for b in range(2):
        ro, rl = O.decode_sequence(qb[b], ks[b], vs[b], lens[b] - 1, th, 1 / math.sqrt(d))
        assert np.abs(o[b].cpu().numpy() - ro).max() < 2e-3
        assert np.abs(l[b].cpu().numpy() - rl).max() < 2e-3
    cache.free()


def test_graph_replays_fused_paged(dk):
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    hkv, hq, d, hid, th, B = 8, 32, 128, 1024, 5e5, 3
    lens = [100, 1500, 40]
    ntok = [L + 1 for L in lens]
    ks, vs = kv_raw(62, lens, hkv, d)
    pt, nh, nd = paged_table(62, ntok, 16, 0.8)
    cache = paged_cache(hkv, d, ntok, pt, nh, nd, ks, vs, th, upto=lens)
    x = torch.from_numpy(normal_bf16(62, TensorId.X, (B, hid)).view(np.int16)).cuda()
    wk = torch.from_numpy(normal_bf16(62, TensorId.WK, (hid, hkv * d), std=0.02).view(np.int16)).cuda()
    wv = torch.from_numpy(normal_bf16(62, TensorId.WV, (hid, hkv * d), std=0.02).view(np.int16)).cuda()
    q = torch.from_numpy(query(62, B, hq, d).view(np.int16)).cuda()
    pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sidx = torch.arange(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(dk.append_workspace_bytes(B, hid, hkv * d), dtype=torch.uint8, device="cuda")
    bufs = dk.alloc_decode_buffers(cache, B, hq, ntok, 0.0)
    ntok_dev = torch.tensor(ntok, dtype=torch.int32, device="cuda")

    def step():
        dk.project_rope_append(cache, B, None, 0.0, sidx, pos, x=x, wk=wk, wv=wv, rope_theta=th,
                               workspace=ws)
        dk.decode_attn_split(cache, q, pos, ntok_dev, 0.0, 1 / math.sqrt(d), th, bufs=bufs)
        dk.merge_lse(bufs.part_o, bufs.part_lse, bufs.split_offsets, B, hq, d, out_o=bufs.out_o,
                     out_lse=bufs.out_lse)

    _check_replays(dk, step, bufs)
    cache.free()


def test_graph_replays_fused_prefill(dk):
    # the fused prefill step (append of the new rows, staging, prefill launch
    # with writer workgroups for the cache slots, merge): the captured graph
    # must replay it exactly
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    lens, news, hq, hkv, d, r, th = [900, 300], [400, 300], 32, 8, 128, 0.7, 5e5
    ks, vs = kv_raw(63, lens, hkv, d)
    pre = [L - n for L, n in zip(lens, news)]
    cache = contiguous_cache(hkv, d, lens, r, ks, vs, th, upto=pre)
    q = torch.from_numpy(np.concatenate([normal_bf16(63 + b, 1, (n, hq, d)) for b, n in enumerate(news)])
                         .view(np.int16)).cuda()
    kn = torch.from_numpy(np.concatenate([k[p:] for k, p in zip(ks, pre)]).view(np.int16)).cuda()
    vn = torch.from_numpy(np.concatenate([v[p:] for v, p in zip(vs, pre)]).view(np.int16)).cuda()
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    T = int(q_start[-1])
    info = dk.prefill_fused_plan(cache, 2, hq, q_start, pre, lens, r)
    ws = torch.empty(info["workspace_bytes"], dtype=torch.uint8, device="cuda")

    class Bufs:
        out_o = torch.empty((T, hq, d), dtype=torch.float32, device="cuda")
        out_lse = torch.empty((T, hq), dtype=torch.float32, device="cuda")

    def step():
        dk.prefill_fused(cache, q, q_start, pre, lens, r, 1 / math.sqrt(d), th, k_new=kn, v_new=vn,
                         workspace=ws, out_o=Bufs.out_o, out_lse=Bufs.out_lse)

    ref_o, ref_l = _check_replays(dk, step, Bufs)
    ro, rl = O.prefill_sequence(np.concatenate([normal_bf16(63 + 1, 1, (news[1], hq, d))]), ks[1], vs[1], pre[1], th,
                                1 / math.sqrt(d), heads=[0, 9, 31])
    o = ref_o.cpu().numpy().astype(np.float64)[q_start[1]:, [0, 9, 31]]
    l = ref_l.cpu().numpy().astype(np.float64)[q_start[1]:, [0, 9, 31]]
    assert np.abs(o - ro).max() < 2e-3 and np.abs(l - rl).max() < 2e-3
    # the captured plan is held while its graph may replay, and released on
    # request once the graph is gone (the helper's graph went out of scope)
    torch.cuda.synchronize()
    st = dk.plan_cache_stats()
    assert st["captured"] >= 1 and st["pinned_bytes"] > 0, st
    dk.plan_cache_release_captured()
    st2 = dk.plan_cache_stats()
    assert st2["captured"] == 0 and st2["entries"] >= 1, st2
    # the plan still serves eager calls
    step()
    torch.cuda.synchronize()
    assert torch.equal(Bufs.out_o, ref_o) and torch.equal(Bufs.out_lse, ref_l)
    cache.free()
