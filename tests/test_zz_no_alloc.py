"""The allocation-free decode step (dkv_decode_step_static) against the step on
a caller workspace (dkv_decode_step): same outputs within the parity bar and
the same appended cache rows, on calls in a row: the second smaller, so the
static scratch holds the first call's contents when the second starts, and a
third larger than both, whose counters would reach where the earlier calls kept
partials and page lists if the scratch did not keep its counters apart."""
import math

import numpy as np
import pytest

import oracle as O
from synth import kv_raw, paged_table, query

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


def _bits(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _dev(a):
    import torch
    return torch.tensor(np.asarray(a, dtype=np.int32), dtype=torch.int32, device="cuda")


def _case(dk, lens, hq, hkv, d, frac, seed):
    """Both entry points on two identical paged caches; returns (outputs, pools)."""
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    th = 5e5
    full = [L + 1 for L in lens]
    ks, vs = kv_raw(seed, full, hkv, d)
    qb = query(seed, len(lens), hq, d)
    pt, nh, nd = paged_table(seed, full, 16, frac)
    caches = [paged_cache(hkv, d, full, pt, nh, nd, ks, vs, th, upto=lens) for _ in range(2)]
    k_new = _bits(np.stack([k[L] for k, L in zip(ks, lens)]))
    v_new = _bits(np.stack([v[L] for v, L in zip(vs, lens)]))
    B = len(lens)
    outs = []
    for i, cache in enumerate(caches):
        oo = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
        ol = torch.empty((B, hq), dtype=torch.float32, device="cuda")
        args = (cache, _bits(qb), _dev(lens), _dev(lens), 0.0, 1 / math.sqrt(d), th)
        if i == 0:
            dk.decode_step(*args, k_new=k_new, v_new=v_new, out_o=oo, out_lse=ol)
        else:
            dk.decode_step_static(*args, k_new=k_new, v_new=v_new, out_o=oo, out_lse=ol)
        torch.cuda.synchronize()
        outs.append((oo.cpu().numpy(), ol.cpu().numpy()))
    # the rows of tokens 0 .. L_b of every sequence (the last one appended by the call)
    rows = []
    for cache in caches:
        pools = {(1, "k"): cache.host_view("k"), (1, "v"): cache.host_view("v"),
                 (0, "k"): cache.dev_k.view(torch.int16).cpu().numpy(),
                 (0, "v"): cache.dev_v.view(torch.int16).cpu().numpy()}
        got = []
        for b, L in enumerate(lens):
            for t in range(L + 1):
                tier, row = O.paged_slot(pt, b, t, 16)
                got.append(np.stack([pools[(tier, "k")][row].view(np.int16), pools[(tier, "v")][row].view(np.int16)]))
        rows.append(np.stack(got))
        cache.free()
    return outs, rows


def test_static_scratch_step_matches_workspace_step_in_a_row(dk):
    # first call: 3 sequences, 32 / 8 heads; second call smaller: 1 sequence, 8 / 2 heads, D = 64;
    # third call larger: 6 sequences, 32 / 8 heads
    for lens, hq, hkv, d, frac, seed in (([700, 16, 1500], 32, 8, 128, 0.8, 91), ([300], 8, 2, 64, 0.5, 92),
                                         ([2000, 5, 900, 64, 3100, 1], 32, 8, 128, 0.3, 93)):
        (ref, got), (ra, rb) = _case(dk, lens, hq, hkv, d, frac, seed)
        eo = float(np.abs(got[0] - ref[0]).max())
        el = float(np.abs(got[1] - ref[1]).max())
        print(f"lens {lens}: max|do|={eo:.3g} max|dlse|={el:.3g}", flush=True)
        assert eo <= TOL and el <= TOL
        assert np.array_equal(ra, rb)  # every token's rows, the appended one included


def test_static_scratch_rejects_oversized_shapes(dk):
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    from decode_attention_host_amd._lib import DkvError
    # 512 sequences x 128 query heads: the partial slots (about 1800 of
    # 128 x 128 fp32) exceed the static scratch
    B, hq, hkv, d = 512, 128, 16, 128
    pt = np.zeros((B, 1), dtype=np.int32)
    cache = dk.KVCache(hkv, d, host_rows=0, dev_rows=16, page_size=16, page_table=pt)
    q = torch.zeros((B, hq, d), dtype=torch.int16, device="cuda")
    sl = torch.zeros(B, dtype=torch.int32, device="cuda")
    oo = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
    with pytest.raises(DkvError, match="static"):
        dk.decode_step_static(cache, q, sl, sl, 0.0, 0.1, 1e4, out_o=oo)
    cache.free()
