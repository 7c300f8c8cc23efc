"""Measurement self-consistency on the GPU.

The bandwidth probe and the live kernel timing feed every roofline figure, so
they are checked against what the hardware can do: a zero-copy read of mapped
host memory and a DMA copy stay at or below the host link's nominal rate, an
HBM streaming read stays below the HBM peak, and the per-kernel HIP-event
timing of an attention call fits inside the same call timed around it on the
stream.  (SplitKernel README, Overview: the planner splits work by the tiers'
measured bandwidth, so these numbers must be physically possible.)
"""
import glob
import math
import os

import numpy as np
import pytest
import torch

from synth import normal_bf16

pytestmark = pytest.mark.gpu

HBM_PEAK_GBS = 8000.0


@pytest.fixture(scope="module")
def dk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import decode_attention_host_amd as dk
    dk.reset_tuning()
    return dk


def link_nominal_gbs():
    """PCIe link speed x width of the visible GPU from sysfs (128b/130b), per
    direction; 64 GB/s (5.0 x16) when sysfs does not say."""
    bus = torch.cuda.get_device_properties(0).pci_bus_id
    for dev in glob.glob("/sys/class/drm/card*/device"):
        try:
            sp = float(open(os.path.join(dev, "current_link_speed")).read().split()[0])
            wd = int(open(os.path.join(dev, "current_link_width")).read().strip())
            uevent = open(os.path.join(dev, "uevent")).read().lower()
        except (OSError, ValueError, IndexError):
            continue
        if f":{bus:02x}:" in uevent:
            return sp * wd * (128.0 / 130.0) / 8.0
    return 64.0


def test_host_probe_within_link_nominal(dk):
    nominal = link_nominal_gbs()
    n = 64 << 20
    hb = dk.HostBuffer(n)
    try:
        hb.numpy(np.uint8)[:] = 7
        for nt in (True, False):
            r = dk.probe_read(hb.dev_ptr, n, 32, nontemporal=nt, iters=2)
            print(f"zero-copy nt={nt}: {r['read_gbs']:.2f} GB/s (nominal {nominal:.1f})", flush=True)
            assert 1.0 < r["read_gbs"] <= 1.02 * nominal
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        r = dk.probe_read(hb.dev_ptr, n, 32, iters=2, dma_dst=dst, dma_src_host=hb.host_ptr)
        torch.cuda.synchronize()
        print(f"DMA: {r['dma_gbs']:.2f} GB/s", flush=True)
        assert 1.0 < r["dma_gbs"] <= 1.02 * nominal
        # the DMA copy moved the bytes
        assert bool((dst == 7).all())
    finally:
        hb.free()


def test_hbm_probe_below_peak(dk):
    big = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    r = dk.probe_read(big.data_ptr(), big.numel(), 512, nontemporal=True, iters=3)
    print(f"HBM read: {r['read_gbs']:.0f} GB/s", flush=True)
    assert 1000.0 < r["read_gbs"] <= HBM_PEAK_GBS
    del big


def test_kernel_timing_fits_inside_the_call(dk):
    hq, hkv, d, L, ratio, theta = 32, 8, 128, 8192, 0.5, 5e5
    from decode_attention_host_amd.cache_build import contiguous_cache
    k = normal_bf16(3, 1, (L, hkv, d))
    v = normal_bf16(3, 2, (L, hkv, d))
    q = torch.from_numpy(normal_bf16(3, 0, (1, hq, d)).view(np.int16)).cuda()
    lens = [L]
    cache = contiguous_cache(hkv, d, lens, ratio, [k], [v], theta)
    try:
        qpos = torch.tensor([L - 1], dtype=torch.int32, device="cuda")
        bufs = None
        for _ in range(3):
            _, _, bufs = dk.decode(cache, q, qpos, lens, ratio, 1 / math.sqrt(d), theta, bufs=bufs)
        torch.cuda.synchronize()
        dk.kernel_timing(True)
        dk.kernel_timing_read("attn")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        iters = 10
        e0.record()
        for _ in range(iters):
            dk.decode(cache, q, qpos, lens, ratio, 1 / math.sqrt(d), theta, bufs=bufs)
        e1.record()
        torch.cuda.synchronize()
        c, ms = dk.kernel_timing_read("attn")
        dk.kernel_timing(False)
        call_ms = e0.elapsed_time(e1)
        print(f"attention kernel {ms / max(c, 1):.4f} ms x {c}; calls {call_ms / iters:.4f} ms", flush=True)
        assert c == iters
        assert 0.0 < ms <= call_ms * 1.001
        # the host-tier bytes cannot have moved faster than the link allows
        host_bytes = int(math.floor(ratio * L)) * hkv * d * 2 * 2
        assert host_bytes / (ms / c * 1e-3) / 1e9 <= 1.02 * link_nominal_gbs()
    finally:
        dk.kernel_timing(False)
        cache.free()


@pytest.mark.parametrize("form", ["split", "fused"])
def test_workgroup_trace_accounts_for_every_unit(dk, form):
    """dkv_attn_trace: every workgroup of a decode launch records its role,
    a start no later than its end, and its units; the units of each role add up
    to the work the host enumeration of the same call lists (items x KV heads)."""
    hq, hkv, d, lens, ratio, theta = 32, 8, 128, [9000, 3000], 0.4, 5e5
    from decode_attention_host_amd.cache_build import contiguous_cache
    ks = [normal_bf16(4, 1 + b, (L, hkv, d)) for b, L in enumerate(lens)]
    vs = [normal_bf16(4, 5 + b, (L, hkv, d)) for b, L in enumerate(lens)]
    q = torch.from_numpy(normal_bf16(4, 0, (2, hq, d)).view(np.int16)).cuda()
    cache = contiguous_cache(hkv, d, lens, ratio, ks, vs, theta)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    items, _, _, info = dk.plan_inspect(cache.desc(), 2, hq, lens, ratio, cus)
    n_host = int((items[:, 0] == 1).sum())
    n_dev = int((items[:, 0] == 0).sum())
    grid = 4096
    buf = torch.zeros((grid, 4), dtype=torch.int64, device="cuda")
    try:
        qpos = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device="cuda")
        dk.attn_trace(buf)
        if form == "split":
            dk.decode(cache, q, qpos, lens, ratio, 1 / math.sqrt(d), theta)
        else:
            ws = dk.decode_step_workspace(cache, 2, hq, ratio)
            dk.decode_step(cache, q, qpos, torch.tensor(lens, dtype=torch.int32, device="cuda"), ratio,
                           1 / math.sqrt(d), theta, workspace=ws)
        torch.cuda.synchronize()
    finally:
        dk.attn_trace(None)
        cache.free()
    t = buf.cpu().numpy()
    used = t[t[:, 0] != 0]
    print(f"{form}: {len(used)} workgroups traced, host items {n_host}, HBM items {n_dev}", flush=True)
    assert len(used) == info["host_wgs"] + info["dev_wgs"]
    assert np.all(used[:, 1] >= used[:, 0])
    host = used[used[:, 2] == 1]
    dev = used[used[:, 2] == 0]
    assert len(host) == info["host_wgs"] and len(dev) == info["dev_wgs"]
    # every (item, KV head) is processed once: the items the host enumeration
    # lists per KV head, times the KV heads
    assert int(host[:, 3].sum()) == n_host * hkv
    assert int(dev[:, 3].sum()) == n_dev * hkv
