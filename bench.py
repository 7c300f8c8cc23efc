#!/usr/bin/env python3
"""Decode-attention benchmark: effective KV GB/s and latency per step vs offload ratio.

A step is one pass of the whole path on one batch: append of each sequence's
newest token (Neox RoPE of its key, bf16 store into its tier), split decode
attention over both tiers, and the LSE merge.  Inputs are seeded synthetic
tensors with the layer shapes of the workload (no weights, no datasets).

Default workload: LLaMA-3-8B attention layer, batch 1, 32 query / 8 KV heads,
head_dim 128, 32768 cached tokens, all of them in host-pinned memory.

Prints ONE JSON line with the headline value, the roofline of the attention
kernel (timed live with HIP events on its stream), the in-run bandwidth probe,
the offload-ratio sweep and the fp64 oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn effective KV GB/s & latency/token vs offload ratio; % of roofline"
PCIE_PEAK_GBS = 64.0      # PCIe 5.0 x16 per direction (128 GB/s bidirectional)
HBM_PEAK_GBS = 8000.0     # HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pcie_nominal_gbs(pci_bus_id: int | None):
    """Link speed x width from sysfs, 128b/130b encoding, per direction."""
    for dev in glob.glob("/sys/class/drm/card*/device"):
        try:
            sp = open(os.path.join(dev, "current_link_speed")).read().split()[0]
            wd = int(open(os.path.join(dev, "current_link_width")).read().strip())
            uevent = open(os.path.join(dev, "uevent")).read()
        except OSError:
            continue
        if pci_bus_id is not None and f":{pci_bus_id:02x}:" not in uevent.lower():
            continue
        gts = float(sp)
        return gts * wd * (128.0 / 130.0) / 8.0, f"{sp} GT/s x{wd}"
    return None, None


def kernel_src_sha():
    """Hash of the split attention kernel's own source: its definition, its
    launcher and the plan/argument structures it reads.  The stored traffic
    figure of that kernel stays valid while this hash matches."""
    import re
    csrc = os.path.join(ROOT, "decode_attention_host_amd", "csrc")
    k = open(os.path.join(csrc, "dkv_kernels.hip")).read()
    h_src = open(os.path.join(csrc, "dkv_internal.h")).read()
    a = re.search(r"__global__ __launch_bounds__\([^)]*\) void attn_split_kernel", k).start()
    a = k.rindex("template", 0, a)
    b = k.index("// ----", a)
    parts = [k[a:b]]
    parts += re.findall(r"static hipError_t launch_attn_d.*?\n}\n", k, re.S)
    for struct in ("PlanItem", "AttnArgs"):
        parts.append(re.search(r"struct %s \{.*?\n\};" % struct, h_src, re.S).group(0))
    parts += re.findall(r"constexpr int k(?:Tile|Threads) = \d+;", h_src)
    h = hashlib.sha256()
    for x in parts:
        h.update(x.encode())
    return h.hexdigest()[:16]


def build_workload(cfg, seed, host_flags):
    import numpy as np
    import torch

    import decode_attention_host_amd as dk
    from decode_attention_host_amd.cache_build import contiguous_cache
    from synth import kv_raw, query

    B, hq, hkv, d, lens = cfg["batch"], cfg["hq"], cfg["hkv"], cfg["d"], cfg["lens"]
    t0 = time.time()
    ks, vs = kv_raw(seed, lens, hkv, d)
    qb = query(seed, B, hq, d)
    log(f"[bench] inputs drawn in {time.time() - t0:.1f}s")
    t0 = time.time()
    cache = contiguous_cache(hkv, d, lens, cfg["ratio"], ks, vs, cfg["theta"], host_flags=host_flags)
    log(f"[bench] cache built (ratio {cfg['ratio']}) in {time.time() - t0:.1f}s")
    q = torch.from_numpy(qb.view(np.int16)).cuda()
    qpos = torch.tensor([n - 1 for n in lens], dtype=torch.int32, device="cuda")
    # the newest token of each sequence, appended every step
    k_new = torch.from_numpy(np.stack([k[-1] for k in ks]).view(np.int16)).cuda()
    v_new = torch.from_numpy(np.stack([v[-1] for v in vs]).view(np.int16)).cuda()
    return dict(ks=ks, vs=vs, qb=qb, q=q, qpos=qpos, cache=cache, k_new=k_new, v_new=v_new,
                seq_lens_dev=torch.tensor(lens, dtype=torch.int32, device="cuda"),
                sidx=torch.arange(B, dtype=torch.int32, device="cuda"))


def make_step(dk, cfg, w, cache, ratio, bufs):
    B, hq, d = cfg["batch"], cfg["hq"], cfg["d"]
    scale = 1.0 / math.sqrt(d)
    lens = cfg["lens"]

    def step():
        dk.project_rope_append(cache, B, w["seq_lens_dev"], ratio, w["sidx"], w["qpos"],
                               k_new=w["k_new"], v_new=w["v_new"], rope_theta=cfg["theta"])
        dk.decode_attn_split(cache, w["q"], w["qpos"], w["seq_lens_dev"], ratio, scale, cfg["theta"], bufs=bufs)
        dk.merge_lse(bufs.part_o, bufs.part_lse, bufs.split_offsets, B, hq, d, out_o=bufs.out_o,
                     out_lse=bufs.out_lse)
    return step


def run_probe(dk, w, nbytes_host):
    import torch
    cache = w["cache"]
    res = {}
    hb = cache.host_k
    if hb is not None:
        n = min(nbytes_host, hb.nbytes) // 16 * 16
        best = None
        sweep = []
        for nt in (True, False):
            for nwg in (32, 64, 128, 256, 512, 1024):
                r = dk.probe_read(hb.dev_ptr, n, nwg, nontemporal=nt, iters=5)
                sweep.append({"nwg": nwg, "nt": nt, "gbs": round(r["read_gbs"], 2)})
                if best is None or r["read_gbs"] > best[0]:
                    best = (r["read_gbs"], nwg, nt)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        dma = dk.probe_read(hb.dev_ptr, n, 256, iters=5, dma_dst=dst, dma_src_host=hb.host_ptr)
        res.update(host_zero_copy_gbs=round(best[0], 2), host_zero_copy_wgs=best[1],
                   host_zero_copy_nt=best[2], host_dma_gbs=round(dma["dma_gbs"], 2),
                   host_sweep=sweep)
        del dst
    big = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    best = (0.0, 0, False)
    hsweep = []
    for nt in (True, False):
        for nwg in (256, 512, 1024, 2048, 4096, 8192):
            r = dk.probe_read(big.data_ptr(), big.numel(), nwg, nontemporal=nt, iters=5)
            hsweep.append({"nwg": nwg, "nt": nt, "gbs": round(r["read_gbs"], 1)})
            if r["read_gbs"] > best[0]:
                best = (r["read_gbs"], nwg, nt)
    res["hbm_read_gbs"] = round(best[0], 1)
    res["hbm_read_wgs"] = best[1]
    res["hbm_read_nt"] = best[2]
    res["hbm_sweep"] = hsweep
    del big
    return res


def gpu_warm(step, seconds=0.3):
    """Run the step until the GPU is back at working clocks (it idles while the
    host builds caches or runs the oracle)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        step()
        torch.cuda.synchronize()


def graph_timing(dk, step, steps):
    """The same step captured once into a HIP graph, K replays timed back to back."""
    import torch
    g = dk.StepGraph(step)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def timed_loop(step, steps, warmup):
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def flushed_steps(dk, step, iters, flush):
    """Per-step times of `iters` steps with a read-only cache flush between
    them, and the library's per-kernel timing over the same steps."""
    import torch
    gpu_warm(step, 0.3)
    dk.kernel_timing(True)
    for k in dk.api.KERNELS:
        dk.kernel_timing_read(k)
    # steps back to back with a flush between them; the host runs ahead, so
    # each event pair brackets GPU work only
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    sink = torch.empty(iters, dtype=torch.float32, device="cuda")
    for i in range(iters):
        torch.sum(flush, dim=0, out=sink[i])
        ev[i][0].record()
        step()
        ev[i][1].record()
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in ev]
    kt = {k: dk.kernel_timing_read(k) for k in dk.api.KERNELS}
    dk.kernel_timing(False)
    return times, kt


def paged_hbm_point(dk, cfg, w, iters, contiguous_ms):
    """The same tokens in a paged cache of permuted 16-token pages, all in HBM."""
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    from synth import paged_table
    L, hq, hkv, d = cfg["lens"][0], cfg["hq"], cfg["hkv"], cfg["d"]
    pt, nh, nd = paged_table(1, [L], 16, 0.0)
    cache = paged_cache(hkv, d, [L], pt, nh, nd, w["ks"], w["vs"], cfg["theta"])
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    bufs = dk.alloc_decode_buffers(cache, 1, hq, [L], 0.0)
    times, kt = flushed_steps(dk, make_step(dk, cfg, w, cache, 0.0, bufs), iters, flush)
    med = statistics.median(times)
    db = L * hkv * d * 2 * 2
    out = {"page": 16, "pages": "permuted, all in HBM", "ms_median": round(med, 4),
           "eff_gbs": round(db / (med * 1e6), 2),
           "kernel_ms": {k: round(v[1] / max(1, v[0]), 5) for k, v in kt.items()},
           "vs_contiguous": round(contiguous_ms / med, 3) if contiguous_ms else None}
    log(f"[bench] paged HBM: {med:.3f} ms ({out['vs_contiguous']} of the contiguous speed)")
    del flush
    cache.free()
    return out


def ratio_sweep(dk, cfg, w, ratios, iters, bw_h, bw_d):
    """Per-ratio latency from full host and device copies of the same cache."""
    import torch
    from decode_attention_host_amd.cache_build import SplitView, contiguous_cache
    assert cfg["batch"] == 1
    L = cfg["lens"][0]
    hq, hkv, d = cfg["hq"], cfg["hkv"], cfg["d"]
    host_full = w["cache"] if w["cache"].host_rows == L else contiguous_cache(
        hkv, d, [L], 1.0, w["ks"], w["vs"], cfg["theta"])
    dev_full = contiguous_cache(hkv, d, [L], 0.0, w["ks"], w["vs"], cfg["theta"])
    # read-only cache flush between steps (a write flush would leave dirty
    # lines to write back during the timed step)
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    row = hkv * d * 2 * 2
    out = []
    for r in ratios:
        view = SplitView(host_full, dev_full, L, r)
        nh = view.n_host
        bufs = dk.alloc_decode_buffers(view, 1, hq, [L], r)
        step = make_step(dk, cfg, w, view, r, bufs)
        times, kt = flushed_steps(dk, step, iters, flush)
        med = statistics.median(times)
        hb, db = nh * row, (L - nh) * row
        t_star = max(hb / (bw_h * 1e6), db / (bw_d * 1e6))
        t_nom = max(hb / (PCIE_PEAK_GBS * 1e6), db / (HBM_PEAK_GBS * 1e6))
        out.append({"ratio": round(r, 5), "n_host": nh, "host_bytes": hb, "hbm_bytes": db,
                    "ms_median": round(med, 4), "ms_p10": round(sorted(times)[len(times) // 10], 4),
                    "ms_p90": round(sorted(times)[(9 * len(times)) // 10], 4),
                    "eff_gbs": round((hb + db) / (med * 1e6), 2),
                    "roofline_ms_measured": round(t_star, 4), "frac_measured": round(t_star / med, 3),
                    "roofline_ms_nominal": round(t_nom, 4), "frac_nominal": round(t_nom / med, 3),
                    "hbm_bytes_saved": hb,
                    "kernel_ms": {k: round(v[1] / max(1, v[0]), 5) for k, v in kt.items()},
                    "plan": {k: bufs.info[k] for k in ("host_wgs", "dev_wgs", "host_chunk", "dev_chunk")}})
        log(f"[bench] sweep r={r:.4f}: {med:.3f} ms, {out[-1]['eff_gbs']} GB/s, "
            f"frac(measured) {out[-1]['frac_measured']}")
    del flush
    if host_full is not w["cache"]:
        host_full.free()
    dev_full.free()
    return out


def best_split(sweep, bw_h, bw_d):
    """Fastest measured ratio vs the combined roofline total / (BW_h + BW_d)."""
    best = min(sweep, key=lambda e: e["ms_median"])
    total = best["host_bytes"] + best["hbm_bytes"]
    t_comb = total / ((bw_h + bw_d) * 1e6)
    t_comb_nom = total / ((PCIE_PEAK_GBS + HBM_PEAK_GBS) * 1e6)
    return {"ratio": best["ratio"], "ms_median": best["ms_median"],
            "combined_roofline_ms_measured": round(t_comb, 4),
            "frac_combined_measured": round(t_comb / best["ms_median"], 3),
            "combined_roofline_ms_nominal": round(t_comb_nom, 4),
            "frac_combined_nominal": round(t_comb_nom / best["ms_median"], 3),
            "attn_ms": best["kernel_ms"]["attn"],
            "frac_combined_measured_attn": round(t_comb / best["kernel_ms"]["attn"], 3)}


def cpu_baseline(cfg, w, budget_s):
    """The fp64 oracle as it stands, on the host: numpy with BLAS on every core
    of this process's affinity set (numpy's elementwise steps use one core)."""
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    limiter, blas_threads = None, None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        blas_threads = max((p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"),
                           default=None)
    except Exception:  # pragma: no cover
        pass
    B, d, lens = cfg["batch"], cfg["d"], cfg["lens"]
    scale = 1.0 / math.sqrt(d)
    t0 = time.perf_counter()
    done_bytes = 0
    seqs = 0
    while True:
        b = seqs % B
        O.decode_sequence(w["qb"][b], w["ks"][b], w["vs"][b], lens[b] - 1, cfg["theta"], scale)
        done_bytes += lens[b] * cfg["hkv"] * d * 4
        seqs += 1
        if time.perf_counter() - t0 >= budget_s:  # whole calls until the budget is spent
            break
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    used = blas_threads or cores
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"{seqs} full decode_sequence call(s) of the workload ({done_bytes} KV bytes incl. "
                      f"key rotation) in {dt:.1f}s, numpy float64, BLAS on {used} thread(s) of {cores} "
                      f"cores in the affinity set (elementwise steps single-threaded)",
            "ms_per_step": round(dt / seqs * B * 1e3, 1)}


def measure_contiguous(dk, cfg, seed, flags, steps, warmup):
    """One contiguous-split workload: timed steps, attention kernel time, roofline."""
    w = build_workload(cfg, seed, flags)
    B, hq, d, lens, ratio = cfg["batch"], cfg["hq"], cfg["d"], cfg["lens"], cfg["ratio"]
    bufs = dk.alloc_decode_buffers(w["cache"], B, hq, lens, ratio)
    step = make_step(dk, cfg, w, w["cache"], ratio, bufs)
    gpu_warm(step)
    dk.kernel_timing(True)
    for k in dk.api.KERNELS:
        dk.kernel_timing_read(k)
    ms, _ = timed_loop(step, steps, warmup)
    kt = {k: dk.kernel_timing_read(k) for k in dk.api.KERNELS}
    dk.kernel_timing(False)
    info = bufs.info
    res = summarize(cfg, info, ms, kt)
    gms = graph_timing(dk, step, steps)
    res["graph_ms_per_step"] = round(gms, 4)
    res["graph_eff_kv_gbs"] = round((info["host_bytes"] + info["dev_bytes"]) / (gms * 1e6), 2)
    return res, w


def summarize(cfg, info, ms, kt, extra_bytes=0):
    attn_ms = kt["attn"][1] / max(1, kt["attn"][0])
    kv = info["host_bytes"] + info["dev_bytes"]
    t_star = max(info["host_bytes"] / (PCIE_PEAK_GBS * 1e6), info["dev_bytes"] / (HBM_PEAK_GBS * 1e6))
    return {"workload": cfg["name"], "batch": cfg["batch"], "ms_per_step": round(ms, 4),
            "latency_ms_per_token": round(ms / cfg["batch"], 5),
            "kv_bytes_per_step": kv, "host_bytes": info["host_bytes"], "hbm_bytes": info["dev_bytes"],
            "eff_kv_gbs": round(kv / (ms * 1e6), 2), "attn_kernel_ms": round(attn_ms, 4),
            "attn_kv_gbs": round(kv / (attn_ms * 1e6), 2),
            "host_gbs_in_attn": round(info["host_bytes"] / (attn_ms * 1e6), 2),
            "roofline_ms_nominal": round(t_star, 4), "frac_nominal_step": round(t_star / ms, 4),
            "frac_nominal_attn": round(t_star / attn_ms, 4),
            "kernel_ms": {k: round(v[1] / max(1, v[0]), 5) for k, v in kt.items()},
            "plan": {k: info[k] for k in ("num_splits", "host_wgs", "dev_wgs", "host_chunk", "dev_chunk")},
            "extra_bytes": extra_bytes}


def measure_fused_paged(dk, cfg, seed, flags, steps, warmup):
    """Ragged batch over a paged cache: projected new token appended at L_b
    (fused projection + RoPE + append), then attention over L_b + 1 tokens."""
    import numpy as np
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    from synth import TensorId, kv_raw, normal_bf16, paged_table, query

    B, hq, hkv, d, lens = cfg["batch"], cfg["hq"], cfg["hkv"], cfg["d"], cfg["lens"]
    ntok = [L + 1 for L in lens]
    t0 = time.time()
    ks, vs = kv_raw(seed, lens, hkv, d)
    pt, nh, nd = paged_table(seed, ntok, cfg["page"], cfg["ratio"])
    cache = paged_cache(hkv, d, ntok, pt, nh, nd, ks, vs, cfg["theta"], page=cfg["page"],
                        host_flags=flags, upto=lens)
    log(f"[bench] {cfg['name']}: {sum(ntok)} tokens, {nh} host / {nd} HBM pages, built in "
        f"{time.time() - t0:.1f}s")
    del ks, vs
    hid = cfg["hidden"]
    x = torch.from_numpy(normal_bf16(seed, TensorId.X, (B, hid)).view(np.int16)).cuda()
    wk = torch.from_numpy(normal_bf16(seed, TensorId.WK, (hid, hkv * d), std=cfg["w_std"]).view(np.int16)).cuda()
    wv = torch.from_numpy(normal_bf16(seed, TensorId.WV, (hid, hkv * d), std=cfg["w_std"]).view(np.int16)).cuda()
    q = torch.from_numpy(query(seed, B, hq, d).view(np.int16)).cuda()
    pos = torch.tensor(lens, dtype=torch.int32, device="cuda")   # new token at position L_b
    sidx = torch.arange(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(dk.append_workspace_bytes(B, hid, hkv * d), dtype=torch.uint8, device="cuda")
    bufs = dk.alloc_decode_buffers(cache, B, hq, ntok, 0.0)
    ntok_dev = torch.tensor(ntok, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)

    def step():
        dk.project_rope_append(cache, B, None, 0.0, sidx, pos, x=x, wk=wk, wv=wv,
                               rope_theta=cfg["theta"], workspace=ws)
        dk.decode_attn_split(cache, q, pos, ntok_dev, 0.0, scale, cfg["theta"], bufs=bufs)
        dk.merge_lse(bufs.part_o, bufs.part_lse, bufs.split_offsets, B, hq, d, out_o=bufs.out_o,
                     out_lse=bufs.out_lse)

    gpu_warm(step)
    dk.kernel_timing(True)
    for k in dk.api.KERNELS:
        dk.kernel_timing_read(k)
    ms, _ = timed_loop(step, steps, warmup)
    kt = {k: dk.kernel_timing_read(k) for k in dk.api.KERNELS}
    dk.kernel_timing(False)
    res = summarize(cfg, bufs.info, ms, kt, extra_bytes=2 * hid * hkv * d * 2)
    res["lens"] = {"min": min(lens), "max": max(lens), "sum": sum(lens)}
    gms = graph_timing(dk, step, steps)
    res["graph_ms_per_step"] = round(gms, 4)
    cache.free()
    return res


def measure_long_sweep(dk, cfg, seed, flags, iters, bw_h, bw_d):
    import numpy as np
    from decode_attention_host_amd.cache_build import contiguous_cache
    from synth import kv_raw, query
    import torch
    L = cfg["lens"][0]
    hkv, d = cfg["hkv"], cfg["d"]
    t0 = time.time()
    ks, vs = kv_raw(seed, [L], hkv, d)
    host_full = contiguous_cache(hkv, d, [L], 1.0, ks, vs, cfg["theta"], host_flags=flags)
    log(f"[bench] {cfg['name']}: host copy built in {time.time() - t0:.1f}s")
    qb = query(seed, 1, cfg["hq"], d)
    w = dict(ks=ks, vs=vs, qb=qb, cache=host_full,
             q=torch.from_numpy(qb.view(np.int16)).cuda(),
             qpos=torch.tensor([L - 1], dtype=torch.int32, device="cuda"),
             k_new=torch.from_numpy(ks[0][-1:].copy().view(np.int16)).cuda(),
             v_new=torch.from_numpy(vs[0][-1:].copy().view(np.int16)).cuda(),
             seq_lens_dev=torch.tensor([L], dtype=torch.int32, device="cuda"),
             sidx=torch.zeros(1, dtype=torch.int32, device="cuda"))
    r_star = bw_h / (bw_h + bw_d)
    ratios = [0.0, r_star, 0.25, 0.5, 0.75, 0.9, 1.0]
    out = ratio_sweep(dk, cfg, w, ratios, iters, bw_h, bw_d)
    paged = paged_hbm_point(dk, cfg, w, iters, next((x["ms_median"] for x in out if x["ratio"] == 0.0), None))
    host_full.free()
    return {"sweep": out, "best_split": best_split(out, bw_h, bw_d), "paged_hbm": paged}


def measure_prefill(dk, cfg, seed, flags, steps, warmup):
    """Causal prefill of new tokens, per offload ratio in cfg["ratios"]:
    the fused step (append of the new rows into their tier plus an HBM copy,
    prefill attention, merge: one library call) and the two-call path
    (append; prefill attention over the cache; merge)."""
    import numpy as np
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    from synth import kv_raw, normal_bf16

    hq, hkv, d, lens, news = cfg["hq"], cfg["hkv"], cfg["d"], cfg["lens"], cfg["new"]
    B = cfg["batch"]
    th = cfg["theta"]
    ks, vs = kv_raw(seed, lens, hkv, d)
    q = torch.from_numpy(np.concatenate([normal_bf16(seed + b, 1, (n, hq, d)) for b, n in enumerate(news)])
                         .view(np.int16)).cuda()
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q_pos0 = [L - n for L, n in zip(lens, news)]
    T = int(q_start[-1])
    k_new = torch.from_numpy(np.concatenate([k[L - n:] for k, L, n in zip(ks, lens, news)]).view(np.int16)).cuda()
    v_new = torch.from_numpy(np.concatenate([v[L - n:] for v, L, n in zip(vs, lens, news)]).view(np.int16)).cuda()
    sidx = torch.from_numpy(np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(news)])).cuda()
    pos = torch.from_numpy(np.concatenate([np.arange(L - n, L, dtype=np.int32) for L, n in zip(lens, news)])).cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    flops = 0
    for L, n, p0 in zip(lens, news, q_pos0):
        flops += 4 * hq * d * sum(p0 + j + 1 for j in range(n))

    def timed(step):
        # median of five timed loops: a step of ~0.1 ms leaves the GPU idle
        # through any host-side stall of a few ms inside a single loop
        gpu_warm(step)
        dk.kernel_timing(True)
        for k in dk.api.KERNELS:
            dk.kernel_timing_read(k)
        ms = statistics.median(timed_loop(step, steps, warmup)[0] for _ in range(5))
        kt = {k: dk.kernel_timing_read(k) for k in dk.api.KERNELS}
        dk.kernel_timing(False)
        return ms, {k: v[1] / max(1, v[0]) for k, v in kt.items() if v[0]}

    out = []
    for r in cfg.get("ratios", [cfg["ratio"]]):
        # fused step over a cache holding only the prefix
        cache = contiguous_cache(hkv, d, lens, r, ks, vs, th, host_flags=flags, upto=q_pos0)
        info = dk.prefill_fused_plan(cache, B, hq, q_start, q_pos0, lens, r)
        ws = torch.empty(max(256, info["workspace_bytes"]), dtype=torch.uint8, device="cuda")
        oo = torch.empty((T, hq, d), dtype=torch.float32, device="cuda")
        ol = torch.empty((T, hq), dtype=torch.float32, device="cuda")
        f_ms, f_kt = timed(lambda: dk.prefill_fused(cache, q, q_start, q_pos0, lens, r, scale, th, k_new=k_new,
                                                    v_new=v_new, workspace=ws, out_o=oo, out_lse=ol))
        cache.free()
        # two-call path over the full cache
        cache = contiguous_cache(hkv, d, lens, r, ks, vs, th, host_flags=flags)
        bufs = dk.alloc_prefill_buffers(cache, B, hq, q_start, q_pos0, lens, r)

        def step():
            dk.project_rope_append(cache, B, sl, r, sidx, pos, k_new=k_new, v_new=v_new, rope_theta=th)
            dk.prefill_attn_split(cache, q, q_start, q_pos0, lens, r, scale, th, bufs=bufs)
            dk.merge_lse(bufs.part_o, bufs.part_lse, bufs.split_offsets, T, hq, d, out_o=bufs.out_o,
                         out_lse=bufs.out_lse)

        s_ms, s_kt = timed(step)
        # attention-only launch time: the two-call path's prefill kernel (the
        # fused launch also carries the writer workgroups' host-slot writes)
        pf_ms = s_kt["prefill"]
        # MFMA work executed: Q.K and P.V each run twice (high and low bf16
        # parts of the fp32 operand), so the executed rate is 2x the useful one
        two = bufs.info
        out.append({"ratio": r, "new_tokens": T,
                    "fused_ms_per_step": round(f_ms, 4),
                    "fused_kernel_ms": {k: round(v, 5) for k, v in f_kt.items()},
                    "fused_kv_reads": {"host_bytes": info["host_bytes"], "hbm_bytes": info["dev_bytes"],
                                       "staged_bytes": info["staged_bytes"]},
                    "two_call_ms_per_step": round(s_ms, 4),
                    "two_call_kernel_ms": {k: round(v, 5) for k, v in s_kt.items()},
                    "two_call_kv_reads": {"host_bytes": two["host_bytes"], "hbm_bytes": two["dev_bytes"],
                                          "staged_bytes": two["staged_bytes"]},
                    "prefill_kernel_ms": round(pf_ms, 4),
                    "fused_prefill_launch_ms": round(f_kt["prefill"], 4),
                    "useful_tflops": round(flops / (pf_ms * 1e9), 2),
                    "frac_bf16_mfma_peak_useful": round(flops / (pf_ms * 1e9) / 2500.0, 4),
                    "frac_bf16_mfma_peak_executed": round(2 * flops / (pf_ms * 1e9) / 2500.0, 4),
                    "plan": {k: info[k] for k in ("num_splits", "host_wgs", "dev_wgs", "host_chunk", "dev_chunk")}})
        log(f"[bench] prefill r={r}: fused {f_ms:.4f} ms, two-call {s_ms:.4f} ms, prefill kernel {pf_ms:.4f} ms")
        cache.free()
    return {"flops_per_step": flops, "per_ratio": out}


def measure_linear(dk, cfg, seed, iters, bw_h, bw_d):
    """Offloaded linear y = x W^T, W split by output rows; per (ratio, tokens):
    median call time with a read-only cache flush between calls, effective
    weight GB/s and the split roofline max(host_bytes/BW_h, hbm_bytes/BW_d)."""
    import numpy as np
    import torch
    from synth import normal_bf16
    N, K = cfg["out_features"], cfg["in_features"]
    w = normal_bf16(seed, 5, (N, K), std=cfg["w_std"])
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    r_star = bw_h / (bw_h + bw_d)
    out = []
    for r in [0.0, r_star, 0.25, 0.5, 1.0]:
        lin = dk.OffloadedLinear(w, r)
        hb, db = lin.n_host * K * 2, (N - lin.n_host) * K * 2
        for m in cfg["tokens"]:
            x = torch.from_numpy(normal_bf16(seed, 4, (m, K)).view(np.int16)).cuda()
            y = torch.empty((m, N), dtype=torch.float32, device="cuda")
            ws = torch.empty(max(256, lin.plan(m)["workspace_bytes"]), dtype=torch.uint8, device="cuda")
            gpu_warm(lambda: lin(x, y, ws), 0.2)
            dk.kernel_timing(True)
            dk.kernel_timing_read("linear")
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
            sink = torch.empty(iters, dtype=torch.float32, device="cuda")
            for i in range(iters):
                torch.sum(flush, dim=0, out=sink[i])
                ev[i][0].record()
                lin(x, y, ws)
                ev[i][1].record()
            torch.cuda.synchronize()
            n_k, k_ms = dk.kernel_timing_read("linear")
            dk.kernel_timing(False)
            times = sorted(a.elapsed_time(b) for a, b in ev)
            med = statistics.median(times)
            t_star = max(hb / (bw_h * 1e6), db / (bw_d * 1e6))
            t_nom = max(hb / (PCIE_PEAK_GBS * 1e6), db / (HBM_PEAK_GBS * 1e6))
            out.append({"ratio": round(r, 5), "tokens": m, "host_bytes": hb, "hbm_bytes": db,
                        "ms_median": round(med, 4), "kernel_ms": round(k_ms / max(1, n_k), 4),
                        "eff_weight_gbs": round((hb + db) / (med * 1e6), 1),
                        "roofline_ms_measured": round(t_star, 4), "frac_measured": round(t_star / med, 3),
                        "roofline_ms_nominal": round(t_nom, 4), "frac_nominal": round(t_nom / med, 3)})
            log(f"[bench] linear r={r:.4f} m={m}: {med:.4f} ms, {out[-1]['eff_weight_gbs']} GB/s, "
                f"frac(measured) {out[-1]['frac_measured']}")
        lin.free()
    del flush
    return {"sweep": out}


def load_traffic(workload_name):
    p = os.path.join(ROOT, "profiles", f"attn_{workload_name}_traffic.json")
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("kernel_src_sha") != kernel_src_sha():
        return None
    return t.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b_32k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--ratio", type=float, default=None,
                    help="offload ratio for the main workload instead of its own (profiling runs)")
    ap.add_argument("--host-flags", choices=["coherent", "noncoherent"], default="coherent")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep-iters", type=int, default=20)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--tune", default="", help="comma list of dkv_tuning fields, e.g. host_wgs=256")
    ap.add_argument("--extra", default="tiny,opt_6_7b_b8,fused_ragged,llama3_8b_1m,llama3_8b_prefill_2k,"
                                       "llama3_8b_mlp_up_linear",
                    help="other workloads measured after the headline ('' for none)")
    ap.add_argument("--profile-run", action="store_true",
                    help="short run for rocprofv3: headline steps plus two calibration reads of known "
                         "size (a 256 MiB HBM copy and a 64 MiB zero-copy read of the host pool)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this path runs on one GPU: bench.py measures N=1 only; "
                          "sharding over several GPUs is a design note, not built"}), flush=True)
        sys.exit(2)

    import torch
    import decode_attention_host_amd as dk
    from synth import workload

    torch.cuda.set_device(0)
    cfg = workload(args.workload, seed=args.seed)
    if args.ratio is not None:
        cfg["ratio"] = float(args.ratio)
    if args.tune:
        kw = {}
        for item in args.tune.split(","):
            k, v = item.split("=")
            kw[k.strip()] = float(v) if "bw" in k else int(v)
        dk.set_tuning(**kw)
    flags = dk.DKV_HOST_NONCOHERENT if args.host_flags == "noncoherent" else dk.DKV_HOST_COHERENT
    log(f"[bench] workload {cfg['name']}: B={cfg['batch']} Hq={cfg['hq']} Hkv={cfg['hkv']} D={cfg['d']} "
        f"L={cfg['lens'] if len(cfg['lens']) <= 4 else str(len(cfg['lens'])) + ' seqs'} r={cfg['ratio']}")
    w = build_workload(cfg, args.seed, flags)
    cache = w["cache"]
    B, hq, d, lens, ratio = cfg["batch"], cfg["hq"], cfg["d"], cfg["lens"], cfg["ratio"]
    bufs = dk.alloc_decode_buffers(cache, B, hq, lens, ratio)
    info = bufs.info
    kv_bytes = info["host_bytes"] + info["dev_bytes"]
    step = make_step(dk, cfg, w, cache, ratio, bufs)

    if args.profile_run:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(3)
        dst.copy_(src)
        if cache.host_k is not None and cache.host_rows * cfg["hkv"] * cfg["d"] * 2 >= (64 << 20):
            dk.probe_read(cache.host_k.dev_ptr, 64 << 20, 64, nontemporal=True, iters=1)
        torch.cuda.synchronize()
        gpu_warm(step, 0.5)
        ms, _ = timed_loop(step, args.steps, args.warmup)
        log(f"[bench] profile run: {args.steps} steps, {ms:.4f} ms/step")
        cache.free()
        return
    # bring the GPU to its working clocks before anything is measured
    gpu_warm(step, 0.5)
    dk.kernel_timing(False)
    # headline: W warm-up steps, then exactly K timed steps
    dk.kernel_timing(True)
    for k in dk.api.KERNELS:
        dk.kernel_timing_read(k)  # clear
    ms, wall = timed_loop(step, args.steps, args.warmup)
    kt = {k: dk.kernel_timing_read(k) for k in dk.api.KERNELS}
    dk.kernel_timing(False)
    n_attn, attn_total = kt["attn"]
    attn_ms = attn_total / max(1, n_attn)
    log(f"[bench] step {ms:.4f} ms (wall {wall / args.steps * 1e3:.4f} ms), attention kernel {attn_ms:.4f} ms "
        f"over {n_attn} launches")
    value = kv_bytes / (ms * 1e6)
    graph_ms = graph_timing(dk, step, args.steps)
    log(f"[bench] graph replay of the same step: {graph_ms:.4f} ms")

    probe = {}
    if not args.no_probe:
        probe = run_probe(dk, w, 128 << 20)
        log(f"[bench] probe: {json.dumps({k: v for k, v in probe.items() if 'sweep' not in k})}")
    nominal, link = pcie_nominal_gbs(getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None))
    probe["host_link_nominal_gbs"] = round(nominal, 2) if nominal else None
    probe["host_link"] = link

    host_dominant = info["host_bytes"] * HBM_PEAK_GBS >= info["dev_bytes"] * PCIE_PEAK_GBS
    if host_dominant:
        achieved = info["host_bytes"] / (attn_ms * 1e6)
        peak = PCIE_PEAK_GBS
        meas = max(probe.get("host_zero_copy_gbs", 0.0), probe.get("host_dma_gbs", 0.0)) or None
    else:
        achieved = info["dev_bytes"] / (attn_ms * 1e6)
        peak = HBM_PEAK_GBS
        meas = probe.get("hbm_read_gbs")
    roofline = {"bound": "host_link" if host_dominant else "hbm", "achieved": round(achieved, 3),
                "peak": peak, "unit": "GB/s", "frac": round(achieved / peak, 4),
                "traffic": load_traffic(cfg["name"]),
                "kernel": "attn_split_kernel", "kernel_ms": round(attn_ms, 5),
                "algorithmic_bytes": info["host_bytes"] if host_dominant else info["dev_bytes"],
                "peak_measured": meas,
                "frac_measured": round(achieved / meas, 4) if meas else None}

    sweep = None
    if not args.no_sweep and B == 1:
        bw_h = probe.get("host_zero_copy_gbs") or 50.0
        bw_d = probe.get("hbm_read_gbs") or 5000.0
        r_star = bw_h / (bw_h + bw_d)
        ratios = [0.0, r_star, 0.25, 0.5, 0.75, 0.9, 1.0]
        sweep = ratio_sweep(dk, cfg, w, ratios, args.sweep_iters, bw_h, bw_d)
        sweep = {"sweep": sweep, "best_split": best_split(sweep, bw_h, bw_d)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, w, args.cpu_budget)
        log(f"[bench] cpu baseline: {cpu}")

    workloads = {}
    for name in [x for x in args.extra.split(",") if x]:
        wcfg = workload(name, seed=args.seed)
        t0 = time.time()
        if wcfg.get("layout") == "linear":
            bw_h = probe.get("host_zero_copy_gbs") or 50.0
            bw_d = probe.get("hbm_read_gbs") or 5000.0
            workloads[name] = measure_linear(dk, wcfg, args.seed, 20, bw_h, bw_d)
        elif "new" in wcfg:
            workloads[name] = measure_prefill(dk, wcfg, args.seed, flags, 10, 3)
        elif name == "llama3_8b_1m":
            bw_h = probe.get("host_zero_copy_gbs") or 50.0
            bw_d = probe.get("hbm_read_gbs") or 5000.0
            workloads[name] = measure_long_sweep(dk, wcfg, args.seed, flags, 10, bw_h, bw_d)
        elif wcfg["layout"] == "paged":
            workloads[name] = measure_fused_paged(dk, wcfg, args.seed, flags, 20, 5)
        else:
            res, ww = measure_contiguous(dk, wcfg, args.seed, flags, 20, 5)
            ww["cache"].free()
            workloads[name] = res
        log(f"[bench] {name} measured in {time.time() - t0:.1f}s: "
            f"{json.dumps({k: v for k, v in workloads[name].items() if k in ('ms_per_step', 'graph_ms_per_step', 'eff_kv_gbs', 'attn_kv_gbs', 'frac_nominal_attn', 'best_split', 'per_ratio')})}")

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": B, "q_heads": hq, "kv_heads": cfg["hkv"],
                   "head_dim": d, "context": lens[0] if len(set(lens)) == 1 else lens,
                   "offload_ratio": ratio, "layout": cfg["layout"], "rope_theta": cfg["theta"],
                   "host_memory": args.host_flags, "kv_bytes_per_step": kv_bytes},
        "latency_ms_per_token": round(ms / B, 5),
        "graph": {"ms_per_step": round(graph_ms, 5), "eff_kv_gbs": round(kv_bytes / (graph_ms * 1e6), 3),
                  "note": "the same step captured into one HIP graph and replayed"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "probe": probe,
        "plan": info,
        "kernel_ms": {k: round(v[1] / max(1, v[0]), 5) for k, v in kt.items()},
        "sweep": sweep,
        "workloads": workloads,
    }
    print(json.dumps(out), flush=True)
    cache.free()


if __name__ == "__main__":
    main()
