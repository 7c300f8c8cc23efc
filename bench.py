#!/usr/bin/env python3
"""Decode-attention benchmark: effective KV GB/s and latency per step vs offload ratio.

A step is one pass of the whole path over one batch: each sequence's newest
token is appended (Neox RoPE of its key in fp64, one bf16 rounding, stored in
its tier), the query attends over both tiers, and the partials are merged by
log-sum-exp.  The one-launch form (dkv_decode_step) does all of it in one
kernel; the split form is append, split attention and merge as three calls.
Inputs are seeded synthetic tensors with the layer shapes of the workload (no
weights, no datasets), already resident in HBM / host-pinned memory.

Default workload: LLaMA-3-8B attention layer, batch 1, 32 query / 8 KV heads,
head_dim 128, 1,048,576 cached tokens (4 GiB of K+V), all in host-pinned memory
(offload ratio 1).

Prints ONE JSON line: the headline value, the roofline of the decode kernel
(timed live with HIP events on its stream), the in-run bandwidth probe, the
offload-ratio sweep, the growing decode loop, the other workloads and the fp64
oracle timed on the host cores.
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
PCIE_RAW_GBS = 64.0       # PCIe 5.0 x16 per direction before 128b/130b encoding
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
    """Hash of the decode kernel's own sources (kernel file, work-split header,
    device helpers, argument structure).  A stored traffic figure of that
    kernel stays valid while this hash matches."""
    import re
    csrc = os.path.join(ROOT, "decode_attention_host_amd", "csrc")
    h = hashlib.sha256()
    for f in ("dkv_decode.hip", "dkv_decomp.h", "dkv_device.h"):
        h.update(open(os.path.join(csrc, f)).read().encode())
    h_src = open(os.path.join(csrc, "dkv_internal.h")).read()
    h.update(re.search(r"struct DecodeArgs \{.*?\n\};", h_src, re.S).group(0).encode())
    for x in re.findall(r"constexpr int k(?:Tile|Threads) = \d+;", h_src):
        h.update(x.encode())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------- timing

def gpu_warm(step, seconds=0.3):
    """Run the step until the GPU is back at working clocks (it idles while the
    host builds caches or runs the oracle)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        step()
        torch.cuda.synchronize()


def timed_loop(step, steps, warmup):
    """W untimed steps, then exactly K steps between two events (back to back)."""
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
    return e0.elapsed_time(e1) / steps, time.perf_counter() - t0


def kernel_times(dk, step, iters):
    """The library's per-kernel HIP-event timing over `iters` steps."""
    import torch
    dk.kernel_timing(True)
    for k in dk.api.KERNELS:
        dk.kernel_timing_read(k)
    for _ in range(iters):
        step()
    torch.cuda.synchronize()
    kt = {k: dk.kernel_timing_read(k) for k in dk.api.KERNELS}
    dk.kernel_timing(False)
    return {k: round(v[1] / v[0], 5) for k, v in kt.items() if v[0]}


def flushed_steps(dk, step, iters, flush):
    """Per-step times of `iters` steps with a read-only cache flush between
    them (median, p10, p90), then the per-kernel times over a second pass of
    the same steps (the library's event pair around each launch would
    otherwise add to the step times)."""
    import torch
    gpu_warm(step, 0.2)
    sink = torch.empty(iters, dtype=torch.float32, device="cuda")

    def run(ev):
        for i in range(iters):
            torch.sum(flush, dim=0, out=sink[i])
            if ev:
                ev[i][0].record()
            step()
            if ev:
                ev[i][1].record()
        torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    run(ev)
    t = sorted(a.elapsed_time(b) for a, b in ev)
    dk.kernel_timing(True)
    for k in dk.api.KERNELS:
        dk.kernel_timing_read(k)
    run(None)
    kt = {k: dk.kernel_timing_read(k) for k in dk.api.KERNELS}
    dk.kernel_timing(False)
    return {"ms_median": round(statistics.median(t), 5), "ms_p10": round(t[len(t) // 10], 5),
            "ms_p90": round(t[(9 * len(t)) // 10], 5),
            "kernel_ms": {k: round(v[1] / v[0], 5) for k, v in kt.items() if v[0]}}


def graph_ms(dk, step, steps):
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


# ----------------------------------------------------------------- steps

class DecodeSteps:
    """Both forms of the decode step over one cache.  The cache holds L_b tokens;
    a step re-appends token L_b - 1 (position L_b - 1, same bits: idempotent) and
    attends over all L_b tokens, so every timed step reads the whole cache."""

    def __init__(self, dk, cfg, cache, ratio, q, k_new, v_new, lens, *, x=None, wk=None, wv=None):
        import torch
        B, hq, d = cfg["batch"], cfg["hq"], cfg["d"]
        self.dk, self.cfg, self.cache, self.ratio = dk, cfg, cache, ratio
        self.q, self.k_new, self.v_new, self.x, self.wk, self.wv = q, k_new, v_new, x, wk, wv
        self.B, self.hq, self.d = B, hq, d
        self.scale = 1.0 / math.sqrt(d)
        self.theta = cfg["theta"]
        self.lens = [int(n) for n in lens]
        self.full = torch.tensor(self.lens, dtype=torch.int32, device="cuda")        # tokens after the append
        self.cached = torch.tensor([n - 1 for n in self.lens], dtype=torch.int32, device="cuda")
        self.pos = self.cached.clone()                                               # the appended token
        self.sidx = torch.arange(B, dtype=torch.int32, device="cuda")
        self.bufs = dk.alloc_decode_buffers(cache, B, hq, self.lens, ratio)
        hidden = int(x.shape[1]) if x is not None else 0
        self.ws = dk.decode_step_workspace(cache, B, hq, ratio, hidden)
        self.app_ws = (torch.empty(dk.append_workspace_bytes(B, hidden, cfg["hkv"] * d), dtype=torch.uint8,
                                   device="cuda") if hidden else None)
        self.out_o = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
        self.out_l = torch.empty((B, hq), dtype=torch.float32, device="cuda")

    def info(self):
        return self.bufs.info

    def split(self):
        dk = self.dk
        dk.project_rope_append(self.cache, self.B, self.full, self.ratio, self.sidx, self.pos, k_new=self.k_new,
                               v_new=self.v_new, x=self.x, wk=self.wk, wv=self.wv, rope_theta=self.theta,
                               workspace=self.app_ws)
        dk.decode_attn_split(self.cache, self.q, self.pos, self.full, self.ratio, self.scale, self.theta,
                             bufs=self.bufs)
        dk.merge_lse(self.bufs.part_o, self.bufs.part_lse, self.bufs.split_offsets, self.B, self.hq, self.d,
                     out_o=self.bufs.out_o, out_lse=self.bufs.out_lse)

    def fused(self):
        self.dk.decode_step(self.cache, self.q, self.pos, self.cached, self.ratio, self.scale, self.theta,
                            k_new=self.k_new, v_new=self.v_new, x=self.x, wk=self.wk, wv=self.wv,
                            workspace=self.ws, out_o=self.out_o, out_lse=self.out_l)


def contiguous_steps(dk, cfg, seed, flags, ratio=None, host_full=None, dev_full=None, raw=None):
    """DecodeSteps over a contiguous-split cache (built here, or a SplitView of
    full host and HBM copies)."""
    import numpy as np
    import torch
    from decode_attention_host_amd.cache_build import SplitView, contiguous_cache
    from synth import kv_raw, query
    B, hq, hkv, d, lens = cfg["batch"], cfg["hq"], cfg["hkv"], cfg["d"], cfg["lens"]
    r = cfg["ratio"] if ratio is None else ratio
    ks, vs = raw if raw is not None else kv_raw(seed, lens, hkv, d)
    if host_full is not None:
        cache = SplitView(host_full, dev_full, lens[0], r)
    else:
        cache = contiguous_cache(hkv, d, lens, r, ks, vs, cfg["theta"], host_flags=flags)
    q = torch.from_numpy(query(seed, B, hq, d).view(np.int16)).cuda()
    k_new = torch.from_numpy(np.stack([k[-1] for k in ks]).view(np.int16)).cuda()
    v_new = torch.from_numpy(np.stack([v[-1] for v in vs]).view(np.int16)).cuda()
    return DecodeSteps(dk, cfg, cache, r, q, k_new, v_new, lens), (ks, vs)


def measure_forms(dk, st, steps, warmup, flush=None, iters=10, graph=True):
    """Back-to-back and (optionally) flushed times of both forms, kernel times, graph replay."""
    out = {}
    for form in ("fused", "split"):
        fn = getattr(st, form)
        gpu_warm(fn, 0.2)
        ms, _ = timed_loop(fn, steps, warmup)
        rec = {"ms_per_step": round(ms, 5), "kernel_ms": kernel_times(dk, fn, min(steps, 20))}
        if flush is not None:
            rec["flushed"] = flushed_steps(dk, fn, iters, flush)
        if graph:
            rec["graph_ms_per_step"] = round(graph_ms(dk, fn, steps), 5)
        out[form] = rec
    return out


def kv_bytes(info):
    return info["host_bytes"] + info["dev_bytes"]


# ----------------------------------------------------------------- probe

def run_probe(dk, host_k, host_v, host_bytes, hbm_bytes=4 << 30):
    """In-run ceilings: zero-copy reads of the host pools (best over workgroup
    counts, grid-stride and blocked, normal and non-temporal loads, one pool or
    the K and V pools at once; best of 5 passes each over >= 1 GiB per pool),
    the DMA engine on the same block, and an HBM streaming read."""
    import torch
    res = {}
    if host_k is not None:
        n = min(host_bytes, host_k.nbytes, host_v.nbytes) // 16 * 16
        best, sweep = None, []
        for pair in (False, True):
            for layout in ("grid", "blocked", "segments"):
                for nt in (True, False):
                    for nwg in (32, 48, 64, 96, 128):
                        r = dk.probe_read(host_k.dev_ptr, n, nwg, nontemporal=nt, iters=5,
                                          blocked=layout == "blocked", segments=layout == "segments",
                                          src2_dev_ptr=host_v.dev_ptr if pair else None)
                        sweep.append({"nwg": nwg, "nt": nt, "layout": layout, "k_and_v": pair,
                                      "gbs": round(r["read_gbs"], 2)})
                        if best is None or r["read_gbs"] > best[0]:
                            best = (r["read_gbs"], nwg, nt, layout, pair)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        dma = dk.probe_read(host_k.dev_ptr, n, 64, iters=5, dma_dst=dst, dma_src_host=host_k.host_ptr)
        del dst
        res.update(host_bytes_read=n, host_zero_copy_gbs=round(best[0], 2), host_zero_copy_wgs=best[1],
                   host_zero_copy_nt=best[2], host_zero_copy_layout=best[3], host_zero_copy_k_and_v=best[4],
                   host_dma_gbs=round(dma["dma_gbs"], 2), host_sweep=sweep)
    big = torch.empty(hbm_bytes, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    best, hs = (0.0, 0, False, False), []
    for blocked in (False, True):
        for nt in (True, False):
            for nwg in (256, 512, 1024, 2048, 4096):
                r = dk.probe_read(big.data_ptr(), big.numel(), nwg, nontemporal=nt, iters=5, blocked=blocked)
                hs.append({"nwg": nwg, "nt": nt, "blocked": blocked, "gbs": round(r["read_gbs"], 1)})
                if r["read_gbs"] > best[0]:
                    best = (r["read_gbs"], nwg, nt, blocked)
    res.update(hbm_read_gbs=round(best[0], 1), hbm_read_wgs=best[1], hbm_read_nt=best[2],
               hbm_read_blocked=best[3], hbm_sweep=hs)
    del big
    return res


# ----------------------------------------------------------------- workloads

def ratio_sweep(dk, cfg, seed, flags, ratios, iters, bw_h, bw_d, raw=None):
    """Both forms at each offload ratio, from full host and HBM copies of the same cache."""
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache
    from synth import kv_raw
    assert cfg["batch"] == 1
    L = cfg["lens"][0]
    hkv, d = cfg["hkv"], cfg["d"]
    ks, vs = raw if raw is not None else kv_raw(seed, [L], hkv, d)
    host_full = contiguous_cache(hkv, d, [L], 1.0, ks, vs, cfg["theta"], host_flags=flags)
    dev_full = contiguous_cache(hkv, d, [L], 0.0, ks, vs, cfg["theta"])
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")  # read-only flush of L2 and MALL
    out = []
    for r in ratios:
        st, _ = contiguous_steps(dk, cfg, seed, flags, ratio=r, host_full=host_full, dev_full=dev_full,
                                 raw=(ks, vs))
        info = st.info()
        hb, db = info["host_bytes"], info["dev_bytes"]
        t_star = max(hb / (bw_h * 1e6), db / (bw_d * 1e6))
        t_nom = max(hb / (PCIE_RAW_GBS * 1e6), db / (HBM_PEAK_GBS * 1e6))
        rec = {"ratio": round(r, 5), "host_bytes": hb, "hbm_bytes": db, "hbm_bytes_saved": hb,
               "roofline_ms_measured": round(t_star, 5), "roofline_ms_nominal": round(t_nom, 5),
               "plan": {k: info[k] for k in ("host_wgs", "dev_wgs", "host_chunk", "dev_chunk",
                                             "host_items", "dev_items")}}
        # cold (cache flushed before each step): 50 steps where a step is
        # short, `iters` otherwise; warm: the same count back to back
        n_it = max(iters, 50) if r < 0.5 else iters
        for form in ("fused", "split"):
            f = flushed_steps(dk, getattr(st, form), n_it, flush)
            f["steps"] = n_it
            f["warm_ms"] = round(timed_loop(getattr(st, form), n_it, 3)[0], 5)
            f["eff_gbs"] = round((hb + db) / (f["ms_median"] * 1e6), 2)
            f["frac_measured"] = round(t_star / f["ms_median"], 3)
            f["frac_nominal"] = round(t_nom / f["ms_median"], 3)
            rec[form] = f
        best = min(("fused", "split"), key=lambda k: rec[k]["ms_median"])
        rec["best_form"] = best
        rec["ms_median"] = rec[best]["ms_median"]
        out.append(rec)
        log(f"[bench] {cfg['name']} r={r:.4f}: fused {rec['fused']['ms_median']:.4f} ms, "
            f"split {rec['split']['ms_median']:.4f} ms, frac(measured) {rec[best]['frac_measured']}")
    del flush
    host_full.free()
    dev_full.free()
    return out


def paged_hbm_point(dk, cfg, seed, ks, vs, iters, flush, bw_d, sweep):
    """The same tokens in a paged cache of 16-token pages, all in HBM, at
    seeded permuted physical pages: both forms timed like the sweep, against
    the contiguous r = 0 point."""
    import numpy as np
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    from synth import paged_table, query
    L, hq, hkv, d = cfg["lens"][0], cfg["hq"], cfg["hkv"], cfg["d"]
    pt, nh, nd = paged_table(seed + 1, [L], 16, 0.0)
    cache = paged_cache(hkv, d, [L], pt, nh, nd, ks, vs, cfg["theta"])
    q = torch.from_numpy(query(seed, 1, hq, d).view(np.int16)).cuda()
    k_new = torch.from_numpy(np.ascontiguousarray(ks[0][-1:]).view(np.int16)).cuda()
    v_new = torch.from_numpy(np.ascontiguousarray(vs[0][-1:]).view(np.int16)).cuda()
    st = DecodeSteps(dk, cfg, cache, 0.0, q, k_new, v_new, [L])
    db = st.info()["dev_bytes"]
    rec = {"layout": "paged, 16-token pages permuted in HBM", "hbm_bytes": db,
           "roofline_ms_measured": round(db / (bw_d * 1e6), 5)}
    for form in ("fused", "split"):
        rec[form] = flushed_steps(dk, getattr(st, form), iters, flush)
    rec["best_form"] = min(("fused", "split"), key=lambda k: rec[k]["ms_median"])
    rec["ms_median"] = rec[rec["best_form"]]["ms_median"]
    r0 = next((e for e in sweep if e["ratio"] == 0.0), None)
    if r0:
        rec["vs_contiguous_r0"] = round(r0["ms_median"] / rec["ms_median"], 3)
    log(f"[bench] {cfg['name']} paged in HBM: fused {rec['fused']['ms_median']:.4f} ms, "
        f"split {rec['split']['ms_median']:.4f} ms, vs contiguous r=0 {rec.get('vs_contiguous_r0')}")
    cache.free()
    return rec


def best_split(sweep, bw_h, bw_d):
    """Fastest measured point vs the combined roofline total / (BW_h + BW_d)."""
    best = min(sweep, key=lambda e: e["ms_median"])
    total = best["host_bytes"] + best["hbm_bytes"]
    t_comb = total / ((bw_h + bw_d) * 1e6)
    t_comb_nom = total / ((PCIE_RAW_GBS + HBM_PEAK_GBS) * 1e6)
    k = best[best["best_form"]]["kernel_ms"]["attn"]
    r0 = next((e for e in sweep if e["ratio"] == 0.0), None)
    return {"ratio": best["ratio"], "form": best["best_form"], "ms_median": best["ms_median"],
            "combined_roofline_ms_measured": round(t_comb, 5),
            "frac_combined_measured": round(t_comb / best["ms_median"], 3),
            "combined_roofline_ms_nominal": round(t_comb_nom, 5),
            "frac_combined_nominal": round(t_comb_nom / best["ms_median"], 3),
            "attn_ms": k, "frac_combined_measured_attn": round(t_comb / k, 3),
            "r0_ms_median": r0["ms_median"] if r0 else None}


def measure_staged(dk, cfg, seed, flags, ratios, chunks, iters, bw_h, bw_d):
    """The staged-prefetch comparator against the zero-copy path on the same
    cache (SplitKernel README, Overview: the conventional design copies the
    offloaded data into GPU memory before computing): attention only (no
    append), flushed steps.  Staging writes the host-tier bytes into HBM and
    reads them back, so it adds 2x those bytes of HBM traffic and holds a ring
    of 2 x chunk rows of K and V."""
    import numpy as np
    import torch
    from decode_attention_host_amd.cache_build import SplitView, contiguous_cache
    from synth import kv_raw, query
    L, hq, hkv, d, th = cfg["lens"][0], cfg["hq"], cfg["hkv"], cfg["d"], cfg["theta"]
    ks, vs = kv_raw(seed, [L], hkv, d)
    host_full = contiguous_cache(hkv, d, [L], 1.0, ks, vs, th, host_flags=flags)
    dev_full = contiguous_cache(hkv, d, [L], 0.0, ks, vs, th)
    del ks, vs
    q = torch.from_numpy(query(seed, 1, hq, d).view(np.int16)).cuda()
    qpos = torch.tensor([L - 1], dtype=torch.int32, device="cuda")
    sl = torch.tensor([L], dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    row = hkv * d * 2 * 2
    out = []
    for r in ratios:
        view = SplitView(host_full, dev_full, L, r)
        bufs = dk.alloc_decode_buffers(view, 1, hq, [L], r)
        zc = flushed_steps(dk, lambda: dk.decode(view, q, qpos, sl, r, scale, th, bufs=bufs), iters, flush)
        nh = view.n_host
        hb, db = nh * row, (L - nh) * row
        t_star = max(hb / (bw_h * 1e6), db / (bw_d * 1e6))
        rec = {"ratio": round(r, 5), "host_bytes": hb, "hbm_bytes": db, "roofline_ms_measured": round(t_star, 5),
               "zero_copy_ms": zc["ms_median"], "zero_copy_kernel_ms": zc["kernel_ms"], "staged": []}
        for chunk in chunks:
            info = dk.decode_staged_plan(view, hq, L, r, chunk)
            ws = torch.zeros(max(256, info["workspace_bytes"]), dtype=torch.uint8, device="cuda")
            oo = torch.empty((hq, d), dtype=torch.float32, device="cuda")
            ol = torch.empty((hq,), dtype=torch.float32, device="cuda")
            f = flushed_steps(dk, lambda: dk.decode_staged(view, q, qpos, L, r, scale, th, chunk, workspace=ws,
                                                             out_o=oo, out_lse=ol), iters, flush)
            diff = float((oo - bufs.out_o[0]).abs().max())
            rec["staged"].append({"chunk_tokens": chunk, "chunks": info["host_items"], "ms_median": f["ms_median"],
                                  "ms_p90": f["ms_p90"], "vs_zero_copy": round(f["ms_median"] / zc["ms_median"], 4),
                                  "ring_bytes": 2 * chunk * row, "staging_hbm_bytes": 2 * info["staged_bytes"],
                                  "hbm_traffic_factor": round((db + 2 * info["staged_bytes"]) / max(1, db), 3)
                                  if db else None,
                                  "max_abs_diff_vs_zero_copy": diff})
            del ws
            log(f"[bench] staged {cfg['name']} r={r:.4f} chunk={chunk}: {f['ms_median']:.4f} ms vs zero-copy "
                f"{zc['ms_median']:.4f} ms")
        out.append(rec)
    del flush
    host_full.free()
    dev_full.free()
    return out


def measure_fused_paged(dk, cfg, seed, flags, steps, warmup):
    """Ragged batch over a paged cache: the new token projected from its hidden
    state (x Wk, x Wv), rotated and appended at L_b, then attention over L_b + 1."""
    import numpy as np
    import torch
    from decode_attention_host_amd.cache_build import paged_cache
    from synth import TensorId, kv_raw, normal_bf16, paged_table, query
    B, hq, hkv, d, lens = cfg["batch"], cfg["hq"], cfg["hkv"], cfg["d"], cfg["lens"]
    ntok = [L + 1 for L in lens]
    t0 = time.time()
    ks, vs = kv_raw(seed, lens, hkv, d)
    pt, nh, nd = paged_table(seed, ntok, cfg["page"], cfg["ratio"])
    cache = paged_cache(hkv, d, ntok, pt, nh, nd, ks, vs, cfg["theta"], page=cfg["page"], host_flags=flags,
                        upto=lens)
    log(f"[bench] {cfg['name']}: {sum(ntok)} tokens, {nh} host / {nd} HBM pages, built in {time.time() - t0:.1f}s")
    del ks, vs
    hid = cfg["hidden"]
    x = torch.from_numpy(normal_bf16(seed, TensorId.X, (B, hid)).view(np.int16)).cuda()
    wk = torch.from_numpy(normal_bf16(seed, TensorId.WK, (hid, hkv * d), std=cfg["w_std"]).view(np.int16)).cuda()
    wv = torch.from_numpy(normal_bf16(seed, TensorId.WV, (hid, hkv * d), std=cfg["w_std"]).view(np.int16)).cuda()
    q = torch.from_numpy(query(seed, B, hq, d).view(np.int16)).cuda()
    st = DecodeSteps(dk, cfg, cache, 0.0, q, None, None, ntok, x=x, wk=wk, wv=wv)
    res = {"workload": cfg["name"], "batch": B, "lens": {"min": min(lens), "max": max(lens), "sum": sum(lens)},
           "kv_bytes_per_step": kv_bytes(st.info()), "host_bytes": st.info()["host_bytes"],
           "hbm_bytes": st.info()["dev_bytes"], "weight_bytes": 2 * hid * hkv * d * 2}
    res.update(measure_forms(dk, st, steps, warmup))
    t_nom = max(res["host_bytes"] / (PCIE_RAW_GBS * 1e6), res["hbm_bytes"] / (HBM_PEAK_GBS * 1e6))
    for form in ("fused", "split"):
        r = res[form]
        r["eff_kv_gbs"] = round(res["kv_bytes_per_step"] / (r["ms_per_step"] * 1e6), 2)
        r["frac_nominal_step"] = round(t_nom / r["ms_per_step"], 4)
    cache.free()
    return res


def measure_contiguous(dk, cfg, seed, flags, steps, warmup):
    st, _ = contiguous_steps(dk, cfg, seed, flags)
    info = st.info()
    res = {"workload": cfg["name"], "batch": cfg["batch"], "ratio": cfg["ratio"],
           "kv_bytes_per_step": kv_bytes(info), "host_bytes": info["host_bytes"], "hbm_bytes": info["dev_bytes"],
           "plan": {k: info[k] for k in ("host_wgs", "dev_wgs", "host_chunk", "dev_chunk", "host_items",
                                         "dev_items")}}
    res.update(measure_forms(dk, st, steps, warmup))
    t_nom = max(res["host_bytes"] / (PCIE_RAW_GBS * 1e6), res["hbm_bytes"] / (HBM_PEAK_GBS * 1e6))
    for form in ("fused", "split"):
        r = res[form]
        r["eff_kv_gbs"] = round(res["kv_bytes_per_step"] / (r["ms_per_step"] * 1e6), 2)
        r["latency_ms_per_token"] = round(r["ms_per_step"] / cfg["batch"], 5)
        r["frac_nominal_step"] = round(t_nom / r["ms_per_step"], 4)
    st.cache.free()
    return res


def decode_loop(dk, cfg, seed, flags, steps, warmup):
    """The growing decode loop (DirectKV README, Artifact Evaluation, Figure 11(a):
    decode latency vs sequence length): each step appends at position L_b,
    attends over L_b + 1 tokens and advances L_b by one, in one launch of
    dkv_decode_step (plus the paged tier lists and, with a hidden state, the
    projection).  Timed eagerly and as replays of one captured graph that also
    advances the lengths."""
    import numpy as np
    import torch
    from decode_attention_host_amd.cache_build import contiguous_cache, paged_cache
    from synth import TensorId, kv_raw, normal_bf16, paged_table, query
    B, hq, hkv, d, th = cfg["batch"], cfg["hq"], cfg["hkv"], cfg["d"], cfg["theta"]
    total = warmup + steps + 8
    lens = [int(n) for n in cfg["lens"]]
    x = wk = wv = None
    if cfg["layout"] == "paged":
        L0 = lens
        cap = [L + total + 1 for L in L0]
        ks, vs = kv_raw(seed, L0, hkv, d)
        pt, nh, nd = paged_table(seed, cap, cfg["page"], cfg["ratio"])
        cache = paged_cache(hkv, d, cap, pt, nh, nd, ks, vs, th, page=cfg["page"], host_flags=flags, upto=L0)
        hid = cfg["hidden"]
        x = torch.from_numpy(normal_bf16(seed, TensorId.X, (B, hid)).view(np.int16)).cuda()
        wk = torch.from_numpy(normal_bf16(seed, TensorId.WK, (hid, hkv * d), std=cfg["w_std"]).view(np.int16)).cuda()
        wv = torch.from_numpy(normal_bf16(seed, TensorId.WV, (hid, hkv * d), std=cfg["w_std"]).view(np.int16)).cuda()
        k_new = v_new = None
        ratio = 0.0
    else:
        # the cache ends at the workload's length after the timed steps
        L0 = [L - total for L in lens]
        ks, vs = kv_raw(seed, lens, hkv, d)
        ratio = cfg["ratio"]
        assert ratio in (0.0, 1.0), "a growing contiguous cache keeps its split point only at r = 0 or 1"
        cache = contiguous_cache(hkv, d, lens, ratio, ks, vs, th, host_flags=flags, upto=L0)
        k_new = torch.from_numpy(np.stack([k[L] for k, L in zip(ks, L0)]).view(np.int16)).cuda()
        v_new = torch.from_numpy(np.stack([v[L] for v, L in zip(vs, L0)]).view(np.int16)).cuda()
    del ks, vs
    q = torch.from_numpy(query(seed, B, hq, d).view(np.int16)).cuda()
    sl = torch.tensor(L0, dtype=torch.int32, device="cuda")
    pos = sl.clone()
    start = sl.clone()
    ws = dk.decode_step_workspace(cache, B, hq, ratio, int(x.shape[1]) if x is not None else 0)
    oo = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
    ol = torch.empty((B, hq), dtype=torch.float32, device="cuda")

    def step():
        dk.decode_step(cache, q, pos, sl, ratio, 1.0 / math.sqrt(d), th, k_new=k_new, v_new=v_new, x=x, wk=wk,
                       wv=wv, workspace=ws, out_o=oo, out_lse=ol)
        sl.add_(1)
        pos.add_(1)

    def run(fn):
        sl.copy_(start)
        pos.copy_(start)
        ms, _ = timed_loop(fn, steps, warmup)
        return ms, int(sl[0].item()) - L0[0]

    eager_ms, grown = run(step)
    sl.copy_(start)
    pos.copy_(start)
    g = dk.StepGraph(step, warmup=1)
    graph_ms_, grown_g = run(g.replay)
    errors = dk.decode_errors(cache, ws)
    kv0 = sum(L0) * hkv * d * 4
    kv1 = sum(L + steps + warmup for L in L0) * hkv * d * 4
    res = {"workload": cfg["name"], "layout": cfg["layout"], "offload_ratio": ratio, "timed_steps": steps,
           "warmup_steps": warmup, "first_len": L0 if B <= 4 else {"sum": sum(L0)},
           "eager_ms_per_step": round(eager_ms, 5), "graph_ms_per_step": round(graph_ms_, 5),
           "eff_kv_gbs_eager": round((kv0 + kv1) / 2 / (eager_ms * 1e6), 2),
           "lengths_advanced_eager": grown, "lengths_advanced_graph": grown_g, "error_flags": errors,
           "note": "one captured graph replayed while every sequence grows by one token per step"}
    log(f"[bench] decode loop {cfg['name']}: eager {eager_ms:.4f} ms/step, graph {graph_ms_:.4f} ms/step "
        f"({grown} steps of growth)")
    cache.free()
    return res


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
        # (step times without the library's per-launch event pairs; kernel
        # times from one more loop with them)
        gpu_warm(step)
        ms = statistics.median(timed_loop(step, steps, warmup)[0] for _ in range(5))
        return ms, kernel_times(dk, step, steps)

    out = []
    for r in cfg.get("ratios", [cfg["ratio"]]):
        cache = contiguous_cache(hkv, d, lens, r, ks, vs, th, host_flags=flags, upto=q_pos0)
        info = dk.prefill_fused_plan(cache, B, hq, q_start, q_pos0, lens, r)
        ws = torch.empty(max(256, info["workspace_bytes"]), dtype=torch.uint8, device="cuda")
        oo = torch.empty((T, hq, d), dtype=torch.float32, device="cuda")
        ol = torch.empty((T, hq), dtype=torch.float32, device="cuda")
        f_ms, f_kt = timed(lambda: dk.prefill_fused(cache, q, q_start, q_pos0, lens, r, scale, th, k_new=k_new,
                                                    v_new=v_new, workspace=ws, out_o=oo, out_lse=ol))
        cache.free()
        cache = contiguous_cache(hkv, d, lens, r, ks, vs, th, host_flags=flags)
        bufs = dk.alloc_prefill_buffers(cache, B, hq, q_start, q_pos0, lens, r)

        def step():
            dk.project_rope_append(cache, B, sl, r, sidx, pos, k_new=k_new, v_new=v_new, rope_theta=th)
            dk.prefill_attn_split(cache, q, q_start, q_pos0, lens, r, scale, th, bufs=bufs)
            dk.merge_lse(bufs.part_o, bufs.part_lse, bufs.split_offsets, T, hq, d, out_o=bufs.out_o,
                         out_lse=bufs.out_lse)
        s_ms, s_kt = timed(step)
        pf_ms = s_kt["prefill"]
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
            ws = lin.workspace(m)
            f = flushed_steps(dk, lambda: lin(x, y, ws), iters, flush)
            med = f["ms_median"]
            t_star = max(hb / (bw_h * 1e6), db / (bw_d * 1e6))
            t_nom = max(hb / (PCIE_RAW_GBS * 1e6), db / (HBM_PEAK_GBS * 1e6))
            out.append({"ratio": round(r, 5), "tokens": m, "host_bytes": hb, "hbm_bytes": db,
                        "ms_median": med, "kernel_ms": f["kernel_ms"].get("linear"),
                        "eff_weight_gbs": round((hb + db) / (med * 1e6), 1),
                        "roofline_ms_measured": round(t_star, 4), "frac_measured": round(t_star / med, 3),
                        "roofline_ms_nominal": round(t_nom, 4), "frac_nominal": round(t_nom / med, 3)})
            log(f"[bench] linear r={r:.4f} m={m}: {med:.4f} ms, {out[-1]['eff_weight_gbs']} GB/s")
        lin.free()
    del flush
    return {"sweep": out}


def cpu_baseline(cfg, raw, budget_s):
    """The fp64 oracle as it stands, on the host, over the same workload: numpy
    with BLAS on every core of this process's affinity set (numpy's elementwise
    steps use one core).  The oracle processes one KV head at a time; whole KV
    heads are run until the budget is spent, at least one."""
    import oracle as O
    from synth import query
    cores = len(os.sched_getaffinity(0))
    limiter, blas_threads = None, None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        blas_threads = max((p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"),
                           default=None)
    except Exception:  # pragma: no cover
        pass
    ks, vs = raw
    L, hq, hkv, d = cfg["lens"][0], cfg["hq"], cfg["hkv"], cfg["d"]
    g = hq // hkv
    qb = query(cfg.get("seed", 0), 1, hq, d)
    t0 = time.perf_counter()
    done = 0
    for kvh in range(hkv):
        O.decode_sequence(qb[0], ks[0], vs[0], L - 1, cfg["theta"], 1.0 / math.sqrt(d),
                          heads=list(range(kvh * g, kvh * g + g)))
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    used = blas_threads or cores
    done_bytes = L * done * d * 4
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"{done} of {hkv} KV heads ({g} query heads each) of the {cfg['name']} workload "
                      f"({L} tokens), the oracle's decode_sequence per KV head including the key rotation, "
                      f"{done_bytes} KV bytes in {dt:.1f}s; numpy float64, BLAS on {used} thread(s) of {cores} "
                      f"cores in the affinity set (elementwise steps single-threaded)",
            "ms_per_step_extrapolated": round(dt / done * hkv * 1e3, 1)}


def load_traffic(workload_name, ratio, form):
    """HBM + host-link bytes per launch of the decode kernel from the stored
    rocprofv3 FETCH_SIZE / WRITE_SIZE passes of this workload, offload ratio
    and step form, or None when none is stored or the kernel sources changed
    since."""
    p = os.path.join(ROOT, "profiles", f"decode_{workload_name}_traffic.json")
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("kernel_src_sha") != kernel_src_sha() or t.get("offload_ratio") != ratio:
        return None
    return t.get("forms", {}).get(form, {}).get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b_1m")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--ratio", type=float, default=None,
                    help="offload ratio for the main workload instead of its own (profiling runs)")
    ap.add_argument("--form", choices=["fused", "split"], default=None,
                    help="time only this form of the step for the headline (default: both, the faster "
                         "one is the headline); profiling runs time one form (default fused)")
    ap.add_argument("--host-flags", choices=["coherent", "noncoherent"], default="coherent")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-loop", action="store_true")
    ap.add_argument("--sweep-iters", type=int, default=10)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--tune", default="", help="comma list of dkv_tuning fields, e.g. host_wgs=256")
    ap.add_argument("--extra", default="tiny,llama3_8b_32k,opt_6_7b_b8,fused_ragged,llama3_8b_prefill_2k,"
                                       "llama3_8b_mlp_up_linear,staged_prefetch",
                    help="other workloads measured after the headline ('' for none)")
    ap.add_argument("--profile-run", action="store_true",
                    help="short run for rocprofv3: headline steps plus two calibration reads of known "
                         "size (a 256 MiB HBM copy and a 1 GiB zero-copy read of the host pool, or "
                         "all of it when smaller)")
    args = ap.parse_args()
    args.form_fixed = args.form is not None
    if args.form is None:
        args.form = "fused"

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
    B, hq, hkv, d, lens, ratio = cfg["batch"], cfg["hq"], cfg["hkv"], cfg["d"], cfg["lens"], cfg["ratio"]
    log(f"[bench] workload {cfg['name']}: B={B} Hq={hq} Hkv={hkv} D={d} "
        f"L={lens if len(lens) <= 4 else str(len(lens)) + ' seqs'} r={ratio}")
    t0 = time.time()
    st, raw = contiguous_steps(dk, cfg, args.seed, flags)
    log(f"[bench] cache built in {time.time() - t0:.1f}s")
    info = st.info()
    kvb = kv_bytes(info)
    step = getattr(st, args.form)

    if args.profile_run:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(3)
        dst.copy_(src)
        cache = st.cache
        host_bytes = cache.host_rows * hkv * d * 2 if cache.host_k is not None else 0
        if host_bytes >= (64 << 20):
            dk.probe_read(cache.host_k.dev_ptr, min(host_bytes, 1 << 30) // (1 << 20) << 20, 64,
                          nontemporal=True, iters=1)
        torch.cuda.synchronize()
        gpu_warm(step, 0.5)
        ms, _ = timed_loop(step, args.steps, args.warmup)
        log(f"[bench] profile run ({args.form}): {args.steps} steps, {ms:.4f} ms/step")
        st.cache.free()
        return

    # headline: W warm-up steps, then exactly K timed steps, for both forms of
    # the step; the faster one is the headline (--form fixes one)
    timed = {}
    for form in ((args.form,) if args.form_fixed else ("fused", "split")):
        fn = getattr(st, form)
        gpu_warm(fn, 0.5)
        dk.kernel_timing(True)
        for k in dk.api.KERNELS:
            dk.kernel_timing_read(k)
        f_ms, f_wall = timed_loop(fn, args.steps, args.warmup)
        f_kt = {k: dk.kernel_timing_read(k) for k in dk.api.KERNELS}
        dk.kernel_timing(False)
        timed[form] = (f_ms, f_wall, f_kt)
        log(f"[bench] {form} step {f_ms:.4f} ms (wall {f_wall / args.steps * 1e3:.4f} ms)")
    form = min(timed, key=lambda k: timed[k][0])
    ms, wall, kt = timed[form]
    step = getattr(st, form)
    n_attn, attn_total = kt["attn"]
    attn_ms = attn_total / max(1, n_attn)
    value = kvb / (ms * 1e6)
    log(f"[bench] headline {form} step {ms:.4f} ms, decode kernel {attn_ms:.4f} ms over {n_attn} launches, "
        f"{value:.2f} GB/s")
    other = "split" if form == "fused" else "fused"
    other_ms = timed[other][0] if other in timed else None
    graph = graph_ms(dk, step, max(5, args.steps // 2))
    log(f"[bench] graph replay of the {form} step {graph:.4f} ms")

    probe = {}
    if not args.no_probe:
        probe = run_probe(dk, st.cache.host_k, st.cache.host_v, 1 << 30)
        log(f"[bench] probe: {json.dumps({k: v for k, v in probe.items() if 'sweep' not in k})}")
    nominal, link = pcie_nominal_gbs(getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None))
    probe["host_link_nominal_gbs"] = round(nominal, 2) if nominal else None
    probe["host_link"] = link

    host_dominant = info["host_bytes"] * HBM_PEAK_GBS >= info["dev_bytes"] * PCIE_RAW_GBS
    if host_dominant:
        achieved = info["host_bytes"] / (attn_ms * 1e6)
        peak = round(nominal, 2) if nominal else PCIE_RAW_GBS
        meas = probe.get("host_zero_copy_gbs")
        meas_dma = probe.get("host_dma_gbs")
    else:
        achieved = info["dev_bytes"] / (attn_ms * 1e6)
        peak = HBM_PEAK_GBS
        meas = probe.get("hbm_read_gbs")
        meas_dma = None
    roofline = {"bound": "hbm" if not host_dominant else "host_link", "achieved": round(achieved, 3),
                "peak": peak, "unit": "GB/s", "frac": round(achieved / peak, 4),
                "traffic": load_traffic(cfg["name"], ratio, form),
                "kernel": "decode_kernel (one-launch step: append + attention + merge)" if form == "fused"
                else "decode_kernel (split attention)",
                "kernel_ms": round(attn_ms, 5),
                "algorithmic_bytes": info["host_bytes"] if host_dominant else info["dev_bytes"],
                "peak_note": ("PCIe 5.0 x16 per direction from the sysfs link speed and width, 128b/130b "
                              f"encoding ({PCIE_RAW_GBS:.0f} GB/s raw)") if host_dominant else "HBM3E",
                "frac_of_raw_link": round(achieved / PCIE_RAW_GBS, 4) if host_dominant else None,
                "peak_measured": meas, "peak_measured_dma": meas_dma,
                "frac_measured": round(achieved / meas, 4) if meas else None}

    bw_h = probe.get("host_zero_copy_gbs") or 50.0
    bw_d = probe.get("hbm_read_gbs") or 5000.0
    sweep = None
    if not args.no_sweep and B == 1:
        r_star = bw_h / (bw_h + bw_d)
        ratios = [0.0, r_star / 2, r_star, 0.25, 0.5, 0.75, 0.9, 1.0]
        pts = ratio_sweep(dk, cfg, args.seed, flags, ratios, args.sweep_iters, bw_h, bw_d, raw=raw)
        sweep = {"r_star": round(r_star, 5), "points": pts, "best_split": best_split(pts, bw_h, bw_d)}
        flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        sweep["paged_hbm"] = paged_hbm_point(dk, cfg, args.seed, raw[0], raw[1], args.sweep_iters, flush, bw_d, pts)
        del flush

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, raw, args.cpu_budget)
        log(f"[bench] cpu baseline: {cpu}")
    del raw
    st.cache.free()

    loops = {}
    if not args.no_loop:
        for name in ("llama3_8b_32k", "fused_ragged"):
            loops[name] = decode_loop(dk, workload(name, seed=args.seed), args.seed, flags, 200, 20)

    workloads = {}
    for name in [x for x in args.extra.split(",") if x]:
        t0 = time.time()
        if name == "staged_prefetch":
            r_star = bw_h / (bw_h + bw_d)
            workloads[name] = {
                "llama3_8b_32k": measure_staged(dk, workload("llama3_8b_32k", seed=args.seed), args.seed, flags,
                                                [r_star, 0.25, 1.0], [2048, 8192], 10, bw_h, bw_d),
                "llama3_8b_1m": measure_staged(dk, workload("llama3_8b_1m", seed=args.seed), args.seed, flags,
                                               [r_star, 0.25, 1.0], [4096, 16384, 65536], 5, bw_h, bw_d)}
            log(f"[bench] {name} measured in {time.time() - t0:.1f}s")
            continue
        wcfg = workload(name, seed=args.seed)
        if wcfg.get("layout") == "linear":
            workloads[name] = measure_linear(dk, wcfg, args.seed, 20, bw_h, bw_d)
        elif "new" in wcfg:
            workloads[name] = measure_prefill(dk, wcfg, args.seed, flags, 10, 3)
        elif wcfg["layout"] == "paged":
            workloads[name] = measure_fused_paged(dk, wcfg, args.seed, flags, 10, 3)
        else:
            workloads[name] = measure_contiguous(dk, wcfg, args.seed, flags, 20, 5)
            if name == "llama3_8b_32k" and not args.no_sweep:
                r_star = bw_h / (bw_h + bw_d)
                workloads[name]["sweep"] = ratio_sweep(dk, wcfg, args.seed, flags,
                                                       [0.0, r_star, 0.25, 0.5, 0.75, 0.9, 1.0], 20, bw_h, bw_d)
        log(f"[bench] {name} measured in {time.time() - t0:.1f}s")
        if name in loops and "fused" in workloads[name]:
            f = workloads[name]["fused"]["ms_per_step"]
            loops[name]["fixed_len_ms_per_step"] = f
            loops[name]["eager_vs_fixed"] = round(loops[name]["eager_ms_per_step"] / f, 4)
            loops[name]["graph_vs_fixed"] = round(loops[name]["graph_ms_per_step"] / f, 4)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": B, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": d, "context": lens[0] if len(set(lens)) == 1 else lens,
                   "offload_ratio": ratio, "layout": cfg["layout"], "rope_theta": cfg["theta"],
                   "step_form": form, "host_memory": args.host_flags, "kv_bytes_per_step": kvb},
        "latency_ms_per_token": round(ms / B, 5),
        "other_form": {"form": other, "ms_per_step": round(other_ms, 5) if other_ms else None},
        "graph": {"ms_per_step": round(graph, 5), "eff_kv_gbs": round(kvb / (graph * 1e6), 3),
                  "note": "the same step captured into one HIP graph and replayed"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "probe": probe,
        "plan": info,
        "kernel_ms": {k: round(v[1] / max(1, v[0]), 5) for k, v in kt.items() if v[0]},
        "sweep": sweep,
        "decode_loop": loops,
        "workloads": workloads,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
