#!/usr/bin/env python3
"""Benchmark: decode step of an interleaved CSA+HCA layer pair on one MI355X.

A step = one pass of the whole decode hot path for a batch of requests:
  CSA layer: append+compress -> indexer scoring -> top-k -> sparse MQA
  HCA layer: append+compress -> dense MQA
at the V4-Pro shape (128 heads x d 512, RoPE 64, window 128, indexer 64x128,
top-1024), batch 32 at 128K context (32768 CSA entries, 1024 HCA entries per
request), FP8/BF16 cache.  Every step appends the next token of every request,
so one step in four completes a CSA entry and the compressor runs as in a real
decode.  Inputs are synthetic, seeded, already resident in HBM when timing
starts.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--batch B] [--ctx N]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0
METRIC = "CSA/HCA decode queries/s at 128K–1M ctx; % HBM BW and % MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=None,
                    help="requests (decode) or tokens (out_proj, index_q); default 32, for index_q 8192 (a prefill "
                         "chunk)")
    ap.add_argument("--ctx", type=int, default=131072)
    ap.add_argument("--policy", default="auto", choices=["auto", "hi", "lo"])
    ap.add_argument("--idx-store", default="fp8", choices=["fp8", "mxfp4"],
                    help="indexer query / key rows: E4M3 with one scale per row (fp8), or MXFP4 (E2M1 with a "
                         "power-of-two scale per 32 dims); decode and prefill workloads")
    ap.add_argument("--cpu-sample", type=int, default=8,
                    help="requests whose caches the CPU-oracle baseline prepares; it then times queries over them "
                         "for about 12 s (0: skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this size (traffic calibration under --pmc)")
    ap.add_argument("--layers", type=int, default=4,
                    help="decode: layer pairs in rotation (step s runs layer s %% L); 4 keeps each step's caches "
                         "out of the 256 MB Infinity Cache, 1 measures a warm cache")
    ap.add_argument("--calibrate", type=int, default=1,
                    help="measure the device's copy / read bandwidth and matrix-core rates (1) or not (0)")
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "hca_decode", "pair_1m", "out_proj", "index_q"],
                    help="decode: the CSA+HCA decode step, batch 32 at 128K (the headline); prefill: one "
                         "8192-token CSA chunk on a 256K-token prefix; hca_decode: the HCA decode step, batch 16 at "
                         "64K; pair_1m: the CSA+HCA decode step for 4 requests at 1M/512K/64K/4K; out_proj: the "
                         "grouped output projection (128 heads x 512 -> 16 groups of rank 1024 -> 7168) of --batch "
                         "tokens; index_q: the indexer's query path (7168 -> 1024 -> 64 x 128, MXFP4 weights, MXFP8 "
                         "activations) of --batch tokens")
    return ap.parse_args()


def main():
    a = parse()
    if a.batch is None:
        a.batch = 8192 if a.workload == "index_q" else 32
    if a.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1", "n_gpus": a.gpus}))
        sys.exit(2)
    if a.workload == "prefill":
        return prefill_main(a)
    if a.workload in ("hca_decode", "pair_1m"):
        return decode_mix_main(a)
    if a.workload == "out_proj":
        return out_proj_main(a)
    if a.workload == "index_q":
        return index_q_main(a)
    import torch
    from long_context_compressed_02_amd import binding as B
    from long_context_compressed_02_amd import synth

    dev = "cuda"
    torch.cuda.set_device(0)
    w = synth.CSA_DECODE_128K
    Bsz, ctx = a.batch, a.ctx
    steps, warm = a.steps, a.warmup
    R = max(1, a.layers)
    n_graph = warm + steps                        # steps captured as graphs (warm-up, then the timed K)
    n_eager = 2 * steps                           # two eager passes with the per-kernel timers on
    n_total = n_graph + n_eager
    mx = a.idx_store == "mxfp4"
    cfg = B.make_cfg(idx_store=B.DSV4_STORE_MXFP4 if mx else B.DSV4_STORE_FP8, **w.shape())
    policy = {"auto": B.DSV4_POLICY_AUTO, "hi": B.DSV4_POLICY_HI, "lo": B.DSV4_POLICY_LO}[a.policy]
    H, d, HI_, dI, k = w.n_heads, w.d, w.idx_heads, w.idx_dim, w.topk

    # ---------------------------------------------------------------- caches
    # R layer pairs (CSA + HCA), each with its own pools at its own addresses:
    # step s runs layer s % R at position ctx + s // R, as a model's decode
    # walks its layers, so a layer's cache was last touched R-1 layer-steps
    # earlier (R >= 3 puts more than the 256 MB Infinity Cache in between).
    pos_max = ctx + (n_total + R - 1) // R + 1
    need_blocks = (pos_max + 127) // 128
    bt = torch.arange(Bsz * need_blocks, dtype=torch.int32, device=dev).view(Bsz, need_blocks)
    # interleave requests' blocks so physical placement is not contiguous per request
    perm = torch.from_numpy(synth.permutation(w.wid, Bsz * need_blocks)).to(dev).to(torch.int32)
    bt = perm[bt.view(-1).long()].view(Bsz, need_blocks).contiguous()
    n_csa, n_hca = ctx // 4, ctx // 128
    t_setup = time.time()
    layers = []
    for li in range(R):
        csa = B.LayerCache(cfg, B.DSV4_CSA, Bsz, need_blocks, Bsz * need_blocks, bt)
        hca = B.LayerCache(cfg, B.DSV4_HCA, Bsz, need_blocks, Bsz * need_blocks, bt)
        if li == 0:
            for r in range(Bsz):
                rr = torch.full((n_csa,), r, dtype=torch.int32, device=dev)
                ar = torch.arange(n_csa, dtype=torch.int32, device=dev)
                B.dsv4_cache_write_entries(cfg, csa, B.DSV4_TARGET_ENTRY, rr, ar,
                                           torch.from_numpy(synth.entries(w, r, n_csa, 0)).to(dev))
                B.dsv4_cache_write_entries(cfg, csa, B.DSV4_TARGET_INDEX_KEY, rr, ar,
                                           torch.from_numpy(synth.index_keys(w, r, n_csa)).to(dev))
                rh = torch.full((n_hca,), r, dtype=torch.int32, device=dev)
                B.dsv4_cache_write_entries(cfg, hca, B.DSV4_TARGET_ENTRY, rh,
                                           torch.arange(n_hca, dtype=torch.int32, device=dev),
                                           torch.from_numpy(synth.entries(w, r, n_hca, 1)).to(dev))
                kv, gate, kI, gI = synth.window_tokens(w, r, 128, 0)
                bf = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16)
                B.dsv4_state_write_tokens(cfg, csa, r, ctx - 128, bf(kv), bf(gate), bf(kI), bf(gI))
                kv, gate, _, _ = synth.window_tokens(w, r, 128, 1)
                B.dsv4_state_write_tokens(cfg, hca, r, ctx - 128, bf(kv), bf(gate))
        else:                                     # the same contents at other addresses
            c0, h0 = layers[0]
            csa.entries.copy_(c0.entries)
            csa.index_keys.copy_(c0.index_keys)
            csa.state.copy_(c0.state)
            hca.entries.copy_(h0.entries)
            hca.state.copy_(h0.state)
        layers.append((csa, hca))
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    # ---------------------------------------------------------------- per-step inputs (resident)
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    rn = lambda *s: torch.randn(*s, generator=g, device=dev, dtype=torch.float32)
    steps_in = []
    for s in range(n_total):
        steps_in.append(dict(
            kv=rn(Bsz, d).bfloat16(), gate=rn(Bsz, d).bfloat16(), kI=rn(Bsz, dI).bfloat16(), gI=rn(Bsz, dI).bfloat16(),
            kvh=rn(Bsz, d).bfloat16(), gateh=rn(Bsz, d).bfloat16(),
            q=rn(Bsz, H, d).bfloat16(), qh=rn(Bsz, H, d).bfloat16(),
            qI=rn(Bsz, HI_, dI).bfloat16(), w=rn(Bsz, HI_) / 8.0,
            pos=torch.full((Bsz,), ctx + s // R, dtype=torch.int32, device=dev)))
    req = torch.arange(Bsz, dtype=torch.int32, device=dev)
    sinks = torch.from_numpy(synth.sinks(w)).to(dev)
    ws = torch.empty(B.dsv4_workspace_bytes(cfg, Bsz, need_blocks * 32), dtype=torch.uint8, device=dev)
    topk = torch.empty((Bsz, k), dtype=torch.int32, device=dev)
    out_c = torch.empty((Bsz, H, d), dtype=torch.bfloat16, device=dev)
    out_h = torch.empty((Bsz, H, d), dtype=torch.bfloat16, device=dev)

    def step(s, stream, layer=None):
        x = steps_in[s]
        csa, hca = layers[s % R if layer is None else layer]
        B.dsv4_compress_kv_decode(cfg, csa, x["kv"], x["gate"], x["kI"], x["gI"], req, x["pos"], stream)
        B.dsv4_index_topk_decode(cfg, csa, x["qI"], x["w"], req, x["pos"], topk, ws, stream)
        B.dsv4_csa_attend_decode(cfg, csa, x["q"], req, x["pos"], topk, sinks, out_c, policy, stream)
        B.dsv4_compress_kv_decode(cfg, hca, x["kvh"], x["gateh"], None, None, req, x["pos"], stream)
        B.dsv4_hca_attend_decode(cfg, hca, x["qh"], req, x["pos"], sinks, out_h, policy, stream)

    for kid in range(B.DSV4_K_COUNT):
        B.dsv4_timer_enable(kid, False)
        B.dsv4_timer_read(kid, True)
    # the read-only calls once, eagerly, before capture (module load, LDS limits)
    x0, (c0, h0) = steps_in[0], layers[0]
    p_prev = torch.full((Bsz,), ctx - 1, dtype=torch.int32, device=dev)
    cur = torch.cuda.current_stream()
    B.dsv4_index_topk_decode(cfg, c0, x0["qI"], x0["w"], req, p_prev, topk, ws, cur)
    B.dsv4_csa_attend_decode(cfg, c0, x0["q"], req, p_prev, topk, sinks, out_c, policy, cur)
    B.dsv4_hca_attend_decode(cfg, h0, x0["qh"], req, p_prev, sinks, out_h, policy, cur)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- one hipGraph per step
    graphs = []
    cap = torch.cuda.Stream()
    for s in range(n_graph):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=cap):
            step(s, torch.cuda.current_stream())
        graphs.append(gr)
    torch.cuda.synchronize()
    for s in range(warm):
        graphs[s].replay()
    torch.cuda.synchronize()
    # timed region: the K steps, each one graph replay, in order (state advances)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(warm, n_graph):
        graphs[s].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps

    # median over >= 100 replays, each timed on its own: the K step graphs
    # cycled (cold rotation; positions repeat, so the cache contents drift but
    # every replay does a step's work), and one layer's step replayed back to
    # back (warm: its data stays in the Infinity Cache)
    def replay_median(order):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i, s in enumerate(order):
            graphs[s].replay()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(len(order))]))
    n_rep = max(100, steps)
    timed = list(range(warm, n_graph))
    med_cold = replay_median([timed[i % len(timed)] for i in range(n_rep)])
    med_warm = replay_median([timed[0]] * n_rep)

    # per-kernel durations: eager steps continuing the timeline with the
    # library's HIP-event timers on the launch stream -- K rotating steps
    # (cold), then K steps on one layer (warm)
    names = {B.DSV4_K_COMPRESS: "compress", B.DSV4_K_INDEX_SCORE: "index_score", B.DSV4_K_TOPK: "topk",
             B.DSV4_K_ATTEND: "attend"}

    def timer_pass(ss, layer):
        for kid in range(B.DSV4_K_COUNT):
            B.dsv4_timer_enable(kid, True)
        hold_stream(stream, 1.0e-3 * len(ss))
        for s in ss:
            step(s, stream, layer)
        torch.cuda.synchronize()
        out = {}
        for kid, nm in names.items():
            ms, n = B.dsv4_timer_read(kid, True)
            out[nm] = dict(total_ms=ms, launches=n, avg_us=1e3 * ms / max(n, 1))
        for kid in range(B.DSV4_K_COUNT):
            B.dsv4_timer_enable(kid, False)
        return out
    kern = timer_pass(range(n_graph, n_graph + steps), None)
    kern_warm = timer_pass(range(n_graph + steps, n_total), 0)

    if a.calib_copy_mib:
        # a copy of known size through the calibration library's copy kernel
        # (the traffic counters' calibration under rocprofv3 --pmc)
        src = torch.empty(a.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        calib_lib().dsv4calib_copy_gbs(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                       src.numel(), 0)
        torch.cuda.synchronize()
        del src, dst
    cal = calibrate() if a.calibrate else None

    # ---------------------------------------------------------------- roofline
    # algorithmic work per step (positions of the eager cold pass, averaged)
    tpos = [ctx + s // R for s in range(n_graph, n_graph + steps)]
    n_vis = np.mean([(t + 1) // 4 for t in tpos])
    n_h = np.mean([(t + 1) // 128 for t in tpos])
    row_b = (dI // 2 if mx else dI) + 4                 # E2M1 codes + 4 E8M0 bytes, or E4M3 codes + fp32 scale
    score_bytes = Bsz * n_vis * (row_b + 4) + Bsz * HI_ * row_b       # keys+scales read, scores written, queries
    rec_b = (d - 64) + 2 * 64 + 4                        # 580 B per stored record
    csa_recs = Bsz * (k + 128)
    hca_recs = Bsz * (n_h + 128)
    attend_bytes_step = (csa_recs + hca_recs) * rec_b + 2 * (2 * Bsz * H * d * 2)
    attend_flops_step = (csa_recs + hca_recs) * H * 4 * d
    per_launch = {
        "index_score": dict(bound="hbm", work=score_bytes, unit="GB/s", peak=HBM_PEAK_GBS,
                            measured=None if cal is None else cal["read_GBps"]),
        "attend": dict(bound="mfma", work=attend_flops_step / 2, unit="TFLOP/s", peak=BF16_PEAK_TFLOPS,
                       measured=None if cal is None else max(cal["bf16_TFLOPs"], cal["bf16_32x32_TFLOPs"])),
    }

    def roofline(kn):
        dom = max(kn, key=lambda n_: kn[n_]["total_ms"])
        if dom not in per_launch:
            dom = "index_score"
        pl = per_launch[dom]
        achieved = pl["work"] / (kn[dom]["avg_us"] * 1e-6) / (1e9 if pl["unit"] == "GB/s" else 1e12)
        kname = {"index_score": "k_index_score_decode",
                 "attend": lo_kernel(d, max(k + 128, need_blocks + 128))}[dom]
        out = {"kernel": kname, "bound": pl["bound"], "achieved": round(achieved, 2), "peak": pl["peak"],
               "unit": pl["unit"], "frac": round(achieved / pl["peak"], 4),
               "traffic": measured_traffic(dom) if (Bsz, ctx, R, mx) == (32, 131072, 4, False) else None}
        if pl["measured"]:
            out["peak_measured"] = round(pl["measured"], 1)
            out["frac_measured"] = round(achieved / pl["measured"], 4)
        return out
    roof = roofline(kern)
    step_bytes = score_bytes + attend_bytes_step
    value = Bsz / (ms_step * 1e-3)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if a.cpu_sample > 0:
        cpu = cpu_baseline(w, a.cpu_sample, ctx + warm, idx_mode=2 if mx else 1)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "queries/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4/fp8/bf16" if mx else "fp8/bf16", "data": "synthetic",
        "config": {"workload": f"V4-Pro CSA+HCA layer-pair decode, batch {Bsz} x {ctx // 1024}K ctx "
                               f"({ctx // 4} CSA / {ctx // 128} HCA entries per request), top-{k}, "
                               f"{H} heads x d {d}, window 128" + (", MXFP4 indexer" if mx else "") +
                               f"; {R} layer pairs in rotation (each step's caches cold), one hipGraph per step",
                   "batch": Bsz, "ctx": ctx, "topk": k, "heads": H, "d": d, "policy": a.policy,
                   "idx_store": a.idx_store, "layers_in_rotation": R},
        "roofline": roof,
        "cpu_baseline": cpu,
        "breakdown_us": {n_: round(v["avg_us"], 2) for n_, v in kern.items()},
        "launches_per_step": {n_: v["launches"] / steps for n_, v in kern.items()},
        "graph_replay_median_us": {"cold": round(1e3 * med_cold, 2), "warm": round(1e3 * med_warm, 2),
                                   "replays": n_rep},
        "warm": {"queries_per_s": round(Bsz / (med_warm * 1e-3), 1),
                 "breakdown_us": {n_: round(v["avg_us"], 2) for n_, v in kern_warm.items()},
                 "roofline": roofline(kern_warm)},
        "step_algorithmic_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "attend_TFLOPs": round(attend_flops_step / (kern["attend"]["total_ms"] / steps * 1e-3) / 1e12, 1),
        "calibration": cal,
        "setup_s": round(t_setup, 1),
    }
    print(json.dumps(res), flush=True)


def prefill_main(a):
    """One prefill chunk of a CSA layer: 8192 new tokens appended to a
    262144-token prefix (65536 entries and index keys), top-512.  A step =
    compress + indexer + top-k + sparse attend over the chunk.  Inputs are
    synthetic N(0,1) values generated on the device before timing."""
    import torch
    from long_context_compressed_02_amd import binding as B
    from long_context_compressed_02_amd import synth

    dev = "cuda"
    torch.cuda.set_device(0)
    w = synth.CSA_PREFILL_8K
    mx = a.idx_store == "mxfp4"
    cfg = B.make_cfg(idx_store=B.DSV4_STORE_MXFP4 if mx else B.DSV4_STORE_FP8, **w.shape())
    idx_peak = FP4_PEAK_TFLOPS if mx else FP8_PEAK_TFLOPS
    H, d, HI_, dI, k = w.n_heads, w.d, w.idx_heads, w.idx_dim, w.topk
    P, C = w.ctx[0], w.chunk
    T = P + C
    steps, warm = a.steps, a.warmup
    nb = (T + 127) // 128 + 1
    perm = torch.from_numpy(synth.permutation(w.wid, nb)).to(dev).to(torch.int32)
    bt = perm.view(1, nb).contiguous()
    csa = B.LayerCache(cfg, B.DSV4_CSA, 1, nb, nb, bt)
    g = torch.Generator(device=dev)
    g.manual_seed(4321)
    rn = lambda *s_: torch.randn(*s_, generator=g, device=dev, dtype=torch.float32)
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    t_setup = time.time()
    n_csa = P // 4
    for a0 in range(0, n_csa, 1 << 15):
        nn = min(1 << 15, n_csa - a0)
        idx = torch.arange(a0, a0 + nn, dtype=torch.int32, device=dev)
        rr = torch.zeros(nn, dtype=torch.int32, device=dev)
        B.dsv4_cache_write_entries(cfg, csa, B.DSV4_TARGET_ENTRY, rr, idx, rn(nn, d))
        B.dsv4_cache_write_entries(cfg, csa, B.DSV4_TARGET_INDEX_KEY, rr, idx, rn(nn, dI))
    bf = lambda *s_: rn(*s_).to(torch.bfloat16)
    B.dsv4_state_write_tokens(cfg, csa, 0, P - 128, bf(128, d), bf(128, d), bf(128, dI), bf(128, dI))
    x = dict(kv=bf(C, d), gate=bf(C, d), kI=bf(C, dI), gI=bf(C, dI), q=bf(C, H, d), qI=bf(C, HI_, dI),
             w=rn(C, HI_) / 8.0)
    sinks = torch.from_numpy(synth.sinks(w)).to(dev)
    cu = torch.tensor([0, C], dtype=torch.int32, device=dev)
    p0 = torch.tensor([P], dtype=torch.int32, device=dev)
    lay = csa.layout
    winc = torch.empty((C + 128) * lay.record_bytes, dtype=torch.uint8, device=dev)
    ws = torch.empty(B.dsv4_workspace_bytes(cfg, C, nb * 32), dtype=torch.uint8, device=dev)
    topk = torch.empty((C, k), dtype=torch.int32, device=dev)
    out_c = torch.empty((C, H, d), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup
    stream = torch.cuda.current_stream()

    def step():
        B.dsv4_compress_kv_prefill(cfg, csa, x["kv"], x["gate"], x["kI"], x["gI"], cu, zero, p0, C, winc, stream)
        B.dsv4_index_topk_prefill(cfg, csa, x["qI"], x["w"], cu, zero, p0, C, topk, ws, stream)
        B.dsv4_csa_attend_prefill(cfg, csa, x["q"], cu, zero, p0, C, topk, winc, sinks, out_c, stream)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    for kid in range(B.DSV4_K_COUNT):
        B.dsv4_timer_enable(kid, True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kern = {}
    names = {B.DSV4_K_COMPRESS: "compress", B.DSV4_K_INDEX_SCORE: "index_score", B.DSV4_K_TOPK: "topk",
             B.DSV4_K_ATTEND: "attend"}
    for kid, nm in names.items():
        ms, n = B.dsv4_timer_read(kid, True)
        B.dsv4_timer_enable(kid, False)
        kern[nm] = dict(total_ms=ms, launches=n, avg_us=1e3 * ms / max(n, 1))
    # algorithmic work of the chunk: indexer flops over the visible keys of every
    # query, attention flops over its records (top-512 + window)
    n_vis = sum((P + i + 1) // 4 for i in range(C))
    idx_flops = n_vis * HI_ * dI * 2
    csa_recs = C * (min(k, n_csa) + 128)
    att_flops = csa_recs * H * 4 * d
    idx_ms = kern["index_score"]["total_ms"] / steps
    att_ms = kern["attend"]["total_ms"] / steps
    idx_tf = idx_flops / (idx_ms * 1e-3) / 1e12 if idx_ms > 0 else 0.0
    att_tf = att_flops / (att_ms * 1e-3) / 1e12 if att_ms > 0 else 0.0
    dom = "index_score" if kern["index_score"]["total_ms"] >= kern["attend"]["total_ms"] else "attend"
    roof = ({"kernel": "k_index_score_prefill", "bound": "mfma", "achieved": round(idx_tf, 2),
             "peak": idx_peak, "unit": "TFLOP/s", "frac": round(idx_tf / idx_peak, 4), "traffic": None}
            if dom == "index_score" else
            {"kernel": "k_attend", "bound": "mfma", "achieved": round(att_tf, 2), "peak": BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(att_tf / BF16_PEAK_TFLOPS, 4), "traffic": None})
    res = {
        "metric": "CSA prefill tokens/s (8192-token chunk on a 262144-token prefix)",
        "value": round(C / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4/fp8/bf16" if mx else "fp8/bf16", "data": "synthetic",
        "config": {"workload": f"V4 CSA layer prefill, chunk {C} on a {P // 1024}K prefix, top-{k}, "
                               f"{H} heads x d {d}" + (", MXFP4 indexer" if mx else ""), "chunk": C, "prefix": P,
                   "topk": k, "idx_store": a.idx_store},
        "roofline": roof,
        "breakdown_ms": {n_: round(v["total_ms"] / steps, 3) for n_, v in kern.items()},
        "indexer_TFLOPs": round(idx_tf, 1), "attend_TFLOPs": round(att_tf, 1),
        "setup_s": round(t_setup, 1),
    }
    print(json.dumps(res), flush=True)


def out_proj_main(a):
    """The grouped output projection of --batch tokens' attention outputs
    (V4-Pro: 128 heads x 512 dims, 16 groups, group rank 1024, model width
    7168), bf16 weights and activations generated on the device before
    timing.  Small batches stream the 369 MB of weights once (HBM-bound);
    large batches are MFMA-bound."""
    import torch
    from long_context_compressed_02_amd import binding as B

    dev = "cuda"
    torch.cuda.set_device(0)
    H, d, G, r, hidden = 128, 512, 16, 1024, 7168
    T = a.batch
    cfg = B.make_cfg()
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    rn = lambda *s_: torch.randn(*s_, generator=g, device=dev, dtype=torch.float32)
    gd = H // G * d
    o = rn(T, H, d).to(torch.bfloat16)
    w1 = (rn(G, r, gd) / gd ** 0.5).to(torch.bfloat16)
    w2 = (rn(hidden, G * r) / (G * r) ** 0.5).to(torch.bfloat16)
    y = torch.empty((T, G * r), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, hidden), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    w1p, w2p = torch.empty_like(w1), torch.empty_like(w2)
    B.dsv4_out_proj_pack(cfg, G, r, hidden, w1, w2, w1p, w2p, stream)     # once, before timing
    del w1, w2

    def step(_s):
        B.dsv4_out_proj(cfg, G, r, hidden, o, w1p, w2p, y, out, stream)

    ms, kern = _timed_steps(step, a.steps, a.warmup)
    flops = 2.0 * T * (G * r * gd + hidden * G * r)
    wbytes = 2.0 * (G * r * gd + hidden * G * r)
    abytes = 2.0 * T * (H * d + 2 * G * r + hidden)
    sec = ms * 1e-3
    small = T <= 256
    achieved = (wbytes + abytes) / sec / 1e9 if small else flops / sec / 1e12
    peak = HBM_PEAK_GBS if small else BF16_PEAK_TFLOPS
    roof = {"kernel": "k_gemm_nt", "bound": "hbm" if small else "mfma", "achieved": round(achieved, 2),
            "peak": peak, "unit": "GB/s" if small else "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None}
    res = {
        "metric": "grouped output projection tokens/s", "value": round(T / sec, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"grouped output projection of {T} tokens: {H} heads x {d} -> {G} groups of rank "
                               f"{r} -> {hidden}", "tokens": T, "heads": H, "d": d, "groups": G, "rank": r,
                   "hidden": hidden},
        "roofline": roof,
        "TFLOPs": round(flops / sec / 1e12, 1), "GBps": round((wbytes + abytes) / sec / 1e9, 1),
        "breakdown_us": {n_: round(v["avg_us"], 2) for n_, v in kern.items() if v["launches"]},
    }
    print(json.dumps(res), flush=True)


def index_q_main(a):
    """The indexer's query path of --batch tokens: x [T, 7168] bf16 -> d_c =
    1024 (bf16) -> 64 heads x 128 (bf16), both products on MXFP4 weights
    (quantised and packed once, before timing) with the activations quantised
    to MXFP8 on the way in.  Small batches stream the 7.8 MB of packed weights
    (HBM-bound); a prefill chunk is bound by the matrix cores."""
    import torch
    from long_context_compressed_02_amd import binding as B

    dev = "cuda"
    torch.cuda.set_device(0)
    hidden, dc, HI, dI = 7168, 1024, 64, 128
    T = a.batch
    cfg = B.make_cfg()                                         # bf16 activations
    g = torch.Generator(device=dev)
    g.manual_seed(78)
    rn = lambda *s_: torch.randn(*s_, generator=g, device=dev, dtype=torch.float32)
    x = rn(T, hidden).to(torch.bfloat16)
    wdq = (rn(dc, hidden) / hidden ** 0.5).to(torch.bfloat16)
    wuq = (rn(HI * dI, dc) / dc ** 0.5).to(torch.bfloat16)
    stream = torch.cuda.current_stream()
    wdq_p = torch.empty(B.dsv4_mx_pack_bytes(dc, hidden, False), dtype=torch.uint8, device=dev)
    wuq_p = torch.empty(B.dsv4_mx_pack_bytes(HI * dI, dc, False), dtype=torch.uint8, device=dev)
    B.dsv4_mx_pack_weight(wdq, wdq_p, stream)                  # once, before timing
    B.dsv4_mx_pack_weight(wuq, wuq_p, stream)
    del wdq, wuq
    ws = torch.empty(B.dsv4_index_q_proj_ws_bytes(cfg, T, hidden, dc), dtype=torch.uint8, device=dev)
    qI = torch.empty((T, HI, dI), dtype=torch.bfloat16, device=dev)

    def step(_s):
        B.dsv4_index_q_proj(cfg, x, dc, wdq_p, wuq_p, ws, qI, stream)

    ms, kern = _timed_steps(step, a.steps, a.warmup)
    flops = 2.0 * T * (dc * hidden + HI * dI * dc)
    # algorithmic bytes: packed weights once; x read; MXFP8 written and read
    # (1 + 1/32 bytes per value) and d_c written and read (bf16), for both
    # products; queries written
    wbytes = float(wdq_p.numel() + wuq_p.numel())
    abytes = T * (2.0 * hidden + 2 * (33 / 32) * (hidden + dc) + 2 * 2.0 * dc + 2.0 * HI * dI)
    sec = ms * 1e-3
    small = T <= 256
    achieved = (wbytes + abytes) / sec / 1e9 if small else flops / sec / 1e12
    peak = HBM_PEAK_GBS if small else FP8_PEAK_TFLOPS
    roof = {"kernel": "k_mx_gemm", "bound": "hbm" if small else "mfma", "achieved": round(achieved, 2),
            "peak": peak, "unit": "GB/s" if small else "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None}
    res = {
        "metric": "indexer query projection tokens/s", "value": round(T / sec, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8xfp4", "data": "synthetic",
        "config": {"workload": f"indexer query path of {T} tokens: {hidden} -> {dc} -> {HI} x {dI}, MXFP4 "
                               f"weights, MXFP8 activations", "tokens": T, "hidden": hidden, "dc": dc,
                   "idx_heads": HI, "idx_dim": dI},
        "roofline": roof,
        "TFLOPs": round(flops / sec / 1e12, 1), "GBps": round((wbytes + abytes) / sec / 1e9, 1),
        "breakdown_us": {n_: round(v["avg_us"], 2) for n_, v in kern.items() if v["launches"]},
    }
    print(json.dumps(res), flush=True)


def _timed_steps(step, steps, warm):
    """Warm up, time `steps` steps with events on the current stream, then run
    them again with the library's per-kernel timers on."""
    import torch
    from long_context_compressed_02_amd import binding as B
    for s in range(warm):
        step(s)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(warm, warm + steps):
        step(s)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    for kid in range(B.DSV4_K_COUNT):
        B.dsv4_timer_enable(kid, True)
    hold_stream(stream, 1.0e-3 * steps)
    for s in range(warm, warm + steps):
        step(s)
    torch.cuda.synchronize()
    names = {B.DSV4_K_COMPRESS: "compress", B.DSV4_K_INDEX_SCORE: "index_score", B.DSV4_K_TOPK: "topk",
             B.DSV4_K_ATTEND: "attend", B.DSV4_K_PROJ: "out_proj", B.DSV4_K_MX: "mx_linear"}
    kern = {}
    for kid, nm in names.items():
        ms, n = B.dsv4_timer_read(kid, True)
        B.dsv4_timer_enable(kid, False)
        kern[nm] = dict(total_ms=ms, launches=n, avg_us=1e3 * ms / max(n, 1))
    return ms_step, kern


def decode_mix_main(a):
    """Decode steps of the other two decode workloads.  hca_decode: an HCA layer,
    16 requests at 65536 tokens (512 entries each); a step = append/compress +
    dense attention.  pair_1m: a CSA+HCA layer pair for 4 requests at
    1048576 / 524288 / 65536 / 4096 tokens; a step = the whole decode path of
    both layers.  Entries, keys and window tokens are N(0,1) values generated on
    the device; every step appends the next token of every request."""
    import torch
    from long_context_compressed_02_amd import binding as B
    from long_context_compressed_02_amd import synth

    dev = "cuda"
    torch.cuda.set_device(0)
    pair = a.workload == "pair_1m"
    w = synth.PAIR_DECODE_1M if pair else synth.HCA_DECODE_64K
    ctxs = list(w.ctx)
    Bsz = len(ctxs)
    steps, warm = a.steps, a.warmup
    total_new = steps + warm
    cfg = B.make_cfg(**w.shape())
    policy = {"auto": B.DSV4_POLICY_AUTO, "hi": B.DSV4_POLICY_HI, "lo": B.DSV4_POLICY_LO}[a.policy]
    H, d, HI_, dI, k = w.n_heads, w.d, w.idx_heads, w.idx_dim, w.topk
    need = [(c + total_new + 127) // 128 for c in ctxs]
    mb = max(need)
    perm = synth.permutation(w.wid, sum(need))
    bt_h = np.full((Bsz, mb), -1, dtype=np.int32)
    o = 0
    for r, nb in enumerate(need):
        bt_h[r, :nb] = perm[o:o + nb]
        o += nb
    bt = torch.from_numpy(bt_h).to(dev)
    csa = B.LayerCache(cfg, B.DSV4_CSA, Bsz, mb, sum(need), bt) if pair else None
    hca = B.LayerCache(cfg, B.DSV4_HCA, Bsz, mb, sum(need), bt)
    g = torch.Generator(device=dev)
    g.manual_seed(5678)
    rn = lambda *s_: torch.randn(*s_, generator=g, device=dev, dtype=torch.float32)
    bf = lambda *s_: rn(*s_).to(torch.bfloat16)
    t_setup = time.time()

    def fill(cache, target, r, n, dim):
        for a0 in range(0, n, 1 << 15):
            nn = min(1 << 15, n - a0)
            B.dsv4_cache_write_entries(cfg, cache, target, torch.full((nn,), r, dtype=torch.int32, device=dev),
                                       torch.arange(a0, a0 + nn, dtype=torch.int32, device=dev), rn(nn, dim))
    for r, c in enumerate(ctxs):
        if pair:
            fill(csa, B.DSV4_TARGET_ENTRY, r, c // 4, d)
            fill(csa, B.DSV4_TARGET_INDEX_KEY, r, c // 4, dI)
            B.dsv4_state_write_tokens(cfg, csa, r, c - 128, bf(128, d), bf(128, d), bf(128, dI), bf(128, dI))
        fill(hca, B.DSV4_TARGET_ENTRY, r, c // 128, d)
        B.dsv4_state_write_tokens(cfg, hca, r, c - 128, bf(128, d), bf(128, d))
    steps_in = []
    for s in range(total_new):
        steps_in.append(dict(
            kv=bf(Bsz, d), gate=bf(Bsz, d), kI=bf(Bsz, dI), gI=bf(Bsz, dI), kvh=bf(Bsz, d), gateh=bf(Bsz, d),
            q=bf(Bsz, H, d), qh=bf(Bsz, H, d), qI=bf(Bsz, HI_, dI), w=rn(Bsz, HI_) / 8.0,
            pos=torch.tensor([c + s for c in ctxs], dtype=torch.int32, device=dev)))
    req = torch.arange(Bsz, dtype=torch.int32, device=dev)
    sinks = torch.from_numpy(synth.sinks(w)).to(dev)
    ws = torch.empty(B.dsv4_workspace_bytes(cfg, Bsz, mb * 32), dtype=torch.uint8, device=dev) if pair else None
    topk = torch.empty((Bsz, k), dtype=torch.int32, device=dev)
    out_c = torch.empty((Bsz, H, d), dtype=torch.bfloat16, device=dev)
    out_h = torch.empty((Bsz, H, d), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup
    stream = torch.cuda.current_stream()

    def step(s):
        x = steps_in[s]
        if pair:
            B.dsv4_compress_kv_decode(cfg, csa, x["kv"], x["gate"], x["kI"], x["gI"], req, x["pos"], stream)
            B.dsv4_index_topk_decode(cfg, csa, x["qI"], x["w"], req, x["pos"], topk, ws, stream)
            B.dsv4_csa_attend_decode(cfg, csa, x["q"], req, x["pos"], topk, sinks, out_c, policy, stream)
        B.dsv4_compress_kv_decode(cfg, hca, x["kvh"], x["gateh"], None, None, req, x["pos"], stream)
        B.dsv4_hca_attend_decode(cfg, hca, x["qh"], req, x["pos"], sinks, out_h, policy, stream)

    ms_step, kern = _timed_steps(step, steps, warm)
    # algorithmic work per step at the timed positions (averaged over the steps)
    ts = [[c + s for c in ctxs] for s in range(warm, total_new)]
    n_vis = np.mean([sum((t + 1) // 4 for t in row) for row in ts]) if pair else 0.0
    n_h = np.mean([sum((t + 1) // 128 for t in row) for row in ts])
    csa_recs = sum(min(k, (t + 1) // 4) + 128 for t in ts[0]) if pair else 0
    hca_recs = n_h + 128 * Bsz
    rec_b = (d - 64) + 2 * 64 + 4
    att_flops = (csa_recs + hca_recs) * H * 4 * d
    att_bytes = (csa_recs + hca_recs) * rec_b + (2 if pair else 1) * 2 * Bsz * H * d * 2
    score_bytes = n_vis * (dI + 4 + 4)
    att_s = kern["attend"]["total_ms"] / steps * 1e-3
    att_tf = att_flops / att_s / 1e12
    att_gbs = att_bytes / att_s / 1e9
    dom = "attend" if (not pair or kern["attend"]["total_ms"] >= kern["index_score"]["total_ms"]) else "index_score"
    if dom == "attend":
        kn_h = lo_kernel(d, mb + 128)
        kn = (lo_kernel(d, k + 128) + " (CSA), " + kn_h + " (HCA)") if pair else kn_h
        roof = {"kernel": kn, "bound": "mfma", "achieved": round(att_tf, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(att_tf / BF16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        sc_gbs = score_bytes / (kern["index_score"]["total_ms"] / steps * 1e-3) / 1e9
        roof = {"kernel": "k_index_score_decode", "bound": "hbm", "achieved": round(sc_gbs, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(sc_gbs / HBM_PEAK_GBS, 4), "traffic": None}
    name = ("CSA/HCA decode queries/s (4 requests at 1M/512K/64K/4K context)" if pair else
            "HCA decode queries/s (16 requests at 64K context)")
    res = {
        "metric": name, "value": round(Bsz / (ms_step * 1e-3), 1), "unit": "queries/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8/bf16", "data": "synthetic",
        "config": {"workload": ("V4 CSA+HCA layer-pair decode, contexts " + "/".join(f"{c // 1024}K" for c in ctxs)
                                if pair else f"V4 HCA layer decode, batch {Bsz} x {ctxs[0] // 1024}K"),
                   "batch": Bsz, "ctx": ctxs, "topk": k if pair else None, "heads": H, "d": d, "policy": a.policy},
        "roofline": roof,
        "breakdown_us": {n_: round(v["avg_us"], 2) for n_, v in kern.items() if v["launches"]},
        "launches_per_step": {n_: v["launches"] / steps for n_, v in kern.items() if v["launches"]},
        "attend_TFLOPs": round(att_tf, 1), "attend_GBps": round(att_gbs, 1),
        "setup_s": round(t_setup, 1),
    }
    print(json.dumps(res), flush=True)


HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "long_context_compressed_02_amd", "csrc")
# per kernel: the committed traffic summary of the headline workload and the
# source whose SHA-256 it records
TRAFFIC = {
    "attend": (os.path.join(HERE, "profiles", "k_attend_decode_128k_b32_hbm_traffic.txt"),
               os.path.join(CSRC, "k_attend.hip"), "k_attend_src_sha256"),
    "index_score": (os.path.join(HERE, "profiles", "k_index_score_decode_128k_b32_hbm_traffic.txt"),
                    os.path.join(CSRC, "k_index.hip"), "k_index_src_sha256"),
}


LO8_MAX_LIST = 2048   # records: the eight-wave LO attention kernel takes lists up to this length (d = 512)


def lo_kernel(d, list_max):
    """Name of the LO attention kernel the library launches for this shape."""
    return "k_attend_lo8" if d == 512 and list_max <= LO8_MAX_LIST else "k_attend_lo"


_SPIN_PER_MS = None


def hold_stream(stream, ms):
    """Queue a spin kernel of about `ms` milliseconds on `stream` (torch's
    bounded clock-wait kernel), so that the launches issued after it are all
    queued before the GPU reaches them: per-launch HIP-event timers then see
    back-to-back kernels, not the host's launch gaps."""
    import torch
    global _SPIN_PER_MS
    with torch.cuda.stream(stream):
        if _SPIN_PER_MS is None:
            n = 1 << 20
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(n)
            a.record()
            torch.cuda._sleep(n)
            b.record()
            b.synchronize()
            _SPIN_PER_MS = n / max(a.elapsed_time(b), 1e-3)
        torch.cuda._sleep(int(min(ms, 200.0) * _SPIN_PER_MS))


def measured_traffic(kernel):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated on a plain
    copy) from the committed rocprofv3 summary of this workload -- only if the
    summary was taken on the kernel's source as it is now."""
    summary, source, key = TRAFFIC[kernel]
    try:
        text = open(summary).read()
        src = open(source, "rb").read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    h = re.search(key + r": ([0-9a-f]+)", text)
    if not m or not h or hashlib.sha256(src).hexdigest() != h.group(1):
        return None
    return int(m.group(1))


_calib = None


def calib_lib():
    global _calib
    if _calib is None:
        path = os.path.join(HERE, "long_context_compressed_02_amd", "libdsv4calib.so")
        L = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.dsv4calib_copy_gbs.argtypes = [vp, vp, i64, i32]
        L.dsv4calib_read_gbs.argtypes = [vp, i64, vp, i32]
        L.dsv4calib_mfma_tflops.argtypes = [i32, i32, i32, vp, i32]
        for f in (L.dsv4calib_copy_gbs, L.dsv4calib_read_gbs, L.dsv4calib_mfma_tflops):
            f.restype = ctypes.c_double
        _calib = L
    return _calib


def calibrate():
    """The device's own rates: a 1 GiB copy and a 1 GiB read (best of 5), and
    back-to-back matrix instructions from every SIMD (bf16 16x16x32, fp8 and
    fp4 16x16x128, bf16 32x32x16, fp8 32x32x64; 2048 workgroups of 4 waves,
    8 independent accumulators per wave; best of 3).  The measured bf16
    peak a kernel is priced against is the faster bf16 shape."""
    import torch
    L = calib_lib()
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    copy = L.dsv4calib_copy_gbs(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n, 5)
    read = L.dsv4calib_read_gbs(ctypes.c_void_p(src.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()), 5)
    del src, dst
    blocks = 2048                                  # 8 waves per SIMD: enough to keep the matrix pipes full
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    tf = [L.dsv4calib_mfma_tflops(kd, blocks, 256, ctypes.c_void_p(out.data_ptr()), 3) for kd in (0, 1, 2, 3, 4)]
    torch.cuda.synchronize()
    return {"copy_GBps": round(copy, 1), "read_GBps": round(read, 1), "bf16_TFLOPs": round(tf[0], 1),
            "fp8_TFLOPs": round(tf[1], 1), "fp4_TFLOPs": round(tf[2], 1), "bf16_32x32_TFLOPs": round(tf[3], 1),
            "fp8_32x32_TFLOPs": round(tf[4], 1),
            "spec": {"hbm_GBps": HBM_PEAK_GBS, "bf16_TFLOPs": BF16_PEAK_TFLOPS, "fp8_TFLOPs": FP8_PEAK_TFLOPS,
                     "fp4_TFLOPs": FP4_PEAK_TFLOPS}}


def cpu_baseline(w, nreq, t, idx_mode=1, budget_s=12.0, max_queries=2000):
    """The oracle (as it stands) on a bounded sample of the same workload:
    nreq requests' caches (prepared once, untimed), then CSA+HCA queries at
    position t -- index keys, top-k and attention, each query with its own
    query vectors over one of those caches in turn -- timed until about
    budget_s seconds of oracle work."""
    from long_context_compressed_02_amd import synth
    from oracle import oracle as O
    oc = O.OCfg(idx_mode=idx_mode, **w.shape())
    n = (t + 1) // 4
    nh = (t + 1) // 128
    sinks = synth.sinks(w)
    prep = []
    for r in range(nreq):
        prep.append(dict(keys=O.store_index_rows(synth.index_keys(w, r, n), oc), ent_raw=synth.entries(w, r, n, 0),
                         hents=O.entries_from_values("hca", synth.entries(w, r, nh, 1), range(nh), oc),
                         win=synth.window_tokens(w, r, 128, 0)[0], winh=synth.window_tokens(w, r, 128, 1)[0]))
    el, done = 0.0, 0
    while el < budget_s and done < max_queries:
        q, qI, wt = synth.decode_queries(w, 1, sub=10000 + done)
        qh, _, _ = synth.decode_queries(w, 1, sub=20000 + done)
        p = prep[done % nreq]
        t0 = time.time()
        idx, _ = O.csa_select(t, qI[0], wt[0].astype(np.float64), p["keys"], oc)
        sel = [int(j) for j in idx if j >= 0]
        ents = O.entries_from_values("csa", p["ent_raw"][sel], sel, oc)
        win = O.window_records(p["win"], np.arange(t - 127, t + 1), oc)
        O.attend(O.query_rot(q[0], t, oc), sinks, np.concatenate([ents, win]), oc.tau)
        winh = O.window_records(p["winh"], np.arange(t - 127, t + 1), oc)
        O.attend(O.query_rot(qh[0], t, oc), sinks, np.concatenate([p["hents"], winh]), oc.tau)
        el += time.time() - t0
        done += 1
    return {"value": round(done / el, 3), "unit": "queries/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{done} queries over {nreq} requests' caches of the same workload (per query: CSA indexer "
                      f"over {n} keys + top-{oc.topk} + sparse MQA, and HCA MQA over {nh}+128 records), fp64, "
                      f"{el:.1f} s of oracle time (the caches' storage quantisation done once, untimed)"}


if __name__ == "__main__":
    main()
