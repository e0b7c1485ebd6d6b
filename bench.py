#!/usr/bin/env python3
"""Throughput of the Medusa verify step on one MI355X.

A step is one pass of the whole hot path over one batch: the K Medusa heads
with top-s (W1 stage; W2 stream with a fused per-workgroup top-s; merge of
those lists), one tree attention pass over the KV prefix and the tree, and
tree acceptance.  Inputs are seeded synthetic tensors resident in HBM before
timing starts.

Prints one JSON line.  Per-call durations come from HIP events recorded on
the stream the library launches on (torch's current stream).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from medusa_tree_verification_amd import workloads as W  # noqa: E402

METRIC = "tree-verify steps/s (heads+tree-attn+accept); achieved HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, published
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_vocab_typical", choices=W.WORKLOAD_ORDER,
                    help="default: the largest workload (K=5 heads, V=128256, batch 8, "
                         "256-node tree, typical acceptance)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="wall-clock budget of the oracle timing")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="MiB read before each step of the per-call breakdown pass, outside "
                         "its events (more than the last-level cache and the L2s; 0: none)")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of whole steps run before the measured passes (unreported)")
    ap.add_argument("--forward-blocks", type=int, default=4,
                    help="attention blocks of the synthetic verify forward (a next-row timing)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def algorithmic_bytes(wl, prefix_len, n_internal):
    """Bytes each call must move at least once (inputs read + outputs written)."""
    w = 2 if wl.dtype == W.BF16 else 4
    B, K, d, V, s, T = wl.B, wl.K, wl.d, wl.V, wl.s, wl.T
    stage1 = K * d * d * w + B * d * w + B * K * d * w              # W1, h in; z out
    stage2 = K * V * d * w + B * K * d * w                          # W2, z in (stream kernel)
    merge = B * K * s * 8                                           # ids + vals out
    Ltot = int(np.minimum(prefix_len, wl.Lcap).sum())
    attn = (2 * wl.Hkv * Ltot * wl.dh * w + 2 * B * wl.Hkv * T * wl.dh * w
            + 2 * B * wl.Hq * T * wl.dh * w)                         # KV prefix + tree KV + q in, out
    accept = B * (n_internal + 1) * V * w                            # internal rows + best row
    return {"heads_stage1": stage1, "heads_stage2": stage2, "heads_merge": merge,
            "tree_attention": attn, "tree_accept": accept}


def attention_flops(wl, prefix_len, tree):
    depth = np.array([len(p) for p in tree.paths])
    Ltot = int(np.minimum(prefix_len, wl.Lcap).sum())
    return 4 * wl.dh * wl.Hq * (wl.T * Ltot + wl.B * int((depth + 1).sum()))


def src_digest():
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "medusa_tree_verification_amd", "csrc", "heads.hip"), "rb") as f:
        h.update(f.read())
    with open(os.path.join(ROOT, "medusa_tree_verification_amd", "csrc", "common.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    digest = src_digest()
    for line in open(TRAFFIC_FILE):
        parts = line.split()
        if len(parts) >= 4 and not line.startswith("#") and parts[0] == workload \
                and parts[1] == "heads_stage2" and parts[2] == digest:
            return int(float(parts[3]))
    return None


def calibrate_copy(mib, reps):
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "reps": reps}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (the verify step "
              "would shard by sequence, kv head or vocabulary). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib, args.steps)
        return
    from medusa_tree_verification_amd import binding as mv

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    tree = W.workload_tree(wl)

    def dv(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    t0 = time.time()
    hx = W.heads_inputs(wl)
    ax = W.attention_inputs(wl)
    hidden, w1, w2 = dv(hx["hidden"]), dv(hx["w1"]), dv(hx["w2"])
    q, kc, vc, kt, vt = (dv(ax[k]) for k in ("q", "k_cache", "v_cache", "k_tree", "v_tree"))
    plen = dv(ax["prefix_len"])
    B, K, d, V, s, T = wl.B, wl.K, wl.d, wl.V, wl.s, wl.T
    dt = mv.BF16 if wl.dtype == W.BF16 else mv.F32
    mode = mv.GREEDY if wl.mode == "greedy" else mv.TYPICAL

    ws_h = mv.workspace(mv.lib.medusa_heads_topk_workspace_bytes(B, K, d, V, s, dt), dev)
    ws_a = mv.workspace(mv.lib.tree_attention_workspace_bytes(B, wl.Hq, wl.Hkv, wl.Lcap, wl.dh, T,
                                                              dt), dev)
    ws_c = mv.workspace(mv.lib.tree_accept_workspace_bytes(B, T, V, K, s), dev)
    ids = torch.empty((B, K, s), dtype=torch.int32, device=dev)
    vals = torch.empty((B, K, s), dtype=torch.float32, device=dev)
    attn_out = torch.empty_like(q)
    i32 = dict(dtype=torch.int32, device=dev)
    acc = {"accept_len": torch.empty(B, **i32), "best_node": torch.empty(B, **i32),
           "accepted_tokens": torch.empty((B, K), **i32), "node_tokens": torch.empty((B, T), **i32),
           "next_token": torch.empty(B, **i32)}

    # LM-head weights for the root-token variant of the heads (a next-row
    # measurement): random, N(0, 0.02), in the workload's dtype
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 * wl.cid + 14)
    w_lm = (torch.randn((V, d), generator=gen, device=dev) * 0.02).to(w2.dtype)

    # uniforms for the sampled bonus token (a next-row measurement)
    uni = torch.from_numpy(np.random.default_rng(1000 * wl.cid + 13).random(B)
                           .astype(np.float32)).to(dev)
    samp = torch.empty(B, dtype=torch.int32, device=dev)

    # verification logits: planted on the candidates the heads actually propose
    mv.medusa_heads_stage1(hidden, w1, B, K, d, V, s, ws_h)
    mv.medusa_heads_stage2(w2, B, K, d, V, s, ids, ws_h, topk_vals=vals)
    torch.cuda.synchronize()
    cand = ids.cpu().numpy()
    vlog_np = W.verify_logits(wl, tree, W.path_tokens(tree, cand))
    vlog = dv(vlog_np)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        mv.medusa_heads_stage1(hidden, w1, B, K, d, V, s, ws_h)
        if ev is not None:
            ev[1].record()
        if ev is None:
            mv.medusa_heads_stage2(w2, B, K, d, V, s, ids, ws_h, topk_vals=vals)
        else:
            # the same two kernels as two calls, so that the weight stream is
            # timed alone
            mv.medusa_heads_stage2_stream(w2, B, K, d, V, s, ws_h)
            ev[2].record()
            mv.medusa_heads_stage2_merge(B, K, d, V, s, dt, ids, ws_h, topk_vals=vals)
            ev[3].record()
        mv.tree_attention(q, kc, vc, plen, kt, vt, tree.parent, wl.scale, ws=ws_a, out=attn_out)
        if ev is not None:
            ev[4].record()
        mv.tree_accept(vlog, ids, tree.parent, mode, wl.temperature, wl.eps, wl.delta, ws=ws_c,
                       out=acc)
        if ev is not None:
            ev[5].record()

    # Settle: whole steps for a fixed span of GPU time before any measured
    # pass.  Right after an idle spell (here: the input set-up on the host)
    # the attention's first few dozen calls run 7-17% slower while the
    # chip's clock settles; the passes below then measure the steady state
    # of a serving loop.  Nothing of this span is reported.
    settle_steps = 0
    t_settle = time.time()
    while time.time() - t_settle < args.settle_s:
        for _ in range(8):
            step()
        settle_steps += 8
        torch.cuda.synchronize()

    # The per-call breakdown: a pass of the same steps with an event between
    # calls (each event costs a little time of its own), every step starting
    # with cold caches (a buffer larger than the last-level cache is read, a
    # sum, before the step's first event; a read leaves no dirty lines, while
    # after a written flush their write-back ran into the step's first
    # kernels).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    flush = torch.ones(args.flush_mib << 17, dtype=torch.int64, device=dev) if args.flush_mib > 0 else None
    sink = torch.zeros((), dtype=torch.int64, device=dev)
    for i in range(args.steps):
        if flush is not None:
            torch.sum(flush, dim=0, out=sink)
        step(evs[i])
    torch.cuda.synchronize()
    del flush, sink

    # W untimed warm-up steps, then the K timed steps back to back with
    # nothing else on the stream
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    names = ["heads_stage1", "heads_stage2", "heads_merge", "tree_attention", "tree_accept"]
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in
           enumerate(names)}

    n_internal = len(set(int(x) for x in tree.parent[1:]))
    nbytes = algorithmic_bytes(wl, ax["prefix_len"], n_internal)
    flops = attention_flops(wl, ax["prefix_len"], tree)
    stages = {n: {"us": round(per[n] * 1e3, 2), "bytes": int(nbytes[n]),
                  "GBps": round(nbytes[n] / (per[n] * 1e-3) / 1e9, 1)} for n in names}
    stages["tree_attention"]["TFLOPs"] = round(flops / (per["tree_attention"] * 1e-3) / 1e12, 1)
    step_bytes = sum(nbytes.values())
    # roofline time of every stage (HBM at the published peak; the tree
    # attention at max(HBM, bf16 MFMA peak) since long prefixes are
    # MFMA-bound) and each stage's and the step's fraction of it
    roof_us = {n: nbytes[n] / (PEAK_HBM_GBS * 1e9) * 1e6 for n in names}
    roof_us["tree_attention"] = max(roof_us["tree_attention"], flops / (PEAK_MFMA_TFLOPS * 1e12) * 1e6)
    for n in names:
        stages[n]["roofline_frac"] = round(roof_us[n] / (per[n] * 1e3), 4)
    stages["tree_attention"]["bound"] = ("mfma" if flops / (PEAK_MFMA_TFLOPS * 1e12) >
                                         nbytes["tree_attention"] / (PEAK_HBM_GBS * 1e9) else "hbm")
    step_us = np.array([e[0].elapsed_time(e[5]) for e in evs]) * 1e3

    dom = "heads_stage2"
    achieved = nbytes[dom] / (per[dom] * 1e-3) / 1e9
    traffic = measured_traffic(wl.name)
    attn_bound = stages["tree_attention"]["bound"]
    attn_tf = flops / (per["tree_attention"] * 1e-3) / 1e12
    attn_gbs = nbytes["tree_attention"] / (per["tree_attention"] * 1e-3) / 1e9
    # the library's choice: the pipelined kernel for bf16, dh = 128 and at
    # least five 32-row waves per m-tile (G * T query rows per kv head)
    row_waves = min((wl.Hq // wl.Hkv * T + 31) // 32, 8)
    attn_main = ("tree_attn_pipe_kernel" if wl.dtype == W.BF16 and wl.dh == 128 and row_waves > 4
                 else "tree_attn_fwd_kernel")
    attn_kernel = (attn_main + " (+ tree_attn_combine_kernel when the prefix is split): "
                   "the tree_attention call")
    result = {
        "metric": METRIC,
        "value": round(1e3 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == W.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "heads": K, "hidden": d, "vocab": V,
                   "top_s": s, "tree_nodes": T, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
                   "head_dim": wl.dh, "prefix_len": [int(ax["prefix_len"].min()),
                                                     int(ax["prefix_len"].max())],
                   "acceptance": wl.mode, "parallelism": "single GPU"},
        "step_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_roofline_frac": round(sum(roof_us.values()) / (ms_per_step * 1e3), 4),
        "step_us_p50_p90": [round(float(np.percentile(step_us, 50)), 2),
                            round(float(np.percentile(step_us, 90)), 2)],
        "roofline": {"kernel": "heads_stage2_kernel (medusa_heads_stage2_stream: W2 stream + fused per-workgroup top-s)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic},
        "roofline_tree_attention": (
            {"kernel": attn_kernel, "bound": "mfma",
             "achieved": round(attn_tf, 1), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
             "frac": round(attn_tf / PEAK_MFMA_TFLOPS, 4), "hbm_GBps": round(attn_gbs, 1),
             "flops": int(flops)} if attn_bound == "mfma" else
            {"kernel": attn_kernel, "bound": "hbm",
             "achieved": round(attn_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(attn_gbs / PEAK_HBM_GBS, 4), "TFLOPs": round(attn_tf, 1),
             "bytes": int(nbytes["tree_attention"])}),
        "stages": stages,
    }

    peaks = measure_peaks(mv, dev)
    result["measured_peaks"] = peaks
    result["roofline"]["frac_of_measured"] = round(achieved / peaks["hbm_read_GBps"], 4)
    rt = result["roofline_tree_attention"]
    rt["frac_of_measured"] = round(rt["achieved"] / (peaks["mfma_bf16_TFLOPs"] if rt["bound"] == "mfma"
                                                     else peaks["hbm_read_GBps"]), 4)
    result["next_rows"] = {
        "kv_commit": measure_commit(mv, wl, tree, kc, vc, kt, vt, plen, acc["best_node"],
                                    args.steps),
        "accept_typical_loglik": time_call(
            lambda: mv.tree_accept(vlog, ids, tree.parent, mv.TYPICAL_LOGLIK,
                                   wl.temperature if wl.mode != "greedy" else 1.0, wl.eps,
                                   wl.delta, ws=ws_c, out=acc), args.steps,
            nbytes["tree_accept"]),
        "heads_with_root": time_call(
            lambda: mv.medusa_heads_topk_root(hidden, w1, w2, w_lm, s, ws=ws_h), args.steps,
            nbytes["heads_stage1"] + nbytes["heads_stage2"] + V * d * w_lm.element_size()),
        "sample_token": time_call(
            lambda: mv.medusa_sample_token(vlog, acc["best_node"], uni,
                                           wl.temperature if wl.mode != "greedy" else 1.0,
                                           token=samp), args.steps,
            B * V * (2 if wl.dtype == W.BF16 else 4)),          # the best rows, read once
        "verify_forward": measure_forward(mv, wl, tree, plen, ax["prefix_len"], args.steps,
                                          args.forward_blocks),
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, hx, ax, tree, cand, vlog_np, args.cpu_seconds)
    result["setup_s"] = round(setup_s, 1)
    print(json.dumps(result), flush=True)


def measure_peaks(mv, dev, read_mib=2048, reps=10):
    """The two ceilings measured on this device with the library's probes: a
    linear 16-byte-load read of read_mib MiB (more than the last-level
    cache) and independent bf16 32x32x16 MFMA chains on every CU."""
    import torch
    sink = torch.empty(mv.lib.medusa_probe_sink_bytes() // 4, dtype=torch.int32, device=dev)
    buf = torch.ones(read_mib << 18, dtype=torch.int32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(3):
        mv.probe_read(buf, sink)
    ev[0].record()
    for _ in range(reps):
        mv.probe_read(buf, sink)
    ev[1].record()
    torch.cuda.synchronize()
    read_gbs = buf.numel() * 4 * reps / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
    # the same stream with per-workgroup clock stamps: workgroup w reads its
    # share on XCD w mod 8, so the ends show each XCD's streaming time
    # (pattern 0: linear; 1: 8-row tiles of 8 KiB rows, the heads' W2 pattern)
    nwg = mv.lib.medusa_probe_read_workgroups()
    mhz = mv.lib.medusa_probe_clock_mhz()
    by_xcd = {}
    for pattern, name in ((0, "linear"), (1, "rows8")):
        stamps = torch.zeros(2 * nwg, dtype=torch.int32, device=dev)
        mv.probe_read_timed(buf, sink, stamps, pattern)
        mv.probe_read_timed(buf, sink, stamps, pattern)
        torch.cuda.synchronize()
        st = stamps.cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        if mhz > 0:
            t0 = st[0::2].min()
            ends = ((st[1::2] - t0) % (1 << 32)) / mhz
            by_xcd[name] = [round(float(np.median(ends[x::8])), 1) for x in range(8)]
    del buf
    iters = 16384
    mv.probe_mfma(iters, sink)
    ev[0].record()
    flops = 0.0
    for _ in range(reps):
        flops += mv.probe_mfma(iters, sink)
    ev[1].record()
    torch.cuda.synchronize()
    tflops = flops / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e12
    return {"hbm_read_GBps": round(read_gbs, 1), "mfma_bf16_TFLOPs": round(tflops, 1),
            "read_us_by_xcd": by_xcd or None,
            "method": f"medusa_probe_read over {read_mib} MiB x {reps}; medusa_probe_mfma "
                      f"{iters} iterations x {reps} (events on the launch stream); read_us_by_xcd: "
                      f"the second of two medusa_probe_read_timed passes per pattern (linear; "
                      f"8-row tiles of 8 KiB rows), the median end per XCD (workgroup w on XCD "
                      f"w mod 8, an equal share each), microseconds from the first start"}


def time_call(fn, steps, nbytes):
    """Mean time of one call, each bracketed by events (after 3 untimed calls)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for _ in range(3):
        fn()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    return {"us": round(us, 2), "bytes": int(nbytes), "GBps": round(nbytes / (us * 1e-6) / 1e9, 2)}


def measure_commit(mv, wl, tree, kc, vc, kt, vt, plen, best_node, steps):
    """The accepted-path KV commit (the step after acceptance) on its own: the
    caches get T rows of spare capacity, the lengths are reset before every
    call (outside the timed interval) and each call is bracketed by events."""
    import torch
    B, Hkv, Lcap, dh = kc.shape
    kc2 = torch.zeros((B, Hkv, Lcap + wl.T, dh), dtype=kc.dtype, device=kc.device)
    vc2 = torch.zeros_like(kc2)
    kc2[:, :, :Lcap].copy_(kc)
    vc2[:, :, :Lcap].copy_(vc)
    lens = plen.clone()
    com = torch.empty(B, dtype=torch.int32, device=kc.device)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps + 3):
        lens.copy_(plen)
        e = ev[i - 3] if i >= 3 else None
        if e:
            e[0].record()
        mv.tree_commit_kv(kc2, vc2, lens, kt, vt, best_node, tree.parent, committed=com)
        if e:
            e[1].record()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    rows = int(com.sum().item())
    w = kc.element_size()
    nbytes = 2 * 2 * Hkv * rows * dh * w          # K and V rows: read from the tree, written to the cache
    return {"us": round(us, 2), "rows": rows, "bytes": nbytes,
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 2)}


def measure_forward(mv, wl, tree, plen, plen_np, steps, N):
    """The multi-block synthetic verify forward (logits of every tree node
    from N attention blocks + the LM head) on its own.  Random-init weights
    and caches of the workload's shape, generated on the device, every block
    with its own weights and caches (nothing is re-read from a cache that a
    previous block warmed).  Bytes: weights, the cached prefix keys/values
    of every block, and the logits written once."""
    import torch
    dev = plen.device
    dt = torch.bfloat16 if wl.dtype == W.BF16 else torch.float32
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 * wl.cid + 17)
    B, T, d, V, Hq, Hkv, dh = wl.B, wl.T, wl.d, wl.V, wl.Hq, wl.Hkv, wl.dh

    def rnd(shape, std, mean=0.0):
        return (torch.randn(shape, generator=gen, device=dev) * std + mean).to(dt)

    layers = [{"g": rnd((d,), 0.1, 1.0), "wq": rnd((Hq * dh, d), d ** -0.5),
               "wk": rnd((Hkv * dh, d), d ** -0.5), "wv": rnd((Hkv * dh, d), d ** -0.5),
               "wo": rnd((d, Hq * dh), (Hq * dh) ** -0.5)} for _ in range(N)]
    kcs = [rnd((B, Hkv, wl.Lcap, dh), 1.0) for _ in range(N)]
    vcs = [rnd((B, Hkv, wl.Lcap, dh), 1.0) for _ in range(N)]
    h0, g_final, w_lm = rnd((B, T, d), 1.0), rnd((d,), 0.1, 1.0), rnd((V, d), 0.02)
    ws = mv.workspace(mv.lib.medusa_verify_forward_workspace_bytes(B, T, d, Hq, Hkv, dh, wl.Lcap,
                                                                   V, mv.BF16 if dt == torch.bfloat16
                                                                   else mv.F32), dev)
    out = {"logits": torch.empty((B, T, V), dtype=torch.float32, device=dev)}
    w = 2 if dt == torch.bfloat16 else 4
    Ltot = int(np.minimum(plen_np, wl.Lcap).sum())
    nbytes = (N * ((2 * Hq + 2 * Hkv) * dh * d * w + 2 * Hkv * Ltot * dh * w)
              + V * d * w + B * T * V * 4)
    r = time_call(lambda: mv.medusa_verify_forward(h0, layers, g_final, w_lm, kcs, vcs, plen,
                                                   tree.parent, Hq, Hkv, dh, ws=ws, out=out),
                  steps, nbytes)
    r["blocks"] = N
    del layers, kcs, vcs
    return r


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, hx, ax, tree, cand, vlog_np, budget_s):
    """The oracle, as it stands, on the host cores: the time of one verify
    step of the same workload (same input bytes).  Heads and acceptance run
    whole; the tree attention runs on an evenly spaced sample of its output
    rows sized to the time budget, and its time is scaled to all rows."""
    import oracle
    t0 = time.perf_counter()
    oracle.heads_topk(hx["hidden"], hx["w1"], hx["w2"], wl.s, wl.dtype)
    t_heads = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.tree_accept(vlog_np, cand, tree.parent, wl.dtype, wl.mode, wl.temperature)
    t_acc = time.perf_counter() - t0
    nrows = wl.B * wl.Hq * wl.T
    allrows = np.stack(np.meshgrid(np.arange(wl.B), np.arange(wl.Hq), np.arange(wl.T),
                                   indexing="ij"), axis=-1).reshape(-1, 3).astype(np.int32)

    def attn(rows):
        t = time.perf_counter()
        oracle.tree_attention(ax["q"], ax["k_cache"], ax["v_cache"], ax["prefix_len"],
                              ax["k_tree"], ax["v_tree"], tree.parent, wl.scale, wl.dtype,
                              rows=rows)
        return time.perf_counter() - t

    probe = allrows[:: max(1, nrows // 256)]
    t_probe = attn(probe)
    left = max(budget_s - t_heads - t_acc - t_probe, 1.0)
    n = int(min(nrows, max(len(probe), len(probe) * left / max(t_probe, 1e-6))))
    stride = max(1, nrows // n)
    sample = allrows[::stride]
    t_attn = attn(sample) * nrows / len(sample)
    step_s = t_heads + t_attn + t_acc
    return {"value": round(1.0 / step_s, 4), "unit": "steps/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(),
            "stage_s": {"heads": round(t_heads, 3), "tree_attention": round(t_attn, 3),
                        "tree_accept": round(t_acc, 3)},
            "sample": f"one verify step of {wl.name}: heads (all {wl.B} sequences, "
                      f"{wl.K} heads) and acceptance in full; tree attention on "
                      + (f"all {nrows} output rows" if stride == 1 else
                         f"every {stride}th of its {nrows} output rows ({len(sample)} rows, "
                         f"time scaled to all rows)")}


if __name__ == "__main__":
    main()
