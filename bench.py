#!/usr/bin/env python3
"""Benchmark of one DFlash-style draft step on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2]

One step = fuse_ctx + inject_kv of the rows committed by the previous step,
draft_block (5-layer Qwen3-8B-shaped drafter, block 16, context 1024 at the
start) and verify_accept against a synthetic target argmax whose accepted
prefix lengths follow a geometric law with p = 0.8, truncated at B-1. The
target tokens depend on the step's own drafts, so they are built in an untimed
first pass over the same steps; the state is then reset and the steps replayed
(bit-identically) with the recorded targets, so the timed region holds only
library calls. Inputs are seeded synthetic tensors resident in HBM.

Prints one JSON line: drafted tokens/s (batch*(B-1) per step), the step
latency, the roofline of the dominant kernel (the LM-head GEMM with fused
argmax: it streams the whole [V, H] head once per step) and, on rank 0, the
fp64 oracle timed on the host cores for the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "draft-step latency (µs) + drafted tokens/s, 5-layer drafter, block 16; %roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# What the LM-head kernel compiles from: its source, the device helpers and,
# of the launch header, the GEMM parameter block and modes. The PMC summary
# records their hash, and a change to any of them voids its traffic figure.
TRAFFIC_SOURCES = ("gemm_stream.hip", "common.h")


def kernel_source_hash(root):
    import hashlib
    import re
    csrc = os.path.join(root, "block_diffusion_drafter_target_amd", "csrc")
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    hdr = open(os.path.join(csrc, "internal.h")).read()
    for pat in (r"struct GemmParams \{.*?\n\};", r"enum GemmMode \{[^}]*\};"):
        m = re.search(pat, hdr, re.S)
        h.update(m.group(0).encode() if m else b"?")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes of the LM-head kernel from the committed rocprofv3 PMC summary,
    or None when the kernel's sources changed since the counters were taken."""
    root = os.path.dirname(os.path.abspath(__file__))
    summary = os.path.join(root, "profiles", "lm_head_argmax_c2_pmc.txt")
    try:
        kv = dict(line.split(": ", 1) for line in open(summary).read().splitlines() if ": " in line)
        sha = kernel_source_hash(root)
    except OSError:
        return None
    if kv.get("kernel_source_sha256", "").strip() != sha:
        return None
    return int(kv["traffic_fetch_bytes"]) + int(kv["traffic_write_bytes"])


def synth_target(torch, draft, m, rnd, vocab):
    """Target argmax rows [batch, B] whose accepted prefix with draft is m."""
    batch, bm1 = draft.shape
    j = torch.arange(bm1 + 1, device=draft.device)[None, :]
    d_ext = torch.nn.functional.pad(draft, (0, 1))
    t = torch.where(j < m[:, None], d_ext, rnd)
    return torch.where((j == m[:, None]) & (m[:, None] < bm1), (d_ext + 1) % (vocab - 1), t)


def sampling_steps(torch, dr, cfg, args, taps_step, state):
    """The step in sampling mode at temperature args.temperature: fuse + inject
    of the committed rows, the sampled draft block (its logits written), and
    speculative-sampling verification against synthetic target logits of the
    block rows (seeded N(0, 2), resident before timing). Timed like the greedy
    steps, from the state after the greedy warmup."""
    from block_diffusion_drafter_target_amd import binding as bd
    B, V, batch = cfg.block, cfg.vocab, cfg.batch
    for k, v in state.items():
        getattr(dr, k).copy_(v)
    g = torch.Generator(device="cuda").manual_seed(4)
    zt = torch.randn((batch * B, V), generator=g, device="cuda") * 2.0
    T, seed = args.temperature, 2024

    def step(i):
        dr.fuse_ctx(taps_step, batch * B, dr.ctx)
        dr.inject_kv(dr.ctx, batch * B, dr.commit_rows, dr.n_commit, batch * B)
        dr.draft_block_sample(T, seed, i, anchor=dr.anchor_out)
        dr.verify_sample(zt, T, seed, i)

    for i in range(args.warmup):
        step(1 + i)
    torch.cuda.synchronize()
    bd.dflash_profile_enable(["lm_head", "verify"])
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(1 + args.warmup + i)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    v_ms, v_n = bd.dflash_profile_read("verify")
    bd.dflash_profile_enable([])
    assert int(dr.status.abs().max()) == 0, "a sequence ran out of cache"
    return {"temperature": T, "us_per_step": round(ms * 1e3, 1),
            "drafted_tokens_per_s": round(batch * (B - 1) / (ms * 1e-3), 1),
            "us_verify_sample": round(1e3 * v_ms / max(1, v_n), 1),
            "note": ("fuse + inject + sampled draft block (logits written, Gumbel-max tokens) + "
                     "speculative-sampling verify against synthetic target logits")}


def target_verify(cfg, W, lens, args, dr):
    """The target side of a step: one causal pass of the target model over the
    B block tokens of every sequence (argmax + taps), timed over repeated
    passes at the workload's context (each pass rewrites the same speculative
    slots; nothing is committed); a one-token pass (greedy decoding's cost per
    token); and a whole speculative step on the device (draft, target pass,
    verify, both commits) replayed from a captured graph."""
    import torch

    from block_diffusion_drafter_target_amd import DeviceTarget, synth
    from block_diffusion_drafter_target_amd.drafter import _LoopState, device_step

    if not cfg.target_layers:
        raise SystemExit(f"config {cfg.name} has no target model")
    B, batch, H = cfg.block, cfg.batch, cfg.hidden
    t0 = time.time()
    TW = synth.make_target_weights(cfg, W)
    log(f"target weights ({cfg.target_layers} layers) generated in {time.time() - t0:.1f} s")
    L = int(lens.max())
    loop_steps = 16
    tgt = DeviceTarget(cfg, TW, cfg.target_layers, cfg.tap_layers, batch=batch,
                       max_ctx=L + (2 * loop_steps + 4) * B + 64, max_n=B)
    del TW
    # prefill every sequence's context in passes of B tokens (ragged contexts:
    # a sequence keeps only its own length through the commit of all rows
    # below it)
    dev = tgt.device
    for i0 in range(0, L, B):
        n = min(B, L - i0)
        toks = torch.from_numpy(np.stack([synth.make_prompt(cfg, n, seed=1000 + 7 * b + i0)
                                          for b in range(batch)]).astype(np.int32)).to(dev)
        tgt.pass_tokens(toks)
        rows = [(b * n + j, b, i0 + j) for b in range(batch) for j in range(n) if i0 + j < int(lens[b])]
        if rows:
            tgt.commit(torch.tensor(rows, dtype=torch.int32, device=dev),
                       torch.tensor([len(rows)], dtype=torch.int32, device=dev), len(rows))
    torch.cuda.synchronize()
    assert tgt.ctx_len.cpu().numpy().tolist() == lens.tolist()
    toks = torch.from_numpy(np.stack([synth.make_prompt(cfg, B, seed=5000 + b) for b in range(batch)])
                            .astype(np.int32)).to(dev)
    for _ in range(3):
        tgt.pass_tokens(toks)
    torch.cuda.synchronize()
    reps = max(5, min(args.steps, 50))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        tgt.pass_tokens(toks)
    stop.record()
    torch.cuda.synchronize()
    us = 1e3 * start.elapsed_time(stop) / reps
    assert int(tgt.status.abs().max()) == 0
    # one token per sequence: greedy decoding's cost per token
    one = toks[:, :1].contiguous()
    tgt.pass_tokens(one)
    start.record()
    for _ in range(reps):
        tgt.pass_tokens(one)
    stop.record()
    torch.cuda.synchronize()
    us_one = 1e3 * start.elapsed_time(stop) / reps
    # whole steps on the device, captured in a graph (the drafter keeps its
    # own context from the timed draft steps; both caches grow by the
    # accepted rows of every step)
    st = _LoopState(torch, batch, B, 2 * loop_steps + 2, dev, None)
    st.budget.fill_(1 << 30)
    dr.status.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(loop_steps):
                device_step(dr, tgt, st)
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    acc0 = int(st.cursor.sum())
    start.record()
    g.replay()
    stop.record()
    torch.cuda.synchronize()
    us_step = 1e3 * start.elapsed_time(stop) / loop_steps
    emitted = (int(st.cursor.sum()) - acc0) / (loop_steps * batch)
    assert int(tgt.status.abs().max()) == 0 and int(dr.status.abs().max()) == 0
    del g
    V, I, NLt = cfg.vocab, cfg.intermediate, cfg.target_layers
    layer_bytes = 2 * H * (cfg.qkv_width + cfg.q_width + 2 * I) + 2 * I * H
    wbytes = NLt * layer_bytes + V * H * 2
    res = {"layers": NLt, "taps": list(cfg.tap_layers), "tokens_per_pass": batch * B, "context": L,
           "us_per_pass": round(us, 1), "weight_bytes": wbytes,
           "weight_stream_GBps": round(wbytes / (us * 1e-6) / 1e9, 1),
           "weight_stream_frac": round(wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "us_per_one_token_pass": round(us_one, 1),
           "device_step_us": round(us_step, 1),
           "device_step_tokens_per_seq": round(emitted, 3),
           "device_step_note": ("draft + target pass + verify + both commits, graph-replayed; "
                                "tokens per step measured with untrained synthetic weights")}
    del tgt
    torch.cuda.empty_cache()
    return res


def cpu_baseline(cfg, W, L, repeats: int, seconds: float, threads: int | None = None):
    """The fp64 oracle's draft step on the host cores: steps repeated until at
    least `repeats` of them and `seconds` of timed work have run; the median.
    threads: BLAS threads (None: the library's default, one per core)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from block_diffusion_drafter_target_amd import synth
    from oracle import ref
    ocfg = ref.OracleConfig.from_any(cfg)
    t0 = time.time()
    WO = {k: synth.bf16_to_f64(v) for k, v in W.items()}
    prep = time.time() - t0
    B, batch = cfg.block, cfg.batch
    g = np.random.default_rng(0)
    cache = ref.new_cache(ocfg, batch, L + B)
    cache["k"][:, :, :L] = g.standard_normal(cache["k"][:, :, :L].shape)
    cache["v"][:, :, :L] = g.standard_normal(cache["v"][:, :, :L].shape)
    taps = synth.bf16_to_f64(synth.make_taps(cfg, batch * B, tid=999))
    anchor = synth.make_anchors(cfg)
    times = []
    with threadpool_limits(limits=threads, user_api="blas"):
        t_all = time.perf_counter()
        while len(times) < repeats or (time.perf_counter() - t_all < seconds and len(times) < 10000):
            t = time.perf_counter()
            ctx = ref.fuse_ctx(ocfg, WO, taps)
            ref.inject_kv(ocfg, WO, ctx, [(b * B + i, b, L - B + i) for b in range(batch) for i in range(B)], cache)
            r = ref.draft_block(ocfg, WO, cache, [L] * batch, anchor)
            tgt = np.concatenate([r["draft"], np.zeros((batch, 1), np.int64)], axis=1)
            ref.verify_accept(r["draft"], tgt, [L] * batch)
            times.append(time.perf_counter() - t)
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = int(blas[0]["num_threads"]) if blas else (os.cpu_count() or 1)
    t_step = float(np.median(times))
    return {"value": batch * (B - 1) / t_step, "unit": "drafted tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"one full draft step (fuse+inject of {batch * B} rows, {cfg.n_layers} layers at "
                       f"context {L}, full LM head, verify) in fp64 numpy, median of {len(times)} steps "
                       f"({sum(times):.1f} s of timed work); step {t_step * 1e3:.0f} ms; weight upcast to "
                       f"fp64 ({prep:.1f} s) not timed"),
            "ms_per_step": t_step * 1e3}


def phase_roofline(cfg, phases, ctx0, ctx1):
    """Achieved fraction of the MI355X roofline of every timed phase of the
    step, from its per-step time (library HIP events, breakdown steps) and its
    algorithmic work: weight bytes (HBM) and GEMM flops (MFMA) of the GEMMs,
    K/V bytes of the attention (at the breakdown steps' mean context)."""
    B, batch, NL, H = cfg.block, cfg.batch, cfg.n_layers, cfg.hidden
    I, V, D, Hkv = cfg.intermediate, cfg.vocab, cfg.head_dim, cfg.n_kv_heads
    Mb, Ml = batch * B, batch * (B - 1)
    gemms = {  # name: (weight bytes, activation rows) per step
        "qkv": (NL * 2 * cfg.qkv_width * H, Mb), "o": (NL * 2 * H * cfg.q_width, Mb),
        "gate_up": (NL * 2 * 2 * I * H, Mb), "down": (NL * 2 * H * I, Mb), "lm_head": (2 * V * H, Ml),
        "fuse": (2 * H * cfg.tap_width, Mb), "inject": (NL * 2 * 2 * cfg.kv_width * H, Mb)}
    out = {}
    tot_b = tot_us = 0.0
    for name, (wb, rows) in gemms.items():
        if name not in phases:
            continue
        us = phases[name]["us_per_step"]
        flops = rows * wb  # 2 flops per weight (2 bytes) and activation row
        out[name] = {"us_per_step": us, "weight_bytes": wb, "GBps": round(wb / us * 1e-3, 1),
                     "hbm_frac": round(wb / us * 1e-3 / HBM_PEAK_GBS, 4),
                     "tflops": round(flops / us * 1e-6, 1),
                     "mfma_frac": round(flops / us * 1e-6 / MFMA_PEAK_TFLOPS, 4)}
        tot_b += wb
        tot_us += us
    if tot_us:
        out["weight_gemms"] = {"us_per_step": round(tot_us, 2), "weight_bytes": int(tot_b),
                               "GBps": round(tot_b / tot_us * 1e-3, 1),
                               "hbm_frac": round(tot_b / tot_us * 1e-3 / HBM_PEAK_GBS, 4)}
    keys = float(np.mean((ctx0 + ctx1) / 2.0 + B)) * batch  # keys read per kv head and layer
    kv_bytes = keys * Hkv * D * 2 * 2 * NL
    for name, parts in (("attention", ("attention",)), ("attention_with_merge", ("attention", "merge"))):
        if all(p in phases for p in parts):
            us = sum(phases[p]["us_per_step"] for p in parts)
            out[name] = {"us_per_step": round(us, 2), "kv_bytes": int(kv_bytes),
                         "GBps": round(kv_bytes / us * 1e-3, 1),
                         "hbm_frac": round(kv_bytes / us * 1e-3 / HBM_PEAK_GBS, 4)}
    return out


def library_gemms(torch, cfg, rows_list):
    """The step's weight GEMMs in torch's bf16 linear (hipBLASLt on ROCm), for
    comparison with the library's kernels on the same shapes: Y = X W^T with W
    [N, K] bf16, X [M, K] bf16, weights cycled over copies that together exceed
    the 256 MB Infinity Cache (cold, as in the step), launches captured in one
    graph and replayed. Returns one record per (rows, product)."""
    import math
    F = torch.nn.functional
    H, qw = cfg.hidden, cfg.n_q_heads * cfg.head_dim
    shapes = {"qkv": (qw + 2 * cfg.n_kv_heads * cfg.head_dim, H), "o": (H, qw),
              "gate_up": (2 * cfg.intermediate, H), "down": (H, cfg.intermediate),
              "lm_head": (cfg.vocab, H), "fuse": (H, cfg.n_tap * H)}
    out = []
    dev = torch.device("cuda")
    side = torch.cuda.Stream()
    for M in rows_list:
        for name, (N, K) in shapes.items():
            nc = max(2, math.ceil(1.2e9 / (N * K * 2)))
            Ws = [torch.randn(N, K, device=dev, dtype=torch.bfloat16) * 0.02 for _ in range(nc)]
            X = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
            Y = [None] * nc
            with torch.cuda.stream(side):
                for i in range(nc):
                    Y[i] = F.linear(X, Ws[i])
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for i in range(nc):
                    Y[i] = F.linear(X, Ws[i])
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, 40 // nc)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = 1e3 * e0.elapsed_time(e1) / (reps * nc)
            flop = 2.0 * M * N * K
            out.append({"rows": M, "gemm": name, "N": N, "K": K, "us": round(us, 1),
                        "weight_TBps": round(N * K * 2 / us / 1e6, 2), "mfma_frac": round(flop / us / 1e6 / MFMA_PEAK_TFLOPS, 3)})
            log(f"library GEMM {name} M={M}: {us:.1f} us")
            del g, Ws, X, Y
            torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--block", type=int, default=0, help="override the block size")
    ap.add_argument("--batch", type=int, default=0, help="override the batch")
    ap.add_argument("--cpu-repeats", type=int, default=3, help="fewest oracle steps of the CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="least timed work of the CPU baseline (seconds)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--target-verify", action="store_true",
                    help="also time the target's causal verify pass (Qwen3-8B-shaped 36-layer target)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="also time the step in sampling mode at this temperature")
    ap.add_argument("--graph", action="store_true",
                    help="also time the same steps captured in one HIP graph")
    ap.add_argument("--evict-mb", type=int, default=0,
                    help="also time steps one by one with this many MiB written between them (outside "
                         "each step's events), so that no step finds the previous one's data in the "
                         "256 MB Infinity Cache")
    ap.add_argument("--library-gemms", action="store_true",
                    help="instead of the step: time torch's bf16 linear (hipBLASLt) on the step's weight "
                         "GEMM shapes at the block rows of the workload and of 16, 128 and 512 rows")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; runs on several GPUs are not implemented",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from block_diffusion_drafter_target_amd import Drafter, synth
    from block_diffusion_drafter_target_amd import binding as bd

    cfg = synth.CONFIGS[args.config]
    if args.block:
        cfg = cfg.with_(block=args.block)
    if args.batch:
        cfg = cfg.with_(batch=args.batch)
    B, V, H, batch = cfg.block, cfg.vocab, cfg.hidden, cfg.batch
    if args.library_gemms:
        rows = sorted({batch * B, 16, 128, 512})
        print(json.dumps({"library_gemms": "torch bf16 linear (hipBLASLt), cold weights, graph-replayed",
                          "config": {"workload": cfg.name}, "results": library_gemms(torch, cfg, rows)}))
        return
    lens = synth.make_ctx_lens(cfg)
    n_break = min(args.steps, 20)  # steps of the per-phase breakdown pass
    n_steps = 1 + args.warmup + args.steps + n_break + (args.warmup if args.temperature > 0 else 0)
    max_ctx = int(lens.max()) + (n_steps + 2) * B + 64
    t0 = time.time()
    W = synth.make_weights(cfg)
    log(f"weights generated in {time.time() - t0:.1f} s")
    dev = torch.device("cuda")
    dr = Drafter(cfg, W, batch=batch, max_ctx=max_ctx, max_rows=max(int(lens.max()), batch * B), device=dev)

    # context ingest (fuse + inject of the whole prompt), timed on its own:
    # every sequence is ingested twice (the same rows into the same slots) and
    # the second pass is timed, so that first-launch costs stay out of it
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ingest_ms = 0.0
    for b in range(batch):
        taps = torch.from_numpy(synth.make_taps(cfg, int(lens[b]), tid=b).view(np.int16)).view(torch.bfloat16).to(dev)
        dr.ingest(b, taps)
        torch.cuda.synchronize()
        ev0.record()
        dr.ingest(b, taps)
        ev1.record()
        torch.cuda.synchronize()
        ingest_ms += ev0.elapsed_time(ev1)
        del taps
    assert dr.ctx_len.cpu().numpy().tolist() == lens.tolist()
    ingest_rows = int(lens.sum())
    ingest_flop = 2.0 * ingest_rows * H * (cfg.tap_width + cfg.n_layers * cfg.kv_width * 2)

    # per-step synthetic inputs, resident before timing
    taps_step = torch.from_numpy(synth.make_taps(cfg, batch * B, tid=999).view(np.int16)).view(torch.bfloat16).to(dev)
    m_all = torch.from_numpy(np.stack([synth.geometric_accept(batch, B, 0.8, step=i) for i in range(n_steps)])).to(dev)
    g = np.random.default_rng(synth.SEED_TARGET)
    rnd_all = torch.from_numpy(g.integers(0, V - 1, size=(n_steps, batch, B)).astype(np.int32)).to(dev)
    dr.anchor.copy_(torch.from_numpy(synth.make_anchors(cfg)))

    # bootstrap: one draft + verify so that the first step has committed rows
    dr.draft_block(anchor=dr.anchor)
    dr.verify_accept(synth_target(torch, dr.draft, m_all[0], rnd_all[0], V))
    saved = {k: getattr(dr, k).clone() for k in ("ctx_len", "anchor_out", "commit_rows", "n_commit")}

    def step(tgt):
        dr.fuse_ctx(taps_step, batch * B, dr.ctx)
        dr.inject_kv(dr.ctx, batch * B, dr.commit_rows, dr.n_commit, batch * B)
        dr.draft_block(anchor=dr.anchor_out)
        dr.verify_accept(tgt)

    # pass 1 (untimed): the target tokens of every step
    targets = [None]
    for i in range(1, n_steps):
        dr.fuse_ctx(taps_step, batch * B, dr.ctx)
        dr.inject_kv(dr.ctx, batch * B, dr.commit_rows, dr.n_commit, batch * B)
        dr.draft_block(anchor=dr.anchor_out)
        targets.append(synth_target(torch, dr.draft, m_all[i], rnd_all[i], V).clone())
        dr.verify_accept(targets[i])
    torch.cuda.synchronize()
    for k, v in saved.items():
        getattr(dr, k).copy_(v)

    # pass 2: warmup, timed steps, per-phase breakdown steps
    for i in range(args.warmup):
        step(targets[1 + i])
    torch.cuda.synchronize()
    assert int(dr.status.abs().max()) == 0, "a sequence ran out of cache"
    after_warmup = {k: getattr(dr, k).clone() for k in ("ctx_len", "anchor_out", "commit_rows", "n_commit")}
    # The timed region: K steps between two events. The LM head is timed live
    # inside it by the library's phase events on every LM_STRIDE-th step (an
    # event pair costs the stream a few microseconds per step; the per-step
    # spread comes from a replay of the same steps below).
    LM_STRIDE = 8
    bd.dflash_profile_enable(["lm_head"])
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        bd.dflash_profile_pause(i % LM_STRIDE != 0)
        step(targets[1 + args.warmup + i])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    lm_ms, lm_n = bd.dflash_profile_read("lm_head")
    bd.dflash_profile_enable([])
    ctx_after = dr.ctx_len.cpu().numpy()
    assert int(dr.status.abs().max()) == 0
    # the replay accepted exactly the recorded prefix lengths
    assert dr.accept_len.cpu().numpy().tolist() == m_all[args.warmup + args.steps].cpu().numpy().tolist()

    # spread of single steps (p10, median, p90): the same K steps replayed from
    # the same state with an event at every step boundary; the replay must
    # reach the timed run's end state
    end_state = {k: getattr(dr, k).clone() for k in ("ctx_len", "anchor_out", "commit_rows", "n_commit")}
    for k, v in after_warmup.items():
        getattr(dr, k).copy_(v)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        step(targets[1 + args.warmup + i])
        evs[i + 1].record()
    torch.cuda.synchronize()
    for k, v in end_state.items():
        assert torch.equal(getattr(dr, k), v), f"the spread replay diverged from the timed steps ({k})"
    per_step = np.array([1e3 * evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    spread = {"p10": round(float(np.percentile(per_step, 10)), 1), "median": round(float(np.median(per_step)), 1),
              "p90": round(float(np.percentile(per_step, 90)), 1)}

    cold = None
    if args.evict_mb:
        # the same timed steps again from the same state, each bracketed by its
        # own events, with a scratch write of evict_mb MiB between steps
        end_state = {k: getattr(dr, k).clone() for k in ("ctx_len", "anchor_out", "commit_rows", "n_commit")}
        for k, v in after_warmup.items():
            getattr(dr, k).copy_(v)
        scratch = torch.empty(args.evict_mb << 20, dtype=torch.uint8, device=dev)
        ea = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        eb = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            scratch.fill_(i & 255)
            ea[i].record()
            step(targets[1 + args.warmup + i])
            eb[i].record()
        torch.cuda.synchronize()
        cold_us = np.array([1e3 * ea[i].elapsed_time(eb[i]) for i in range(args.steps)])
        for k, v in end_state.items():
            assert torch.equal(getattr(dr, k), v), f"the cold-cache replay diverged ({k})"
        del scratch
        cold = {"evict_mb": args.evict_mb, "us_per_step_median": round(float(np.median(cold_us)), 1),
                "us_per_step_mean": round(float(cold_us.mean()), 1),
                "drafted_tokens_per_s": round(batch * (B - 1) / (float(np.median(cold_us)) * 1e-6), 1)}

    graph_ms = None
    if args.graph:
        # the same timed steps, launched as one captured graph from the same state
        end_state = {k: getattr(dr, k).clone() for k in ("ctx_len", "anchor_out", "commit_rows", "n_commit")}
        for k, v in after_warmup.items():
            getattr(dr, k).copy_(v)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(targets[1 + args.warmup + i])
        for k, v in after_warmup.items():
            getattr(dr, k).copy_(v)
        torch.cuda.synchronize()
        start.record()
        graph.replay()
        stop.record()
        torch.cuda.synchronize()
        graph_ms = start.elapsed_time(stop) / args.steps
        for k, v in end_state.items():
            assert torch.equal(getattr(dr, k), v), f"graph replay diverged from the eager steps ({k})"
        del graph

    sampling = None
    if args.temperature > 0:
        sampling = sampling_steps(torch, dr, cfg, args, taps_step, after_warmup)

    ctx_break0 = dr.ctx_len.cpu().numpy().astype(np.int64)
    bd.dflash_profile_enable(list(bd.PHASES))
    for i in range(n_break):
        step(targets[1 + args.warmup + args.steps + i])
    torch.cuda.synchronize()
    ctx_break1 = dr.ctx_len.cpu().numpy().astype(np.int64)
    phases = {}
    for name in bd.PHASES:
        t, n = bd.dflash_profile_read(name)
        if n:
            phases[name] = {"us_per_step": round(1e3 * t / n_break, 2), "launches_per_step": n / n_break,
                            "us_per_launch": round(1e3 * t / n, 2)}
    bd.dflash_profile_enable([])

    if args.calib_copy_mb:
        # a plain copy of known size: rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of
        # this kernel calibrate the counters against bytes actually moved
        src = torch.ones(args.calib_copy_mb << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # roofline of the dominant kernel: the LM head streams V*H bf16 weights
    Ml = batch * (B - 1)
    lm_bytes = V * H * 2 + Ml * H * 2 + Ml * 8
    lm_us = 1e3 * lm_ms / max(1, lm_n)
    achieved = lm_bytes / (lm_us * 1e-6) / 1e9
    # the library streams up to 32 LM rows per workgroup tile; more take the
    # LDS-tiled kernel (64- or 128-row tiles)
    lm_kernel = (f"gemm_stream_kernel<{1 if Ml <= 16 else 2},2,argmax>" if Ml <= 32 else
                 f"gemm_tile_kernel<2,{4 if Ml <= 64 else 8},argmax>")
    roofline = {"kernel": f"{lm_kernel} (LM head + fused argmax)", "bound": "hbm",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "bytes_per_launch": lm_bytes, "us_per_launch": round(lm_us, 2)}
    # whole-step weight streaming, for context
    layer_bytes = 2 * H * (cfg.qkv_width + cfg.q_width + 2 * cfg.intermediate) + 2 * cfg.intermediate * H
    step_weight_bytes = cfg.n_layers * layer_bytes + V * H * 2 + H * cfg.tap_width * 2 + \
        cfg.n_layers * 2 * cfg.kv_width * H * 2
    drafted = batch * (B - 1)
    out = {
        "metric": METRIC,
        "value": round(drafted / (ms * 1e-3), 1),
        "unit": "drafted tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "latency_us": round(ms * 1e3, 1),
        "latency_us_spread": spread,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": (f"{cfg.name} drafter: H {H}, {cfg.n_q_heads}/{cfg.n_kv_heads} heads of "
                                f"{cfg.head_dim}, I {cfg.intermediate}, V {V}, {cfg.n_tap} taps; batch {batch}, "
                                f"block {B}, context {int(lens.min())}..{int(lens.max())} at start "
                                f"(ends at {int(ctx_after.max())}); geometric acceptance p=0.8"),
                   "batch": batch, "block": B, "context": int(lens.max()), "layers": cfg.n_layers},
        "roofline": roofline,
        "step_weight_bytes": step_weight_bytes,
        "step_weight_stream_frac": round(step_weight_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "ingest_ms": round(ingest_ms, 3),
        "ingest": {"rows": ingest_rows, "gflop": round(ingest_flop * 1e-9, 1),
                   "tflops": round(ingest_flop / (ingest_ms * 1e-3) * 1e-12, 1),
                   "mfma_frac": round(ingest_flop / (ingest_ms * 1e-3) * 1e-12 / MFMA_PEAK_TFLOPS, 4),
                   "note": "fuse + inject of every context row (GEMM flops), second pass timed"},
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "cold_cache": cold,
        "sampling": sampling,
        "phases": phases,
        "phase_roofline": phase_roofline(cfg, phases, ctx_break0, ctx_break1),
    }
    if args.target_verify:
        out["target_verify"] = target_verify(cfg, W, lens, args, dr)
    del dr
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host ...")
        cb = cpu_baseline(cfg, W, int(lens.max()), args.cpu_repeats, args.cpu_seconds)
        # the same step on one BLAS thread: a bounded sample of a few steps
        one = cpu_baseline(cfg, W, int(lens.max()), 2, min(6.0, args.cpu_seconds), threads=1)
        cb["single_thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample", "ms_per_step")}
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
