#!/usr/bin/env python3
"""Benchmark of the batched verify forward (DFlash block speculative decoding) on one MI355X.

Workload (the target-shaped verify): 42 decoder layers, hidden 2560, 8 query heads of 256; sliding
layers KV row 2 x 256 floats/position with window 512, every 6th layer full with 2 x 512; layers
24..41 KV-shared; FFN 10240 (20480 on shared layers); Q4_1 weights; bf16 tied head of 262144
rows; 1024 cached positions; k = 8 verified rows. All inputs are seeded synthetic draws (seed 0).

A step = one verify pass over the k rows (embed, 42 layers, final norm, head, logits_all and taps),
the greedy accept (argmax + longest prefix) and commit_verify_rows(0), which rolls the appended rows
back so every step verifies at the same 1024 cached positions.

Prints one JSON line: verified rows/s, the Q4_1 weight stream in GB/s and as a fraction of the
8 TB/s HBM peak, the roofline of the dominant kernel -- the Q4_1 GEMM, over all its launches of a
pass, with each launch class (q|k|v, o, gate|up, down) beside it, timed with HIP events on the
model's stream, and the HBM traffic the committed rocprofv3 counter summary gives for the same GEMM
source --, the k = 1 step for comparison, and the CPU oracle timed on this host's cores
(cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
import numpy as np

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "q4_1_gemm.target_k8.pmc_traffic.txt")
GEMM_SRC = os.path.join(ROOT, "block_verify_forward_amd", "csrc", "gemm.hip")


def measured_traffic(cls: str):
    """HBM bytes per launch of a GEMM class (gate_up, down) from the committed rocprofv3 counter
    summary, or None when the GEMM source has changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    key = f"traffic_bytes_per_launch.{cls}"
    if fields.get("gemm_hip_sha256") != src or key not in fields:
        return None
    return int(fields[key])
METRIC = "verified rows/s and Q4_1 weight-stream HBM GB/s (% of peak), k=8 verify pass"


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def planes(m, args, verify: bool = True):
    """The model with the memory variants asked for: bf16 K/V planes (--kv-bf16), and on the verify
    model ring sliding planes (--kv-ring) and per-layer embeddings of width --ple-dim."""
    import dataclasses
    if args.kv_bf16:
        m = dataclasses.replace(m, kv_bf16=1)
    if verify and args.kv_ring:
        m = dataclasses.replace(m, kv_ring=1)
    if verify and args.ple_dim:
        m = dataclasses.replace(m, ple_dim=args.ple_dim)
    return m


def build_weights(m, seed: int, threads: int):
    from block_verify_forward_amd import synth
    return synth.make_weights(m, seed, threads=threads)


def cpu_baseline(m, w, kv, ctx, toks, budget_s: float):
    """The CPU oracle, as it stands, on this host: one k-row verify of the same workload. If one
    full pass would take longer than the budget, a prefix of the layers is timed and the pass time
    is scaled by Q4_1 bytes (the sample is named in the result)."""
    import oracle
    from block_verify_forward_amd import synth
    k = len(toks)
    threads = oracle.threads()
    # time a 1-layer model (plus head) to estimate the full pass
    import dataclasses
    m1 = dataclasses.replace(m, n_layers=1, layers=m.layers[:1], tap_layers=())
    w1 = {"layers": w["layers"][:1], "embed": w["embed"], "final_norm": w["final_norm"]}
    o1 = oracle.Model(m1, w1)
    o1.set_kv(kv[:1], ctx)
    t = time.perf_counter()
    o1.verify_batch(toks)
    t1 = time.perf_counter() - t
    full_est = t1 * synth.q4_1_bytes(m) / synth.q4_1_bytes(m1)
    if full_est <= budget_s:
        # whole passes of the workload, repeated until about 10 s of CPU work (or the budget)
        o = oracle.Model(m, w)
        o.set_kv(kv, ctx)
        n, t = 0, time.perf_counter()
        while True:
            o.verify_batch(toks)
            o.commit_verify_rows(0)
            n += 1
            el = time.perf_counter() - t
            if el >= min(10.0, budget_s) or el + el / n > budget_s:
                break
        dt = el / n
        sample = f"{n} full k={k} verify passes of the same workload ({m.n_layers} layers + head), {el:.1f} s"
    else:
        n_s = max(1, min(24, int(budget_s / t1)))
        ms = dataclasses.replace(m, n_layers=n_s, layers=m.layers[:n_s], tap_layers=())
        ws = {"layers": w["layers"][:n_s], "embed": w["embed"], "final_norm": w["final_norm"]}
        o = oracle.Model(ms, ws)
        o.set_kv(kv[:n_s], ctx)
        t = time.perf_counter()
        o.verify_batch(toks)
        ds = time.perf_counter() - t
        dt = ds * synth.q4_1_bytes(m) / synth.q4_1_bytes(ms)
        sample = (f"first {n_s} layers + head of the workload, k={k}, timed {ds:.1f} s; pass time scaled by "
                  f"Q4_1 bytes to {m.n_layers} layers")
    one = cpu_one_core(m, w, kv, ctx, toks)
    return {"value": round(k / dt, 4), "unit": "verified rows/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds_per_pass": round(dt, 3), "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "one_core": one}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_one_core(m, w, kv, ctx, toks):
    """The oracle on one thread: a 1-layer and a 2-layer prefix of the workload (each with the
    head) give the time of layer 0, of layer 1 and of the head; the pass time is the head plus every
    layer scaled by its Q4_1 bytes from the measured layer of the same kind."""
    import dataclasses
    import oracle
    from block_verify_forward_amd import synth
    k = len(toks)
    all_threads = oracle.threads()
    oracle.set_threads(1)
    try:
        def prefix(n):
            mp = dataclasses.replace(m, n_layers=n, layers=m.layers[:n], tap_layers=())
            wp = {"layers": w["layers"][:n], "embed": w["embed"], "final_norm": w["final_norm"]}
            o = oracle.Model(mp, wp)
            o.set_kv(kv[:n], ctx)
            t = time.perf_counter()
            o.verify_batch(toks)
            return time.perf_counter() - t, mp
        t1, m1 = prefix(1)
        t2, m2 = prefix(2)
    finally:
        oracle.set_threads(all_threads)
    t_layer1 = max(t2 - t1, 1e-9)
    t_head = max(t1 - t_layer1, 0.0)
    b1 = synth.q4_1_bytes(m2) - synth.q4_1_bytes(m1)
    dt = t_head + t_layer1 * synth.q4_1_bytes(m) / b1
    return {"value": round(k / dt, 4), "unit": "verified rows/s", "cores": 1, "seconds_per_pass": round(dt, 2),
            "sample": f"layers 0 and 1 plus the head at one thread ({t1 + t2:.1f} s); the pass is the head "
                      f"({t_head:.2f} s) plus {m.n_layers} layers scaled by Q4_1 bytes from layer 1 ({t_layer1:.2f} s)"}


def run_loop(args):
    """The full speculative loop: target (42 layers) and draft (5 layers, hidden 2560, block 8) at full
    size, args.ctx cached positions on both, rounds until args.loop tokens; per round the accept
    length is drawn from the truncated geometric of the acceptance workload (mean 3.8) and imposed
    by steering the verify logits (synthetic weights accept nothing by themselves)."""
    import dataclasses
    import torch
    from block_verify_forward_amd import bvf, synth
    from block_verify_forward_amd.loop import SpecLoop

    threads = min(16, os.cpu_count() or 8)
    max_ctx = args.ctx + args.loop + 64
    m = planes(synth.target_model(max_ctx=max_ctx, n_layers=args.layers, vocab=args.vocab), args)
    dm = planes(synth.draft_model(max_ctx=max_ctx), args, verify=False)
    t0 = time.time()
    w = synth.make_weights(m, args.seed, threads=threads)
    dw = synth.make_weights(dm, args.seed, threads=threads)
    kv = synth.make_kv(m, args.ctx, args.seed, threads=threads)
    kvd = synth.make_kv(dm, args.ctx, args.seed, threads=threads)
    log(f"synthetic target, draft and contexts drawn in {time.time() - t0:.1f} s")
    T = bvf.Model(m)
    T.load_weights(w)
    T.set_context(kv, args.ctx)
    D = bvf.Model(dataclasses.replace(dm, vocab=m.vocab))
    D.load_weights(dw)
    D.set_context(kvd, args.ctx)
    if args.graph and not args.no_graph:
        T.set_graph_mode(True)
        D.set_graph_mode(True)
    rounds_max = args.loop
    steer = synth.accept_lengths(args.seed, rounds_max, max_a=7)
    loop = SpecLoop(T, D, 8, temperature=args.temperature, seed=args.seed)
    snap_t, snap_d = T.snapshot_take(), D.snapshot_take()
    loop.start(17)
    for i in range(3):   # warm-up rounds, then back to the start
        loop.round(int(steer[i]))
    T.restore(snap_t)
    D.restore(snap_d)
    loop.start(17)
    torch.cuda.synchronize()
    # events around each draft block (recorded on the stream, no synchronisation): the round's split
    draft_ev = []
    draft_call = D.draft_block_forward

    def timed_draft(*a, **kw):
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        ev[0].record()
        draft_call(*a, **kw)
        ev[1].record()
        draft_ev.append(ev)

    D.draft_block_forward = timed_draft
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    toks = loop.run(args.loop, steer)
    e1.record()
    torch.cuda.synchronize()
    D.draft_block_forward = draft_call
    ms = e0.elapsed_time(e1)
    draft_ms = float(np.mean([a.elapsed_time(b) for a, b in draft_ev]))
    rounds = len(loop.accepted)
    assert loop.accepted == [int(a) for a in steer[:rounds]], "steered accept lengths not reproduced"
    res = {
        "metric": "speculative decode tokens/s (draft block 8 + batched verify k=8 + "
                  + (f"sampled accept T={args.temperature}" if args.temperature > 0 else "greedy accept") + " + commit)",
        "value": round(len(toks) / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "vs_baseline": None,
        "data": f"synthetic (seeded draws, seed {args.seed}); acceptance steered: truncated geometric p=0.8467",
        "config": {"workload": f"speculative loop: target {m.n_layers} layers hidden {m.hidden} Q4_1, draft 5 layers "
                               f"hidden 2560, block 8, {args.ctx} cached positions, {args.loop} tokens",
                   "kv_planes": ("bf16" if args.kv_bf16 else "fp32") + (", ring" if args.kv_ring else ""),
                   "ple_dim": args.ple_dim,
                   "launches": "graph replay" if args.graph and not args.no_graph else "direct"},
        "tokens": len(toks),
        "rounds": rounds,
        "tokens_per_target_pass": round(len(toks) / rounds, 3),
        "mean_accepted_drafts": round(float(np.mean(loop.accepted)), 3),
        "ms_per_round": round(ms / rounds, 4),
        "draft_block_ms": round(draft_ms, 4),
        "verify_graph_captures": T.graph_captures(),
        "draft_graph_captures": D.graph_captures(),
    }
    print(json.dumps(res), flush=True)


def run_draft(args):
    """The draft block forward at its real size: 5 layers (hidden 2560, 32 query / 8 KV heads of 128,
    FFN 5120, window 1024), fc over 5 tapped target rows, a block of 8, args.ctx cached context
    positions, and the target's tied bf16 head (args.vocab rows) on rows 1..7. Times args.steps blocks
    with 1 and with 8 new context rows (HIP events; the draft restored from a snapshot before each
    series) and reports ms per block and the bytes a block streams (the draft's Q4_1 layers, the bf16
    fc, the head, the visible context K/V) over that time against the 8 TB/s HBM peak."""
    import dataclasses
    import torch
    from block_verify_forward_amd import bvf, synth

    threads = min(16, os.cpu_count() or 8)
    B = 8
    max_ctx = args.ctx + 8 * (args.steps + args.warmup) + 64
    tm = synth.target_model(max_ctx=max_ctx, n_layers=1, vocab=args.vocab)   # the embedding and head only
    dm = planes(synth.draft_model(max_ctx=max_ctx), args, verify=False)
    t0 = time.time()
    tw = synth.make_weights(tm, args.seed, threads=threads)
    dw = synth.make_weights(dm, args.seed, threads=threads)
    kvd = synth.make_kv(dm, args.ctx, args.seed, threads=threads)
    log(f"synthetic draft, head and context drawn in {time.time() - t0:.1f} s")
    T = bvf.Model(tm)
    T.load_weights(tw)
    D = bvf.Model(dataclasses.replace(dm, vocab=tm.vocab))
    D.load_weights(dw)
    D.set_context(kvd, args.ctx)
    if args.graph and not args.no_graph:
        D.set_graph_mode(True)
    taps = torch.from_numpy(synth.bf16_normal(args.seed, "bench.draft.taps", (B, len(dm.tap_layers), dm.hidden))).cuda()
    last = torch.full((1,), 17, dtype=torch.int32, device="cuda")
    props = torch.zeros(B - 1, dtype=torch.int32, device="cuda")
    snap = D.snapshot_take()
    res = {}
    for n_new in (1, 8):
        D.restore(snap)
        for _ in range(args.warmup):
            D.draft_block_forward(T, taps[:n_new], n_new, last, B, 1.0, tm.vocab - 1, props)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            D.draft_block_forward(T, taps[:n_new], n_new, last, B, 1.0, tm.vocab - 1, props)
        e1.record()
        torch.cuda.synchronize()
        res[n_new] = e0.elapsed_time(e1) / args.steps
        log(f"draft block, {n_new} new context rows: {res[n_new]:.4f} ms")
    q4, _ = D.pass_bytes()
    _, head = T.pass_bytes()
    fc = len(dm.tap_layers) * dm.hidden * dm.hidden * 2
    kv_w = sum(2 * L.n_kv_heads * L.head_dim for L in dm.layers)   # K and V floats per position, all layers
    kv = (min(args.ctx, dm.draft_window) + B) * kv_w * (2 if args.kv_bf16 else 4)
    total = q4 + fc + head + kv
    gbs = total / (res[8] * 1e-3) / 1e9
    out = {
        "metric": "draft block forward ms (block 8: fc over the new taps, 5 layers, head on rows 1..7, argmax)",
        "value": round(res[8], 4),
        "unit": "ms per block",
        "n_gpus": 1,
        "higher_is_better": False,
        "vs_baseline": None,
        "data": f"synthetic (seeded draws, seed {args.seed})",
        "config": {"workload": f"draft block forward: 5 layers hidden 2560 Q4_1, fc 12800x2560 bf16, head {tm.vocab}x2560 "
                               f"bf16, {args.ctx} cached context positions, block 8, 8 new context rows",
                   "kv_planes": "bf16" if args.kv_bf16 else "fp32",
                   "launches": "graph replay" if args.graph and not args.no_graph else "direct"},
        "ms_per_block_1_new_row": round(res[1], 4),
        "bytes_per_block": {"q4_1": q4, "fc_bf16": fc, "head_bf16": head, "context_kv": kv, "total": total},
        "gbs": round(gbs, 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "ms_at_hbm_peak": round(total / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
    }
    print(json.dumps(out), flush=True)


def run_prefill(args):
    """Chunked prefill: args.prefill prompt tokens on top of args.ctx cached positions, in batched
    passes of up to 64 rows (one pass over the weights per chunk, four 16-row MFMA tiles per weight
    superblock), the head on the last row only; the context is restored from a snapshot before every
    timed run. Also times each Q4_1 GEMM class at 64 rows (HIP events over 3 x n_layers launches)
    and reports its weight-stream GB/s and useful bf16 MFMA TFLOP/s."""
    import torch
    from block_verify_forward_amd import bvf, synth

    threads = min(16, os.cpu_count() or 8)
    m = planes(synth.target_model(max_ctx=args.ctx + args.prefill + 64, n_layers=args.layers, vocab=args.vocab), args)
    w = build_weights(m, args.seed, threads)
    kv = synth.make_kv(m, args.ctx, args.seed, threads=threads)
    g = bvf.Model(m)
    g.load_weights(w)
    g.set_context(kv, args.ctx)
    toks = torch.from_numpy(synth.tokens(args.seed, "bench.prefill", args.prefill, m.vocab)).cuda()
    last = torch.empty(m.vocab, dtype=torch.float32, device="cuda")
    snap = g.snapshot_take()
    for _ in range(max(1, args.warmup // 2)):
        g.prefill(toks, last)
        g.restore(snap)
    torch.cuda.synchronize()
    times = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.prefill(toks, last)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
        assert g.positions_held() == args.ctx + args.prefill
        g.restore(snap)
    ms = float(np.median(times))
    # snapshot costs at ctx + prefill positions: a first take allocates, an update and a restore copy
    g.prefill(toks, last)
    torch.cuda.synchronize()
    t0 = time.time()
    s2 = g.snapshot_take()
    take_ms = (time.time() - t0) * 1e3
    t0 = time.time()
    g.snapshot_update(s2)
    update_ms = (time.time() - t0) * 1e3
    t0 = time.time()
    g.restore(s2)
    restore_ms = (time.time() - t0) * 1e3
    snap_mb = float(np.sum(s2.floats())) * (2 if args.kv_bf16 else 4) / 1e6
    del s2
    g.restore(snap)
    chunk = 64
    n_chunks = (args.prefill + chunk - 1) // chunk
    cls_ms, cls_bytes = g.time_gemms(chunk, 3)
    gemm = {}
    for i, name in enumerate(("qkv", "o", "gate_up", "down")):
        t = float(cls_ms[i]) * 1e-3
        flops = 2.0 * chunk * float(cls_bytes[i]) / 0.625   # Q4_1: 0.625 bytes per weight
        gemm[name] = {"us_per_launch": round(t * 1e6, 2), "gbs": round(float(cls_bytes[i]) / t / 1e9, 1),
                      "tflops_useful_bf16": round(flops / t / 1e12, 1),
                      "frac_of_mfma_peak": round(flops / t / 2.5e15, 4)}
    log(f"per-class GEMM at {chunk} rows: " + ", ".join(f"{k} {v['us_per_launch']} us ({v['gbs']} GB/s, "
                                                         f"{v['tflops_useful_bf16']} TFLOP/s)" for k, v in gemm.items()))
    res = {
        "metric": "chunked prefill tokens/s (64-row batched passes)",
        "value": round(args.prefill / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded draws, seed {args.seed})",
        "config": {"workload": f"prefill of {args.prefill} tokens on {args.ctx} cached positions, target {m.n_layers} "
                               f"layers hidden {m.hidden} Q4_1, chunks of {chunk} rows",
                   "kv_planes": ("bf16" if args.kv_bf16 else "fp32") + (", ring" if args.kv_ring else ""),
                   "ple_dim": args.ple_dim},
        "ms": round(ms, 3),
        "chunks": n_chunks,
        "ms_per_chunk": round(ms / n_chunks, 4),
        "gemm_64_rows": gemm,
        "snapshot_ms": {"positions": args.ctx + args.prefill, "mb": round(snap_mb, 1), "take": round(take_ms, 3),
                        "update": round(update_ms, 3), "restore": round(restore_ms, 3)},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--k", type=int, default=8)
    ap.add_argument("--ctx", type=int, default=1024)
    ap.add_argument("--layers", type=int, default=42, help="decoder layers (42 = the workload)")
    ap.add_argument("--vocab", type=int, default=262144)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--prefill", type=int, default=0,
                    help="instead of the verify step: chunked prefill of this many prompt tokens")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: the step (or the loop) uses the sampled accept at this temperature instead of greedy")
    ap.add_argument("--cpu-budget-s", type=float, default=25.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-bf16", action="store_true", help="K/V planes hold bf16 values (half the plane bytes)")
    ap.add_argument("--kv-ring", action="store_true",
                    help="the verify model's own sliding planes are rings of window + 16 slots")
    ap.add_argument("--ple-dim", type=int, default=0,
                    help="> 0: the verify model runs per-layer embeddings of this width (vocab x layers x width table)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the captured verify pass (and draft block) from HIP graphs; the default is direct "
                         "launches, measured faster on MI355X (k = 8 step 2.498 vs 2.511-2.515 ms, loop 1618-1620 vs "
                         "1594-1597 tokens/s, same box)")
    ap.add_argument("--no-graph", action="store_true", help="direct launches (the default; overrides --graph)")
    ap.add_argument("--loop", type=int, default=0,
                    help="instead of the verify step: the speculative loop (draft block of 8 + batched verify + "
                         "accept + commit) until this many tokens, steered acceptance, full-size draft and target")
    ap.add_argument("--draft", action="store_true",
                    help="instead of the verify step: the draft block forward alone at its real size (1 and 8 new "
                         "context rows), ms per block and bytes over time")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run a plain fp32 copy kernel (neg) of this many MiB three times first: the known-size "
                         "dispatch that scales HBM counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus}: this benchmark runs the verify pass on one GPU only; "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_verify_forward_amd import bvf, synth

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    if args.loop > 0:
        return run_loop(args)
    if args.draft:
        return run_draft(args)
    if args.prefill > 0:
        return run_prefill(args)
    threads = min(16, os.cpu_count() or 8)
    m = planes(synth.target_model(max_ctx=args.ctx + 64, n_layers=args.layers, vocab=args.vocab), args)
    t0 = time.time()
    w = build_weights(m, args.seed, threads)
    kv = synth.make_kv(m, args.ctx, args.seed)
    log(f"synthetic weights and context drawn in {time.time() - t0:.1f} s")
    t0 = time.time()
    g = bvf.Model(m)
    g.load_weights(w)
    g.set_context(kv, args.ctx)
    if args.graph and not args.no_graph:
        g.set_graph_mode(True)
    torch.cuda.synchronize()
    log(f"loaded and packed on the GPU in {time.time() - t0:.1f} s; arena {g.arena.numel() / 2**30:.2f} GiB")

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: 3 x neg over {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")

    k, V, H, T = args.k, m.vocab, m.hidden, len(m.tap_layers)
    toks_h = synth.tokens(args.seed, "bench.tokens", k, V)
    toks = torch.from_numpy(toks_h).cuda()
    logits = torch.empty((k, V), dtype=torch.float32, device="cuda")
    taps = torch.empty((k, T, H), dtype=torch.int16, device="cuda")
    out_tok = torch.zeros(k, dtype=torch.int32, device="cuda")
    n_acc = torch.zeros(1, dtype=torch.int32, device="cuda")

    n_steps = [0]

    def step(tk, lg, tp):
        g.verify_batch(tk, lg, tp)
        if args.temperature > 0:
            g.accept_sampled(lg, tk, out_tok, n_acc, args.temperature, args.seed, n_steps[0])
            n_steps[0] += 1
        else:
            g.accept_greedy(lg, tk, out_tok, n_acc)
        g.commit_verify_rows(0)

    def timed(nsteps, tk, lg, tp):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(nsteps):
            step(tk, lg, tp)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / nsteps

    for _ in range(args.warmup):
        step(toks, logits, taps)
    ms = timed(args.steps, toks, logits, taps)
    log(f"k={k}: {ms:.3f} ms per step")
    assert g.positions_held() == args.ctx

    # k = 1 step (same kernels, one row)
    toks1 = toks[:1].contiguous()
    lg1 = torch.empty((1, V), dtype=torch.float32, device="cuda")
    tp1 = torch.empty((1, T, H), dtype=torch.int16, device="cuda")
    for _ in range(2):
        step(toks1, lg1, tp1)
    ms1 = timed(max(3, args.steps // 2), toks1, lg1, tp1)
    log(f"k=1: {ms1:.3f} ms per step")

    # per-class GEMM timing with HIP events on the model's stream (the launches of the pass)
    cls_ms, cls_bytes = g.time_gemms(k, 3)
    cls_ms = [float(v) for v in cls_ms]
    cls_bytes = [int(v) for v in cls_bytes]
    names = ["qkv", "o", "gate_up", "down", "head"]
    per_pass = [m.n_layers] * 4 + [1]
    cls_total_ms = [cls_ms[i] * per_pass[i] for i in range(5)]
    q4_ms = sum(cls_total_ms[:4])
    q4_bytes, head_bytes = g.pass_bytes()
    q4_gbs = q4_bytes / (q4_ms * 1e-3) / 1e9
    dom = int(np.argmax(cls_total_ms[:4]))
    cls_gbs = [float(cls_bytes[i] / (cls_ms[i] * 1e-3) / 1e9) for i in range(5)]
    # the Q4_1 GEMM kernel over its 4 n_layers launches of a pass: bytes per launch and the average
    # launch duration (q|k|v, o, gate|up, down of every layer)
    n_q4_launches = 4 * m.n_layers
    q4_launch_bytes = q4_bytes / n_q4_launches
    q4_launch_ms = q4_ms / n_q4_launches
    log("per-class GEMM ms/launch: " + ", ".join(f"{names[i]} {cls_ms[i]:.4f} ({cls_bytes[i] / cls_ms[i] / 1e6:.0f} GB/s)"
                                                  for i in range(5)))

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(m, w, kv, args.ctx, toks_h, args.cpu_budget_s)
        log(f"cpu baseline in {time.time() - t0:.1f} s: {cpu}")

    rows_s = k / (ms * 1e-3)
    res = {
        "metric": METRIC,
        "value": round(rows_s, 1),
        "unit": "verified rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded draws, seed 0)",
        "config": {"workload": f"target-shaped verify: {m.n_layers} layers, hidden {H}, Q4_1, head {V}x{H} bf16, "
                               f"{args.ctx} cached positions, k={k}",
                   "arithmetic": "Q4_1 weights (codes exact in bf16), bf16 x bf16 -> fp32 MFMA, fp32 residual, "
                                 "norms and softmax",
                   "k": k, "cached_positions": args.ctx, "layers": m.n_layers, "vocab": V,
                   "accept": "greedy" if args.temperature <= 0 else f"sampled, T={args.temperature}",
                   "kv_planes": ("bf16" if args.kv_bf16 else "fp32") + (", ring" if args.kv_ring else ""),
                   "ple_dim": args.ple_dim,
                   "launches": "graph replay" if args.graph and not args.no_graph else "direct"},
        "q4_1_weight_stream_gbs": round(q4_gbs, 1),
        "q4_1_weight_stream_frac_of_peak": round(q4_gbs / HBM_PEAK_GBS, 4),
        "q4_1_bytes_per_pass": q4_bytes,
        "head_bytes_per_pass": head_bytes,
        "pass_gbs_all_weights": round((q4_bytes + head_bytes) / (ms * 1e-3) / 1e9, 1),
        "k1_ms_per_step": round(ms1, 4),
        "k8_over_k1": round(ms / ms1, 4),
        "gemm_ms_per_launch": {names[i]: round(float(cls_ms[i]), 5) for i in range(5)},
        "gemm_gbs": {names[i]: round(float(cls_bytes[i] / (cls_ms[i] * 1e-3) / 1e9), 1) for i in range(5)},
        "gemm_alg_bytes": {names[i]: cls_bytes[i] for i in range(5)},
        "roofline": {"bound": "hbm",
                     "kernel": f"Q4_1 GEMM (k_gemm), all {n_q4_launches} launches of a pass: "
                               f"{q4_launch_bytes / 1e6:.2f} MB per launch in {q4_launch_ms * 1e3:.2f} us on average",
                     "achieved": round(q4_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(q4_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("all"),
                     "classes": {names[i]: {"achieved": round(cls_gbs[i], 1), "frac": round(cls_gbs[i] / HBM_PEAK_GBS, 4),
                                            "us_per_launch": round(cls_ms[i] * 1e3, 2),
                                            "traffic": measured_traffic(names[i])} for i in range(4)},
                     "dominant_class": names[dom]},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
