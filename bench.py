#!/usr/bin/env python3
"""RMA-layer decode benchmark on one MI355X.

One step = one decode token through the whole RMA stack: for each of the 8
layers, the local-ring read, the anchor-bank read, the signed gate, the
ring write and the pending append; plus, every 256 tokens, the admit of
all layers.  Workload: 512 sequences, state pre-filled as after a 32K
prompt (ring and bank full), synthetic N(0,1)/16 bf16 inputs from a
device-resident pool of 16 input sets per layer (the pool changes none of
the state traffic).  Prints ONE JSON line: the headline decode figure with
its HBM roofline and the CPU oracle beside it, plus the admit round, the
same batch with per-sequence positions and with a separate anchor query,
batch-1 token latency (eager and HIP-graph replay) and the MFMA prefill
block at batch 1 and 8.

    python bench.py [--gpus 1] [--steps 1024] [--warmup 16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
POOL = 16                  # input sets per layer kept on the device

# Algorithmic bytes of one (sequence, layer, group) decode step.
#   read : ring K/V 1,023 x 1,024 B, bank K/V 1,024 x 1,024 B,
#          q of 4 heads 2,048 B, current K/V 1,024 B, candidate K/V 1,024 B
#          + score 4 B
#   write: out of 4 heads 2,048 B, ring slot 1,024 B, pending slot 1,024 B
#          + score 4 B
RING_BYTES = 1023 * 1024
BANK_BYTES = 1024 * 1024
UNIT_READ = RING_BYTES + BANK_BYTES + 2048 + 1024 + 1028
UNIT_WRITE = 2048 + 1024 + 1028
UNIT_BYTES = UNIT_READ + UNIT_WRITE          # 2,104,328


# Sources that define the decode kernel; the committed counter summary is
# used only while their hash matches.
DECODE_SOURCES = ("rma_decode.hip", "rma_kernels.h", "rma_admit_unit.h")


def kernel_sources_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bounded_memory_decode_amd", "csrc")
    for name in DECODE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def make_state(w, seed, device):
    """RMA state of workload `w` on `device`, filled with seeded synthetic
    records drawn on the device (torch generator per tensor and layer)."""
    import torch
    from bounded_memory_decode_amd import rma, synth
    cfg = rma.config_default(layers=w.L, q_heads=w.H, kv_groups=w.G, head_dim=w.d,
                             window=w.R + 1, bank_cap=w.N, commit=w.C, scale=w.d ** -0.5)
    S = rma.State(cfg, w.B, device, start_pos=w.t0, bank_n=w.bank_n)
    filled = min(w.t0, w.R)
    for l in range(w.L):
        for name, kind, slots in (("ring_k", 1, w.R), ("ring_v", 2, w.R),
                                  ("bank_k", 3, w.N), ("bank_v", 4, w.N)):
            x = synth.torch_normal_bf16((1, w.B, w.G, slots, w.d), w.qkv_std, seed, device,
                                        (w.wid, synth.KIND[name], l))
            if name.startswith("ring") and filled < w.R:
                x[:, :, :, filled:] = 0
            if name.startswith("bank") and w.bank_n < w.N:
                x[:, :, :, w.bank_n:] = 0
            S.write(name, x.view(torch.int16), layers=slice(l, l + 1))
            del x
        sc = synth.torch_scores((1, w.B, w.G, w.N), w, seed, device, (w.wid, synth.KIND["bscore"], l))
        sc[..., w.bank_n:] = 0
        S.write("bscore", sc, layers=slice(l, l + 1))
        src = torch.arange(w.N, dtype=torch.int32, device=device).expand(1, w.B, w.G, w.N)
        S.write("bsrc", src, layers=slice(l, l + 1))
    zero16 = torch.zeros((), dtype=torch.int16, device=device)
    S.region_view("pend_k").fill_(zero16)
    S.region_view("pend_v").fill_(zero16)
    S.region_view("pscore").zero_()
    torch.cuda.synchronize(device)
    return S


def make_pool(w, seed, device, pool=POOL):
    """Per layer, `pool` sets of step inputs and the gate weights."""
    import torch
    from bounded_memory_decode_amd import synth
    sets = []
    for l in range(w.L):
        per = []
        for p in range(pool):
            key = lambda kind: (w.wid, synth.KIND[kind], l, p, 1)
            per.append({
                "q": synth.torch_normal_bf16((w.B, w.H, w.d), w.qkv_std, seed, device, key("q")),
                "k": synth.torch_normal_bf16((w.B, w.G, w.d), w.qkv_std, seed, device, key("k")),
                "v": synth.torch_normal_bf16((w.B, w.G, w.d), w.qkv_std, seed, device, key("v")),
                "ck": synth.torch_normal_bf16((w.B, w.G, w.d), w.qkv_std, seed, device, key("ck")),
                "cv": synth.torch_normal_bf16((w.B, w.G, w.d), w.qkv_std, seed, device, key("cv")),
                "cs": synth.torch_scores((w.B, w.G), w, seed, device, key("cs")),
            })
        sets.append(per)
    g = torch.Generator(device=device)
    g.manual_seed(seed * 7919 + w.wid)
    wg = (torch.randn((w.L, w.H, w.d), generator=g, device=device) * w.w_std).contiguous()
    outs = [torch.empty((w.B, w.H, w.d), dtype=torch.bfloat16, device=device) for _ in range(w.L)]
    return sets, wg, outs


def run_step(S, sets, wg, outs, step, events=None, admit_events=None):
    """One token through all layers (+ admit at the block end)."""
    L = S.cfg.layers
    for l in range(L):
        x = sets[l][step % len(sets[l])]
        if events is not None:
            events[l][0].record()
        S.decode_step(l, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[l], outs[l])
        if events is not None:
            events[l][1].record()
    if S.pend_n[0] == S.cfg.commit:
        if admit_events is not None:
            admit_events.append((_event(), _event()))
            admit_events[-1][0].record()
        S.admit(-1)
        if admit_events is not None:
            admit_events[-1][1].record()
        return True
    return False


def _event():
    import torch
    return torch.cuda.Event(enable_timing=True)


# Prefill work of one 256-token block of one layer with a full ring and
# bank, masked work excluded: per group, 1,024 query rows (256 tokens x 4
# heads) each against 1,024 local keys and 1,024 anchors, QK and PV at
# 2 flop per multiply-add over 256 dims.
PREFILL_FLOP_PER_GROUP = 1024 * (1024 + 1024) * 256 * 2 * 2   # 2.147 GFLOP
MFMA_BF16_PEAK_TFLOPS = 2500.0
EVENT_EVERY = 8  # headline loop: steps between two steps with per-launch events


def bench_prefill(device, seed, batch, blocks):
    """Time rma_prefill_block on full-history states: `blocks` blocks of
    256 tokens through all 8 layers, admit after each block."""
    import torch
    from bounded_memory_decode_amd import synth
    w = synth.WORKLOADS["stack_b512"].with_(B=batch)
    S = make_state(w, seed, device)
    n = w.C
    ins = []
    for l in range(w.L):
        key = lambda kind: (w.wid, synth.KIND[kind], l, 99, 2)
        ins.append({
            "q": synth.torch_normal_bf16((w.B, n, w.H, w.d), w.qkv_std, seed, device, key("q")),
            "k": synth.torch_normal_bf16((w.B, n, w.G, w.d), w.qkv_std, seed, device, key("k")),
            "v": synth.torch_normal_bf16((w.B, n, w.G, w.d), w.qkv_std, seed, device, key("v")),
            "ck": synth.torch_normal_bf16((w.B, n, w.G, w.d), w.qkv_std, seed, device, key("ck")),
            "cv": synth.torch_normal_bf16((w.B, n, w.G, w.d), w.qkv_std, seed, device, key("cv")),
            "cs": synth.torch_scores((w.B, n, w.G), w, seed, device, key("cs")),
        })
    wg = (torch.randn((w.L, w.H, w.d), device=device) * w.w_std).contiguous()
    outs = [torch.empty((w.B, n, w.H, w.d), dtype=torch.bfloat16, device=device) for _ in range(w.L)]

    def block(ev=None):
        for l in range(w.L):
            x = ins[l]
            if ev is not None:
                ev[l][0].record()
            S.prefill_block(l, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[l], outs[l])
            if ev is not None:
                ev[l][1].record()
        S.admit(-1)

    block()  # warm-up
    torch.cuda.synchronize()
    evs = [[(_event(), _event()) for _ in range(w.L)] for _ in range(blocks)]
    for b in range(blocks):
        block(evs[b])
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for ev in evs for e0, e1 in ev]
    avg_ms = sum(ms) / len(ms)
    flop = PREFILL_FLOP_PER_GROUP * w.G * w.B
    tflops = flop / (avg_ms * 1e-3) / 1e12
    del S
    torch.cuda.empty_cache()
    return {"workload": f"{w.L} layers x batch {w.B}, 256-token blocks on a full ring and bank "
                        f"(position {w.t0})",
            "batch": w.B, "blocks": blocks, "us_per_block_layer": round(avg_ms * 1e3, 2),
            "prefill_tokens_per_s": round(w.B * n / (avg_ms * 1e-3 * w.L), 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "flop_per_launch": flop,
                         "kernel": "prefill_attn_kernel + prefill_commit_kernel (one layer, one block)"}}


def bench_latency(device, seed, steps, warmup):
    """One sequence, 8 layers, decoding after a 131,072-token prompt (ring
    and bank full): the token step launched call by call (lockstep calls,
    admit every 256 tokens) and the same step captured once in a HIP graph
    (per-sequence calls with the admit inside, plus the position increment)
    and replayed.  The state of one sequence (64 MiB) stays in the 256 MB
    last-level cache, so this is a latency figure, not an HBM one."""
    import torch
    from bounded_memory_decode_amd import synth
    w = synth.WORKLOADS["long_b1"].with_(t0=131072, bank_n=1024, ring_full=True)
    S = make_state(w, seed, device)
    sets, wg, outs = make_pool(w, seed, device, pool=4)
    for s in range(warmup):
        run_step(S, sets, wg, outs, s)
    torch.cuda.synchronize()
    e0, e1 = _event(), _event()
    e0.record()
    for s in range(steps):
        run_step(S, sets, wg, outs, warmup + s)
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / steps

    pos = torch.full((w.B,), S.t[0], dtype=torch.int32, device=device)
    x = [sets[l][0] for l in range(w.L)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(w.L):
            S.decode_step_at(l, pos, x[l]["q"], x[l]["k"], x[l]["v"], x[l]["ck"], x[l]["cv"],
                             x[l]["cs"], wg[l], outs[l])
        pos.add_(1)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / steps
    del graph, S
    torch.cuda.empty_cache()
    return {"workload": f"long_b1 decode: 1 sequence x {w.L} layers after a {w.t0}-token prompt "
                        f"(ring and bank full)",
            "steps": steps,
            "eager_us_per_token": round(eager_us, 2),
            "graph_us_per_token": round(graph_us, 2),
            "graph_tokens_per_s": round(1e6 / graph_us, 1),
            "graph": "8 x rma_decode_step_at (attention, combine, admit-if-block-end) + "
                     "position increment, captured once"}


def bench_staggered(S, w, sets, wg, outs, steps):
    """The headline batch with every sequence at its own offset inside the
    256-token block (sequence b at t + b mod 256): per-sequence calls, so
    each step admits the sequences whose block ends there, one layer at a
    time, instead of all of them every 256th step."""
    import torch
    t = S.t[0]
    pos = (t + torch.arange(w.B, device=S.device, dtype=torch.int32) % w.C).to(torch.int32)
    e0, e1 = _event(), _event()
    torch.cuda.synchronize()
    e0.record()
    for s in range(steps):
        for l in range(w.L):
            x = sets[l][s % len(sets[l])]
            S.decode_step_at(l, pos, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[l],
                             outs[l])
        pos += 1
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    return {"workload": f"{w.name} with sequence b at block offset b mod {w.C} (per-sequence "
                        f"positions; every sequence admitted once per layer per {w.C} steps)",
            "steps": steps, "ms_per_step": round(ms / steps, 4),
            "tokens_per_s": round(w.B * steps / (ms * 1e-3), 1)}


def bench_anchor_query(S, w, sets, wg, outs, steps):
    """The headline batch through the per-sequence call with a separate
    anchor query (the anchor read and the gate use q_anchor; here the q of
    another input set of the pool), every sequence at the same position."""
    import torch
    pos = torch.full((w.B,), S.t[0], dtype=torch.int32, device=S.device)
    e0, e1 = _event(), _event()
    ev = [(_event(), _event()) for _ in range(steps * w.L)]
    torch.cuda.synchronize()
    e0.record()
    for s in range(steps):
        for l in range(w.L):
            x = sets[l][s % len(sets[l])]
            qa = sets[l][(s + 1) % len(sets[l])]["q"]
            ev[s * w.L + l][0].record()
            S.decode_step_at(l, pos, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[l],
                             outs[l], q_anchor=qa)
            ev[s * w.L + l][1].record()
        pos += 1
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    launch_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    return {"workload": f"{w.name} through rma_decode_step_at with a separate anchor query",
            "steps": steps, "ms_per_step": round(ms / steps, 4),
            "tokens_per_s": round(w.B * steps / (ms * 1e-3), 1),
            "decode_launch_us": round(launch_ms * 1e3, 1),
            "GBps": round(w.B * w.G * (UNIT_BYTES + 2048) / (launch_ms * 1e-3) / 1e9, 1)}


def cpu_baseline(S, w, sets, wg, sample_b: int, seed: int, steps: int = 8):
    """The oracle, timed on the host cores on a bounded sample: `sample_b`
    sequences of the same state, `steps` tokens through all layers."""
    import numpy as np
    import torch
    import oracle
    from oracle import OracleState
    b_idx = list(range(sample_b))
    o = OracleState(L=w.L, B=sample_b, H=w.H, G=w.G, d=w.d, R=w.R, N=w.N, C=w.C,
                    scale=float(S.cfg.scale))
    for name in ("ring_k", "ring_v", "bank_k", "bank_v", "pend_k", "pend_v"):
        getattr(o, name)[...] = S.read(name, batch=b_idx).cpu().numpy().view(np.uint16)
    for name in ("bscore", "bsrc", "pscore", "bank_n"):
        getattr(o, name)[...] = S.read(name, batch=b_idx).cpu().numpy()
    o.t[:] = S.t[:w.L]
    o.pend_n[:] = S.pend_n[:w.L]
    ins = [[{k: (v[:sample_b].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                 if v.dtype == torch.bfloat16 else v[:sample_b].cpu().numpy())
             for k, v in sets[l][p].items()} for p in range(len(sets[l]))] for l in range(w.L)]
    wgn = wg.cpu().numpy()
    admits = 0
    t0 = time.perf_counter()
    for s in range(steps):
        for l in range(w.L):
            x = ins[l][s % len(ins[l])]
            o.decode_step(l, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wgn[l])
        if o.pend_n[0] == w.C:
            for l in range(w.L):
                o.admit(l)
            admits += 1
    dt = time.perf_counter() - t0
    cores = oracle.num_threads()
    return {"value": sample_b * steps / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{sample_b} of {w.B} sequences, {steps} tokens through all {w.L} layers "
                      f"(decode, ring write, pending append; {admits} admit rounds), "
                      f"{dt:.2f} s wall on {cores} threads"}


def read_traffic(sha: str):
    """HBM traffic per decode launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "decode_stack_b512_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha") != sha:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="stack_b512")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--repeats", type=int, default=3,
                    help="timed runs of --steps steps each; the median run is reported")
    ap.add_argument("--cpu-sample", type=int, default=64,
                    help="sequences in the CPU-oracle sample (0: skip)")
    ap.add_argument("--cpu-steps", type=int, default=32,
                    help="tokens per sequence in the CPU-oracle sample")
    ap.add_argument("--latency-steps", type=int, default=512,
                    help="batch-1 token steps timed eager and as graph replays (0: skip)")
    ap.add_argument("--staggered-steps", type=int, default=256,
                    help="steps of the per-sequence-position run at the headline batch (0: skip)")
    ap.add_argument("--anchor-steps", type=int, default=64,
                    help="steps with a separate anchor query at the headline batch (0: skip)")
    ap.add_argument("--prefill-blocks", type=int, default=4,
                    help="256-token blocks timed per prefill batch size (0: skip)")
    ap.add_argument("--calibration-copy-gib", type=int, default=0,
                    help="before timing, copy a buffer of this many GiB three times "
                         "(a plain copy kernel of known size, for scaling HBM counters)")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the RMA state of a sequence never leaves its GPU, "
              f"so --gpus {args.gpus} is not a supported configuration (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from bounded_memory_decode_amd import rma, synth
    rma.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    w = synth.WORKLOADS[args.workload]

    def say(m):
        if not args.quiet:
            print(m, file=sys.stderr, flush=True)

    say(f"[bench] building state: {w.name} B={w.B} L={w.L}")
    S = make_state(w, args.seed, device)
    sets, wg, outs = make_pool(w, args.seed, device)
    if args.calibration_copy_gib > 0:
        n = args.calibration_copy_gib << 30
        src = torch.ones(n, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        say(f"[bench] calibration copy: 3 x {n} bytes")
        del src, dst
    say(f"[bench] state {S.buf.numel() / 2**30:.2f} GiB; warmup {args.warmup} steps")
    for s in range(args.warmup):
        run_step(S, sets, wg, outs, s)
    torch.cuda.synchronize()

    K = args.steps
    runs = []
    step0 = args.warmup
    # Per-launch events on every EVENT_EVERY-th step only: each event is a
    # marker packet on the stream, and events around all 8 launches of
    # every step cost about 0.9% of the step time on MI355X (measured).
    sampled = [s for s in range(K) if s % EVENT_EVERY == 0]
    for r in range(max(1, args.repeats)):
        ev = [[(_event(), _event()) for _ in range(w.L)] if s % EVENT_EVERY == 0 else None
              for s in range(K)]
        start, stop = _event(), _event()
        say(f"[bench] timing {K} steps (run {r + 1})")
        admits = 0
        admit_ev = []
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        start.record()
        for s in range(K):
            admits += run_step(S, sets, wg, outs, step0 + s, ev[s], admit_ev)
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_wall
        step0 += K
        ms_total = start.elapsed_time(stop)
        dec_ms = [ev[s][l][0].elapsed_time(ev[s][l][1]) for s in sampled for l in range(w.L)]
        runs.append({"ms_total": ms_total, "dec_avg_ms": sum(dec_ms) / len(dec_ms),
                     "admits": admits, "admit_ev": admit_ev, "wall": wall})
        say(f"[bench] run {r + 1}: {w.B * K / (ms_total * 1e-3):,.0f} tok/s, decode launch "
            f"{runs[-1]['dec_avg_ms'] * 1e3:.1f} us")
    med = sorted(runs, key=lambda x: x["ms_total"])[len(runs) // 2]
    ms_total, dec_avg_ms, admits = med["ms_total"], med["dec_avg_ms"], med["admits"]
    admit_ev, wall = med["admit_ev"], med["wall"]
    ms_step = ms_total / K

    units = w.B * w.G
    launch_bytes = units * UNIT_BYTES
    step_bytes = launch_bytes * w.L
    achieved = launch_bytes / (dec_avg_ms * 1e-3) / 1e9
    tokens_s = w.B * K / (ms_total * 1e-3)
    sha = kernel_sources_sha()
    traffic = read_traffic(sha)

    result = {
        "metric": "RMA-layer decode tokens/s at batch 512x8 layers; achieved HBM GB/s vs peak",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: RMA stack, {w.L} layers x batch {w.B}, 16 q heads, "
                               f"4 KV groups, head_dim 256, ring 1023 + current, bank 1024, "
                               f"commit 256, start position {w.t0} (ring and bank full)",
                   "batch": w.B, "layers": w.L, "admit_rounds": admits,
                   "runs": len(runs), "run_tokens_per_s": [round(w.B * K / (x["ms_total"] * 1e-3), 1)
                                                          for x in runs],
                   "step_bytes_algorithmic": step_bytes,
                   "step_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "decode_attn_kernel<true, false, 1>: the whole decode step of one layer "
                               "(one launch at this batch)",
                     "avg_launch_ms": round(dec_avg_ms, 5),
                     "launches_timed": len(sampled) * w.L,
                     "bytes_per_launch": launch_bytes,
                     "kernel_sources_sha": sha},
        "cpu_baseline": None,
    }
    if admit_ev:
        adm_ms = [a.elapsed_time(b) for a, b in admit_ev]
        result["admit"] = {"workload": f"all {w.L} layers x batch {w.B} x 4 groups: top-1024 of "
                                       f"1024 anchors + 256 candidates each",
                           "rounds": len(adm_ms), "ms_per_round": round(sum(adm_ms) / len(adm_ms), 4),
                           "selections_per_s": round(w.L * w.B * w.G / (sum(adm_ms) / len(adm_ms) * 1e-3))}
    say(f"[bench] {tokens_s:,.0f} tok/s, {ms_step:.3f} ms/step, decode launch {dec_avg_ms*1e3:.1f} us "
        f"= {achieved:,.0f} GB/s ({100*achieved/HBM_PEAK_GBS:.1f}% of peak); wall {wall:.2f} s")
    if args.cpu_sample > 0:
        say(f"[bench] CPU oracle on {args.cpu_sample} sequences x {args.cpu_steps} tokens")
        result["cpu_baseline"] = cpu_baseline(S, w, sets, wg, args.cpu_sample, args.seed,
                                              args.cpu_steps)
    if args.staggered_steps > 0:
        say(f"[bench] per-sequence positions, {args.staggered_steps} steps")
        result["staggered"] = bench_staggered(S, w, sets, wg, outs, args.staggered_steps)
        say(f"[bench] staggered: {result['staggered']['tokens_per_s']:,.0f} tok/s")
    if args.anchor_steps > 0:
        say(f"[bench] separate anchor query, {args.anchor_steps} steps")
        result["anchor_query"] = bench_anchor_query(S, w, sets, wg, outs, args.anchor_steps)
        say(f"[bench] anchor query: {result['anchor_query']['tokens_per_s']:,.0f} tok/s, decode "
            f"launch {result['anchor_query']['decode_launch_us']} us")
    del S, sets, outs
    torch.cuda.empty_cache()
    if args.latency_steps > 0:
        say(f"[bench] batch-1 latency, {args.latency_steps} steps")
        result["latency"] = bench_latency(device, args.seed, args.latency_steps, 16)
        say(f"[bench] batch 1: eager {result['latency']['eager_us_per_token']} us/token, "
            f"graph {result['latency']['graph_us_per_token']} us/token")
    if args.prefill_blocks > 0:
        torch.cuda.empty_cache()
        result["prefill"] = []
        for pb in (1, 8):
            say(f"[bench] prefill, batch {pb}")
            r = bench_prefill(device, args.seed, pb, args.prefill_blocks)
            say(f"[bench] prefill batch {pb}: {r['us_per_block_layer']} us per block-layer, "
                f"{r['roofline']['achieved']} TFLOP/s ({100 * r['roofline']['frac']:.1f}% of bf16 MFMA peak)")
            result["prefill"].append(r)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
