#!/usr/bin/env python3
"""RMA-layer decode benchmark on one MI355X.

One step = one decode token through the whole RMA stack: for each of the 8
layers, the local-ring read, the anchor-bank read, the signed gate, the
ring write and the pending append; plus, every 256 tokens, the admit of
all layers.  Workload: 512 sequences, state pre-filled as after a 32K
prompt (ring and bank full), synthetic N(0,1)/16 bf16 inputs from a
device-resident pool of 16 input sets per layer (the pool changes none of
the state traffic).  The timed window always ends with a step that
completes a block, so it contains at least one admit of all layers.

Prints ONE JSON line: the headline decode figure with its HBM roofline, a
streaming-read calibration and the CPU oracle beside it, plus
  admit_stress  one all-layer admit with scores on 64 levels (heavy ties);
  staggered     the same batch with per-sequence positions;
  anchor_query  the same batch with a separate anchor query;
  long          one sequence: a 131,072-token prompt in 256-token prefill
                blocks (admit after each), then decode as HIP-graph replays;
  layers        one layer at batch 1 and 64 through its whole decode run
                (512 and 2,048 steps with their admits), eager and as graph
                replays;
  prefill       the MFMA prefill block at batch 1 and 8.

    python bench.py [--gpus 1] [--steps 1024] [--warmup 16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
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

# Algorithmic bytes of one (sequence, layer, group) admit, given n anchors,
# C candidates and m records moved: read n + C scores; for each moved
# record read its K/V (1,024 B) and score; write its K/V, score and source
# position into the bank; write the bank count.
REC_BYTES = 1024


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


def run_step(S, sets, wg, outs, step, admit_events=None):
    """One token through all layers (+ admit at the block end)."""
    L = S.cfg.layers
    for l in range(L):
        x = sets[l][step % len(sets[l])]
        S.decode_step(l, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[l], outs[l])
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


def _median(xs):
    s = sorted(xs)
    return s[len(s) // 2]


# Prefill work of one 256-token block of one layer with a full ring and
# bank, masked work excluded: per group, 1,024 query rows (256 tokens x 4
# heads) each against 1,024 local keys and 1,024 anchors, QK and PV at
# 2 flop per multiply-add over 256 dims.
PREFILL_FLOP_PER_GROUP = 1024 * (1024 + 1024) * 256 * 2 * 2   # 2.147 GFLOP
MFMA_BF16_PEAK_TFLOPS = 2500.0


def _time_stream(rma, buf, waves, sink, reps, warm):
    """Best and median ms of `reps` timed streaming reads of `buf`."""
    import torch
    for _ in range(warm):
        rma.calib_stream_read(buf, waves, sink)
    ms = []
    for _ in range(reps):
        e0, e1 = _event(), _event()
        e0.record()
        rma.calib_stream_read(buf, waves, sink)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return min(ms), _median(ms)


def bench_calibration(device, gib=8, waves=1024, reps=9, warm=3, launch_bytes=None):
    """Achievable read bandwidth: rma_calib_stream_read (a streaming-read
    kernel of this library, 16-byte non-temporal loads, 16 in flight per
    lane) over a `gib` GiB buffer with `waves` waves (the decode kernel's
    resident wave count).  `warm` untimed passes, then `reps` passes timed
    with events; the best pass is the achievable figure (the median is
    listed beside it).  Run first, before the state is allocated: after a
    minute of load it read up to 6% lower on the same box.  With
    `launch_bytes`, the same probe also reads a prefix of the buffer of
    that size (rounded up to the probe's granularity): a launch as long as
    the decode's, whose ramp-up and tail weigh as much as the decode's do."""
    import torch
    from bounded_memory_decode_amd import rma
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device=device)
    buf.fill_(1)
    sink = torch.empty(waves, dtype=torch.int32, device=device)
    best, med = _time_stream(rma, buf, waves, sink, reps, warm)
    r = {"kernel": "stream_read_kernel (rma_calib_stream_read): every wave reads its own "
                   "contiguous share with 16-byte non-temporal loads",
         "bytes": n, "waves": waves, "passes": reps, "ms": round(best, 4),
         "GBps": round(n / (best * 1e-3) / 1e9, 1),
         "median_GBps": round(n / (med * 1e-3) / 1e9, 1)}
    if launch_bytes:
        gran = waves * 16 * 1024
        nb = min(n, -(-launch_bytes // gran) * gran)
        lb, lm = _time_stream(rma, buf[:nb], waves, sink, reps, warm)
        r["launch_size"] = {"bytes": nb, "ms": round(lb, 4),
                            "GBps": round(nb / (lb * 1e-3) / 1e9, 1),
                            "median_GBps": round(nb / (lm * 1e-3) / 1e9, 1)}
    del buf, sink
    torch.cuda.empty_cache()
    return r


def bench_admit_stress(S, w, seed, reps=5):
    """Config of the admit stress: every (sequence, layer, group) of the
    headline state gets a full pending buffer and scores on 64 levels
    (integers 0..63, so ties straddle the cut in nearly every group), then
    one admit of all layers is timed; the bank metadata is restored
    between passes.  Moved records are counted from the result."""
    import torch
    from bounded_memory_decode_amd import synth
    ws = synth.WORKLOADS["admit_b512"].with_(B=w.B, L=w.L)
    dev = S.device
    C, N = w.C, w.N
    # a block-aligned position for the lockstep admit; source positions
    # 0 .. N-1 for the anchors, so that every record the admit moves in
    # (source position >= the block start > N) can be counted
    t_al = (S.t[0] // C + 1) * C
    S.region_view("bsrc").copy_(torch.arange(N, dtype=torch.int32, device=dev).expand(
        w.L, w.B, w.G, N))
    for l in range(w.L):
        sc = synth.torch_scores((1, w.B, w.G, N), ws, seed, dev, (ws.wid, synth.KIND["bscore"], l))
        S.write("bscore", sc, layers=slice(l, l + 1))
        ps = synth.torch_scores((1, w.B, w.G, C), ws, seed, dev, (ws.wid, synth.KIND["pscore"], l))
        S.write("pscore", ps, layers=slice(l, l + 1))
        for name in ("pend_k", "pend_v"):
            x = synth.torch_normal_bf16((1, w.B, w.G, C, w.d), ws.qkv_std, seed, dev,
                                        (ws.wid, synth.KIND[name], l))
            S.write(name, x.view(torch.int16), layers=slice(l, l + 1))
    saved = {k: S.region_view(k).clone() for k in ("bscore", "bsrc", "bank_n")}
    n_before = S.region_view("bank_n").to(torch.int64)
    host_n = list(S.bank_n)
    ms = []
    moved = None
    for r in range(reps):
        for k, v in saved.items():
            S.region_view(k).copy_(v)
        for l in range(w.L):
            S._st.t[l] = t_al
            S._st.pend_n[l] = C
            S._st.bank_n[l] = host_n[l]
        torch.cuda.synchronize()
        e0, e1 = _event(), _event()
        e0.record()
        S.admit(-1)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
        if moved is None:
            moved = int((S.region_view("bsrc") >= N).sum().item())
    m = _median(ms)
    units = w.L * w.B * w.G
    nsum = int(n_before.sum().item())
    bytes_round = (nsum + units * C) * 4 + moved * (REC_BYTES + 4) + moved * (REC_BYTES + 8) + \
        units * 4
    return {"workload": f"admit_b512: {w.L} layers x batch {w.B} x {w.G} groups, each the top "
                        f"{N} of {N} anchors + {C} candidates, scores integers 0..63 (heavy ties)",
            "selections": units, "passes": reps, "ms_per_round": round(m, 4),
            "selections_per_s": round(units / (m * 1e-3)),
            "records_moved": moved, "bytes_per_round": bytes_round,
            "roofline": {"bound": "hbm", "achieved": round(bytes_round / (m * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(bytes_round / (m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "kernel": "admit_kernel"}}


def sdpa_reference(device, batch, reps=20):
    """Yardstick for the prefill roofline: torch's own fused attention
    (scaled_dot_product_attention, flash backend) on a dense problem of the
    same algorithmic flop as one block-layer at this batch: per sequence 16
    heads x 256 queries against 2,048 keys, head_dim 256, no mask, each
    head with its own K/V rows (so the flop equals the block's 1,024 query
    rows x 2,048 keys per group).  Measurement only; nothing on the
    library's path uses it.  None where the backend is unavailable."""
    import torch
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        g = torch.Generator(device=device)
        g.manual_seed(7)
        H, T, S, D = 16, 256, 2048, 256
        q, k, v = ((torch.randn((batch, H, n, D), generator=g, device=device) / 16)
                   .to(torch.bfloat16).contiguous() for n in (T, S, S))
        f = torch.nn.functional.scaled_dot_product_attention
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            for _ in range(3):
                f(q, k, v)
            torch.cuda.synchronize()
            e0, e1 = _event(), _event()
            e0.record()
            for _ in range(reps):
                f(q, k, v)
            e1.record()
            torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
    except Exception as ex:  # backend missing on this build: report, do not fail the bench
        return {"kernel": "torch scaled_dot_product_attention (flash)", "error": str(ex)[:200]}
    flop = 4.0 * batch * H * T * S * D
    return {"kernel": "torch scaled_dot_product_attention (flash backend), bf16",
            "shape": f"batch {batch} x 16 heads x 256 queries x 2048 keys x head_dim 256, no mask",
            "flop": flop, "us": round(us, 2), "TFLOP/s": round(flop / us / 1e6, 2),
            "frac": round(flop / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)}


def bench_prefill(device, seed, batch, blocks):
    """Time rma_prefill_block on full-history states: `blocks` blocks of
    256 tokens through all 8 layers, admit after each block."""
    import torch
    from bounded_memory_decode_amd import synth
    w = synth.WORKLOADS["stack_b512"].with_(B=batch)
    S = make_state(w, seed, device)
    n = w.C
    ins = [synth.torch_block_inputs(w, seed, l, 99, device, sets=2) for l in range(w.L)]
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
    del S, ins, outs
    torch.cuda.empty_cache()
    ref = sdpa_reference(device, batch)
    return {"workload": f"{w.L} layers x batch {w.B}, 256-token blocks on a full ring and bank "
                        f"(position {w.t0})",
            "library_reference": ref,
            "batch": w.B, "blocks": blocks, "us_per_block_layer": round(avg_ms * 1e3, 2),
            "prefill_tokens_per_s": round(w.B * n / (avg_ms * 1e-3 * w.L), 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "flop_per_launch": flop,
                         "kernel": "prefill_attn_kernel + prefill_commit_kernel (one layer, one block)"}}


def bench_long(device, seed, prompt_blocks, decode_steps, eager_steps):
    """The long single-sequence path: one sequence, 8 layers, from an empty
    history.  A prompt of prompt_blocks x 256 tokens through
    rma_prefill_block (all layers admitted after every block), timed as a
    whole; then decode: `eager_steps` token steps launched call by call
    (lockstep calls, admit every 256 tokens), then `decode_steps` token
    steps as replays of one captured HIP graph (8 per-sequence calls with
    the admit inside, plus the position increment).  The state of one
    sequence (64 MiB) stays in the 256 MB last-level cache, so these are
    latency figures, not HBM ones."""
    import torch
    from bounded_memory_decode_amd import rma, synth
    w = synth.WORKLOADS["long_b1"]
    cfg = rma.config_default(layers=w.L)
    S = rma.State(cfg, 1, device, start_pos=0, bank_n=0)
    S.buf.zero_()
    ins = [[synth.torch_block_inputs(w, seed, l, p, device, sets=4) for p in range(4)]
           for l in range(w.L)]
    g = torch.Generator(device=device)
    g.manual_seed(seed * 7919 + w.wid)
    wg = (torch.randn((w.L, w.H, w.d), generator=g, device=device) * w.w_std).contiguous()
    pout = [torch.empty((1, w.C, w.H, w.d), dtype=torch.bfloat16, device=device)
            for _ in range(w.L)]
    torch.cuda.synchronize()
    e0, e1 = _event(), _event()
    e0.record()
    for blk in range(prompt_blocks):
        for l in range(w.L):
            x = ins[l][blk % 4]
            S.prefill_block(l, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[l], pout[l])
        S.admit(-1)
    e1.record()
    torch.cuda.synchronize()
    prompt_ms = e0.elapsed_time(e1)
    prompt_tokens = prompt_blocks * w.C

    # decode inputs: token i of the pool's blocks, per layer
    sets = [[{k: v[:, i].contiguous() for k, v in ins[l][i % 4].items()} for i in range(4)]
            for l in range(w.L)]
    outs = [torch.empty((1, w.H, w.d), dtype=torch.bfloat16, device=device) for _ in range(w.L)]
    e0.record()
    for s in range(eager_steps):
        run_step(S, sets, wg, outs, s)
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / max(1, eager_steps)

    pos = torch.full((1,), S.t[0], dtype=torch.int32, device=device)
    x = [sets[l][0] for l in range(w.L)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(w.L):
            S.decode_step_at(l, pos, x[l]["q"], x[l]["k"], x[l]["v"], x[l]["ck"], x[l]["cv"],
                             x[l]["cs"], wg[l], outs[l])
        pos.add_(1)
    for _ in range(16):
        graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(decode_steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / max(1, decode_steps)
    end_pos = int(pos.item())
    del graph, S
    torch.cuda.empty_cache()
    return {"workload": f"long_b1: 1 sequence x {w.L} layers from an empty history: a "
                        f"{prompt_tokens}-token prompt in {w.C}-token prefill blocks (all layers "
                        f"admitted after each block), then decode",
            "prompt_tokens": prompt_tokens, "prompt_ms": round(prompt_ms, 3),
            "prefill_tokens_per_s": round(prompt_tokens / (prompt_ms * 1e-3), 1),
            "us_per_block_layer_with_admit": round(prompt_ms * 1e3 / (prompt_blocks * w.L), 2),
            "eager_steps": eager_steps, "eager_us_per_token": round(eager_us, 2),
            "decode_steps": decode_steps, "graph_us_per_token": round(graph_us, 2),
            "decode_tokens_per_s": round(1e6 / graph_us, 1),
            "end_position": end_pos,
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
    another input set of the pool), every sequence at the same position,
    no block end inside the window."""
    import torch
    pos = torch.full((w.B,), S.t[0], dtype=torch.int32, device=S.device)
    e0, e1 = _event(), _event()
    torch.cuda.synchronize()
    e0.record()
    for s in range(steps):
        for l in range(w.L):
            x = sets[l][s % len(sets[l])]
            qa = sets[l][(s + 1) % len(sets[l])]["q"]
            S.decode_step_at(l, pos, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[l],
                             outs[l], q_anchor=qa)
        pos += 1
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    launch_ms = ms / (steps * w.L)
    return {"workload": f"{w.name} through rma_decode_step_at with a separate anchor query",
            "steps": steps, "ms_per_step": round(ms / steps, 4),
            "tokens_per_s": round(w.B * steps / (ms * 1e-3), 1),
            "decode_launch_us": round(launch_ms * 1e3, 1),
            "GBps": round(w.B * w.G * (UNIT_BYTES + 2048) / (launch_ms * 1e-3) / 1e9, 1)}


def bench_layer_config(device, seed, name):
    """One RMA layer at its own batch, from the pre-filled state (ring and
    bank full at position 32,768): the workload's full decode run, all its
    steps and admits, two ways on two copies of the state.
      eager: lockstep rma_decode_step per token, rma_admit at each block
             end (event pairs around the admits);
      graph: 16 captured token steps (rma_decode_step_at, which admits
             inside the call at a block end, plus the position increment;
             each step with its own input set of the pool), replayed
             steps / 16 times, so that the host's graph launch is shared
             by 16 tokens.
    Batch 1 keeps its whole state (8 MiB) in the 256 MB last-level cache,
    so its figures are latency; batch 64 (537 MB) and batch 288 (2.4 GB,
    decoded in two launches: whole units for 256 sequences, the split
    launch for 32) stream from HBM."""
    import torch
    from bounded_memory_decode_amd import synth
    w = synth.WORKLOADS[name]
    steps = w.steps
    S = make_state(w, seed, device)
    sets, wg, outs = make_pool(w, seed, device)
    torch.cuda.synchronize()
    adm = []
    e0, e1 = _event(), _event()
    e0.record()
    for s in range(steps):
        run_step(S, sets, wg, outs, s, adm)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1)
    adm_ms = [a.elapsed_time(b) for a, b in adm]
    dec_ms = (eager_ms - sum(adm_ms)) / (steps * w.L)
    del S
    torch.cuda.empty_cache()

    S = make_state(w, seed, device)
    per = 16
    pos = torch.full((w.B,), S.t[0], dtype=torch.int32, device=device)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(per):
            for l in range(w.L):
                x = sets[l][i % len(sets[l])]
                S.decode_step_at(l, pos, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"],
                                 wg[l], outs[l])
            pos.add_(1)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps // per):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1)
    end_pos = int(pos[0].item())
    del graph, S, sets, outs
    torch.cuda.empty_cache()
    launch_bytes = w.B * w.G * UNIT_BYTES
    r = {"workload": f"{name}: one RMA layer, batch {w.B}, {steps} decode steps from position "
                     f"{w.t0} (ring and bank full), {len(adm_ms)} admits",
         "batch": w.B, "steps": steps,
         "eager_tokens_per_s": round(w.B * steps / (eager_ms * 1e-3), 1),
         "eager_us_per_step": round(eager_ms * 1e3 / steps, 2),
         "eager_decode_launch_us": round(dec_ms * 1e3, 2),
         "admits": len(adm_ms),
         "admit_us": round(1e3 * sum(adm_ms) / max(1, len(adm_ms)), 2),
         "graph_tokens_per_s": round(w.B * (steps // per * per) / (graph_ms * 1e-3), 1),
         "graph_us_per_step": round(graph_ms * 1e3 / (steps // per * per), 2),
         "graph_steps_per_replay": per,
         "graph_end_position": end_pos,
         "bytes_per_launch": launch_bytes}
    if w.B > 1:
        gbs = launch_bytes / (dec_ms * 1e-3) / 1e9
        r["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "launch_time": "eager window minus its admits, per decode launch"}
        # the streaming-read probe over a launch of the same size (its ramp-up
        # and tail weigh as much as this short launch's do)
        gib = -(-launch_bytes // (1 << 30))
        probe = bench_calibration(device, gib, launch_bytes=launch_bytes)["launch_size"]
        r["roofline"]["stream_probe_same_size"] = probe
        r["roofline"]["frac_of_probe"] = round(gbs / probe["GBps"], 4)
    else:
        r["note"] = "state resident in the last-level cache: latency, not HBM bandwidth"
    return r


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(S, w, sets, wg, sample_b: int, steps: int, one_b: int, one_steps: int):
    """The oracle, timed on the host cores on a bounded sample of the same
    state: `sample_b` sequences, `steps` tokens through all layers with
    every thread, crossing a block end (so the admit is in the sample);
    then `one_b` sequences x `one_steps` tokens on one thread.  The state
    is copied to the host when S's layers stand a few tokens before a
    block end."""
    import numpy as np
    import torch
    import oracle
    from oracle import OracleState

    def load(nb):
        b_idx = list(range(nb))
        o = OracleState(L=w.L, B=nb, H=w.H, G=w.G, d=w.d, R=w.R, N=w.N, C=w.C,
                        scale=float(S.cfg.scale))
        for name in ("ring_k", "ring_v", "bank_k", "bank_v", "pend_k", "pend_v"):
            getattr(o, name)[...] = S.read(name, batch=b_idx).cpu().numpy().view(np.uint16)
        for name in ("bscore", "bsrc", "pscore", "bank_n"):
            getattr(o, name)[...] = S.read(name, batch=b_idx).cpu().numpy()
        o.t[:] = S.t[:w.L]
        o.pend_n[:] = S.pend_n[:w.L]
        return o

    def run(o, nb, n_steps):
        ins = [[{k: (v[:nb].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                     if v.dtype == torch.bfloat16 else v[:nb].cpu().numpy())
                 for k, v in sets[l][p].items()} for p in range(len(sets[l]))]
               for l in range(w.L)]
        wgn = wg.cpu().numpy()
        admits = 0
        t0 = time.perf_counter()
        for s in range(n_steps):
            for l in range(w.L):
                x = ins[l][s % len(ins[l])]
                o.decode_step(l, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wgn[l])
            if o.pend_n[0] == w.C:
                for l in range(w.L):
                    o.admit(l)
                admits += 1
        return time.perf_counter() - t0, admits

    cores = oracle.num_threads()
    dt, admits = run(load(sample_b), sample_b, steps)
    oracle.set_num_threads(1)
    try:
        dt1, admits1 = run(load(one_b), one_b, one_steps)
    finally:
        oracle.set_num_threads(cores)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"value": sample_b * steps / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{sample_b} of {w.B} sequences, {steps} tokens through all {w.L} layers "
                      f"(decode, ring write, pending append; {admits} admit round of all layers "
                      f"for these sequences), {dt:.2f} s wall on {cores} threads",
            "value_1_thread": one_b * one_steps / dt1,
            "sample_1_thread": f"{one_b} sequences, {one_steps} tokens through all {w.L} layers "
                               f"({admits1} admit rounds), {dt1:.2f} s wall on 1 thread",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": affinity}


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
    ap.add_argument("--calibration-gib", type=int, default=8,
                    help="GiB read by the streaming-read calibration (0: skip)")
    ap.add_argument("--admit-passes", type=int, default=5,
                    help="timed passes of the admit stress (0: skip)")
    ap.add_argument("--cpu-sample", type=int, default=64,
                    help="sequences in the CPU-oracle sample (0: skip)")
    ap.add_argument("--cpu-steps", type=int, default=32,
                    help="tokens per sequence in the CPU-oracle sample")
    ap.add_argument("--staggered-steps", type=int, default=256,
                    help="steps of the per-sequence-position run at the headline batch (0: skip)")
    ap.add_argument("--anchor-steps", type=int, default=64,
                    help="steps with a separate anchor query at the headline batch (0: skip)")
    ap.add_argument("--long-blocks", type=int, default=512,
                    help="256-token prompt blocks of the long single-sequence run (0: skip)")
    ap.add_argument("--long-decode", type=int, default=131072,
                    help="decode tokens (graph replays) after the long prompt")
    ap.add_argument("--long-eager", type=int, default=512,
                    help="decode tokens launched call by call before the graph replays")
    ap.add_argument("--prefill-blocks", type=int, default=4,
                    help="256-token blocks timed per prefill batch size (0: skip)")
    ap.add_argument("--layer-configs", type=int, default=1,
                    help="1: time the one-layer workloads at batch 1, 64 and 288 (0: skip)")
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

    cal = None
    if args.calibration_gib > 0:
        # first, on a device with nothing else allocated
        say(f"[bench] streaming-read calibration, {args.calibration_gib} GiB")
        cal = bench_calibration(device, args.calibration_gib,
                                launch_bytes=w.B * w.G * UNIT_BYTES)
        say(f"[bench] stream read: {cal['GBps']} GB/s; a launch of the decode's "
            f"{cal['launch_size']['bytes']:,} B: {cal['launch_size']['GBps']} GB/s")
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
    step = 0
    for _ in range(args.warmup):
        run_step(S, sets, wg, outs, step)
        step += 1
    K = args.steps
    C = w.C

    def align():
        """Untimed steps so that the next K steps end on a block end."""
        nonlocal step
        extra = (-(S.pend_n[0] + K)) % C
        for _ in range(extra):
            run_step(S, sets, wg, outs, step)
            step += 1
        return extra

    torch.cuda.synchronize()
    runs = []
    for r in range(max(1, args.repeats)):
        extra = align()
        torch.cuda.synchronize()
        start, stop = _event(), _event()
        say(f"[bench] timing {K} steps (run {r + 1}, after {extra} alignment steps)")
        admits = 0
        admit_ev = []
        t_wall = time.perf_counter()
        start.record()
        for s in range(K):
            admits += run_step(S, sets, wg, outs, step, admit_ev)
            step += 1
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_wall
        ms_total = start.elapsed_time(stop)
        adm_ms = [a.elapsed_time(b) for a, b in admit_ev]
        runs.append({"ms_total": ms_total, "admits": admits, "admit_ms": adm_ms, "wall": wall})
        dec = (ms_total - sum(adm_ms)) / (K * w.L)
        say(f"[bench] run {r + 1}: {w.B * K / (ms_total * 1e-3):,.0f} tok/s, {admits} admit "
            f"rounds, decode launch {dec * 1e3:.1f} us")
    med = sorted(runs, key=lambda x: x["ms_total"])[len(runs) // 2]
    ms_total, admits, adm_ms, wall = med["ms_total"], med["admits"], med["admit_ms"], med["wall"]
    ms_step = ms_total / K
    # decode launch time: the timed window minus its admits, per launch
    # (launch gaps included, so at most the kernel's own duration)
    dec_avg_ms = (ms_total - sum(adm_ms)) / (K * w.L)

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
                   "admit_ms_in_window": round(sum(adm_ms), 4),
                   "alignment": "untimed steps before each run so that the timed window ends on "
                                "a block end (every run holds at least one admit of all layers)",
                   "runs": len(runs), "run_tokens_per_s": [round(w.B * K / (x["ms_total"] * 1e-3), 1)
                                                          for x in runs],
                   "step_bytes_algorithmic": step_bytes,
                   "step_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1)},
        # the same run's decode launch time and admit round, with one admit
        # per C steps as in a long decode (a short window holds one admit in
        # K steps, more than its share)
        "amortized": None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "decode_attn_kernel<true, false, 1, false>: the whole decode step of one layer "
                               "(one launch at this batch)",
                     "avg_launch_ms": round(dec_avg_ms, 5),
                     "launch_time": "timed window minus its admit rounds, divided by the decode "
                                    "launches in it (gaps between launches included)",
                     "bytes_per_launch": launch_bytes,
                     "kernel_sources_sha": sha},
        "cpu_baseline": None,
    }
    if adm_ms:
        adm_round = sum(adm_ms) / len(adm_ms)
        amort_ms = w.L * dec_avg_ms + adm_round / C
        result["amortized"] = {"ms_per_step": round(amort_ms, 4),
                               "tokens_per_s": round(w.B / (amort_ms * 1e-3), 1),
                               "rule": f"{w.L} decode launches + one all-layer admit per {C} steps"}
        result["admit"] = {"workload": f"all {w.L} layers x batch {w.B} x 4 groups inside the timed "
                                       f"window: top-1024 of 1024 anchors + 256 candidates each",
                           "rounds": len(adm_ms),
                           "ms_per_round": round(sum(adm_ms) / len(adm_ms), 4),
                           "selections_per_s": round(w.L * w.B * w.G / (sum(adm_ms) / len(adm_ms) * 1e-3))}
    say(f"[bench] {tokens_s:,.0f} tok/s, {ms_step:.3f} ms/step, decode launch {dec_avg_ms*1e3:.1f} us "
        f"= {achieved:,.0f} GB/s ({100*achieved/HBM_PEAK_GBS:.1f}% of peak); wall {wall:.2f} s")
    if args.cpu_sample > 0:
        # stand a few tokens before a block end so that the sample holds an admit
        lead = min(8, args.cpu_steps)
        while (C - S.pend_n[0]) != lead:
            run_step(S, sets, wg, outs, step)
            step += 1
        torch.cuda.synchronize()
        say(f"[bench] CPU oracle on {args.cpu_sample} sequences x {args.cpu_steps} tokens, "
            f"then 1 thread")
        result["cpu_baseline"] = cpu_baseline(S, w, sets, wg, args.cpu_sample, args.cpu_steps,
                                              one_b=4, one_steps=lead + 2)
    if args.staggered_steps > 0:
        say(f"[bench] per-sequence positions, {args.staggered_steps} steps")
        result["staggered"] = bench_staggered(S, w, sets, wg, outs, args.staggered_steps)
        say(f"[bench] staggered: {result['staggered']['tokens_per_s']:,.0f} tok/s")
    if args.anchor_steps > 0:
        say(f"[bench] separate anchor query, {args.anchor_steps} steps")
        result["anchor_query"] = bench_anchor_query(S, w, sets, wg, outs, args.anchor_steps)
        say(f"[bench] anchor query: {result['anchor_query']['tokens_per_s']:,.0f} tok/s, decode "
            f"launch {result['anchor_query']['decode_launch_us']} us")
    if args.admit_passes > 0:
        say(f"[bench] admit stress, {args.admit_passes} passes")
        result["admit_stress"] = bench_admit_stress(S, w, args.seed, args.admit_passes)
        a = result["admit_stress"]
        say(f"[bench] admit stress: {a['ms_per_round']} ms per round, {a['records_moved']} records "
            f"moved, {a['roofline']['achieved']} GB/s")
    del S, sets, outs
    torch.cuda.empty_cache()
    if cal is not None:
        cal["decode_frac_of_stream"] = round(achieved / cal["GBps"], 4)
        cal["decode_frac_of_stream_launch_size"] = round(achieved / cal["launch_size"]["GBps"], 4)
        result["calibration"] = cal
        say(f"[bench] decode at {100 * cal['decode_frac_of_stream']:.1f}% of the stream read, "
            f"{100 * cal['decode_frac_of_stream_launch_size']:.1f}% of a stream read of its own size")
    if args.long_blocks > 0:
        say(f"[bench] long path: {args.long_blocks} prompt blocks, {args.long_decode} decode tokens")
        result["long"] = bench_long(device, args.seed, args.long_blocks, args.long_decode,
                                    args.long_eager)
        r = result["long"]
        say(f"[bench] long: prefill {r['prefill_tokens_per_s']:,.0f} tok/s "
            f"({r['us_per_block_layer_with_admit']} us per block-layer), decode "
            f"{r['graph_us_per_token']} us/token as graph replays, {r['eager_us_per_token']} eager")
    if args.layer_configs > 0:
        result["layers"] = []
        for name in ("layer_b1", "layer_b64", "layer_b288"):
            say(f"[bench] one layer: {name}")
            r = bench_layer_config(device, args.seed, name)
            say(f"[bench] {name}: eager {r['eager_us_per_step']} us/step (decode launch "
                f"{r['eager_decode_launch_us']} us, admit {r['admit_us']} us), graph "
                f"{r['graph_us_per_step']} us/step")
            if "roofline" in r:
                rf = r["roofline"]
                say(f"[bench] {name}: decode launch {rf['achieved']} GB/s, "
                    f"{100 * rf['frac_of_probe']:.1f}% of a stream read of its size "
                    f"({rf['stream_probe_same_size']['GBps']} GB/s)")
            result["layers"].append(r)
    if args.prefill_blocks > 0:
        torch.cuda.empty_cache()
        result["prefill"] = []
        for pb in (1, 8):
            say(f"[bench] prefill, batch {pb}")
            r = bench_prefill(device, args.seed, pb, args.prefill_blocks)
            say(f"[bench] prefill batch {pb}: {r['us_per_block_layer']} us per block-layer, "
                f"{r['roofline']['achieved']} TFLOP/s ({100 * r['roofline']['frac']:.1f}% of bf16 MFMA peak)")
            ref = r["library_reference"]
            if "us" in ref:
                say(f"[bench] torch flash attention, same flop: {ref['us']} us, {ref['TFLOP/s']} TFLOP/s "
                    f"({100 * ref['frac']:.1f}% of peak)")
            result["prefill"].append(r)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
