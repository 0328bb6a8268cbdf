"""GPU parity of the per-group gate (rma_config.gate = RMA_GATE_GROUP: one
gate per token and KV group, tanh of the group's mean anchor query against
one weight vector per group) against the oracle, in every launch that
computes the gate: the whole-unit decode finish (with and without a
separate anchor query), the split decode's combine, and the prefill block
(split and unsplit plans)."""
import numpy as np
import pytest
import torch

from bounded_memory_decode_amd import rma, synth
from oracle import OracleState
import gpu_util as gu

pytestmark = pytest.mark.gpu

GROUP = rma.RMA_GATE_GROUP


def _setup(w, seed):
    st = synth.initial_state(w, seed)
    S = gu.gpu_state(w, st, gate=GROUP)
    o = OracleState.from_synth(st, H=w.H, G=w.G, d=w.d, R=w.R, N=w.N, C=w.C, gate_group=True)
    wg = synth.gate_weights(w, seed, per_group=True)
    return S, o, wg, gu.to_dev(wg[0])


@pytest.mark.parametrize("B,anchor_query", [(448, False), (448, True), (300, False), (300, True),
                                             (3, False), (4, True)],
                         ids=["whole-unit", "whole-unit-qa", "two-launch", "two-launch-qa", "split",
                              "split-qa"])
def test_group_gate_decode(B, anchor_query):
    """Decode across block ends with the per-group gate.  Batches 448 and
    300 run on a small geometry (ring 63, bank 64, commit 16: 1,792 units,
    the whole-unit launch; 1,200 units, the whole-unit launch for sequences
    0-255 and the split launch for the rest), batches 3 and 4 on the
    EdgeRock geometry (the split launch).  Per-sequence calls with a
    separate anchor query, lockstep calls without; every output every few
    steps and the state at the end (in both parts of the two-launch batch)."""
    gu.log(f"case group gate decode B={B} q_anchor={anchor_query}")
    if B >= 160:
        w = synth.WORKLOADS["sharp_b1"].with_(name=f"group_b{B}", B=B, R=63, N=64, C=16,
                                              t0=64 * 16 + 5, bank_n=64)
        steps, every = 30, 3
    else:
        w = synth.WORKLOADS["sharp_b1"].with_(name=f"group_b{B}", B=B, t0=32768 - 20,
                                              bank_n=700)
        steps, every = 40, 1
    seed = 100 + B
    S, o, wg, wg_dev = _setup(w, seed)
    pos = torch.full((B,), w.t0, dtype=torch.int32, device=gu.DEV)
    worst = 0.0
    for s in range(steps):
        x = synth.step_inputs(w, seed, 0, s)
        xd = gu.inputs_to_dev(x)
        want = s % every == 0 or s == steps - 1
        if anchor_query:
            qa = synth.anchor_query(w, seed, 0, s)
            out = S.decode_step_at(0, pos, xd["q"], xd["k"], xd["v"], xd["ck"], xd["cv"],
                                   xd["cs"], wg_dev, q_anchor=gu.to_dev(qa))
            pos += 1
        else:
            qa = None
            out = gu.decode(S, 0, xd, wg_dev)
        ref = o.decode_step(0, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[0],
                            compute_out=want, q_anchor=qa)
        if want:
            e, _ = gu.check_out(out, ref, f"group gate B={B} step {s}")
            worst = max(worst, e)
        if o.pend_n[0] == w.C:
            if not anchor_query:
                S.admit(0)
            o.admit(0)
    torch.cuda.synchronize()
    for b in sorted({0, B // 2, min(B - 1, 255), min(B - 1, 256), B - 1}):
        gu.check_seq_state(S, b, _one(o, b), f"group gate B={B}")
    gu.log(f"group gate decode B={B}: worst error {worst:.3e}")


def _one(o, b):
    """Sequence b of an oracle state as a one-sequence state."""
    r = OracleState(o.L, 1, o.H, o.G, o.d, o.R, o.N, o.C, o.scale, o.gate_group)
    for name in OracleState.ARRAYS:
        a = getattr(o, name)
        if name in ("t", "pend_n"):
            getattr(r, name)[...] = a
        else:
            getattr(r, name)[...] = a[:, b:b + 1]
    return r


@pytest.mark.parametrize("B,anchor_query", [(1, False), (1, True), (2, True), (8, False),
                                             (8, True)],
                         ids=["b1", "b1-qa", "b2-qa", "b8", "b8-qa"])
def test_group_gate_prefill(B, anchor_query):
    """Prefill blocks with the per-group gate: batch 1 and 2 (split launch:
    the gate in the merge kernel), batch 8 (unsplit: the gate in the
    attention kernel), a full block and a 100-token one, each completed by
    decode steps and admitted; every output against the oracle."""
    gu.log(f"case group gate prefill B={B} q_anchor={anchor_query}")
    w = synth.WORKLOADS["sharp_b1"].with_(name=f"group_pf_b{B}", B=B, bank_n=900)
    seed = 120 + B
    S, o, wg, wg_dev = _setup(w, seed)
    pos = torch.full((B,), w.t0, dtype=torch.int32, device=gu.DEV)
    step = 0
    for n in (256, 100):
        x = synth.block_inputs(w, seed, 0, step, n)
        d = gu.inputs_to_dev(x)
        qa = synth.block_anchor_query(w, seed, 0, step, n) if anchor_query else None
        vm = gu.vmax(o.ring_v, o.bank_v, x["v"])
        if anchor_query:
            out = S.prefill_block_at(0, pos, d["q"], d["k"], d["v"], d["ck"], d["cv"], d["cs"],
                                     wg_dev, q_anchor=gu.to_dev(qa))
        else:
            out = S.prefill_block(0, d["q"], d["k"], d["v"], d["ck"], d["cv"], d["cs"], wg_dev)
        ref = o.prefill_block(0, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[0],
                              q_anchor=qa)
        gu.check_out(out, ref, f"group gate prefill B={B} n={n}", p_bf16_vmax=vm)
        step += n
        pos += n
        while o.pend_n[0] < w.C:  # complete the block
            xs = synth.step_inputs(w, seed, 0, step)
            xsd = gu.inputs_to_dev(xs)
            qs = synth.anchor_query(w, seed, 0, step) if anchor_query else None
            if anchor_query:
                outd = S.decode_step_at(0, pos, xsd["q"], xsd["k"], xsd["v"], xsd["ck"],
                                        xsd["cv"], xsd["cs"], wg_dev, q_anchor=gu.to_dev(qs))
                pos += 1
            else:
                outd = gu.decode(S, 0, xsd, wg_dev)
            refd = o.decode_step(0, xs["q"], xs["k"], xs["v"], xs["ck"], xs["cv"], xs["cs"],
                                 wg[0], q_anchor=qs)
            gu.check_out(outd, refd, f"group gate B={B} decode step {step}")
            step += 1
        if not anchor_query:
            S.admit(0)
        o.admit(0)
    torch.cuda.synchronize()
    for b in range(B):
        gu.check_seq_state(S, b, _one(o, b), f"group gate prefill B={B}")
