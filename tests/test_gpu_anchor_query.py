"""GPU parity of the separate anchor query (q_anchor of rma_decode_step_at
and rma_prefill_block_at): the anchor read and the gate use q_anchor, the
local read keeps q.  Checked against one-sequence oracles that take the
same q_anchor, in the split launch (small batch), the whole-unit launch
(batch 256) and the prefill block; and q_anchor == q must give the bits of
the one-query path."""
import numpy as np
import pytest
import torch

from bounded_memory_decode_amd import rma, synth
from oracle import OracleState
import gpu_util as gu
from test_gpu_positions import SENTINEL, _decode_at, _rows, _seq_oracles

pytestmark = pytest.mark.gpu


def _oracle_decode_qa(o: OracleState, layer: int, xb: dict, qab, wg) -> np.ndarray:
    ref = o.decode_step(layer, xb["q"], xb["k"], xb["v"], xb["ck"], xb["cv"], xb["cs"], wg,
                        q_anchor=qab)
    if o.pend_n[layer] == o.C:
        o.admit(layer)
    return ref


def _decode_at_qa(S, layer, pos_list, xd, qa_dev, wg_dev):
    pos = torch.tensor(pos_list, dtype=torch.int32, device=gu.DEV)
    out = torch.full((S.batch, S.cfg.q_heads, S.cfg.head_dim), SENTINEL, dtype=torch.bfloat16,
                     device=gu.DEV)
    S.decode_step_at(layer, pos, xd["q"], xd["k"], xd["v"], xd["ck"], xd["cv"], xd["cs"],
                     wg_dev, out=out, q_anchor=qa_dev)
    return out


@pytest.mark.parametrize("B", [4, 256])
def test_anchor_query_equal_to_q_gives_the_same_bits(B):
    """q_anchor == q: outputs and state identical to the one-query call
    (split launch at B=4, whole-unit launch at B=256), across an admit."""
    gu.log(f"case q_anchor == q, B={B}")
    w = synth.WORKLOADS["layer_b1"].with_(B=B, t0=32768 + 250, bank_n=800)
    seed = 70
    if B <= 8:
        st = synth.initial_state(w, seed)
        A, D = gu.gpu_state(w, st), gu.gpu_state(w, st)
    else:  # device-drawn records: the comparison is GPU against GPU
        A = rma.State(gu.cfg_for(w), B, gu.DEV, start_pos=w.t0, bank_n=w.bank_n)
        g = torch.Generator(device=gu.DEV)
        g.manual_seed(seed)
        for name in ("ring_k", "ring_v", "bank_k", "bank_v"):
            v = A.region_view(name)
            v.copy_((torch.randn(v.shape, generator=g, device=gu.DEV) / 16)
                    .to(torch.bfloat16).view(torch.int16))
        A.region_view("bscore").copy_(torch.randn(A.region_view("bscore").shape, generator=g,
                                                  device=gu.DEV))
        for name in ("bsrc", "pend_k", "pend_v", "pscore"):
            A.region_view(name).zero_()
        D = rma.State(gu.cfg_for(w), B, gu.DEV, start_pos=w.t0, bank_n=w.bank_n)
        D.buf.copy_(A.buf)
        torch.cuda.synchronize()
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    pos = [w.t0] * B
    for s in range(10):
        xd = gu.inputs_to_dev(synth.step_inputs(w, seed, 0, s))
        oa = _decode_at_qa(A, 0, pos, xd, xd["q"].clone(), wg_dev)
        od = _decode_at(D, 0, pos, xd, wg_dev)
        assert torch.equal(oa.view(torch.int16), od.view(torch.int16)), f"step {s}"
        pos = [p + 1 for p in pos]
    torch.cuda.synchronize()
    for name in gu.REGIONS + ("bank_n",):
        assert torch.equal(A.read(name), D.read(name)), name


def test_anchor_query_split_launch_vs_oracle():
    """Batch 3 at unrelated positions, each crossing a block end, with a
    distinct q_anchor every step."""
    gu.log("case q_anchor split launch, B=3")
    base = synth.WORKLOADS["layer_b1"]
    specs = [(32768 - 5, 1024), (1020, 300), (32768 + 240, 0)]
    seed = 71
    states, oracles = _seq_oracles(base, specs, seed)
    w = base.with_(B=len(specs))
    S = gu.assemble_state(w, states)
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    pos = [t0 for t0, _ in specs]
    for s in range(24):
        x = synth.step_inputs(w, seed, 0, s)
        qa = synth.anchor_query(w, seed, 0, s)
        out = _decode_at_qa(S, 0, pos, gu.inputs_to_dev(x), gu.to_dev(qa), wg_dev)
        for b in range(w.B):
            ref = _oracle_decode_qa(oracles[b], 0, _rows(x, b), qa[b:b + 1], wg[0])
            gu.check_out(out[b:b + 1], ref, f"q_anchor step {s} sequence {b}")
        pos = [p + 1 for p in pos]
    torch.cuda.synchronize()
    for b in range(w.B):
        gu.check_seq_state(S, b, oracles[b], "q_anchor split end")
    assert [int(o.bank_n[0, 0, 0]) for o in oracles] == [1024, 556, 256]


def test_anchor_query_whole_unit_launch_vs_oracle():
    """Batch 256 (whole-unit launch) from an empty state at staggered
    positions; four sampled sequences against their oracles."""
    gu.log("case q_anchor whole-unit launch, B=256")
    base = synth.WORKLOADS["layer_b1"]
    B = 256
    sampled = {1: (250, 1024), 64: (33000, 1024), 130: (767, 512), 255: (1023 - 3, 0)}
    seed = 72
    states, oracles = _seq_oracles(base, list(sampled.values()), seed)
    w = base.with_(B=B)
    S = rma.State(gu.cfg_for(w), B, gu.DEV, start_pos=0, bank_n=0)
    S.buf.zero_()
    S.seq_reset(0, B, 1024)
    for (b, _), st in zip(sampled.items(), states):
        for name in gu.REGIONS + ("bank_n",):
            S.write(name, st[name], batch=slice(b, b + 1))
    torch.cuda.synchronize()
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    pos = [(b * 53) % 4096 for b in range(B)]
    for b, (t0, _) in sampled.items():
        pos[b] = t0
    for s in range(20):
        x = synth.step_inputs(w, seed, 0, s)
        qa = synth.anchor_query(w, seed, 0, s)
        out = _decode_at_qa(S, 0, pos, gu.inputs_to_dev(x), gu.to_dev(qa), wg_dev)
        for i, b in enumerate(sampled):
            ref = _oracle_decode_qa(oracles[i], 0, _rows(x, b), qa[b:b + 1], wg[0])
            gu.check_out(out[b:b + 1], ref, f"q_anchor step {s} sequence {b}")
        pos = [p + 1 for p in pos]
    torch.cuda.synchronize()
    for i, b in enumerate(sampled):
        gu.check_seq_state(S, b, oracles[i], "q_anchor whole-unit end")


def test_anchor_query_prefill_vs_oracle():
    """Prefill blocks with a distinct q_anchor (full block with its admit,
    then a short block), an empty-bank sequence (the gate still takes
    q_anchor), then decode steps."""
    gu.log("case q_anchor prefill, B=2")
    base = synth.WORKLOADS["layer_b1"]
    specs = [(32768, 1024), (512, 0)]
    seed = 73
    states, oracles = _seq_oracles(base, specs, seed)
    w = base.with_(B=2)
    S = gu.assemble_state(w, states)
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    pos = [t0 for t0, _ in specs]
    step = 0
    for n in (256, 60):
        x = synth.block_inputs(w, seed, 0, step, n)
        qa = synth.block_anchor_query(w, seed, 0, step, n)
        d = gu.inputs_to_dev(x)
        out = S.prefill_block_at(0, torch.tensor(pos, dtype=torch.int32, device=gu.DEV), d["q"],
                                 d["k"], d["v"], d["ck"], d["cv"], d["cs"], wg_dev,
                                 q_anchor=gu.to_dev(qa))
        for b in range(2):
            o = oracles[b]
            xb = _rows(x, b)
            vm = gu.vmax(o.ring_v, o.bank_v, xb["v"])
            ref = o.prefill_block(0, xb["q"], xb["k"], xb["v"], xb["ck"], xb["cv"], xb["cs"],
                                  wg[0], q_anchor=qa[b:b + 1])
            if o.pend_n[0] == o.C:
                o.admit(0)
            gu.check_out(out[b:b + 1], ref, f"q_anchor prefill n={n} sequence {b}", p_bf16_vmax=vm)
        pos = [p + n for p in pos]
        step += n
    for s in range(4):
        x = synth.step_inputs(w, seed, 0, step + s)
        qa = synth.anchor_query(w, seed, 0, step + s)
        out = _decode_at_qa(S, 0, pos, gu.inputs_to_dev(x), gu.to_dev(qa), wg_dev)
        for b in range(2):
            ref = _oracle_decode_qa(oracles[b], 0, _rows(x, b), qa[b:b + 1], wg[0])
            gu.check_out(out[b:b + 1], ref, f"q_anchor decode after prefill, sequence {b}")
        pos = [p + 1 for p in pos]
    torch.cuda.synchronize()
    for b in range(2):
        gu.check_seq_state(S, b, oracles[b], "q_anchor prefill end")


def test_anchor_query_equal_to_q_prefill_same_bits():
    """Prefill with q_anchor == q: outputs and state identical to the
    one-query prefill (the anchor-query rows are reloaded at the first bank
    tile and for the gate)."""
    gu.log("case q_anchor == q prefill, B=2")
    w = synth.WORKLOADS["layer_b1"].with_(B=2, bank_n=700)
    seed = 74
    st = synth.initial_state(w, seed)
    A, D = gu.gpu_state(w, st), gu.gpu_state(w, st)
    wg_dev = gu.to_dev(synth.gate_weights(w, seed)[0])
    x = gu.inputs_to_dev(synth.block_inputs(w, seed, 0, 0, 256))
    pos = torch.full((2,), w.t0, dtype=torch.int32, device=gu.DEV)
    oa = A.prefill_block_at(0, pos, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg_dev,
                            q_anchor=x["q"].clone())
    od = D.prefill_block_at(0, pos, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg_dev)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), od.view(torch.int16))
    for name in gu.REGIONS + ("bank_n",):
        assert torch.equal(A.read(name), D.read(name)), name
