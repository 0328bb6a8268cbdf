"""GPU parity of the per-sequence-position calls (rma_decode_step_at,
rma_prefill_block_at, rma_seq_reset) and of a token step captured in a HIP
graph.

Each sequence of a batch is checked against a one-sequence CPU oracle that
runs the method at that sequence's own position, so sequences cross their
block boundaries (and are admitted) at different steps; sequences left out
(negative position) must keep their state and output rows untouched."""
import numpy as np
import pytest
import torch

from bounded_memory_decode_amd import rma, synth
from oracle import OracleState
import gpu_util as gu

pytestmark = pytest.mark.gpu

SENTINEL = 7.0  # exact in bf16; written into out before each call


def _one_seq_workload(base: synth.Workload, t0: int, bank_n: int) -> synth.Workload:
    return base.with_(B=1, t0=t0, bank_n=bank_n, ring_full=True)


def _seq_oracles(base, specs, seed):
    """(start states, oracles) of one-sequence workloads at (t0, bank_n)."""
    states, oracles = [], []
    for b, (t0, n) in enumerate(specs):
        w1 = _one_seq_workload(base, t0, n)
        st = synth.initial_state(w1, seed + b)
        states.append(st)
        oracles.append(OracleState.from_synth(st, H=w1.H, G=w1.G, d=w1.d, R=w1.R, N=w1.N,
                                              C=w1.C))
    return states, oracles


def _rows(x: dict, b: int) -> dict:
    return {k: v[b:b + 1] for k, v in x.items()}


def _oracle_decode(o: OracleState, layer: int, xb: dict, wg) -> np.ndarray:
    ref = o.decode_step(layer, xb["q"], xb["k"], xb["v"], xb["ck"], xb["cv"], xb["cs"], wg)
    if o.pend_n[layer] == o.C:
        o.admit(layer)
    return ref


def _decode_at(S, layer, pos_list, xd, wg_dev):
    pos = torch.tensor(pos_list, dtype=torch.int32, device=gu.DEV)
    out = torch.full((S.batch, S.cfg.q_heads, S.cfg.head_dim), SENTINEL, dtype=torch.bfloat16,
                     device=gu.DEV)
    S.decode_step_at(layer, pos, xd["q"], xd["k"], xd["v"], xd["ck"], xd["cv"], xd["cs"],
                     wg_dev, out=out)
    return out


def _check_left_out(out: torch.Tensor, b: int, tag: str):
    row = out[b].float()
    assert torch.all(row == SENTINEL), f"{tag}: output row of left-out sequence {b} written"


def test_at_equals_lockstep_bitwise():
    """All sequences at one position: the per-sequence calls give the same
    bits as the lockstep calls (outputs and every region), across an
    admit, in two layers."""
    gu.log("case decode_at == lockstep, B=4, 2 layers")
    w = synth.WORKLOADS["layer_b1"].with_(B=4, L=2, t0=32768 + 200, bank_n=700)
    seed = 60
    st = synth.initial_state(w, seed)
    A = gu.gpu_state(w, st)
    D = gu.gpu_state(w, st)
    wg = synth.gate_weights(w, seed)
    wg_dev = [gu.to_dev(wg[l]) for l in range(w.L)]
    pos = torch.full((w.B,), w.t0, dtype=torch.int32, device=gu.DEV)
    for s in range(70):
        for l in range(w.L):
            xd = gu.inputs_to_dev(synth.step_inputs(w, seed, l, s))
            oa = A.decode_step_at(l, pos, xd["q"], xd["k"], xd["v"], xd["ck"], xd["cv"],
                                  xd["cs"], wg_dev[l])
            od = gu.decode(D, l, xd, wg_dev[l])
            if D.pend_n[l] == w.C:
                D.admit(l)
            assert torch.equal(oa.view(torch.int16), od.view(torch.int16)), f"step {s} layer {l}"
        pos += 1
    torch.cuda.synchronize()
    for name in gu.REGIONS + ("bank_n",):
        assert torch.equal(A.read(name), D.read(name)), name
    assert int(A.read("bank_n").min()) == 956  # 700 + 256 after the admit


def test_staggered_positions_and_idle_sequence_vs_oracle():
    """Four sequences at unrelated positions (full ring, ring still filling,
    empty and partial banks), one of them idle every third step; each
    crosses a block boundary at its own step."""
    gu.log("case staggered positions, B=4 (split launch)")
    base = synth.WORKLOADS["layer_b1"]
    specs = [(32768 - 3, 1024), (32768 + 220, 600), (1013, 768), (500, 0)]
    seed = 61
    states, oracles = _seq_oracles(base, specs, seed)
    w = base.with_(B=len(specs))
    S = gu.assemble_state(w, states)
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    pos = [t0 for t0, _ in specs]
    for s in range(70):
        active = [not (b == 1 and s % 3 == 1) for b in range(w.B)]
        x = synth.step_inputs(w, seed, 0, s)
        out = _decode_at(S, 0, [p if a else -1 for p, a in zip(pos, active)],
                         gu.inputs_to_dev(x), wg_dev)
        for b in range(w.B):
            tag = f"step {s} sequence {b} at {pos[b]}"
            if not active[b]:
                _check_left_out(out, b, tag)
                continue
            ref = _oracle_decode(oracles[b], 0, _rows(x, b), wg[0])
            gu.check_out(out[b:b + 1], ref, tag)
            pos[b] += 1
    torch.cuda.synchronize()
    for b in range(w.B):
        assert oracles[b].t[0] == pos[b]
        gu.check_seq_state(S, b, oracles[b], "staggered end")
    # every sequence went through an admit
    assert [int(o.bank_n[0, 0, 0]) for o in oracles] == [1024, 856, 1024, 256]


@pytest.mark.parametrize("B", [256, 300])
def test_whole_unit_launch_staggered_sampled(B):
    """Batch 256 (the whole-unit launch, one wave per sequence and group)
    and batch 300 (two launches: sequences 0-255 whole-unit with the admit
    launch, 256-299 the split launch of a batch of 44 with the admit in its
    combine): every sequence at its own position, some idle on even steps;
    six sampled sequences against their oracles, every step."""
    gu.log(f"case staggered positions, B={B} (whole-unit launch), 6 sampled sequences")
    base = synth.WORKLOADS["layer_b1"]
    sampled = {0: (250, 1024), 3: (0, 0), 7: (1020, 768), 100: (511, 256), 203: (33010, 1024),
               255: (767, 512)}
    if B == 300:
        sampled = {0: (250, 1024), 255: (0, 0), 256: (1020, 768), 263: (511, 256),
                   280: (33010, 1024), 299: (767, 512)}
    seed = 62
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
    pos = [(b * 37) % 2048 for b in range(B)]
    for b, (t0, _) in sampled.items():
        pos[b] = t0
    for s in range(40):
        active = [not (b % 5 == 3 and s % 2 == 0) for b in range(B)]
        x = synth.step_inputs(w, seed, 0, s)
        out = _decode_at(S, 0, [p if a else -1 for p, a in zip(pos, active)],
                         gu.inputs_to_dev(x), wg_dev)
        for i, b in enumerate(sampled):
            tag = f"step {s} sequence {b} at {pos[b]}"
            if not active[b]:
                _check_left_out(out, b, tag)
            else:
                ref = _oracle_decode(oracles[i], 0, _rows(x, b), wg[0])
                gu.check_out(out[b:b + 1], ref, tag)
        pos = [p + 1 if a else p for p, a in zip(pos, active)]
    torch.cuda.synchronize()
    for i, b in enumerate(sampled):
        gu.check_seq_state(S, b, oracles[i], "whole-unit staggered end")
    assert [int(o.bank_n[0, 0, 0]) for o in oracles] == [1024, 0, 1024, 512, 1024, 768]


def test_prefill_at_mixed_positions():
    """Block prefill for the sequences at a block start; a sequence off a
    block start is left out (state and output rows untouched); a full block
    is admitted by the same call, a short one is not; then every sequence
    decodes at its own position."""
    gu.log("case prefill_at, B=3")
    base = synth.WORKLOADS["layer_b1"]
    specs = [(32768, 1024), (32768 + 100, 900), (512, 256)]
    seed = 63
    states, oracles = _seq_oracles(base, specs, seed)
    w = base.with_(B=3)
    S = gu.assemble_state(w, states)
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    pos = [t0 for t0, _ in specs]
    step = 0
    for n in (256, 100):
        x = synth.block_inputs(w, seed, 0, step, n)
        d = gu.inputs_to_dev(x)
        before1 = {name: S.read(name, slice(None), slice(1, 2)) for name in gu.REGIONS}
        out = torch.full((w.B, n, w.H, w.d), SENTINEL, dtype=torch.bfloat16, device=gu.DEV)
        S.prefill_block_at(0, torch.tensor(pos, dtype=torch.int32, device=gu.DEV), d["q"],
                           d["k"], d["v"], d["ck"], d["cv"], d["cs"], wg_dev, out=out)
        for b in (0, 2):
            o = oracles[b]
            xb = _rows(x, b)
            vm = gu.vmax(o.ring_v, o.bank_v, xb["v"])
            ref = o.prefill_block(0, xb["q"], xb["k"], xb["v"], xb["ck"], xb["cv"], xb["cs"],
                                  wg[0])
            if o.pend_n[0] == o.C:
                o.admit(0)
            gu.check_out(out[b:b + 1], ref, f"prefill n={n} sequence {b}", p_bf16_vmax=vm)
            pos[b] += n
        _check_left_out(out, 1, f"prefill n={n}")
        torch.cuda.synchronize()
        for name in gu.REGIONS:
            assert torch.equal(S.read(name, slice(None), slice(1, 2)), before1[name]), name
        step += n
    # then everybody decodes at its own position
    for s in range(6):
        x = synth.step_inputs(w, seed, 0, step + s)
        out = _decode_at(S, 0, pos, gu.inputs_to_dev(x), wg_dev)
        for b in range(3):
            ref = _oracle_decode(oracles[b], 0, _rows(x, b), wg[0])
            gu.check_out(out[b:b + 1], ref, f"decode after prefill, sequence {b}")
            pos[b] += 1
    torch.cuda.synchronize()
    for b in range(3):
        gu.check_seq_state(S, b, oracles[b], "prefill_at end")
    assert [int(o.bank_n[0, 0, 0]) for o in oracles] == [1024, 900, 512]


@pytest.mark.parametrize("B", [4, 300, 448])
def test_every_sequence_left_out_changes_nothing(B):
    """Per-sequence decode and prefill calls with every position negative
    (an empty batch): no output row and no byte of the history changes.
    Batch 4 takes the split launches; batch 448 (ring 63, bank 64, commit
    16) the whole-unit decode launch with its admit launch, and the
    unsplit prefill; batch 300 both decode launches in turn."""
    gu.log(f"case every sequence left out, B={B}")
    w = synth.WORKLOADS["layer_b1"].with_(name=f"idle_b{B}", B=B, R=63, N=64, C=16,
                                          t0=64 * 16, bank_n=64)
    seed = 67
    st = synth.initial_state(w, seed)
    S = gu.gpu_state(w, st)
    before = {name: S.read(name).clone() for name in gu.REGIONS + ("bank_n",)}
    wg_dev = gu.to_dev(synth.gate_weights(w, seed)[0])
    idle = torch.full((B,), -1, dtype=torch.int32, device=gu.DEV)
    out = _decode_at(S, 0, [-1] * B, gu.inputs_to_dev(synth.step_inputs(w, seed, 0, 0)), wg_dev)
    d = gu.inputs_to_dev(synth.block_inputs(w, seed, 0, 0, w.C))
    pout = torch.full((B, w.C, w.H, w.d), SENTINEL, dtype=torch.bfloat16, device=gu.DEV)
    S.prefill_block_at(0, idle, d["q"], d["k"], d["v"], d["ck"], d["cv"], d["cs"], wg_dev,
                       out=pout)
    torch.cuda.synchronize()
    assert torch.all(out.float() == SENTINEL), "decode wrote an output row"
    assert torch.all(pout.float() == SENTINEL), "prefill wrote an output row"
    for name, v in before.items():
        assert torch.equal(S.read(name), v), name


@pytest.mark.parametrize("B", [2, 448])
def test_positions_at_the_int32_limit(B):
    """Sequences whose last block ends at the last int32 position
    (2^31 - 1; 256 divides 2^31, so that token completes a block): a
    prompt block that ends there (admitted by the call), then decode steps
    of other sequences across that same block end (admitted by the decode
    call).  Batch 2 takes the split launches (the decode's admit runs in
    its combine), batch 448 the whole-unit decode, its admit launch and
    the unsplit prefill."""
    gu.log(f"case positions at the int32 limit, B={B}")
    base = synth.WORKLOADS["layer_b1"]
    top = rma.RMA_MAX_POS
    sampled = {0: (top + 1 - 3, 1024), B - 1: (top + 1 - 256, 700)}
    seed = 68
    states, oracles = _seq_oracles(base, list(sampled.values()), seed)
    orc = dict(zip(sampled, oracles))
    w = base.with_(B=B)
    if B == len(sampled):
        S = gu.assemble_state(w, states)
    else:
        S = rma.State(gu.cfg_for(w), B, gu.DEV, start_pos=0, bank_n=0)
        S.buf.zero_()
        S.seq_reset(0, B, 512)
        for b, st in zip(sampled, states):
            for name in gu.REGIONS + ("bank_n",):
                S.write(name, st[name], batch=slice(b, b + 1))
        torch.cuda.synchronize()
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    pos = [(b * 53) % 4096 for b in range(B)]
    for b, (t0, _) in sampled.items():
        pos[b] = t0

    # the prompt block [2^31 - 256, 2^31) of the last sequence; the first
    # is off a block start and left out
    n = 256
    x = synth.block_inputs(w, seed, 0, 0, n)
    d = gu.inputs_to_dev(x)
    out = torch.full((B, n, w.H, w.d), SENTINEL, dtype=torch.bfloat16, device=gu.DEV)
    S.prefill_block_at(0, torch.tensor(pos, dtype=torch.int32, device=gu.DEV), d["q"], d["k"],
                       d["v"], d["ck"], d["cv"], d["cs"], wg_dev, out=out)
    o = orc[B - 1]
    xb = _rows(x, B - 1)
    ref = o.prefill_block(0, xb["q"], xb["k"], xb["v"], xb["ck"], xb["cv"], xb["cs"], wg[0])
    assert o.pend_n[0] == o.C
    o.admit(0)
    gu.check_out(out[B - 1:B], ref, "prefill ending at 2^31 - 1",
                 p_bf16_vmax=gu.vmax(o.ring_v, o.bank_v, xb["v"]))
    _check_left_out(out, 0, "prefill at the int32 limit")
    torch.cuda.synchronize()
    gu.check_seq_state(S, B - 1, o, "after the prefill ending at 2^31 - 1")
    assert int(o.bank_n[0, 0, 0]) == 956 and int(o.bsrc[0, 0, 0, :956].max()) >= top - 255

    # decode: the first sequence crosses the same block end; the last has
    # no position left and is left out
    pos = [p + n if (b != 0 and p % 256 == 0) else p for b, p in enumerate(pos)]
    pos[B - 1] = -1
    for s in range(3):
        x = synth.step_inputs(w, seed, 0, n + s)
        out = _decode_at(S, 0, pos, gu.inputs_to_dev(x), wg_dev)
        ref = _oracle_decode(orc[0], 0, _rows(x, 0), wg[0])
        gu.check_out(out[0:1], ref, f"decode step {s} at {pos[0]}")
        _check_left_out(out, B - 1, f"decode step {s}")
        pos = [p + 1 if (p >= 0 and p < top) else -1 for p in pos]
    torch.cuda.synchronize()
    assert orc[0].t[0] == top + 1 and orc[0].pend_n[0] == 0  # admitted
    for b in sampled:
        gu.check_seq_state(S, b, orc[b], "int32 limit end")

def test_seq_reset_starts_a_new_sequence_in_a_used_slot():
    """A slot that held a long sequence is given a new one: bank count 0 in
    every layer, position 0; its stale ring and bank are never read."""
    gu.log("case seq_reset, B=2, 2 layers")
    base = synth.WORKLOADS["layer_b1"].with_(L=2)
    seed = 64
    old_states, _ = _seq_oracles(base, [(32768, 1024), (40000, 1024)], seed)
    w = base.with_(B=2)
    S = gu.assemble_state(w, old_states)
    S.seq_reset(1, 1, 0)
    torch.cuda.synchronize()
    bn = S.read("bank_n")
    assert torch.all(bn[:, 0] == 1024) and torch.all(bn[:, 1] == 0)
    fresh = synth.initial_state(base.with_(B=1, t0=0, bank_n=0, ring_full=False), seed)
    o_new = OracleState.from_synth(fresh)
    o_old = OracleState.from_synth(old_states[0])
    wg = synth.gate_weights(w, seed)
    wg_dev = [gu.to_dev(wg[l]) for l in range(w.L)]
    pos = [32768, 0]
    for s in range(5):
        for l in range(w.L):
            x = synth.step_inputs(w, seed, l, s)
            out = _decode_at(S, l, pos, gu.inputs_to_dev(x), wg_dev[l])
            for b, o in ((0, o_old), (1, o_new)):
                ref = _oracle_decode(o, l, _rows(x, b), wg[l])
                gu.check_out(out[b:b + 1], ref, f"step {s} layer {l} sequence {b}")
        pos = [p + 1 for p in pos]
    torch.cuda.synchronize()
    gu.check_seq_state(S, 0, o_old, "reset: untouched sequence")
    # the new sequence: its written ring and pending slots, and its counts
    ring_v = S.read("ring_v", slice(None), slice(1, 2)).cpu().numpy()
    pend_k = S.read("pend_k", slice(None), slice(1, 2)).cpu().numpy()
    assert np.array_equal(ring_v[:, :, :, :5], o_new.ring_v[:, :, :, :5].view(np.int16))
    assert np.array_equal(pend_k[:, :, :, :5], o_new.pend_k[:, :, :, :5].view(np.int16))
    assert torch.all(S.read("bank_n")[:, 1] == 0)


def test_token_step_graph_replays_match_eager_and_oracle():
    """Eight layers of one token captured once in a HIP graph together with
    the position increment, replayed with new inputs each time (eager copies
    and synchronisations between replays); crosses a block boundary, so the
    admit inside the graph runs on one replay and is skipped on the others.
    Every replay equals the eager per-sequence calls bit for bit and the
    oracle within the bound."""
    gu.log("case graph replay, B=1, 8 layers")
    base = synth.WORKLOADS["layer_b1"].with_(L=8)
    seed = 65
    t0 = 32768 - 4
    w = base.with_(t0=t0, bank_n=1024)
    st = synth.initial_state(w, seed)
    A = gu.gpu_state(w, st)
    D = gu.gpu_state(w, st)
    o = OracleState.from_synth(st)
    wg = synth.gate_weights(w, seed)
    wg_dev = [gu.to_dev(wg[l]) for l in range(w.L)]
    L, B, H, G, d = w.L, w.B, w.H, w.G, w.d
    q_s = torch.zeros((L, B, H, d), dtype=torch.bfloat16, device=gu.DEV)
    kv_s = {k: torch.zeros((L, B, G, d), dtype=torch.bfloat16, device=gu.DEV)
            for k in ("k", "v", "ck", "cv")}
    cs_s = torch.zeros((L, B, G), dtype=torch.float32, device=gu.DEV)
    out_s = torch.zeros((L, B, H, d), dtype=torch.bfloat16, device=gu.DEV)
    pos_a = torch.full((B,), t0, dtype=torch.int32, device=gu.DEV)
    pos_d = pos_a.clone()

    # a throwaway call first, so nothing but launches happens under capture
    Wst = rma.State(gu.cfg_for(w), B, gu.DEV, start_pos=0, bank_n=0)
    Wst.decode_step_at(0, torch.zeros((B,), dtype=torch.int32, device=gu.DEV), q_s[0],
                       kv_s["k"][0], kv_s["v"][0], kv_s["ck"][0], kv_s["cv"][0], cs_s[0],
                       wg_dev[0])
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l in range(L):
            A.decode_step_at(l, pos_a, q_s[l], kv_s["k"][l], kv_s["v"][l], kv_s["ck"][l],
                             kv_s["cv"][l], cs_s[l], wg_dev[l], out=out_s[l])
        pos_a.add_(1)
    torch.cuda.synchronize()

    for s in range(10):
        xs = [synth.step_inputs(w, seed, l, s) for l in range(L)]
        for l in range(L):
            xd = gu.inputs_to_dev(xs[l])
            q_s[l].copy_(xd["q"])
            for k in kv_s:
                kv_s[k][l].copy_(xd[k])
            cs_s[l].copy_(xd["cs"])
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            xd = gu.inputs_to_dev(xs[l])
            od = D.decode_step_at(l, pos_d, xd["q"], xd["k"], xd["v"], xd["ck"], xd["cv"],
                                  xd["cs"], wg_dev[l])
            torch.cuda.synchronize()
            assert torch.equal(out_s[l].view(torch.int16), od.view(torch.int16)), \
                f"replay {s} layer {l}"
            ref = _oracle_decode(o, l, xs[l], wg[l])
            gu.check_out(out_s[l], ref, f"graph replay {s} layer {l}")
        pos_d += 1
        torch.cuda.synchronize()
        assert int(pos_a[0]) == t0 + s + 1
    for name in gu.REGIONS + ("bank_n",):
        assert torch.equal(A.read(name), D.read(name)), name
    gu.check_seq_state(A, 0, o, "graph end")


def test_graph_replays_of_the_two_launch_batch():
    """Batch 300 on a small geometry (ring 63, bank 64, commit 16): the
    per-sequence decode takes two launches (whole units for sequences
    0-255 with their admit launch, the split launch with the admit in its
    combine for 256-299).  Two layers of one token, captured once with the
    position increment, replayed across block ends with staggered
    positions: every replay equals the eager calls bit for bit, and so does
    the whole history at the end."""
    gu.log("case graph replay, B=300 (two launches), 2 layers")
    B = 300
    w = synth.WORKLOADS["layer_b1"].with_(name="graph_b300", B=B, L=2, R=63, N=64, C=16,
                                          t0=64 * 16, bank_n=64)
    seed = 66
    st = synth.initial_state(w, seed)
    A = gu.gpu_state(w, st)
    D = gu.gpu_state(w, st)
    wg = synth.gate_weights(w, seed)
    wg_dev = [gu.to_dev(wg[l]) for l in range(w.L)]
    L, H, G, d = w.L, w.H, w.G, w.d
    q_s = torch.zeros((L, B, H, d), dtype=torch.bfloat16, device=gu.DEV)
    kv_s = {k: torch.zeros((L, B, G, d), dtype=torch.bfloat16, device=gu.DEV)
            for k in ("k", "v", "ck", "cv")}
    cs_s = torch.zeros((L, B, G), dtype=torch.float32, device=gu.DEV)
    out_s = torch.zeros((L, B, H, d), dtype=torch.bfloat16, device=gu.DEV)
    # staggered: sequence b at block offset b mod 16, so every replay ends
    # some sequences' blocks on both sides of the two launches
    pos0 = torch.tensor([w.t0 + (b % 16) for b in range(B)], dtype=torch.int32, device=gu.DEV)
    pos_a, pos_d = pos0.clone(), pos0.clone()

    Wst = rma.State(gu.cfg_for(w), B, gu.DEV, start_pos=0, bank_n=0)
    Wst.decode_step_at(0, torch.zeros((B,), dtype=torch.int32, device=gu.DEV), q_s[0],
                       kv_s["k"][0], kv_s["v"][0], kv_s["ck"][0], kv_s["cv"][0], cs_s[0],
                       wg_dev[0])
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l in range(L):
            A.decode_step_at(l, pos_a, q_s[l], kv_s["k"][l], kv_s["v"][l], kv_s["ck"][l],
                             kv_s["cv"][l], cs_s[l], wg_dev[l], out=out_s[l])
        pos_a.add_(1)
    torch.cuda.synchronize()

    for s in range(20):
        for l in range(L):
            xd = gu.inputs_to_dev(synth.step_inputs(w, seed, l, s))
            q_s[l].copy_(xd["q"])
            for k in kv_s:
                kv_s[k][l].copy_(xd[k])
            cs_s[l].copy_(xd["cs"])
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            xd = gu.inputs_to_dev(synth.step_inputs(w, seed, l, s))
            od = D.decode_step_at(l, pos_d, xd["q"], xd["k"], xd["v"], xd["ck"], xd["cv"],
                                  xd["cs"], wg_dev[l])
            torch.cuda.synchronize()
            assert torch.equal(out_s[l].view(torch.int16), od.view(torch.int16)), \
                f"replay {s} layer {l}"
        pos_d += 1
    torch.cuda.synchronize()
    assert torch.equal(pos_a, pos_d)
    for name in gu.REGIONS + ("bank_n",):
        assert torch.equal(A.read(name), D.read(name)), name
