"""GPU parity over seeded random geometries, against one-sequence oracles of
the same geometry.

Each case draws a ring R (1 .. 4,096 slots), a commit interval C
(1 .. min(256, R)) log-uniformly and a bank capacity N (1 .. 2,048 - C)
log-uniformly or uniformly, or
takes one of the edge geometries listed below (a one-slot ring with
single-token blocks, blocks as long as the ring, a one-record bank beside
the largest window, a two-slot ring beside the largest pool).  Then:

- per-sequence decode of three sequences at unrelated positions (ring still
  filling or full, bank empty to full), each crossing its own block end and
  admitted inside the call;
- a per-sequence prefill block of a drawn length for the sequences at a
  block start (one sequence off a block start is left out and must keep
  its state and output rows), then decode on from there.

Three cases run drawn geometries at batch 448, where the decode takes the
whole-unit launch with its admit launch and the prefill its unsplit
launch, and check sampled sequences.  Four geometries run with a separate
anchor query, under the per-head and the per-group gate.  Outputs are compared within the
decode tolerance, the history bit for bit.  Every draw is fixed by the
case's seed and logged before the case runs."""
import zlib

import numpy as np
import pytest
import torch

from bounded_memory_decode_amd import rma, synth
from oracle import OracleState
import gpu_util as gu

pytestmark = pytest.mark.gpu

SENTINEL = 7.0  # exact in bf16; written into out before each call
BASE = synth.WORKLOADS["layer_b1"]

# name: (R, N, C); the RANDOM cases draw theirs from their names
EDGES = {
    "ring1_commit1": (1, 1, 1),
    "commit_eq_ring": (96, 300, 96),
    "bank1_window_max": (4096, 1, 256),
    "ring2_pool_max": (2, 2046, 2),
}
RANDOM = [f"draw{i}" for i in range(16)]


def _logu(rng, lo: int, hi: int) -> int:
    if hi <= lo:
        return lo
    x = np.exp(rng.uniform(np.log(lo), np.log(hi + 1)))
    return int(min(hi, max(lo, np.floor(x))))


def _geometry(name: str):
    """(rng, R, N, C) of a case: the rng drives the case's later draws."""
    rng = np.random.default_rng([0x67656f, zlib.crc32(name.encode())])
    if name in EDGES:
        R, N, C = EDGES[name]
    else:
        R = _logu(rng, 1, 4096)
        C = _logu(rng, 1, min(256, R))
        N = _logu(rng, 1, 2048 - C) if rng.random() < 0.5 else int(rng.integers(1, 2049 - C))
    return rng, R, N, C


def _seq_oracles(w, specs, seed):
    states, oracles = [], []
    for b, (t0, n) in enumerate(specs):
        w1 = w.with_(B=1, t0=t0, bank_n=n)
        st = synth.initial_state(w1, seed + b)
        states.append(st)
        oracles.append(OracleState.from_synth(st, H=w1.H, G=w1.G, d=w1.d, R=w1.R, N=w1.N,
                                              C=w1.C))
    return states, oracles


def _rows(x: dict, b: int) -> dict:
    return {k: v[b:b + 1] for k, v in x.items()}


def _decode_at(S, pos_list, x, wg_dev):
    xd = gu.inputs_to_dev(x)
    pos = torch.tensor(pos_list, dtype=torch.int32, device=gu.DEV)
    out = torch.full((S.batch, S.cfg.q_heads, S.cfg.head_dim), SENTINEL, dtype=torch.bfloat16,
                     device=gu.DEV)
    S.decode_step_at(0, pos, xd["q"], xd["k"], xd["v"], xd["ck"], xd["cv"], xd["cs"], wg_dev,
                     out=out)
    return out


def _oracle_decode(o, xb, wg):
    ref = o.decode_step(0, xb["q"], xb["k"], xb["v"], xb["ck"], xb["cv"], xb["cs"], wg)
    if o.pend_n[0] == o.C:
        o.admit(0)
    return ref


def _before_block_end(rng, R, C):
    """A position 1 .. min(C, 6) tokens before a block end, ring still
    filling or already full."""
    k = int(rng.integers(1, max(2, (3 * R) // C + 3)))
    return k * C - int(rng.integers(1, min(C, 6) + 1))


def _decode_steps(S, oracles, seqs, pos, w, seed, step0, steps, wg, wg_dev, tag):
    """`steps` per-sequence decode steps; sequences not in `seqs` are left
    out (position -1) and must keep their output rows."""
    for s in range(steps):
        x = synth.step_inputs(w, seed, 0, step0 + s)
        out = _decode_at(S, [pos[b] if b in seqs else -1 for b in range(S.batch)], x, wg_dev)
        for b in range(S.batch):
            if b not in seqs:
                assert torch.all(out[b].float() == SENTINEL), f"{tag}: row {b} written"
                continue
            ref = _oracle_decode(oracles[seqs.index(b)], _rows(x, b), wg)
            gu.check_out(out[b:b + 1], ref, f"{tag} step {s} sequence {b} at {pos[b]}")
            pos[b] += 1


@pytest.mark.parametrize("name", list(EDGES) + RANDOM)
def test_random_geometry_decode_admit_prefill(name):
    rng, R, N, C = _geometry(name)
    w = BASE.with_(name=name, R=R, N=N, C=C)
    seed = 90 + sum(map(ord, name)) % 97

    # per-sequence decode across each sequence's own block end
    specs = [(_before_block_end(rng, R, C), int(rng.integers(0, N + 1))) for _ in range(3)]
    gu.log(f"case {name}: R={R} N={N} C={C}; decode_at from {specs}")
    states, oracles = _seq_oracles(w, specs, seed)
    wb = w.with_(B=len(specs))
    S = gu.assemble_state(wb, states)
    wg = synth.gate_weights(wb, seed)
    wg_dev = gu.to_dev(wg[0])
    pos = [t0 for t0, _ in specs]
    _decode_steps(S, oracles, [0, 1, 2], pos, wb, seed, 0, 8, wg[0], wg_dev, f"{name} decode")
    torch.cuda.synchronize()
    for b in range(3):
        assert oracles[b].t[0] == pos[b]
        gu.check_seq_state(S, b, oracles[b], f"{name} decode end")

    # per-sequence prefill of a drawn length at block starts, one sequence
    # off a block start left out, then decode on
    n = C if rng.random() < 0.5 else _logu(rng, 1, C)
    blk = lambda: C * int(rng.integers(0, max(1, (3 * R) // C + 3)))
    off = blk() + (int(rng.integers(1, C)) if C > 1 else -1)
    specs = [(blk(), int(rng.integers(0, N + 1))), (off if off >= 0 else 0, N),
             (blk(), int(rng.integers(0, N + 1)))]
    left_out = 1 if C > 1 else None  # with C = 1 every position starts a block
    gu.log(f"case {name}: prefill_at n={n} from {specs}")
    states, oracles = _seq_oracles(w, specs, seed + 10)
    S = gu.assemble_state(wb, states)
    pos = [t0 for t0, _ in specs]
    x = synth.block_inputs(wb, seed, 0, 0, n)
    d = gu.inputs_to_dev(x)
    before = {r: S.read(r, slice(None), slice(1, 2)) for r in gu.REGIONS} if left_out else None
    out = torch.full((3, n, w.H, w.d), SENTINEL, dtype=torch.bfloat16, device=gu.DEV)
    S.prefill_block_at(0, torch.tensor(pos, dtype=torch.int32, device=gu.DEV), d["q"], d["k"],
                       d["v"], d["ck"], d["cv"], d["cs"], wg_dev, out=out)
    for b in range(3):
        if b == left_out:
            assert torch.all(out[b].float() == SENTINEL), f"{name}: prefill wrote row {b}"
            continue
        o = oracles[b]
        xb = _rows(x, b)
        vm = gu.vmax(o.ring_v, o.bank_v, xb["v"])
        ref = o.prefill_block(0, xb["q"], xb["k"], xb["v"], xb["ck"], xb["cv"], xb["cs"], wg[0])
        if o.pend_n[0] == o.C:
            o.admit(0)
        gu.check_out(out[b:b + 1], ref, f"{name} prefill n={n} sequence {b}", p_bf16_vmax=vm)
        pos[b] += n
    torch.cuda.synchronize()
    if left_out is not None:
        for r in gu.REGIONS:
            assert torch.equal(S.read(r, slice(None), slice(1, 2)), before[r]), f"{name}: {r}"
    live = [b for b in range(3) if b != left_out]
    steps = min(C - n, 6) + 2 if n < C else 4
    _decode_steps(S, [oracles[b] for b in live], live, pos, wb, seed, n, steps, wg[0], wg_dev,
                  f"{name} decode after prefill")
    torch.cuda.synchronize()
    for b in live:
        gu.check_seq_state(S, b, oracles[b], f"{name} prefill end")


@pytest.mark.parametrize("name", ["wide0", "wide2", "wide3"])
def test_random_geometry_whole_unit_launch(name):
    """Batch 448: whole-unit decode launch and its admit launch, unsplit
    prefill (wide0: a block nearly as long as the ring; wide2: a ring of
    1,411 slots; wide3: a one-slot ring, an admit after every token).
    Four sampled sequences start 8 tokens before a block end, so they
    cross it (admitted by the admit launch) and then sit at a block start
    for the prefill; one of them is left out of the prefill.  The rest of
    the batch decodes and prefills at unrelated positions with a zero
    history."""
    rng, R, N, C = _geometry(name)
    w = BASE.with_(name=name, R=R, N=N, C=C)
    seed = 95 + zlib.crc32(name.encode()) % 7
    B = 448
    sampled = [0, 101, 250, 447]
    specs = [(C * int(rng.integers(-(-8 // C), -(-8 // C) + (3 * R) // C + 3)) - 8,
              int(rng.integers(0, N + 1))) for _ in sampled]
    gu.log(f"case {name}: B={B} R={R} N={N} C={C}; decode_at of {sampled} from {specs}")
    states, oracles = _seq_oracles(w, specs, seed)
    orc = dict(zip(sampled, oracles))
    wb = w.with_(B=B)
    S = rma.State(gu.cfg_for(wb), B, gu.DEV, start_pos=0, bank_n=0)
    S.buf.zero_()
    S.seq_reset(0, B, int(rng.integers(0, N + 1)))
    for b, st in zip(sampled, states):
        for r in gu.REGIONS + ("bank_n",):
            S.write(r, st[r], batch=slice(b, b + 1))
    torch.cuda.synchronize()
    wg = synth.gate_weights(wb, seed)
    wg_dev = gu.to_dev(wg[0])
    pos = [int(rng.integers(0, 4 * C + R)) for _ in range(B)]
    for b, (t0, _) in zip(sampled, specs):
        pos[b] = t0

    for s in range(8):
        x = synth.step_inputs(wb, seed, 0, s)
        out = _decode_at(S, pos, x, wg_dev)
        for b in sampled:
            ref = _oracle_decode(orc[b], _rows(x, b), wg[0])
            gu.check_out(out[b:b + 1], ref, f"{name} step {s} sequence {b} at {pos[b]}")
        pos = [p + 1 for p in pos]
    torch.cuda.synchronize()
    for b in sampled:
        assert pos[b] % C == 0 and orc[b].t[0] == pos[b]
        gu.check_seq_state(S, b, orc[b], f"{name} decode end")

    n = _logu(rng, 1, C)
    skip = sampled[1]
    gu.log(f"case {name}: prefill_at n={n}, sequence {skip} left out")
    call = list(pos)
    call[skip] = -1
    x = synth.block_inputs(wb, seed, 0, 8, n)
    d = gu.inputs_to_dev(x)
    out = torch.full((B, n, w.H, w.d), SENTINEL, dtype=torch.bfloat16, device=gu.DEV)
    S.prefill_block_at(0, torch.tensor(call, dtype=torch.int32, device=gu.DEV), d["q"], d["k"],
                       d["v"], d["ck"], d["cv"], d["cs"], wg_dev, out=out)
    for b in sampled:
        if b == skip:
            assert torch.all(out[b].float() == SENTINEL), f"{name}: prefill wrote row {b}"
            continue
        o = orc[b]
        xb = _rows(x, b)
        vm = gu.vmax(o.ring_v, o.bank_v, xb["v"])
        ref = o.prefill_block(0, xb["q"], xb["k"], xb["v"], xb["ck"], xb["cv"], xb["cs"], wg[0])
        if o.pend_n[0] == o.C:
            o.admit(0)
        gu.check_out(out[b:b + 1], ref, f"{name} prefill sequence {b}", p_bf16_vmax=vm)
    torch.cuda.synchronize()
    for b in sampled:
        gu.check_seq_state(S, b, orc[b], f"{name} prefill end")


def _states_and_oracles(w, specs, seed, gate_group):
    states, oracles = [], []
    for b, (t0, n) in enumerate(specs):
        w1 = w.with_(B=1, t0=t0, bank_n=n)
        st = synth.initial_state(w1, seed + b)
        states.append(st)
        oracles.append(OracleState.from_synth(st, H=w1.H, G=w1.G, d=w1.d, R=w1.R, N=w1.N,
                                              C=w1.C, gate_group=gate_group))
    return states, oracles


@pytest.mark.parametrize("gate", ["head", "group"])
@pytest.mark.parametrize("name", ["ring1_commit1", "bank1_window_max", "draw1", "draw3"])
def test_random_geometry_anchor_query_and_gate(name, gate):
    """The separate anchor query and both gate forms at drawn and edge
    geometries: per-sequence decode of three sequences with a q_anchor
    across their block ends, then a prefill block with a q_anchor for the
    sequences at a block start (the others are left out)."""
    rng, R, N, C = _geometry(name)
    w = BASE.with_(name=name, R=R, N=N, C=C)
    group = gate == "group"
    seed = 120 + zlib.crc32(f"{name}/{gate}".encode()) % 50
    # sequences 0 and 1 start 8 tokens before a block end (so the prefill
    # finds them at a block start), sequence 2 at a drawn offset
    k0 = -(-8 // C)
    specs = [(C * int(rng.integers(k0, k0 + (3 * R) // C + 3)) - 8, int(rng.integers(0, N + 1)))
             for _ in range(2)]
    specs.append((_before_block_end(rng, R, C), int(rng.integers(0, N + 1))))
    gu.log(f"case {name} gate={gate}: R={R} N={N} C={C}; decode_at with q_anchor from {specs}")
    states, oracles = _states_and_oracles(w, specs, seed, group)
    wb = w.with_(B=3)
    S = rma.State(gu.cfg_for(wb, gate=rma.RMA_GATE_GROUP if group else rma.RMA_GATE_HEAD), 3,
                  gu.DEV, start_pos=0, bank_n=0)
    S.buf.zero_()
    for b, st in enumerate(states):
        for r in gu.REGIONS + ("bank_n",):
            S.write(r, st[r], batch=slice(b, b + 1))
    torch.cuda.synchronize()
    wg = synth.gate_weights(wb, seed, per_group=group)
    wg_dev = gu.to_dev(wg[0])
    pos = [t0 for t0, _ in specs]
    for s in range(8):
        x = synth.step_inputs(wb, seed, 0, s)
        qa = synth.anchor_query(wb, seed, 0, s)
        xd = gu.inputs_to_dev(x)
        out = S.decode_step_at(0, torch.tensor(pos, dtype=torch.int32, device=gu.DEV), xd["q"],
                               xd["k"], xd["v"], xd["ck"], xd["cv"], xd["cs"], wg_dev,
                               q_anchor=gu.to_dev(qa))
        for b in range(3):
            o = oracles[b]
            xb = _rows(x, b)
            ref = o.decode_step(0, xb["q"], xb["k"], xb["v"], xb["ck"], xb["cv"], xb["cs"], wg[0],
                                q_anchor=qa[b:b + 1])
            if o.pend_n[0] == o.C:
                o.admit(0)
            gu.check_out(out[b:b + 1], ref, f"{name} {gate} step {s} sequence {b} at {pos[b]}")
            pos[b] += 1
    torch.cuda.synchronize()
    for b in range(3):
        gu.check_seq_state(S, b, oracles[b], f"{name} {gate} decode end")

    # the sequences now at a block start take a prefill block with a q_anchor
    n = _logu(rng, 1, C)
    at_start = [b for b in range(3) if pos[b] % C == 0]
    assert 0 in at_start and 1 in at_start
    gu.log(f"case {name} gate={gate}: prefill_at n={n}, sequences at a block start {at_start}")
    x = synth.block_inputs(wb, seed, 0, 8, n)
    qa = synth.block_anchor_query(wb, seed, 0, 8, n)
    d = gu.inputs_to_dev(x)
    out = torch.full((3, n, w.H, w.d), SENTINEL, dtype=torch.bfloat16, device=gu.DEV)
    S.prefill_block_at(0, torch.tensor(pos, dtype=torch.int32, device=gu.DEV), d["q"], d["k"],
                       d["v"], d["ck"], d["cv"], d["cs"], wg_dev, out=out, q_anchor=gu.to_dev(qa))
    for b in range(3):
        if b not in at_start:
            assert torch.all(out[b].float() == SENTINEL), f"{name}: prefill wrote row {b}"
            continue
        o = oracles[b]
        xb = _rows(x, b)
        ref = o.prefill_block(0, xb["q"], xb["k"], xb["v"], xb["ck"], xb["cv"], xb["cs"], wg[0],
                              q_anchor=qa[b:b + 1])
        if o.pend_n[0] == o.C:
            o.admit(0)
        gu.check_out(out[b:b + 1], ref, f"{name} {gate} prefill sequence {b}",
                      p_bf16_vmax=gu.vmax(o.ring_v, o.bank_v, xb["v"]))
    torch.cuda.synchronize()
    for b in range(3):
        gu.check_seq_state(S, b, oracles[b], f"{name} {gate} prefill end")
