"""GPU parity of the decode path (local read, anchor read, gate, ring write,
pending append) and of admit inside decode trajectories, through the C ABI,
against the CPU oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

from bounded_memory_decode_amd import rma, synth
from oracle import OracleState
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run_trajectory(w, seed, steps, check_every=1, state_at_admit=True, out_batch=None):
    """Decode `steps` tokens of layer 0 on both sides, admitting at every
    block end; compare outputs (for `out_batch` sequences every
    `check_every` steps) and the whole state after every admit."""
    st = synth.initial_state(w, seed)
    S = gu.gpu_state(w, st)
    o_state = OracleState.from_synth(st, H=w.H, G=w.G, d=w.d, R=w.R, N=w.N, C=w.C)
    ob = list(range(w.B)) if out_batch is None else list(out_batch)
    o_out = OracleState.from_synth(synth.initial_state(w, seed, batch=ob), H=w.H, G=w.G, d=w.d,
                                   R=w.R, N=w.N, C=w.C) if out_batch is not None else o_state
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    worst = 0.0
    for s in range(steps):
        x = synth.step_inputs(w, seed, 0, s)
        out = gu.decode(S, 0, gu.inputs_to_dev(x), wg_dev)
        want = (s % check_every == 0) or (s == steps - 1)
        if out_batch is not None:
            o_state.decode_step(0, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[0],
                                compute_out=False)
            xs = {k: v[ob] for k, v in x.items()}
            ref = o_out.decode_step(0, xs["q"], xs["k"], xs["v"], xs["ck"], xs["cv"], xs["cs"],
                                    wg[0], compute_out=want)
        else:
            ref = o_state.decode_step(0, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[0],
                                      compute_out=want)
        if want:
            e, _ = gu.check_out(out[ob], ref, f"{w.name} step {s}")
            worst = max(worst, e)
        if o_state.pend_n[0] == w.C:
            S.admit(0)
            o_state.admit(0)
            if out_batch is not None:
                o_out.admit(0)
            if state_at_admit:
                torch.cuda.synchronize()
                gu.check_state(S, o_state, f"{w.name} after admit at step {s}")
    torch.cuda.synchronize()
    gu.check_state(S, o_state, f"{w.name} end")
    gu.log(f"{w.name}: {steps} steps, worst output error {worst:.3e}")
    return worst


@pytest.mark.parametrize("B,kind", [(300, "two launches: 256 whole-unit sequences, 44 split"),
                                     (448, "whole-unit, a partial second round")])
def test_launch_shapes_large_batch(B, kind):
    """Launch shapes that depend only on the number of units, run on a small
    geometry (ring 63, bank 64, commit 16) so that every sequence's state
    and outputs can be checked: batch 300 (1,200 units; a second round of
    whole units would leave most waves idle, so sequences 0-255 take the
    whole-unit launch and 256-299 the split launch of a batch of 44) and
    448 (1,792 units: whole units in one-wave workgroups, the second round
    partial).  40 steps across three block ends; every output every 4th step,
    the whole state at each admit and at the end."""
    gu.log(f"case launch shape B={B} ({kind})")
    w = synth.WORKLOADS["layer_b1"].with_(name=f"shape_b{B}", B=B, R=63, N=64, C=16,
                                          t0=64 * 16 + 5, bank_n=64, steps=40)
    _run_trajectory(w, 9, 40, check_every=4)


def test_layer_b1_512_steps_two_admits():
    """One layer, batch 1, ring and bank full, 512 decode steps with two
    admits; every output and the whole state after each admit."""
    gu.log("case layer_b1 seed 0")
    _run_trajectory(synth.WORKLOADS["layer_b1"], 0, 512)


def test_sharp_inputs():
    """q, K, V ~ N(0,1): peaked softmaxes, gate arguments of order one, so
    the 2e-2 bound is a real constraint."""
    gu.log("case sharp_b1 seed 1")
    _run_trajectory(synth.WORKLOADS["sharp_b1"], 1, 300)


def test_from_empty_history_ragged():
    """Start at position 0 with an empty ring and bank: the local window
    grows one key at a time (ragged tiles, t < ring size), the bank is
    empty for the first block and then partially filled (n = 256, 512)."""
    gu.log("case empty start B=2 seed 2")
    w = synth.WORKLOADS["layer_b1"].with_(B=2, t0=0, bank_n=0, ring_full=False)
    _run_trajectory(w, 2, 600, check_every=3)


def test_partial_bank_ragged_tail():
    """A bank of 300 anchors (not a multiple of the 64-key tile) and a
    ring of 200 filled slots."""
    gu.log("case partial bank seed 3")
    w = synth.WORKLOADS["layer_b1"].with_(B=3, t0=256, bank_n=300, ring_full=False)
    _run_trajectory(w, 3, 70)


def test_sharp_from_empty_history():
    gu.log("case sharp empty start seed 4")
    w = synth.WORKLOADS["sharp_b1"].with_(t0=0, bank_n=0, ring_full=False)
    _run_trajectory(w, 4, 300, check_every=2)


def test_layer_b64_2048_steps_eight_admits():
    """One layer, batch 64, 2,048 steps (8 admits): outputs of 3 sampled
    sequences every 8th step, the whole state of all 64 after every
    admit."""
    gu.log("case layer_b64 seed 0")
    _run_trajectory(synth.WORKLOADS["layer_b64"], 0, 2048, check_every=8,
                    out_batch=[0, 29, 63])


def test_new_anchor_invisible_until_next_block():
    """A candidate with a huge score and a key aligned with the next
    block's first query: every output of its own block is bit-identical to
    a run without it; the first output of the next block changes."""
    gu.log("case visibility")
    w = synth.WORKLOADS["layer_b1"]
    seed = 5
    st = synth.initial_state(w, seed)
    A = gu.gpu_state(w, st)
    Bst = gu.gpu_state(w, st)
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    xf = synth.step_inputs(w, seed, 0, w.C)
    h, g = 6, 1
    plant_k = synth.bf16_bits(1024.0 * synth.bf16_to_f32(xf["q"][0, h]))
    for s in range(w.C):
        x = synth.step_inputs(w, seed, 0, s)
        a = gu.decode(A, 0, gu.inputs_to_dev(x), wg_dev).clone()
        if s == 3:
            x["ck"][0, g] = plant_k
            x["cs"][0, g] = 1e30
        b = gu.decode(Bst, 0, gu.inputs_to_dev(x), wg_dev).clone()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"step {s}"
    A.admit(0)
    Bst.admit(0)
    x = gu.inputs_to_dev(synth.step_inputs(w, seed, 0, w.C))
    a = gu.decode(A, 0, x, wg_dev).float()
    b = gu.decode(Bst, 0, x, wg_dev).float()
    assert (a[0, h] - b[0, h]).abs().max().item() > 1e-3
    assert torch.equal(a[0, :4], b[0, :4])
    bsrc = Bst.read("bsrc")[0, 0, g].cpu().numpy()
    assert (bsrc == w.t0 + 3).sum() == 1


def test_pending_full_is_reported_and_state_unchanged():
    w = synth.WORKLOADS["layer_b1"]
    seed = 6
    st = synth.initial_state(w, seed)
    S = gu.gpu_state(w, st)
    wg_dev = gu.to_dev(synth.gate_weights(w, seed)[0])
    for s in range(w.C):
        gu.decode(S, 0, gu.inputs_to_dev(synth.step_inputs(w, seed, 0, s)), wg_dev)
    x = gu.inputs_to_dev(synth.step_inputs(w, seed, 0, w.C))
    with pytest.raises(rma.RmaError) as e:
        gu.decode(S, 0, x, wg_dev)
    assert e.value.code == rma.RMA_E_PENDING_FULL
    assert S.t[0] == w.t0 + w.C and S.pend_n[0] == w.C
    S.admit(0)
    gu.decode(S, 0, x, wg_dev)
    assert S.t[0] == w.t0 + w.C + 1


@pytest.mark.parametrize("B,out_batch", [(16, [0, 9, 15]), (64, [0, 37, 63]),
                                         (144, [0, 77, 143]), (160, [0, 77, 159])])
def test_launch_shapes(B, out_batch):
    """Batch sizes whose launch differs from the other tests: 16 (the
    one-tile part kernel with 2,048 parts), 64 and 144 (8-tile and 2-tile
    parts of the persistent kernel) and 160 (the whole-unit kernel with 640
    units, fewer than its resident waves, in four-wave workgroups).  40
    steps across a block end; sampled outputs every 5th step, the whole
    state at the admit and at the end."""
    gu.log(f"case launch shape B={B}")
    w = synth.WORKLOADS["layer_b1"].with_(name=f"split_b{B}", B=B, t0=32768 + 230, steps=40)
    _run_trajectory(w, 7, 40, check_every=5, out_batch=out_batch)
