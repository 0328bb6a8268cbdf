"""GPU parity of the chunked-prefill block (MFMA path) against the CPU
oracle, which defines a block as its tokens decoded in order with no admit
inside; plus prefill/decode equivalence on the GPU itself."""
import numpy as np
import pytest
import torch

from bounded_memory_decode_amd import rma, synth
from oracle import OracleState
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _prefill(S, layer, x, wg_dev):
    d = gu.inputs_to_dev(x)
    return S.prefill_block(layer, d["q"], d["k"], d["v"], d["ck"], d["cv"], d["cs"], wg_dev)


def _run_blocks(w, seed, sizes, decode_after=0, check_state_each=True):
    """Prefill blocks of the given sizes (each starting on a block
    boundary: a short block is completed by decode steps), admitting at
    every block end; compare every output and the state."""
    st = synth.initial_state(w, seed)
    S = gu.gpu_state(w, st)
    o = OracleState.from_synth(st, H=w.H, G=w.G, d=w.d, R=w.R, N=w.N, C=w.C)
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    step = 0
    worst = 0.0
    for n in sizes:
        x = synth.block_inputs(w, seed, 0, step, n)
        vm = gu.vmax(o.ring_v, o.bank_v, x["v"])
        out = _prefill(S, 0, x, wg_dev)
        ref = o.prefill_block(0, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[0])
        e, _ = gu.check_out(out, ref, f"{w.name} prefill n={n} at step {step}", p_bf16_vmax=vm)
        worst = max(worst, e)
        step += n
        # finish the block with decode steps, then admit
        while o.pend_n[0] < w.C:
            xs = synth.step_inputs(w, seed, 0, step)
            outd = gu.decode(S, 0, gu.inputs_to_dev(xs), wg_dev)
            refd = o.decode_step(0, xs["q"], xs["k"], xs["v"], xs["ck"], xs["cv"], xs["cs"], wg[0])
            gu.check_out(outd, refd, f"{w.name} decode after prefill, step {step}")
            step += 1
        if check_state_each:
            torch.cuda.synchronize()
            gu.check_state(S, o, f"{w.name} block ending at {step}")
        S.admit(0)
        o.admit(0)
    for _ in range(decode_after):
        xs = synth.step_inputs(w, seed, 0, step)
        outd = gu.decode(S, 0, gu.inputs_to_dev(xs), wg_dev)
        refd = o.decode_step(0, xs["q"], xs["k"], xs["v"], xs["ck"], xs["cv"], xs["cs"], wg[0])
        gu.check_out(outd, refd, f"{w.name} decode step {step}")
        step += 1
    torch.cuda.synchronize()
    gu.check_state(S, o, f"{w.name} end")
    gu.log(f"{w.name}: blocks {sizes}, worst prefill error {worst:.3e}")


def test_full_block_on_full_history():
    gu.log("case prefill full block, B=2, full ring and bank")
    w = synth.WORKLOADS["layer_b1"].with_(B=2)
    _run_blocks(w, 50, [256, 256], decode_after=3)


def test_ragged_blocks_and_query_tile_edges():
    """Blocks of 1, 17, 100 and 255 tokens (query tiles of 16 tokens with
    ragged tails), each completed by decode steps."""
    gu.log("case prefill ragged blocks")
    w = synth.WORKLOADS["layer_b1"].with_(B=1, bank_n=600)
    _run_blocks(w, 51, [1, 17, 100, 255])


def test_from_empty_history():
    """Position 0: the ring fills over the first four blocks (P < R), the
    bank starts empty and grows by 256 per admit."""
    gu.log("case prefill from empty history")
    w = synth.WORKLOADS["layer_b1"].with_(B=2, t0=0, bank_n=0, ring_full=False)
    _run_blocks(w, 52, [256, 256, 256, 256, 256], decode_after=2)


def test_sharp_inputs():
    gu.log("case prefill sharp")
    w = synth.WORKLOADS["sharp_b1"]
    _run_blocks(w, 53, [256, 130])


def test_prefill_equals_decode_on_gpu():
    """The same 256 tokens through one prefill call and through 256 decode
    calls: identical state bit for bit, outputs within the bound."""
    gu.log("case prefill == decode")
    w = synth.WORKLOADS["layer_b1"].with_(B=3, bank_n=900)
    seed = 54
    st = synth.initial_state(w, seed)
    A = gu.gpu_state(w, st)
    D = gu.gpu_state(w, st)
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    x = synth.block_inputs(w, seed, 0, 0, w.C)
    outp = _prefill(A, 0, x, wg_dev)
    outs = []
    for i in range(w.C):
        xs = {k: v[:, i] for k, v in x.items()}
        outs.append(gu.decode(D, 0, gu.inputs_to_dev(xs), wg_dev).clone())
    outd = torch.stack(outs, dim=1)
    err = (outp.float() - outd.float()).abs().max().item()
    scale = outd.float().abs().max().item()
    assert err <= 2e-2 and err <= 1e-2 * scale, err
    torch.cuda.synchronize()
    for name in gu.REGIONS + ("bank_n",):
        assert torch.equal(A.read(name), D.read(name)), name
    assert A.t == D.t and A.pend_n == D.pend_n


@pytest.mark.parametrize("n", [256, 60])
@pytest.mark.parametrize("B", [2, 4, 8])
def test_launch_plans(B, n):
    """The launch plans above batch 1: batch 2 splits each query tile's
    local and anchor reads in 2 slices each, batch 4 in 1 each (one
    workgroup per read), batch 8 runs unsplit; a full block and a 60-token
    one (its last query tile partial).  Sequences at their own
    block-aligned positions (per-sequence call); two sampled sequences (a
    full history and an empty or short one) against one-sequence oracles,
    outputs and state."""
    from test_gpu_positions import _rows, _seq_oracles
    gu.log(f"case prefill batch {B}, n={n}")
    base = synth.WORKLOADS["layer_b1"]
    specs = [(32768, 1024), (33024, 700), (256, 0), (1024, 1024), (32768, 512), (0, 0),
             (4096, 1000), (768, 64)]
    specs = specs[:B] if B >= 6 else [specs[0], specs[5], specs[1], specs[7]][:B]
    sampled = (0, 5) if B >= 6 else (0, 1)
    seed = 56
    states, oracles = _seq_oracles(base, specs, seed)
    w = base.with_(B=len(specs))
    S = gu.assemble_state(w, states)
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    x = synth.block_inputs(w, seed, 0, 0, n)
    d = gu.inputs_to_dev(x)
    pos = torch.tensor([t0 for t0, _ in specs], dtype=torch.int32, device=gu.DEV)
    out = S.prefill_block_at(0, pos, d["q"], d["k"], d["v"], d["ck"], d["cv"], d["cs"], wg_dev)
    for b in sampled:
        o = oracles[b]
        xb = _rows(x, b)
        vm = gu.vmax(o.ring_v, o.bank_v, xb["v"])
        ref = o.prefill_block(0, xb["q"], xb["k"], xb["v"], xb["ck"], xb["cv"], xb["cs"], wg[0])
        if o.pend_n[0] == o.C:
            o.admit(0)
        gu.check_out(out[b:b + 1], ref, f"batch {B} prefill n={n} sequence {b}", p_bf16_vmax=vm)
    torch.cuda.synchronize()
    for b in sampled:
        gu.check_seq_state(S, b, oracles[b], f"batch {B} prefill n={n}")
