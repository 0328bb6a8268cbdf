"""The allocation-free decode entry point (rma_decode_step_at_static)
against rma_decode_step_at: same inputs, same positions, two identical
states; the outputs and every state region must agree bit for bit.  Calls
in a row with ever smaller batches (the static array keeps the previous
call's partials): batch 300 (two launches, the second split), 152 (the
largest partials of any accepted configuration), 32 and 4."""
import numpy as np
import pytest
import torch

from bounded_memory_decode_amd import rma, synth
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run_pair(B, seed, steps, anchor_query):
    w = synth.WORKLOADS["layer_b1"].with_(B=B, bank_n=900)
    st = synth.initial_state(w, seed)
    A = gu.gpu_state(w, st)   # allocation-free entry point
    D = gu.gpu_state(w, st)   # the entry point it is a variant of
    wg = gu.to_dev(synth.gate_weights(w, seed)[0])
    # positions a few tokens before a block end, so that some sequences
    # complete their block (and are admitted) inside the run
    pos0 = torch.tensor([w.t0 - 3 + (b % 5) for b in range(B)], dtype=torch.int32,
                        device=gu.DEV)
    pa, pd = pos0.clone(), pos0.clone()
    oa = torch.empty((B, w.H, w.d), dtype=torch.bfloat16, device=gu.DEV)
    od = torch.empty_like(oa)
    for s in range(steps):
        x = gu.inputs_to_dev(synth.step_inputs(w, seed, 0, s))
        qa = gu.to_dev(synth.anchor_query(w, seed, 0, s)) if anchor_query else None
        A.decode_step_at_static(0, pa, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg, oa,
                                q_anchor=qa)
        D.decode_step_at(0, pd, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg, od,
                         q_anchor=qa)
        assert torch.equal(oa.view(torch.int16), od.view(torch.int16)), f"batch {B} step {s}"
        pa += 1
        pd += 1
    torch.cuda.synchronize()
    for name in gu.REGIONS + ("bank_n",):
        assert torch.equal(A.read(name), D.read(name)), f"batch {B}: region {name}"


def test_static_scratch_decode_matches_state_scratch_decode():
    gu.log("case allocation-free decode: batch 300, then 152, 32 and 4")
    _run_pair(300, 89, 4, anchor_query=False)  # whole-unit launch for 256, split for 44
    _run_pair(152, 88, 4, anchor_query=False)  # the largest need: 608 units x 32 parts, 76.6 MiB
    _run_pair(32, 90, 6, anchor_query=False)   # one-tile parts: 16.1 MiB of partials
    _run_pair(4, 91, 6, anchor_query=True)     # smaller input, separate anchor query

