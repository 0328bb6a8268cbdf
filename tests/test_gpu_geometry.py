"""GPU parity at geometries other than EdgeRock's: the largest admit pool
(bank 1,792 + commit 256 = 2,048 keys), the largest window (4,097: a ring
of 4,096 positions, 64 decode tiles), a small odd one (ring 99, bank 40,
commit 16: no tile is full, ragged everywhere) and commit 1 (an admit after
every token).  Decode (lockstep and per-sequence), admit and prefill
against the oracle built with the same geometry."""
import numpy as np
import pytest
import torch

from bounded_memory_decode_amd import rma, synth
from oracle import OracleState
import gpu_util as gu

pytestmark = pytest.mark.gpu

GEOMETRIES = {
    # name: (ring R, bank N, commit C, t0, bank_n, B, steps)
    "max_pool": (1535, 1792, 256, 8192, 1792, 2, 300),
    "max_window": (4096, 1024, 256, 8192, 1024, 2, 300),
    "small_odd": (99, 40, 16, 96, 33, 3, 70),
    "commit_1": (63, 20, 1, 70, 20, 2, 30),
}


def _setup(name, seed):
    R, N, C, t0, bank_n, B, steps = GEOMETRIES[name]
    w = synth.WORKLOADS["layer_b1"].with_(name=name, B=B, R=R, N=N, C=C, t0=t0, bank_n=bank_n,
                                          steps=steps)
    st = synth.initial_state(w, seed)
    S = gu.gpu_state(w, st)
    S.write("bank_n", st["bank_n"])
    o = OracleState.from_synth(st, H=w.H, G=w.G, d=w.d, R=R, N=N, C=C)
    torch.cuda.synchronize()
    return w, S, o


@pytest.mark.parametrize("name", list(GEOMETRIES))
def test_decode_and_admit_at_other_geometries(name):
    """Lockstep decode with an admit at every block end, over several
    blocks; every output and the final state bit for bit."""
    gu.log(f"case geometry {name}: lockstep decode + admit")
    seed = 80
    w, S, o = _setup(name, seed)
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    admits = 0
    for s in range(w.steps):
        x = synth.step_inputs(w, seed, 0, s)
        out = gu.decode(S, 0, gu.inputs_to_dev(x), wg_dev)
        ref = o.decode_step(0, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[0])
        gu.check_out(out, ref, f"{name} step {s}")
        if o.pend_n[0] == w.C:
            S.admit(0)
            o.admit(0)
            admits += 1
    torch.cuda.synchronize()
    gu.check_state(S, o, f"{name} end")
    assert admits >= 1


@pytest.mark.parametrize("name", ["max_pool", "max_window", "small_odd"])
def test_per_sequence_decode_and_prefill_at_other_geometries(name):
    """Per-sequence calls at these geometries: a prefill block from a block
    start (admitted in the call when full), then decode steps across the
    next block end; every output and the final state."""
    gu.log(f"case geometry {name}: prefill_at + decode_at")
    seed = 81
    w, S, o = _setup(name, seed)
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    assert w.t0 % w.C == 0
    pos = torch.full((w.B,), w.t0, dtype=torch.int32, device=gu.DEV)
    n = w.C
    x = synth.block_inputs(w, seed, 0, 0, n)
    d = gu.inputs_to_dev(x)
    vm = gu.vmax(o.ring_v, o.bank_v, x["v"])
    out = S.prefill_block_at(0, pos, d["q"], d["k"], d["v"], d["ck"], d["cv"], d["cs"], wg_dev)
    ref = o.prefill_block(0, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[0])
    o.admit(0)
    gu.check_out(out, ref, f"{name} prefill", p_bf16_vmax=vm)
    pos += n
    for s in range(w.C + 3):
        xs = synth.step_inputs(w, seed, 0, n + s)
        xd = gu.inputs_to_dev(xs)
        outd = S.decode_step_at(0, pos, xd["q"], xd["k"], xd["v"], xd["ck"], xd["cv"], xd["cs"],
                                wg_dev)
        refd = o.decode_step(0, xs["q"], xs["k"], xs["v"], xs["ck"], xs["cv"], xs["cs"], wg[0])
        if o.pend_n[0] == w.C:
            o.admit(0)
        gu.check_out(outd, refd, f"{name} decode_at step {s}")
        pos += 1
    torch.cuda.synchronize()
    for b in range(w.B):
        for region in gu.REGIONS + ("bank_n",):
            g = gu.bits(S.read(region, slice(None), slice(b, b + 1)))
            r = getattr(o, region)[:, b:b + 1]
            if r.dtype == np.uint16:
                r = r.view(np.int16)
            if r.dtype == np.float32:
                g, r = g.view(np.uint32), r.view(np.uint32)
            assert np.array_equal(g, r), f"{name}: sequence {b} region {region}"
