"""GPU parity at batch sizes where the decode step runs as one launch per
layer (a wave owns a whole (sequence, group) unit), including the exact
configuration bench.py times: 512 sequences x 8 layers, state drawn on the
device.  Sampled sequences are checked against the CPU oracle; the oracle
gets copies of the generated inputs taken before any kernel ran."""
import numpy as np
import pytest
import torch

import bench
from bounded_memory_decode_amd import rma, synth
from oracle import OracleState
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle_from_device(S: rma.State, w, batch):
    o = OracleState(L=w.L, B=len(batch), H=w.H, G=w.G, d=w.d, R=w.R, N=w.N, C=w.C)
    for name in ("ring_k", "ring_v", "bank_k", "bank_v", "pend_k", "pend_v"):
        getattr(o, name)[...] = S.read(name, batch=batch).cpu().numpy().view(np.uint16)
    for name in ("bscore", "bsrc", "pscore", "bank_n"):
        getattr(o, name)[...] = S.read(name, batch=batch).cpu().numpy()
    o.t[:] = S.t[:w.L]
    o.pend_n[:] = S.pend_n[:w.L]
    return o


def test_whole_unit_batch256_from_empty_history():
    """256 sequences (1,024 units): one launch per token.  Start at
    position 0 (empty ring and bank), 300 tokens, one admit; sampled
    outputs every 5th token, the whole state of every sequence at the end."""
    gu.log("case whole-unit B=256 from empty history")
    w = synth.WORKLOADS["layer_b1"].with_(B=256, t0=0, bank_n=0, ring_full=False)
    seed = 41
    st = synth.initial_state(w, seed)
    S = gu.gpu_state(w, st)
    o_all = OracleState.from_synth(st)
    sample = [0, 97, 255]
    o_s = OracleState.from_synth(synth.initial_state(w, seed, batch=sample))
    wg = synth.gate_weights(w, seed)
    wg_dev = gu.to_dev(wg[0])
    for s in range(300):
        x = synth.step_inputs(w, seed, 0, s)
        out = gu.decode(S, 0, gu.inputs_to_dev(x), wg_dev)
        o_all.decode_step(0, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg[0],
                          compute_out=False)
        xs = {k: v[sample] for k, v in x.items()}
        want = s % 5 == 0 or s in (255, 256)
        ref = o_s.decode_step(0, xs["q"], xs["k"], xs["v"], xs["ck"], xs["cv"], xs["cs"], wg[0],
                              compute_out=want)
        if want:
            gu.check_out(out[sample], ref, f"B=256 step {s}")
        if o_all.pend_n[0] == w.C:
            S.admit(0)
            o_all.admit(0)
            o_s.admit(0)
    torch.cuda.synchronize()
    gu.check_state(S, o_all, "B=256 end")


@pytest.mark.parametrize("bank_n", [1024, 555])
def test_bench_configuration_batch512_8_layers(bank_n):
    """The launch configuration bench.py times: 512 sequences x 8 layers,
    ring full, bank full (or partial), starting 3 tokens before a block
    end; 6 tokens through all layers, so every layer is admitted after the
    third.  Sampled sequences: outputs of every layer and token, and their
    whole state at the end, bit for bit.  Every sequence: the admit's
    selection (scores, source positions, counts of all 512 x 8 x 4 groups)
    against an oracle that carries the same scores with stand-in records
    of width 2 (the selection depends on the scores alone)."""
    gu.log(f"case bench configuration bank_n={bank_n}")
    w = synth.WORKLOADS["stack_b512"].with_(bank_n=bank_n, t0=32768 - 3)
    seed = 3
    dev = torch.device("cuda", 0)
    S = bench.make_state(w, seed, dev)
    sets, wg, outs = bench.make_pool(w, seed, dev, pool=6)
    sample = [0, 257, 511]
    o = _oracle_from_device(S, w, sample)
    # all sequences, scores only
    oa = OracleState(L=w.L, B=w.B, H=w.H, G=w.G, d=2, R=w.R, N=w.N, C=w.C)
    for name in ("bscore", "bsrc", "pscore", "bank_n"):
        getattr(oa, name)[...] = S.read(name).cpu().numpy()
    oa.t[:] = S.t[:w.L]
    oa.pend_n[:] = S.pend_n[:w.L]
    assert oa.pend_n[0] == w.C - 3
    wgn = wg.cpu().numpy()
    ins = [[{k: (_host_bits(v[sample]) if v.dtype == torch.bfloat16 else v[sample].cpu().numpy())
             for k, v in sets[l][p].items()} for p in range(6)] for l in range(w.L)]
    rec2 = np.zeros((w.B, w.G, 2), np.uint16)
    admitted = 0
    for step in range(6):
        admitted += bench.run_step(S, sets, wg, outs, step)
        torch.cuda.synchronize()
        for l in range(w.L):
            x = ins[l][step]
            ref = o.decode_step(l, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wgn[l])
            gu.check_out(outs[l][sample], ref, f"bench config step {step} layer {l}")
            cs = sets[l][step]["cs"].cpu().numpy()
            oa.decode_step(l, np.zeros((w.B, w.H, 2), np.uint16), rec2, rec2, rec2, rec2, cs,
                           np.zeros((w.H, 2), np.float32), compute_out=False)
        if o.pend_n[0] == w.C:
            for l in range(w.L):
                o.admit(l)
                oa.admit(l)
    assert admitted == 1
    for name in gu.REGIONS + ("bank_n",):
        g = gu.bits(S.read(name, batch=sample))
        r = getattr(o, name)
        r = r.view(np.int16) if r.dtype == np.uint16 else r
        if r.dtype == np.float32:
            g, r = g.view(np.uint32), r.view(np.uint32)
        assert np.array_equal(g, r), f"sampled sequences: {name}"
    assert S.t == list(o.t) and S.pend_n == list(o.pend_n)
    for name in ("bscore", "bsrc", "bank_n"):
        g = gu.bits(S.read(name))
        r = getattr(oa, name)
        if r.dtype == np.float32:
            g, r = g.view(np.uint32), r.view(np.uint32)
        assert np.array_equal(g, r), f"all sequences: {name}"
