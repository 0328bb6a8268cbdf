"""The long single-sequence path on the GPU against the CPU oracle: a
131,072-token prompt fed in 256-token prefill blocks through 8 RMA layers
(all layers admitted after every block), then decode.

The committed state (ring, bank, pending, scores, source positions) is a
function of the inputs alone, never of the attention outputs, so the
oracle can follow the whole prompt without computing its outputs: it
replays every block's writes and admits (state only) and computes outputs
where they are checked.

  - the first 8 blocks: every output of every layer, the bank metadata
    after every admit, the whole state at the end;
  - the whole prompt, then 2,048 decode tokens: the bank metadata after
    every admit (520 of them), the whole state at five points of the
    prompt and at the end, the outputs of the prompt's last block (two
    layers) and of every 16th decode token (all layers).
"""
import numpy as np
import pytest
import torch

from bounded_memory_decode_amd import synth
from oracle import OracleState
import gpu_util as gu

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS["long_b1"]
META = ("bscore", "bsrc", "bank_n")


def _host(x: dict) -> dict:
    """Device inputs -> numpy (bf16 as uint16 bits, scores as float32)."""
    out = {}
    for k, v in x.items():
        if v.dtype == torch.bfloat16:
            out[k] = v.view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            out[k] = v.cpu().numpy()
    return out


def _check_meta(S, o, tag):
    for name in META:
        g = gu.bits(S.read(name))
        r = getattr(o, name)
        if r.dtype == np.float32:
            g, r = g.view(np.uint32), r.view(np.uint32)
        if not np.array_equal(g, r):
            idx = np.argwhere(g != r)
            raise AssertionError(f"{tag}: {name} differs at {len(idx)} places, first "
                                 f"{idx[0].tolist()}")


def _setup(seed):
    st = synth.initial_state(W, seed)
    S = gu.gpu_state(W, st)
    o = OracleState.from_synth(st)
    wg = synth.gate_weights(W, seed)
    wg_dev = [gu.to_dev(wg[l]) for l in range(W.L)]
    return S, o, wg, wg_dev


def _admit_all(S, o):
    S.admit(-1)
    for l in range(W.L):
        o.admit(l)


def test_long_prompt_first_eight_blocks():
    """The prompt's first 8 blocks (positions 0 .. 2,047) through all 8
    layers from an empty history: the ring fills during the first four
    blocks and the bank grows by 256 records per admit until it is full.
    Every output of every block and layer against the oracle."""
    gu.log("case long prompt: first 8 blocks x 8 layers, every output")
    seed = 55
    S, o, wg, wg_dev = _setup(seed)
    worst = 0.0
    for blk in range(8):
        for l in range(W.L):
            x = synth.torch_block_inputs(W, seed, l, blk, gu.DEV)
            xh = _host(x)
            vm = gu.vmax(o.ring_v[l], o.bank_v[l], xh["v"])
            out = S.prefill_block(l, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg_dev[l])
            ref = o.prefill_block(l, xh["q"], xh["k"], xh["v"], xh["ck"], xh["cv"], xh["cs"],
                                  wg[l])
            e, _ = gu.check_out(out, ref, f"long block {blk} layer {l}", p_bf16_vmax=vm)
            worst = max(worst, e)
        _admit_all(S, o)
        torch.cuda.synchronize()
        _check_meta(S, o, f"long admit after block {blk}")
        assert all(int(n) == min(W.N, W.C * (blk + 1)) for n in o.bank_n.ravel())
    gu.check_state(S, o, "long after 8 blocks")
    gu.log(f"long prompt, first 8 blocks: worst output error {worst:.3e}")


def test_long_prompt_whole_then_decode():
    """The whole 131,072-token prompt (512 blocks x 8 layers, an admit of
    all layers after each block), then 2,048 decode tokens (8 more
    admits)."""
    seed = 57
    blocks, decode_steps, sample_every = 512, 2048, 16
    S, o, wg, wg_dev = _setup(seed)
    full_checks = {0, 127, 255, 383, blocks - 1}
    zero_q = np.zeros((1, W.C, W.H, W.d), np.uint16)
    gu.log(f"case long prompt: {blocks} blocks x {W.L} layers, state replay")
    for blk in range(blocks):
        last = blk == blocks - 1
        for l in range(W.L):
            x = synth.torch_block_inputs(W, seed, l, blk, gu.DEV)
            out = S.prefill_block(l, x["q"], x["k"], x["v"], x["ck"], x["cv"], x["cs"], wg_dev[l])
            with_out = last and l in (0, W.L - 1)
            if not with_out:
                del x["q"]
            xh = _host(x)
            if with_out:
                vm = gu.vmax(o.ring_v[l], o.bank_v[l], xh["v"])
                ref = o.prefill_block(l, xh["q"], xh["k"], xh["v"], xh["ck"], xh["cv"], xh["cs"],
                                      wg[l])
                gu.check_out(out, ref, f"long block {blk} layer {l}", p_bf16_vmax=vm)
            else:
                o.prefill_block(l, zero_q, xh["k"], xh["v"], xh["ck"], xh["cv"], xh["cs"], wg[l],
                                compute_out=False)
        if blk in full_checks:
            torch.cuda.synchronize()
            gu.check_state(S, o, f"long before the admit of block {blk}")
        _admit_all(S, o)
        torch.cuda.synchronize()
        _check_meta(S, o, f"long admit after block {blk}")
        if blk in full_checks:
            gu.check_state(S, o, f"long after the admit of block {blk}")
        if blk % 64 == 63:
            gu.log(f"long prompt: {blk + 1} blocks")
    assert S.t == [blocks * W.C] * W.L

    gu.log(f"case long decode: {decode_steps} tokens after the prompt")
    checked = 0
    for j in range(decode_steps // W.C):
        blk = blocks + j
        xs = [synth.torch_block_inputs(W, seed, l, blk, gu.DEV) for l in range(W.L)]
        xh = [_host(x) for x in xs]
        for i in range(W.C):
            step = j * W.C + i
            sampled = step % sample_every == 0
            for l in range(W.L):
                xd = {k: v[:, i].contiguous() for k, v in xs[l].items()}
                out = gu.decode(S, l, xd, wg_dev[l])
                xi = {k: np.ascontiguousarray(v[:, i]) for k, v in xh[l].items()}
                ref = o.decode_step(l, xi["q"], xi["k"], xi["v"], xi["ck"], xi["cv"], xi["cs"],
                                    wg[l], compute_out=sampled)
                if sampled:
                    gu.check_out(out, ref, f"long decode token {step} layer {l}")
                    checked += 1
        _admit_all(S, o)
        torch.cuda.synchronize()
        _check_meta(S, o, f"long decode admit {j}")
    torch.cuda.synchronize()
    gu.check_state(S, o, "long end")
    assert checked == decode_steps // sample_every * W.L
    gu.log(f"long path: {blocks} blocks + {decode_steps} tokens, {checked} decode outputs checked")
