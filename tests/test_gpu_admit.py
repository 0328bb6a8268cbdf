"""GPU parity of the admit step (top-min(N, n+C) selection with the
deterministic tie-break, in-place compaction) against the CPU oracle,
bit for bit, including heavy ties (scores on 64 integer levels)."""
import numpy as np
import pytest
import torch

from bounded_memory_decode_amd import rma, synth
from oracle import OracleState
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _admit_case(w, seed, bank_n, layers=None, mutate=None):
    w = w.with_(bank_n=bank_n)
    st = synth.initial_state(w, seed)
    pf = synth.pending_fill(w, seed)
    st.update(pf)
    if mutate is not None:
        mutate(st)
    # a full pending block at position t0 + C
    w2 = w.with_(t0=w.t0 + w.C)
    S = rma.State(gu.cfg_for(w2), w2.B, gu.DEV, start_pos=w2.t0, bank_n=bank_n)
    for name in gu.REGIONS:
        S.write(name, st[name])
    # the state starts on a block boundary with no candidates; mark the
    # pending block as full the way decode would have left it
    for l in range(w.L):
        S._st.pend_n[l] = w.C
    o = OracleState.from_synth({**st, "t0": np.int64(w2.t0)}, H=w.H, G=w.G, d=w.d, R=w.R,
                               N=w.N, C=w.C)
    o.pend_n[:] = w.C
    return S, o


@pytest.mark.parametrize("bank_n", [1024, 1000, 800, 768, 300, 0])
def test_admit_bit_exact_heavy_ties(bank_n):
    gu.log(f"case admit B=8 L=8 bank_n={bank_n}")
    w = synth.WORKLOADS["admit_b512"].with_(B=8)
    S, o = _admit_case(w, 31, bank_n)
    S.admit(-1)
    for l in range(w.L):
        o.admit(l)
    torch.cuda.synchronize()
    gu.check_state(S, o, f"admit bank_n={bank_n}")
    assert S.bank_n == [min(w.N, bank_n + w.C)] * w.L


# Scores the total order has to place by rule: quiet NaNs of several
# payloads and both signs (all equal, below -inf), +-inf, +-0 (equal),
# the smallest denormals, the largest finite values and +-1.  Quiet NaNs
# only: their bits survive every host copy unchanged.
_SPECIAL_SCORES = np.array([0x7FC00000, 0xFFC00000, 0x7FC12345, 0x7F800000, 0xFF800000,
                            0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x7F7FFFFF,
                            0xFF7FFFFF, 0x3F800000, 0xBF800000], np.uint32).view(np.float32)


@pytest.mark.parametrize("bank_n", [1024, 900, 0])
def test_admit_special_scores_bit_exact(bank_n):
    """Bank and pending scores drawn, with heavy repetition, from NaNs,
    infinities, signed zeros, denormals and the extreme finite values: the
    kept set (score descending, then global index ascending, NaNs below
    -inf, -0 equal to +0), the compaction and every moved record and score
    (NaN payloads included) match the oracle bit for bit."""
    gu.log(f"case admit special scores bank_n={bank_n}")
    rng = np.random.default_rng(77 + bank_n)

    def mutate(st):
        for name in ("bscore", "pscore"):
            st[name] = _SPECIAL_SCORES[rng.integers(0, len(_SPECIAL_SCORES),
                                                    size=st[name].shape)].copy()

    w = synth.WORKLOADS["admit_b512"].with_(B=4, L=2)
    S, o = _admit_case(w, 41, bank_n, mutate=mutate)
    S.admit(-1)
    for l in range(w.L):
        o.admit(l)
    torch.cuda.synchronize()
    gu.check_state(S, o, f"admit special scores bank_n={bank_n}")


def test_admit_one_layer_at_a_time():
    gu.log("case admit per layer")
    w = synth.WORKLOADS["admit_b512"].with_(B=4, L=3, scores="normal")
    S, o = _admit_case(w, 32, 1024)
    for l in (2, 0, 1):
        S.admit(l)
        o.admit(l)
        torch.cuda.synchronize()
        gu.check_state(S, o, f"admit layer {l}")


def test_admit_full_size_batch512_all_layers():
    """Full admit stress: 512 sequences x 8 layers x 4 groups, scores on 64
    levels.  Selection and compaction (scores, source positions, counts)
    are checked for every group against the oracle run on the same scores
    with 2-value stand-in records; the moved K/V records are checked bit
    for bit on sampled sequences against the full-width oracle."""
    w = synth.WORKLOADS["admit_b512"]
    seed = 33
    gu.log("case admit full size: generating scores")
    B, L, G, N, C, d = w.B, w.L, w.G, w.N, w.C, w.d
    rng = np.random.default_rng(seed)
    bscore = rng.integers(0, 64, size=(L, B, G, N)).astype(np.float32)
    pscore = rng.integers(0, 64, size=(L, B, G, C)).astype(np.float32)
    bsrc = np.broadcast_to(np.arange(N, dtype=np.int32) * 7, (L, B, G, N)).copy()

    w2 = w.with_(t0=w.t0 + C)
    S = rma.State(gu.cfg_for(w2), B, gu.DEV, start_pos=w2.t0, bank_n=N)
    gu.log("case admit full size: filling records on the device")
    for l in range(L):
        for name, shape, kind in (("bank_k", (1, B, G, N, d), 3), ("bank_v", (1, B, G, N, d), 4),
                                  ("pend_k", (1, B, G, C, d), 14), ("pend_v", (1, B, G, C, d), 15)):
            x = synth.torch_normal_bf16(shape, w.qkv_std, seed, gu.DEV, (w.wid, kind, l))
            S.write(name, x.view(torch.int16), layers=slice(l, l + 1))
            del x
    S.write("bscore", bscore)
    S.write("pscore", pscore)
    S.write("bsrc", bsrc)
    for l in range(L):
        S._st.pend_n[l] = C
    sample = [0, 255, 511]
    before = {name: gu.bits(S.read(name, batch=sample)) for name in
              ("bank_k", "bank_v", "pend_k", "pend_v")}
    torch.cuda.synchronize()

    gu.log("case admit full size: admit on the GPU")
    S.admit(-1)
    torch.cuda.synchronize()

    # oracle with stand-in records of width 2
    o = OracleState(L=L, B=B, H=4 * G, G=G, d=2, R=3, N=N, C=C)
    o.bscore[...] = bscore
    o.pscore[...] = pscore
    o.bsrc[...] = bsrc
    o.bank_n[...] = N
    o.t[:] = w2.t0
    o.pend_n[:] = C
    for l in range(L):
        o.admit(l)
    gu.log("case admit full size: comparing")
    for name in ("bscore", "bsrc", "bank_n"):
        g = gu.bits(S.read(name))
        r = getattr(o, name)
        if r.dtype == np.float32:
            g, r = g.view(np.uint32), r.view(np.uint32)
        assert np.array_equal(g, r), name

    # full-width records for the sampled sequences
    os_ = OracleState(L=L, B=len(sample), H=4 * G, G=G, d=d, R=w.R, N=N, C=C)
    os_.bank_k[...] = before["bank_k"].view(np.uint16)
    os_.bank_v[...] = before["bank_v"].view(np.uint16)
    os_.pend_k[...] = before["pend_k"].view(np.uint16)
    os_.pend_v[...] = before["pend_v"].view(np.uint16)
    os_.bscore[...] = bscore[:, sample]
    os_.pscore[...] = pscore[:, sample]
    os_.bsrc[...] = bsrc[:, sample]
    os_.bank_n[...] = N
    os_.t[:] = w2.t0
    os_.pend_n[:] = C
    for l in range(L):
        os_.admit(l)
    for name in ("bank_k", "bank_v"):
        g = gu.bits(S.read(name, batch=sample))
        assert np.array_equal(g, getattr(os_, name).view(np.int16)), name
