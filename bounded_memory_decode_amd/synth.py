"""Seeded synthetic inputs for the RMA layer step.

This module only draws random numbers and names workload shapes; it holds
none of the layer's arithmetic.  Both the HIP path (tests, bench) and the
CPU oracle (tests) take their inputs from here, so the two sides see the
same bytes.

Shapes follow the EdgeRock pages: 8 RMA layers, 16 query heads in 4 KV
groups, a 1,023-slot local ring plus the current token, 1,024 anchors per
group and 256 pending candidates (EdgeRock model card, "How Rock Memory
Anchors work" history-component table; Rock Matrix models page, spec
list).  The head dimension 256 is the one the card's persistent-history
table (32.00 / 8.00 / 31.97 MiB) implies for bf16 records.

Value recipe: q, K, V and candidate records are N(0,1)/16 drawn in fp32
and rounded to bf16 (nearest, ties to even); gate weights are N(0, 1/256)
in fp32; scores are N(0,1) fp32, or uniform integers 0..63 for the admit
stress.  The "sharp" variant uses N(0,1) for q/K/V so that softmaxes are
far from uniform.

Two generators:
  * numpy: one ``SeedSequence(seed, spawn_key=(workload, kind, layer,
    step, b))`` stream per tensor (start state: per sequence, so one
    sequence can be regenerated on its own; step inputs: per token for the
    whole batch);
  * torch: one seeded ``torch.Generator`` per (kind, layer[, step]) on the
    target device, used only where numpy would be too slow (full-size bench
    state).  Its values differ from the numpy stream; parity at that size
    copies the generated tensors to the host before any kernel runs.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np

KIND = {
    "ring_k": 1, "ring_v": 2, "bank_k": 3, "bank_v": 4, "bscore": 5, "bsrc": 6,
    "q": 7, "k": 8, "v": 9, "ck": 10, "cv": 11, "cs": 12, "w_g": 13,
    "pend_k": 14, "pend_v": 15, "pscore": 16, "q_anchor": 17,
}


@dataclasses.dataclass(frozen=True)
class Workload:
    """A synthetic workload: layer geometry, batch, start state, steps."""
    name: str
    wid: int                 # numeric id used in the seed
    B: int
    L: int
    steps: int
    t0: int                  # position of the first decoded token
    bank_n: int              # committed anchors at t0
    H: int = 16
    G: int = 4
    d: int = 256
    R: int = 1023
    N: int = 1024
    C: int = 256
    qkv_std: float = 1.0 / 16.0
    w_std: float = 1.0 / 16.0
    scores: str = "normal"   # "normal" | "levels64"
    ring_full: bool = True

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads.  t0 = 32,768 is a block-aligned position after a 32K
# prompt: ring full (positions t0-1023 .. t0-1), bank full, pending empty.
WORKLOADS: Dict[str, Workload] = {
    # one layer, batch 1, 512 decode steps (2 admits)
    "layer_b1": Workload("layer_b1", 1, B=1, L=1, steps=512, t0=32768, bank_n=1024),
    # one layer, batch 64, 2,048 decode steps (8 admits)
    "layer_b64": Workload("layer_b64", 2, B=64, L=1, steps=2048, t0=32768, bank_n=1024),
    # the full 8-layer stack at batch 512, 1,024 decode steps
    "stack_b512": Workload("stack_b512", 3, B=512, L=8, steps=1024, t0=32768, bank_n=1024),
    # admit stress: batch 512 x 8 layers x 4 groups, scores on 64 levels
    "admit_b512": Workload("admit_b512", 4, B=512, L=8, steps=0, t0=32768, bank_n=1024,
                           scores="levels64"),
    # long single sequence: 131,072-token prompt in 256-token blocks, then decode
    "long_b1": Workload("long_b1", 5, B=1, L=8, steps=131072, t0=0, bank_n=0,
                        ring_full=False),
    # sharp variant of layer_b1: q/K/V ~ N(0,1)
    "sharp_b1": Workload("sharp_b1", 6, B=1, L=1, steps=512, t0=32768, bank_n=1024,
                         qkv_std=1.0),
    # one layer, batch 288 (a full round of whole units and 32 more
    # sequences), 512 decode steps (2 admits)
    "layer_b288": Workload("layer_b288", 7, B=288, L=1, steps=512, t0=32768, bank_n=1024),
}


# ---------------------------------------------------------------- helpers

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    # finite values and infinities cannot carry out of 32 bits; NaNs are
    # replaced below
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    r = r.astype(np.uint16)
    r[np.isnan(f)] = 0x7FC0
    return r


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, w: Workload, kind: str, layer: int = 0, step: int = 0,
         b: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(w.wid, KIND[kind], layer, step, b))
    return np.random.Generator(np.random.PCG64(ss))


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def _scores(rng: np.random.Generator, shape, w: Workload) -> np.ndarray:
    if w.scores == "levels64":
        return rng.integers(0, 64, size=shape).astype(np.float32)
    return rng.standard_normal(shape, dtype=np.float32)


def _batch(w: Workload, batch: Optional[Sequence[int]]):
    return list(range(w.B)) if batch is None else [int(b) for b in batch]


# ----------------------------------------------------------------- numpy side

def gate_weights(w: Workload, seed: int = 0, per_group: bool = False) -> np.ndarray:
    """w_g [L][H][d] fp32, N(0, w_std^2); [L][G][d] for a gate per KV
    group."""
    rng = _rng(seed, w, "w_g")
    rows = w.G if per_group else w.H
    return (rng.standard_normal((w.L, rows, w.d), dtype=np.float32)
            * np.float32(w.w_std))


def initial_state(w: Workload, seed: int = 0, layers: Optional[Sequence[int]] = None,
                  batch: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Start state in the natural layout, for the listed layers/sequences.

    Returns ring_k/ring_v [l][b][G][R][d], bank_k/bank_v [l][b][G][N][d]
    (bf16 bits), bscore [l][b][G][N] f32, bsrc [l][b][G][N] i32,
    bank_n [l][b][G] i32, pending buffers zeroed, and t0.  Ring slots that
    hold no position yet (t0 < R) are left zero; bank slots >= bank_n are
    zero.  bsrc of pre-filled anchors are distinct positions below
    t0 - R (ascending, synthetic)."""
    layers = list(range(w.L)) if layers is None else [int(x) for x in layers]
    bl = _batch(w, batch)
    nl, nb = len(layers), len(bl)
    G, d, R, N, C = w.G, w.d, w.R, w.N, w.C
    out = {
        "ring_k": np.zeros((nl, nb, G, R, d), np.uint16),
        "ring_v": np.zeros((nl, nb, G, R, d), np.uint16),
        "bank_k": np.zeros((nl, nb, G, N, d), np.uint16),
        "bank_v": np.zeros((nl, nb, G, N, d), np.uint16),
        "bscore": np.zeros((nl, nb, G, N), np.float32),
        "bsrc": np.zeros((nl, nb, G, N), np.int32),
        "bank_n": np.full((nl, nb, G), w.bank_n, np.int32),
        "pend_k": np.zeros((nl, nb, G, C, d), np.uint16),
        "pend_v": np.zeros((nl, nb, G, C, d), np.uint16),
        "pscore": np.zeros((nl, nb, G, C), np.float32),
    }
    filled = min(w.t0, R)
    n = w.bank_n
    for li, l in enumerate(layers):
        for bi, b in enumerate(bl):
            if filled:
                out["ring_k"][li, bi, :, :filled] = _normal_bf16(
                    _rng(seed, w, "ring_k", l, 0, b), (G, filled, d), w.qkv_std)
                out["ring_v"][li, bi, :, :filled] = _normal_bf16(
                    _rng(seed, w, "ring_v", l, 0, b), (G, filled, d), w.qkv_std)
            if n:
                out["bank_k"][li, bi, :, :n] = _normal_bf16(
                    _rng(seed, w, "bank_k", l, 0, b), (G, n, d), w.qkv_std)
                out["bank_v"][li, bi, :, :n] = _normal_bf16(
                    _rng(seed, w, "bank_v", l, 0, b), (G, n, d), w.qkv_std)
                out["bscore"][li, bi, :, :n] = _scores(
                    _rng(seed, w, "bscore", l, 0, b), (G, n), w)
                hi = max(w.t0 - R, n)
                r = _rng(seed, w, "bsrc", l, 0, b)
                for g in range(G):
                    out["bsrc"][li, bi, g, :n] = np.sort(
                        r.choice(hi, size=n, replace=False)).astype(np.int32)
    out["t0"] = np.int64(w.t0)
    return out


def pending_fill(w: Workload, seed: int = 0, layers: Optional[Sequence[int]] = None,
                 batch: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """A full pending buffer (admit-only stress): pend_k/pend_v [l][b][G][C][d]
    bf16 bits and pscore [l][b][G][C] f32."""
    layers = list(range(w.L)) if layers is None else [int(x) for x in layers]
    bl = _batch(w, batch)
    G, d, C = w.G, w.d, w.C
    pk = np.zeros((len(layers), len(bl), G, C, d), np.uint16)
    pv = np.zeros_like(pk)
    ps = np.zeros((len(layers), len(bl), G, C), np.float32)
    for li, l in enumerate(layers):
        for bi, b in enumerate(bl):
            pk[li, bi] = _normal_bf16(_rng(seed, w, "pend_k", l, 0, b), (G, C, d), w.qkv_std)
            pv[li, bi] = _normal_bf16(_rng(seed, w, "pend_v", l, 0, b), (G, C, d), w.qkv_std)
            ps[li, bi] = _scores(_rng(seed, w, "pscore", l, 0, b), (G, C), w)
    return {"pend_k": pk, "pend_v": pv, "pscore": ps}


def step_inputs(w: Workload, seed: int, layer: int, step: int,
                batch: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Inputs of one decode token of one layer: q [b][H][d], k, v, ck, cv
    [b][G][d] (bf16 bits) and cs [b][G] f32.  `step` counts tokens from
    t0, so the same (layer, step) always gives the same values.  One stream
    per (tensor, layer, step) covers the whole batch; `batch` selects rows."""
    H, G, d = w.H, w.G, w.d
    out = {"q": _normal_bf16(_rng(seed, w, "q", layer, step), (w.B, H, d), w.qkv_std)}
    for kind in ("k", "v", "ck", "cv"):
        out[kind] = _normal_bf16(_rng(seed, w, kind, layer, step), (w.B, G, d), w.qkv_std)
    out["cs"] = _scores(_rng(seed, w, "cs", layer, step), (w.B, G), w)
    if batch is not None:
        idx = [int(b) for b in batch]
        out = {k: np.ascontiguousarray(v[idx]) for k, v in out.items()}
    return out


def anchor_query(w: Workload, seed: int, layer: int, step: int,
                 batch: Optional[Sequence[int]] = None) -> np.ndarray:
    """A second query per head, [b][H][d] bf16 bits, drawn like q from its
    own stream (one per (layer, step), the whole batch)."""
    qa = _normal_bf16(_rng(seed, w, "q_anchor", layer, step), (w.B, w.H, w.d), w.qkv_std)
    if batch is not None:
        qa = np.ascontiguousarray(qa[[int(b) for b in batch]])
    return qa


def block_anchor_query(w: Workload, seed: int, layer: int, step0: int, n: int,
                       batch: Optional[Sequence[int]] = None) -> np.ndarray:
    """anchor_query for n consecutive tokens: [b][n][H][d]."""
    return np.stack([anchor_query(w, seed, layer, step0 + i, batch) for i in range(n)], axis=1)


def block_inputs(w: Workload, seed: int, layer: int, step0: int, n: int,
                 batch: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """n consecutive tokens starting at `step0`, stacked on a token axis
    after the batch axis: q [b][n][H][d], k.. [b][n][G][d], cs [b][n][G].
    Token i carries exactly step_inputs(w, seed, layer, step0 + i)."""
    per = [step_inputs(w, seed, layer, step0 + i, batch) for i in range(n)]
    return {k: np.stack([p[k] for p in per], axis=1) for k in per[0]}


# ----------------------------------------------------------------- torch side

def torch_normal_bf16(shape, std: float, seed: int, device, generator_key: Sequence[int]):
    """Device-side N(0, std^2) in fp32 rounded to bf16 (torch's round to
    nearest even), from a torch.Generator seeded by (seed, key)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, generator_key))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    return x.to(torch.bfloat16)


def torch_scores(shape, w: Workload, seed: int, device, generator_key: Sequence[int]):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, generator_key))
    if w.scores == "levels64":
        return torch.randint(0, 64, shape, generator=g, device=device).to(torch.float32)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _torch_seed(seed: int, key: Sequence[int]) -> int:
    ss = np.random.SeedSequence(seed, spawn_key=tuple(int(k) for k in key))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def torch_block_inputs(w: Workload, seed: int, layer: int, block: int, device,
                       n: Optional[int] = None, sets: int = 3):
    """Inputs of n (default C) consecutive tokens of one layer, drawn on
    `device`: q [B][n][H][d], k, v, ck, cv [B][n][G][d] bf16 and cs [B][n][G]
    f32, one torch.Generator per (layer, block, tensor).  `block` names the
    draw (the long prompt uses the index of the 256-token block, decode
    continues the count); `sets` separates this family of draws from the
    bench's other torch streams.  Used where a prompt of 131,072 tokens
    makes the per-token numpy streams too slow."""
    n = w.C if n is None else int(n)
    B, H, G, d = w.B, w.H, w.G, w.d

    def key(kind):
        return (w.wid, KIND[kind], layer, block, sets)

    out = {"q": torch_normal_bf16((B, n, H, d), w.qkv_std, seed, device, key("q"))}
    for kind in ("k", "v", "ck", "cv"):
        out[kind] = torch_normal_bf16((B, n, G, d), w.qkv_std, seed, device, key(kind))
    out["cs"] = torch_scores((B, n, G), w, seed, device, key("cs"))
    return out
