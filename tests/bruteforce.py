"""Full-history brute force of the RMA layer step (tiny shapes only).

An independent formulation used to pin the oracle: it keeps every token's
K/V by absolute position (no ring buffer) and the anchor bank as a list of
records (no slot bookkeeping), and recomputes each output from those
lists with a plain float64 softmax.  Selection uses numpy's stable argsort
of the scores; with continuous scores no tie sits on the cut, which the
model asserts.

Semantics (EdgeRock model card, "How Rock Memory Anchors work" and the
persistent-history table; ai-primer "three operations" list):
  local window = the 1,023 preceding positions plus the current token;
  anchor read = softmax attention over the committed records of the
  query's KV group; out = local + tanh(q . w_g) * anchor;
  every C tokens the pending candidates and the anchors compete for N
  records per group; the best scores stay.
"""
from __future__ import annotations

import numpy as np


def _f(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _softmax_read(q, K, V, scale):
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w / w.sum()) @ V


class BruteForce:
    def __init__(self, H, G, d, R, N, C, scale, t0, ring_k, ring_v, bank_k, bank_v,
                 bscore, bsrc, bank_n, gate_group=False):
        """ring_*/bank_* [G][slots][d] bf16 bits for ONE sequence of ONE layer.
        Ring slot s holds the position p in [t0-R, t0) with p % R == s.
        gate_group: one gate per KV group, tanh of the mean anchor query of
        the group against w_g[g] (w_g [G][d]), instead of one per head."""
        self.H, self.G, self.d, self.R, self.N, self.C = H, G, d, R, N, C
        self.gate_group = gate_group
        self.scale = scale
        self.t = int(t0)
        self.hist_k = [dict() for _ in range(G)]
        self.hist_v = [dict() for _ in range(G)]
        for g in range(G):
            for p in range(max(0, t0 - R), t0):
                self.hist_k[g][p] = _f(ring_k[g, p % R])
                self.hist_v[g][p] = _f(ring_v[g, p % R])
        # bank: list of records per group (order irrelevant)
        self.bank = [[{"score": float(bscore[g, i]), "pos": int(bsrc[g, i]),
                       "k": _f(bank_k[g, i]), "v": _f(bank_v[g, i])}
                      for i in range(int(bank_n[g]))] for g in range(G)]
        self.pending = [[] for _ in range(G)]

    def step(self, q, k, v, ck, cv, cs, w_g, q_anchor=None):
        """q [H][d], k/v/ck/cv [G][d] bf16 bits, cs [G], w_g [H][d] f32;
        q_anchor [H][d] (optional): the query of the anchor read and of the
        gate, else q.  Returns out [H][d] float64."""
        H, G, d = self.H, self.G, self.d
        hpg = H // G
        t = self.t
        out = np.zeros((H, d))
        for g in range(G):
            kc, vc = _f(k[g]), _f(v[g])
            self.hist_k[g][t] = kc
            self.hist_v[g][t] = vc
            lo = max(0, t - self.R)
            Kl = np.stack([self.hist_k[g][p] for p in range(lo, t + 1)])
            Vl = np.stack([self.hist_v[g][p] for p in range(lo, t + 1)])
            qsrc = q if q_anchor is None else q_anchor
            qbar = np.mean([_f(qsrc[g * hpg + i]) for i in range(hpg)], axis=0)
            for hh in range(hpg):
                h = g * hpg + hh
                qh = _f(q[h])
                qa = qh if q_anchor is None else _f(q_anchor[h])
                ol = _softmax_read(qh, Kl, Vl, self.scale)
                if self.bank[g]:
                    Kb = np.stack([r["k"] for r in self.bank[g]])
                    Vb = np.stack([r["v"] for r in self.bank[g]])
                    oa = _softmax_read(qa, Kb, Vb, self.scale)
                else:
                    oa = np.zeros(d)
                if self.gate_group:
                    z = qbar @ np.asarray(w_g[g], np.float64)
                else:
                    z = qa @ np.asarray(w_g[h], np.float64)
                out[h] = ol + np.tanh(z) * oa
            self.pending[g].append({"score": float(cs[g]), "pos": t,
                                    "k": _f(ck[g]), "v": _f(cv[g])})
            # positions older than the window are never read again
            self.hist_k[g].pop(t - self.R - 1, None)
            self.hist_v[g].pop(t - self.R - 1, None)
        self.t += 1
        if self.t % self.C == 0:
            self._admit()
        return out

    def _admit(self):
        for g in range(self.G):
            pool = self.bank[g] + self.pending[g]
            sc = np.array([r["score"] for r in pool])
            order = np.argsort(-sc, kind="stable")
            K = min(self.N, len(pool))
            if K < len(pool):
                assert sc[order[K - 1]] != sc[order[K]], "tie on the cut"
            self.bank[g] = [pool[i] for i in order[:K]]
            self.pending[g] = []

    def bank_positions(self, g):
        return sorted(r["pos"] for r in self.bank[g])
