"""CPU oracle of the RMA layer step: TEST INFRASTRUCTURE ONLY.

A ctypes wrapper around ``rma_oracle.c`` (plain C, double arithmetic).
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the product path never does.

``OracleState`` keeps the whole state in numpy arrays in the natural
layout documented in ``rma_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rma_oracle.c")
_LIB = os.path.join(_HERE, "librma_oracle.so")
# RMA_ORACLE_LIBRARY may name another build of this source, used as is: the
# mutation test (tests/test_oracle_mutations.py) points it at copies with a
# planted mistake to show that the pins fail on them.
_OVERRIDE = os.environ.get("RMA_ORACLE_LIBRARY")

ORC_OK, ORC_E_ARG, ORC_E_PENDING_FULL, ORC_E_NOT_BOUNDARY = 0, -1, -2, -3


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, IEEE double: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-Wall", "-Wextra",
                               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("H", ctypes.c_int32), ("G", ctypes.c_int32),
                ("d", ctypes.c_int32), ("R", ctypes.c_int32), ("N", ctypes.c_int32),
                ("C", ctypes.c_int32), ("scale", ctypes.c_double),
                ("gate_group", ctypes.c_int32)]


_P = ctypes.c_void_p


class _State(ctypes.Structure):
    _fields_ = [("cfg", _Cfg), ("B", ctypes.c_int32),
                ("ring_k", _P), ("ring_v", _P), ("bank_k", _P), ("bank_v", _P),
                ("bscore", _P), ("bsrc", _P), ("bank_n", _P),
                ("pend_k", _P), ("pend_v", _P), ("pscore", _P), ("t", _P), ("pend_n", _P)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _OVERRIDE:
            L = ctypes.CDLL(_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = ctypes.CDLL(_LIB)
        L.orc_decode_step.argtypes = [ctypes.POINTER(_State), ctypes.c_int32] + [_P] * 8 + [_P, ctypes.c_int32]
        L.orc_decode_step.restype = ctypes.c_int
        L.orc_admit.argtypes = [ctypes.POINTER(_State), ctypes.c_int32, _P]
        L.orc_admit.restype = ctypes.c_int
        L.orc_prefill_block.argtypes = [ctypes.POINTER(_State), ctypes.c_int32, ctypes.c_int32] + [_P] * 8 + [_P]
        L.orc_prefill_block.restype = ctypes.c_int
        L.orc_round_bf16.argtypes = [ctypes.c_double]
        L.orc_round_bf16.restype = ctypes.c_uint16
        L.orc_round_bf16_array.argtypes = [_P, _P, ctypes.c_int64]
        L.orc_round_bf16_array.restype = None
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_set_num_threads.argtypes = [ctypes.c_int]
        L.orc_set_num_threads.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Exact round-to-nearest-even of doubles to bf16 bit patterns."""
    x = _c(x, np.float64)
    y = np.empty(x.shape, np.uint16)
    lib().orc_round_bf16_array(_ptr(x), _ptr(y), x.size)
    return y


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (results do not
    depend on it)."""
    lib().orc_set_num_threads(int(n))


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle status {code}")
        self.code = code


class OracleState:
    """The RMA state of L layers x B sequences on the host (natural layout)."""

    def __init__(self, L: int, B: int, H: int = 16, G: int = 4, d: int = 256,
                 R: int = 1023, N: int = 1024, C: int = 256,
                 scale: Optional[float] = None, gate_group: bool = False):
        """gate_group: one gate per (token, KV group) from the mean of the
        group's anchor queries and gate weights [G][d] per layer, instead
        of one gate per (token, head) with weights [H][d]."""
        self.L, self.B, self.H, self.G, self.d = L, B, H, G, d
        self.R, self.N, self.C = R, N, C
        self.scale = float(d) ** -0.5 if scale is None else float(scale)
        self.gate_group = bool(gate_group)
        self.ring_k = np.zeros((L, B, G, R, d), np.uint16)
        self.ring_v = np.zeros((L, B, G, R, d), np.uint16)
        self.bank_k = np.zeros((L, B, G, N, d), np.uint16)
        self.bank_v = np.zeros((L, B, G, N, d), np.uint16)
        self.bscore = np.zeros((L, B, G, N), np.float32)
        self.bsrc = np.zeros((L, B, G, N), np.int32)
        self.bank_n = np.zeros((L, B, G), np.int32)
        self.pend_k = np.zeros((L, B, G, C, d), np.uint16)
        self.pend_v = np.zeros((L, B, G, C, d), np.uint16)
        self.pscore = np.zeros((L, B, G, C), np.float32)
        self.t = np.zeros((L,), np.int64)
        self.pend_n = np.zeros((L,), np.int32)

    ARRAYS = ("ring_k", "ring_v", "bank_k", "bank_v", "bscore", "bsrc", "bank_n",
              "pend_k", "pend_v", "pscore", "t", "pend_n")

    @classmethod
    def from_synth(cls, st: Dict[str, np.ndarray], H=16, G=4, d=256, R=1023, N=1024,
                   C=256, scale=None, gate_group=False) -> "OracleState":
        """Build from synth.initial_state() output (t0 must be block aligned,
        or the caller sets pend_n/pending contents itself)."""
        L, B = st["ring_k"].shape[:2]
        o = cls(L, B, H, G, d, R, N, C, scale, gate_group)
        for k in ("ring_k", "ring_v", "bank_k", "bank_v", "bscore", "bsrc", "bank_n",
                  "pend_k", "pend_v", "pscore"):
            getattr(o, k)[...] = st[k]
        o.t[:] = int(st["t0"])
        o.pend_n[:] = int(st["t0"]) % C
        return o

    def clone(self) -> "OracleState":
        o = OracleState(self.L, self.B, self.H, self.G, self.d, self.R, self.N, self.C,
                        self.scale, self.gate_group)
        for k in self.ARRAYS:
            getattr(o, k)[...] = getattr(self, k)
        return o

    def _struct(self) -> _State:
        s = _State()
        s.cfg = _Cfg(self.L, self.H, self.G, self.d, self.R, self.N, self.C, self.scale,
                     int(self.gate_group))
        s.B = self.B
        for k in self.ARRAYS:
            setattr(s, k, _ptr(getattr(self, k)))
        return s

    def _wg_rows(self) -> int:
        return self.G if self.gate_group else self.H

    def decode_step(self, layer: int, q, k, v, ck, cv, cs, w_g,
                    compute_out: bool = True, q_anchor=None) -> Optional[np.ndarray]:
        """One token for all B sequences of `layer`; returns out [B][H][d]
        float64 (unrounded) or None when compute_out is False.  q_anchor
        [B][H][d] (bf16 bits), if given, is the query of the anchor read and
        the gate; else q serves both reads."""
        B, H, G, d = self.B, self.H, self.G, self.d
        qa = None if q_anchor is None else _c(q_anchor, np.uint16).reshape(B, H, d)
        arrs = [_c(x, np.uint16).reshape(B, G, d) for x in (k, v, ck, cv)] + \
               [_c(cs, np.float32).reshape(B, G), _c(w_g, np.float32).reshape(self._wg_rows(), d)]
        q = _c(q, np.uint16).reshape(B, H, d)
        out = np.empty((B, H, d), np.float64) if compute_out else None
        st = self._struct()
        rc = lib().orc_decode_step(ctypes.byref(st), layer, _ptr(q),
                                   _ptr(qa) if qa is not None else None,
                                   *[_ptr(a) for a in arrs],
                                   _ptr(out) if out is not None else None, int(compute_out))
        if rc != ORC_OK:
            raise OracleError(rc, "decode_step")
        return out

    def admit(self, layer: int) -> np.ndarray:
        """Admit of `layer`; returns moved-record counts [B][G]."""
        moved = np.zeros((self.B, self.G), np.int32)
        st = self._struct()
        rc = lib().orc_admit(ctypes.byref(st), layer, _ptr(moved))
        if rc != ORC_OK:
            raise OracleError(rc, "admit")
        return moved

    def prefill_block(self, layer: int, q, k, v, ck, cv, cs, w_g,
                      compute_out: bool = True, q_anchor=None) -> Optional[np.ndarray]:
        B, H, G, d = self.B, self.H, self.G, self.d
        q = _c(q, np.uint16)
        n = q.shape[1]
        q = q.reshape(B, n, H, d)
        qa = None if q_anchor is None else _c(q_anchor, np.uint16).reshape(B, n, H, d)
        arrs = [_c(x, np.uint16).reshape(B, n, G, d) for x in (k, v, ck, cv)] + \
               [_c(cs, np.float32).reshape(B, n, G), _c(w_g, np.float32).reshape(self._wg_rows(), d)]
        out = np.empty((B, n, H, d), np.float64) if compute_out else None
        st = self._struct()
        rc = lib().orc_prefill_block(ctypes.byref(st), layer, n, _ptr(q),
                                     _ptr(qa) if qa is not None else None,
                                     *[_ptr(a) for a in arrs],
                                     _ptr(out) if out is not None else None)
        if rc != ORC_OK:
            raise OracleError(rc, "prefill_block")
        return out
