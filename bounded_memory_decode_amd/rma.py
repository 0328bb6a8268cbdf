"""Thin ctypes binding of librma.so (include/rma.h).

Argument marshalling only: tensors are checked for device, dtype, shape
and contiguity, and their device pointers are passed to the C ABI together
with torch's current HIP stream.  Every step of the layer runs in the HIP
kernels of librma.so; there is no host fallback, and loading fails loudly
when the library has not been built.

``State`` owns the device buffer of one rma_state (a torch uint8 tensor)
and offers views of its regions in the natural layout for filling and
inspecting the history (a permutation of bytes, no arithmetic).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# RMA_LIBRARY may name another build of the same library (e.g. a tuning
# variant); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("RMA_LIBRARY") or os.path.join(_HERE, "librma.so")

RMA_MAX_LAYERS = 64
RMA_OK, RMA_E_ARG, RMA_E_PENDING_FULL, RMA_E_NOT_BOUNDARY, RMA_E_HIP, RMA_E_UNSUPPORTED = \
    0, -1, -2, -3, -4, -5
RMA_E_SCRATCH = -6
RMA_GATE_HEAD, RMA_GATE_GROUP = 0, 1
RMA_STATIC_SCRATCH_BYTES = 80 << 20
RMA_MAX_POS = 2 ** 31 - 1

# every symbol include/rma.h and include/rma_calib.h declare
EXPORTS = ("rma_config_default", "rma_state_bytes", "rma_state_layout", "rma_state_init",
           "rma_decode_step", "rma_prefill_block", "rma_admit", "rma_decode_step_at",
           "rma_prefill_block_at", "rma_seq_reset", "rma_strerror",
           "rma_decode_step_at_static", "rma_calib_stream_read")


class Config(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("q_heads", ctypes.c_int32),
                ("kv_groups", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("bank_cap", ctypes.c_int32),
                ("commit", ctypes.c_int32), ("scale", ctypes.c_float),
                ("gate", ctypes.c_int32)]

    def __repr__(self):
        return "Config(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "ring_k", "ring_v", "bank_k", "bank_v", "pend_k", "pend_v", "bscore", "bsrc",
        "pscore", "bank_n", "scratch", "scratch_bytes", "total_bytes", "ring_bytes",
        "bank_bytes", "pend_bytes", "meta_bytes", "ring_k_slots")]


class _State(ctypes.Structure):
    _fields_ = [("cfg", Config), ("batch", ctypes.c_int32), ("hip_error", ctypes.c_int32),
                ("base", ctypes.c_void_p), ("bytes", ctypes.c_uint64), ("layout", Layout),
                ("t", ctypes.c_int64 * RMA_MAX_LAYERS),
                ("bank_n", ctypes.c_int32 * RMA_MAX_LAYERS),
                ("pend_n", ctypes.c_int32 * RMA_MAX_LAYERS)]


_P = ctypes.c_void_p
_lib = None


def lib() -> ctypes.CDLL:
    """Load librma.so (built by __graft_entry__.build() or
    ``python -m bounded_memory_decode_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bounded_memory_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.rma_config_default.argtypes = [ctypes.POINTER(Config)]
        L.rma_config_default.restype = ctypes.c_int
        L.rma_state_bytes.argtypes = [ctypes.POINTER(Config), ctypes.c_int32]
        L.rma_state_bytes.restype = ctypes.c_size_t
        L.rma_state_layout.argtypes = [ctypes.POINTER(Config), ctypes.c_int32, ctypes.POINTER(Layout)]
        L.rma_state_layout.restype = ctypes.c_int
        L.rma_state_init.argtypes = [ctypes.POINTER(_State), ctypes.POINTER(Config), ctypes.c_int32,
                                     _P, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int32, _P]
        L.rma_state_init.restype = ctypes.c_int
        L.rma_decode_step.argtypes = [ctypes.POINTER(_State), ctypes.c_int32] + [_P] * 9
        L.rma_decode_step.restype = ctypes.c_int
        L.rma_prefill_block.argtypes = [ctypes.POINTER(_State), ctypes.c_int32, ctypes.c_int32] + [_P] * 9
        L.rma_prefill_block.restype = ctypes.c_int
        L.rma_admit.argtypes = [ctypes.POINTER(_State), ctypes.c_int32, _P]
        L.rma_admit.restype = ctypes.c_int
        L.rma_decode_step_at.argtypes = [ctypes.POINTER(_State), ctypes.c_int32] + [_P] * 11
        L.rma_decode_step_at.restype = ctypes.c_int
        L.rma_decode_step_at_static.argtypes = [ctypes.POINTER(_State), ctypes.c_int32] + [_P] * 11
        L.rma_decode_step_at_static.restype = ctypes.c_int
        L.rma_prefill_block_at.argtypes = [ctypes.POINTER(_State), ctypes.c_int32,
                                           ctypes.c_int32] + [_P] * 11
        L.rma_prefill_block_at.restype = ctypes.c_int
        L.rma_seq_reset.argtypes = [ctypes.POINTER(_State), ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, _P]
        L.rma_seq_reset.restype = ctypes.c_int
        L.rma_calib_stream_read.argtypes = [_P, ctypes.c_size_t, ctypes.c_int32, _P, _P]
        L.rma_calib_stream_read.restype = ctypes.c_int
        L.rma_strerror.argtypes = [ctypes.c_int]
        L.rma_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


class RmaError(RuntimeError):
    def __init__(self, code: int, what: str):
        msg = lib().rma_strerror(code).decode()
        super().__init__(f"{what}: {msg} (status {code})")
        self.code = code


def _check(rc: int, what: str):
    if rc != RMA_OK:
        raise RmaError(rc, what)


def config_default(**override) -> Config:
    c = Config()
    _check(lib().rma_config_default(ctypes.byref(c)), "rma_config_default")
    for k, v in override.items():
        setattr(c, k, v)
    return c


def state_bytes(cfg: Config, batch: int) -> int:
    return int(lib().rma_state_bytes(ctypes.byref(cfg), batch))


def state_layout(cfg: Config, batch: int) -> Layout:
    out = Layout()
    _check(lib().rma_state_layout(ctypes.byref(cfg), batch, ctypes.byref(out)), "rma_state_layout")
    return out


def calib_stream_read(buf: torch.Tensor, waves: int, sink: torch.Tensor):
    """Enqueue one streaming read of the whole device buffer `buf` (a
    contiguous tensor whose byte size is a multiple of waves * 16 KiB) with
    `waves` waves; each wave's xor of its words goes to sink[w] (a device
    int32 tensor of `waves` entries).  Measurement support, not part of the
    layer step."""
    if not buf.is_contiguous() or sink.dtype != torch.int32 or sink.numel() < waves or \
            sink.device != buf.device:
        raise ValueError("calib_stream_read: contiguous buffer and an int32 sink of `waves` "
                         "entries on the same device expected")
    nbytes = buf.numel() * buf.element_size()
    rc = lib().rma_calib_stream_read(buf.data_ptr(), nbytes, int(waves), sink.data_ptr(),
                                     _stream_handle(buf.device))
    if rc != 0:
        raise RuntimeError(f"rma_calib_stream_read: status {rc}")


def _stream_handle(device) -> Optional[int]:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, dtype, shape, name: str, device) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, state is on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


class State:
    """One RMA state (all layers, `batch` sequences) in one device buffer."""

    def __init__(self, cfg: Config, batch: int, device="cuda", start_pos: int = 0,
                 bank_n: int = 0):
        self.cfg = cfg
        self.batch = int(batch)
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        nbytes = state_bytes(cfg, batch)
        if nbytes == 0:
            raise RmaError(RMA_E_ARG, "rma_state_bytes")
        self.layout = state_layout(cfg, batch)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self._st = _State()
        _check(lib().rma_state_init(ctypes.byref(self._st), ctypes.byref(cfg), self.batch,
                                    self.buf.data_ptr(), nbytes, int(start_pos), int(bank_n),
                                    _stream_handle(self.device)), "rma_state_init")

    # ------------------------------------------------------------ counters
    @property
    def t(self):
        return [int(self._st.t[i]) for i in range(self.cfg.layers)]

    @property
    def bank_n(self):
        return [int(self._st.bank_n[i]) for i in range(self.cfg.layers)]

    @property
    def pend_n(self):
        return [int(self._st.pend_n[i]) for i in range(self.cfg.layers)]

    def snapshot(self):
        """(copy of the device buffer, copy of the host counters)."""
        return self.buf.clone(), bytes(self._st)

    def restore(self, snap):
        buf, raw = snap
        self.buf.copy_(buf)
        ctypes.memmove(ctypes.byref(self._st), raw, ctypes.sizeof(self._st))
        self._st.base = self.buf.data_ptr()

    # -------------------------------------------------------------- regions
    def _region(self, name: str, dtype, count: int) -> torch.Tensor:
        off = getattr(self.layout, name)
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return self.buf[off:off + nbytes].view(dtype)

    def region_view(self, name: str) -> torch.Tensor:
        """A view of one region in its stored layout (int16 for bf16 bits):
        ring_k/bank_k [L][B][G][slots*d] (16-byte chunks, chunk-major, see
        include/rma.h; a ring K plane has layout.ring_k_slots slots, the
        ring's R rounded up to a multiple of 64), ring_v/bank_v
        [L][B][G][slots][d],
        pend_k/pend_v [L][B][G][C][d], bscore/bsrc [L][B][G][N],
        pscore [L][B][G][C], bank_n [L][B][G]."""
        c = self.cfg
        L, B, G, d = c.layers, self.batch, c.kv_groups, c.head_dim
        R, N, C = c.window - 1, c.bank_cap, c.commit
        shapes = {
            "ring_k": ((L, B, G, int(self.layout.ring_k_slots) * d), torch.int16),
            "ring_v": ((L, B, G, R, d), torch.int16),
            "bank_k": ((L, B, G, N * d), torch.int16),
            "bank_v": ((L, B, G, N, d), torch.int16),
            "pend_k": ((L, B, G, C, d), torch.int16),
            "pend_v": ((L, B, G, C, d), torch.int16),
            "bscore": ((L, B, G, N), torch.float32),
            "bsrc": ((L, B, G, N), torch.int32),
            "pscore": ((L, B, G, C), torch.float32),
            "bank_n": ((L, B, G), torch.int32),
        }
        shape, dt = shapes[name]
        n = 1
        for s in shape:
            n *= s
        return self._region(name, dt, n).view(shape)

    def write(self, name: str, value: torch.Tensor, layers=slice(None), batch=slice(None)):
        """Copy `value` (natural layout, bf16 bits as int16/uint16/bf16) into
        region `name` for the given layer/sequence slices."""
        v = self.region_view(name)
        if name in ("ring_k", "bank_k"):
            dst = v[layers, batch]
            src = _as_bits(value).to(self.device).reshape(*dst.shape[:3], -1, self.cfg.head_dim)
            slots = dst.shape[-1] // self.cfg.head_dim
            if src.shape[-2] < slots:  # ring K plane padding slots
                pad = torch.zeros((*src.shape[:-2], slots - src.shape[-2], src.shape[-1]),
                                  dtype=src.dtype, device=src.device)
                src = torch.cat([src, pad], dim=-2)
            dst.copy_(_k_to_stored(src))
        else:
            dst = v[layers, batch]
            if dst.dtype == torch.int16:
                src = _as_bits(value)
            else:
                src = _as_tensor(value)
            dst.copy_(src.to(self.device).reshape(dst.shape).to(dst.dtype))

    def read(self, name: str, layers=slice(None), batch=slice(None)) -> torch.Tensor:
        """Copy of region `name` in the natural layout (bf16 bits as int16)."""
        v = self.region_view(name)
        if name == "ring_k":  # without the plane's padding slots
            nat = _k_to_natural(v[layers, batch], self.cfg.head_dim)
            return nat[..., :self.cfg.window - 1, :].contiguous()
        if name == "bank_k":
            return _k_to_natural(v[layers, batch], self.cfg.head_dim)
        return v[layers, batch].clone()

    # ------------------------------------------------------------- compute
    def _wg_rows(self) -> int:
        """Rows of the gate weights: one per query head, or one per KV group
        with cfg.gate == RMA_GATE_GROUP."""
        return self.cfg.kv_groups if self.cfg.gate == RMA_GATE_GROUP else self.cfg.q_heads

    def _decode_ptrs(self, q, k, v, cand_k, cand_v, cand_score, w_g, out):
        c, B = self.cfg, self.batch
        H, G, d = c.q_heads, c.kv_groups, c.head_dim
        if out is None:
            out = torch.empty((B, H, d), dtype=torch.bfloat16, device=self.device)
        bf, f32, dev = torch.bfloat16, torch.float32, self.device
        ptrs = [_dev(q, bf, (B, H, d), "q", dev), _dev(k, bf, (B, G, d), "k", dev),
                _dev(v, bf, (B, G, d), "v", dev), _dev(cand_k, bf, (B, G, d), "cand_k", dev),
                _dev(cand_v, bf, (B, G, d), "cand_v", dev),
                _dev(cand_score, f32, (B, G), "cand_score", dev),
                _dev(w_g, f32, (self._wg_rows(), d), "w_g", dev),
                _dev(out, bf, (B, H, d), "out", dev)]
        return out, ptrs

    def _prefill_ptrs(self, q, k, v, cand_k, cand_v, cand_score, w_g, out):
        c, B = self.cfg, self.batch
        H, G, d = c.q_heads, c.kv_groups, c.head_dim
        n = q.shape[1]
        if out is None:
            out = torch.empty((B, n, H, d), dtype=torch.bfloat16, device=self.device)
        bf, f32, dev = torch.bfloat16, torch.float32, self.device
        ptrs = [_dev(q, bf, (B, n, H, d), "q", dev), _dev(k, bf, (B, n, G, d), "k", dev),
                _dev(v, bf, (B, n, G, d), "v", dev), _dev(cand_k, bf, (B, n, G, d), "cand_k", dev),
                _dev(cand_v, bf, (B, n, G, d), "cand_v", dev),
                _dev(cand_score, f32, (B, n, G), "cand_score", dev),
                _dev(w_g, f32, (self._wg_rows(), d), "w_g", dev),
                _dev(out, bf, (B, n, H, d), "out", dev)]
        return n, out, ptrs

    def decode_step(self, layer: int, q, k, v, cand_k, cand_v, cand_score, w_g,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
        out, ptrs = self._decode_ptrs(q, k, v, cand_k, cand_v, cand_score, w_g, out)
        _check(lib().rma_decode_step(ctypes.byref(self._st), int(layer), *ptrs,
                                     _stream_handle(self.device)), "rma_decode_step")
        return out

    def prefill_block(self, layer: int, q, k, v, cand_k, cand_v, cand_score, w_g,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
        n, out, ptrs = self._prefill_ptrs(q, k, v, cand_k, cand_v, cand_score, w_g, out)
        _check(lib().rma_prefill_block(ctypes.byref(self._st), int(layer), int(n), *ptrs,
                                       _stream_handle(self.device)), "rma_prefill_block")
        return out

    def decode_step_at(self, layer: int, pos: torch.Tensor, q, k, v, cand_k, cand_v, cand_score,
                       w_g, out: Optional[torch.Tensor] = None,
                       q_anchor: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Decode with per-sequence positions: `pos` is a device int32
        tensor [batch] (negative: sequence left out, its `out` rows are not
        written).  Admits the blocks the step completes.  `q_anchor` (shape
        of q), if given, is the query of the anchor read and the gate.  The
        host counters (t, pend_n, bank_n) are not used or updated."""
        out, ptrs = self._decode_ptrs(q, k, v, cand_k, cand_v, cand_score, w_g, out)
        p = _dev(pos, torch.int32, (self.batch,), "pos", self.device)
        qa = None if q_anchor is None else _dev(q_anchor, torch.bfloat16, tuple(q.shape),
                                                "q_anchor", self.device)
        _check(lib().rma_decode_step_at(ctypes.byref(self._st), int(layer), p, ptrs[0], qa,
                                        *ptrs[1:], _stream_handle(self.device)),
               "rma_decode_step_at")
        return out

    def decode_step_at_static(self, layer: int, pos: torch.Tensor, q, k, v, cand_k, cand_v,
                              cand_score, w_g, out: torch.Tensor,
                              q_anchor: Optional[torch.Tensor] = None) -> torch.Tensor:
        """decode_step_at through the allocation-free entry point: the
        split-K partials go to the library's static device array, not to the
        state's scratch region.  `out` must be given (nothing is allocated
        here either).  Calls that overlap on one GPU race on that array."""
        if out is None:
            raise ValueError("decode_step_at_static: pass `out` (the call allocates nothing)")
        out, ptrs = self._decode_ptrs(q, k, v, cand_k, cand_v, cand_score, w_g, out)
        p = _dev(pos, torch.int32, (self.batch,), "pos", self.device)
        qa = None if q_anchor is None else _dev(q_anchor, torch.bfloat16, tuple(q.shape),
                                                "q_anchor", self.device)
        _check(lib().rma_decode_step_at_static(ctypes.byref(self._st), int(layer), p, ptrs[0], qa,
                                               *ptrs[1:], _stream_handle(self.device)),
               "rma_decode_step_at_static")
        return out

    def prefill_block_at(self, layer: int, pos: torch.Tensor, q, k, v, cand_k, cand_v,
                         cand_score, w_g, out: Optional[torch.Tensor] = None,
                         q_anchor: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Prefill block with per-sequence block starts in `pos` (device
        int32 [batch]; sequences whose entry is negative or not a multiple of
        the commit interval are left out).  A full block is admitted.
        `q_anchor` as in decode_step_at, with the token axis."""
        n, out, ptrs = self._prefill_ptrs(q, k, v, cand_k, cand_v, cand_score, w_g, out)
        p = _dev(pos, torch.int32, (self.batch,), "pos", self.device)
        qa = None if q_anchor is None else _dev(q_anchor, torch.bfloat16, tuple(q.shape),
                                                "q_anchor", self.device)
        _check(lib().rma_prefill_block_at(ctypes.byref(self._st), int(layer), int(n), p,
                                          ptrs[0], qa, *ptrs[1:], _stream_handle(self.device)),
               "rma_prefill_block_at")
        return out

    def seq_reset(self, first: int, count: int = 1, bank_n: int = 0):
        """Set the bank count of sequences first .. first+count-1 (all
        layers and groups), e.g. for a new sequence in a reused slot."""
        _check(lib().rma_seq_reset(ctypes.byref(self._st), int(first), int(count), int(bank_n),
                                   _stream_handle(self.device)), "rma_seq_reset")

    def admit(self, layer: int = -1):
        _check(lib().rma_admit(ctypes.byref(self._st), int(layer), _stream_handle(self.device)),
               "rma_admit")

    @property
    def hip_error(self) -> int:
        return int(self._st.hip_error)


def _as_bits(x) -> torch.Tensor:
    """bf16 bit patterns as an int16 tensor (numpy uint16, torch bf16/int16)."""
    import numpy as np
    if isinstance(x, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16)
    if x.dtype == torch.int16:
        return x
    raise TypeError(f"expected bf16 bits, got {x.dtype}")


def _k_to_stored(nat: torch.Tensor) -> torch.Tensor:
    """[..., S, d] K rows -> [..., S*d] in the stored K order: 16-byte
    chunks of 8 dims, chunk-major over the plane."""
    *lead, S, d = nat.shape
    return nat.reshape(*lead, S, d // 8, 8).transpose(-3, -2).reshape(*lead, S * d)


def _k_to_natural(stored: torch.Tensor, d: int) -> torch.Tensor:
    """Inverse of _k_to_stored: [..., S*d] -> [..., S, d] (a copy)."""
    *lead, n = stored.shape
    S = n // d
    return stored.reshape(*lead, d // 8, S, 8).transpose(-3, -2).reshape(*lead, S, d)


def _as_tensor(x) -> torch.Tensor:
    import numpy as np
    if isinstance(x, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(x))
    return x


def bf16_from_bits(x) -> torch.Tensor:
    """numpy uint16 bit patterns -> torch bfloat16 tensor (host)."""
    return _as_bits(x).view(torch.bfloat16)
