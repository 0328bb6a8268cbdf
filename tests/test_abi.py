"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/*.h declares, reproduces the pages' memory accounting, and
rejects bad arguments on the host before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

from bounded_memory_decode_amd import rma

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            src = open(os.path.join(INCLUDE, h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(rma_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(rma.EXPORTS)
    L = rma.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", rma.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (rma_\w+)", out))
    assert set(names) <= exported


def test_default_config_is_edgerock_geometry():
    c = rma.config_default()
    assert (c.layers, c.q_heads, c.kv_groups, c.head_dim) == (8, 16, 4, 256)
    assert (c.window, c.bank_cap, c.commit) == (1024, 1024, 256)
    assert c.scale == 1.0 / 16


def _golden():
    vals = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "memory_table.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()
            vals[k] = float(v)
    return vals


def test_layout_matches_the_pages_memory_table():
    """Per-sequence region sizes equal the persistent-history table of the
    model card (32.00 / 8.00 / 31.97 MiB, 72 MiB of attention KV)."""
    g = _golden()
    c = rma.config_default()
    L = rma.state_layout(c, 1)
    mib = 2.0 ** 20
    assert L.bank_bytes == 33_554_432 and round(L.bank_bytes / mib, 2) == g["committed_anchors_mib"]
    assert L.pend_bytes == 8_388_608 and round(L.pend_bytes / mib, 2) == g["pending_candidates_mib"]
    assert L.ring_bytes == 33_521_664 and round(L.ring_bytes / mib, 2) == g["local_window_kv_mib"]
    assert round((L.ring_bytes + L.bank_bytes + L.pend_bytes) / mib) == g["attention_kv_mib"]
    # metadata: the page prints 0.29 MiB without a layout; ours is scores,
    # source positions and counts
    assert 0.25 < L.meta_bytes / mib < 0.30
    # linear in the batch apart from alignment and scratch
    L512 = rma.state_layout(c, 512)
    assert L512.ring_bytes == 512 * L.ring_bytes and L512.bank_bytes == 512 * L.bank_bytes
    assert rma.state_bytes(c, 512) == L512.total_bytes
    for name in ("ring_k", "ring_v", "bank_k", "bank_v", "pend_k", "pend_v", "bscore", "bsrc",
                 "pscore", "bank_n", "scratch"):
        assert getattr(L512, name) % 256 == 0
    # ring K planes are padded to 1,024 slots (1 KiB-aligned chunk planes);
    # the padding is alignment, not records
    assert L.ring_k_slots == 1024
    assert L512.ring_v - L512.ring_k >= 512 * 4 * 8 * 1024 * 512
    # regions do not overlap and are in order
    offs = [L512.ring_k, L512.ring_v, L512.bank_k, L512.bank_v, L512.pend_k, L512.pend_v,
            L512.bscore, L512.bsrc, L512.pscore, L512.bank_n, L512.scratch]
    assert offs == sorted(offs)
    assert L512.scratch + L512.scratch_bytes <= L512.total_bytes


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 128, rma.RMA_E_UNSUPPORTED),
    ("q_heads", 8, rma.RMA_E_UNSUPPORTED),
    ("q_heads", 6, rma.RMA_E_ARG),
    ("layers", 0, rma.RMA_E_ARG),
    ("layers", 65, rma.RMA_E_ARG),
    ("window", 1, rma.RMA_E_ARG),
    ("commit", 512, rma.RMA_E_UNSUPPORTED),
    ("window", 4098, rma.RMA_E_UNSUPPORTED),
    ("window", 256, rma.RMA_E_UNSUPPORTED),   # commit 256 > ring 255
    ("bank_cap", 1900, rma.RMA_E_UNSUPPORTED),
    ("scale", float("nan"), rma.RMA_E_ARG),
    ("gate", 2, rma.RMA_E_ARG),
])
def test_invalid_configs_are_rejected(field, value, code):
    c = rma.config_default(**{field: value})
    assert rma.state_bytes(c, 4) == 0
    with pytest.raises(rma.RmaError) as e:
        rma.state_layout(c, 4)
    assert e.value.code == code


def test_zero_batch_is_rejected():
    c = rma.config_default()
    assert rma.state_bytes(c, 0) == 0
    with pytest.raises(rma.RmaError):
        rma.state_layout(c, 0)


def _fake_state(pend_n=0, t=32768):
    """A host-only rma_state bound to a fake device address; only calls
    that fail validation may be made with it."""
    c = rma.config_default()
    st = rma._State()
    st.cfg = c
    st.batch = 2
    st.base = 0x10000000
    st.layout = rma.state_layout(c, 2)
    st.bytes = st.layout.total_bytes
    for i in range(c.layers):
        st.t[i] = t
        st.pend_n[i] = pend_n
        st.bank_n[i] = 1024
    return st


FAKE = 0x20000000  # 16-byte aligned, never dereferenced


def _decode(st, layer=0, ptrs=None):
    ptrs = ptrs or [FAKE] * 9
    return rma.lib().rma_decode_step(ctypes.byref(st), layer, *ptrs)


def test_decode_validation_on_host():
    L = rma.lib()
    st = _fake_state()
    assert L.rma_decode_step(None, 0, *([FAKE] * 9)) == rma.RMA_E_ARG
    assert _decode(st, layer=8) == rma.RMA_E_ARG
    assert _decode(st, layer=-1) == rma.RMA_E_ARG
    ptrs = [FAKE] * 9
    ptrs[0] = FAKE + 2  # misaligned q
    assert _decode(st, ptrs=ptrs) == rma.RMA_E_ARG
    ptrs = [FAKE] * 9
    ptrs[7] = None  # no output
    assert _decode(st, ptrs=ptrs) == rma.RMA_E_ARG
    full = _fake_state(pend_n=256)
    assert _decode(full) == rma.RMA_E_PENDING_FULL
    assert full.t[0] == 32768 and full.pend_n[0] == 256  # unchanged


def test_positions_past_the_int32_range_are_rejected_on_host():
    """Source positions are int32: a lockstep decode at position
    RMA_MAX_POS + 1, a prefill block reaching past it, and a state started
    past it are refused before anything is enqueued."""
    L = rma.lib()
    top = rma.RMA_MAX_POS + 1  # 2^31, a multiple of the commit interval 256
    st = _fake_state(pend_n=0, t=top)
    assert _decode(st) == rma.RMA_E_ARG
    assert L.rma_prefill_block(ctypes.byref(st), 0, 1, *([FAKE] * 9)) == rma.RMA_E_ARG
    assert st.t[0] == top and st.pend_n[0] == 0  # unchanged
    c = rma.config_default()
    s0 = rma._State()
    n = rma.state_bytes(c, 2)
    assert L.rma_state_init(ctypes.byref(s0), ctypes.byref(c), 2, FAKE, n, top, 0,
                            None) == rma.RMA_E_ARG


def test_admit_and_prefill_sequencing_on_host():
    L = rma.lib()
    st = _fake_state(pend_n=100, t=32768 + 100)
    assert L.rma_admit(ctypes.byref(st), 0, None) == rma.RMA_E_NOT_BOUNDARY
    assert L.rma_admit(ctypes.byref(st), -1, None) == rma.RMA_E_NOT_BOUNDARY
    assert L.rma_admit(ctypes.byref(st), -2, None) == rma.RMA_E_ARG
    assert L.rma_admit(ctypes.byref(st), 8, None) == rma.RMA_E_ARG
    assert L.rma_prefill_block(ctypes.byref(st), 0, 16, *([FAKE] * 9)) == rma.RMA_E_NOT_BOUNDARY
    st2 = _fake_state(pend_n=256)
    assert L.rma_prefill_block(ctypes.byref(st2), 0, 16, *([FAKE] * 9)) == rma.RMA_E_NOT_BOUNDARY
    st3 = _fake_state(pend_n=0)
    assert L.rma_prefill_block(ctypes.byref(st3), 0, 0, *([FAKE] * 9)) == rma.RMA_E_ARG
    assert L.rma_prefill_block(ctypes.byref(st3), 0, 257, *([FAKE] * 9)) == rma.RMA_E_ARG
    assert st.bank_n[0] == 1024 and st.pend_n[0] == 100


def test_state_init_validation_on_host():
    L = rma.lib()
    c = rma.config_default()
    st = rma._State()
    n = rma.state_bytes(c, 2)
    assert L.rma_state_init(ctypes.byref(st), ctypes.byref(c), 2, None, n, 0, 0, None) == rma.RMA_E_ARG
    assert L.rma_state_init(ctypes.byref(st), ctypes.byref(c), 2, FAKE + 16, n, 0, 0, None) == rma.RMA_E_ARG
    assert L.rma_state_init(ctypes.byref(st), ctypes.byref(c), 2, FAKE, n - 1, 0, 0, None) == rma.RMA_E_ARG
    assert L.rma_state_init(ctypes.byref(st), ctypes.byref(c), 2, FAKE, n, -1, 0, None) == rma.RMA_E_ARG
    assert L.rma_state_init(ctypes.byref(st), ctypes.byref(c), 2, FAKE, n, 0, 1025, None) == rma.RMA_E_ARG
    assert L.rma_state_init(None, ctypes.byref(c), 2, FAKE, n, 0, 0, None) == rma.RMA_E_ARG


def test_strerror_covers_every_code():
    L = rma.lib()
    seen = set()
    for code in (rma.RMA_OK, rma.RMA_E_ARG, rma.RMA_E_PENDING_FULL, rma.RMA_E_NOT_BOUNDARY,
                 rma.RMA_E_HIP, rma.RMA_E_UNSUPPORTED):
        s = L.rma_strerror(code).decode()
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 6
    assert L.rma_strerror(12345).decode() == "unknown status"


@pytest.mark.parametrize("S", [1023, 1024, 64, 63, 130, 1])
def test_k_plane_layout_helpers_follow_the_header(S):
    """The binding's natural <-> stored K conversion puts chunk c of slot s
    at uint4 index c*S + s, as include/rma.h states."""
    import torch
    from bounded_memory_decode_amd.rma import _k_to_natural, _k_to_stored
    d = 256
    nat = torch.arange(S * d, dtype=torch.int64).reshape(1, S, d)
    st = _k_to_stored(nat)[0]
    for s in sorted({x for x in (0, 5, 63, S - 1, S // 2) if x < S}):
        for c in (0, 7, 31):
            i = (c * S + s) * 8
            assert torch.equal(st[i:i + 8], nat[0, s, 8 * c:8 * c + 8])
    assert torch.equal(_k_to_natural(st[None], d), nat)


def test_positioned_calls_validation_on_host():
    """The per-sequence calls check pointers, layer, block size and the
    reset range on the host; nothing is enqueued on failure."""
    L = rma.lib()
    st = _fake_state()
    P = [FAKE] * 10  # q, q_anchor, k, v, cand_k, cand_v, cand_score, w_g, out, stream
    assert L.rma_decode_step_at(ctypes.byref(st), 0, None, *P) == rma.RMA_E_ARG
    assert L.rma_decode_step_at(ctypes.byref(st), 0, FAKE + 2, *P) == rma.RMA_E_ARG
    assert L.rma_decode_step_at(ctypes.byref(st), 8, FAKE, *P) == rma.RMA_E_ARG
    bad = list(P)
    bad[2] = FAKE + 8  # misaligned k
    assert L.rma_decode_step_at(ctypes.byref(st), 0, FAKE, *bad) == rma.RMA_E_ARG
    bad = list(P)
    bad[1] = FAKE + 8  # misaligned q_anchor
    assert L.rma_decode_step_at(ctypes.byref(st), 0, FAKE, *bad) == rma.RMA_E_ARG
    assert L.rma_prefill_block_at(ctypes.byref(st), 0, 16, FAKE, *bad) == rma.RMA_E_ARG
    assert L.rma_decode_step_at(None, 0, FAKE, *P) == rma.RMA_E_ARG
    assert L.rma_prefill_block_at(ctypes.byref(st), 0, 0, FAKE, *P) == rma.RMA_E_ARG
    assert L.rma_prefill_block_at(ctypes.byref(st), 0, 257, FAKE, *P) == rma.RMA_E_ARG
    assert L.rma_prefill_block_at(ctypes.byref(st), 0, 16, None, *P) == rma.RMA_E_ARG
    assert L.rma_prefill_block_at(ctypes.byref(st), -1, 16, FAKE, *P) == rma.RMA_E_ARG
    for first, count, n in ((-1, 1, 0), (0, 0, 0), (1, 2, 0), (2, 1, 0), (0, 1, -1),
                            (0, 1, 1025)):
        assert L.rma_seq_reset(ctypes.byref(st), first, count, n, None) == rma.RMA_E_ARG
    assert L.rma_seq_reset(None, 0, 1, 0, None) == rma.RMA_E_ARG
    # host counters untouched by failed calls
    assert st.t[0] == 32768 and st.pend_n[0] == 0 and st.bank_n[0] == 1024


@pytest.mark.parametrize("buf,nbytes,waves,sink", [
    (0, 1 << 20, 1024, FAKE),            # null buffer
    (FAKE + 8, 1 << 24, 1024, FAKE),     # misaligned buffer
    (FAKE, 1 << 24, 1026, FAKE),         # waves not a multiple of 4
    (FAKE, 1 << 24, 0, FAKE),            # no waves
    (FAKE, (1 << 24) + 16, 1024, FAKE),  # bytes not a multiple of waves * 16 KiB
    (FAKE, 0, 1024, FAKE),               # nothing to read
    (FAKE, 1 << 24, 1024, 0),            # null sink
])
def test_calibration_probe_rejects_bad_arguments(buf, nbytes, waves, sink):
    """rma_calib_stream_read refuses bad arguments on the host (-1) before
    anything is launched."""
    assert rma.lib().rma_calib_stream_read(buf, nbytes, waves, sink, None) == -1


def test_binding_constants_follow_the_header():
    """The binding's copies of the header's size constants are the header's."""
    import re
    h = open(os.path.join(ROOT, "include", "rma.h")).read()
    m = re.search(r"#define RMA_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", h)
    assert m, "RMA_STATIC_SCRATCH_BYTES not found in include/rma.h"
    assert rma.RMA_STATIC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
    # the largest split-K partials of an accepted configuration: 608 units
    # (batch 152 of the EdgeRock geometry) in 32 one-tile parts of 4,128 B
    assert 608 * 32 * 4128 <= rma.RMA_STATIC_SCRATCH_BYTES
