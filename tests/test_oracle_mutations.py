"""The pins catch what they claim to catch: each plausible mistake below is
planted in a copy of the oracle's C source (on the CPU), the copy is built
into a temporary directory, and the pins of tests/test_oracle_pins.py that
should notice it run against that build in a child process
(RMA_ORACLE_LIBRARY).  At least one of them must fail.

Every mutation keeps all indices in range; each changes one fact of the
method: the window, the current token, the softmax scale, the gate's sign
or its group mean, the query of the anchor read, the ring slot written,
the tie-break, the NaN order, the compaction order, the source positions,
and the token/batch slicing of a prompt block."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "rma_oracle.c")
HDR = os.path.join(ROOT, "oracle", "rma_oracle.h")
PINS = os.path.join(HERE, "test_oracle_pins.py")

READS = "bruteforce or sdpa or constant or identical or planted"
MUTATIONS = {
    # (text in rma_oracle.c, replacement, pins to run)
    "window_short_by_one": (
        "const int64_t first = t - R > 0 ? t - R : 0;",
        "const int64_t first = t - R + 1 > 0 ? t - R + 1 : 0;", READS + " or ring_holds"),
    "current_token_dropped": (
        "attend(d, c->scale, q, nloc, lk, lv, s, oloc);",
        "attend(d, c->scale, q, nloc > 1 ? nloc - 1 : nloc, lk, lv, s, oloc);", READS),
    "scale_dropped": ("s[j] = scale * acc;", "s[j] = acc;", READS),
    "gate_sign_flipped": (
        "out[(size_t)h * d + i] = oloc[i] + gate * oanc[i];",
        "out[(size_t)h * d + i] = oloc[i] - gate * oanc[i];", READS),
    "anchor_read_uses_q": (
        "attend(d, c->scale, qa, n, ak, av, s, oanc);",
        "attend(d, c->scale, q, n, ak, av, s, oanc);", "anchor"),
    "group_gate_without_mean": (
        "zg += (qm[i] / hpg) * (double)w_g[(size_t)g * d + i];",
        "zg += qm[i] * (double)w_g[(size_t)g * d + i];", "group_gate"),
    "ring_slot_off_by_one": (
        "const size_t rs = (size_t)(t % c->R), ps = (size_t)(t % c->C);",
        "const size_t rs = (size_t)((t + 1) % c->R), ps = (size_t)(t % c->C);",
        READS + " or ring_holds"),
    "tie_break_reversed": (
        "return (a->gidx > b->gidx) - (a->gidx < b->gidx);",
        "return (a->gidx < b->gidx) - (a->gidx > b->gidx);", "lexsort or hand_worked"),
    "nan_ranked_first": (
        "  if (isnan(a)) return 0;\n  if (isnan(b)) return 1;",
        "  if (isnan(a)) return !isnan(b);\n  if (isnan(b)) return 0;", "lexsort or hand_worked"),
    "compaction_order_reversed": (
        "const int dst = a < ne ? evicted[a] : n + (a - ne);",
        "const int dst = a < ne ? evicted[ne - 1 - a] : n + (a - ne);",
        "hand_worked or compaction"),
    "source_position_off_by_one": (
        "st->bsrc[u * N + dst] = (int32_t)(block_start + j);",
        "st->bsrc[u * N + dst] = (int32_t)(block_start + j + 1);", "hand_worked or bruteforce"),
    "prefill_query_sliced_n_major": (
        "memcpy(tq + (size_t)b * H * d, q + ((size_t)b * n + i) * H * d,",
        "memcpy(tq + (size_t)b * H * d, q + ((size_t)i * B + b) * H * d,", "prefill"),
}


def _run_pins(tmp_path, source: str, select: str):
    """Build `source` as the oracle library in tmp_path and run the pins
    matching `select` against it in a child process."""
    (tmp_path / "rma_oracle.c").write_text(source)
    shutil.copy(HDR, tmp_path / "rma_oracle.h")
    lib = tmp_path / "librma_oracle.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC",
                    str(tmp_path / "rma_oracle.c"), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, RMA_ORACLE_LIBRARY=str(lib))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "-m", "not gpu", PINS, "-k", select],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_pins_pass_on_an_unmodified_copy(tmp_path):
    """Control: the same harness with the source unchanged passes every
    selection used below, so a failure there comes from the mistake."""
    select = " or ".join(f"({m[2]})" for m in MUTATIONS.values())
    r = _run_pins(tmp_path, open(SRC).read(), select)
    assert r.returncode == 0, f"unmodified oracle failed (exit {r.returncode}):\n{r.stdout[-1500:]}"


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_fail_on_a_planted_mistake(name, tmp_path):
    old, new, select = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"{name}: the mutated text must occur once in rma_oracle.c"
    r = _run_pins(tmp_path, src.replace(old, new), select)
    # pytest exits 1 when a test failed; 0 (all passed) or 5 (nothing
    # selected) mean the pins missed the mistake
    assert r.returncode == 1, (f"mutation {name}: the pins selected by {select!r} did not "
                               f"fail (exit {r.returncode}):\n{r.stdout[-1500:]}")
