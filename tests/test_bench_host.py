"""Host-side checks of bench.py (no GPU): the one-GPU contract, the
algorithmic byte and flop counts its rooflines divide by, and the rule
that the committed HBM counters are used only for the sources they were
taken on."""
import os
import subprocess
import sys

import bench
from bounded_memory_decode_amd import rma

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unit_bytes_follow_the_library_layout():
    """The ring and bank bytes per (sequence, layer, group) in the roofline
    are the record bytes the library's own layout accounts for (the pages'
    31.97 / 32.00 MiB per sequence), and the unit total is the sum of its
    reads and writes."""
    cfg = rma.config_default()
    L = rma.state_layout(cfg, 1)
    units = cfg.layers * cfg.kv_groups
    assert bench.RING_BYTES == L.ring_bytes // units == 1023 * 1024
    assert bench.BANK_BYTES == L.bank_bytes // units == 1024 * 1024
    assert bench.UNIT_BYTES == bench.UNIT_READ + bench.UNIT_WRITE == 2_104_328


def test_prefill_flop_per_block_layer():
    """4 groups x 1,024 query rows x 2,048 keys x 256 dims x 2 products x
    2 flop: 8.59 GFLOP per 256-token block of one layer."""
    assert 4 * bench.PREFILL_FLOP_PER_GROUP == 8_589_934_592


def test_traffic_only_for_the_profiled_sources():
    sha = bench.kernel_sources_sha()
    assert bench.read_traffic("0" * 16) is None
    t = bench.read_traffic(sha)
    if t is not None:  # the committed profile matches these sources
        algorithmic = 512 * 4 * bench.UNIT_BYTES  # one batch-512 launch
        assert algorithmic <= t < 1.5 * algorithmic
