"""GPU check of the streaming-read probe behind the bench's achievable-
bandwidth figure (include/rma_calib.h): every wave must read every byte
of its share, so each wave's sink value equals the xor of all 32-bit
words of that share, computed here on the host."""
import numpy as np
import pytest
import torch

from bounded_memory_decode_amd import rma
import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("waves,turns", [(4, 1), (8, 3), (1024, 1)])
def test_stream_read_folds_every_word_of_each_share(waves, turns):
    gu.log(f"case calib waves={waves} turns={turns}")
    nbytes = waves * 16384 * turns  # a whole number of turns: waves x 64 lanes x 16 loads x 16 B
    rng = np.random.default_rng(waves * 7 + turns)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((waves,), -1, dtype=torch.int32, device="cuda")
    rma.calib_stream_read(buf, waves, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.reshape(waves, -1), axis=1)
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want)
