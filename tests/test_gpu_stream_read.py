"""The stream-read calibration kernel reads every byte it is given.

A measurement aid (the achievable HBM read rate beside the 8 TB/s peak), not
an operation of the method: its folds must XOR to the XOR of the buffer's
32-bit words, so no load was skipped or read twice an odd number of times.
"""
import numpy as np
import pytest

from pa_harness import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [0, 4, 4 * 1000 + 4, (64 << 20) // 4 + 12])
def test_folds_cover_every_word(gpu, words):
    import torch
    say(f"stream read: {words} words")
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2 ** 32, words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((gpu.pa_stream_read_sink_words(),), 12345, dtype=torch.int32, device="cuda")
    gpu.pa_stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host) if words else np.uint32(0)
    assert got == want
