"""The streaming-read yardstick reads exactly the bytes it is given: each
wave folds its chunks into one word per lane, and a lane's word is stored
only when it equals the caller's `never`. Choosing `never` as the fold the
host computes for the lane that holds the last byte (bytes past the end
counted as zeros) checks that the launch covered the tail and read nothing
past it, while the allocation behind the end holds random bytes."""
from __future__ import annotations

import numpy as np
import pytest

import w4a16_mixed_precision_amd as w4
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _host_folds(data: np.ndarray, n: int) -> np.ndarray:
    """[waves, 64] folds of the first n bytes (zeros past n), in the launch
    shape the library uses: 12 chunks of 1 KiB per wave up to 12288 chunks,
    4 above."""
    chunks = (n + 1023) // 1024
    U = 12 if chunks <= 256 * 4 * 12 else 4
    waves = (chunks + U - 1) // U
    buf = np.zeros(waves * U * 1024, dtype=np.uint8)
    buf[:n] = data[:n]
    words = buf.view(np.uint32).reshape(waves, U, 64, 4)
    return np.bitwise_xor.reduce(np.bitwise_xor.reduce(words, axis=1), axis=2)


@pytest.mark.parametrize("n", [16, 1024, 2 * 12 * 1024 + 7 * 16, 12 * 1024 * 1024 + 5 * 1024 + 256])
def test_stream_read_covers_exactly_the_buffer(n):
    import torch
    say(f"stream read n={n}")
    rng = np.random.default_rng(n)
    data = rng.integers(0, 256, size=n + 65536, dtype=np.uint8)
    folds = _host_folds(data, n)
    wave, lane = ((n - 1) // 1024) // (12 if (n + 1023) // 1024 <= 12288 else 4), ((n - 1) % 1024) // 16
    never = int(folds[wave, lane])
    assert never != 0xFFFFFFFF
    buf = dev(data)
    sink = torch.full((64,), -1, dtype=torch.int32, device="cuda")
    w4.w4a16_stream_read(buf, sink, nbytes=n, never=never)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    hit = (folds == never).any(axis=0)
    assert got[lane] == never
    assert np.all(got[hit] == never) and np.all(got[~hit] == 0xFFFFFFFF)
