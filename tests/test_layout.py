"""The packed weight format, checked on the CPU (no GPU needed).

The pages ask of the offline packing pass only that it be a lossless relayout
of the 4-bit codes into the order the matrix instructions consume them in
("LMDeploy Guide: Fast Mixed-Precision LLM Inference Engine", section 1
"Hardware-Aware Weight Packing (GEMM Pipeline)", steps 3 and 4). These tests
pin the written-out format in ``oracle`` to that: it is a bijection, it has
the documented size, each 1 KiB tile holds exactly one 128 x 16 block of
codes, and the shift-and-mask the kernels use on each 32-bit word yields
consecutive k pairs in the two fp16 halves.
"""
import numpy as np
import pytest

import oracle


def _rand(K, N, G, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    z = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    s = rng.standard_normal((K // G, N)).astype(np.float16)
    return q, z, s


@pytest.mark.parametrize("K,N,G", [(128, 16, 128), (256, 48, 64), (384, 32, 32), (512, 80, 256), (1024, 16, 128)])
def test_round_trip_is_bit_exact(K, N, G):
    q, z, s = _rand(K, N, G, seed=K + N)
    buf = oracle.layout_pack(q, z, s, G)
    assert buf.size == oracle.packed_bytes(K, N, G) == K * N // 2 + 5 * N * (K // G) // 2
    q2, z2, s2 = oracle.layout_unpack(buf, K, N, G)
    assert np.array_equal(q, q2) and np.array_equal(z, z2)
    assert np.array_equal(s.view(np.uint16), s2.view(np.uint16))


def test_pack_is_injective_on_single_code_changes():
    K, N, G = 256, 32, 128
    q, z, s = _rand(K, N, G, seed=3)
    base = oracle.layout_pack(q, z, s, G)
    rng = np.random.default_rng(4)
    seen = set()
    for _ in range(64):
        k, n = int(rng.integers(K)), int(rng.integers(N))
        q2 = q.copy()
        q2[k, n] ^= 0x5
        diff = np.nonzero(oracle.layout_pack(q2, z, s, G) != base)[0]
        assert diff.size == 1          # exactly one byte changes
        assert diff[0] < K * N // 2    # inside the weight region
        seen.add((int(diff[0]), k, n))
    # distinct (k, n) land in distinct (byte, nibble) places
    assert len({(b) for b, _, _ in seen}) >= len({(k // 2, n) for _, k, n in seen}) // 2


def test_each_tile_holds_one_128_by_16_block():
    K, N, G = 512, 64, 128
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    q = ((k // 128) * 5 + (n // 16) * 3) % 16
    q = q.astype(np.uint8) + np.zeros((K, N), np.uint8)
    z = np.zeros((K // G, N), np.uint8)
    s = np.ones((K // G, N), np.float16)
    buf = oracle.layout_pack(q, z, s, G)
    tiles = buf[: K * N // 2].reshape(N // 16, K // 128, 1024)
    for sn in range(N // 16):
        for kb in range(K // 128):
            v = (kb * 5 + sn * 3) % 16
            assert np.all(tiles[sn, kb] == v | (v << 4))


def test_word_masks_give_consecutive_k_pairs_of_each_step():
    # For lane l and word v of a tile, with w the word and w8 = w >> 8:
    #   w  & 0x000F000F -> codes of (k, k+1) of step 0,
    #   w8 & 0x000F000F -> step 1,
    #   w  & 0x00F000F0 -> step 2 (times 16),
    #   w8 & 0x00F000F0 -> step 3 (times 16),
    # where k = 128 kb + 32 t + 8 (l // 16) + 2 v, column 16 sn + l % 16.
    K, N, G = 256, 32, 128
    q, z, s = _rand(K, N, G, seed=9)
    buf = oracle.layout_pack(q, z, s, G)
    words = buf[: K * N // 2].view(np.uint32).reshape(N // 16, K // 128, 64, 4)
    for sn in range(N // 16):
        for kb in range(K // 128):
            for lane in range(64):
                n = 16 * sn + lane % 16
                for v in range(4):
                    w = int(words[sn, kb, lane, v])
                    w8 = w >> 8
                    got = {0: w & 0x000F000F, 1: w8 & 0x000F000F,
                           2: (w & 0x00F000F0) >> 4, 3: (w8 & 0x00F000F0) >> 4}
                    for t in range(4):
                        k = 128 * kb + 32 * t + 8 * (lane // 16) + 2 * v
                        assert got[t] & 0xFFFF == q[k, n]
                        assert got[t] >> 16 == q[k + 1, n]


def test_scale_and_zero_records():
    K, N, G = 256, 32, 64
    q, z, s = _rand(K, N, G, seed=11)
    buf = oracle.layout_pack(q, z, s, G)
    base = K * N // 2
    sreg = buf[base: base + 2 * N * (K // G)].view(np.uint16).reshape(N // 16, K // G, 16)
    zreg = buf[base + 2 * N * (K // G):].reshape(N // 16, K // G, 8)
    for g in range(K // G):
        for n in range(N):
            assert sreg[n // 16, g, n % 16] == s.view(np.uint16)[g, n]
            assert (zreg[n // 16, g, (n % 16) // 2] >> (4 * (n % 2))) & 15 == z[g, n]


@pytest.mark.parametrize("K,N,G", [(100, 16, 4), (128, 8, 128), (128, 16, 96), (128, 16, 512), (0, 16, 128)])
def test_rejects_unsupported_shapes(K, N, G):
    with pytest.raises(ValueError):
        oracle.packed_bytes(K, N, G)


def test_rejects_out_of_range_codes():
    q, z, s = _rand(128, 16, 128)
    q[3, 3] = 16
    with pytest.raises(ValueError):
        oracle.layout_pack(q, z, s, 128)
