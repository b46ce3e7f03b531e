"""HIP-graph replays of the KV-cache attention (attention + chunk merge
kernels) and the W8A8 GEMM (activation quantization + GEMM + split-K sum):
every replay must reproduce the eager result bit for bit, with eager calls
on the same buffers between replays."""
import math

import numpy as np
import pytest

import w4a16_mixed_precision_amd as w4
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def _replay_check(run, outputs):
    import torch
    ref = [host(t).copy() for t in run(None)]
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        run(st)
        st.synchronize()
        with torch.cuda.graph(g, stream=st):
            run(st)
    for i in range(4):
        for t in outputs:
            t.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outputs, ref):
            assert np.array_equal(host(t).view(np.uint8), r.view(np.uint8)), f"replay {i}"
        eager = [host(t).copy() for t in run(None)]
        torch.cuda.synchronize()
        for e, r in zip(eager, ref):
            assert np.array_equal(e.view(np.uint8), r.view(np.uint8)), f"eager after replay {i}"


@pytest.mark.parametrize("bits", [8, 4])
def test_kv_attention_graph_replays(bits):
    import torch
    say(f"graph replay kv attention bits={bits}")
    B, hq, hkv, T = 3, 8, 2, 300
    nb = (T + 63) // 64
    table = torch.arange(B * nb, dtype=torch.int32, device="cuda").reshape(B, nb)
    slots = (table[:, :, None] * 64 + torch.arange(64, dtype=torch.int32, device="cuda")).reshape(B, -1)[:, :T]
    cache = torch.zeros(B * nb * w4.w4a16_kv_block_bytes(bits, hkv), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(bits)
    k = dev(rng.standard_normal((B * T, hkv, 128)).astype(np.float16))
    v = dev(rng.standard_normal((B * T, hkv, 128)).astype(np.float16))
    w4.w4a16_kv_append(k, v, slots.reshape(-1).contiguous(), bits, cache)
    q = dev(rng.standard_normal((B, hq, 128)).astype(np.float16))
    lengths = torch.tensor([T, 17, 200], dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(w4.w4a16_kv_attention_workspace_bytes(B, hkv, nb), dtype=torch.uint8, device="cuda")

    def run(stream):
        w4.w4a16_kv_attention(q, cache, table, lengths, bits, hkv, 1 / math.sqrt(128), out=out, workspace=ws,
                              stream=stream)
        return [out]

    _replay_check(run, [out])


@pytest.mark.parametrize("M", [1, 16, 100])
def test_w8a8_graph_replays(M):
    import torch
    say(f"graph replay w8a8 M={M}")
    K, N = 2048, 512
    rng = np.random.default_rng(M)
    W = dev((rng.standard_normal((K, N)) * 0.02).astype(np.float16))
    X = dev(rng.standard_normal((M, K)).astype(np.float16))
    packed, wsc = w4.w4a16_w8a8_quantize_weights(W)
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    need = w4.w4a16_w8a8_workspace_bytes(M, N, K)
    wsp = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def run(stream):
        s = stream if stream is not None else torch.cuda.current_stream()
        w4.lib().w4a16_w8a8_quantize_act(X.data_ptr(), M, K, xq.data_ptr(), xs.data_ptr(), s.cuda_stream)
        w4.w4a16_w8a8_gemm(xq, xs, packed, wsc, N, Y=Y, workspace=wsp, stream=stream)
        return [xq, xs, Y]

    _replay_check(run, [xq, xs, Y])
