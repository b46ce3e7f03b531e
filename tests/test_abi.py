"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects bad arguments before any HIP call (so this runs without a GPU)."""
import ctypes
import os
import re

import pytest

import oracle
import w4a16_mixed_precision_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")
FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("w4a16_packed_bytes", "w4a16_pack", "w4a16_unpack", "w4a16_workspace_bytes",
              "w4a16_gemm", "w4a16_gemm_ex", "w4a16_status_string", "w4a16_last_error",
              "w4a16_layout_version", "w4a16_auto_path", "w4a16_quantize", "w4a16_quantize_pack",
              "w4a16_kv_block_bytes", "w4a16_kv_append", "w4a16_kv_attention_workspace_bytes",
              "w4a16_kv_attention", "w4a16_w8a8_packed_bytes", "w4a16_w8a8_quantize_weights",
              "w4a16_w8a8_quantize_act", "w4a16_w8a8_workspace_bytes", "w4a16_w8a8_gemm"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = w4.lib()
    for n in _declared():
        assert hasattr(L, n), n


def test_packed_bytes_matches_layout_spec():
    for K, N, G in [(256, 256, 128), (4096, 6144, 128), (29568, 8192, 64), (512, 16, 32), (512, 32, 256)]:
        assert w4.w4a16_packed_bytes(K, N, G) == oracle.packed_bytes(K, N, G)
    for K, N, G in [(100, 16, 4), (128, 8, 128), (128, 16, 96), (0, 16, 128), (192, 16, 64), (128, 16, 512)]:
        assert w4.w4a16_packed_bytes(K, N, G) == 0


def test_layout_version():
    assert w4.w4a16_layout_version() == 2


def test_auto_path_rule():
    D, P = w4.W4A16_PATH_DECODE, w4.W4A16_PATH_PREFILL
    assert w4.w4a16_auto_path(1, 6144, 4096, 128) == D
    assert w4.w4a16_auto_path(32, 57344, 8192, 128) == D
    assert w4.w4a16_auto_path(33, 57344, 8192, 128) == P
    assert w4.w4a16_auto_path(64, 6144, 4096, 128) == D
    assert w4.w4a16_auto_path(64, 8192, 28672, 128) == P
    assert w4.w4a16_auto_path(65, 4096, 14336, 128) == P
    assert w4.lib().w4a16_auto_path(1, 6144, 100, 128) == w4.W4A16_ERR_SHAPE


def test_gemm_validation_before_any_hip_call():
    L = w4.lib()
    assert L.w4a16_gemm(None, FAKE, 1, 256, 256, 128, FAKE, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_gemm(FAKE, FAKE, 0, 256, 256, 128, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_gemm(FAKE, FAKE, 1, 250, 256, 128, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_gemm(FAKE, FAKE, 1, 256, 200, 128, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_gemm(FAKE, FAKE, 1, 256, 256, 96, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_gemm(MISALIGNED, FAKE, 1, 256, 256, 128, FAKE, None) == w4.W4A16_ERR_ALIGN
    assert "16-byte" in w4.w4a16_last_error()
    assert L.w4a16_gemm(FAKE, FAKE, 1, 256, 256, 128, MISALIGNED, None) == w4.W4A16_ERR_ALIGN


def test_gemm_ex_plan_and_workspace_validation():
    L = w4.lib()
    # path out of range
    assert L.w4a16_gemm_ex(FAKE, FAKE, 4, 256, 256, 128, FAKE, None, 0, 7, 1, None) == w4.W4A16_ERR_ARG
    # decode path is limited to M <= 64
    assert L.w4a16_gemm_ex(FAKE, FAKE, 65, 256, 256, 128, FAKE, None, 0, 1, 1, None) == w4.W4A16_ERR_ARG
    # more splits than 128-row blocks
    assert L.w4a16_gemm_ex(FAKE, FAKE, 4, 256, 256, 128, FAKE, None, 0, 1, 3, None) == w4.W4A16_ERR_ARG
    # negative split counts
    assert L.w4a16_gemm_ex(FAKE, FAKE, 4, 256, 256, 128, FAKE, None, 0, 2, -1, None) == w4.W4A16_ERR_ARG
    # a split plan without (enough) workspace
    assert L.w4a16_gemm_ex(FAKE, FAKE, 4, 256, 256, 128, FAKE, None, 0, 1, 2, None) == w4.W4A16_ERR_WORKSPACE
    need = w4.w4a16_workspace_bytes(4, 256, 256, 128, w4.W4A16_PATH_DECODE, 2)
    assert need > 0
    assert L.w4a16_gemm_ex(FAKE, FAKE, 4, 256, 256, 128, FAKE, FAKE, need - 1, 1, 2, None) == w4.W4A16_ERR_WORKSPACE
    # unsplit plans need none
    assert w4.w4a16_workspace_bytes(4, 256, 256, 128, w4.W4A16_PATH_DECODE, 1) == 0
    assert w4.w4a16_workspace_bytes(4, 256, 256, 128, w4.W4A16_PATH_PREFILL, 1) == 0
    assert w4.w4a16_workspace_bytes(512, 8192, 8192, 64, w4.W4A16_PATH_PREFILL, 4) == 4 * 512 * 8192 * 4
    # split workspace covers S * M * N fp32 partials plus counters
    assert w4.w4a16_workspace_bytes(16, 4096, 14336, 128, w4.W4A16_PATH_DECODE, 8) >= 8 * 16 * 4096 * 4


def test_pack_validation_before_any_hip_call():
    L = w4.lib()
    assert L.w4a16_pack(None, FAKE, FAKE, 256, 256, 128, FAKE, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_pack(FAKE, FAKE, FAKE, 256, 250, 128, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_pack(FAKE, FAKE, FAKE, 256, 256, 128, MISALIGNED, None) == w4.W4A16_ERR_ALIGN
    assert L.w4a16_unpack(FAKE, 256, 256, 128, None, FAKE, FAKE, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_unpack(FAKE, 256, 256, 100, FAKE, FAKE, FAKE, None) == w4.W4A16_ERR_SHAPE


def test_quantize_validation_before_any_hip_call():
    L = w4.lib()
    assert L.w4a16_quantize(None, 256, 256, 128, FAKE, FAKE, FAKE, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_quantize(FAKE, 256, 256, 128, FAKE, None, FAKE, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_quantize(FAKE, 256, 250, 128, FAKE, FAKE, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_quantize(FAKE, 192, 256, 64, FAKE, FAKE, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_quantize(MISALIGNED, 256, 256, 128, FAKE, FAKE, FAKE, None) == w4.W4A16_ERR_ALIGN
    assert L.w4a16_quantize(FAKE, 256, 256, 128, FAKE, MISALIGNED, FAKE, None) == w4.W4A16_ERR_ALIGN
    assert L.w4a16_quantize_pack(FAKE, 256, 256, 128, None, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_quantize_pack(FAKE, 256, 256, 96, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_quantize_pack(FAKE, 256, 256, 128, MISALIGNED, None) == w4.W4A16_ERR_ALIGN


def test_kv_and_w8a8_validation_before_any_hip_call():
    L = w4.lib()
    assert w4.w4a16_kv_block_bytes(8, 8) == 8 * (2 * 64 * 128 + 512)
    assert w4.w4a16_kv_block_bytes(4, 2) == 2 * (2 * 64 * 64 + 512)
    assert w4.w4a16_kv_block_bytes(5, 2) == 0
    assert L.w4a16_kv_append(None, FAKE, FAKE, 1, 8, 8, FAKE, 1, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_kv_append(FAKE, FAKE, FAKE, 1, 8, 6, FAKE, 1, None) == w4.W4A16_ERR_ARG
    assert L.w4a16_kv_append(FAKE, FAKE, MISALIGNED, 1, 8, 8, FAKE, 1, None) == w4.W4A16_ERR_ALIGN
    # 12 query heads over 8 KV heads, and 17 query heads per KV head, are refused
    args = lambda hq, hkv: L.w4a16_kv_attention(FAKE, FAKE, 1, FAKE, 1, FAKE, 1, hq, hkv, 8,
                                                 ctypes.c_float(0.1), FAKE, FAKE, 1 << 20, None)
    assert args(12, 8) == w4.W4A16_ERR_SHAPE and args(17, 1) == w4.W4A16_ERR_SHAPE
    big = L.w4a16_kv_attention(FAKE, FAKE, 1, FAKE, (1 << 24) + 1, FAKE, 1, 8, 8, 8, ctypes.c_float(0.1),
                               FAKE, FAKE, 1 << 20, None)
    assert big == w4.W4A16_ERR_SHAPE and w4.w4a16_kv_attention_workspace_bytes(1 << 20, 128, 4) == 0
    assert w4.w4a16_w8a8_packed_bytes(512, 64) == 512 * 64
    assert w4.w4a16_w8a8_packed_bytes(320, 64) == 0 and w4.w4a16_w8a8_packed_bytes(1 << 18, 16) == 0
    assert L.w4a16_w8a8_gemm(FAKE, FAKE, FAKE, FAKE, 1, 64, 320, FAKE, None, 0, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_w8a8_gemm(FAKE, None, FAKE, FAKE, 1, 64, 256, FAKE, None, 0, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_w8a8_quantize_act(FAKE, 0, 256, FAKE, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_w8a8_quantize_weights(FAKE, 256, 24, FAKE, FAKE, None) == w4.W4A16_ERR_SHAPE


def test_stream_read_validation_before_any_hip_call():
    L = w4.lib()
    assert L.w4a16_stream_read(FAKE, 0, 0, FAKE, None) == w4.W4A16_ERR_SHAPE
    # offsets past the end are steered to 2^31, so the buffer stays below it
    assert L.w4a16_stream_read(FAKE, 1 << 31, 0, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_stream_read(None, 1024, 0, FAKE, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_stream_read(MISALIGNED, 1024, 0, FAKE, None) == w4.W4A16_ERR_ALIGN


def test_status_strings():
    for code in range(-7, 1):
        assert w4.w4a16_status_string(code) not in ("", "unknown status")
    assert w4.w4a16_status_string(-99) == "unknown status"


def test_python_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    X = torch.zeros((1, 256), dtype=torch.float16)
    packed = torch.zeros(w4.w4a16_packed_bytes(256, 256, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):
        w4.w4a16_gemm(X, packed, 256, 256, 128)


def test_weight_bytes_bound_rejects_shapes_the_prefill_descriptors_cannot_address():
    """The prefill kernel reaches the whole packed weight region through one
    buffer descriptor with a 32-bit byte count, so the boundary refuses
    K * N / 2 >= 2^31 (e.g. K = N = 65536, and K = N = 131072, whose 8 GiB
    would wrap a 32-bit count to 0 and read zeros)."""
    L = w4.lib()
    for K, N in [(65536, 65536), (131072, 131072), (1 << 22, 1024)]:
        assert w4.w4a16_packed_bytes(K, N, 128) == 0
        assert L.w4a16_gemm(FAKE, FAKE, 1, N, K, 128, FAKE, None) == w4.W4A16_ERR_SHAPE
        assert "2^31" in w4.w4a16_last_error()
        assert L.w4a16_pack(FAKE, FAKE, FAKE, K, N, 128, FAKE, None) == w4.W4A16_ERR_SHAPE
        assert L.w4a16_quantize_pack(FAKE, K, N, 128, FAKE, None) == w4.W4A16_ERR_SHAPE
    # just below the bound is accepted: 65536 x 65520 / 2 < 2^31
    assert w4.w4a16_packed_bytes(65536, 65520, 128) == oracle.packed_bytes(65536, 65520, 128)


def test_python_binding_checks_the_packed_size_before_any_launch():
    """A packed tensor one byte short of w4a16_packed_bytes(K, N, G) is refused
    in the binding (the kernels size their reads from K, N and G, not from the
    allocation); the check runs before the tensors are even looked at as
    device pointers, so it holds without a GPU."""
    torch = pytest.importorskip("torch")
    K, N, G = 256, 256, 128
    need = w4.w4a16_packed_bytes(K, N, G)
    X = torch.zeros((1, K), dtype=torch.float16)
    short = torch.zeros(need - 1, dtype=torch.uint8)
    for call in (lambda: w4.w4a16_gemm(X, short, N, K, G),
                 lambda: w4.w4a16_gemm_ex(X, short, N, K, G),
                 lambda: w4.w4a16_unpack(short, K, N, G)):
        with pytest.raises(ValueError, match="needs"):
            call()
    q = torch.zeros((K, N), dtype=torch.uint8)
    z = torch.zeros((K // G, N), dtype=torch.uint8)
    s = torch.zeros((K // G, N), dtype=torch.float16)
    with pytest.raises(ValueError, match="needs"):
        w4.w4a16_pack(q, z, s, G, packed=short)


def test_noalloc_gemm_validation_before_any_hip_call():
    L = w4.lib()
    assert w4.W4A16_NOALLOC_SCRATCH_BYTES == 64 << 20
    assert L.w4a16_gemm_noalloc(None, FAKE, 1, 256, 256, 128, FAKE, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_gemm_noalloc(FAKE, FAKE, 1, 250, 256, 128, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_gemm_noalloc(FAKE, FAKE, 0, 256, 256, 128, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_gemm_noalloc(FAKE, FAKE, 1, 65536, 65536, 128, FAKE, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_gemm_noalloc(MISALIGNED, FAKE, 1, 256, 256, 128, FAKE, None) == w4.W4A16_ERR_ALIGN


def test_binding_loads_the_library_on_torchs_hip_runtime():
    """ROCm wheels of torch carry their own libamdhip64 (same soname as the
    system one): loading libw4a16.so first would put two HIP runtimes in the
    process and torch would see no GPU. The binding imports torch first, so
    only torch's copy is mapped (checked in a fresh interpreter)."""
    import subprocess
    import sys
    pytest.importorskip("torch")
    code = ("import w4a16_mixed_precision_amd as w4; w4.lib(); "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    mapped = eval(out.stdout.strip().splitlines()[-1])
    assert len(mapped) == 1 and "torch" in mapped[0], mapped
