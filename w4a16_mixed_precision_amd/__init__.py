"""Python binding of libw4a16.so, the W4A16 GEMM library for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/w4a16.h``. PyTorch supplies
device memory and streams; tensors are passed as raw device pointers. The
functions carry the C names and follow the C argument order; shapes are
taken from the tensors where the C call needs them explicitly.

If the library is not built, every call raises: there is no fallback.

PyTorch wheels for ROCm carry their own HIP runtime (libamdhip64.so, the
same soname as the system one libw4a16.so links against). Whichever copy is
loaded first serves the whole process; if the system copy came first, the
wheel's runtime would load beside it and torch would find no GPU. ``lib()``
therefore imports torch before it loads libw4a16.so, so the library binds
to torch's runtime: one HIP runtime per process, shared with the tensors
and streams it is handed.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "W4A16Error", "lib", "library_path",
    "W4A16_OK", "W4A16_ERR_NULL", "W4A16_ERR_SHAPE", "W4A16_ERR_ALIGN", "W4A16_ERR_RANGE",
    "W4A16_ERR_HIP", "W4A16_ERR_WORKSPACE", "W4A16_ERR_ARG",
    "W4A16_PATH_AUTO", "W4A16_PATH_DECODE", "W4A16_PATH_PREFILL",
    "w4a16_packed_bytes", "w4a16_pack", "w4a16_unpack", "w4a16_workspace_bytes",
    "w4a16_gemm", "w4a16_gemm_ex", "w4a16_gemm_noalloc", "W4A16_NOALLOC_SCRATCH_BYTES", "w4a16_status_string", "w4a16_last_error",
    "w4a16_layout_version", "w4a16_auto_path", "w4a16_quantize", "w4a16_quantize_pack",
    "w4a16_kv_block_bytes", "w4a16_kv_append", "w4a16_kv_attention_workspace_bytes", "w4a16_kv_attention",
    "w4a16_w8a8_packed_bytes", "w4a16_w8a8_quantize_weights", "w4a16_w8a8_quantize_act",
    "w4a16_w8a8_workspace_bytes", "w4a16_w8a8_gemm", "w4a16_stream_read",
]

W4A16_OK = 0
W4A16_ERR_NULL = -1
W4A16_ERR_SHAPE = -2
W4A16_ERR_ALIGN = -3
W4A16_ERR_RANGE = -4
W4A16_ERR_HIP = -5
W4A16_ERR_WORKSPACE = -6
W4A16_ERR_ARG = -7
W4A16_PATH_AUTO = 0
W4A16_PATH_DECODE = 1
W4A16_PATH_PREFILL = 2
W4A16_NOALLOC_SCRATCH_BYTES = 64 << 20

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a16.so")
_lib = None


class W4A16Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def lib():
    """The loaded C library (ctypes.CDLL). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(
            f"{library_path} is missing: build it with `python -m w4a16_mixed_precision_amd.build`")
    try:  # torch's HIP runtime first (see the module docstring)
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(library_path)
    P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    L.w4a16_packed_bytes.argtypes = [I64, I64, I64]
    L.w4a16_packed_bytes.restype = SZ
    L.w4a16_pack.argtypes = [P, P, P, I64, I64, I64, P, P]
    L.w4a16_pack.restype = I
    L.w4a16_unpack.argtypes = [P, I64, I64, I64, P, P, P, P]
    L.w4a16_unpack.restype = I
    L.w4a16_workspace_bytes.argtypes = [I64, I64, I64, I64, I, I]
    L.w4a16_workspace_bytes.restype = SZ
    L.w4a16_gemm.argtypes = [P, P, I64, I64, I64, I64, P, P]
    L.w4a16_gemm.restype = I
    L.w4a16_gemm_ex.argtypes = [P, P, I64, I64, I64, I64, P, P, SZ, I, I, P]
    L.w4a16_gemm_ex.restype = I
    L.w4a16_gemm_noalloc.argtypes = [P, P, I64, I64, I64, I64, P, P]
    L.w4a16_gemm_noalloc.restype = I
    L.w4a16_status_string.argtypes = [I]
    L.w4a16_status_string.restype = ctypes.c_char_p
    L.w4a16_last_error.argtypes = []
    L.w4a16_last_error.restype = ctypes.c_char_p
    L.w4a16_layout_version.argtypes = []
    L.w4a16_layout_version.restype = I
    L.w4a16_auto_path.argtypes = [I64, I64, I64, I64]
    L.w4a16_quantize.argtypes = [P, I64, I64, I64, P, P, P, P]
    L.w4a16_quantize.restype = I
    L.w4a16_quantize_pack.argtypes = [P, I64, I64, I64, P, P]
    L.w4a16_quantize_pack.restype = I
    L.w4a16_kv_block_bytes.argtypes = [I, I64]
    L.w4a16_kv_block_bytes.restype = SZ
    L.w4a16_kv_append.argtypes = [P, P, P, I64, I64, I, P, I64, P]
    L.w4a16_kv_append.restype = I
    L.w4a16_kv_attention_workspace_bytes.argtypes = [I64, I64, I64]
    L.w4a16_kv_attention_workspace_bytes.restype = SZ
    L.w4a16_kv_attention.argtypes = [P, P, I64, P, I64, P, I64, I64, I64, I, ctypes.c_float, P, P, SZ, P]
    L.w4a16_kv_attention.restype = I
    L.w4a16_w8a8_packed_bytes.argtypes = [I64, I64]
    L.w4a16_w8a8_packed_bytes.restype = SZ
    L.w4a16_w8a8_quantize_weights.argtypes = [P, I64, I64, P, P, P]
    L.w4a16_w8a8_quantize_weights.restype = I
    L.w4a16_w8a8_quantize_act.argtypes = [P, I64, I64, P, P, P]
    L.w4a16_w8a8_quantize_act.restype = I
    L.w4a16_w8a8_workspace_bytes.argtypes = [I64, I64, I64]
    L.w4a16_w8a8_workspace_bytes.restype = SZ
    L.w4a16_w8a8_gemm.argtypes = [P, P, P, P, I64, I64, I64, P, P, SZ, P]
    L.w4a16_w8a8_gemm.restype = I
    L.w4a16_auto_path.restype = I
    L.w4a16_stream_read.argtypes = [P, SZ, ctypes.c_uint32, P, P]
    L.w4a16_stream_read.restype = I
    _lib = L
    return L


def _check(rc: int):
    if rc != W4A16_OK:
        raise W4A16Error(rc, lib().w4a16_last_error().decode() or
                         lib().w4a16_status_string(rc).decode())


def _dev_ptr(t, dtype, name):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _same_device(*named):
    """Raise ValueError unless every given tensor sits on one device."""
    devs = {(n, t.device) for n, t in named if t is not None}
    if len({d for _, d in devs}) > 1:
        raise ValueError("tensors on different devices: " +
                         ", ".join(f"{n} on {d}" for n, d in sorted(devs, key=lambda x: x[0])))


def _check_packed(packed, K: int, N: int, G: int, name: str = "packed"):
    """Raise before any launch if `packed` cannot hold the packed layout of a
    K x N weight with groups of G: the kernels size their buffer
    descriptors from K, N and G, not from the allocation."""
    need = w4a16_packed_bytes(K, N, G)
    if need == 0:
        raise ValueError(f"unsupported shape K={K} N={N} G={G}")
    have = packed.numel() * packed.element_size()
    if have < need:
        raise ValueError(f"{name} holds {have} bytes, K={K} N={N} G={G} needs {need}")


def _stream(stream, device):
    import torch
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def w4a16_status_string(status: int) -> str:
    return lib().w4a16_status_string(int(status)).decode()


def w4a16_last_error() -> str:
    return lib().w4a16_last_error().decode()


def w4a16_layout_version() -> int:
    return int(lib().w4a16_layout_version())


def w4a16_auto_path(M: int, N: int, K: int, G: int) -> int:
    """Path the automatic plan takes for this shape (W4A16_PATH_DECODE or
    W4A16_PATH_PREFILL)."""
    rc = int(lib().w4a16_auto_path(M, N, K, G))
    _check(rc if rc < 0 else 0)
    return rc


def w4a16_packed_bytes(K: int, N: int, G: int) -> int:
    return int(lib().w4a16_packed_bytes(K, N, G))


def w4a16_workspace_bytes(M: int, N: int, K: int, G: int, path: int = W4A16_PATH_AUTO,
                          splits: int = 0) -> int:
    return int(lib().w4a16_workspace_bytes(M, N, K, G, path, splits))


def w4a16_pack(q, zeros, scales, G: int, packed=None, stream=None):
    """Pack uint8 q [K][N], uint8 zeros [K/G][N], fp16 scales [K/G][N] (device
    tensors) into a uint8 device tensor of w4a16_packed_bytes(K, N, G) bytes."""
    import torch
    K, N = q.shape
    nbytes = w4a16_packed_bytes(K, N, G)
    if packed is None:
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    if tuple(zeros.shape) != (K // G, N) or tuple(scales.shape) != (K // G, N):
        raise ValueError("zeros and scales must be [K/G][N]")
    _same_device(("q", q), ("zeros", zeros), ("scales", scales), ("packed", packed))
    if nbytes:
        _check_packed(packed, K, N, G)
    _check(lib().w4a16_pack(_dev_ptr(q, torch.uint8, "q"), _dev_ptr(zeros, torch.uint8, "zeros"),
                            _dev_ptr(scales, torch.float16, "scales"), K, N, G,
                            _dev_ptr(packed, torch.uint8, "packed"), _stream(stream, q.device)))
    return packed


def w4a16_quantize(W, G: int, stream=None):
    """Quantize fp16 W [K][N] (device tensor) group-wise to 4 bits: returns
    (q uint8 [K][N], zeros uint8 [K/G][N], scales fp16 [K/G][N]) device tensors.
    Synchronizes the stream."""
    import torch
    K, N = W.shape
    dev = W.device
    q = torch.empty((K, N), dtype=torch.uint8, device=dev)
    z = torch.empty((K // G, N), dtype=torch.uint8, device=dev)
    s = torch.empty((K // G, N), dtype=torch.float16, device=dev)
    _check(lib().w4a16_quantize(_dev_ptr(W, torch.float16, "W"), K, N, G, q.data_ptr(), z.data_ptr(),
                                s.data_ptr(), _stream(stream, dev)))
    return q, z, s


def w4a16_quantize_pack(W, G: int, packed=None, stream=None):
    """Quantize fp16 W [K][N] (device tensor) straight into the packed layout
    (a uint8 device tensor of w4a16_packed_bytes(K, N, G) bytes, the same
    bytes as w4a16_pack of w4a16_quantize's output). Synchronizes the stream."""
    import torch
    K, N = W.shape
    nbytes = w4a16_packed_bytes(K, N, G)
    if packed is None:
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=W.device)
    _same_device(("W", W), ("packed", packed))
    if nbytes:
        _check_packed(packed, K, N, G)
    _check(lib().w4a16_quantize_pack(_dev_ptr(W, torch.float16, "W"), K, N, G,
                                     _dev_ptr(packed, torch.uint8, "packed"), _stream(stream, W.device)))
    return packed


def w4a16_kv_block_bytes(bits: int, kv_heads: int) -> int:
    return int(lib().w4a16_kv_block_bytes(bits, kv_heads))


def w4a16_kv_append(k, v, slots, bits: int, cache, stream=None):
    """Quantize fp16 k, v [ntok][kv_heads][128] (device) into the cache
    (uint8 device tensor of whole blocks) at int32 `slots` [ntok]. Asynchronous."""
    import torch
    ntok, hkv, d = k.shape
    if d != 128 or tuple(v.shape) != tuple(k.shape) or slots.numel() != ntok:
        raise ValueError("k and v must be [ntok][kv_heads][128], slots [ntok]")
    nb = cache.numel() // max(w4a16_kv_block_bytes(bits, hkv), 1)
    _check(lib().w4a16_kv_append(_dev_ptr(k, torch.float16, "k"), _dev_ptr(v, torch.float16, "v"),
                                 _dev_ptr(slots, torch.int32, "slots"), ntok, hkv, bits,
                                 _dev_ptr(cache, torch.uint8, "cache"), nb, _stream(stream, k.device)))


def w4a16_kv_attention_workspace_bytes(B: int, kv_heads: int, max_blocks: int) -> int:
    return int(lib().w4a16_kv_attention_workspace_bytes(B, kv_heads, max_blocks))


def w4a16_kv_attention(q, cache, block_table, lengths, bits: int, kv_heads: int, sm_scale: float,
                       out=None, workspace=None, stream=None):
    """fp16 out [B][q_heads][128] = softmax(sm_scale q K^T) V over each
    sequence's cached tokens. Asynchronous."""
    import torch
    B, hq, d = q.shape
    max_blocks = block_table.shape[1]
    if d != 128 or tuple(block_table.shape) != (B, max_blocks) or lengths.numel() != B:
        raise ValueError("q must be [B][q_heads][128], block_table [B][max_blocks], lengths [B]")
    if out is None:
        out = torch.empty_like(q)
    need = w4a16_kv_attention_workspace_bytes(B, kv_heads, max_blocks)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    nb = cache.numel() // max(w4a16_kv_block_bytes(bits, kv_heads), 1)
    _check(lib().w4a16_kv_attention(_dev_ptr(q, torch.float16, "q"), _dev_ptr(cache, torch.uint8, "cache"), nb,
                                    _dev_ptr(block_table, torch.int32, "block_table"), max_blocks,
                                    _dev_ptr(lengths, torch.int32, "lengths"), B, hq, kv_heads, bits,
                                    float(sm_scale), _dev_ptr(out, torch.float16, "out"),
                                    _dev_ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                    _stream(stream, q.device)))
    return out


def w4a16_w8a8_packed_bytes(K: int, N: int) -> int:
    return int(lib().w4a16_w8a8_packed_bytes(K, N))


def w4a16_w8a8_quantize_weights(W, stream=None):
    """fp16 W [K][N] (device) -> (packed uint8 [K*N], w_scales float32 [N]). Asynchronous."""
    import torch
    K, N = W.shape
    packed = torch.empty(max(w4a16_w8a8_packed_bytes(K, N), 1), dtype=torch.uint8, device=W.device)
    ws = torch.empty(N, dtype=torch.float32, device=W.device)
    _check(lib().w4a16_w8a8_quantize_weights(_dev_ptr(W, torch.float16, "W"), K, N, packed.data_ptr(),
                                             ws.data_ptr(), _stream(stream, W.device)))
    return packed, ws


def w4a16_w8a8_quantize_act(X, stream=None, xq=None, xs=None):
    """fp16 X [M][K] (device) -> (xq int8 [M][K], x_scales float32 [M]),
    into xq / xs when given. Asynchronous."""
    import torch
    M, K = X.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if xs is None:
        xs = torch.empty(M, dtype=torch.float32, device=X.device)
    if tuple(xq.shape) != (M, K) or xs.numel() < M:
        raise ValueError("xq must be [M][K] and xs hold M floats")
    _check(lib().w4a16_w8a8_quantize_act(_dev_ptr(X, torch.float16, "X"), M, K, xq.data_ptr(), xs.data_ptr(),
                                         _stream(stream, X.device)))
    return xq, xs


def w4a16_w8a8_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().w4a16_w8a8_workspace_bytes(M, N, K))


def w4a16_w8a8_gemm(xq, x_scales, packed, w_scales, N: int, Y=None, workspace=None, stream=None):
    """Y fp16 [M][N] from int8 activation codes and packed int8 weights. Asynchronous."""
    import torch
    M, K = xq.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=xq.device)
    need = w4a16_w8a8_workspace_bytes(M, N, K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=xq.device)
    wptr = _dev_ptr(workspace, None, "workspace") if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().w4a16_w8a8_gemm(_dev_ptr(xq, torch.int8, "xq"), _dev_ptr(x_scales, torch.float32, "x_scales"),
                                 _dev_ptr(packed, torch.uint8, "packed"), _dev_ptr(w_scales, torch.float32, "w_scales"),
                                 M, N, K, _dev_ptr(Y, torch.float16, "Y"), wptr, wbytes, _stream(stream, xq.device)))
    return Y


def w4a16_unpack(packed, K: int, N: int, G: int, stream=None):
    """Inverse of w4a16_pack: (q, zeros, scales) device tensors."""
    import torch
    dev = packed.device
    if w4a16_packed_bytes(K, N, G):
        _check_packed(packed, K, N, G)
    q = torch.empty((K, N), dtype=torch.uint8, device=dev)
    z = torch.empty((K // G, N), dtype=torch.uint8, device=dev)
    s = torch.empty((K // G, N), dtype=torch.float16, device=dev)
    _check(lib().w4a16_unpack(_dev_ptr(packed, torch.uint8, "packed"), K, N, G, q.data_ptr(),
                              z.data_ptr(), s.data_ptr(), _stream(stream, dev)))
    return q, z, s


def w4a16_gemm(X, packed, N: int, K: int, G: int, Y=None, stream=None):
    """Y[M][N] (fp16) = X[M][K] (fp16) . dequant(packed). Asynchronous."""
    import torch
    M = X.shape[0]
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [M][K]")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    elif tuple(Y.shape) != (M, N):
        raise ValueError("Y must be [M][N]")
    _same_device(("X", X), ("packed", packed), ("Y", Y))
    if w4a16_packed_bytes(K, N, G):
        _check_packed(packed, K, N, G)
    _check(lib().w4a16_gemm(_dev_ptr(X, torch.float16, "X"), _dev_ptr(packed, torch.uint8, "packed"),
                            M, N, K, G, _dev_ptr(Y, torch.float16, "Y"), _stream(stream, X.device)))
    return Y


def w4a16_gemm_ex(X, packed, N: int, K: int, G: int, Y=None, workspace=None,
                  path: int = W4A16_PATH_AUTO, splits: int = 0, stream=None):
    """w4a16_gemm with an explicit plan and caller-owned workspace (a uint8
    device tensor of at least w4a16_workspace_bytes(...) bytes, any contents)."""
    import torch
    M = X.shape[0]
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [M][K]")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    elif tuple(Y.shape) != (M, N):
        raise ValueError("Y must be [M][N]")
    _same_device(("X", X), ("packed", packed), ("Y", Y), ("workspace", workspace))
    if w4a16_packed_bytes(K, N, G):
        _check_packed(packed, K, N, G)
    ws_ptr = _dev_ptr(workspace, torch.uint8, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(lib().w4a16_gemm_ex(_dev_ptr(X, torch.float16, "X"), _dev_ptr(packed, torch.uint8, "packed"),
                               M, N, K, G, _dev_ptr(Y, torch.float16, "Y"), ws_ptr, ws_bytes,
                               path, splits, _stream(stream, X.device)))
    return Y


def w4a16_gemm_noalloc(X, packed, N: int, K: int, G: int, Y, stream=None):
    """w4a16_gemm whose split-K partials use the library's fixed per-GPU
    scratch: the call allocates nothing (Y, the output, is the caller's).
    Calls that overlap on one GPU share that scratch and must be ordered."""
    import torch
    M = X.shape[0]
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [M][K]")
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y must be [M][N]")
    _same_device(("X", X), ("packed", packed), ("Y", Y))
    if w4a16_packed_bytes(K, N, G):
        _check_packed(packed, K, N, G)
    _check(lib().w4a16_gemm_noalloc(_dev_ptr(X, torch.float16, "X"), _dev_ptr(packed, torch.uint8, "packed"),
                                    M, N, K, G, _dev_ptr(Y, torch.float16, "Y"), _stream(stream, X.device)))
    return Y


def w4a16_stream_read(buf, sink, nbytes=None, never: int = 0x9E3779B9, stream=None):
    """Read `nbytes` (default: all) bytes of the device tensor `buf` in one
    launch and nothing else (the achievable-bandwidth yardstick); `sink` is a
    device tensor of at least 64 uint32 (written only if the data fold to
    `never`). Asynchronous."""
    import torch
    have = buf.numel() * buf.element_size()
    n = have if nbytes is None else int(nbytes)
    if n > have:
        raise ValueError(f"buf holds {have} bytes, asked to read {n}")
    if sink.numel() * sink.element_size() < 256:
        raise ValueError("sink must hold 64 uint32")
    _same_device(("buf", buf), ("sink", sink))
    _check(lib().w4a16_stream_read(_dev_ptr(buf, None, "buf"), n, never & 0xFFFFFFFF,
                                   _dev_ptr(sink, None, "sink"), _stream(stream, buf.device)))
