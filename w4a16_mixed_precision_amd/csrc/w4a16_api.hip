// C ABI of the W4A16 library: argument validation, plan selection and the
// per-device state (a small status word for pack and the quantizer, the lazily grown split-K
// workspace of w4a16_gemm). The declarations and their contract are in
// include/w4a16.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/w4a16.h"
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

int fail_hip(hipError_t e, const char *what) {
    return fail(W4A16_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // M
constexpr int64_t kMaxKN = (int64_t)1 << 22;   // K and N (32-bit buffer offsets)
// The prefill kernel reaches the whole packed weight region through one
// buffer descriptor with a 32-bit byte count and 32-bit tile offsets, so the
// 4-bit weights must stay below 2^31 bytes.
constexpr int64_t kMaxWeightBytes = (int64_t)1 << 31;

bool shape_ok(int64_t K, int64_t N, int64_t G) {
    if (K <= 0 || N <= 0 || K > kMaxKN || N > kMaxKN) return false;
    if (K * N / 2 >= kMaxWeightBytes) return false;
    if (K % 128 != 0 || N % 16 != 0) return false;
    if (G != 32 && G != 64 && G != 128 && G != 256) return false;
    return K % G == 0;
}

int check_shape(int64_t K, int64_t N, int64_t G) {
    if (!shape_ok(K, N, G))
        return fail(W4A16_ERR_SHAPE,
                    "unsupported shape K=%lld N=%lld G=%lld (need K%%128==0, N%%16==0, "
                    "G in {32,64,128,256}, K%%G==0, K and N <= 2^22, K*N/2 < 2^31)",
                    (long long)K, (long long)N, (long long)G);
    return W4A16_OK;
}

// ------------------------------------------------------------- device state
constexpr int kMaxDevices = 64;

struct DeviceState {
    std::mutex mu;
    int num_cus = 0;
    int *flag = nullptr;       // pack range / quantizer finiteness error word (pinned host memory)
    void *ws = nullptr;        // w4a16_gemm split-K workspace
    size_t ws_bytes = 0;
    // Workspaces outgrown by a larger plan. They are never freed: work
    // already enqueued (or captured into a graph) may still use them.
    std::vector<void *> retired;
    void *scratch = nullptr;   // this device's address of `scratch` (w4a16_gemm_noalloc)
};

DeviceState g_dev[kMaxDevices];

int current_device(int *dev) {
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    if (*dev < 0 || *dev >= kMaxDevices) return fail(W4A16_ERR_HIP, "device index %d out of range", *dev);
    return W4A16_OK;
}

int device_cus(int dev, int *cus) {
    DeviceState &d = g_dev[dev];
    std::lock_guard<std::mutex> lk(d.mu);
    if (d.num_cus == 0) {
        int v = 0;
        hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute");
        d.num_cus = v > 0 ? v : 1;
    }
    *cus = d.num_cus;
    return W4A16_OK;
}

// The status word of the synchronous offline calls (pack, quantize) lives in
// pinned, device-mapped host memory: the host clears it before the launch and
// reads it after the stream synchronization, so a call costs no fill kernel
// and no device-to-host copy. Kernels only ever store 1 into it.
int device_flag(int dev, int **flag) {
    DeviceState &d = g_dev[dev];
    std::lock_guard<std::mutex> lk(d.mu);
    if (!d.flag) {
        hipError_t e = hipHostMalloc((void **)&d.flag, 256, hipHostMallocMapped | hipHostMallocCoherent);
        if (e != hipSuccess) return fail_hip(e, "hipHostMalloc(status word)");
    }
    *flag = d.flag;
    return W4A16_OK;
}

// Clears the status word, runs `launch_fn(flag)` on `st`, synchronizes `st`
// and reports whether a kernel set the word.
template <class Launch>
int run_flagged(hipStream_t st, const char *what, Launch &&launch_fn, bool *raised) {
    int dev, rc;
    if ((rc = current_device(&dev))) return rc;
    int *flag;
    if ((rc = device_flag(dev, &flag))) return rc;
    *(volatile int *)flag = 0;
    hipError_t e = launch_fn(flag);
    if (e != hipSuccess) return fail_hip(e, what);
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
    *raised = *(volatile int *)flag != 0;
    return W4A16_OK;
}

// Grows the per-device split-K workspace to at least `bytes`. A buffer that a
// larger plan outgrows is retired, not freed, so that work already enqueued
// or captured into a HIP graph keeps valid memory; growing is refused while
// `stream` is being captured (a capture must not allocate).
int device_workspace(int dev, size_t bytes, void **ws, hipStream_t stream) {
    DeviceState &d = g_dev[dev];
    std::lock_guard<std::mutex> lk(d.mu);
    if (d.ws_bytes < bytes) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t ce = hipStreamIsCapturing(stream, &cs);
        if (ce != hipSuccess) return fail_hip(ce, "hipStreamIsCapturing");
        if (cs != hipStreamCaptureStatusNone)
            return fail(W4A16_ERR_WORKSPACE,
                        "w4a16_gemm needs a larger library workspace (%zu bytes) during stream capture; "
                        "run the shape once before capturing, or use w4a16_gemm_ex with a caller workspace",
                        bytes);
        if (d.ws) d.retired.push_back(d.ws);
        d.ws = nullptr;
        d.ws_bytes = 0;
        size_t want = bytes < ((size_t)1 << 20) ? ((size_t)1 << 20) : bytes;
        hipError_t e = hipMalloc(&d.ws, want);
        if (e != hipSuccess) return fail_hip(e, "hipMalloc(workspace)");
        d.ws_bytes = want;
    }
    *ws = d.ws;
    return W4A16_OK;
}

// ------------------------------------------------------------- fixed scratch
// Split-K partials of w4a16_gemm_noalloc: a fixed array in the library's code
// object, one copy on every GPU the library runs on, held until the process
// ends. In host code the name `scratch` is only a stand-in for the symbol:
// kernels get this device's address of it, looked up once per device by
// hipGetSymbolAddress with that device current, and every use in host code
// goes through that address.
static __device__ __align__(256) uint8_t scratch[W4A16_NOALLOC_SCRATCH_BYTES];

int device_scratch(int dev, void **ptr) {
    DeviceState &d = g_dev[dev];
    std::lock_guard<std::mutex> lk(d.mu);
    if (!d.scratch) {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(W4A16_ERR_HIP, "hipGetSymbolAddress(scratch) returned no address");
        d.scratch = p;
    }
    *ptr = d.scratch;
    return W4A16_OK;
}

// ------------------------------------------------------------- planning
struct Plan {
    int path;
    int splits;
};

// Decode up to 32 rows; up to 64 on narrow matrices (graph-timed on MI355X:
// at M = 64 the decode ring took 12.2 / 21.8 us against 23.2 / 26.8 us for
// the tiled kernel on the Llama-3-8B QKV and down projections, but 129 / 72
// against 100 / 53 us on the Llama-3-70B gate/up and down projections).
int auto_path(int64_t M, int64_t N) {
    return (M <= 32 || (M <= 64 && N <= 6144)) ? W4A16_PATH_DECODE : W4A16_PATH_PREFILL;
}

int make_plan(int64_t M, int64_t N, int64_t K, int64_t G, int path, int splits, int num_cus, Plan *p) {
    if (path != W4A16_PATH_AUTO && path != W4A16_PATH_DECODE && path != W4A16_PATH_PREFILL)
        return fail(W4A16_ERR_ARG, "path %d is not one of W4A16_PATH_*", path);
    if (path == W4A16_PATH_AUTO) path = auto_path(M, N);
    if (path == W4A16_PATH_DECODE && M > w4a16::kDecodeMaxM)
        return fail(W4A16_ERR_ARG, "decode path needs M <= %d (M=%lld)", w4a16::kDecodeMaxM, (long long)M);
    const int maxs = (int)(K / 128);
    if (splits < 0 || splits > maxs) return fail(W4A16_ERR_ARG, "splits=%d outside 0..%d", splits, maxs);
    if (splits == 0)
        splits = path == W4A16_PATH_DECODE
                     ? w4a16::decode_auto_splits((int)M, (int)N, (int)K, (int)G, num_cus)
                     : w4a16::prefill_auto_splits((int)M, (int)N, (int)K, (int)G, num_cus);
    p->path = path;
    p->splits = splits;
    return W4A16_OK;
}

size_t plan_workspace(const Plan &p, int64_t M, int64_t N, int64_t K, int64_t G, int num_cus) {
    if (p.path == W4A16_PATH_DECODE)
        return w4a16::decode_workspace_bytes((int)M, (int)N, (int)K, (int)G, p.splits, num_cus);
    return w4a16::prefill_workspace_bytes((int)M, (int)N, (int)K, (int)G, p.splits);
}

int check_gemm_args(const uint16_t *X, const void *packed, int64_t M, int64_t N, int64_t K,
                    int64_t G, uint16_t *Y) {
    if (!X || !packed || !Y) return fail(W4A16_ERR_NULL, "X, packed and Y must be non-NULL");
    if (M < 1 || M > kMaxDim) return fail(W4A16_ERR_SHAPE, "M=%lld out of range", (long long)M);
    int rc = check_shape(K, N, G);
    if (rc) return rc;
    if (!aligned16(X) || !aligned16(packed) || !aligned16(Y))
        return fail(W4A16_ERR_ALIGN, "X, packed and Y must be 16-byte aligned");
    return W4A16_OK;
}

int launch(const uint16_t *X, const void *packed, int64_t M, int64_t N, int64_t K, int64_t G,
           uint16_t *Y, void *ws, const Plan &p, int num_cus, hipStream_t stream) {
    hipError_t e;
    if (p.path == W4A16_PATH_DECODE)
        e = w4a16::launch_decode(X, (const uint8_t *)packed, (int)M, (int)N, (int)K, (int)G, Y, ws,
                                 p.splits, num_cus, stream);
    else
        e = w4a16::launch_prefill(X, (const uint8_t *)packed, (int)M, (int)N, (int)K, (int)G, Y, ws,
                                  p.splits, num_cus, stream);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    g_last_error[0] = 0;
    return W4A16_OK;
}

// One quantizer launch with the finiteness status word; synchronizes `st`.
template <class Launch>
int run_quantizer(hipStream_t st, Launch &&launch_fn) {
    bool raised = false;
    int rc = run_flagged(st, "quantize launch", launch_fn, &raised);
    if (rc) return rc;
    if (raised)
        return fail(W4A16_ERR_RANGE,
                    "a weight is not finite (Inf or NaN), or a group's codes dequantize beyond the fp16 range "
                    "(|(q - z) * s| >= 65520)");
    g_last_error[0] = 0;
    return W4A16_OK;
}

}  // namespace

extern "C" {

size_t w4a16_packed_bytes(int64_t K, int64_t N, int64_t G) {
    if (!shape_ok(K, N, G)) return 0;
    return w4a16::weight_bytes(K, N) + w4a16::scale_bytes(K, N, G) + w4a16::zero_bytes(K, N, G);
}

int w4a16_pack(const uint8_t *q, const uint8_t *zeros, const uint16_t *scales, int64_t K, int64_t N,
               int64_t G, void *packed, void *stream) {
    if (!q || !zeros || !scales || !packed)
        return fail(W4A16_ERR_NULL, "q, zeros, scales and packed must be non-NULL");
    int rc = check_shape(K, N, G);
    if (rc) return rc;
    if (!aligned16(packed)) return fail(W4A16_ERR_ALIGN, "packed must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    bool host_flag = false;
    rc = run_flagged(st, "pack launch", [&](int *flag) {
        return w4a16::launch_pack(q, zeros, scales, (int)K, (int)N, (int)G, (uint8_t *)packed, flag, st);
    }, &host_flag);
    if (rc) return rc;
    if (host_flag)
        return fail(W4A16_ERR_RANGE,
                    "a q or zero code is larger than 15, or a dequantized weight (q - z) * s is not a finite "
                    "fp16 value (non-finite scale, or |(q - z) * s| >= 65520)");
    g_last_error[0] = 0;
    return W4A16_OK;
}

int w4a16_quantize(const uint16_t *W, int64_t K, int64_t N, int64_t G, uint8_t *q, uint8_t *zeros,
                   uint16_t *scales, void *stream) {
    if (!W || !q || !zeros || !scales)
        return fail(W4A16_ERR_NULL, "W, q, zeros and scales must be non-NULL");
    int rc = check_shape(K, N, G);
    if (rc) return rc;
    if (!aligned16(W) || !aligned16(q) || !aligned16(zeros) || !aligned16(scales))
        return fail(W4A16_ERR_ALIGN, "W, q, zeros and scales must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    return run_quantizer(st, [&](int *flag) {
        return w4a16::launch_quantize(W, (int)K, (int)N, (int)G, q, zeros, scales, flag, st);
    });
}

int w4a16_quantize_pack(const uint16_t *W, int64_t K, int64_t N, int64_t G, void *packed, void *stream) {
    if (!W || !packed) return fail(W4A16_ERR_NULL, "W and packed must be non-NULL");
    int rc = check_shape(K, N, G);
    if (rc) return rc;
    if (!aligned16(W) || !aligned16(packed)) return fail(W4A16_ERR_ALIGN, "W and packed must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    return run_quantizer(st, [&](int *flag) {
        return w4a16::launch_quantize_pack(W, (int)K, (int)N, (int)G, (uint8_t *)packed, flag, st);
    });
}

int w4a16_unpack(const void *packed, int64_t K, int64_t N, int64_t G, uint8_t *q, uint8_t *zeros,
                 uint16_t *scales, void *stream) {
    if (!q || !zeros || !scales || !packed)
        return fail(W4A16_ERR_NULL, "packed, q, zeros and scales must be non-NULL");
    int rc = check_shape(K, N, G);
    if (rc) return rc;
    if (!aligned16(packed)) return fail(W4A16_ERR_ALIGN, "packed must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = w4a16::launch_unpack((const uint8_t *)packed, (int)K, (int)N, (int)G, q, zeros,
                                        scales, st);
    if (e != hipSuccess) return fail_hip(e, "unpack launch");
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
    g_last_error[0] = 0;
    return W4A16_OK;
}

size_t w4a16_kv_block_bytes(int bits, int64_t kv_heads) {
    if ((bits != 4 && bits != 8) || kv_heads < 1 || kv_heads > 65535) return 0;
    return (size_t)kv_heads * w4a16::kv_region_bytes(bits);
}

int w4a16_kv_append(const uint16_t *k, const uint16_t *v, const int32_t *slots, int64_t ntok, int64_t kv_heads,
                    int bits, void *cache, int64_t num_blocks, void *stream) {
    if (!k || !v || !slots || !cache) return fail(W4A16_ERR_NULL, "k, v, slots and cache must be non-NULL");
    if (bits != 4 && bits != 8) return fail(W4A16_ERR_ARG, "bits must be 4 or 8 (got %d)", bits);
    if (ntok < 0 || ntok > kMaxDim || kv_heads < 1 || kv_heads > 65535 || num_blocks < 1)
        return fail(W4A16_ERR_SHAPE, "bad KV append shape ntok=%lld kv_heads=%lld num_blocks=%lld", (long long)ntok,
                    (long long)kv_heads, (long long)num_blocks);
    if (!aligned16(k) || !aligned16(v) || !aligned16(slots) || !aligned16(cache))
        return fail(W4A16_ERR_ALIGN, "k, v, slots and cache must be 16-byte aligned");
    int dev = 0, cus = 0, rc;
    if ((rc = current_device(&dev)) || (rc = device_cus(dev, &cus))) return rc;
    hipError_t e = w4a16::launch_kv_append(k, v, slots, (int)ntok, (int)kv_heads, bits, num_blocks, (uint8_t *)cache,
                                           cus, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "KV append launch");
    g_last_error[0] = 0;
    return W4A16_OK;
}

size_t w4a16_kv_attention_workspace_bytes(int64_t B, int64_t kv_heads, int64_t max_blocks) {
    if (B < 1 || B > kMaxDim || kv_heads < 1 || kv_heads > 65535 || max_blocks < 1 || max_blocks > (1 << 24) ||
        B * kv_heads > (1 << 26))
        return 0;
    int cus = 256, dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
        int v = 0;
        if (device_cus(dev, &v) == W4A16_OK) cus = v;
    }
    return w4a16::kv_workspace_bytes((int)B, (int)kv_heads, (int)max_blocks, cus);
}

int w4a16_kv_attention(const uint16_t *q, const void *cache, int64_t num_blocks, const int32_t *block_table,
                       int64_t max_blocks, const int32_t *lengths, int64_t B, int64_t q_heads, int64_t kv_heads,
                       int bits, float sm_scale, uint16_t *out, void *workspace, size_t workspace_bytes,
                       void *stream) {
    if (!q || !cache || !block_table || !lengths || !out)
        return fail(W4A16_ERR_NULL, "q, cache, block_table, lengths and out must be non-NULL");
    if (bits != 4 && bits != 8) return fail(W4A16_ERR_ARG, "bits must be 4 or 8 (got %d)", bits);
    // (max_blocks * 64 and the per-(sequence, KV head) work count stay in int)
    if (B < 1 || B > kMaxDim || kv_heads < 1 || kv_heads > 65535 || q_heads < kv_heads ||
        q_heads % kv_heads != 0 || q_heads / kv_heads > 16 || max_blocks < 1 || max_blocks > (1 << 24) ||
        num_blocks < 1 || B * q_heads > kMaxDim || B * kv_heads > (1 << 26))
        return fail(W4A16_ERR_SHAPE,
                    "bad KV attention shape B=%lld q_heads=%lld kv_heads=%lld max_blocks=%lld num_blocks=%lld "
                    "(need q_heads a multiple of kv_heads, at most 16 query heads per KV head)",
                    (long long)B, (long long)q_heads, (long long)kv_heads, (long long)max_blocks,
                    (long long)num_blocks);
    if (!aligned16(q) || !aligned16(cache) || !aligned16(out) || !aligned16(block_table) || !aligned16(lengths))
        return fail(W4A16_ERR_ALIGN, "q, cache, block_table, lengths and out must be 16-byte aligned");
    int dev, rc, cus;
    if ((rc = current_device(&dev))) return rc;
    if ((rc = device_cus(dev, &cus))) return rc;
    const size_t need = w4a16::kv_workspace_bytes((int)B, (int)kv_heads, (int)max_blocks, cus);
    if (!workspace || workspace_bytes < need)
        return fail(W4A16_ERR_WORKSPACE, "KV attention needs a workspace of %zu bytes (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(W4A16_ERR_ALIGN, "workspace must be 16-byte aligned");
    hipError_t e = w4a16::launch_kv_attention(q, (const uint8_t *)cache, block_table, (int)max_blocks, lengths,
                                              (int)B, (int)q_heads, (int)kv_heads, bits, num_blocks, sm_scale, out,
                                              workspace, cus, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "KV attention launch");
    g_last_error[0] = 0;
    return W4A16_OK;
}

// ------------------------------------------------------------- W8A8
static bool w8a8_shape_ok(int64_t K, int64_t N) {
    return K > 0 && N > 0 && K % 256 == 0 && N % 16 == 0 && K <= (1 << 17) && N <= kMaxKN &&
           K * N <= (int64_t)0xFFFFFFFF;
}

static int w8a8_check_shape(int64_t K, int64_t N) {
    if (!w8a8_shape_ok(K, N))
        return fail(W4A16_ERR_SHAPE,
                    "unsupported W8A8 shape K=%lld N=%lld (need K %% 256 == 0, K <= 131072, N %% 16 == 0, "
                    "K * N < 2^32)",
                    (long long)K, (long long)N);
    return W4A16_OK;
}

size_t w4a16_w8a8_packed_bytes(int64_t K, int64_t N) { return w8a8_shape_ok(K, N) ? (size_t)(K * N) : 0; }

int w4a16_w8a8_quantize_weights(const uint16_t *W, int64_t K, int64_t N, void *packed, float *w_scales,
                                void *stream) {
    if (!W || !packed || !w_scales) return fail(W4A16_ERR_NULL, "W, packed and w_scales must be non-NULL");
    int rc = w8a8_check_shape(K, N);
    if (rc) return rc;
    if (!aligned16(W) || !aligned16(packed) || !aligned16(w_scales))
        return fail(W4A16_ERR_ALIGN, "W, packed and w_scales must be 16-byte aligned");
    hipError_t e = w4a16::launch_w8a8_quant_weights(W, (int)K, (int)N, (uint8_t *)packed, w_scales,
                                                    (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "W8A8 weight quantization launch");
    g_last_error[0] = 0;
    return W4A16_OK;
}

int w4a16_w8a8_quantize_act(const uint16_t *X, int64_t M, int64_t K, int8_t *xq, float *x_scales, void *stream) {
    if (!X || !xq || !x_scales) return fail(W4A16_ERR_NULL, "X, xq and x_scales must be non-NULL");
    if (M < 1 || M > kMaxDim) return fail(W4A16_ERR_SHAPE, "M=%lld out of range", (long long)M);
    int rc = w8a8_check_shape(K, 16);
    if (rc) return rc;
    if (!aligned16(X) || !aligned16(xq) || !aligned16(x_scales))
        return fail(W4A16_ERR_ALIGN, "X, xq and x_scales must be 16-byte aligned");
    hipError_t e = w4a16::launch_w8a8_quant_act(X, (int)M, (int)K, xq, x_scales, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "W8A8 activation quantization launch");
    g_last_error[0] = 0;
    return W4A16_OK;
}

size_t w4a16_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || M > kMaxDim || !w8a8_shape_ok(K, N)) return 0;
    int cus = 256, dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
        int v = 0;
        if (device_cus(dev, &v) == W4A16_OK) cus = v;
    }
    return w4a16::w8a8_workspace_bytes((int)M, (int)N, (int)K, cus);
}

int w4a16_w8a8_gemm(const int8_t *xq, const float *x_scales, const void *packed, const float *w_scales, int64_t M,
                    int64_t N, int64_t K, uint16_t *Y, void *workspace, size_t workspace_bytes, void *stream) {
    if (!xq || !x_scales || !packed || !w_scales || !Y)
        return fail(W4A16_ERR_NULL, "xq, x_scales, packed, w_scales and Y must be non-NULL");
    if (M < 1 || M > kMaxDim) return fail(W4A16_ERR_SHAPE, "M=%lld out of range", (long long)M);
    int rc = w8a8_check_shape(K, N);
    if (rc) return rc;
    if (!aligned16(xq) || !aligned16(packed) || !aligned16(Y) || !aligned16(x_scales) || !aligned16(w_scales))
        return fail(W4A16_ERR_ALIGN, "xq, x_scales, packed, w_scales and Y must be 16-byte aligned");
    int dev, cus;
    if ((rc = current_device(&dev))) return rc;
    if ((rc = device_cus(dev, &cus))) return rc;
    const size_t need = w4a16::w8a8_workspace_bytes((int)M, (int)N, (int)K, cus);
    if (need && (!workspace || workspace_bytes < need))
        return fail(W4A16_ERR_WORKSPACE, "W8A8 GEMM needs a workspace of %zu bytes (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    hipError_t e = w4a16::launch_w8a8_gemm(xq, x_scales, (const uint8_t *)packed, w_scales, (int)M, (int)N, (int)K,
                                           Y, workspace, cus, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "W8A8 GEMM launch");
    g_last_error[0] = 0;
    return W4A16_OK;
}

size_t w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G, int path, int splits) {
    if (M < 1 || M > kMaxDim || !shape_ok(K, N, G)) return 0;
    // The plan depends on the device's CU count; size for the current device
    // when one is available, else for 256 CUs.
    int cus = 256, dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
        int v = 0;
        if (device_cus(dev, &v) == W4A16_OK) cus = v;
    }
    Plan p;
    if (make_plan(M, N, K, G, path, splits, cus, &p) != W4A16_OK) return 0;
    return plan_workspace(p, M, N, K, G, cus);
}

int w4a16_gemm(const uint16_t *X, const void *packed, int64_t M, int64_t N, int64_t K, int64_t G,
               uint16_t *Y, void *stream) {
    int rc = check_gemm_args(X, packed, M, N, K, G, Y);
    if (rc) return rc;
    int dev, cus;
    if ((rc = current_device(&dev)) || (rc = device_cus(dev, &cus))) return rc;
    Plan p;
    if ((rc = make_plan(M, N, K, G, W4A16_PATH_AUTO, 0, cus, &p))) return rc;
    void *ws = nullptr;
    const size_t need = plan_workspace(p, M, N, K, G, cus);
    if (need && (rc = device_workspace(dev, need, &ws, (hipStream_t)stream))) return rc;
    return launch(X, packed, M, N, K, G, Y, ws, p, cus, (hipStream_t)stream);
}

int w4a16_gemm_noalloc(const uint16_t *X, const void *packed, int64_t M, int64_t N, int64_t K, int64_t G,
                       uint16_t *Y, void *stream) {
    int rc = check_gemm_args(X, packed, M, N, K, G, Y);
    if (rc) return rc;
    int dev, cus;
    if ((rc = current_device(&dev)) || (rc = device_cus(dev, &cus))) return rc;
    Plan p;
    if ((rc = make_plan(M, N, K, G, W4A16_PATH_AUTO, 0, cus, &p))) return rc;
    const size_t need = plan_workspace(p, M, N, K, G, cus);
    if (need > (size_t)W4A16_NOALLOC_SCRATCH_BYTES)
        return fail(W4A16_ERR_WORKSPACE,
                    "the plan for M=%lld N=%lld K=%lld G=%lld needs %zu bytes of split-K partials; the fixed "
                    "scratch of w4a16_gemm_noalloc holds %zu (use w4a16_gemm_ex with a caller workspace)",
                    (long long)M, (long long)N, (long long)K, (long long)G, need,
                    (size_t)W4A16_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need && (rc = device_scratch(dev, &ws))) return rc;
    return launch(X, packed, M, N, K, G, Y, ws, p, cus, (hipStream_t)stream);
}

int w4a16_gemm_ex(const uint16_t *X, const void *packed, int64_t M, int64_t N, int64_t K, int64_t G,
                  uint16_t *Y, void *workspace, size_t workspace_bytes, int path, int splits,
                  void *stream) {
    int rc = check_gemm_args(X, packed, M, N, K, G, Y);
    if (rc) return rc;
    // Plan and workspace checks first: they need no device.
    Plan p;
    if (splits != 0) {
        if ((rc = make_plan(M, N, K, G, path, splits, 256, &p))) return rc;
        const size_t need = plan_workspace(p, M, N, K, G, 256);
        if (need && (!workspace || workspace_bytes < need))
            return fail(W4A16_ERR_WORKSPACE, "plan needs %zu workspace bytes, got %zu", need,
                        workspace ? workspace_bytes : (size_t)0);
    }
    int dev, cus;
    if ((rc = current_device(&dev)) || (rc = device_cus(dev, &cus))) return rc;
    if ((rc = make_plan(M, N, K, G, path, splits, cus, &p))) return rc;
    const size_t need = plan_workspace(p, M, N, K, G, cus);
    if (need && (!workspace || workspace_bytes < need))
        return fail(W4A16_ERR_WORKSPACE, "plan needs %zu workspace bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (need && !aligned16(workspace)) return fail(W4A16_ERR_ALIGN, "workspace must be 16-byte aligned");
    return launch(X, packed, M, N, K, G, Y, workspace, p, cus, (hipStream_t)stream);
}

int w4a16_stream_read(const void *buf, size_t bytes, uint32_t never, uint32_t *sink, void *stream) {
    if (!buf || !sink) return fail(W4A16_ERR_NULL, "buf and sink must be non-NULL");
    if (bytes == 0 || bytes >= ((size_t)1 << 31))
        return fail(W4A16_ERR_SHAPE, "stream read needs 0 < bytes < 2^31 (got %zu)", bytes);
    if (!aligned16(buf) || !aligned16(sink)) return fail(W4A16_ERR_ALIGN, "buf and sink must be 16-byte aligned");
    hipError_t e = w4a16::launch_stream_read((const uint8_t *)buf, bytes, never, sink, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "stream read launch");
    g_last_error[0] = 0;
    return W4A16_OK;
}

const char *w4a16_status_string(int status) {
    switch (status) {
        case W4A16_OK: return "ok";
        case W4A16_ERR_NULL: return "null pointer";
        case W4A16_ERR_SHAPE: return "unsupported shape";
        case W4A16_ERR_ALIGN: return "misaligned pointer";
        case W4A16_ERR_RANGE: return "code out of range";
        case W4A16_ERR_HIP: return "HIP runtime error";
        case W4A16_ERR_WORKSPACE: return "workspace too small";
        case W4A16_ERR_ARG: return "invalid argument";
        default: return "unknown status";
    }
}

const char *w4a16_last_error(void) { return g_last_error; }

int w4a16_layout_version(void) { return W4A16_LAYOUT_VERSION; }

int w4a16_auto_path(int64_t M, int64_t N, int64_t K, int64_t G) {
    if (M < 1 || M > kMaxDim) return fail(W4A16_ERR_SHAPE, "M=%lld out of range", (long long)M);
    const int rc = check_shape(K, N, G);
    if (rc) return rc;
    return auto_path(M, N);
}

}  // extern "C"
