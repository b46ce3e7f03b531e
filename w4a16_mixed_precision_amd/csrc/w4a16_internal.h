// Host-side interfaces between the C ABI layer and the kernel launchers.
// Internal header: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

// Offline relayout (pack) and its inverse (unpack). `bad` is a
// device-visible int (pinned host memory) that pack sets to 1 when a code is
// larger than 15 or a dequantized weight (q - z) * s is not a finite fp16.
hipError_t launch_pack(const uint8_t *q, const uint8_t *z, const uint16_t *s, int K, int N, int G,
                       uint8_t *packed, int *bad, hipStream_t stream);
hipError_t launch_unpack(const uint8_t *packed, int K, int N, int G, uint8_t *q, uint8_t *z,
                         uint16_t *s, hipStream_t stream);

// Group-wise 4-bit quantizer: fp16 W[K][N] -> plain (q, z, s) arrays, or
// straight into the packed layout. `bad` (as for pack) is set to 1 when a
// weight is not finite.
hipError_t launch_quantize(const uint16_t *W, int K, int N, int G, uint8_t *q, uint8_t *z, uint16_t *s,
                           int *bad, hipStream_t stream);
hipError_t launch_quantize_pack(const uint16_t *W, int K, int N, int G, uint8_t *packed, int *bad,
                                hipStream_t stream);

// Low-bit KV cache (8 or 4 bits, blocks of 64 tokens, head dimension 128)
// and decode attention over it.
size_t kv_region_bytes(int bits);  // one (block, KV head) region
struct KvPlan {
    int chunk_blocks, nchunks;
};
KvPlan kv_plan(int B, int Hkv, int max_blocks, int num_cus, int bits);
size_t kv_workspace_bytes(int B, int Hkv, int max_blocks, int num_cus);
hipError_t launch_kv_append(const uint16_t *k, const uint16_t *v, const int32_t *slots, int ntok, int Hkv, int bits,
                            int64_t num_blocks, uint8_t *cache, int num_cus, hipStream_t stream);
hipError_t launch_kv_attention(const uint16_t *q, const uint8_t *cache, const int32_t *block_table, int max_blocks,
                               const int32_t *lengths, int B, int Hq, int Hkv, int bits, int64_t num_blocks,
                               float sm_scale, uint16_t *out, void *workspace, int num_cus, hipStream_t stream);

// W8A8 GEMM: int8 codes (symmetric, per token / per output channel) on the
// int8 matrix cores.
size_t w8a8_workspace_bytes(int M, int N, int K, int num_cus);
hipError_t launch_w8a8_quant_act(const uint16_t *X, int M, int K, int8_t *xq, float *xs, hipStream_t stream);
hipError_t launch_w8a8_quant_weights(const uint16_t *W, int K, int N, uint8_t *packed, float *ws, hipStream_t stream);
hipError_t launch_w8a8_gemm(const int8_t *xq, const float *xs, const uint8_t *packed, const float *ws, int M, int N,
                            int K, uint16_t *Y, void *workspace, int num_cus, hipStream_t stream);

// Decode path (M <= 64): one 16-column strip per workgroup, waves split K,
// MFMA with M padded to 16; optional split of K across workgroups (narrow N)
// with fp32 partials in a workspace and a second reduce kernel.
constexpr int kDecodeMaxM = 64;
int decode_auto_splits(int M, int N, int K, int G, int num_cus);
int decode_max_splits(int M, int N, int K);
// (the plan, and so the workspace, can depend on the CU count of the device)
size_t decode_workspace_bytes(int M, int N, int K, int G, int splits, int num_cus);
hipError_t launch_decode(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G,
                         uint16_t *Y, void *workspace, int splits, int num_cus, hipStream_t stream);

// Prefill path (any M): LDS-staged activations, MFMA tiles, optional split
// of K across workgroups (fp32 partials + reduce kernel) for small grids.
int prefill_auto_splits(int M, int N, int K, int G, int num_cus);
size_t prefill_workspace_bytes(int M, int N, int K, int G, int splits);
hipError_t launch_prefill(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G,
                          uint16_t *Y, void *workspace, int splits, int num_cus, hipStream_t stream);

// Streaming read of `bytes` bytes of `buf` (measurement yardstick).
hipError_t launch_stream_read(const uint8_t *buf, size_t bytes, uint32_t never, uint32_t *sink, hipStream_t stream);

}  // namespace w4a16
