/*
 * w4a16.h -- W4A16 mixed-precision GEMM for AMD Instinct MI355X (gfx950).
 *
 *   Y[M][N] = X[M][K] . W[K][N],   W[k][n] = (q[k][n] - z[k/G][n]) * s[k/G][n]
 *
 * X and Y are fp16, q and z are unsigned 4-bit codes (0..15), s is fp16, and
 * all products are accumulated in fp32. The dequantization formula is the one
 * given in "LMDeploy Guide: Fast Mixed-Precision LLM Inference Engine",
 * section 3 "Instruction-Level Parallelism (ILP) for Zero-Overhead
 * Dequantization"; 4-bit weights in groups with one scale per group and
 * 16-bit activations are W4A16 as "LMDeploy, in depth" defines it (section
 * "Quantization: AWQ weights and KV cache"). Groups run along K: rows
 * [g*G, (g+1)*G) of column n share s[g][n] and z[g][n].
 *
 * The library has two parts, as the GEMM pipeline on those pages does
 * ("LMDeploy Accelerates Mixed-Precision LLM Inference with TurboMind",
 * abstract: offline weight packing plus online acceleration):
 *   - w4a16_pack: an offline, lossless relayout of (q, z, s) into one packed
 *     buffer laid out in the order the gfx950 matrix instructions consume it
 *     (w4a16_quantize produces (q, z, s) from fp16 weights;
 *     w4a16_quantize_pack does both in one pass);
 *   - w4a16_gemm: the online dequantize-and-multiply.
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers (memory from hipMalloc or
 *     torch), C-contiguous, row-major, and at least 16-byte aligned.
 *   - fp16 tensors are passed as uint16_t bit patterns.
 *   - The caller owns every buffer; the library keeps no pointer after a call
 *     returns (apart from its own internal workspace, see w4a16_gemm).
 *   - `stream` is a hipStream_t (0 = the null stream).
 *   - Every argument is validated on the host before any HIP call; on a
 *     validation error nothing is launched and outputs are untouched.
 *   - Return value: W4A16_OK (0) or a negative W4A16_ERR_* code;
 *     w4a16_last_error() gives a message for the calling thread.
 *   - Shapes: K % 128 == 0, N % 16 == 0, G in {32, 64, 128, 256} with
 *     K % G == 0, 1 <= M <= 2^30, K and N <= 2^22, and K * N / 2 < 2^31
 *     (the 4-bit weights of one matrix stay below 2 GiB). Anything else is
 *     W4A16_ERR_SHAPE.
 *
 * Packed layout, version 2 (bytes, little-endian):
 *   [0, K*N/2)            weights. Weight (k, n) lives in the 1024-byte tile
 *                         (n/16)*(K/128) + k/128, in the 32-bit word at byte
 *                         16*(16*((k%32)/8) + n%16) + 4*((k%8)/2) of the tile,
 *                         in nibble slot 4*(k%2) + 2*(t%2) + t/2 with step
 *                         t = (k%128)/32. One wave64 load of 16 bytes per
 *                         lane reads one whole tile; lane l then holds the
 *                         B-operand codes of column l%16, rows 8*(l/16)..+7,
 *                         of all four 32-row steps, and the masks 0x000F000F
 *                         and 0x00F000F0 on a word and on the word shifted
 *                         right by 8 give the (k, k+1) code pairs of steps
 *                         0, 2, 1 and 3 in the two 16-bit halves.
 *   next 2*N*(K/G)        fp16 scales, s[g][n] at element ((n/16)*(K/G)+g)*16 + n%16.
 *   next N*(K/G)/2        4-bit zeros, z[g][n] in byte ((n/16)*(K/G)+g)*8 + (n%16)/2,
 *                         low nibble for even n, high nibble for odd n.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_LAYOUT_VERSION 2

#define W4A16_OK 0
#define W4A16_ERR_NULL (-1)      /* a required pointer is NULL */
#define W4A16_ERR_SHAPE (-2)     /* M, N, K or G outside the supported set */
#define W4A16_ERR_ALIGN (-3)     /* a device pointer is not 16-byte aligned */
#define W4A16_ERR_RANGE (-4)     /* pack: a q or z code is larger than 15, or a
                                    dequantized weight is not a finite fp16;
                                    quantize: a weight is Inf or NaN, or a
                                    group's codes dequantize beyond fp16 */
#define W4A16_ERR_HIP (-5)       /* a HIP runtime call or kernel launch failed */
#define W4A16_ERR_WORKSPACE (-6) /* workspace missing or smaller than required */
#define W4A16_ERR_ARG (-7)       /* path or split selector out of range */

/* Execution paths for w4a16_gemm_ex. */
#define W4A16_PATH_AUTO 0    /* see w4a16_auto_path */
#define W4A16_PATH_DECODE 1  /* weight-streaming, HBM-bound; M <= 64 */
#define W4A16_PATH_PREFILL 2 /* LDS-tiled MFMA, compute-bound; any M */

/*
 * Size in bytes of the packed buffer for a K x N weight with groups of G;
 * 0 if the shape is not supported. Host-only, no HIP call.
 * Equals K*N/2 + 2.5*N*K/G.
 */
size_t w4a16_packed_bytes(int64_t K, int64_t N, int64_t G);

/*
 * Offline packing ("LMDeploy Guide: Fast Mixed-Precision LLM Inference
 * Engine", section 1 "Hardware-Aware Weight Packing (GEMM Pipeline)"): writes
 * the packed buffer from
 *   q       uint8 [K][N]     codes 0..15 (one code per byte)
 *   zeros   uint8 [K/G][N]   codes 0..15
 *   scales  fp16  [K/G][N]
 * into `packed` (w4a16_packed_bytes(K, N, G) bytes, caller-allocated).
 * The dequantized weight (q - z) * s is an fp16 value on the pages (the
 * formula above), so every one must be finite in fp16: W4A16_ERR_RANGE if
 * any code exceeds 15, a scale is Inf or NaN, or |(q - z) * s| >= 65520
 * (which rounds to infinity); on that error the packed contents are
 * unspecified. With this rule neither GEMM path can overflow while
 * dequantizing.
 * Enqueued on `stream` (so that it is ordered after the caller's writes of
 * q, zeros and scales on that stream), then synchronizes that stream (the
 * pass is offline) to report the status.
 */
int w4a16_pack(const uint8_t *q, const uint8_t *zeros, const uint16_t *scales,
               int64_t K, int64_t N, int64_t G, void *packed, void *stream);

/*
 * Group-wise asymmetric 4-bit quantizer, the step that produces the inputs
 * of w4a16_pack from fp16 weights. The pages quantize weights to uniform
 * 4-bit codes in groups of 128 rows with one scale per group ("LMDeploy, in
 * depth", section "Quantization: AWQ weights and KV cache", paragraph
 * "Weight quantization (W4A16)"), dequantized by the formula above, and call
 * the plain form round-to-nearest ("LMDeploy" interview notes, the answer on
 * AWQ versus naive RTN INT4; AWQ's calibrated channel scaling, applied to
 * the weights before this step, is not part of it). The scale and zero
 * spread the group's range [min, max] over 15 steps; per group g and
 * column n, in float32 unless stated:
 *   s   = fp16(max((max - min) / 15, 2^-14))     (round to nearest even)
 *   inv = 1 / s
 *   z   = clamp(rint(-min * inv), 0, 15)
 *   q   = clamp(rint(w * inv) + z, 0, 15)         for every weight w
 * where each product is exact and rint rounds it once to the nearest
 * integer, ties to even. A group of equal weights gets the scale 2^-14 (all
 * zeros give q = z = 0); codes saturate at 0 and 15.
 *
 *   W       fp16  [K][N]     weights (finite)
 *   q       uint8 [K][N]     codes 0..15, one per byte
 *   zeros   uint8 [K/G][N]   codes 0..15
 *   scales  fp16  [K/G][N]
 * Shapes as for w4a16_pack. Enqueued on `stream`, then synchronizes it
 * (offline pass) to report W4A16_ERR_RANGE if a weight is Inf or NaN; on that
 * error the outputs are unspecified.
 */
int w4a16_quantize(const uint16_t *W, int64_t K, int64_t N, int64_t G,
                   uint8_t *q, uint8_t *zeros, uint16_t *scales, void *stream);

/*
 * w4a16_quantize fused with w4a16_pack: one pass over W writes the packed
 * buffer (w4a16_packed_bytes(K, N, G) bytes, caller-allocated), byte for
 * byte what w4a16_pack makes of w4a16_quantize's output. Synchronizes
 * `stream`; W4A16_ERR_RANGE as for w4a16_quantize.
 */
int w4a16_quantize_pack(const uint16_t *W, int64_t K, int64_t N, int64_t G,
                        void *packed, void *stream);

/*
 * Exact inverse of w4a16_pack: recovers q, zeros and scales (same layouts as
 * the inputs of w4a16_pack) from a packed buffer. Enqueued on `stream`, then
 * synchronizes it.
 */
int w4a16_unpack(const void *packed, int64_t K, int64_t N, int64_t G,
                 uint8_t *q, uint8_t *zeros, uint16_t *scales, void *stream);

/*
 * Online GEMM ("LMDeploy Guide: Fast Mixed-Precision LLM Inference Engine",
 * architecture figure, pipeline A, and section 3): Y[M][N] (fp16) =
 * X[M][K] (fp16) . dequant(packed). The 4-bit codes are turned into fp16 by
 * an exponent-OR bit trick, the zero is subtracted exactly and the scale is
 * applied, all inside the kernel; products accumulate in fp32 and Y is
 * rounded to nearest-even once.
 *
 * Asynchronous: enqueued on `stream`, no host synchronization. If the chosen
 * plan splits K across workgroups (see w4a16_workspace_bytes), a per-device
 * library workspace is allocated with hipMalloc on first need and reused;
 * calls that need it must therefore not run concurrently on two streams of
 * one device (use w4a16_gemm_ex with separate workspaces for that). When a
 * larger plan outgrows the workspace, a new one is allocated and the old one
 * is kept (never freed) so that enqueued or graph-captured work stays valid;
 * growing it while `stream` is being captured is refused with
 * W4A16_ERR_WORKSPACE (run the shape once before capturing, or capture
 * w4a16_gemm_ex with a caller-owned workspace).
 */
int w4a16_gemm(const uint16_t *X, const void *packed, int64_t M, int64_t N, int64_t K,
               int64_t G, uint16_t *Y, void *stream);

/*
 * Workspace bytes w4a16_gemm_ex needs for this shape and plan (`path` one of
 * W4A16_PATH_*, `splits` 0 = automatic, else the number of K splits across
 * workgroups). 0 means the plan needs none. Host-only apart from reading the
 * current device's CU count (the plan depends on it; without a device the
 * size is for 256 CUs).
 */
size_t w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G, int path, int splits);

/*
 * w4a16_gemm with an explicit plan and a caller-owned workspace.
 *   path     W4A16_PATH_AUTO / _DECODE / _PREFILL (decode requires M <= 64)
 *   splits   0 = automatic; otherwise 1 .. K/128 workgroup splits of K
 *            (rounded to whole quantization groups per split, and raised
 *            where the decode path's on-chip staging needs it)
 *   workspace, workspace_bytes: at least w4a16_workspace_bytes(...) bytes of
 *            device memory (any contents), or NULL/0 if that is 0. It holds
 *            the fp32 partial sums of the K splits between the GEMM kernel
 *            and the reduce kernel, so calls sharing one workspace must be
 *            ordered (same stream).
 * Rounding depends on the plan, the exact result does not: the decode path
 * multiplies the exact integers (q - z) by X and applies each group's scale
 * to the group's fp32 partial sum; the prefill path rounds every dequantized
 * weight (q - z) * s to fp16 once before multiplying; both accumulate in fp32
 * (in an order that depends on `splits`) and round Y to fp16 once. Results
 * of different plans therefore differ by a few fp16 units at most, within
 * max|dY| <= 4e-3 max|Y| and ||dY||_F <= 1e-3 ||Y||_F of the exact product;
 * for a fixed plan the result is bitwise reproducible.
 */
int w4a16_gemm_ex(const uint16_t *X, const void *packed, int64_t M, int64_t N, int64_t K,
                  int64_t G, uint16_t *Y, void *workspace, size_t workspace_bytes,
                  int path, int splits, void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * w4a16_gemm with the same automatic plan and kernels (results bitwise equal
 * to w4a16_gemm's), whose split-K partials go to a fixed scratch array
 * inside the library instead of an allocated workspace:
 * W4A16_NOALLOC_SCRATCH_BYTES per GPU, placed when the library's code object
 * is loaded on that GPU and held until the process ends. The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks up that device's address of the array. Returns
 * W4A16_ERR_WORKSPACE, launching nothing, if the plan's partials exceed the
 * scratch (every automatic plan fits on a 256-CU MI355X). All calls on one
 * GPU share its scratch, which keeps the last call's partials (every plan
 * writes each partial before reading it, so nothing needs clearing): calls
 * that overlap on one GPU (two streams, or two threads) race; calls ordered
 * on one stream are safe. Other arguments and errors as for w4a16_gemm.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (64u << 20)
int w4a16_gemm_noalloc(const uint16_t *X, const void *packed, int64_t M, int64_t N, int64_t K,
                       int64_t G, uint16_t *Y, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Low-bit KV cache and decode attention (the pages' second pipeline:
 * "LMDeploy Guide: Fast Mixed-Precision LLM Inference Engine", architecture
 * figure, pipeline B, sections 2 "Adaptive Head Alignment" and 4
 * "Asynchronous KV Memory Loading Pipeline"; "LMDeploy, in depth", the
 * blocked KV cache (64 tokens per block) and KV cache quantization: online,
 * asymmetric, per head and per token, 8 or 4 bits).
 *
 * Head dimension 128. Every key and value vector of one (token, KV head) is
 * quantized on its own, with L = 2^bits - 1 steps over its range (the same
 * reading as w4a16_quantize): s = fp16(max((max - min) / L, 2^-14)),
 * z = clamp(rint(-min / s), 0, L), c = clamp(rint(x / s) + z, 0, L), the
 * products with the float32 reciprocal of s exact and rounded once.
 *
 * Cache: an array of num_blocks blocks of w4a16_kv_block_bytes(bits,
 * kv_heads) bytes; block b holds kv_heads regions, region (b, h) at byte
 * (b * kv_heads + h) * (w4a16_kv_block_bytes / kv_heads). Inside a region,
 * KC = 64 * 128 * bits / 8:
 *   [0, KC)          K codes, token-major rows of 128 codes
 *   [KC, 2 KC)       V codes, rows of 64 bytes, token t's byte at position
 *                    p(t) = 16 ((t % 16) / 4) + 8 (t / 32) + 4 ((t / 16) % 2) + t % 4;
 *                    8-bit: row d = 0..127 holds dimension d; 4-bit: row
 *                    r = 0..63 holds dimension r (low nibble) and r + 64
 *                    (high nibble)
 *   [2 KC, +256)     K parameters, 4 bytes per token: fp16 scale, zero, 0
 *   [2 KC + 256, +256) V parameters
 * 4-bit K codes are two per byte, the even index in the low nibble. Token i
 * of a sequence lives in block block_table[b][i / 64] at offset i % 64.
 * ---------------------------------------------------------------------------
 */

/* Bytes of one cache block for kv_heads heads; 0 if bits is not 4 or 8. */
size_t w4a16_kv_block_bytes(int bits, int64_t kv_heads);

/*
 * Quantize and store new tokens:
 *   k, v    fp16 [ntok][kv_heads][128]
 *   slots   int32 [ntok], block * 64 + offset of each token; a negative
 *           slot, or one past num_blocks blocks, skips that token
 *   cache   the cache (num_blocks blocks)
 * Asynchronous on `stream`. Tokens of one call may share cache blocks;
 * two tokens of one call must not share a slot. Non-finite inputs give
 * unspecified codes.
 */
int w4a16_kv_append(const uint16_t *k, const uint16_t *v, const int32_t *slots, int64_t ntok,
                    int64_t kv_heads, int bits, void *cache, int64_t num_blocks, void *stream);

/* Workspace bytes of w4a16_kv_attention for this batch (depends on the
 * current device's CU count; 0 for an invalid shape). */
size_t w4a16_kv_attention_workspace_bytes(int64_t B, int64_t kv_heads, int64_t max_blocks);

/*
 * Decode attention of one new query token per sequence:
 *   out[b][h] = softmax(sm_scale * q[b][h] . K_b^T) . V_b
 * over the lengths[b] tokens of sequence b, with K and V dequantized as
 * (c - z) * s and query head h reading KV head h / (q_heads / kv_heads).
 *   q, out       fp16 [B][q_heads][128]
 *   block_table  int32 [B][max_blocks]; entries outside [0, num_blocks) are
 *                read as empty blocks
 *   lengths      int32 [B]; a length <= 0 gives zeros, one above
 *                max_blocks * 64 is clamped
 *   workspace    at least w4a16_kv_attention_workspace_bytes(B, kv_heads,
 *                max_blocks) bytes of device memory (any contents)
 * q_heads must be a multiple of kv_heads, at most 16 query heads per KV
 * head; max_blocks <= 2^24, B * kv_heads <= 2^26, B * q_heads <= 2^30.
 * Asynchronous on `stream`; calls sharing a workspace must be ordered.
 */
int w4a16_kv_attention(const uint16_t *q, const void *cache, int64_t num_blocks,
                       const int32_t *block_table, int64_t max_blocks, const int32_t *lengths,
                       int64_t B, int64_t q_heads, int64_t kv_heads, int bits, float sm_scale,
                       uint16_t *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ---------------------------------------------------------------------------
 * W8A8 GEMM: 8-bit weights times 8-bit activations on the int8 matrix cores
 * (W8A8 is the precision format "LMDeploy Guide: Fast Mixed-Precision LLM
 * Inference Engine" lists beside W4A16; the pages give no formula). Symmetric
 * scales: one per output channel for W (offline), one per token for X (per
 * call): s = max|v| / 127 in float32 (1 for an all-zero vector), code =
 * clamp(rint(v / s), -127, 127) with the product of v and the float32
 * reciprocal of s exact and rounded once; Y[m][n] =
 * fp16(float32(float32(acc) * s_x[m]) * s_w[n]) with acc the exact int32 sum
 * of code products.
 *
 * Shapes: K % 256 == 0, K <= 131072 (the int32 sum cannot overflow),
 * N % 16 == 0, K * N < 2^32, 1 <= M <= 2^30.
 * Packed weights (K * N bytes): 1 KiB tiles of 16 columns x 64 rows of K,
 * tile (n / 16) * (K / 64) + k / 64; inside a tile, 16 bytes per lane
 * l = 16 * ((k % 64) / 16) + n % 16, byte k % 16 (int8 codes).
 * ---------------------------------------------------------------------------
 */

/* Bytes of the packed W8A8 weights (K * N); 0 for an unsupported shape. */
size_t w4a16_w8a8_packed_bytes(int64_t K, int64_t N);

/* Offline: fp16 W [K][N] -> packed int8 codes and float32 w_scales [N].
 * Asynchronous on `stream`; non-finite weights give unspecified codes. */
int w4a16_w8a8_quantize_weights(const uint16_t *W, int64_t K, int64_t N, void *packed, float *w_scales,
                                void *stream);

/* Per call: fp16 X [M][K] -> int8 xq [M][K] and float32 x_scales [M].
 * Asynchronous on `stream`. */
int w4a16_w8a8_quantize_act(const uint16_t *X, int64_t M, int64_t K, int8_t *xq, float *x_scales,
                            void *stream);

/* Workspace bytes of w4a16_w8a8_gemm (int32 partial sums when K is split
 * across workgroups, which happens only above 16 rows: up to M = 16 one
 * launch sums K inside each workgroup; depends on the current device's CU
 * count; 0 if none). */
size_t w4a16_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Y[M][N] (fp16) from the codes and scales above. Asynchronous on `stream`;
 * calls sharing a workspace must be ordered. */
int w4a16_w8a8_gemm(const int8_t *xq, const float *x_scales, const void *packed, const float *w_scales,
                    int64_t M, int64_t N, int64_t K, uint16_t *Y, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * Measurement yardstick, not part of the GEMM: one kernel launch that reads
 * `bytes` bytes of the device buffer `buf` (16-byte loads, each byte once,
 * non-temporal) and nothing else, the plainest bound on a launch that
 * streams that many bytes ("LMDeploy" interview notes: each decode step
 * streams every weight byte once). Folds the data into one word per lane and
 * writes it to `sink` (64 uint32, device) only where it equals `never`, so
 * in practice nothing is written. 0 < bytes < 2^31. Asynchronous on `stream`.
 */
int w4a16_stream_read(const void *buf, size_t bytes, uint32_t never, uint32_t *sink, void *stream);

/* Static description of a status code. */
const char *w4a16_status_string(int status);

/* Message of the last failing call on the calling thread ("" if none). */
const char *w4a16_last_error(void);

/* W4A16_LAYOUT_VERSION of the compiled library. */
int w4a16_layout_version(void);

/*
 * The path W4A16_PATH_AUTO takes for this shape: W4A16_PATH_DECODE for
 * M <= 32, and for M <= 64 when N <= 6144 (narrow matrices, where the
 * weight-streaming kernel measured faster than the tiled one); otherwise
 * W4A16_PATH_PREFILL. Host-only. Returns W4A16_ERR_SHAPE for an
 * unsupported shape.
 */
int w4a16_auto_path(int64_t M, int64_t N, int64_t K, int64_t G);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
