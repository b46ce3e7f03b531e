// Decode path of the W4A16 GEMM: small M (<= 64), bound by HBM bandwidth.
//
// Each generated token streams every weight byte once, so at small M the
// GEMM is limited by memory bandwidth, not arithmetic ("LMDeploy" interview
// notes, answer to why W4A16 raises throughput although FLOPs do not change;
// "LMDeploy, in depth", section "Quantization: AWQ weights and KV cache").
// The kernel is therefore built around the weight stream:
//
// * Work unit: one 1 KiB packed tile (16 columns x 128 rows of K), read by
//   one wave64 with one 16-byte load per lane. A workgroup owns NS adjacent
//   strips (16 NS columns) and one of S contiguous slices of K; its waves
//   take the 128-row blocks of that slice in turn, NB blocks at a time, and
//   issue every tile load of a batch before touching the data.
// * Dequantization ("LMDeploy Guide: Fast Mixed-Precision LLM Inference
//   Engine", section 3, FP16 = (INT4 - ZeroPoint) x Scale): the exponent-OR
//   trick turns each code into the fp16 value 1024 + q, a packed fp16 add of
//   -(1024 + z) leaves the exact integer q - z, and the matrix instruction
//   multiplies that with X. The scale is applied in fp32 once per group and
//   column to the group's partial sum. The integer work of one tile is
//   independent of the others in the batch, so it interleaves with the
//   matrix instructions of neighbouring tiles (the pages' ILP point).
// * Activations: X is padded to 16 rows per MFMA tile by zero lanes; each
//   lane loads its 8 consecutive fp16 of X straight into the A operand.
// * Reduction: partial sums of the waves of a workgroup are added in LDS in
//   fixed wave order. With S > 1 each workgroup writes fp32 partials to a
//   workspace, and the last workgroup of a column tile to finish (counted
//   with a device-scope atomic) adds the S partials in fixed split order and
//   writes fp16 Y, then resets the counter. Results are bitwise reproducible
//   for a fixed plan.
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

template <int MT, int NS, int WAVES, int NB, int GS>
__global__ void __launch_bounds__(WAVES * 64)
decode_kernel(const uint16_t *__restrict__ X, const uint8_t *__restrict__ packed,
              uint16_t *__restrict__ Y, float *__restrict__ part, uint32_t *__restrict__ counters,
              int M, int N, int K, int S) {
    constexpr int F = GS < 4 ? GS : 4;  // 32-row k-steps per scale group inside a block
    constexpr int NF = 4 / F;            // scale groups per 128-row block
    __shared__ floatx4 red[WAVES][MT * NS][64];
    __shared__ int is_last;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int nblk = K / kBlockK;
    const int ngrp = K / (32 * GS);
    const int nstrip = N / kStripCols;
    const int strip0 = blockIdx.x * NS;
    const int split = blockIdx.y;
    const int bb = (int)((int64_t)split * nblk / S);
    const int be = (int)((int64_t)(split + 1) * nblk / S);
    const PackedView pv = packed_view(packed, K, N, 32 * GS);

    floatx4 acc[MT][NS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[mt][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int b0 = bb + wave * NB; b0 < be; b0 += WAVES * NB) {
        u32x4 w[NB][NS];
        half8 a[NB][4][MT];
        uint32_t sz[NB][NF][NS];
        // 1. the weight stream: one 16-byte load per lane per tile
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const int b = b0 + i, s = strip0 + j;
                if (b < be && s < nstrip)
                    w[i][j] = __builtin_nontemporal_load(&pv.w[((size_t)s * nblk + b) * 64 + lane]);
                else
                    w[i][j] = u32x4{0u, 0u, 0u, 0u};
            }
        // 2. activations: 8 consecutive k of one row per lane
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int b = b0 + i, row = mt * 16 + col;
                    if (b < be && row < M)
                        a[i][t][mt] = *reinterpret_cast<const half8 *>(
                            X + (size_t)row * K + b * kBlockK + t * 32 + kq * 8);
                    else
                        a[i][t][mt] = half8{0, 0, 0, 0, 0, 0, 0, 0};
                }
        // 3. scale and zero of every group the batch touches
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    const int b = b0 + i, s = strip0 + j;
                    if (b < be && s < nstrip) {
                        const int g = (b * 4 + f * F) / GS;
                        sz[i][f][j] = load_scale_zero(pv, (size_t)s * ngrp + g, col);
                    } else {
                        sz[i][f][j] = 0u;
                    }
                }
        // 4. dequantize and multiply
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                floatx4 accg[MT][NS];
#pragma unroll
                for (int tt = 0; tt < F; ++tt) {
                    const int t = f * F + tt;
#pragma unroll
                    for (int j = 0; j < NS; ++j) {
                        const half8 bq = dequant_qz(w[i][j][t], neg_bias_pair(sz[i][f][j]));
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            accg[mt][j] = mfma16x16x32(a[i][t][mt], bq,
                                                       tt == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : accg[mt][j]);
                    }
                }
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    const float sc = scale_of(sz[i][f][j]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[mt][j][e] = __builtin_fmaf(sc, accg[mt][j][e], acc[mt][j][e]);
                }
            }
    }

    // Sum the waves' partial tiles in LDS, wave 0 first.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NS; ++j) red[wave][mt * NS + j][lane] = acc[mt][j];
    __syncthreads();

    const int rows = M < MT * 16 ? M : MT * 16;
    const int outs = rows * NS * 16;
    for (int o = threadIdx.x; o < outs; o += WAVES * 64) {
        const int r = o / (NS * 16), c = o % (NS * 16);
        const int j = c >> 4, cl = c & 15, mt = r >> 4, rr = r & 15;
        const int ln = (rr >> 2) * 16 + cl, e = rr & 3;
        float v = 0.f;
#pragma unroll
        for (int wv = 0; wv < WAVES; ++wv) v += red[wv][mt * NS + j][ln][e];
        if (strip0 + j < nstrip) {
            const size_t n = (size_t)(strip0 + j) * kStripCols + cl;
            if (S == 1)
                Y[(size_t)r * N + n] = f32_to_f16_bits(v);
            else
                part[((size_t)split * M + r) * N + n] = v;
        }
    }
    if (S == 1) return;

    // Cross-workgroup reduction: the last of the S workgroups of this column
    // tile to arrive adds all partials in split order.
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&counters[blockIdx.x], 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        is_last = (prev == (uint32_t)(S - 1));
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    for (int o = threadIdx.x; o < outs; o += WAVES * 64) {
        const int r = o / (NS * 16), c = o % (NS * 16);
        const int j = c >> 4, cl = c & 15;
        if (strip0 + j >= nstrip) continue;
        const size_t n = (size_t)(strip0 + j) * kStripCols + cl;
        float v = 0.f;
        for (int sp = 0; sp < S; ++sp)
            v += __hip_atomic_load(&part[((size_t)sp * M + r) * N + n], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        Y[(size_t)r * N + n] = f32_to_f16_bits(v);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&counters[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Launch shapes per row-tile count MT: strips per workgroup, waves, blocks
// per wave batch.
struct DecodeShape {
    int ns, waves, nb;
};

inline DecodeShape decode_shape(int mt) {
    switch (mt) {
        case 1: return {4, 4, 2};
        case 2: return {4, 4, 2};
        default: return {4, 4, 1};
    }
}

inline int decode_mt(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

template <int MT, int GS>
hipError_t launch_mt_gs(const uint16_t *X, const uint8_t *packed, int M, int N, int K, uint16_t *Y,
                        float *part, uint32_t *counters, int S, hipStream_t stream) {
    constexpr int NS = 4, WAVES = 4, NB = (MT <= 2 ? 2 : 1);
    const int tiles = (N / kStripCols + NS - 1) / NS;
    hipLaunchKernelGGL((decode_kernel<MT, NS, WAVES, NB, GS>), dim3(tiles, S), dim3(WAVES * 64), 0,
                       stream, X, packed, Y, part, counters, M, N, K, S);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G,
                     uint16_t *Y, float *part, uint32_t *counters, int S, hipStream_t stream) {
    switch (G) {
        case 32: return launch_mt_gs<MT, 1>(X, packed, M, N, K, Y, part, counters, S, stream);
        case 64: return launch_mt_gs<MT, 2>(X, packed, M, N, K, Y, part, counters, S, stream);
        case 128: return launch_mt_gs<MT, 4>(X, packed, M, N, K, Y, part, counters, S, stream);
        case 256: return launch_mt_gs<MT, 8>(X, packed, M, N, K, Y, part, counters, S, stream);
        default: return hipErrorInvalidValue;
    }
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

int decode_max_splits(int M, int N, int K) {
    (void)M;
    (void)N;
    return K / kBlockK;
}

int decode_auto_splits(int M, int N, int K, int G, int num_cus) {
    (void)G;
    const DecodeShape sh = decode_shape(decode_mt(M));
    const int tiles = (N / kStripCols + sh.ns - 1) / sh.ns;
    const int nblk = K / kBlockK;
    // Aim for about 8 resident waves per compute unit, but give each wave
    // at least one full batch of blocks.
    const int want_waves = 8 * num_cus;
    int s = (want_waves + tiles * sh.waves - 1) / (tiles * sh.waves);
    const int cap = nblk / (sh.waves * sh.nb);
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    return s;
}

size_t decode_workspace_bytes(int M, int N, int K, int G, int splits) {
    (void)K;
    (void)G;
    if (splits <= 1) return 0;
    const DecodeShape sh = decode_shape(decode_mt(M));
    const int tiles = (N / kStripCols + sh.ns - 1) / sh.ns;
    return align_up((size_t)tiles * sizeof(uint32_t), 256) +
           (size_t)splits * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_decode(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G,
                         uint16_t *Y, void *workspace, int splits, hipStream_t stream) {
    const int mt = decode_mt(M);
    const DecodeShape sh = decode_shape(mt);
    const int tiles = (N / kStripCols + sh.ns - 1) / sh.ns;
    uint32_t *counters = nullptr;
    float *part = nullptr;
    if (splits > 1) {
        counters = static_cast<uint32_t *>(workspace);
        part = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) +
                                         align_up((size_t)tiles * sizeof(uint32_t), 256));
    }
    switch (mt) {
        case 1: return launch_mt<1>(X, packed, M, N, K, G, Y, part, counters, splits, stream);
        case 2: return launch_mt<2>(X, packed, M, N, K, G, Y, part, counters, splits, stream);
        default: return launch_mt<4>(X, packed, M, N, K, G, Y, part, counters, splits, stream);
    }
}

}  // namespace w4a16
