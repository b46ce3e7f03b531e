// Prefill path of the W4A16 GEMM: large M, bound by the matrix cores.
//
// Prefill is compute-bound ("LMDeploy" interview notes: prefill gains less
// from 4-bit weights because it is compute-bound), so this path is organised
// around keeping the MFMA units busy, following the GEMM pipeline of
// "LMDeploy Guide: Fast Mixed-Precision LLM Inference Engine" (architecture
// figure, pipeline A: asynchronous global load, bank-conflict-free on-chip
// staging, dequantization interleaved with the math, direct matrix-core
// execution), re-shaped for gfx950:
//
// * Workgroup tile BM x (64 NSW): four waves side by side along N, each
//   owning all BM rows and NSW 16-column strips, so no two waves dequantize
//   the same weight.
// * Activations: the BM x 128 tile of X for the next K block is copied
//   global -> LDS by direct 16-byte loads (no register staging) while the
//   current block is being multiplied (two LDS stages). Inside a 256-byte
//   LDS row the sixteen 16-byte chunks are stored XOR-swizzled by the row
//   index, so the 16 lanes that read one k chunk from 16 consecutive rows hit
//   16 different bank groups.
// * Weights: each wave loads its packed tiles straight into registers, one
//   16-byte load per lane per strip and K block (the packed order is the
//   operand order, so there is no run-time swizzle), one block ahead.
// * Dequantization (section 3 of the same page, FP16 = (INT4 - ZeroPoint) x
//   Scale): exponent-OR gives 1024 + q, a packed fp16 add of -(1024 + z)
//   gives q - z exactly, a packed fp16 multiply by s gives the weight
//   rounded once to fp16. The B operand of every 16 x 16 x 32 MFMA is
//   produced this way and reused for all BM/16 row tiles.
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

template <int MTW, int NSW, int GS>
__global__ void __launch_bounds__(256)
prefill_kernel(const uint16_t *__restrict__ X, const uint8_t *__restrict__ packed,
               uint16_t *__restrict__ Y, int M, int N, int K, int tiles_m) {
    constexpr int BM = 16 * MTW;
    constexpr int STAGE = BM * 256;  // BM rows x 128 k x 2 bytes
    constexpr int F = GS < 4 ? GS : 4;
    constexpr int NF = 4 / F;
    constexpr int XLOADS = BM / 16;  // 16-byte direct loads per thread per stage
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int nblk = K / kBlockK;
    const int ngrp = K / (32 * GS);
    const int nstrip = N / kStripCols;
    const int tm = blockIdx.x % tiles_m;
    const int tn = blockIdx.x / tiles_m;
    const int m0 = tm * BM;
    const int strip_w = tn * 4 * NSW + wave * NSW;  // first strip of this wave
    const PackedView pv = packed_view(packed, K, N, 32 * GS);
    const uint32_t magic = kMagic;

    // Global source of this thread's X chunks (row clamped into [0, M)).
    const uint16_t *xsrc[XLOADS];
#pragma unroll
    for (int i = 0; i < XLOADS; ++i) {
        const int f = (i * 4 + wave) * 64 + lane;
        const int row = f >> 4;
        const int chunk = (f & 15) ^ (row & 15);
        int grow = m0 + row;
        grow = grow < M ? grow : M - 1;
        xsrc[i] = X + (size_t)grow * K + chunk * 8;
    }
    auto issue_x = [&](int b, int stage) {
#pragma unroll
        for (int i = 0; i < XLOADS; ++i) {
            __builtin_amdgcn_global_load_lds(
                (const void *)(xsrc[i] + b * kBlockK),
                (lds_void *)(lds + stage * STAGE + (i * 4 + wave) * 1024), 16, 0, 0);
        }
    };
    auto load_w = [&](int b, u32x4 *w, uint32_t (*sz)[NSW]) {
#pragma unroll
        for (int j = 0; j < NSW; ++j) {
            const int s = strip_w + j;
            if (s < nstrip) {
                w[j] = pv.w[((size_t)s * nblk + b) * 64 + lane];
#pragma unroll
                for (int f = 0; f < NF; ++f)
                    sz[f][j] = load_scale_zero(pv, (size_t)s * ngrp + (b * 4 + f * F) / GS, col);
            } else {
                w[j] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int f = 0; f < NF; ++f) sz[f][j] = 0u;
            }
        }
    };

    floatx4 acc[MTW][NSW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int j = 0; j < NSW; ++j) acc[mt][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    u32x4 wc[NSW], wn[NSW];
    uint32_t szc[NF][NSW], szn[NF][NSW];
    issue_x(0, 0);
    load_w(0, wc, szc);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int b = 0; b < nblk; ++b) {
        const int cur = b & 1;
        if (b + 1 < nblk) {
            issue_x(b + 1, cur ^ 1);
            load_w(b + 1, wn, szn);
        }
        const uint8_t *st = lds + cur * STAGE;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int f = t / F;
            half8 bw[NSW];
#pragma unroll
            for (int j = 0; j < NSW; ++j) {
                const uint32_t sz = szc[f][j];
                const uint32_t s2 = (sz & 0xFFFFu) | (sz << 16);
                bw[j] = dequant_w(t, wc[j], neg_bias_pair(sz), s2, magic);
            }
            const int chunk = (4 * t + kq) ^ col;
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) {
                const half8 a = *reinterpret_cast<const half8 *>(st + (mt * 16 + col) * 256 + chunk * 16);
#pragma unroll
                for (int j = 0; j < NSW; ++j) acc[mt][j] = mfma16x16x32(a, bw[j], acc[mt][j]);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NSW; ++j) {
            wc[j] = wn[j];
#pragma unroll
            for (int f = 0; f < NF; ++f) szc[f][j] = szn[f][j];
        }
    }

    // Epilogue: fp32 -> fp16 (round to nearest even), rows beyond M dropped.
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int j = 0; j < NSW; ++j) {
            const int s = strip_w + j;
            if (s >= nstrip) continue;
            const size_t n = (size_t)s * kStripCols + col;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + mt * 16 + 4 * kq + e;
                if (row < M) Y[(size_t)row * N + n] = f32_to_f16_bits(acc[mt][j][e]);
            }
        }
}

template <int MTW, int NSW>
hipError_t launch_shape(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G,
                        uint16_t *Y, hipStream_t stream) {
    constexpr int BM = 16 * MTW, BN = 64 * NSW;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    switch (G) {
        case 32: hipLaunchKernelGGL((prefill_kernel<MTW, NSW, 1>), grid, dim3(256), 0, stream, X, packed, Y, M, N, K, tiles_m); break;
        case 64: hipLaunchKernelGGL((prefill_kernel<MTW, NSW, 2>), grid, dim3(256), 0, stream, X, packed, Y, M, N, K, tiles_m); break;
        case 128: hipLaunchKernelGGL((prefill_kernel<MTW, NSW, 4>), grid, dim3(256), 0, stream, X, packed, Y, M, N, K, tiles_m); break;
        case 256: hipLaunchKernelGGL((prefill_kernel<MTW, NSW, 8>), grid, dim3(256), 0, stream, X, packed, Y, M, N, K, tiles_m); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G,
                          uint16_t *Y, hipStream_t stream) {
    if (M <= 64) return launch_shape<4, 4>(X, packed, M, N, K, G, Y, stream);
    if (M <= 128) return launch_shape<8, 4>(X, packed, M, N, K, G, Y, stream);
    return launch_shape<16, 4>(X, packed, M, N, K, G, Y, stream);
}

}  // namespace w4a16
