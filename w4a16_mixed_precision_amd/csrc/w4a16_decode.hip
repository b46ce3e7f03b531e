// Decode path of the W4A16 GEMM: small M (<= 64), bound by HBM bandwidth.
//
// Each generated token streams every weight byte once, so at small M the
// GEMM is limited by memory bandwidth, not arithmetic ("LMDeploy" interview
// notes, answer to why W4A16 raises throughput although FLOPs do not change;
// "LMDeploy, in depth", section "Quantization: AWQ weights and KV cache").
// The kernel is built so that streaming the weights costs as few vector
// memory instructions as possible: on gfx950 the per-CU address unit, not
// DRAM, is what runs out first when every 1 KiB weight tile also drags in
// activation and scale loads.
//
// * Work unit: one 1 KiB packed tile (16 columns x 128 rows of K), read by
//   one wave64 with one 16-byte buffer load per lane. A workgroup owns NS
//   adjacent 16-column strips and one of S slices of K; its WK waves split
//   the slice into contiguous runs of 128-row blocks and each wave streams
//   all NS strips of its run, two batches of tiles in flight.
// * Scales and zeros of the workgroup's strips and slice are staged in LDS
//   once, already turned into the fp16 pair -(1024 + z) and the fp32 scale,
//   so the main loop reads them with one LDS load per group and strip.
// * Activations: for M <= 4 the rows of X in the slice are staged in LDS too
//   (a few KiB) and every lane reads its A operand from there; for larger M
//   each wave loads its A operands from global memory once per 32-row step
//   and uses them for all NS strips, so X costs 4/NS loads per tile.
//   Rows >= M of the 16-row MFMA tile are padding: their results are never
//   stored.
// * Dequantization ("LMDeploy Guide: Fast Mixed-Precision LLM Inference
//   Engine", section 3, FP16 = (INT4 - ZeroPoint) x Scale): one v_and_or_b32
//   per pair of codes sets the fp16 exponent field and yields 1024 + q (or
//   1024 + 16 q for the two steps stored in the high nibbles); a packed fp16
//   add of -(1024 + z) (or -(1024 + 16 z)) leaves the exact integer q - z (or
//   16 (q - z)), which the matrix instruction multiplies with X. The scale
//   (and the 1/16) is applied in fp32 once per group and column to the
//   group's partial sum. The integer work of one tile is independent of the
//   other tiles in flight, so it interleaves with the matrix instructions and
//   the loads (the pages' ILP point).
// * Reduction: the WK partial tiles of each strip are added in LDS in fixed
//   order. With S == 1 the workgroup writes fp16 Y directly. With S > 1 each
//   workgroup writes its fp32 partial to a workspace and a second small
//   kernel adds the S partials in split order; the kernel boundary orders the
//   two, so no device-scope fence is needed (on the multi-XCD gfx950 such a
//   fence writes back the whole L2, which costs more than the GEMM itself at
//   these sizes). Results are bitwise reproducible for a fixed plan.
#include <stdlib.h>

#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

// Per (strip, group, column) record in LDS: -(1024 + z) as an fp16 pair and
// the fp32 scale.
struct SZ {
    uint32_t nb;
    float sc;
};

template <int MT, int NS, int NB>
struct DecodeBatch {
    u32x4 w[NB][NS];
    half8 a[NB][4][MT];  // register-X mode only
};

// Dynamic LDS layout: [ sz records | X rows (LDS-X mode) or reduction ].
struct DecodeLds {
    uint32_t sz_bytes, x_bytes, red_bytes, x_stride;
    __host__ __device__ uint32_t total() const {
        return sz_bytes + (x_bytes > red_bytes ? x_bytes : red_bytes);
    }
};

__host__ __device__ inline DecodeLds decode_lds(int M, int MT, int NS, int WK, int slice_blocks, int G,
                                                 bool xlds) {
    DecodeLds l;
    const int groups = (slice_blocks * kBlockK + G - 1) / G;
    l.sz_bytes = (uint32_t)(NS * groups * 16 * sizeof(SZ));
    l.x_stride = (uint32_t)(slice_blocks * kBlockK * 2 + 16);  // +16 B: rows in different banks
    l.x_bytes = xlds ? (uint32_t)M * l.x_stride : 0u;
    l.red_bytes = (uint32_t)(WK * NS * MT * 64 * 16);
    return l;
}

template <int MT, int NS, int WK, int NB, int GS, bool XLDS>
__global__ void __launch_bounds__(WK * 64)
decode_kernel(const uint16_t *__restrict__ X, const uint8_t *__restrict__ packed,
              uint16_t *__restrict__ Y, float *__restrict__ part, int M, int N, int K, int S,
              int slice_blocks) {
    constexpr int F = GS < 4 ? GS : 4;  // 32-row k-steps per scale group inside a block
    constexpr int NF = 4 / F;            // scale groups per 128-row block
    constexpr int G = 32 * GS;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int lane = threadIdx.x & 63;
    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int nblk = K / kBlockK;
    const int ngrp = K / G;
    const int nstrip = N / kStripCols;
    const int strip0 = blockIdx.x * NS;
    const int split = blockIdx.y;
    const int bb = split * slice_blocks;
    const int be = bb + slice_blocks < nblk ? bb + slice_blocks : nblk;
    const int per = (be - bb + WK - 1) / WK;
    const int wb = bb + wk * per;
    const int we = wb + per < be ? wb + per : be;
    const int g0 = bb * kBlockK / G;  // slices start on a group boundary
    const int ng = ((be - bb) * kBlockK + G - 1) / G;

    const DecodeLds L = decode_lds(M, MT, NS, WK, slice_blocks, G, XLDS);
    SZ *szl = reinterpret_cast<SZ *>(lds);
    uint8_t *xl = lds + L.sz_bytes;

    __amdgpu_buffer_rsrc_t rw[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int s = strip0 + j < nstrip ? strip0 + j : 0;
        rw[j] = make_rsrc(packed + (size_t)s * nblk * kTileBytes, (uint32_t)nblk * kTileBytes);
    }
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (uint32_t)((size_t)M * K * 2));
    uint32_t xoff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row = mt * 16 + col;
        if constexpr (XLDS)  // rows >= M read row M-1: padding rows are never stored
            xoff[mt] = (uint32_t)((row < M ? row : M - 1) * L.x_stride + kq * 16);
        else
            xoff[mt] = (uint32_t)((row * K + kq * 8) * 2);
    }
    const uint32_t magic = kMagic;

    floatx4 acc[MT][NS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[mt][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    typedef DecodeBatch<MT, NS, NB> Batch;
    auto load = [&](int b0, Batch &bt) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < NS; ++j)
                if (b0 + i < we)
                    bt.w[i][j] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw[j], lane * 16, (b0 + i) * kTileBytes, 0));
        if constexpr (!XLDS) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        if (b0 + i < we && mt * 16 + col < M)
                            bt.a[i][t][mt] = __builtin_bit_cast(
                                half8, __builtin_amdgcn_raw_buffer_load_b128(
                                           rx, xoff[mt], ((b0 + i) * kBlockK + t * 32) * 2, 0));
        }
    };
    auto compute = [&](int b0, const Batch &bt) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int b = b0 + i;
            if (b >= we) break;
            half8 a[4][MT];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if constexpr (XLDS)
                        a[t][mt] = *reinterpret_cast<const half8 *>(
                            xl + xoff[mt] + ((b - bb) * kBlockK + t * 32) * 2);
                    else
                        a[t][mt] = bt.a[i][t][mt];
                }
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                u32x4 w8;
#pragma unroll
                for (int v = 0; v < 4; ++v) w8[v] = bt.w[i][j][v] >> 8;
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const int g = (b * 4 + f * F) / GS;
                    const SZ sz = szl[(j * ng + (g - g0)) * 16 + col];
                    const uint32_t nb_lo = sz.nb;
                    const uint32_t nb_hi = ((nb_lo & 0x000F000Fu) << 4) | 0xE400E400u;
                    floatx4 acc_lo[MT], acc_hi[MT];
                    bool lo_used = false, hi_used = false;
#pragma unroll
                    for (int tt = 0; tt < F; ++tt) {
                        const int t = f * F + tt;
                        const half8 bq = dequant_qz(t, bt.w[i][j], w8, nb_lo, nb_hi, magic);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            if (t < 2)
                                acc_lo[mt] = mfma16x16x32(a[t][mt], bq,
                                                          lo_used ? acc_lo[mt] : floatx4{0.f, 0.f, 0.f, 0.f});
                            else
                                acc_hi[mt] = mfma16x16x32(a[t][mt], bq,
                                                          hi_used ? acc_hi[mt] : floatx4{0.f, 0.f, 0.f, 0.f});
                        }
                        if (t < 2) lo_used = true; else hi_used = true;
                    }
                    const float sc = sz.sc, sc16 = sz.sc * 0.0625f;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (lo_used) acc[mt][j][e] = __builtin_fmaf(sc, acc_lo[mt][e], acc[mt][j][e]);
                            if (hi_used) acc[mt][j][e] = __builtin_fmaf(sc16, acc_hi[mt][e], acc[mt][j][e]);
                        }
                }
            }
        }
    };

    Batch b0, b1;
    if constexpr (!XLDS) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    b0.a[i][t][mt] = half8{0, 0, 0, 0, 0, 0, 0, 0};
                    b1.a[i][t][mt] = half8{0, 0, 0, 0, 0, 0, 0, 0};
                }
    }
    // With LDS-staged X the first two batches of weight tiles go out before
    // the staging, so their latency overlaps it (with register X the extra
    // live registers would cost occupancy; those waves load after staging).
    int b = wb;
    if constexpr (XLDS) {
        if (b < we) load(b, b0);
        if (b + NB < we) load(b + NB, b1);
    }

    // ---- stage scale/zero records of the slice: [NS][ng][16]
    {
        const uint16_t *sreg = reinterpret_cast<const uint16_t *>(packed + weight_bytes(K, N));
        const uint8_t *zreg = packed + weight_bytes(K, N) + scale_bytes(K, N, G);
        for (int e = threadIdx.x; e < NS * ng * 16; e += WK * 64) {
            const int j = e / (ng * 16), r = e % (ng * 16);
            const int g = g0 + r / 16, c = r % 16;
            const int s = strip0 + j;
            SZ v{0u, 0.f};
            if (s < nstrip) {
                const size_t rec = (size_t)s * ngrp + g;
                const uint32_t z = (zreg[rec * 8 + (c >> 1)] >> ((c & 1) * 4)) & 15u;
                const uint32_t h = 0xE400u | z;
                v.nb = h | (h << 16);
                v.sc = (float)__builtin_bit_cast(_Float16, sreg[rec * 16 + c]);
            }
            szl[e] = v;
        }
    }
    // ---- stage the slice's rows of X (LDS-X mode): [M][slice k] + padding
    if constexpr (XLDS) {
        const int kc = (be - bb) * kBlockK / 8;  // 16-byte chunks per row
        for (int e = threadIdx.x; e < M * kc; e += WK * 64) {
            const int r = e / kc, c = e % kc;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(X + (size_t)r * K + (size_t)bb * kBlockK + c * 8);
            *reinterpret_cast<u32x4 *>(xl + r * L.x_stride + c * 16) = v;
        }
    }
    __syncthreads();

    if constexpr (XLDS) {
        while (b < we) {
            compute(b, b0);
            b += NB;
            if (b + NB < we) load(b + NB, b0);
            if (b >= we) break;
            compute(b, b1);
            b += NB;
            if (b + NB < we) load(b + NB, b1);
        }
    } else {
        if (b < we) load(b, b0);
        while (b < we) {
            if (b + NB < we) load(b + NB, b1);
            compute(b, b0);
            b += NB;
            if (b >= we) break;
            if (b + NB < we) load(b + NB, b0);
            compute(b, b1);
            b += NB;
        }
    }

    // ---- add the WK partial tiles of each strip in LDS, run 0 first
    __syncthreads();  // every wave is done with the staged X
    floatx4 *red = reinterpret_cast<floatx4 *>(xl);  // [WK][NS][MT][64]
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[((wk * NS + j) * MT + mt) * 64 + lane] = acc[mt][j];
    __syncthreads();

    const int rows = M < MT * 16 ? M : MT * 16;
    const int outs = rows * NS * 16;
    for (int o = threadIdx.x; o < outs; o += WK * 64) {
        const int r = o / (NS * 16), c = o % (NS * 16);
        const int j = c >> 4, cl = c & 15, mt = r >> 4, rr = r & 15;
        const int ln = (rr >> 2) * 16 + cl, e = rr & 3;
        const int sj = strip0 + j;
        if (sj >= nstrip) continue;
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < WK; ++q) v += red[((q * NS + j) * MT + mt) * 64 + ln][e];
        const size_t n = (size_t)sj * kStripCols + cl;
        if (S == 1)
            Y[(size_t)r * N + n] = f32_to_f16_bits(v);
        else
            part[((size_t)split * M + r) * N + n] = v;
    }
}

// Y = sum over s of part[s] (split order), fp32 -> fp16.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float *__restrict__ part, uint16_t *__restrict__ Y, int64_t MN, int S) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < MN;
         i += (int64_t)gridDim.x * blockDim.x) {
        float v = 0.f;
        for (int s = 0; s < S; ++s) v += part[(size_t)s * MN + i];
        Y[i] = f32_to_f16_bits(v);
    }
}

inline int decode_mt(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

// ---------------------------------------------------------------- planning
constexpr uint32_t kLdsBudget = 64 * 1024;

struct Plan {
    int mt, ns, wk;
    bool xlds;
    bool fixed_splits;  // automatic plan keeps K unsplit
    int splits, slice_blocks;
};

int env_int(const char *name, int dflt) {
    const char *v = getenv(name);
    return v ? atoi(v) : dflt;
}

// Launch shape. LDS-staged X with one strip per wave for M <= 4; for
// larger M register X shared by NS strips per wave, the shape picked from
// measurements on MI355X over the Llama-3-8B/70B decode matrices: narrow N
// with short K (QKV-like) runs best unsplit with 2 strips x 16 waves, the
// rest with 4 strips x 8 waves and K split across workgroups where N is
// narrow. W4A16_DECODE_NS and W4A16_DECODE_WK override NS and WK for tuning
// (instantiated values only).
Plan base_plan(int M, int N, int K) {
    Plan p;
    p.mt = decode_mt(M);
    p.xlds = M <= 4;
    const int nstrip = N / kStripCols, nblk = K / kBlockK;
    const bool short_narrow = nstrip <= 384 && nblk <= 64;
    if (p.xlds) {
        p.ns = 1;
        p.wk = nstrip < 512 ? 16 : 8;
    } else if (short_narrow) {
        p.ns = 2;
        p.wk = p.mt == 1 ? 16 : 8;
    } else {
        p.ns = (M <= 8 && nstrip >= 2048) ? 2 : 4;
        p.wk = 8;
    }
    if (p.mt == 4) p.ns = 2;
    p.fixed_splits = !p.xlds && short_narrow;
    const int ens = env_int("W4A16_DECODE_NS", 0), ewk = env_int("W4A16_DECODE_WK", 0);
    if (ens == 1 || ens == 2 || ens == 4) p.ns = ens;
    if (p.mt == 4 && p.ns == 4) p.ns = 2;
    if (ewk == 4 || ewk == 8 || (ewk == 16 && p.mt == 1)) p.wk = ewk;
    // the cross-wave reduction buffer must leave room for the staged records
    while (p.wk * p.ns * p.mt * 64 * 16 > 32 * 1024 && p.wk > 4) p.wk /= 2;
    while (p.wk * p.ns * p.mt * 64 * 16 > 32 * 1024 && p.ns > 1) p.ns /= 2;
    p.splits = 1;
    p.slice_blocks = 0;
    return p;
}

// Blocks per split for a split count: whole groups per slice.
int slice_for(int K, int G, int splits) {
    const int nblk = K / kBlockK;
    const int unit = G > kBlockK ? G / kBlockK : 1;
    int sb = (nblk + splits - 1) / splits;
    return (sb + unit - 1) / unit * unit;
}

bool lds_fits(const Plan &p, int M, int G, int slice_blocks) {
    return decode_lds(M, p.mt, p.ns, p.wk, slice_blocks, G, p.xlds).total() <= kLdsBudget;
}

Plan make_plan(int M, int N, int K, int G, int splits, int num_cus) {
    Plan p = base_plan(M, N, K);
    const int nblk = K / kBlockK;
    const int tiles = (N / kStripCols + p.ns - 1) / p.ns;
    if (splits <= 0 && p.fixed_splits) splits = 1;
    if (splits <= 0) {
        // Narrow N: about two workgroups per CU, keeping two blocks per wave.
        splits = 1;
        if (tiles < num_cus) {
            splits = (2 * num_cus + tiles - 1) / tiles;
            int cap = nblk / (2 * p.wk);
            if (cap < 1) cap = 1;
            if (splits > cap) splits = cap;
        }
    }
    // enough splits for the LDS budget (also raises a requested count)
    while (splits < nblk && !lds_fits(p, M, G, slice_for(K, G, splits))) ++splits;
    p.slice_blocks = slice_for(K, G, splits);
    p.splits = (nblk + p.slice_blocks - 1) / p.slice_blocks;
    return p;
}

template <int MT, int NS, int WK, int GS, bool XLDS>
hipError_t launch_one(const uint16_t *X, const uint8_t *packed, int M, int N, int K, uint16_t *Y,
                      float *part, const Plan &p, hipStream_t stream) {
    constexpr int NB = (NS == 1 && MT == 1) ? 2 : 1;
    const DecodeLds L = decode_lds(M, MT, NS, WK, p.slice_blocks, 32 * GS, XLDS);
    const int tiles = (N / kStripCols + NS - 1) / NS;
    hipLaunchKernelGGL((decode_kernel<MT, NS, WK, NB, GS, XLDS>), dim3(tiles, p.splits), dim3(WK * 64),
                       L.total(), stream, X, packed, Y, part, M, N, K, p.splits, p.slice_blocks);
    return hipGetLastError();
}

template <int MT, int NS, int WK, bool XLDS>
hipError_t launch_g(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G, uint16_t *Y,
                    float *part, const Plan &p, hipStream_t stream) {
    switch (G) {
        case 32: return launch_one<MT, NS, WK, 1, XLDS>(X, packed, M, N, K, Y, part, p, stream);
        case 64: return launch_one<MT, NS, WK, 2, XLDS>(X, packed, M, N, K, Y, part, p, stream);
        case 128: return launch_one<MT, NS, WK, 4, XLDS>(X, packed, M, N, K, Y, part, p, stream);
        case 256: return launch_one<MT, NS, WK, 8, XLDS>(X, packed, M, N, K, Y, part, p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int MT, int NS, bool XLDS>
hipError_t launch_wk(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G, uint16_t *Y,
                     float *part, const Plan &p, hipStream_t stream) {
    if constexpr (MT == 1) {
        if (p.wk == 16) return launch_g<MT, NS, 16, XLDS>(X, packed, M, N, K, G, Y, part, p, stream);
    }
    if (p.wk == 4) return launch_g<MT, NS, 4, XLDS>(X, packed, M, N, K, G, Y, part, p, stream);
    return launch_g<MT, NS, 8, XLDS>(X, packed, M, N, K, G, Y, part, p, stream);
}

hipError_t launch_plan(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G, uint16_t *Y,
                       float *part, const Plan &p, hipStream_t stream) {
    if (p.xlds) {  // M <= 4
        switch (p.ns) {
            case 1: return launch_wk<1, 1, true>(X, packed, M, N, K, G, Y, part, p, stream);
            case 2: return launch_wk<1, 2, true>(X, packed, M, N, K, G, Y, part, p, stream);
            default: return launch_wk<1, 4, true>(X, packed, M, N, K, G, Y, part, p, stream);
        }
    }
    switch (p.mt) {
        case 1:
            switch (p.ns) {
                case 1: return launch_wk<1, 1, false>(X, packed, M, N, K, G, Y, part, p, stream);
                case 2: return launch_wk<1, 2, false>(X, packed, M, N, K, G, Y, part, p, stream);
                default: return launch_wk<1, 4, false>(X, packed, M, N, K, G, Y, part, p, stream);
            }
        case 2:
            switch (p.ns) {
                case 1: return launch_wk<2, 1, false>(X, packed, M, N, K, G, Y, part, p, stream);
                case 2: return launch_wk<2, 2, false>(X, packed, M, N, K, G, Y, part, p, stream);
                default: return launch_wk<2, 4, false>(X, packed, M, N, K, G, Y, part, p, stream);
            }
        default:
            switch (p.ns) {
                case 1: return launch_wk<4, 1, false>(X, packed, M, N, K, G, Y, part, p, stream);
                default: return launch_wk<4, 2, false>(X, packed, M, N, K, G, Y, part, p, stream);
            }
    }
}

}  // namespace

int decode_max_splits(int M, int N, int K) {
    (void)M;
    (void)N;
    return K / kBlockK;
}

int decode_auto_splits(int M, int N, int K, int G, int num_cus) {
    return make_plan(M, N, K, G, 0, num_cus).splits;
}

size_t decode_workspace_bytes(int M, int N, int K, int G, int splits) {
    // a requested split count is rounded to whole groups per slice and
    // raised until the slice fits the LDS budget
    const Plan p = make_plan(M, N, K, G, splits, 256);
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_decode(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G,
                         uint16_t *Y, void *workspace, int splits, int num_cus, hipStream_t stream) {
    const Plan p = make_plan(M, N, K, G, splits, num_cus);
    if (!lds_fits(p, M, G, p.slice_blocks)) return hipErrorInvalidConfiguration;
    float *part = p.splits > 1 ? static_cast<float *>(workspace) : nullptr;
    hipError_t e = launch_plan(X, packed, M, N, K, G, Y, part, p, stream);
    if (e != hipSuccess || p.splits <= 1) return e;
    const int64_t MN = (int64_t)M * N;
    int64_t blocks = (MN + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, Y, MN,
                       p.splits);
    return hipGetLastError();
}

}  // namespace w4a16
