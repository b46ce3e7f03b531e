// Group-wise asymmetric 4-bit quantizer: fp16 weights W[K][N] -> codes q,
// one fp16 scale s and one 4-bit zero z per group of G rows along K and per
// column, written either as plain arrays or straight into the packed layout
// the GEMM reads.
//
// This is the step before packing. The pages quantize weights to uniform
// 4-bit codes in groups of 128 with a scale per group ("LMDeploy, in depth",
// section "Quantization: AWQ weights and KV cache", paragraph "Weight
// quantization (W4A16)"), dequantized as FP16 = (INT4 - ZeroPoint) x Scale
// ("LMDeploy Guide: Fast Mixed-Precision LLM Inference Engine", section 3),
// and call the plain form round-to-nearest ("LMDeploy" interview notes, the
// answer on AWQ versus naive RTN INT4). The scale and zero follow the plain
// asymmetric reading: the group's range [min, max] spread over 15 steps, and
// every weight goes to the code nearest to it.
//   s   = fp16(max(fp32(fp32(max - min) / 15), 2^-14))
//   z   = clamp(rint(-min / s), 0, 15)
//   q   = clamp(rint(w / s) + z, 0, 15)
// rint is the nearest integer to the exact quotient, ties to even. A group
// whose codes dequantize beyond fp16 (|(q - z) s| >= 65520) has no valid
// encoding and sets the status word, as a non-finite weight does.
//
// One pass over W, bound by HBM: a workgroup stages a KB x CB tile of W in
// LDS (KB = max(128, G) rows, CB columns), takes each column's group minimum
// and maximum with packed fp16 min/max over row slices, turns them into
// (s, 1/s, z) per group and column (z and the range check by float64
// division, which decides rint exactly for these operands), and then either
//   - packed output: each wave builds the 1 KiB tiles of its 16-column
//     strips (one 16-byte store per lane, the bytes the GEMM's lane loads)
//     and the scale and zero records, or
//   - plain output: q[K][N] (one byte per code), z[K/G][N], s[K/G][N].
//
// Code decision per weight (code_float below). Adding 1.5 * 2^23 in float32
// rounds any |x| < 2^22 to an integer with ties to even, so
// y = fma(w, fp32(1/s), 1.5 * 2^23) is 1.5 * 2^23 + c with c the exact
// product w * fp32(1/s) rounded once. With w = a 2^x and s = b 2^y (a, b
// below 2^11, s normal), a quotient w / s that is not a half-integer lies at
// least 2^-12 from every half-integer, and |w * fp32(1/s) - w / s| <=
// |w / s| 2^-24 < 2^-12 wherever the code is not saturated (|w / s| < 2^12),
// so c = rint(w / s) except at an exact tie, where the inexact reciprocal
// may land on either side. The residual w - c s is exact in float32 there
// (at most 12 significant bits above the lower of the two exponents), equals
// +-s/2 exactly at a tie, and then the even neighbour of c wins. y is then
// clamped to [1.5 * 2^23 - z, 1.5 * 2^23 - z + 15]; in that binade the
// float's bit pattern is bits(1.5 * 2^23) - z + code, so the packed word is
// the sum of bits(y) << shift over its eight nibbles plus one per-lane
// constant that removes bits(1.5 * 2^23) - z from every nibble (all modulo
// 2^32, the nibbles never carry into each other).
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

constexpr int kQThreads = 256;

// Per (group, column) parameters of the code decision.
struct QParams {
    float inv;     // fp32(1 / s)
    float lo;      // 1.5 * 2^23 - z
    float hi;      // lo + 15
    uint32_t zb;   // z - bits(1.5 * 2^23)
    float s;       // the stored scale, in float32
};

// 1.5 * 2^23 + clamp(rint(w / s) + z, 0, 15) as a float (w and s are fp16
// values: the corrected reciprocal product decides rint of the exact
// quotient, ties to even)
__device__ inline float code_float(float w, const QParams &p) {
    return __builtin_amdgcn_fmed3f(round_quotient_fp16(w, p.s, p.inv), p.lo, p.hi);
}

template <int KB, int CB>
struct QuantGeom {
    static constexpr int kStride = CB * 2 + 16;           // bytes per staged row
    static constexpr int kChunks = CB / 8;                // 16-byte chunks per row
    static constexpr int kLoads = KB * kChunks / kQThreads;
    static constexpr int kPairs = CB / 2;                 // column pairs
    static constexpr int kSlices = kQThreads / kPairs;    // row slices of the range pass
    static constexpr int kSliceRows = KB / kSlices;
    static_assert(kLoads * kQThreads == KB * kChunks, "tile load split");
};

__device__ inline uint32_t nibble_shift(int t, int e) { return 4u * (4 * e + 2 * (t & 1) + (t >> 1)); }

template <int GS, int CB, bool PACKED>
__global__ void __launch_bounds__(kQThreads)
quantize_kernel(const uint16_t *__restrict__ W, int K, int N, uint8_t *__restrict__ packed,
                uint8_t *__restrict__ qout, uint8_t *__restrict__ zout, uint16_t *__restrict__ sout,
                int *__restrict__ bad, int tpb) {
    constexpr int G = 32 * GS;
    constexpr int KB = G > kBlockK ? G : kBlockK;
    constexpr int NGK = KB / G;  // groups in the tile's rows
    typedef QuantGeom<KB, CB> Geo;
    static_assert(G % Geo::kSliceRows == 0, "a row slice lies inside one group");
    __shared__ __attribute__((aligned(16))) uint8_t tile[KB * Geo::kStride];
    __shared__ uint32_t pmax[Geo::kSlices][Geo::kPairs];
    __shared__ uint32_t pmin[Geo::kSlices][Geo::kPairs];
    __shared__ __attribute__((aligned(16))) QParams prm[NGK][CB];
    __shared__ uint8_t zl[NGK][CB];

    const int tid = threadIdx.x;
    const int c0 = blockIdx.x * CB;  // first column of the tiles
    const int ngrp = K / G;
    const int kt_end = min((int)(blockIdx.y + 1) * tpb, K / KB);

    // Tiles kt = blockIdx.y * tpb .. kt_end - 1 of this column range, one
    // after the other; the 16-byte row-chunk loads of the next tile are in
    // flight while the current one is quantized. Chunks past N read zeros
    // (N % 16 == 0, so a chunk of 8 columns is all in or all out).
    u32x4 v[Geo::kLoads];
    auto issue = [&](int kt) {
        const __amdgpu_buffer_rsrc_t rw =
            make_rsrc(W + (size_t)kt * KB * N + c0, (uint32_t)((size_t)KB * N * 2));
#pragma unroll
        for (int i = 0; i < Geo::kLoads; ++i) {
            const int idx = i * kQThreads + tid;
            const int r = idx / Geo::kChunks, ch = idx % Geo::kChunks;
            const bool ok = c0 + ch * 8 < N;
            v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rw, ok ? (uint32_t)(r * N * 2 + ch * 16) : kOobOffset, 0, 0));
        }
    };
    issue(blockIdx.y * tpb);
    for (int kt = blockIdx.y * tpb; kt < kt_end; ++kt) {
        const int k0 = kt * KB;  // first row of the tile
        // ---- stage the tile in LDS, then send the next tile's loads
#pragma unroll
        for (int i = 0; i < Geo::kLoads; ++i) {
            const int idx = i * kQThreads + tid;
            const int r = idx / Geo::kChunks, ch = idx % Geo::kChunks;
            *reinterpret_cast<u32x4 *>(tile + r * Geo::kStride + ch * 16) = v[i];
        }
        if (kt + 1 < kt_end) issue(kt + 1);
        __syncthreads();

        // ---- range pass: thread = (column pair, row slice); packed fp16
        // maximum/minimum, which propagate NaN (three-input forms on gfx950),
        // so a non-finite weight shows up in its group's range
        {
            const int cp = tid % Geo::kPairs, sl = tid / Geo::kPairs;
            const uint8_t *p = tile + sl * Geo::kSliceRows * Geo::kStride + cp * 4;
            half2v mx = __builtin_bit_cast(half2v, *reinterpret_cast<const uint32_t *>(p));
            half2v mn = mx;
#pragma unroll
            for (int r = 1; r < Geo::kSliceRows; ++r) {
                const half2v x = __builtin_bit_cast(half2v, *reinterpret_cast<const uint32_t *>(p + r * Geo::kStride));
                mx = __builtin_elementwise_maximum(mx, x);
                mn = __builtin_elementwise_minimum(mn, x);
            }
            pmax[sl][cp] = __builtin_bit_cast(uint32_t, mx);
            pmin[sl][cp] = __builtin_bit_cast(uint32_t, mn);
        }
        __syncthreads();

        // ---- scale, reciprocal and zero per (group, column)
        for (int it = tid; it < NGK * CB; it += kQThreads) {
            const int g = it / CB, c = it % CB;
            constexpr int per = G / Geo::kSliceRows;  // slices per group
            float wmax = (float)__builtin_bit_cast(half2v, pmax[g * per][c >> 1])[c & 1];
            float wmin = (float)__builtin_bit_cast(half2v, pmin[g * per][c >> 1])[c & 1];
#pragma unroll
            for (int q = 1; q < per; ++q) {
                const int sl = g * per + q;
                wmax = __builtin_elementwise_maximum(wmax, (float)__builtin_bit_cast(half2v, pmax[sl][c >> 1])[c & 1]);
                wmin = __builtin_elementwise_minimum(wmin, (float)__builtin_bit_cast(half2v, pmin[sl][c >> 1])[c & 1]);
            }
            if (!__builtin_isfinite(wmax) || !__builtin_isfinite(wmin)) *bad = 1;
            // s = fp16(max(fp32(max - min) / 15, 2^-14)): the division in
            // three operations (correctly rounded for every float32
            // difference of fp16 numbers)
            const float s32 = __builtin_fmaxf(div_steps(wmax - wmin, 15.0f, 1.0f / 15.0f), kScaleFloor);
            const _Float16 s16 = (_Float16)s32;
            const float sf = (float)s16;
            QParams pr;
            pr.inv = __builtin_amdgcn_rcpf(sf);  // one ulp is within what the code decision allows
            // z = clamp(rint(-min / s), 0, 15), decided like the codes (the
            // operands are fp16); the codes are monotone in w, so the
            // group's extremes bound |q - z| for the fp16 range check
            const float zf = __builtin_amdgcn_fmed3f(round_quotient_fp16(-wmin, sf, pr.inv), kRoundMagic,
                                                     kRoundMagic + 15.0f);
            const int z = (int)(__builtin_bit_cast(uint32_t, zf) - kRoundMagicBits);
            pr.lo = kRoundMagic - (float)z;
            pr.hi = pr.lo + 15.0f;
            pr.zb = (uint32_t)z - kRoundMagicBits;
            pr.s = sf;
            const int qlo = (int)(__builtin_bit_cast(uint32_t, code_float(wmin, pr)) - kRoundMagicBits);  // q - z
            const int qhi = (int)(__builtin_bit_cast(uint32_t, code_float(wmax, pr)) - kRoundMagicBits);
            const int dmax = qlo < 0 ? (-qlo > qhi ? -qlo : qhi) : qhi;
            if (!((float)dmax * sf < 65520.0f)) *bad = 1;
            prm[g][c] = pr;
            zl[g][c] = (uint8_t)z;
            const int n = c0 + c;
            if (n < N) {
                const int gg = k0 / G + g;
                if constexpr (PACKED) {
                    uint16_t *srec = reinterpret_cast<uint16_t *>(packed + weight_bytes(K, N));
                    srec[((size_t)(n / kStripCols) * ngrp + gg) * kStripCols + n % kStripCols] =
                        __builtin_bit_cast(uint16_t, s16);
                } else {
                    sout[(size_t)gg * N + n] = __builtin_bit_cast(uint16_t, s16);
                    zout[(size_t)gg * N + n] = (uint8_t)z;
                }
            }
        }
        __syncthreads();

        if constexpr (PACKED) {
            // zero records: two columns per byte, low nibble for the even one
            uint8_t *zrec = packed + weight_bytes(K, N) + scale_bytes(K, N, G);
            for (int it = tid; it < NGK * CB / 2; it += kQThreads) {
                const int g = it / (CB / 2), c = 2 * (it % (CB / 2));
                const int n = c0 + c;
                if (n < N)
                    zrec[((size_t)(n / kStripCols) * ngrp + k0 / G + g) * 8 + (n % kStripCols) / 2] =
                        (uint8_t)(zl[g][c] | (zl[g][c + 1] << 4));
            }
            // weight tiles: wave w builds the tiles of strips w, w + 4, ... of
            // the tile's columns, block by block
            const int lane = tid & 63, wave = tid >> 6;
            const int cl = lane & 15, kq = lane >> 4;
            const int nblk = K / kBlockK;
            for (int st = wave; st < CB / kStripCols; st += kQThreads / 64) {
                const int strip = c0 / kStripCols + st;
                if (strip * kStripCols >= N) break;
                const int c = st * kStripCols + cl;
#pragma unroll
                for (int bl = 0; bl < KB / kBlockK; ++bl) {
                    uint32_t word[4];
                    uint32_t base = 0;
                    QParams pt[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        pt[t] = prm[(bl * kBlockK + 32 * t) / G][c];
                        base += pt[t].zb * ((1u << nibble_shift(t, 0)) + (1u << nibble_shift(t, 1)));
                    }
#pragma unroll
                    for (int w = 0; w < 4; ++w) word[w] = base;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const uint8_t *src = tile + (bl * kBlockK + 32 * t + 8 * kq) * Geo::kStride + c * 2;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const _Float16 h = *reinterpret_cast<const _Float16 *>(src + j * Geo::kStride);
                            const float y = code_float((float)h, pt[t]);
                            word[j >> 1] += __builtin_bit_cast(uint32_t, y) << nibble_shift(t, j & 1);
                        }
                    }
                    u32x4 out = {word[0], word[1], word[2], word[3]};
                    *reinterpret_cast<u32x4 *>(packed + ((size_t)strip * nblk + k0 / kBlockK + bl) * kTileBytes +
                                               lane * 16) = out;
                }
            }
        } else {
            // plain codes: thread item = (row, 16 columns), one 16-byte store
            constexpr int kItems = KB * CB / 16;
            for (int it = tid; it < kItems; it += kQThreads) {
                const int r = it / (CB / 16), cc = (it % (CB / 16)) * 16;
                if (c0 + cc >= N) continue;
                const int g = r / G;
                const uint8_t *src = tile + r * Geo::kStride + cc * 2;
                u32x4 out;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint32_t word = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int c = cc + 4 * d + b;
                        const QParams pr = prm[g][c];
                        const _Float16 h = *reinterpret_cast<const _Float16 *>(src + (4 * d + b) * 2);
                        const float y = code_float((float)h, pr);
                        word |= ((__builtin_bit_cast(uint32_t, y) + pr.zb) & 15u) << (8 * b);
                    }
                    out[d] = word;
                }
                *reinterpret_cast<u32x4 *>(qout + (size_t)(k0 + r) * N + c0 + cc) = out;
            }
        }
        __syncthreads();  // the next tile overwrites the LDS tile and parameters
    }
}

template <int GS, bool PACKED>
hipError_t launch_gs(const uint16_t *W, int K, int N, int cb, uint8_t *packed, uint8_t *q, uint8_t *z,
                     uint16_t *s, int *bad, hipStream_t stream) {
    constexpr int KB = 32 * GS > kBlockK ? 32 * GS : kBlockK;
    const int tiles = K / KB;
    if (cb == 256 && !(GS == 2 || GS == 4)) cb = 128;  // 256-column tiles need 64-row range slices
    const int gx = (N + cb - 1) / cb;
    // tiles per workgroup: one (measured fastest on the 8192 x 57344 weight;
    // the pipelined loop is kept for other devices and shapes, via the knob)
    int tpb = 1;
    if (const char *e = getenv("W4A16_QUANTIZE_TPB")) tpb = atoi(e) > 0 ? atoi(e) : 1;
    const unsigned gy = (unsigned)((tiles + tpb - 1) / tpb);
    if constexpr (GS == 2 || GS == 4) {
        if (cb == 256) {
            hipLaunchKernelGGL((quantize_kernel<GS, 256, PACKED>), dim3((unsigned)gx, gy), dim3(kQThreads), 0,
                               stream, W, K, N, packed, q, z, s, bad, tpb);
            return hipGetLastError();
        }
    }
    if (cb == 128) {
        hipLaunchKernelGGL((quantize_kernel<GS, 128, PACKED>), dim3((unsigned)gx, gy), dim3(kQThreads), 0,
                           stream, W, K, N, packed, q, z, s, bad, tpb);
    } else {
        hipLaunchKernelGGL((quantize_kernel<GS, 64, PACKED>), dim3((unsigned)gx, gy), dim3(kQThreads), 0,
                           stream, W, K, N, packed, q, z, s, bad, tpb);
    }
    return hipGetLastError();
}

template <bool PACKED>
hipError_t launch_mode(const uint16_t *W, int K, int N, int G, uint8_t *packed, uint8_t *q, uint8_t *z,
                       uint16_t *s, int *bad, hipStream_t stream) {
    // 128 columns: 256-byte row segments (a read-only probe of this access
    // pattern on the 8192 x 57344 weight: 225 us against 240 us for 64).
    // 256 columns (G = 64, 128; W4A16_QUANTIZE_CB=256) measured 3% faster
    // on that weight (264-268 against 274-276 us) but slower on smaller
    // ones (4096 x 28672: 75-76 against 71-73 us; 4096 x 14336, G = 64: 53
    // against 46 us), with half as many workgroups.
    int cb = 128;
    if (const char *e = getenv("W4A16_QUANTIZE_CB")) cb = atoi(e) == 64 ? 64 : (atoi(e) == 256 ? 256 : 128);
    switch (G) {
        case 32: return launch_gs<1, PACKED>(W, K, N, cb, packed, q, z, s, bad, stream);
        case 64: return launch_gs<2, PACKED>(W, K, N, cb, packed, q, z, s, bad, stream);
        case 128: return launch_gs<4, PACKED>(W, K, N, cb, packed, q, z, s, bad, stream);
        case 256: return launch_gs<8, PACKED>(W, K, N, cb, packed, q, z, s, bad, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_quantize(const uint16_t *W, int K, int N, int G, uint8_t *q, uint8_t *z, uint16_t *s,
                           int *bad, hipStream_t stream) {
    return launch_mode<false>(W, K, N, G, nullptr, q, z, s, bad, stream);
}

hipError_t launch_quantize_pack(const uint16_t *W, int K, int N, int G, uint8_t *packed, int *bad,
                                hipStream_t stream) {
    return launch_mode<true>(W, K, N, G, packed, nullptr, nullptr, nullptr, bad, stream);
}

}  // namespace w4a16
