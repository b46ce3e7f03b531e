// Device-side building blocks shared by the W4A16 kernels (gfx950 only).
//
// Internal header: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Geometry of the packed weight tiles: 16 output columns ("strip") by 128
// rows of K ("block") = 1024 bytes, read by one wave64 as 16 bytes per lane.
constexpr int kStripCols = 16;
constexpr int kBlockK = 128;
constexpr int kTileBytes = 1024;

// Offsets of the three regions of a packed buffer.
struct PackedView {
    const u32x4 *w;       // [N/16][K/128][64 lanes] of 16 bytes
    const uint16_t *s;    // [N/16][K/G][16] fp16 scales
    const uint8_t *z;     // [N/16][K/G][8] two 4-bit zeros per byte
};

__host__ __device__ inline size_t weight_bytes(int64_t K, int64_t N) { return (size_t)(K * N / 2); }
__host__ __device__ inline size_t scale_bytes(int64_t K, int64_t N, int64_t G) { return (size_t)(2 * N * (K / G)); }
__host__ __device__ inline size_t zero_bytes(int64_t K, int64_t N, int64_t G) { return (size_t)(N * (K / G) / 2); }

__device__ inline PackedView packed_view(const uint8_t *p, int K, int N, int G) {
    PackedView v;
    v.w = reinterpret_cast<const u32x4 *>(p);
    v.s = reinterpret_cast<const uint16_t *>(p + weight_bytes(K, N));
    v.z = p + weight_bytes(K, N) + scale_bytes(K, N, G);
    return v;
}

// Scale bits and zero code of (strip, group) for column `col` of the strip,
// combined into one word: bits 0..15 fp16 scale, bits 16..19 zero code.
__device__ inline uint32_t load_scale_zero(const PackedView &pv, size_t rec, int col) {
    uint32_t sc = pv.s[rec * 16 + col];
    uint32_t zc = (pv.z[rec * 8 + (col >> 1)] >> ((col & 1) * 4)) & 15u;
    return sc | (zc << 16);
}

// -(1024 + z) as an fp16 pair: 1024 + z is exponent 10 with z in the low
// mantissa bits (0x6400 | z); the sign bit makes it negative.
__device__ inline uint32_t neg_bias_pair(uint32_t sz) {
    uint32_t h = 0xE400u | (sz >> 16);
    return h | (h << 16);
}

__device__ inline float scale_of(uint32_t sz) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(sz & 0xFFFFu));
}

// Eight 4-bit codes of one packed word -> four fp16 pairs holding 1024 + q.
// Setting the exponent field of a half to 10 (0x6400) and OR-ing the code
// into the low mantissa bits gives exactly 1024 + q without any
// integer-to-float conversion instruction. Nibble slots are ordered so that
// shift i and the mask 0x000F000F yield the codes of k = 2i and 2i + 1.
__device__ inline void biased_halves(uint32_t w, uint32_t h[4]) {
    h[0] = (w & 0x000F000Fu) | 0x64006400u;
    h[1] = ((w >> 4) & 0x000F000Fu) | 0x64006400u;
    h[2] = ((w >> 8) & 0x000F000Fu) | 0x64006400u;
    h[3] = ((w >> 12) & 0x000F000Fu) | 0x64006400u;
}

__device__ inline half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }
__device__ inline uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }

// B operand (8 halves) of exact integers q - z for one packed word:
// (1024 + q) - (1024 + z) is exact in fp16 (both in [1024, 1040)).
__device__ inline half8 dequant_qz(uint32_t w, uint32_t nb2) {
    uint32_t h[4];
    biased_halves(w, h);
    half2v nb = as_h2(nb2);
    half2v r0 = as_h2(h[0]) + nb, r1 = as_h2(h[1]) + nb, r2 = as_h2(h[2]) + nb, r3 = as_h2(h[3]) + nb;
    half8 out;
    out[0] = r0[0]; out[1] = r0[1]; out[2] = r1[0]; out[3] = r1[1];
    out[4] = r2[0]; out[5] = r2[1]; out[6] = r3[0]; out[7] = r3[1];
    return out;
}

// B operand of fp16 weights (q - z) * s, rounded once to nearest-even.
__device__ inline half8 dequant_w(uint32_t w, uint32_t nb2, uint32_t s2) {
    uint32_t h[4];
    biased_halves(w, h);
    half2v nb = as_h2(nb2), sc = as_h2(s2);
    half2v r0 = (as_h2(h[0]) + nb) * sc, r1 = (as_h2(h[1]) + nb) * sc;
    half2v r2 = (as_h2(h[2]) + nb) * sc, r3 = (as_h2(h[3]) + nb) * sc;
    half8 out;
    out[0] = r0[0]; out[1] = r0[1]; out[2] = r1[0]; out[3] = r1[1];
    out[4] = r2[0]; out[5] = r2[1]; out[6] = r3[0]; out[7] = r3[1];
    return out;
}

// D += A . B on a 16 x 16 output tile with K = 32 (fp16 in, fp32 accumulate).
// Lane l holds A[l % 16][8 (l / 16) .. +7], B[8 (l / 16) .. +7][l % 16] and
// D[4 (l / 16) + e][l % 16] for e = 0..3.
__device__ inline floatx4 mfma16x16x32(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

}  // namespace w4a16
