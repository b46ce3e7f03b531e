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
typedef __attribute__((address_space(3))) void lds_void;  // LDS pointer for direct buffer loads

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

// -(1024 + z) and -(1024 + 16 z) as fp16 pairs: 1024 + z is exponent 10
// with z in the low mantissa bits (0x6400 | z), 1024 + 16 z puts z four bits
// higher; the sign bit makes them negative.
__device__ inline uint32_t neg_bias_pair(uint32_t sz) {
    uint32_t h = 0xE400u | (sz >> 16);
    return h | (h << 16);
}
__device__ inline uint32_t neg_bias16_pair(uint32_t sz) {
    uint32_t h = 0xE400u | ((sz >> 16) << 4);
    return h | (h << 16);
}

__device__ inline float scale_of(uint32_t sz) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(sz & 0xFFFFu));
}

// (x & mask) | magic in one VALU op. gfx9 VOP3 reads at most one scalar
// operand, so the mask goes in an SGPR and the magic number in a VGPR.
__device__ inline uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic));
    return r;
}

// Exponent-OR conversion: a half with exponent field 10 (0x6400) and a code
// c in its low mantissa bits is exactly 1024 + c, so OR-ing the code into
// 0x6400 converts it to fp16 without an integer-to-float instruction. Codes
// sitting four bits higher give 1024 + 16 c, also exact.
constexpr uint32_t kMagic = 0x64006400u;
constexpr uint32_t kLoMask = 0x000F000Fu;
constexpr uint32_t kHiMask = 0x00F000F0u;

__device__ inline half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }

__device__ inline half8 pack_h8(half2v r0, half2v r1, half2v r2, half2v r3) {
    half8 out;
    out[0] = r0[0]; out[1] = r0[1]; out[2] = r1[0]; out[3] = r1[1];
    out[4] = r2[0]; out[5] = r2[1]; out[6] = r3[0]; out[7] = r3[1];
    return out;
}

// One lane's 16-byte slice of a packed tile holds four words; word v carries
// the k pair (2v, 2v+1) of each of the four 32-row steps of the tile: steps
// 0 and 1 in the low nibble of bytes 0/2 and 1/3, steps 2 and 3 in their high
// nibble (see the layout in include/w4a16.h).
//
// B operand of exact integers for step T: (q - z) for T = 0, 1 and 16 (q - z)
// for T = 2, 3 (the caller folds the 1/16 into the scale). (1024 + q) -
// (1024 + z) and (1024 + 16 q) - (1024 + 16 z) are exact in fp16 (all
// operands in [1024, 1264]). w8[v] = w[v] >> 8, computed once per word.
template <int T>
__device__ inline half8 dequant_qz_step(const u32x4 &w, const u32x4 &w8, uint32_t nb_lo,
                                        uint32_t nb_hi, uint32_t magic) {
    const uint32_t mask = (T < 2) ? kLoMask : kHiMask;
    const uint32_t nb = (T < 2) ? nb_lo : nb_hi;
    half2v r[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const uint32_t src = (T & 1) ? w8[v] : w[v];
        r[v] = as_h2(and_or(src, mask, magic)) + as_h2(nb);
    }
    return pack_h8(r[0], r[1], r[2], r[3]);
}

// B operand of fp16 weights for step T: ((1024 + q) - (1024 + z)) * s, the
// exact q - z rounded once to fp16 by the multiply with s.
template <int T>
__device__ inline half8 dequant_w_step(const u32x4 &w, uint32_t nb_lo, uint32_t s2, uint32_t magic) {
    constexpr int shift = T == 0 ? 0 : (T == 1 ? 8 : (T == 2 ? 4 : 12));
    half2v r[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const uint32_t src = shift ? (w[v] >> shift) : w[v];
        r[v] = (as_h2(and_or(src, kLoMask, magic)) + as_h2(nb_lo)) * as_h2(s2);
    }
    return pack_h8(r[0], r[1], r[2], r[3]);
}

// Runtime-step dispatch for code that loops over steps.
__device__ inline half8 dequant_w(int t, const u32x4 &w, uint32_t nb_lo, uint32_t s2, uint32_t magic) {
    switch (t) {
        case 0: return dequant_w_step<0>(w, nb_lo, s2, magic);
        case 1: return dequant_w_step<1>(w, nb_lo, s2, magic);
        case 2: return dequant_w_step<2>(w, nb_lo, s2, magic);
        default: return dequant_w_step<3>(w, nb_lo, s2, magic);
    }
}
__device__ inline half8 dequant_qz(int t, const u32x4 &w, const u32x4 &w8, uint32_t nb_lo,
                                   uint32_t nb_hi, uint32_t magic) {
    switch (t) {
        case 0: return dequant_qz_step<0>(w, w8, nb_lo, nb_hi, magic);
        case 1: return dequant_qz_step<1>(w, w8, nb_lo, nb_hi, magic);
        case 2: return dequant_qz_step<2>(w, w8, nb_lo, nb_hi, magic);
        default: return dequant_qz_step<3>(w, w8, nb_lo, nb_hi, magic);
    }
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

// A raw buffer load whose offset reaches past the descriptor's byte count
// returns zeros and makes no memory request. Kernels point loads they do not
// need at this offset instead of branching around them, so every path
// through a loop issues the same loads and the compiler can wait for exactly
// the batch it consumes.
constexpr uint32_t kOobOffset = 0x80000000u;

// Buffer resource over [base, base + bytes) for raw buffer loads (gfx9
// descriptor: stride 0, 32-bit data format word).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

}  // namespace w4a16
