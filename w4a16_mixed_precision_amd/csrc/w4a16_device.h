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

__host__ __device__ inline size_t weight_bytes(int64_t K, int64_t N) { return (size_t)(K * N / 2); }
__host__ __device__ inline size_t scale_bytes(int64_t K, int64_t N, int64_t G) { return (size_t)(2 * N * (K / G)); }
__host__ __device__ inline size_t zero_bytes(int64_t K, int64_t N, int64_t G) { return (size_t)(N * (K / G) / 2); }

// (x & mask) | magic in one VALU op. gfx9 VOP3 reads at most one scalar
// operand, so the mask goes in an SGPR and the magic number in a VGPR.
__device__ inline uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic));
    return r;
}

// Exponent-OR conversion: a half with exponent field 10 (0x6400, the value
// 1024) has a mantissa unit of 1, so OR-ing a code c into its low four bits
// gives exactly 1024 + c without an integer-to-float instruction. With
// exponent 6 (0x5400, the value 64) the unit is 1/16, so a code sitting in
// bits 4..7 gives exactly 64 + c: the high nibble of a byte converts without
// a shift.
constexpr uint32_t kMagic = 0x64006400u;
constexpr uint32_t kMagic64 = 0x54005400u;
constexpr uint32_t kLoMask = 0x000F000Fu;
constexpr uint32_t kHiMask = 0x00F000F0u;

// -(64 + z) as an fp16 pair, from the pair -(1024 + z) (0xE400 | z): the z
// bits move up by four and the exponent becomes that of 64.
__device__ inline uint32_t neg_bias64_from_1024(uint32_t nb_lo) {
    return ((nb_lo & kLoMask) << 4) | 0xD400D400u;
}

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
// nibble (see the layout in include/w4a16.h). With w8[v] = w[v] >> 8 (once
// per word), step T reads its codes from (T odd ? w8 : w) under the low
// (T < 2) or high (T >= 2) nibble mask: one shift per word for all four
// steps.
//
// B operand of exact integers q - z for step T: (1024 + q) - (1024 + z) for
// the low nibbles, (64 + q) - (64 + z) for the high ones; both are exact in
// fp16 (operands in [1024, 1039] and [64, 79]).
struct DequantConsts {
    uint32_t nb_lo;  // -(1024 + z) pair
    uint32_t nb_hi;  // -(64 + z) pair
    uint32_t m_lo;   // kMagic, in a VGPR (gfx9 VOP3 reads one scalar operand)
    uint32_t m_hi;   // kMagic64, likewise
};

template <int T>
__device__ inline half2v dequant_pair(const u32x4 &w, const u32x4 &w8, int v, const DequantConsts &c) {
    const uint32_t src = (T & 1) ? w8[v] : w[v];
    return as_h2(and_or(src, T < 2 ? kLoMask : kHiMask, T < 2 ? c.m_lo : c.m_hi)) + as_h2(T < 2 ? c.nb_lo : c.nb_hi);
}

template <int T>
__device__ inline half8 dequant_qz_step(const u32x4 &w, const u32x4 &w8, const DequantConsts &c) {
    return pack_h8(dequant_pair<T>(w, w8, 0, c), dequant_pair<T>(w, w8, 1, c), dequant_pair<T>(w, w8, 2, c),
                   dequant_pair<T>(w, w8, 3, c));
}

// B operand of fp16 weights for step T: the exact q - z rounded once to fp16
// by the multiply with the scale pair s2.
template <int T>
__device__ inline half8 dequant_w_step(const u32x4 &w, const u32x4 &w8, const DequantConsts &c, uint32_t s2) {
    return pack_h8(dequant_pair<T>(w, w8, 0, c) * as_h2(s2), dequant_pair<T>(w, w8, 1, c) * as_h2(s2),
                   dequant_pair<T>(w, w8, 2, c) * as_h2(s2), dequant_pair<T>(w, w8, 3, c) * as_h2(s2));
}

// Runtime-step dispatch for code that loops over steps.
__device__ inline half8 dequant_w(int t, const u32x4 &w, const u32x4 &w8, const DequantConsts &c, uint32_t s2) {
    switch (t) {
        case 0: return dequant_w_step<0>(w, w8, c, s2);
        case 1: return dequant_w_step<1>(w, w8, c, s2);
        case 2: return dequant_w_step<2>(w, w8, c, s2);
        default: return dequant_w_step<3>(w, w8, c, s2);
    }
}
__device__ inline half8 dequant_qz(int t, const u32x4 &w, const u32x4 &w8, const DequantConsts &c) {
    switch (t) {
        case 0: return dequant_qz_step<0>(w, w8, c);
        case 1: return dequant_qz_step<1>(w, w8, c);
        case 2: return dequant_qz_step<2>(w, w8, c);
        default: return dequant_qz_step<3>(w, w8, c);
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

// s_waitcnt immediate that waits until at most n vector memory operations
// are outstanding (gfx9 encoding; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }
// s_waitcnt immediate that waits for all LDS (and scalar memory) operations
constexpr int kLgkmZero = 15 | (3 << 14) | (7 << 4);

// Rounding to an integer in float32: adding 1.5 * 2^23 rounds any |x| <
// 2^22 to the nearest integer (ties to even) and lands in the binade
// [2^23, 2^24), whose bit pattern is kRoundMagicBits + that integer; a fused
// multiply-add with it rounds an exact product once. Used by the quantizers.
constexpr float kRoundMagic = 12582912.0f;         // 1.5 * 2^23
constexpr uint32_t kRoundMagicBits = 0x4B400000u;  // its bit pattern
// Smallest normal fp16 (2^-14): the floor of the quantizers' scales.
constexpr float kScaleFloor = 6.103515625e-05f;

// 1.5 * 2^23 + rint(x / s): the nearest integer to the exact quotient, ties
// to even, for an fp16 value x and a normal float32 scale s (inv = fp32(1/s),
// half_s = s / 2), valid while |x / s| < 2^12 (larger quotients only move
// further past any clamp of the result).
// The fused multiply-add rounds the exact product x * inv once to an integer
// c; since |x * inv - x / s| <= |x / s| 2^-24, c is rint(x / s) or its
// neighbour across a half-integer within that distance (for an fp16 scale
// only an exact tie qualifies: a quotient of two fp16 numbers that is not a
// half-integer lies at least 2^-12 from every half-integer). The residual
// r = x - c s is exact in float32 in every case that matters (|r| < s, and
// the exponents of x and c s differ by less than the float32 precision
// unless |x / s| < 1/2, where c = 0 and r = x), so comparing |r| with s / 2
// settles the decision: beyond it c moves one step towards x / s, at it
// (an exact tie) the even neighbour wins.
// 1.5 * 2^23 + rint(x / s) for an fp16 value x and an fp16 value s
// (normal; inv = fp32(1/s) or within one ulp of it), valid while
// |x / s| < 2^12. The reciprocal
// product p = x inv and one correction step p' = p + (x - p s) inv give the
// quotient within |x / s| 2^-44 before p' is rounded to float32: an exact
// tie n + 1/2 (representable) comes out exact and rounds to even when the
// magic constant is added, and every other quotient of two fp16 numbers lies
// at least 2^-12 from a half-integer, farther than p' can be off (its
// rounding moves it by at most 2^-20 there). Four operations where the
// residual test of round_quotient_magic takes about nine; not valid for a
// float32 scale, whose quotients can come within 2^-25 of a half-integer.
__device__ inline float round_quotient_fp16(float x, float s, float inv) {
    const float p = x * inv;
    const float r = __builtin_fmaf(-p, s, x);
    const float q = __builtin_fmaf(r, inv, p);
    return q + kRoundMagic;
}

// d / L rounded once to float32, for d in [0, 2^17] and L = 15 or 255
// (rL = float32(1/L)): the product, its exact residual and one correction
// step, three operations where an IEEE division takes about ten. Checked
// against the correctly rounded quotient for every float32 d in that range
// and both L (the quantizers' step counts for 4- and 8-bit codes; d is the
// float32 difference of two fp16 numbers, at most 131008).
__device__ inline float div_steps(float d, float L, float rL) {
    const float q0 = d * rL;
    const float e = __builtin_fmaf(-q0, L, d);
    return __builtin_fmaf(e, rL, q0);
}

__device__ inline float round_quotient_magic(float x, float s, float inv, float half_s) {
    float y = __builtin_fmaf(x, inv, kRoundMagic);
    const float c = y - kRoundMagic;
    const float r = __builtin_fmaf(-c, s, x);
    const float ar = __builtin_fabsf(r);
    const bool step = ar > half_s || (ar == half_s && (__builtin_bit_cast(uint32_t, y) & 1u));
    y += step ? __builtin_copysignf(1.0f, r) : 0.0f;
    return y;
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
