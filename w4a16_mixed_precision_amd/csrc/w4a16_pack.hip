// Offline packing pass and its inverse.
//
// The pages describe packing as a one-time relayout that puts the 4-bit
// codes in the exact per-lane order the matrix instructions consume, so the
// online kernel does no swizzling at run time ("LMDeploy Guide: Fast
// Mixed-Precision LLM Inference Engine", section 1 "Hardware-Aware Weight
// Packing (GEMM Pipeline)"). On NVIDIA that takes four steps (widen to 16
// bits, shared-memory fragment load, compress and permute, coalesced store)
// because the permutation is done by the ldmatrix crossbar. Here the target
// order is known in closed form, so each thread computes the source index of
// every code it writes and the pass is a single gather: one thread per
// 16-byte lane slot of a 1 KiB tile (the bytes one wave64 lane loads at run
// time).
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

// Nibble slot j of word v in a lane's 16 bytes holds k offset
// 32 * step(j) + 2 * v + (j >> 2) from the lane's first row, where the slot
// order (steps 0, 2, 1, 3 in the low and high 16-bit halves) lets one shift
// by 8 plus two masks expose all four 32-row steps of a word.
__device__ inline int slot_step(int j) { return 2 * (j & 1) + ((j >> 1) & 1); }
__device__ inline int slot_k(int v, int j) { return 32 * slot_step(j) + 2 * v + (j >> 2); }

// Largest |(q - z) * s| that rounds to a finite fp16 value is just below
// 65520 (65504 is the largest fp16; 65520 is the midpoint to the next power
// of two and rounds to infinity, ties to even).
constexpr float kFp16Overflow = 65520.0f;

// Packs the codes and checks every dequantized weight: the pages define the
// dequantized weight as an fp16 value ("LMDeploy Guide: Fast Mixed-Precision
// LLM Inference Engine", section 3, FP16 = (INT4 - ZeroPoint) x Scale), so a
// code above 15, a non-finite scale or a product |q - z| * |s| that rounds to
// infinity sets `bad`. The product of a 4-bit difference and an fp16 scale
// is exact in fp32, and the negated comparison also catches NaN.
__global__ void __launch_bounds__(256)
pack_weights_kernel(const uint8_t *__restrict__ q, const uint8_t *__restrict__ z, const uint16_t *__restrict__ s,
                    int K, int N, int G, u32x4 *__restrict__ out, int *__restrict__ bad) {
    const int64_t slots = (int64_t)K * N / 32;
    const int nblk = K / kBlockK;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < slots;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(idx & 63);
        const int64_t tile = idx >> 6;
        const int strip = (int)(tile / nblk);
        const int blk = (int)(tile % nblk);
        const int n = strip * kStripCols + (lane & 15);
        const int kbase = blk * kBlockK + 8 * (lane >> 4);
        u32x4 v;
        uint32_t over = 0;
        bool out_of_range = false;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int k = kbase + slot_k(w, j);
                const uint32_t c = q[(int64_t)k * N + n];
                const int64_t gi = (int64_t)(k / G) * N + n;
                const float sc = (float)__builtin_bit_cast(_Float16, s[gi]);
                const float d = (float)((int)(c & 15u) - (int)(z[gi] & 15u));
                out_of_range |= !(__builtin_fabsf(d * sc) < kFp16Overflow);
                over |= c;
                word |= (c & 15u) << (4 * j);
            }
            v[w] = word;
        }
        out[idx] = v;
        if (over > 15u || out_of_range) *bad = 1;
    }
}

__global__ void __launch_bounds__(256)
pack_scales_zeros_kernel(const uint8_t *__restrict__ z, const uint16_t *__restrict__ s, int K,
                         int N, int G, uint16_t *__restrict__ sout, uint8_t *__restrict__ zout,
                         int *__restrict__ bad) {
    // One thread per (strip, group, column pair).
    const int ngrp = K / G;
    const int64_t pairs = (int64_t)ngrp * N / 2;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < pairs;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int pr = (int)(idx & 7);
        const int64_t rec = idx >> 3;  // strip * ngrp + g
        const int strip = (int)(rec / ngrp);
        const int g = (int)(rec % ngrp);
        const int n = strip * kStripCols + 2 * pr;
        const uint32_t z0 = z[(int64_t)g * N + n], z1 = z[(int64_t)g * N + n + 1];
        if ((z0 | z1) > 15u) *bad = 1;
        zout[idx] = (uint8_t)((z0 & 15u) | ((z1 & 15u) << 4));
        sout[rec * 16 + 2 * pr] = s[(int64_t)g * N + n];
        sout[rec * 16 + 2 * pr + 1] = s[(int64_t)g * N + n + 1];
    }
}

__global__ void __launch_bounds__(256)
unpack_weights_kernel(const u32x4 *__restrict__ in, int K, int N, uint8_t *__restrict__ q) {
    const int64_t slots = (int64_t)K * N / 32;
    const int nblk = K / kBlockK;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < slots;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(idx & 63);
        const int64_t tile = idx >> 6;
        const int strip = (int)(tile / nblk);
        const int blk = (int)(tile % nblk);
        const int n = strip * kStripCols + (lane & 15);
        const int kbase = blk * kBlockK + 8 * (lane >> 4);
        const u32x4 v = in[idx];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int k = kbase + slot_k(w, j);
                q[(int64_t)k * N + n] = (uint8_t)((v[w] >> (4 * j)) & 15u);
            }
        }
    }
}

__global__ void __launch_bounds__(256)
unpack_scales_zeros_kernel(const uint16_t *__restrict__ sin, const uint8_t *__restrict__ zin,
                           int K, int N, int G, uint8_t *__restrict__ z, uint16_t *__restrict__ s) {
    const int ngrp = K / G;
    const int64_t pairs = (int64_t)ngrp * N / 2;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < pairs;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int pr = (int)(idx & 7);
        const int64_t rec = idx >> 3;
        const int strip = (int)(rec / ngrp);
        const int g = (int)(rec % ngrp);
        const int n = strip * kStripCols + 2 * pr;
        const uint8_t b = zin[idx];
        z[(int64_t)g * N + n] = b & 15;
        z[(int64_t)g * N + n + 1] = b >> 4;
        s[(int64_t)g * N + n] = sin[rec * 16 + 2 * pr];
        s[(int64_t)g * N + n + 1] = sin[rec * 16 + 2 * pr + 1];
    }
}

inline unsigned grid_for(int64_t items) {
    int64_t blocks = (items + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    return (unsigned)blocks;
}

}  // namespace

hipError_t launch_pack(const uint8_t *q, const uint8_t *z, const uint16_t *s, int K, int N, int G,
                       uint8_t *packed, int *bad, hipStream_t stream) {
    u32x4 *wout = reinterpret_cast<u32x4 *>(packed);
    uint16_t *sout = reinterpret_cast<uint16_t *>(packed + weight_bytes(K, N));
    uint8_t *zout = packed + weight_bytes(K, N) + scale_bytes(K, N, G);
    const int64_t slots = (int64_t)K * N / 32;
    hipLaunchKernelGGL(pack_weights_kernel, dim3(grid_for(slots)), dim3(256), 0, stream, q, z, s, K, N, G,
                       wout, bad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t pairs = (int64_t)(K / G) * N / 2;
    hipLaunchKernelGGL(pack_scales_zeros_kernel, dim3(grid_for(pairs)), dim3(256), 0, stream, z, s,
                       K, N, G, sout, zout, bad);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int K, int N, int G, uint8_t *q, uint8_t *z,
                         uint16_t *s, hipStream_t stream) {
    const u32x4 *win = reinterpret_cast<const u32x4 *>(packed);
    const uint16_t *sin = reinterpret_cast<const uint16_t *>(packed + weight_bytes(K, N));
    const uint8_t *zin = packed + weight_bytes(K, N) + scale_bytes(K, N, G);
    const int64_t slots = (int64_t)K * N / 32;
    hipLaunchKernelGGL(unpack_weights_kernel, dim3(grid_for(slots)), dim3(256), 0, stream, win, K,
                       N, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t pairs = (int64_t)(K / G) * N / 2;
    hipLaunchKernelGGL(unpack_scales_zeros_kernel, dim3(grid_for(pairs)), dim3(256), 0, stream, sin,
                       zin, K, N, G, z, s);
    return hipGetLastError();
}

}  // namespace w4a16
