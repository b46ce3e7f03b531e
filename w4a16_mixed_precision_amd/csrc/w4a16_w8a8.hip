// W8A8 GEMM: 8-bit weights times 8-bit activations on the int8 matrix
// cores, the precision format the pages list beside W4A16 ("LMDeploy
// Guide: Fast Mixed-Precision LLM Inference Engine", the two pillars and the
// table of quantization formats; SmoothQuant named among the post-training
// methods; the interview notes on the PyTorch engine's w8a8 quantization).
//
// Reading (no formula on the pages): symmetric scales, one per output
// channel for the weights (offline) and one per token for the activations
// (per call): s = max|v| / 127 rounded once to float32 (1 for an all-zero
// vector), code = clamp(rint(v / s), -127, 127) with rint the nearest integer
// to the exact quotient, ties to even (round_quotient_magic).
// Y[m][n] = fp16(float32(float32(acc) * s_x[m]) * s_w[n]) with acc the exact
// int32 sum of code products.
//
// Packed weights: K * N bytes in 1 KiB tiles of 16 columns x 64 rows of K,
// strip-major (tile (n / 16) * (K / 64) + k / 64); in a tile, lane
// l = 16 * ((k % 64) / 16) + n % 16 holds the 16 codes k % 16 = 0..15 of its
// column, the B operand of one v_mfma_i32_16x16x64_i8 step. The activation
// operand takes the same 16 consecutive k per lane group, so A and B agree
// on every k (whatever order the instruction sums them in).
//
// GEMM: workgroup tile BM x 256 (four waves side by side, each 64 columns);
// the BM x 256-byte tile of codes of X for the next 256 rows of K is copied
// global -> LDS by direct 16-byte loads (XOR-swizzled by row, two stages)
// while the current one is multiplied; each wave streams its packed weight
// tiles into registers half a block (two 64-row steps) ahead. Split-K writes int32 partials that
// a second kernel adds (exactly) and scales. Unsplit, the scaled fp16 tile
// is rearranged in LDS and stored as 16-byte row chunks.
#include <stdlib.h>

#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef int int32x4 __attribute__((ext_vector_type(4)));
constexpr int kW8Tile = 1024;   // 16 columns x 64 k
constexpr int kW8Block = 256;   // rows of K per pipeline stage (4 MFMA steps)

// Per-vector quantities of the code decision: the scale, its float32
// reciprocal and half of it.
struct Q8 {
    float s, inv, half_s;
};
__device__ inline Q8 q8_params(float s) { return Q8{s, 1.0f / s, 0.5f * s}; }

// code of v: rint(v / s) clamped to [-127, 127] (round_quotient_magic gives
// 1.5 * 2^23 + rint; the clamp keeps the result in that binade, whose bit
// pattern is bits(1.5 * 2^23) + code)
__device__ inline int code8(float v, const Q8 &p) {
    const float y = __builtin_amdgcn_fmed3f(round_quotient_magic(v, p.s, p.inv, p.half_s), kRoundMagic - 127.f,
                                            kRoundMagic + 127.f);
    return (int)(__builtin_bit_cast(uint32_t, y) - kRoundMagicBits);
}

__device__ inline float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// fp16(float32(float32(acc) * sx) * sw), every product rounded to float32
// first: the empty asm keeps the compiler from fusing the last product with
// the conversion into one mixed-precision instruction (a single rounding
// straight to fp16, which can differ by one fp16 step)
__device__ inline uint16_t scale_out(int32_t acc, float sx, float sw) {
    float y = ((float)acc * sx) * sw;
    asm volatile("" : "+v"(y));
    return f32_to_f16_bits(y);
}

// ------------------------------------------------------------ activations
// One workgroup of 256 threads per token (row); 8 values per thread per
// 16-byte load. K % 256 == 0. Rows of up to 8192 values stay in registers
// between the maximum and the codes (one read of X); longer rows are read
// again.
constexpr int kActRegChunks = 4;  // 16-byte chunks per thread kept in registers

__device__ inline void quant8_store(const u32x4 &v, const Q8 &inv, int8_t *dst) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t c0 = (uint32_t)code8(h2f((uint16_t)(v[d] & 0xFFFF)), inv) & 0xFFu;
        const uint32_t c1 = (uint32_t)code8(h2f((uint16_t)(v[d] >> 16)), inv) & 0xFFu;
        const uint32_t pair = c0 | (c1 << 8);
        if (d < 2)
            lo |= pair << (16 * d);
        else
            hi |= pair << (16 * (d - 2));
    }
    *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
}

__device__ inline float absmax8(const u32x4 &v, float amax) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        amax = __builtin_fmaxf(amax, __builtin_fabsf(h2f((uint16_t)(v[d] & 0xFFFF))));
        amax = __builtin_fmaxf(amax, __builtin_fabsf(h2f((uint16_t)(v[d] >> 16))));
    }
    return amax;
}

__global__ void __launch_bounds__(256)
w8a8_quant_act_kernel(const uint16_t *__restrict__ X, int K, int8_t *__restrict__ xq, float *__restrict__ xs) {
    __shared__ float red[4];
    const int m = blockIdx.x, tid = threadIdx.x;
    const uint16_t *row = X + (size_t)m * K;
    const bool held = K <= kActRegChunks * 256 * 8;
    u32x4 keep[kActRegChunks];
    float amax = 0.f;
    if (held) {
#pragma unroll
        for (int i = 0; i < kActRegChunks; ++i) {
            const int k = (i * 256 + tid) * 8;
            keep[i] = k < K ? *reinterpret_cast<const u32x4 *>(row + k) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kActRegChunks; ++i) amax = absmax8(keep[i], amax);
    } else {
        for (int k = tid * 8; k < K; k += 256 * 8) amax = absmax8(*reinterpret_cast<const u32x4 *>(row + k), amax);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o, 64));
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    const float s = amax > 0.f ? amax / 127.0f : 1.0f;
    const Q8 inv = q8_params(s);
    if (tid == 0) xs[m] = s;
    int8_t *out = xq + (size_t)m * K;
    if (held) {
#pragma unroll
        for (int i = 0; i < kActRegChunks; ++i) {
            const int k = (i * 256 + tid) * 8;
            if (k < K) quant8_store(keep[i], inv, out + k);
        }
    } else {
        for (int k = tid * 8; k < K; k += 256 * 8) quant8_store(*reinterpret_cast<const u32x4 *>(row + k), inv, out + k);
    }
}

// ------------------------------------------------------------ weights
// Per-column maxima of |W| in two passes (the maximum does not depend on
// the order, so the result equals a plain loop over the rows). Pass 1: a
// workgroup takes 64 columns x 256 rows; each thread reads two adjacent
// columns (one 4-byte load) on every eighth row of the slice, so a wave
// reads whole 128-byte row segments, and the eight row phases meet in LDS.
// The partial maxima [K / 256][N] go to `part` (the packed output buffer,
// K * N bytes, which the pack kernel overwrites afterwards). Pass 2: one
// thread per column takes the maximum over the slices and writes the scale.
__global__ void __launch_bounds__(256)
w8a8_weight_colmax_kernel(const uint16_t *__restrict__ W, int K, int N, float *__restrict__ part) {
    __shared__ float red[8][64];
    const int t = threadIdx.x;
    const int p = t & 31, h = t >> 5;
    const int c = blockIdx.x * 64 + 2 * p;
    const int r0 = blockIdx.y * 256;
    float m0 = 0.f, m1 = 0.f;
    if (c < N) {  // N is even: both columns of a pair exist or neither
#pragma unroll 8
        for (int i = 0; i < 32; ++i) {
            const uint32_t v = *reinterpret_cast<const uint32_t *>(W + (size_t)(r0 + h + 8 * i) * N + c);
            m0 = __builtin_fmaxf(m0, __builtin_fabsf(h2f((uint16_t)(v & 0xFFFFu))));
            m1 = __builtin_fmaxf(m1, __builtin_fabsf(h2f((uint16_t)(v >> 16))));
        }
    }
    red[h][2 * p] = m0;
    red[h][2 * p + 1] = m1;
    __syncthreads();
    if (t < 64 && blockIdx.x * 64 + t < N) {
        float m = red[0][t];
#pragma unroll
        for (int q = 1; q < 8; ++q) m = __builtin_fmaxf(m, red[q][t]);
        part[(size_t)blockIdx.y * N + blockIdx.x * 64 + t] = m;
    }
}

__global__ void __launch_bounds__(256)
w8a8_weight_scale_kernel(const float *__restrict__ part, int slices, int N, float *__restrict__ ws) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    float amax = 0.f;
    for (int s = 0; s < slices; ++s) amax = __builtin_fmaxf(amax, part[(size_t)s * N + n]);
    ws[n] = amax > 0.f ? amax / 127.0f : 1.0f;
}

// One thread per 16-byte lane slot of a packed tile.
__global__ void __launch_bounds__(256)
w8a8_weight_pack_kernel(const uint16_t *__restrict__ W, int K, int N, const float *__restrict__ ws,
                        u32x4 *__restrict__ out) {
    const int64_t slots = (int64_t)K * N / 16;
    const int kt = K / 64;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < slots;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(idx & 63);
        const int64_t tile = idx >> 6;
        const int strip = (int)(tile / kt), kb = (int)(tile % kt);
        const int n = strip * 16 + (lane & 15);
        const int k0 = kb * 64 + 16 * (lane >> 4);
        const Q8 inv = q8_params(ws[n]);
        u32x4 v;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int c = code8(h2f(W[(size_t)(k0 + 4 * d + b) * N + n]), inv);
                word |= ((uint32_t)c & 0xFFu) << (8 * b);
            }
            v[d] = word;
        }
        out[idx] = v;
    }
}

// ------------------------------------------------------------ GEMM
template <int MTW, int NSW, int OCC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
w8a8_gemm_kernel(const int8_t *__restrict__ X, const float *__restrict__ xs, const uint8_t *__restrict__ packed,
                 const float *__restrict__ ws, uint16_t *__restrict__ Y, int32_t *__restrict__ part, int M, int N,
                 int K, int tiles_m, int S, int slice_blocks) {
    constexpr int WAVES = 4;
    constexpr int BM = MTW * 16;
    constexpr int STAGE = BM * kW8Block;         // bytes of X per stage
    constexpr int XLOADS = BM * 16 / 256;         // 16-byte copies per thread per stage
    static_assert(XLOADS >= 1 && BM * 16 % 256 == 0, "X tile must split over the threads");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, kq = lane >> 4;
    const int nblk = K / kW8Block;
    const int nstrip = N / 16;
    // XCD-aware remap: workgroups are dispatched round-robin over the eight
    // XCDs. With 8 or more row tiles and tiles that split evenly, XCD x takes
    // half of the row tiles (x % 2) and a quarter of the column slabs (x / 2),
    // M varying fastest:
    // the row tiles that share a slab of weights read it through one L2,
    // and each L2 sees half of X (an XCD taking all rows of a quarter of
    // the slabs, the first form, was 1.3% slower at 2048 x 4096 x 28672 and
    // 1024 x 8192 x 7168). Otherwise each XCD takes a contiguous run of tiles.
    const int ntiles = (int)gridDim.x;  // tiles_m x tiles_n
    const int tiles_n = ntiles / tiles_m;
    int tm, tn;
    if (tiles_m >= 8 && tiles_m % 2 == 0 && tiles_n % 4 == 0) {
        const int x = blockIdx.x % 8, i = blockIdx.x / 8, half_m = tiles_m / 2;
        tm = (x % 2) * half_m + i % half_m;
        tn = (x / 2) * (tiles_n / 4) + i / half_m;
    } else {
        const int tile = ntiles % 8 == 0 ? (blockIdx.x % 8) * (ntiles / 8) + blockIdx.x / 8 : (int)blockIdx.x;
        tm = tile % tiles_m;
        tn = tile / tiles_m;
    }
    const int split = blockIdx.y;
    const int bb = split * slice_blocks;
    const int be = bb + slice_blocks < nblk ? bb + slice_blocks : nblk;
    const int m0 = tm * BM;
    const int strip_w = (tn * WAVES + wave) * NSW;

    // X copies: copy i of this thread moves row r0(i) + lane / 16 of the
    // tile, r0(i) = 4 (i WAVES + wave), source chunk (lane & 15) ^ (row & 15)
    // to LDS position lane: LDS row r holds chunk p ^ (r & 15) at p. Rows at
    // or past M read zeros (one descriptor per copy, ending at row M).
    const int rows_here = M - m0 < BM ? M - m0 : BM;
    __amdgpu_buffer_rsrc_t rx[XLOADS];
#pragma unroll
    for (int i = 0; i < XLOADS; ++i) {
        const int r0 = 4 * (i * WAVES + wave);
        const int nrows = rows_here - r0 > 0 ? rows_here - r0 : 0;
        rx[i] = make_rsrc(X + (size_t)(m0 + (r0 < rows_here ? r0 : 0)) * K, (uint32_t)((size_t)nrows * K));
    }
    const int xrow = lane >> 4;
    const uint32_t xoff = (uint32_t)(xrow * K + (((lane & 15) ^ ((4 * wave + xrow) & 15)) * 16));
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(packed, (uint32_t)((size_t)K * N));
    int sstrip[NSW];
#pragma unroll
    for (int j = 0; j < NSW; ++j) sstrip[j] = strip_w + j < nstrip ? strip_w + j : nstrip - 1;

    auto issue_x = [&](int b, int stage) {
#pragma unroll
        for (int i = 0; i < XLOADS; ++i) {
            const __amdgpu_buffer_rsrc_t r = rx[i];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void *)(lds + stage * STAGE + (i * WAVES + wave) * 1024), 16, xoff, b * kW8Block, 0, 0);
        }
    };
    // packed weights in half blocks (two 64-row steps): the next half is in
    // flight while the current one is multiplied
    typedef u32x4 WHalf[NSW][2];
    auto load_w = [&](int h, WHalf &w) {  // half block h = 2 * block + (0 or 1)
#pragma unroll
        for (int j = 0; j < NSW; ++j)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                w[j][s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rw, lane * 16u, ((size_t)sstrip[j] * (K / 64) + 2 * h + s) * kW8Tile, 0));
    };

    int32x4 acc[MTW][NSW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int j = 0; j < NSW; ++j) acc[mt][j] = int32x4{0, 0, 0, 0};

    // A 64-row step: row tile after row tile, each multiplied with the NSW
    // strips' B operands of the step. A operands stream from LDS two row
    // tiles ahead, across the block's four steps (only three are live, which
    // lets 128-row wave tiles keep two waves per SIMD); a0 and a1 carry the
    // stream from one half block to the next.
    auto a_at = [&](int stage, int s, int mt) {
        return *reinterpret_cast<const int32x4 *>(lds + stage * STAGE + (mt * 16 + col) * kW8Block +
                                                  (((4 * s + kq) ^ col) * 16));
    };
    auto compute = [&](int stage, int half, const WHalf &w, int32x4 &a0, int32x4 &a1) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int s = 2 * half + s2;
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) {
                // the operand two places further along the (step, row tile)
                // stream; nothing past the block's last step
                const int nx = s * MTW + mt + 2;
                const int32x4 a2 = nx < 4 * MTW ? a_at(stage, nx / MTW, nx % MTW) : a0;
#pragma unroll
                for (int j = 0; j < NSW; ++j)
                    acc[mt][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, __builtin_bit_cast(int32x4, w[j][s2]),
                                                                       acc[mt][j], 0, 0, 0);
                a0 = a1;
                a1 = a2;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    if (bb < be) {
        WHalf w0, w1;
        issue_x(bb, 0);
        load_w(2 * bb, w0);
        load_w(2 * bb + 1, w1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // weights two half blocks ahead: three half-block sets rotate, so a
        // half is requested while the two halves before it are multiplied
        const int hlast = 2 * be - 1;
        auto block = [&](int b, WHalf &p, WHalf &q, WHalf &r) {
            const int cur = (b - bb) & 1;
            int32x4 a0 = a_at(cur, 0, 0), a1 = MTW > 1 ? a_at(cur, 0, 1) : a_at(cur, 1, 0);
            if (b + 1 < be) issue_x(b + 1, cur ^ 1);
            // unconditional, clamped to the slice's last half (reloaded,
            // not used) so that every path issues the same loads
            load_w(2 * b + 2 < hlast ? 2 * b + 2 : hlast, r);
            compute(cur, 0, p, a0, a1);
            load_w(2 * b + 3 < hlast ? 2 * b + 3 : hlast, p);
            compute(cur, 1, q, a0, a1);
            // the next block's X copies, issued before the 4 NSW weight
            // loads of this block, have landed; the barrier makes every
            // wave's copies visible and frees the stage just read
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * NSW));
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        WHalf w2;
        for (int b = bb; b < be; b += 3) {
            block(b, w0, w1, w2);
            if (b + 1 < be) block(b + 1, w2, w0, w1);
            if (b + 2 < be) block(b + 2, w1, w2, w0);
        }
    }

    // epilogue: exact int32 sums -> fp16 with the two scales, or partials.
    // Unsplit K: the fp16 tile goes through LDS so that each lane stores 16
    // bytes of a row (8 columns) instead of one 2-byte value per element; the
    // two X stages hold the four waves' tiles. In a wave's region row r,
    // column c sits at r * RB + 16 * ((c / 8) ^ x(r)) + 2 * (c % 8) with
    // x(r) = 2 ((r / 4) % 4) mod the chunks per row: the four row groups a
    // write instruction touches fall in different 16-byte chunks. Rows beyond M and strips beyond N dropped.
    constexpr int RB = NSW * 32;  // bytes per row of a wave's tile
    static_assert(WAVES * MTW * 16 * RB <= 2 * STAGE, "the wave tiles must fit the X stages");
    if (S == 1 && NSW % 2 == 0) {
        __syncthreads();  // every wave is done with the last X stage
        uint8_t *wt = lds + wave * (MTW * 16 * RB);
#pragma unroll
        for (int j = 0; j < NSW; ++j) {
            const int sj = strip_w + j < nstrip ? strip_w + j : nstrip - 1;
            const float swn = ws[sj * 16 + col];
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = mt * 16 + 4 * kq + e, cc = j * 16 + col;
                    const float sx = xs[m0 + r < M ? m0 + r : M - 1];
                    *reinterpret_cast<uint16_t *>(wt + r * RB + 16 * ((cc >> 3) ^ ((2 * ((r >> 2) & 3)) & (RB / 16 - 1))) + 2 * (cc & 7)) =
                        scale_out(acc[mt][j][e], sx, swn);
                }
        }
        constexpr int CPR = RB / 16;   // 16-byte chunks per row
        constexpr int RPI = 64 / CPR;  // rows per read instruction
        const int k = lane % CPR, rr = lane / CPR;
        const int sk = strip_w + k / 2;
#pragma unroll
        for (int i = 0; i < MTW * 16 / RPI; ++i) {
            const int r = i * RPI + rr;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(wt + r * RB + 16 * (k ^ ((2 * ((r >> 2) & 3)) & (CPR - 1))));
            if (m0 + r < M && sk < nstrip)
                *reinterpret_cast<u32x4 *>(Y + (size_t)(m0 + r) * N + (size_t)strip_w * 16 + 8 * k) = v;
        }
        return;
    }
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int j = 0; j < NSW; ++j) {
            const int sj = strip_w + j;
            if (sj >= nstrip) continue;
            const int n = sj * 16 + col;
            const float swn = S == 1 ? ws[n] : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + mt * 16 + 4 * kq + e;
                if (row >= M) continue;
                if (S == 1)
                    Y[(size_t)row * N + n] = scale_out(acc[mt][j][e], xs[row], swn);
                else
                    part[((size_t)split * M + row) * N + n] = acc[mt][j][e];
            }
        }
}

__global__ void __launch_bounds__(256)
w8a8_reduce_kernel(const int32_t *__restrict__ part, const float *__restrict__ xs, const float *__restrict__ ws,
                   uint16_t *__restrict__ Y, int M, int N, int S) {
    const int64_t MN = (int64_t)M * N;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < MN; i += (int64_t)gridDim.x * blockDim.x) {
        int32_t a = 0;
        for (int s = 0; s < S; ++s) a += part[(size_t)s * MN + i];
        const int m = (int)(i / N), n = (int)(i % N);
        Y[i] = scale_out(a, xs[m], ws[n]);
    }
}

// ------------------------------------------------------------ decode GEMM
// Small M (<= 16 rows, one 16-row tile): one workgroup per NS strips of 16
// columns over the whole of K, WK waves splitting the K tiles. Each wave
// streams its weight tiles and the matching codes of X straight into
// operand registers (lane (m, kq) of tile t holds X codes [m][64 t + 16 kq,
// +16); rows at or past M lie outside the codes' descriptor and read zeros), with
// the next batch of tiles in flight, and the waves' exact int32 partial
// tiles are added in LDS: no split-K partials in memory and no second
// launch.
template <int NS, int WK>
__global__ void __launch_bounds__(WK * 64)
w8a8_decode_kernel(const int8_t *__restrict__ X, const float *__restrict__ xs, const uint8_t *__restrict__ packed,
                   const float *__restrict__ ws, uint16_t *__restrict__ Y, int M, int N, int K) {
    static_assert(NS <= WK, "one wave per strip in the epilogue");
    constexpr int TB = 4;  // tiles per batch
    __shared__ int32x4 red[WK][NS][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane & 15, kq = lane >> 4;
    const int kt = K / 64;
    const int nstrip = N / 16;
    const int strip0 = blockIdx.x * NS;
    const int per = (kt + WK - 1) / WK;
    const int t0 = wave * per;
    const int t1 = t0 + per < kt ? t0 + per : kt;
    // one descriptor over the M x K codes: lanes of rows at or past M fall
    // outside it and read zeros
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (uint32_t)(M * K));
    const uint32_t xrow = (uint32_t)(row * K + 16 * kq);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(packed, (uint32_t)((size_t)K * N));
    int sstrip[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) sstrip[j] = strip0 + j < nstrip ? strip0 + j : nstrip - 1;

    struct Batch {
        int32x4 x[TB];
        int32x4 w[TB][NS];
    };
    // tiles past the wave's range load the wave's last tile again (in
    // bounds) and are not multiplied
    auto load = [&](int t, Batch &B) {
#pragma unroll
        for (int i = 0; i < TB; ++i) {
            const int tile = t + i < t1 ? t + i : t1 - 1;
            B.x[i] = __builtin_bit_cast(int32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xrow + (uint32_t)(tile * 64), 0, 0));
#pragma unroll
            for (int j = 0; j < NS; ++j)
                B.w[i][j] = __builtin_bit_cast(int32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                            rw, lane * 16u, ((size_t)sstrip[j] * kt + tile) * kW8Tile, 0));
        }
    };
    int32x4 acc[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[j] = int32x4{0, 0, 0, 0};
    auto compute = [&](int t, const Batch &B) {
#pragma unroll
        for (int i = 0; i < TB; ++i) {
            if (t + i >= t1) break;
#pragma unroll
            for (int j = 0; j < NS; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(B.x[i], B.w[i][j], acc[j], 0, 0, 0);
        }
    };
    if (t0 < t1) {
        Batch b0, b1;
        load(t0, b0);
        for (int t = t0; t < t1; t += 2 * TB) {
            if (t + TB < t1) load(t + TB, b1);
            compute(t, b0);
            if (t + TB >= t1) break;
            if (t + 2 * TB < t1) load(t + 2 * TB, b0);
            compute(t + TB, b1);
        }
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) red[wave][j][lane] = acc[j];
    __syncthreads();
    if (wave < NS && strip0 + wave < nstrip) {
        int32x4 sum = red[0][wave][lane];
#pragma unroll
        for (int w = 1; w < WK; ++w) sum += red[w][wave][lane];
        const int n = (strip0 + wave) * 16 + row;
        const float swn = ws[n];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * kq + e;
            if (m < M) Y[(size_t)m * N + n] = scale_out(sum[e], xs[m], swn);
        }
    }
}

inline unsigned grid_for(int64_t items) {
    int64_t blocks = (items + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return (unsigned)(blocks < 1 ? 1 : blocks);
}

struct W8Plan {
    int bm;  // workgroup rows: 16 or 64
    int splits, slice_blocks;
    int decode, ns, wk;  // the decode kernel (M <= 16): strips per workgroup, waves along K
};

// The decode kernel up to M = 16, tiles of 64 or 128 rows above; split K
// until the tiles times splits fill the GPU's resident slots (two 4-wave
// workgroups per CU), keeping at least two blocks of K per split.
W8Plan w8_plan(int M, int N, int K, int num_cus) {
    W8Plan p;
    p.bm = M <= 16 ? 16 : 64;
    p.decode = M <= 16;
    if (const char *e = getenv("W4A16_W8A8_TILE")) {  // forces the tiled kernel
        const int v = atoi(e);
        if (v == 16 || v == 64 || v == 128) {
            p.bm = v;
            p.decode = 0;
        }
    }
    // decode kernel: at most one workgroup per CU where two strips per
    // workgroup get there (every workgroup reads all of X's codes, so two
    // on one CU read them twice; graph-timed at M = 16, K = 4096, N = 6144:
    // 10.9 us per call with two strips, 12.3-12.7 with one, waves along K
    // 4, 8 or 16 within 2%). W4A16_W8A8_DNS (1, 2) and W4A16_W8A8_DWK (4,
    // 8, 16) override the shape (tuning).
    p.ns = N / 16 > num_cus ? 2 : 1;
    p.wk = 8;
    if (const char *e = getenv("W4A16_W8A8_DNS")) {
        const int v = atoi(e);
        if (v == 1 || v == 2) p.ns = v;
    }
    if (const char *e = getenv("W4A16_W8A8_DWK")) {
        const int v = atoi(e);
        if (v == 4 || v == 8 || v == 16) p.wk = v;
    }
    if (p.decode) {
        p.splits = 1;
        p.slice_blocks = K / kW8Block;
        return p;
    }
    const int nblk = K / kW8Block;
    const int slots = num_cus * 2;  // two 4-wave workgroups per CU
    // 128-row tiles read each weight tile half as often as 64-row ones but
    // give half as many workgroups: taken where 64-row tiles would fill the
    // chip at least twice (graph-timed, 2048 x 4096 x 28672: 269-279 us
    // against 325-378; 1024 x 8192 x 7168, under one round: 91 against 81.5)
    if (getenv("W4A16_W8A8_TILE") == nullptr && M > 16 &&
        ((M + 63) / 64) * ((N + 255) / 256) >= 2 * slots)
        p.bm = 128;
    const int BM = p.bm;
    const int tiles = ((M + BM - 1) / BM) * ((N + 255) / 256);
    int s = tiles >= slots ? 1 : slots / tiles;
    const int cap = nblk / 2 > 1 ? nblk / 2 : 1;
    if (s > cap) s = cap;
    const int sb = (nblk + s - 1) / s;
    p.slice_blocks = sb;
    p.splits = (nblk + sb - 1) / sb;
    return p;
}

}  // namespace

size_t w8a8_workspace_bytes(int M, int N, int K, int num_cus) {
    const W8Plan p = w8_plan(M, N, K, num_cus);
    return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(int32_t) : 0;
}

hipError_t launch_w8a8_quant_act(const uint16_t *X, int M, int K, int8_t *xq, float *xs, hipStream_t stream) {
    hipLaunchKernelGGL(w8a8_quant_act_kernel, dim3((unsigned)M), dim3(256), 0, stream, X, K, xq, xs);
    return hipGetLastError();
}

hipError_t launch_w8a8_quant_weights(const uint16_t *W, int K, int N, uint8_t *packed, float *ws, hipStream_t stream) {
    float *part = reinterpret_cast<float *>(packed);  // [K / 256][N] partial maxima, overwritten by the pack
    hipLaunchKernelGGL(w8a8_weight_colmax_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)(K / 256)), dim3(256), 0,
                       stream, W, K, N, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(w8a8_weight_scale_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, part,
                       K / 256, N, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(w8a8_weight_pack_kernel, dim3(grid_for((int64_t)K * N / 16)), dim3(256), 0, stream, W, K, N,
                       ws, reinterpret_cast<u32x4 *>(packed));
    return hipGetLastError();
}

hipError_t launch_w8a8_gemm(const int8_t *xq, const float *xs, const uint8_t *packed, const float *ws, int M, int N,
                            int K, uint16_t *Y, void *workspace, int num_cus, hipStream_t stream) {
    const W8Plan p = w8_plan(M, N, K, num_cus);
    if (p.decode) {
        const dim3 grid((unsigned)((N / 16 + p.ns - 1) / p.ns));
#define W8_DECODE(NS_, WK_)                                                                                          \
    if (p.ns == NS_ && p.wk == WK_)                                                                                  \
        hipLaunchKernelGGL((w8a8_decode_kernel<NS_, WK_>), grid, dim3(WK_ * 64), 0, stream, xq, xs, packed, ws, Y, M, \
                           N, K);
        W8_DECODE(1, 4) W8_DECODE(1, 8) W8_DECODE(1, 16) W8_DECODE(2, 4) W8_DECODE(2, 8) W8_DECODE(2, 16)
#undef W8_DECODE
        return hipGetLastError();
    }
    int32_t *part = p.splits > 1 ? static_cast<int32_t *>(workspace) : nullptr;
    const int tiles_m = (M + p.bm - 1) / p.bm, tiles_n = (N + 255) / 256;
    const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)p.splits);
    if (p.bm == 128)
        hipLaunchKernelGGL((w8a8_gemm_kernel<8, 4, 2>), grid, dim3(256), 0, stream, xq, xs, packed, ws, Y, part, M, N,
                           K, tiles_m, p.splits, p.slice_blocks);
    else if (p.bm == 64)
        hipLaunchKernelGGL((w8a8_gemm_kernel<4, 4, 2>), grid, dim3(256), 0, stream, xq, xs, packed, ws, Y, part, M, N,
                           K, tiles_m, p.splits, p.slice_blocks);
    else
        hipLaunchKernelGGL((w8a8_gemm_kernel<1, 4, 2>), grid, dim3(256), 0, stream, xq, xs, packed, ws, Y, part, M, N,
                           K, tiles_m, p.splits, p.slice_blocks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits <= 1) return e;
    hipLaunchKernelGGL(w8a8_reduce_kernel, dim3(grid_for((int64_t)M * N)), dim3(256), 0, stream, part, xs, ws, Y, M,
                       N, p.splits);
    return hipGetLastError();
}

}  // namespace w4a16
