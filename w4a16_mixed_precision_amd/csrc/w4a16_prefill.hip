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
// * Workgroup tile BM x BN with WM x WN waves; wave (wm, wn) owns MTW 16-row
//   tiles and NSW 16-column strips. Its accumulators stay in registers for
//   the whole K loop.
// * Activations: the BM x 128 tile of X for the next K block is copied
//   global -> LDS by direct 16-byte loads (no register staging) while the
//   current block is being multiplied (two LDS stages). Inside a 256-byte
//   LDS row the sixteen 16-byte chunks are stored XOR-swizzled by the row
//   index, so the 16 lanes that read one k chunk from 16 consecutive rows hit
//   16 different bank groups. A operands of the next 32-row step are read
//   from LDS while the current step's MFMAs run.
// * Weights: each wave loads its packed tiles straight into registers, one
//   16-byte load per lane per strip and K block (the packed order is the
//   operand order, so there is no run-time swizzle), one block ahead.
// * Dequantization (section 3 of the same page, FP16 = (INT4 - ZeroPoint) x
//   Scale): exponent-OR gives 1024 + q (low nibbles) or 64 + q (high
//   nibbles, unshifted), a packed fp16 add of -(1024 + z) or -(64 + z) gives
//   q - z exactly, a packed fp16 multiply by s gives the weight
//   rounded once to fp16. The B operand of every 16 x 16 x 32 MFMA is
//   produced this way and reused for all MTW row tiles of the wave.
// * Split-K: when the tile grid alone cannot fill the GPU, workgroups also
//   split K; each writes fp32 partials and a second kernel adds them in
//   split order (the kernel boundary orders the two; no device-scope fence).
// * Epilogue: the accumulators hold four rows of one column per lane, so the
//   tile (fp16, or the fp32 partials half a tile at a time) is rearranged in
//   LDS and leaves as 16-byte row chunks, whole lines of Y.
// * Workgroups are dispatched round-robin over the eight XCDs; tile ids are
//   remapped so that the workgroups resident on one XCD share rows of X and
//   columns of W in that XCD's L2.
#include <stdlib.h>

#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {


// Packed weights of one K block for the wave's NSW strips, kept raw until
// use (combining them right after the load would make the compiler wait on
// every load in flight, including the next block's prefetch).
template <int NSW>
struct WSet {
    u32x4 w[NSW];
};

template <int MTW, int NSW, int WM, int WN, int GS, int OCC>
__global__ void __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
prefill_kernel(const uint16_t *__restrict__ X, const uint8_t *__restrict__ packed,
               uint16_t *__restrict__ Y, float *__restrict__ part, int M, int N, int K, int tiles_m,
               int tiles_n, int S, int slice_blocks) {
    constexpr int WAVES = WM * WN;
    constexpr int THREADS = WAVES * 64;
    constexpr int BM = WM * MTW * 16;
    constexpr int STAGE = BM * 256;  // BM rows x 128 k x 2 bytes
    constexpr int F = GS < 4 ? GS : 4;
    constexpr int NF = 4 / F;
    constexpr int XLOADS = BM * 16 / THREADS;  // 16-byte direct loads per thread per stage
    static_assert(BM * 16 % THREADS == 0, "X tile must split evenly over the threads");
    static_assert(MTW == 4 || MTW == 8 || MTW == 16, "row tiles per wave");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int nblk = K / kBlockK;
    const int ngrp = K / (32 * GS);
    const int nstrip = N / kStripCols;

    // XCD-aware remap: dispatch order id -> logical tile. Consecutive ids go
    // to consecutive XCDs. With 8 or more row tiles (X too large for one L2)
    // and tiles that split evenly, XCD x takes half of the row tiles (x % 2)
    // and a quarter of the column slabs (x / 2), M varying fastest, so
    // neighbours share columns of W in one L2 and each L2 sees half of X
    // (2048 x 4096 x 28672: 389-398 against 401-404 us with each XCD taking
    // all rows of a contiguous run of tiles). Otherwise each XCD takes a
    // contiguous run of tiles, which reads every weight once (at M = 256 the
    // half-rows order read the 70B gate/up weights twice and took 221-227
    // against 212-214 us).
    const int ntiles = tiles_m * tiles_n;
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
    const int strip_w = (tn * WN + wn) * NSW;  // first strip of this wave
    const uint32_t m_lo = kMagic, m_hi = kMagic64;

    // X: this thread's chunk i of a stage covers row r0(i) + lane/16 of the
    // tile, r0(i) = 4 (i WAVES + wave). One buffer per i starts at that row
    // group and ends at row M, so rows past M read as zeros (their results
    // are never stored); the per-lane offset is the same for every i.
    const int rows_here = M - m0 < BM ? M - m0 : BM;
    __amdgpu_buffer_rsrc_t rx[XLOADS];
#pragma unroll
    for (int i = 0; i < XLOADS; ++i) {
        const int r0 = 4 * (i * WAVES + wave);
        const int nrows = rows_here - r0 > 0 ? rows_here - r0 : 0;
        rx[i] = make_rsrc(X + (size_t)(m0 + (r0 < rows_here ? r0 : 0)) * K, (uint32_t)((size_t)nrows * K * 2));
    }
    const int xrow = lane >> 4;
    const uint32_t xoff = (uint32_t)(xrow * K * 2 + (((lane & 15) ^ ((4 * wave + xrow) & 15)) * 16));
    static_assert((4 * WAVES) % 16 == 0, "chunk swizzle must not depend on the load index");
    // W, scales, zeros: per-lane offsets shared by all strips, strip offsets
    // in scalar registers (tail strips past N are loaded but not stored).
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(packed, (uint32_t)weight_bytes(K, N));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(packed + weight_bytes(K, N), (uint32_t)scale_bytes(K, N, 32 * GS));
    const __amdgpu_buffer_rsrc_t rz =
        make_rsrc(packed + weight_bytes(K, N) + scale_bytes(K, N, 32 * GS), (uint32_t)zero_bytes(K, N, 32 * GS));
    const uint32_t woff = lane * 16;
    int sstrip[NSW];
#pragma unroll
    for (int j = 0; j < NSW; ++j) sstrip[j] = strip_w + j < nstrip ? strip_w + j : nstrip - 1;

    auto issue_x = [&](int b, int stage) {
#pragma unroll
        for (int i = 0; i < XLOADS; ++i) {
            // (a local copy: passing the array element straight to the
            // builtin makes hipcc's host pass drop this kernel's launch stub)
            const __amdgpu_buffer_rsrc_t r = rx[i];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void *)(lds + stage * STAGE + (i * WAVES + wave) * 1024), 16, xoff, b * 256, 0, 0);
        }
    };
    typedef WSet<NSW> Set;
    auto load_w = [&](int b, Set &w) {
#pragma unroll
        for (int j = 0; j < NSW; ++j)
            w.w[j] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff, (sstrip[j] * nblk + b) * kTileBytes, 0));
    };
    // Scales and zero codes come in windows of four consecutive groups of a
    // strip (GS blocks): lane (col, kq) loads column col's scale and zero
    // byte of group 4 w + kq, so one 16-bit and one 8-bit load per strip
    // serve GS blocks, where every lane loading its own group's pair would
    // take 2 NF loads per strip and block (the four kq rows of a column
    // need the same values). Groups past the strip's last read the next
    // strip's records, or zeros past the last strip (the whole offset is the
    // per-lane one, so the descriptor bound decides); they are not used.
    // The lane's byte offsets within a window, kq 32 + 2 col and kq 8 +
    // col / 2, are woff / 8 and woff / 32: recomputed at each window (the
    // asm keeps the compiler from holding them, or spilling them, across
    // the loop).
    auto load_sz = [&](int b, uint32_t (&sc)[NSW], uint32_t (&zb)[NSW]) {
        uint32_t ls, lz;
        asm volatile("v_lshrrev_b32 %0, 3, %1" : "=v"(ls) : "v"(woff));
        asm volatile("v_lshrrev_b32 %0, 5, %1" : "=v"(lz) : "v"(woff));
#pragma unroll
        for (int j = 0; j < NSW; ++j) {
            const uint32_t rec = (uint32_t)(sstrip[j] * ngrp + (b / GS) * 4);
            sc[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, rec * 32u + ls, 0, 0);
            zb[j] = __builtin_amdgcn_raw_buffer_load_b8(rz, rec * 8u + lz, 0, 0);
        }
    };

    floatx4 acc[MTW][NSW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int j = 0; j < NSW; ++j) acc[mt][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // LDS byte offset of this lane's A operand for row tile mt, step t.
    const int rbase = wm * MTW * 16;
    auto a_off = [&](int mt, int t) { return (rbase + mt * 16 + col) * 256 + (((4 * t + kq) ^ col) * 16); };

    // One K block: four 32-row steps x NSW strips = 4 NSW strip groups of MTW
    // MFMAs each. The B operand of a strip for the next step is dequantized
    // once that strip's group has issued its MFMAs (all four 32-bit words
    // after the group's last MFMA for 8 row tiles per wave, two words after
    // every second one for 4), into the registers those MFMAs read;
    // after the last strip of a step, each row tile's A operand for the next
    // step is read from LDS right behind that row tile's MFMA. The matrix
    // unit thus runs while the VALU converts weights and the LDS serves reads.
    auto compute = [&](int b, int stage, const Set &w, const uint32_t (&sz)[NSW]) {
        const uint8_t *st = lds + stage * STAGE;
        // scale and zero code of each group the block uses, from the lane of
        // the same column that loaded it (row kq = the group's place in its
        // window)
        uint32_t gsz[NF][NSW];
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int src = (((b * 4 + f * F) / GS) & 3) * 64 + col * 4;  // byte index of the source lane
#pragma unroll
            for (int j = 0; j < NSW; ++j) gsz[f][j] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sz[j]);
        }
        // Per strip, the fp16 bias -(1024 + z) or -(64 + z) and the scale
        // of each step, two 16-bit values to a register: steps t and t + 2
        // share register t % NP (low half for t < 2, high half above), and
        // the packed add and multiply read the half they need broadcast.
        constexpr int NP = F == 1 ? 2 : 1;
        uint32_t bp[NP][NSW], sp[NP][NSW];
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int j = 0; j < NSW; ++j) {
                const int f0 = p / F, f1 = (p + 2) / F;  // groups of steps p and p + 2
                bp[p][j] = (0xE400u | (gsz[f0][j] >> 16)) | ((0xD400u | ((gsz[f1][j] >> 16) << 4)) << 16);
                sp[p][j] = (gsz[f0][j] & 0xFFFFu) | (gsz[f1][j] << 16);
            }
        auto half_of = [](uint32_t x, bool hi) -> half2v {
            const half2v h = as_h2(x);
            return hi ? __builtin_shufflevector(h, h, 1, 1) : __builtin_shufflevector(h, h, 0, 0);
        };
        // word v of strip j's B operand for step t: two fp16 weights
        auto bword = [&](int t, int j, int v) -> uint32_t {
            const int p = t % NP;
            const bool hi = t >= 2;
            const uint32_t src = (t & 1) ? (w.w[j][v] >> 8) : w.w[j][v];
            const half2v r = (as_h2(and_or(src, t < 2 ? kLoMask : kHiMask, t < 2 ? m_lo : m_hi)) +
                              half_of(bp[p][j], hi)) *
                             half_of(sp[p][j], hi);
            return __builtin_bit_cast(uint32_t, r);
        };
        half8 a[MTW];
        u32x4 bw[NSW];
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) a[mt] = *reinterpret_cast<const half8 *>(st + a_off(mt, 0));
#pragma unroll
        for (int j = 0; j < NSW; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) bw[j][v] = bword(0, j, v);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < 4 * NSW; ++g) {
            const int t = g / NSW, j = g % NSW;
            // steps 1 and 2 run at raised wave priority, step 0 (behind the
            // block start) and step 3 (ahead of the wait for the next block)
            // at the normal one
            if (g == NSW) __builtin_amdgcn_s_setprio(1);
            if (g == 3 * NSW) __builtin_amdgcn_s_setprio(0);
            const int pg = g - 1;                      // previous strip group
            const int pt = pg / NSW + 1, pj = pg % NSW;  // its strip's next step
            const bool pending = g > 0 && pt < 4;
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) {
                acc[mt][j] = mfma16x16x32(a[mt], __builtin_bit_cast(half8, bw[j]), acc[mt][j]);
                if (t < 3 && j == NSW - 1) a[mt] = *reinterpret_cast<const half8 *>(st + a_off(mt, t + 1));
                // all four words after the group's last MFMA for 8 or more
                // row tiles (graph-timed against two words after every
                // fourth MFMA: 399 against 403 us at 2048 x 4096 x 28672,
                // 98 against 102.5 us at 512 x 8192 x 10240, G = 64; one
                // slot at the first, fourth or sixth MFMA sat in between);
                // two words after every second MFMA for MTW 4
                constexpr int kSlots = MTW >= 8 ? 1 : MTW / 2;  // dequant slots per group
                constexpr int kEvery = MTW / kSlots;
                if (pending && mt % kEvery == kEvery - 1) {
                    const int slot = mt / kEvery;
#pragma unroll
                    for (int v = slot * 4 / kSlots; v < (slot + 1) * 4 / kSlots; ++v) bw[pj][v] = bword(pt, pj, v);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    Set wc, wnext;
    uint32_t scn[NSW], zbn[NSW], sz[NSW];
    issue_x(bb, 0);
    load_w(bb, wc);
    load_sz(bb, scn, zbn);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int b = bb; b < be; ++b) {
        const int cur = (b - bb) & 1;
        if (b == bb || b % GS == 0) {  // a new window (loaded during the previous block)
            // this column's nibble of the zero byte: (woff / 4) & 4 = 4 (col & 1)
            uint32_t zsh;
            asm volatile("v_lshrrev_b32 %0, 2, %1\n\tv_and_b32 %0, 4, %0" : "=&v"(zsh) : "v"(woff));
#pragma unroll
            for (int j = 0; j < NSW; ++j) sz[j] = (scn[j] & 0xFFFFu) | (((zbn[j] >> zsh) & 15u) << 16);
        }
        if (b + 1 < be) issue_x(b + 1, cur ^ 1);
        // unconditional (a conditional reload would keep the old set live
        // beside the new one): after the last block it reloads that block
        load_w(b + 1 < be ? b + 1 : b, wnext);
        if (b + 1 < be && (b + 1) % GS == 0) load_sz(b + 1, scn, zbn);
        compute(b, cur, wc, sz);
        // The middle two steps of each block run at raised wave priority
        // (inside compute), the block start, the last step and the wait for
        // the next block at the normal one: while one wave sets up or waits,
        // the SIMD's other wave (the other workgroup's) issues its matrix
        // work first. Graph-timed: 2048 x 4096 x 28672 378-385 us (387-393
        // with no priority change), Qwen-shaped G = 64 pair 86-88 / 214-220
        // us (93-95 / 224-230), 8192 x 57344 at M = 256 199-207 us (203-215
        // with the whole block raised); raising it for the whole block, from
        // the block start or from the barrier measured 1-4% slower than this
        // window.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        wc = wnext;
    }

    // Epilogue, unsplit K: the fp16 tile goes through LDS so that each lane
    // stores 16 bytes of a row (8 columns) instead of one 2-byte value per
    // accumulator element; the two X stages hold the four waves' tiles
    // (MTW 16 rows x NSW 16 columns x 2 bytes each). In a wave's region row
    // r, column c sits at r * RB + 16 * ((c / 8) ^ x(r)) + 2 * (c % 8) with
    // x(r) = 2 ((r / 4) % 4) mod the chunks per row: the four row groups a
    // write instruction touches fall in different 16-byte chunks. Rows beyond M and strips beyond N dropped.
    constexpr int RB = NSW * 32;  // bytes per row of a wave's tile
    static_assert(WAVES * MTW * 16 * RB <= 2 * STAGE, "the wave tiles must fit the X stages");
    static_assert(NSW % 2 == 0 || NSW == 1, "16-byte row chunks");
    if (S == 1 && NSW % 2 == 0) {
        __syncthreads();  // every wave is done with the last X stage
        uint8_t *wt = lds + wave * (MTW * 16 * RB);
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int j = 0; j < NSW; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = mt * 16 + 4 * kq + e, cc = j * 16 + col;
                    *reinterpret_cast<uint16_t *>(wt + r * RB + 16 * ((cc >> 3) ^ ((2 * ((r >> 2) & 3)) & (RB / 16 - 1))) + 2 * (cc & 7)) =
                        f32_to_f16_bits(acc[mt][j][e]);
                }
        // each read covers RB / 16 chunks of 64 / (RB / 16) rows
        constexpr int CPR = RB / 16;          // 16-byte chunks per row
        constexpr int RPI = 64 / CPR;         // rows per instruction
        const int k = lane % CPR, rr = lane / CPR;
        const int s = strip_w + k / 2;
#pragma unroll
        for (int i = 0; i < MTW * 16 / RPI; ++i) {
            const int r = i * RPI + rr;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(wt + r * RB + 16 * (k ^ ((2 * ((r >> 2) & 3)) & (CPR - 1))));
            const int row = m0 + rbase + r;
            if (row < M && s < nstrip)
                *reinterpret_cast<u32x4 *>(Y + (size_t)row * N + (size_t)strip_w * kStripCols + 8 * k) = v;
        }
        return;
    }
    // Split K: the fp32 partial tile takes the same route, half of the
    // wave's rows at a time (a whole fp32 tile is twice the X stages), with
    // 16-byte chunks of 4 columns and x(r) = 4 ((r / 4) % 4) mod the chunks
    // per row. A wave reuses only its own region, and its LDS operations
    // complete in order, so the halves need no barrier between them.
    if (S > 1 && NSW % 2 == 0) {
        constexpr int RB4 = NSW * 64;   // bytes per fp32 row
        constexpr int HR = MTW * 8;     // rows per half
        constexpr int CPR4 = RB4 / 16;  // 16-byte chunks per row
        constexpr int RPI4 = 64 / CPR4; // rows per read instruction
        static_assert(WAVES * HR * RB4 <= 2 * STAGE, "half wave tiles must fit the X stages");
        __syncthreads();  // every wave is done with the last X stage
        uint8_t *wt = lds + wave * (HR * RB4);
        const int k = lane % CPR4, rr = lane / CPR4;
        const int s = strip_w + k / 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int mt = 0; mt < MTW / 2; ++mt)
#pragma unroll
                for (int j = 0; j < NSW; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = mt * 16 + 4 * kq + e, cc = j * 16 + col;
                        *reinterpret_cast<float *>(wt + r * RB4 + 16 * ((cc >> 2) ^ ((4 * ((r >> 2) & 3)) & (CPR4 - 1))) +
                                                   4 * (cc & 3)) = acc[h * (MTW / 2) + mt][j][e];
                    }
#pragma unroll
            for (int i = 0; i < HR / RPI4; ++i) {
                const int r = i * RPI4 + rr;
                const floatx4 v = *reinterpret_cast<const floatx4 *>(wt + r * RB4 + 16 * (k ^ ((4 * ((r >> 2) & 3)) & (CPR4 - 1))));
                const int row = m0 + rbase + h * HR + r;
                if (row < M && s < nstrip)
                    *reinterpret_cast<floatx4 *>(part + ((size_t)split * M + row) * N + (size_t)strip_w * kStripCols + 4 * k) = v;
            }
        }
        return;
    }
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int j = 0; j < NSW; ++j) {
            const int s = strip_w + j;
            if (s >= nstrip) continue;
            const size_t n = (size_t)s * kStripCols + col;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + rbase + mt * 16 + 4 * kq + e;
                if (row >= M) continue;
                if (S == 1)
                    Y[(size_t)row * N + n] = f32_to_f16_bits(acc[mt][j][e]);
                else
                    part[((size_t)split * M + row) * N + n] = acc[mt][j][e];
            }
        }
}

// Sum of the S fp32 partials in split order, rounded once to fp16: four
// outputs per thread (one 16-byte load per split, one 8-byte store); M N is
// a multiple of four (N % 16 == 0).
__global__ void __launch_bounds__(256)
prefill_reduce_kernel(const floatx4 *__restrict__ part, uint32_t *__restrict__ Y, int64_t n4, int S) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x) {
        floatx4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int s = 0; s < S; ++s) v += part[(size_t)s * n4 + i];
        Y[2 * i] = (uint32_t)f32_to_f16_bits(v[0]) | ((uint32_t)f32_to_f16_bits(v[1]) << 16);
        Y[2 * i + 1] = (uint32_t)f32_to_f16_bits(v[2]) | ((uint32_t)f32_to_f16_bits(v[3]) << 16);
    }
}

// ------------------------------------------------------------- configurations
struct Cfg {
    int mtw, nsw, wm, wn, occ;
};

// Instantiated shapes (index = W4A16_PREFILL_CFG for tuning).
constexpr Cfg kCfgs[] = {
    {16, 4, 1, 4, 1},  // 0: 256 x 256, 4 waves, 1 wave/SIMD
    {8, 4, 2, 4, 2},   // 1: 256 x 256, 8 waves, 2 waves/SIMD
    {8, 4, 1, 4, 2},   // 2: 128 x 256, 4 waves, 2 WGs/CU
    {4, 4, 1, 4, 2},   // 3:  64 x 256
    {8, 2, 2, 4, 2},   // 4: 256 x 128, 8 waves
    {4, 4, 2, 4, 2},   // 5: 128 x 256, 8 waves
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

template <int CI, int GS>
hipError_t launch_cfg_g(const uint16_t *X, const uint8_t *packed, int M, int N, int K, uint16_t *Y,
                        float *part, int S, int slice_blocks, hipStream_t stream) {
    constexpr Cfg c = kCfgs[CI];
    constexpr int BM = c.wm * c.mtw * 16, BN = c.wn * c.nsw * 16;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    hipLaunchKernelGGL((prefill_kernel<c.mtw, c.nsw, c.wm, c.wn, GS, c.occ>),
                       dim3((unsigned)(tiles_m * tiles_n), (unsigned)S), dim3(c.wm * c.wn * 64), 0, stream, X,
                       packed, Y, part, M, N, K, tiles_m, tiles_n, S, slice_blocks);
    return hipGetLastError();
}

template <int CI>
hipError_t launch_cfg(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G, uint16_t *Y,
                      float *part, int S, int slice_blocks, hipStream_t stream) {
    switch (G) {
        case 32: return launch_cfg_g<CI, 1>(X, packed, M, N, K, Y, part, S, slice_blocks, stream);
        case 64: return launch_cfg_g<CI, 2>(X, packed, M, N, K, Y, part, S, slice_blocks, stream);
        case 128: return launch_cfg_g<CI, 4>(X, packed, M, N, K, Y, part, S, slice_blocks, stream);
        case 256: return launch_cfg_g<CI, 8>(X, packed, M, N, K, Y, part, S, slice_blocks, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_index(int ci, const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G,
                        uint16_t *Y, float *part, int S, int slice_blocks, hipStream_t stream) {
    switch (ci) {
        case 0: return launch_cfg<0>(X, packed, M, N, K, G, Y, part, S, slice_blocks, stream);
        case 1: return launch_cfg<1>(X, packed, M, N, K, G, Y, part, S, slice_blocks, stream);
        case 2: return launch_cfg<2>(X, packed, M, N, K, G, Y, part, S, slice_blocks, stream);
        case 3: return launch_cfg<3>(X, packed, M, N, K, G, Y, part, S, slice_blocks, stream);
        case 4: return launch_cfg<4>(X, packed, M, N, K, G, Y, part, S, slice_blocks, stream);
        default: return launch_cfg<5>(X, packed, M, N, K, G, Y, part, S, slice_blocks, stream);
    }
}

struct PrefillPlan {
    int ci, splits, slice_blocks;
};

// Tile shape by M (64-row tiles up to M = 128, 128-row tiles above); split
// K so that one round of resident workgroups covers the GPU: the largest
// split count whose tiles x splits still fit in one round. (A count that
// spills into a second, mostly empty round costs more than it gains:
// graph-timed on MI355X, 8192 x 10240 at M = 512 took 125 us with 3 splits
// of its 160 tiles and 150 us with 4; 8192 x 57344 at M = 256 took 241 us
// unsplit and 297 us with 2 splits of its 448 tiles.)
// W4A16_PREFILL_CFG overrides the shape (tuning).
PrefillPlan prefill_plan(int M, int N, int K, int G, int splits, int num_cus) {
    PrefillPlan p;
    p.ci = M <= 128 ? 3 : 2;
    if (const char *e = getenv("W4A16_PREFILL_CFG")) {
        const int v = atoi(e);
        if (v >= 0 && v < kNumCfgs) p.ci = v;
    }
    const Cfg c = kCfgs[p.ci];
    const int BM = c.wm * c.mtw * 16, BN = c.wn * c.nsw * 16;
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int nblk = K / kBlockK;
    const int per_cu = c.occ * 4 / (c.wm * c.wn) > 0 ? c.occ * 4 / (c.wm * c.wn) : 1;  // resident WGs per CU
    if (splits <= 0) {
        const int slots = num_cus * per_cu;
        splits = tiles >= slots ? 1 : slots / tiles;
        // keep 16+ blocks of K per split: below that the fp32 partials
        // (written, then read back by the reduce kernel) cost more than the
        // idle slots (graph-timed, 3584 x 8192 at M = 1024: 82.3 us with 2
        // splits of 14 blocks, 69.8 us unsplit)
        const int cap = nblk / 16 > 1 ? nblk / 16 : 1;
        if (splits > cap) splits = cap;
    }
    if (splits > nblk) splits = nblk;
    const int unit = G > kBlockK ? G / kBlockK : 1;
    int sb = (nblk + splits - 1) / splits;
    sb = (sb + unit - 1) / unit * unit;
    p.slice_blocks = sb;
    p.splits = (nblk + sb - 1) / sb;
    return p;
}

}  // namespace

int prefill_auto_splits(int M, int N, int K, int G, int num_cus) {
    return prefill_plan(M, N, K, G, 0, num_cus).splits;
}

size_t prefill_workspace_bytes(int M, int N, int K, int G, int splits) {
    const PrefillPlan p = prefill_plan(M, N, K, G, splits, 256);
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_prefill(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G,
                          uint16_t *Y, void *workspace, int splits, int num_cus, hipStream_t stream) {
    const PrefillPlan p = prefill_plan(M, N, K, G, splits, num_cus);
    float *part = p.splits > 1 ? static_cast<float *>(workspace) : nullptr;
    hipError_t e = launch_index(p.ci, X, packed, M, N, K, G, Y, part, p.splits, p.slice_blocks, stream);
    if (e != hipSuccess || p.splits <= 1) return e;
    const int64_t n4 = (int64_t)M * N / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(prefill_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const floatx4 *>(part), reinterpret_cast<uint32_t *>(Y), n4, p.splits);
    return hipGetLastError();
}

}  // namespace w4a16
