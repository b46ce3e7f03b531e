// Decode path of the W4A16 GEMM: small M (<= 64), bound by HBM bandwidth.
//
// Each generated token streams every weight byte once, so at small M the
// GEMM is limited by memory bandwidth, not arithmetic ("LMDeploy" interview
// notes, answer to why W4A16 raises throughput although FLOPs do not change;
// "LMDeploy, in depth", section "Quantization: AWQ weights and KV cache").
// The kernel is built around what runs out first on gfx950 when every 1 KiB
// weight tile also needs activations and scales: not DRAM bandwidth but the
// rate at which a CU can pull cache lines into its L1 (about one 128-byte
// line per 1.1 ns) and its VALU time for the dequantization.
//
// * Work unit: one 1 KiB packed tile (16 columns x 128 rows of K), read by
//   one wave64 with one 16-byte buffer load per lane. A workgroup owns NS
//   adjacent 16-column strips and one of S slices of K; its WK waves split
//   the slice into contiguous runs of 128-row blocks and each wave streams
//   all NS strips of its run, two batches of tiles in flight.
// * Scales and zeros of a wave's strips and run are staged in its own LDS
//   region once, already turned into the fp16 pair -(1024 + z) and the fp32
//   scale, so the main loop reads them with one LDS load per group and strip.
// * Activations. M = 1: the row of X over the wave's run is staged in LDS
//   before the main loop (a few KiB). 2 <= M <= 64: each batch of weight
//   tiles travels with the X rows of its blocks, copied straight into a
//   two-slot LDS ring by 16-byte buffer->LDS loads that each move four rows
//   x 256 bytes (whole 128-byte lines). The per-CU cost of X is the number of
//   cache lines it pulls in; A operands loaded straight into registers (16
//   rows x 64 bytes per instruction) would use half of each line they touch,
//   the ring uses all of it. Rows >= M of the 16-row MFMA tiles are padding:
//   their results are never stored.
// * Dequantization ("LMDeploy Guide: Fast Mixed-Precision LLM Inference
//   Engine", section 3, FP16 = (INT4 - ZeroPoint) x Scale): one v_and_or_b32
//   per pair of codes sets the fp16 exponent field and yields 1024 + q (low
//   nibbles) or 64 + q (high nibbles, no shift needed); a packed fp16 add of
//   -(1024 + z) or -(64 + z) leaves the exact integer q - z, which the matrix
//   instruction multiplies with X. The scale is applied in fp32 once per
//   group and column to the group's partial sum. The integer work of one
//   tile is independent of the other tiles in flight, so it interleaves with
//   the matrix instructions and the loads (the pages' ILP point).
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

// One batch of weight tiles in flight: NB blocks of the wave's NS strips,
// and with RB the scale and zero-code of every group the batch's blocks
// start (one fp16 scale and one byte holding the zero nibble per lane).
template <int NS, int NB, int NF, bool RB>
struct DecodeBatch {
    u32x4 w[NB][NS];
    uint32_t sc[RB ? NB : 1][NS][NF];
    uint32_t zb[RB ? NB : 1][NS][NF];
};

// Dynamic LDS: one private region per wave, back to back, holding the
// records of the wave's groups, [NS][ngw][16], and in staged-run mode the
// rows of X over the wave's run of blocks, [M][x_stride]. X arrives by direct
// buffer-to-LDS loads of 1 KiB (4 blocks of one row) per instruction, so a
// row slot holds whole KiB chunks, plus 16 bytes that put consecutive rows in
// different banks. The cross-wave reduction buffer [WK][NS][MT][64] of float4
// follows the regions where the plan's LDS budget allows (sep), so that a
// wave can write its partial tile while others still read their regions;
// otherwise it reuses the regions after a barrier.
struct DecodeLds {
    uint32_t ngw;         // record groups per wave region
    uint32_t sz_bytes;    // records per wave region
    uint32_t x_stride;    // bytes per staged row of X
    uint32_t wave_bytes;  // one wave region
    uint32_t red_bytes;
    uint32_t regions;     // WK * wave_bytes
    uint32_t red_off;     // byte offset of the reduction buffer
    uint32_t tot;
    __host__ __device__ uint32_t total() const { return tot; }
};

// X modes of decode_kernel
constexpr int kXRun = 1;  // the wave's run of X staged in LDS up front
// 8, 16, 32 or 64: the X rows of each batch's blocks in an LDS ring of that
// many rows (8 for M <= 8, else 16 per 16-row MFMA tile)

__host__ __device__ inline DecodeLds decode_lds(int M, int MT, int NS, int WK, int slice_blocks, int G,
                                                 int xm, bool rb, bool sep = false) {
    DecodeLds l;
    const int per = (slice_blocks + WK - 1) / WK;
    // a run that starts inside a group (G > 128) touches one group more
    l.ngw = (uint32_t)((per * kBlockK + G - 1) / G + (G > kBlockK ? 1 : 0));
    l.sz_bytes = rb ? 0u : (uint32_t)(NS * l.ngw * 16 * sizeof(SZ));
    l.x_stride = (uint32_t)((per + 3) / 4 * 1024 + 16);
    l.wave_bytes = l.sz_bytes + (xm == kXRun ? (uint32_t)M * l.x_stride : 0u);
    l.red_bytes = (uint32_t)(WK * NS * MT * 64 * 16);
    l.regions = (uint32_t)WK * l.wave_bytes;
    l.red_off = sep ? (l.regions + 15u) & ~15u : 0u;
    l.tot = sep ? l.red_off + l.red_bytes : (l.regions > l.red_bytes ? l.regions : l.red_bytes);
    return l;
}

// Cache policy of the weight loads: non-temporal. Every weight byte is read
// once per call, so the stream should not evict the kernel's code, X, the
// scale records or split-K partials from L2.
constexpr int kWeightLoadPolicy = 2;  // nt

// One 128-row block of NS strips: for each of the block's scale groups the
// matrix instruction runs over its 32-row steps with the exact integer
// weights q - z, and the group's partial products are scaled into acc in
// fp32. rec points at the records of the first strip; strip j's records
// start rec_stride groups later, and gbase is the group index of the first
// record.
// With RB the records come from the batch (bsc, bzb: [NS][NF] of block b)
// instead of the LDS region.
template <int MT, int NS, int GS, bool RB>
__device__ __forceinline__ void block_mma(const half8 (&a)[4][MT], const u32x4 (&w)[NS], const SZ *rec,
                                          int rec_stride, int b, int gbase, int col, uint32_t m_lo,
                                          uint32_t m_hi, const uint32_t (&bsc)[NS][GS < 4 ? 4 / GS : 1],
                                          const uint32_t (&bzb)[NS][GS < 4 ? 4 / GS : 1],
                                          floatx4 (&acc)[MT][NS]) {
    constexpr int F = GS < 4 ? GS : 4;  // 32-row k-steps per scale group inside a block
    constexpr int NF = 4 / F;            // scale groups per 128-row block
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        u32x4 w8;
#pragma unroll
        for (int v = 0; v < 4; ++v) w8[v] = w[j][v] >> 8;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            SZ sz;
            if constexpr (RB) {
                const uint32_t hz = 0xE400u | ((bzb[j][f] >> ((col & 1) * 4)) & 15u);
                sz.nb = hz | (hz << 16);
                sz.sc = (float)__builtin_bit_cast(_Float16, (uint16_t)bsc[j][f]);
            } else {
                const int g = (b * 4 + f * F) / GS;
                sz = rec[(j * rec_stride + (g - gbase)) * 16 + col];
            }
            const DequantConsts dc{sz.nb, neg_bias64_from_1024(sz.nb), m_lo, m_hi};
            floatx4 part[MT];
#pragma unroll
            for (int tt = 0; tt < F; ++tt) {
                const int t = f * F + tt;
                const half8 bq = dequant_qz(t, w[j], w8, dc);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    part[mt] = mfma16x16x32(a[t][mt], bq, tt ? part[mt] : floatx4{0.f, 0.f, 0.f, 0.f});
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[mt][j][e] = __builtin_fmaf(sz.sc, part[mt][e], acc[mt][j][e]);
        }
    }
}

// Converts half a group record (8 columns: 8 fp16 scales, 8 four-bit zero
// codes) into 8 LDS records.
__device__ __forceinline__ void store_records(SZ *dst, const u32x4 &sv, uint32_t zv) {
    u32x4 *d = reinterpret_cast<u32x4 *>(dst);
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
        u32x4 rec2;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t hz = 0xE400u | ((zv >> (4 * (2 * c2 + h))) & 15u);
            rec2[2 * h] = hz | (hz << 16);
            rec2[2 * h + 1] =
                __builtin_bit_cast(uint32_t, (float)__builtin_bit_cast(_Float16, (uint16_t)(sv[c2] >> (16 * h))));
        }
        d[c2] = rec2;
    }
}

template <int MT, int NS, int WK, int NB, int GS, int XM, bool RB>
__global__ void __launch_bounds__(WK * 64)
decode_kernel(const uint16_t *__restrict__ X, const uint8_t *__restrict__ packed,
              uint16_t *__restrict__ Y, float *__restrict__ part, int M, int N, int K, int S,
              int slice_blocks, int sep) {
    constexpr int G = 32 * GS;
    constexpr int F = GS < 4 ? GS : 4;
    constexpr int NF = 4 / F;
    constexpr bool kRun = XM == kXRun;
    constexpr bool kRing = XM >= 8;
    static_assert(!kRing || (MT == 1 && XM == 8) || XM == 16 * MT, "ring rows: 8, or 16 per row tile");
    static_assert(kRun || kRing, "X mode");
    // X copies per block: one ring copy per 4 rows (the staged run has none)
    constexpr int kXLoads = kRing ? XM / 4 : 0;
    // loads of one batch and of the two batches issued ahead of the loop
    constexpr int kBatchLoads = NB * (NS * (RB ? 1 + 2 * NF : 1) + kXLoads);
    static_assert(2 * kBatchLoads <= 63, "vmcnt range");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // Ring mode: slot i of ring0 (ring1) holds X rows [0, XM) of block i of
    // the batch in flight in b0 (b1), [row][256 bytes] with the sixteen
    // 16-byte chunks of row r stored at position chunk ^ (r & 15), so the 16
    // lanes that read one chunk of 16 rows hit 16 different bank groups. Two
    // arrays, so that the compiler sees that a batch's reads and the other
    // batch's copies touch different memory.
    constexpr int kSlot = kRing ? XM * kBlockK * 2 : 16;
    static_assert(!kRing || 2 * WK * NB * kSlot <= 160 * 1024, "ring exceeds the LDS");
    __shared__ __attribute__((aligned(16))) uint8_t ring0[kRing ? WK * NB * kSlot : 16];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[kRing ? WK * NB * kSlot : 16];

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
    const int per = (slice_blocks + WK - 1) / WK;
    const int wb = bb + wk * per < be ? bb + wk * per : be;
    const int we = wb + per < be ? wb + per : be;
    const int gw0 = wb * kBlockK / G;  // groups overlapping the wave's run
    const int ngw = (we * kBlockK + G - 1) / G - gw0;

    const DecodeLds L = decode_lds(M, MT, NS, WK, slice_blocks, G, XM, RB, sep != 0);
    SZ *szl = reinterpret_cast<SZ *>(lds + wk * L.wave_bytes);
    uint8_t *xl = lds + wk * L.wave_bytes + L.sz_bytes;
    uint8_t *xr0 = ring0 + wk * NB * kSlot;
    uint8_t *xr1 = ring1 + wk * NB * kSlot;

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
        if constexpr (kRun)  // rows >= M read row M-1: padding rows are never stored
            xoff[mt] = (uint32_t)((row < M ? row : M - 1) * L.x_stride + kq * 16);
        else  // ring rows >= M hold zeros; rows >= XM (M <= 8) repeat rows < 8
            xoff[mt] = (uint32_t)((row & (XM - 1)) * kBlockK * 2);
    }
    // ring copies: copy xi moves rows 4 xi .. 4 xi + 3 of a block, lane ->
    // row 4 xi + lane / 16, 16-byte chunk (lane & 15) ^ row, written to LDS
    // position lane. Copies xi and xi + 4 share the chunk order (rows 16
    // apart), so the per-lane offsets repeat with period 4 and the 16-row
    // step goes into the scalar offset. Rows >= M lie past the end of X's
    // descriptor and read as zeros.
    uint32_t xsrc[4];
#pragma unroll
    for (int xi = 0; xi < 4; ++xi) {
        const int r = xi * 4 + (lane >> 4);
        xsrc[xi] = (uint32_t)(r * K * 2 + (((lane & 15) ^ (r & 15)) * 16));
    }
    const uint32_t m_lo = kMagic, m_hi = kMagic64;

    floatx4 acc[MT][NS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[mt][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // scale and zero-code records of the workgroup's strips (strips past N
    // lie past the descriptors and read as zeros)
    const int nsv = nstrip - strip0 < NS ? nstrip - strip0 : NS;  // strips that exist
    const uint8_t *srec = packed + weight_bytes(K, N) + (size_t)strip0 * ngrp * 32;
    const uint8_t *zrec = packed + weight_bytes(K, N) + scale_bytes(K, N, G) + (size_t)strip0 * ngrp * 8;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(srec, (uint32_t)(nsv * ngrp * 32));
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(zrec, (uint32_t)(nsv * ngrp * 8));

    typedef DecodeBatch<NS, NB, NF, RB> Batch;
    // Blocks at or past the end of the wave's run load from the out-of-range
    // offset: no branch, no memory traffic, and the same instruction count
    // on every path. X rows >= M are out of range of X's descriptor too.
    auto load = [&](int b0, Batch &bt, uint8_t *xr) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const bool in = b0 + i < we;
            const uint32_t wo = in ? (uint32_t)lane * 16u : kOobOffset;
            if constexpr (kRing) {
                // the slots being refilled were read by the previous
                // compute: those LDS reads complete before the copies start
                if (i == 0) __builtin_amdgcn_s_waitcnt(kLgkmZero);
#pragma unroll
                for (int xi = 0; xi < XM / 4; ++xi)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(xr + i * kSlot + xi * 1024), 16,
                                                             in ? xsrc[xi & 3] : kOobOffset,
                                                             (b0 + i) * kBlockK * 2 + (xi >> 2) * 32 * K, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                if constexpr (RB) {
                    // this lane's column: its fp16 scale and the byte holding
                    // its zero code, for each group the block starts
#pragma unroll
                    for (int f = 0; f < NF; ++f) {
                        const uint32_t rec = (uint32_t)(j * ngrp + ((b0 + i) * 4 + f * F) / GS);
                        bt.sc[i][j][f] = __builtin_amdgcn_raw_buffer_load_b16(rs, in ? rec * 32u + col * 2u : kOobOffset,
                                                                              0, 0);
                        bt.zb[i][j][f] = __builtin_amdgcn_raw_buffer_load_b8(rz, in ? rec * 8u + (col >> 1) : kOobOffset,
                                                                             0, 0);
                    }
                }
                bt.w[i][j] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw[j], wo, (b0 + i) * kTileBytes, kWeightLoadPolicy));
            }
        }
    };
    auto compute = [&](int b0, const Batch &bt, const uint8_t *xr) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int b = b0 + i;
            if (b >= we) break;
            half8 a[4][MT];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if constexpr (kRun)
                        a[t][mt] = *reinterpret_cast<const half8 *>(
                            xl + xoff[mt] + ((b - wb) * kBlockK + t * 32) * 2);
                    else
                        a[t][mt] = *reinterpret_cast<const half8 *>(
                            xr + i * kSlot + xoff[mt] + (((4 * t + kq) ^ col) * 16));
                }
            block_mma<MT, NS, GS, RB>(a, bt.w[i], szl, (int)L.ngw, b, gw0, col, m_lo, m_hi, bt.sc[RB ? i : 0],
                                      bt.zb[RB ? i : 0], acc);
        }
    };

    if (wb < we) {  // uniform per wave; waves without blocks only join the reduction
        // ---- staging into the wave's own LDS region: the records of its
        // groups and (LDS-X mode) its rows of X. These loads go out before the
        // first two weight batches, so waiting for them leaves the weight
        // loads in flight (vector loads complete in order). A record unit is
        // half a group record (8 columns: 16 bytes of scales, 4 bytes of zero
        // codes), one per lane; units past the first 64 (long runs only)
        // follow after a full wait. With RB (plans whose runs fit in the two
        // batches issued up front) the records travel with the batches
        // instead: no staging round trip before the first tile, at the cost
        // of two small loads per strip and group.
        const int su_n = NS * ngw * 2;

        auto sz_load = [&](int u, u32x4 &sv, uint32_t &zv) {
            const int j = u / (ngw * 2), r = u % (ngw * 2);
            const bool ok = u < su_n && j < nsv;
            const uint32_t rec = (uint32_t)(j * ngrp + gw0 + (r >> 1));
            sv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rs, ok ? rec * 32u + (r & 1) * 16u : kOobOffset, 0, 0));
            zv = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rz, ok ? rec * 8u + (r & 1) * 4u : kOobOffset,
                                                               0, 0);
        };
        auto sz_store = [&](int u, const u32x4 &sv, uint32_t zv) {
            if (u >= su_n) return;
            const int j = u / (ngw * 2), r = u % (ngw * 2);
            store_records(szl + (j * (int)L.ngw + (r >> 1)) * 16 + (r & 1) * 8, sv, zv);
        };

        u32x4 sv0;
        uint32_t zv0;
        if constexpr (!RB) sz_load(lane, sv0, zv0);
        if constexpr (kRun) {
            // row r, chunk c: blocks [wb + 4c, wb + 4c + 4) of row r; lanes
            // past the run read zeros into the slot's spare bytes
            const int run = we - wb, nch = (run + 3) / 4;
            for (int r = 0; r < M; ++r)
                for (int c = 0; c < nch; ++c) {
                    const bool ok = c * 64 + lane < run * 16;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rx, (lds_void *)(xl + r * L.x_stride + c * 1024), 16,
                        ok ? (uint32_t)(r * K * 2 + lane * 16) : kOobOffset, (wb * kBlockK + c * 512) * 2, 0, 0);
                }
        }
        asm volatile("" ::: "memory");  // staging loads go out first
        Batch b0, b1;
        int b = wb;
        load(b, b0, xr0);
        asm volatile("" ::: "memory");  // keep the two batches apart in issue order
        load(b + NB, b1, xr1);
        asm volatile("" ::: "memory");
        if constexpr (!RB || kRun) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kBatchLoads));  // staging loads landed
            if constexpr (!RB) {
                sz_store(lane, sv0, zv0);
                for (int u = 64 + lane; u - lane < su_n; u += 64) {
                    u32x4 a;
                    uint32_t z;
                    sz_load(u, a, z);
                    sz_store(u, a, z);
                }
            }
            // the region is private to the wave: order its writes before its reads
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }

        // Two batches in flight: consume one, refill it two batches ahead.
        // All rounds but the last refill unconditionally (only the final
        // refill can reach past the run, and those blocks are out of range);
        // the last round only consumes.
        const int rounds = (we - b + 2 * NB - 1) / (2 * NB);
        // The tiles' arithmetic runs at raised wave priority (the SIMD's
        // other waves, waiting on their loads, issue behind it): the same
        // results, up to 0.1 us less per launch (8B down projection at M = 1
        // 7.52 against 7.61 us, graph-timed).
        for (int r = 1; r < rounds; ++r, b += 2 * NB) {
            __builtin_amdgcn_s_setprio(1);
            compute(b, b0, xr0);
            __builtin_amdgcn_s_setprio(0);
            load(b + 2 * NB, b0, xr0);
            __builtin_amdgcn_s_setprio(1);
            compute(b + NB, b1, xr1);
            __builtin_amdgcn_s_setprio(0);
            load(b + 3 * NB, b1, xr1);
        }
        compute(b, b0, xr0);
        compute(b + NB, b1, xr1);
    }

    // ---- add the WK partial tiles of each strip in LDS, run 0 first. Where
    // the reduction buffer reuses the waves' record and X regions, every wave
    // must be done with its region first; where it has its own memory (or
    // there are no regions) a wave writes its tile as soon as its loop ends.
    if (L.regions > 0 && !sep) __syncthreads();
    floatx4 *red = reinterpret_cast<floatx4 *>(lds + L.red_off);  // [WK][NS][MT][64]
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

// Y = sum over s of part[s] in split order, fp32 -> fp16. Each thread owns
// four consecutive outputs and loads up to eight partials before adding any,
// so the reduction costs one memory round trip per eight splits instead of
// one per split; the additions still run in split order (bitwise equal to a
// plain loop).
__global__ void __launch_bounds__(64)
splitk_reduce_kernel(const float *__restrict__ part, uint16_t *__restrict__ Y, int64_t MN, int S) {
    typedef float floatx4_t __attribute__((ext_vector_type(4)));
    const int64_t n4 = MN / 4;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        const floatx4_t *p = reinterpret_cast<const floatx4_t *>(part) + i;
        floatx4_t v = floatx4_t{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < S; s0 += 8) {
            floatx4_t t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < S) t[u] = p[(s0 + u) * n4];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < S) v += t[u];
        }
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = f32_to_f16_bits(v[e]);
        reinterpret_cast<uint2 *>(Y)[i] = uint2{(uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                               (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    }
}

inline int decode_mt(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

// ---------------------------------------------------------------- planning
constexpr uint32_t kLdsBudget = 64 * 1024;
constexpr uint32_t kLdsMax = 160 * 1024;  // per CU on gfx950

struct Plan {
    int mt, ns, wk;
    int xm;             // decode_kernel X mode: kXRun, or ring rows (8, 16, 32, 64)
    bool fixed_splits;  // automatic plan keeps K unsplit
    int splits, slice_blocks;
    bool rb;            // records loaded with each batch (runs of at most two batches)
    bool sep;           // the cross-wave reduction buffer after the wave regions (see DecodeLds)
};

int env_int(const char *name, int dflt) {
    const char *v = getenv(name);
    return v ? atoi(v) : dflt;
}

// Launch shape, picked from graph-timed sweeps on MI355X over the decode
// matrices of Llama-3-8B (QKV 4096 x 6144, down 14336 x 4096) and Llama-3-70B
// (gate/up 8192 x 57344, down 28672 x 8192):
// * M = 1: X staged per run in LDS, 8 waves per workgroup, one strip per
//   wave (two where N is very wide);
// * 2 <= M <= 64: X through the LDS ring. Short K with narrow N (QKV-like):
//   K unsplit, 2 strips x 16 waves (x 4 waves for M > 16). Very wide N: 2
//   strips x 4 waves, plenty of workgroups. Otherwise about one workgroup
//   per CU with K unsplit for M <= 8 (16 waves); for larger M twice the
//   strips per workgroup and K split in two, which halves the X each CU has
//   to read (4 strips x 4 waves for 17 <= M <= 32, 2 x 4 above).
// W4A16_DECODE_XM (1: staged run, M <= 16; 2: ring, M >= 2), _NS and _WK
// override the X mode, NS and WK for tuning (instantiated values only).
Plan base_plan(int M, int N, int K) {
    Plan p;
    p.mt = decode_mt(M);
    p.xm = M == 1 ? kXRun : (M <= 8 ? 8 : 16 * p.mt);
    const int nstrip = N / kStripCols, nblk = K / kBlockK;
    const bool short_narrow = nstrip <= 384 && nblk <= 64;
    if (p.xm == kXRun) {
        p.ns = nstrip >= 2048 ? 2 : 1;
        p.wk = 8;
    } else if (short_narrow || nstrip >= 1024) {
        p.ns = 2;
        p.wk = short_narrow && p.mt == 1 ? 16 : 4;
    } else if (p.mt == 1) {
        int ns = nstrip / 256;
        ns = ns < 1 ? 1 : (ns > 2 ? 2 : ns);
        p.ns = M <= 8 ? ns : 2 * ns;
        p.wk = M <= 8 ? 16 : 8;
    } else {
        p.ns = p.mt == 2 ? 4 : 2;
        p.wk = 4;
    }
    p.fixed_splits = p.xm != kXRun && short_narrow;
    const int exm = env_int("W4A16_DECODE_XM", -1);
    if (exm == 1 && p.mt == 1) p.xm = kXRun;
    if (exm == 2 && M > 1) p.xm = M <= 8 ? 8 : 16 * p.mt;
    const int ens = env_int("W4A16_DECODE_NS", 0), ewk = env_int("W4A16_DECODE_WK", 0);
    if (ens == 1 || ens == 2 || ens == 4) p.ns = ens;
    if (p.mt == 4 && p.ns == 4) p.ns = 2;
    if (ewk == 4 || ewk == 8 || (ewk == 16 && p.mt == 1)) p.wk = ewk;
    if (p.mt > 1 && p.wk > 8) p.wk = 8;
    if (p.xm == 64) p.wk = 4;  // two 64-row slots per wave: 128 KiB of LDS at 4 waves
    p.splits = 1;
    p.slice_blocks = 0;
    p.rb = false;
    p.sep = false;
    // no more waves than blocks of K (idle waves would still hold LDS)
    while (p.wk > 4 && p.wk > nblk) p.wk /= 2;
    // the cross-wave reduction buffer must leave room for the staged records
    while (p.wk * p.ns * p.mt * 64 * 16 > 32 * 1024 && p.wk > 4) p.wk /= 2;
    while (p.wk * p.ns * p.mt * 64 * 16 > 32 * 1024 && p.ns > 1) p.ns /= 2;
    return p;
}

// Blocks per split for a split count: whole groups per slice.
int slice_for(int K, int G, int splits) {
    const int nblk = K / kBlockK;
    const int unit = G > kBlockK ? G / kBlockK : 1;
    int sb = (nblk + splits - 1) / splits;
    return (sb + unit - 1) / unit * unit;
}

// Batches of 2 tiles per wave only for single-strip single-tile waves
// without an LDS ring (the ring holds one block per batch).
constexpr int decode_nb(int MT, int NS, int XM) { return (NS == 1 && MT == 1 && XM <= kXRun) ? 2 : 1; }

// Records with the batches need 2 (NF) more loads per strip and block; the
// two batches issued ahead must stay within the vector-memory counter.
constexpr bool rb_fits(int MT, int NS, int XM, int GS) {
    const int nf = GS < 4 ? 4 / GS : 1;
    const int xloads = XM >= 8 ? XM / 4 : 0;
    return MT == 1 && 2 * decode_nb(MT, NS, XM) * (NS * (1 + 2 * nf) + xloads) <= 63;
}

// Static LDS of the ring mode: two rings of WK x NB slots of XM rows.
uint32_t ring_lds(const Plan &p) {
    return p.xm >= 8 ? (uint32_t)(2 * p.wk * decode_nb(p.mt, p.ns, p.xm) * p.xm * kBlockK * 2) : 0u;
}

uint32_t plan_lds(const Plan &p, int M, int G, int slice_blocks) {
    return decode_lds(M, p.mt, p.ns, p.wk, slice_blocks, G, p.xm, p.rb).total() + ring_lds(p);
}

// A plan may use all of a CU's LDS when it runs one workgroup per CU (the
// ring plans, or at most one workgroup per CU in all); the others keep to a
// budget that leaves room for two.
bool lds_fits(const Plan &p, int M, int G, int slice_blocks, long workgroups, int num_cus) {
    const bool one_per_cu = p.xm >= 8 || workgroups <= num_cus;
    return plan_lds(p, M, G, slice_blocks) <= (one_per_cu ? kLdsMax : kLdsBudget);
}

int plan_tiles(const Plan &p, int N) { return (N / kStripCols + p.ns - 1) / p.ns; }

Plan make_plan(int M, int N, int K, int G, int splits, int num_cus) {
    Plan p = base_plan(M, N, K);
    const int nblk = K / kBlockK;
    // Wider workgroups (more strips, to cut each CU's X reads) rely on
    // splitting K to keep every CU busy; where K is too short to split
    // that far, narrow them back until the workgroups cover the CUs
    // (graph-timed, K = 3584, N = 8192, M = 16: 4 strips unsplit 9.0 us,
    // 2 strips 6.9 us). The shape does not depend on the requested split
    // count, so a plan asked for with its own automatic count is the same.
    if (!p.fixed_splits && env_int("W4A16_DECODE_NS", 0) == 0) {
        auto reach = [&](const Plan &q) {
            const long t = plan_tiles(q, N);
            int cap = nblk / (2 * q.wk);
            if (cap < 1) cap = 1;
            const long sp = t < num_cus ? ((num_cus + t - 1) / t < cap ? (num_cus + t - 1) / t : cap) : 1;
            return t * sp;
        };
        while (p.ns > 1 && reach(p) < num_cus) p.ns /= 2;
    }
    const int tiles = plan_tiles(p, N);
    if (splits <= 0 && p.fixed_splits) splits = 1;
    if (splits <= 0) {
        // Narrow N: about one workgroup per CU, keeping at least two blocks
        // per wave.
        splits = 1;
        if (tiles < num_cus) {
            splits = (num_cus + tiles - 1) / tiles;
            int cap = nblk / (2 * p.wk);
            if (cap < 1) cap = 1;
            if (splits > cap) splits = cap;
        }
    }
    // enough splits for the LDS budget (also raises a requested count)
    auto fits = [&](int sp) {
        const int sb = slice_for(K, G, sp);
        return lds_fits(p, M, G, sb, (long)tiles * ((nblk + sb - 1) / sb), num_cus);
    };
    while (splits < nblk && !fits(splits)) ++splits;
    p.slice_blocks = slice_for(K, G, splits);
    p.splits = (nblk + p.slice_blocks - 1) / p.slice_blocks;
    // Records with the batches when a wave's whole run is in flight after
    // the first two batches (graph-timed on MI355X, 4096 x 6144: M = 1 5.72
    // -> 5.46 us, M = 8 6.44 -> 6.11, M = 16 7.32 -> 6.97; on longer runs
    // the per-batch record loads cost more than the staging saves: 14336 x
    // 4096 at M = 1, 7.97 -> 9.73 us). W4A16_DECODE_RB (0, 1) overrides.
    const int per = (p.slice_blocks + p.wk - 1) / p.wk;
    const bool ok = rb_fits(p.mt, p.ns, p.xm, G / 32);
    p.rb = ok && per <= 2 * decode_nb(p.mt, p.ns, p.xm);
    const int erb = env_int("W4A16_DECODE_RB", -1);
    if (ok && (erb == 0 || erb == 1)) p.rb = erb == 1;
    // a separate reduction buffer where the plan's budget still holds it
    // (the plan itself does not change); at M <= 16 only (graph-timed, 8B
    // shapes: M = 8 and 16 0.12-0.15 us faster per launch, M = 32 0.3 us
    // slower)
    if (p.mt == 1) {
        const long wgs = (long)tiles * p.splits;
        const bool one_per_cu = p.xm >= 8 || wgs <= num_cus;
        const uint32_t sep_lds =
            decode_lds(M, p.mt, p.ns, p.wk, p.slice_blocks, G, p.xm, p.rb, true).total() + ring_lds(p);
        p.sep = sep_lds <= (one_per_cu ? kLdsMax : kLdsBudget);
    }
    return p;
}

template <int MT, int NS, int WK, int GS, int XM, bool RB>
hipError_t launch_one(const uint16_t *X, const uint8_t *packed, int M, int N, int K, uint16_t *Y,
                      float *part, const Plan &p, hipStream_t stream) {
    constexpr int NB = decode_nb(MT, NS, XM);
    const DecodeLds L = decode_lds(M, MT, NS, WK, p.slice_blocks, 32 * GS, XM, RB, p.sep);
    const int tiles = (N / kStripCols + NS - 1) / NS;
    hipLaunchKernelGGL((decode_kernel<MT, NS, WK, NB, GS, XM, RB>), dim3(tiles, p.splits), dim3(WK * 64),
                       L.total(), stream, X, packed, Y, part, M, N, K, p.splits, p.slice_blocks, p.sep ? 1 : 0);
    return hipGetLastError();
}

template <int MT, int NS, int WK, int GS, int XM>
hipError_t launch_rb(const uint16_t *X, const uint8_t *packed, int M, int N, int K, uint16_t *Y, float *part,
                     const Plan &p, hipStream_t stream) {
    if constexpr (rb_fits(MT, NS, XM, GS)) {
        if (p.rb) return launch_one<MT, NS, WK, GS, XM, true>(X, packed, M, N, K, Y, part, p, stream);
    }
    return launch_one<MT, NS, WK, GS, XM, false>(X, packed, M, N, K, Y, part, p, stream);
}

template <int MT, int NS, int WK, int XM>
hipError_t launch_g(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G, uint16_t *Y,
                    float *part, const Plan &p, hipStream_t stream) {
    switch (G) {
        case 32: return launch_rb<MT, NS, WK, 1, XM>(X, packed, M, N, K, Y, part, p, stream);
        case 64: return launch_rb<MT, NS, WK, 2, XM>(X, packed, M, N, K, Y, part, p, stream);
        case 128: return launch_rb<MT, NS, WK, 4, XM>(X, packed, M, N, K, Y, part, p, stream);
        case 256: return launch_rb<MT, NS, WK, 8, XM>(X, packed, M, N, K, Y, part, p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int MT, int NS, int XM>
hipError_t launch_wk(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G, uint16_t *Y,
                     float *part, const Plan &p, hipStream_t stream) {
    if constexpr (XM == 64) {  // two 64-row ring slots per wave: 4 waves only
        return launch_g<MT, NS, 4, XM>(X, packed, M, N, K, G, Y, part, p, stream);
    } else {
        if constexpr (MT == 1) {
            if (p.wk == 16) return launch_g<MT, NS, 16, XM>(X, packed, M, N, K, G, Y, part, p, stream);
        }
        if (p.wk == 4) return launch_g<MT, NS, 4, XM>(X, packed, M, N, K, G, Y, part, p, stream);
        return launch_g<MT, NS, 8, XM>(X, packed, M, N, K, G, Y, part, p, stream);
    }
}

hipError_t launch_plan(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G, uint16_t *Y,
                       float *part, const Plan &p, hipStream_t stream) {
    switch (p.xm) {
        case kXRun:  // M = 1 (M <= 16 when tuning)
            switch (p.ns) {
                case 1: return launch_wk<1, 1, kXRun>(X, packed, M, N, K, G, Y, part, p, stream);
                case 2: return launch_wk<1, 2, kXRun>(X, packed, M, N, K, G, Y, part, p, stream);
                default: return launch_wk<1, 4, kXRun>(X, packed, M, N, K, G, Y, part, p, stream);
            }
        case 8:  // 2 <= M <= 8
            switch (p.ns) {
                case 1: return launch_wk<1, 1, 8>(X, packed, M, N, K, G, Y, part, p, stream);
                case 2: return launch_wk<1, 2, 8>(X, packed, M, N, K, G, Y, part, p, stream);
                default: return launch_wk<1, 4, 8>(X, packed, M, N, K, G, Y, part, p, stream);
            }
        case 16:  // 9 <= M <= 16
            switch (p.ns) {
                case 1: return launch_wk<1, 1, 16>(X, packed, M, N, K, G, Y, part, p, stream);
                case 2: return launch_wk<1, 2, 16>(X, packed, M, N, K, G, Y, part, p, stream);
                default: return launch_wk<1, 4, 16>(X, packed, M, N, K, G, Y, part, p, stream);
            }
        case 32:  // 17 <= M <= 32
            switch (p.ns) {
                case 1: return launch_wk<2, 1, 32>(X, packed, M, N, K, G, Y, part, p, stream);
                case 2: return launch_wk<2, 2, 32>(X, packed, M, N, K, G, Y, part, p, stream);
                default: return launch_wk<2, 4, 32>(X, packed, M, N, K, G, Y, part, p, stream);
            }
        case 64:  // 33 <= M <= 64
            if (p.ns == 1) return launch_wk<4, 1, 64>(X, packed, M, N, K, G, Y, part, p, stream);
            return launch_wk<4, 2, 64>(X, packed, M, N, K, G, Y, part, p, stream);
        default: return hipErrorInvalidValue;
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

size_t decode_workspace_bytes(int M, int N, int K, int G, int splits, int num_cus) {
    // a requested split count is rounded to whole groups per slice and
    // raised until the slice fits the LDS budget
    const Plan p = make_plan(M, N, K, G, splits, num_cus);
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_decode(const uint16_t *X, const uint8_t *packed, int M, int N, int K, int G,
                         uint16_t *Y, void *workspace, int splits, int num_cus, hipStream_t stream) {
    const Plan p = make_plan(M, N, K, G, splits, num_cus);
    if (!lds_fits(p, M, G, p.slice_blocks, (long)plan_tiles(p, N) * p.splits, num_cus))
        return hipErrorInvalidConfiguration;
    float *part = p.splits > 1 ? static_cast<float *>(workspace) : nullptr;
    hipError_t e = launch_plan(X, packed, M, N, K, G, Y, part, p, stream);
    if (e != hipSuccess || p.splits <= 1) return e;
    const int64_t MN = (int64_t)M * N;  // a multiple of 16
    int64_t blocks = (MN / 4 + 63) / 64;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, part, Y, MN,
                       p.splits);
    return hipGetLastError();
}

}  // namespace w4a16
