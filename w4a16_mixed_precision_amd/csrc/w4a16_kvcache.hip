// Low-bit KV cache and decode attention (the pages' second pipeline).
//
// KV quantization is online, asymmetric, per head and per token, 8 or 4 bits
// ("LMDeploy, in depth", "Quantization: AWQ weights and KV cache", paragraph
// on KV cache quantization); the cache is blocked, 64 tokens per block (same
// page, section on the blocked KV cache). Attention of one new query token
// per sequence reads the low-bit K and V straight from the cache
// ("LMDeploy Guide: Fast Mixed-Precision LLM Inference Engine", architecture
// figure, pipeline B; sections 2 "Adaptive Head Alignment" and 4
// "Asynchronous KV Memory Loading Pipeline").
//
// Scale and zero of a vector x of D = 128 numbers (L = 2^bits - 1 steps),
// the reading the weight quantizer uses:
//   s = fp16(max(fp32(max - min) / L, 2^-14)),
//   z = clamp(rint(-min / s), 0, L), c = clamp(rint(x / s) + z, 0, L)
// with rint the nearest integer to the exact quotient, ties to even (the
// zero and the codes by round_quotient_fp16).
//
// Cache region of one (block, KV head), KC = 64 * 128 * bits / 8 bytes:
//   [0, KC)        K codes, token-major rows of 128 codes
//   [KC, 2 KC)     V codes, rows d = 0..127 of 64 tokens in position order
//                  p(t) = 16 ((t % 16) / 4) + 8 (t / 32) + 4 ((t / 16) % 2) + t % 4
//   [2 KC, +256)   K parameters per token: fp16 scale, zero code, 0
//   [2 KC + 256, +256) V parameters per token
// (4-bit codes two per byte, the even index in the low nibble.)
//
// Decode attention on gfx950, one wave per (sequence, KV head, chunk of
// blocks):
// * S^T = K . Q^T on the matrix cores (16 x 16 x 32 fp16 MFMA): rows are 16
//   tokens, columns up to 16 query heads of the KV head's group. A lane's A
//   operand is one token's codes, 32 contiguous dimensions per lane (16 or
//   32 bytes): the dimension order inside the reduction is permuted so that
//   every lane reads contiguous codes, and the query is permuted the same way
//   once per wave (the pages' adaptive head alignment: the query is
//   rearranged once so that its slices match the low-bit key layout). The
//   codes enter as 1024 + c (exponent-OR, one instruction per two codes);
//   each score then loses (1024 + z) * sum(q) and is multiplied by the
//   token's scale times the softmax scale and log2 e.
// * Online softmax in fp32 per head (exp2).
// * O^T = V^T . P^T on the matrix cores: the V rows are stored index-major in
//   the position order above, which puts in each lane exactly the eight
//   tokens whose probabilities that lane already holds after the score
//   product, so P needs no data movement; V's per-token scale is folded into
//   P (rounded to fp16) and its zero subtracted exactly from the codes.
// * The loads of the next cache block are issued before the current one is
//   multiplied (two register sets), the pages' double-buffered KV pipeline.
// * Each wave writes a partial (max, sum, unnormalized O) per head; a second
//   kernel merges the chunks of a sequence (log-sum-exp).
#include <stdlib.h>

#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

constexpr int kHD = 128;    // head dimension
constexpr int kBS = 64;     // tokens per cache block
constexpr float kLog2e = 1.4426950408889634f;

template <int BITS>
struct KvGeom {
    static constexpr int kCodeBytes = kBS * kHD * BITS / 8;  // K (or V) codes of one region
    static constexpr int kRowBytes = kHD * BITS / 8;         // one K row
    static constexpr int kVRowBytes = kBS;                   // one V row: a byte per position
    static constexpr int kKPar = 2 * kCodeBytes;
    static constexpr int kVPar = 2 * kCodeBytes + 4 * kBS;
    static constexpr int kRegion = 2 * kCodeBytes + 8 * kBS;
};

__device__ inline int v_position(int t) { return 16 * ((t & 15) >> 2) + 8 * (t >> 5) + 4 * ((t >> 4) & 1) + (t & 3); }

// One step of a packed-fp16 maximum across lanes: each lane takes the
// maximum of its value and the value DPP control CTRL brings from another
// lane of its row of 16 (rows outside ROW_MASK keep their own value).
template <int CTRL, int ROW_MASK>
__device__ inline half2v dpp_step(half2v v) {
    const int b = __builtin_bit_cast(int, v);
    const int m = ROW_MASK == 0xF ? __builtin_amdgcn_mov_dpp(b, CTRL, 0xF, 0xF, false)
                                  : __builtin_amdgcn_update_dpp(b, b, CTRL, ROW_MASK, 0xF, false);
    return __builtin_elementwise_maximum(v, __builtin_bit_cast(half2v, m));
}

// ------------------------------------------------------------------ append
// One wave per unit of (KV head, 4 consecutive input tokens). Row g of the
// wave (lanes 16 g .. 16 g + 15) takes token g of the unit; lane i of the
// row holds key dimensions 8 i .. 8 i + 7 and value dimensions 4 i .. 4 i + 3
// and 64 + 4 i .. 64 + 4 i + 3 (4-bit: the two nibbles of V bytes
// 4 i .. 4 i + 3, so every byte of the cache has one writer). A vector's
// range is reduced inside its row, so each instruction of the quantization
// serves the four tokens at once. Tokens with a negative slot, or a slot
// past the cache, are skipped. Tokens t .. t + 3 of a block (t % 4 == 0)
// sit in 4 consecutive bytes of every V row, so when the unit's 4 slots are
// such a run the lanes exchange their V bytes (ds_bpermute) and lane L
// stores the run's 32-bit word of V row L (and, 8-bit, of row 64 + L): one
// store instruction covers 64 consecutive rows. Otherwise each lane stores
// its own bytes.

constexpr int kAppendQuad = 4;  // input tokens per unit

// The inputs of one unit, fetched one unit ahead of their use.
struct AppendIn {
    int slot;      // slot of this row's token (-1: none)
    int h, n;      // KV head, tokens present (1..4)
    u32x4 kx, vx;  // this lane's 8 fp16 key and value elements
};

template <int BITS>
__device__ inline void kv_append_fetch(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                       const int32_t *__restrict__ slots, int ntok, int Hkv, int h, int qi, int lane,
                                       AppendIn &in) {
    const int i0 = qi * kAppendQuad;
    const int g = lane >> 4, li = lane & 15;
    in.h = h;
    in.n = ntok - i0 < kAppendQuad ? ntok - i0 : kAppendQuad;
    const int i = i0 + g < ntok ? i0 + g : ntok - 1;  // rows past a short last unit re-read its last token
    const size_t row = ((size_t)i * Hkv + h) * kHD;
    const int s = slots[i];
    in.slot = i0 + g < ntok ? s : -1;
    in.kx = *reinterpret_cast<const u32x4 *>(k + row + 8 * li);
    const uint2 lo = *reinterpret_cast<const uint2 *>(v + row + 4 * li);
    const uint2 hi = *reinterpret_cast<const uint2 *>(v + row + kHD / 2 + 4 * li);
    in.vx = u32x4{lo.x, lo.y, hi.x, hi.y};
}

// (max, -min) of an fp16 pair as an fp16 pair
__device__ inline half2v pair_range(uint32_t p) {
    const half2v h = as_h2(p);
    return __builtin_elementwise_maximum(half2v{h.x, -h.x}, half2v{h.y, -h.y});
}

// Codes c[0..7] of this lane's 8 elements of one vector, and the vector's
// scale and zero (the weight quantizer's reading with L = 2^BITS - 1). The
// vector's 128 elements are the 16 lanes of this lane's row.
template <int BITS>
__device__ inline void kv_quantize_row(const u32x4 &x, uint32_t (&c)[8], uint32_t &par) {
    constexpr int L = (1 << BITS) - 1;
    half2v r = __builtin_elementwise_maximum(__builtin_elementwise_maximum(pair_range(x[0]), pair_range(x[1])),
                                             __builtin_elementwise_maximum(pair_range(x[2]), pair_range(x[3])));
    r = dpp_step<0xB1, 0xF>(r);   // quad_perm 1 0 3 2
    r = dpp_step<0x4E, 0xF>(r);   // quad_perm 2 3 0 1
    r = dpp_step<0x141, 0xF>(r);  // row_half_mirror
    r = dpp_step<0x140, 0xF>(r);  // row_mirror: every lane holds its row's (max, -min)
    const float xmax = (float)r.x, xmin = -(float)r.y;
    const float s32 = __builtin_fmaxf(div_steps(xmax - xmin, (float)L, 1.0f / (float)L), kScaleFloor);
    const _Float16 s16 = (_Float16)s32;
    const float sf = (float)s16;
    // within one ulp of 1/s, which the code decision allows (its corrected
    // product stays within |x/s| 2^-44 of the quotient)
    const float inv = __builtin_amdgcn_rcpf(sf);
    // the zero code: rint(-xmin / s) clamped to [0, L], decided like the
    // codes (-xmin and s are fp16 values)
    const float zf = __builtin_amdgcn_fmed3f(round_quotient_fp16(-xmin, sf, inv), kRoundMagic, kRoundMagic + (float)L);
    const int z = (int)(__builtin_bit_cast(uint32_t, zf) - kRoundMagicBits);
    const float lo = kRoundMagic - (float)z, hi = lo + (float)L;
    const uint32_t off = (uint32_t)z - kRoundMagicBits;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t w = x[e / 2];
        const float xe = (float)__builtin_bit_cast(_Float16, (uint16_t)(e & 1 ? w >> 16 : w & 0xFFFF));
        const float y = __builtin_amdgcn_fmed3f(round_quotient_fp16(xe, sf, inv), lo, hi);
        c[e] = __builtin_bit_cast(uint32_t, y) + off;
    }
    par = (uint32_t)__builtin_bit_cast(uint16_t, s16) | ((uint32_t)z << 16);
}

template <int BITS>
__device__ inline void kv_append_store(const AppendIn &in, int Hkv, int64_t num_blocks, int lane,
                                       uint8_t *__restrict__ cache) {
    typedef KvGeom<BITS> Geo;
    const int g = lane >> 4, li = lane & 15;
    // the unit's four slots (uniform): a 4-aligned run inside one block?
    const int s0 = __builtin_amdgcn_readlane(in.slot, 0);
    bool run = in.n == kAppendQuad && s0 >= 0 && (s0 & 3) == 0 && s0 / kBS < num_blocks;
#pragma unroll
    for (int j = 1; j < kAppendQuad; ++j) run = run && __builtin_amdgcn_readlane(in.slot, 16 * j) == s0 + j;
    const int slot = in.slot;
    const bool valid = slot >= 0 && slot / kBS < num_blocks;
    const int blk = valid ? slot / kBS : 0, t = slot & (kBS - 1);
    uint8_t *region = cache + ((size_t)blk * Hkv + in.h) * Geo::kRegion;

    uint32_t c[8], kpar, vpar;
    kv_quantize_row<BITS>(in.kx, c, kpar);
    if (valid) {
        uint8_t *krow = region + t * Geo::kRowBytes;
        if constexpr (BITS == 8)
            *reinterpret_cast<uint2 *>(krow + 8 * li) =
                make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
        else
            *reinterpret_cast<uint32_t *>(krow + 4 * li) =
                c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12) | (c[4] << 16) | (c[5] << 20) | (c[6] << 24) | (c[7] << 28);
    }
    kv_quantize_row<BITS>(in.vx, c, vpar);
    if (valid && li == 0) {
        *reinterpret_cast<uint32_t *>(region + Geo::kKPar + 4 * t) = kpar;
        *reinterpret_cast<uint32_t *>(region + Geo::kVPar + 4 * t) = vpar;
    }
    // V code bytes of this lane: byte e of vb0 is dimension 4 li + e (4-bit:
    // with dimension 64 + 4 li + e in its high nibble), byte e of vb1
    // (8-bit) dimension 64 + 4 li + e
    uint32_t vb0, vb1 = 0;
    if constexpr (BITS == 8) {
        vb0 = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        vb1 = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    } else {
        vb0 = (c[0] | (c[4] << 4)) | ((c[1] | (c[5] << 4)) << 8) | ((c[2] | (c[6] << 4)) << 16) |
              ((c[3] | (c[7] << 4)) << 24);
    }
    if (run) {
        // row r = lane (+ 64): byte j of its word is token j's byte of that
        // row, byte r % 4 of lane (j, r / 4 % 16)'s vb
        uint8_t *vrows = cache + ((size_t)(s0 / kBS) * Hkv + in.h) * Geo::kRegion + Geo::kCodeBytes;
        const int p = v_position(s0 & (kBS - 1));  // positions p .. p + 3 hold the run's tokens
        const uint32_t b = lane & 3;
        const uint32_t sel = b | ((4 + b) << 8);
#pragma unroll
        for (int half = 0; half < (BITS == 8 ? 2 : 1); ++half) {
            const uint32_t vb = half ? vb1 : vb0;
            uint32_t src[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) src[j] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (16 * j + (lane >> 2)), (int)vb);
            const uint32_t t01 = __builtin_amdgcn_perm(src[1], src[0], sel);
            const uint32_t t23 = __builtin_amdgcn_perm(src[3], src[2], sel);
            *reinterpret_cast<uint32_t *>(vrows + (64 * half + lane) * kBS + p) = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
        }
    } else if (valid) {
        uint8_t *vrows = region + Geo::kCodeBytes;
        const int p = v_position(t);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vrows[(4 * li + e) * kBS + p] = (uint8_t)(vb0 >> (8 * e));
            if constexpr (BITS == 8) vrows[(64 + 4 * li + e) * kBS + p] = (uint8_t)(vb1 >> (8 * e));
        }
    }
}

constexpr int kAppendWaves = 16;   // waves per workgroup: one unit each, 64 tokens per task
constexpr int kAppendWgPerCu = 2;   // resident workgroups per CU (8 waves per SIMD)

// A resident grid over tasks of (KV head, 64 consecutive input tokens),
// one unit of 4 tokens per wave; each wave fetches its unit of the
// workgroup's next task before it quantizes and stores the current one, and
// the workgroup meets at a barrier after every task. When the slots run in
// order a task is one cache block: the 16 partial writes that complete each
// V line all come from one workgroup within one task, and an XCD has only
// its resident workgroups' blocks open at a time, so the lines fill in its
// L2 before they are written back (units dealt to waves across the whole
// grid had drifted apart over the rounds and sent partly written lines to
// memory: 1.9x the cache bytes written for 8-bit codes).
template <int BITS>
__global__ void __launch_bounds__(64 * kAppendWaves)
kv_append_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, const int32_t *__restrict__ slots,
                 int ntok, int Hkv, int64_t num_blocks, uint8_t *__restrict__ cache) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int quads = (ntok + kAppendQuad - 1) / kAppendQuad;
    const int chunks = (quads + kAppendWaves - 1) / kAppendWaves;  // tasks per head
    const int64_t tasks = (int64_t)chunks * Hkv;
    const uint32_t grid = gridDim.x;
    int64_t T = blockIdx.x;
    if (T >= tasks) return;
    // task T = h * chunks + c, advanced by the grid without a division per task
    int h = (int)(T / chunks), c = (int)(T % chunks);
    const int64_t sh = grid / chunks;
    const int sc = (int)(grid % chunks);
    // every task fetches (a unit past the last token re-reads the last one,
    // in bounds, marked empty), so the loads in flight are the same on every
    // path
    auto fetch = [&](int hh, int cc, bool live, AppendIn &in) {
        const int qi = kAppendWaves * cc + wave;
        const bool ok = live && qi < quads;
        kv_append_fetch<BITS>(k, v, slots, ntok, Hkv, ok ? hh : Hkv - 1, ok ? qi : quads - 1, lane, in);
        if (!ok) {
            in.slot = -1;
            in.n = 0;
        }
    };
    AppendIn cur, nxt;
    fetch(h, c, true, cur);
    while (true) {
        const int64_t nT = T + grid;
        int nc = c + sc;
        const int carry = nc >= chunks;
        nc -= carry ? chunks : 0;
        const int64_t hn = h + sh + carry;
        const int nh = hn < Hkv ? (int)hn : Hkv - 1;
        const bool nlive = nT < tasks;  // uniform over the workgroup
        fetch(nh, nc, nlive, nxt);
        kv_append_store<BITS>(cur, Hkv, num_blocks, lane, cache);
        if (!nlive) break;
        __syncthreads();
        cur = nxt;
        h = nh;
        c = nc;
        T = nT;
    }
}

// ------------------------------------------------------------------ attention
// Registers of one half block (32 tokens) for one wave: the pipeline stage.
template <int BITS>
struct KvStage {
    u32x4 kc[2][BITS == 8 ? 2 : 1];  // K codes of the two 16-token tiles, 32 dims per lane
    u32x4 kp[2];                     // K parameters of tokens 16 tt + 4 kq + 0..3
    u32x4 vp[2];                     // V parameters of the same tokens
    // V codes, 8 positions per row: 8-bit, d tiles 0..7; 4-bit, row tiles
    // 0..3 (low nibbles: d tile r, high nibbles: d tile r + 4)
    uint32_t vc[BITS == 8 ? 8 : 4][2];
};

// fp16 pair (1024 + byte 2i, 1024 + byte 2i + 1) of the 8-bit codes in w:
// v_perm_b32 takes bytes 0-3 from its second source and 4-7 from its first
__device__ inline uint32_t bytes_to_h2(uint32_t w, int i) {
    return __builtin_amdgcn_perm(0x64646464u, w, i ? 0x04030402u : 0x04010400u);
}

// Waves per SIMD the attention kernel is built for (register budget: with
// one half block in flight, 8-bit stages fit two waves and 4-bit stages
// three without the compiler reusing registers of loads still in flight).
// Half blocks in flight per wave, and waves per SIMD the kernel is built
// for (measured at 50 x 4000 tokens: 8-bit, one half block at
// two waves 88.7 us per call, two at one wave 92.6, three at one wave 105.5;
// 4-bit, two at two waves 54.9, one at three waves 57).
template <int BITS>
constexpr int kv_depth() { return BITS == 8 ? 1 : 2; }
template <int BITS>
constexpr int kv_waves_per_simd() { return 2; }

template <int BITS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kv_waves_per_simd<BITS>(), kv_waves_per_simd<BITS>())))
kv_attention_kernel(const uint16_t *__restrict__ q, const uint8_t *__restrict__ cache,
                    const int32_t *__restrict__ block_table, int max_blocks, const int32_t *__restrict__ lengths,
                    int B, int Hq, int Hkv, int64_t num_blocks, float score_scale, int chunk_blocks, int nchunks,
                    float *__restrict__ part_o, float2 *__restrict__ part_ml) {
    typedef KvGeom<BITS> Geo;
    typedef KvStage<BITS> Stage;
    const int lane = threadIdx.x & 63;
    const int unit = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int units = B * Hkv * nchunks;
    if (unit >= units) return;  // uniform per wave; no block-wide barrier below
    const int chunk = unit % nchunks;
    const int kh = (unit / nchunks) % Hkv;
    const int b = unit / (nchunks * Hkv);
    const int g = Hq / Hkv;
    const int c = lane & 15, kq = lane >> 4;
    int len = lengths[b];
    if (len > max_blocks * kBS) len = max_blocks * kBS;
    const int nblk = len > 0 ? (len + kBS - 1) / kBS : 0;
    const int bb0 = chunk * chunk_blocks;
    const int bb1 = bb0 + chunk_blocks < nblk ? bb0 + chunk_blocks : nblk;
    // half blocks [h0, h1) of this chunk that hold tokens
    const int h0 = 2 * bb0;
    const int h1 = bb1 > bb0 ? (2 * bb1 < (len + 31) / 32 ? 2 * bb1 : (len + 31) / 32) : h0;

    // query of head kh * g + c in the key's dimension order (B operand of
    // S^T = K . Q^T): step s, slot j of lane group kq holds dimension
    // 32 kq + 8 s + j (8-bit keys) or 32 kq + 8 s + sigma(j) with
    // sigma = 0 4 1 5 2 6 3 7 (4-bit keys, whose nibble extraction yields
    // that order)
    half8 qf[4];
    {
        const bool ok = c < g;
        const uint16_t *qh = q + ((size_t)b * Hq + kh * g + (ok ? c : 0)) * kHD + 32 * kq;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const half8 raw = ok ? *reinterpret_cast<const half8 *>(qh + 8 * s) : half8{};
            if constexpr (BITS == 8) {
                qf[s] = raw;
            } else {
                half8 p;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    p[2 * j] = raw[j];
                    p[2 * j + 1] = raw[j + 4];
                }
                qf[s] = p;
            }
        }
    }
    // The key codes enter the matrix instruction as bias + c: 1024 + c
    // (8-bit codes and the low nibbles of 4-bit ones, exponent-OR) or 64 + c
    // (high nibbles, which need no shift). A score then loses
    // sum_d bias_d q_d + z * sum(q); both sums are per head (the four kq lane
    // groups hold 32 dimensions each). In the 4-bit slot order the slots
    // 0, 1, 4, 5 of a step hold low nibbles and 2, 3, 6, 7 high ones.
    float qsum = 0.f, qbias = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float qv = (float)qf[s][j];
            qsum += qv;
            qbias += qv * (BITS == 8 || ((j >> 1) & 1) == 0 ? 1024.f : 64.f);
        }
    qsum += __shfl_xor(qsum, 16, 64);
    qsum += __shfl_xor(qsum, 32, 64);
    qbias += __shfl_xor(qbias, 16, 64);
    qbias += __shfl_xor(qbias, 32, 64);

    // Half block hb = 2 * block + half. Stages past the chunk, or in a block
    // the table does not name, load through an empty descriptor: no memory
    // traffic and the same instructions on every path.
    auto load = [&](int hb, Stage &S) {
        const int bi = hb >> 1, hf = hb & 1;
        const int bic = bi < max_blocks ? bi : max_blocks - 1;  // stays inside the table
        int id = hb < h1 ? block_table[(size_t)b * max_blocks + bic] : -1;
        if (id >= num_blocks) id = -1;
        const uint8_t *base = cache + (id < 0 ? 0 : ((int64_t)id * Hkv + kh) * Geo::kRegion);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(base, id < 0 ? 0u : (uint32_t)Geo::kRegion);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tt = 2 * hf + u;
            const int tok = 16 * tt + c;
#pragma unroll
            for (int w = 0; w < (BITS == 8 ? 2 : 1); ++w)
                S.kc[u][w] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                           r, (uint32_t)(tok * Geo::kRowBytes + (32 * kq) * BITS / 8 + 16 * w), 0, 0));
            const int t4 = 16 * tt + 4 * kq;
            S.kp[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(Geo::kKPar + 4 * t4), 0, 0));
            S.vp[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(Geo::kVPar + 4 * t4), 0, 0));
        }
#pragma unroll
        for (int dt = 0; dt < (BITS == 8 ? 8 : 4); ++dt) {
            const uint32_t off = (uint32_t)(Geo::kCodeBytes + (16 * dt + c) * Geo::kVRowBytes + 16 * kq + 8 * hf);
            const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
            S.vc[dt][0] = (uint32_t)w2[0];
            S.vc[dt][1] = (uint32_t)w2[1];
        }
    };

    floatx4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff(), l_run = 0.f;

    auto compute = [&](int hb, const Stage &S) {
        const int tok0 = 32 * hb;  // sequence position of the stage's first token
        const int bi = hb >> 1;
        int id = block_table[(size_t)b * max_blocks + bi];
        if (id < 0 || id >= num_blocks) return;  // uniform: an absent block holds no tokens
        const bool full = tok0 + 32 <= len;
        // ---- scores of the 32 tokens (two 16-token tiles): the matrix
        // instruction multiplies the codes as 1024 + c (exponent-OR, no
        // per-code subtraction); the zero enters each score once as
        // -(1024 + z) * sum(q), exact products summed in fp32
        float x[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                half8 a;
                if constexpr (BITS == 8) {
                    const u32x4 &w = S.kc[u][s >> 1];
                    const uint32_t w0 = w[2 * (s & 1)], w1 = w[2 * (s & 1) + 1];
                    a = pack_h8(as_h2(bytes_to_h2(w0, 0)), as_h2(bytes_to_h2(w0, 1)), as_h2(bytes_to_h2(w1, 0)),
                                as_h2(bytes_to_h2(w1, 1)));
                } else {
                    const uint32_t w = S.kc[u][0][s], w8 = w >> 8;
                    a = pack_h8(as_h2(and_or(w, kLoMask, kMagic)), as_h2(and_or(w, kHiMask, kMagic64)),
                                as_h2(and_or(w8, kLoMask, kMagic)), as_h2(and_or(w8, kHiMask, kMagic64)));
                }
                acc = mfma16x16x32(a, qf[s], acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t par = S.kp[u][e];
                const float ks = (float)__builtin_bit_cast(_Float16, (uint16_t)(par & 0xFFFFu));
                const float zk = (float)(par >> 16 & 0xFFu);
                const float sc = __builtin_fmaf(-zk, qsum, acc[e] - qbias) * (ks * score_scale);
                x[u][e] = full || tok0 + 16 * u + 4 * kq + e < len ? sc : -__builtin_inff();
            }
        }
        // ---- online softmax for head c (the four kq lane groups hold
        // different tokens of the same head)
        float mt = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(x[0][0], x[0][1]), __builtin_fmaxf(x[0][2], x[0][3])),
                                   __builtin_fmaxf(__builtin_fmaxf(x[1][0], x[1][1]), __builtin_fmaxf(x[1][2], x[1][3])));
        mt = __builtin_fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32, 64));
        // The running maximum moves only when a head's maximum rises by more
        // than 8 (log2 units): the probabilities stay below 2^8 (exact
        // enough in fp16 after the V scale) and most stages skip the rescale
        // of O. The result does not depend on which maximum is used.
        const float m_new = mt > m_run + 8.f ? mt : m_run;
        if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {  // some head's max moved: rescale
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int e = 0; e < 4; ++e) o[dt][e] *= alpha;
            m_run = m_new;
        }
        // ---- B operand P^T for O^T = V^T . P^T: slot j holds token
        // 4 kq + j (j < 4) or 16 + 4 kq + j - 4 of the stage, times its V
        // scale; masked tokens contribute exactly zero
        half8 pb;
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = __builtin_amdgcn_exp2f(x[u][e] - m_run);
                psum += p;
                const float vs = (float)__builtin_bit_cast(_Float16, (uint16_t)(S.vp[u][e] & 0xFFFFu));
                const _Float16 pv = (_Float16)(x[u][e] == -__builtin_inff() ? 0.f : p * vs);
                const int j = 4 * u + e;
                // 4-bit V: each 16-bit half of a code word yields the tokens
                // e and e + 2 of a 4-token group, so the slots of tokens
                // e = 0 1 2 3 are 0 2 1 3
                const int slot = BITS == 8 ? j : 4 * u + 2 * (e & 1) + (e >> 1);
                pb[slot] = pv;
            }
        l_run += psum;
        uint32_t vzn[4];  // -(1024 + z) pairs of the slot pairs
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
            // slot pair (2 pr, 2 pr + 1): 8-bit tokens j = 2 pr, 2 pr + 1;
            // 4-bit tokens j = 4 (pr / 2) + pr % 2 and that + 2
            const int ja = BITS == 8 ? 2 * pr : 4 * (pr >> 1) + (pr & 1), jb = BITS == 8 ? ja + 1 : ja + 2;
            const uint32_t za = S.vp[ja / 4][ja % 4] >> 16 & 0xFFu;
            const uint32_t zb = S.vp[jb / 4][jb % 4] >> 16 & 0xFFu;
            vzn[pr] = (0xE400u | za) | ((0xE400u | zb) << 16);
        }
        // ---- O^T += V^T . P^T over the 8 tiles of 16 dimensions with the
        // exact integers c - z (the outputs are averages much smaller than
        // the codes, so the zero is not deferred as it is for the scores)
        if constexpr (BITS == 8) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const uint32_t w0 = S.vc[dt][0], w1 = S.vc[dt][1];
                const half8 a = pack_h8(as_h2(bytes_to_h2(w0, 0)) + as_h2(vzn[0]), as_h2(bytes_to_h2(w0, 1)) + as_h2(vzn[1]),
                                        as_h2(bytes_to_h2(w1, 0)) + as_h2(vzn[2]), as_h2(bytes_to_h2(w1, 1)) + as_h2(vzn[3]));
                o[dt] = mfma16x16x32(a, pb, o[dt]);
            }
        } else {
            // low nibbles enter as 1024 + c (d tile r), high nibbles as
            // 64 + c with no shift (d tile r + 4)
            uint32_t vzh[4];
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) vzh[pr] = neg_bias64_from_1024(vzn[pr]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const uint32_t w0 = S.vc[rt][0], w1 = S.vc[rt][1], w0s = w0 >> 8, w1s = w1 >> 8;
                const half8 lo = pack_h8(as_h2(and_or(w0, kLoMask, kMagic)) + as_h2(vzn[0]),
                                         as_h2(and_or(w0s, kLoMask, kMagic)) + as_h2(vzn[1]),
                                         as_h2(and_or(w1, kLoMask, kMagic)) + as_h2(vzn[2]),
                                         as_h2(and_or(w1s, kLoMask, kMagic)) + as_h2(vzn[3]));
                o[rt] = mfma16x16x32(lo, pb, o[rt]);
                const half8 hi = pack_h8(as_h2(and_or(w0, kHiMask, kMagic64)) + as_h2(vzh[0]),
                                         as_h2(and_or(w0s, kHiMask, kMagic64)) + as_h2(vzh[1]),
                                         as_h2(and_or(w1, kHiMask, kMagic64)) + as_h2(vzh[2]),
                                         as_h2(and_or(w1s, kHiMask, kMagic64)) + as_h2(vzh[3]));
                o[rt + 4] = mfma16x16x32(hi, pb, o[rt + 4]);
            }
        }
    };

    // The pages' double-buffered KV loading, D half blocks deep: while D
    // half blocks are multiplied the next D are in flight.
    if (h0 < h1) {
        constexpr int D = kv_depth<BITS>();
        Stage st[2][D];
#pragma unroll
        for (int i = 0; i < D; ++i) load(h0 + i, st[0][i]);
        for (int hb = h0; hb < h1; hb += 2 * D) {
#pragma unroll
            for (int i = 0; i < D; ++i) load(hb + D + i, st[1][i]);
            bool more = true;
#pragma unroll
            for (int i = 0; i < D; ++i) {
                if (hb + i >= h1) more = false;
                if (more) compute(hb + i, st[0][i]);
            }
            if (hb + D >= h1) break;
#pragma unroll
            for (int i = 0; i < D; ++i) load(hb + 2 * D + i, st[0][i]);
#pragma unroll
            for (int i = 0; i < D; ++i) {
                if (hb + D + i >= h1) more = false;
                if (more) compute(hb + D + i, st[1][i]);
            }
        }
    }

    // ---- partial results of this chunk: (max, sum) and unnormalized O^T
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (c < g) {
        if (kq == 0) part_ml[(size_t)unit * 16 + c] = float2{m_run, l_run};
        float *po = part_o + ((size_t)unit * 16 + c) * kHD;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<floatx4 *>(po + 16 * dt + 4 * kq) = o[dt];
    }
}

// O[b][h] = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i over the chunks of
// (b, h / g); one workgroup of 128 threads per (b, h), thread = dimension.
// The chunks' (max, sum) records and outputs are loaded 8 chunks at a time,
// all loads of a batch in flight together, and merged with a running
// maximum (for 8 chunks or fewer that is one pass with the global maximum).
__global__ void __launch_bounds__(128)
kv_combine_kernel(const float *__restrict__ part_o, const float2 *__restrict__ part_ml, int Hq, int Hkv,
                  int nchunks, uint16_t *__restrict__ out) {
    constexpr int CB = 8;
    const int bh = blockIdx.x, d = threadIdx.x;
    const int b = bh / Hq, h = bh % Hq, g = Hq / Hkv;
    const int kh = h / g, c = h % g;
    const size_t u0 = ((size_t)b * Hkv + kh) * nchunks;
    float M = -__builtin_inff(), num = 0.f, den = 0.f;
    for (int i0 = 0; i0 < nchunks; i0 += CB) {
        float2 ml[CB];
        float o[CB];
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            const bool in = i0 + j < nchunks;
            const size_t r = (u0 + (in ? i0 + j : 0)) * 16 + c;
            ml[j] = in ? part_ml[r] : float2{-__builtin_inff(), 0.f};
            o[j] = in ? part_o[r * kHD + d] : 0.f;
        }
        float mb = M;
#pragma unroll
        for (int j = 0; j < CB; ++j) mb = __builtin_fmaxf(mb, ml[j].x);
        if (mb == -__builtin_inff()) continue;  // no tokens so far
        const float sc = __builtin_amdgcn_exp2f(M - mb);  // 0 while M is -inf
        num *= sc;
        den *= sc;
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            if (ml[j].x == -__builtin_inff()) continue;
            const float w = __builtin_amdgcn_exp2f(ml[j].x - mb);
            num += w * o[j];
            den += w * ml[j].y;
        }
        M = mb;
    }
    out[(size_t)bh * kHD + d] = f32_to_f16_bits(den > 0.f ? num / den : 0.f);
}

}  // namespace

size_t kv_region_bytes(int bits) { return bits == 8 ? KvGeom<8>::kRegion : KvGeom<4>::kRegion; }

hipError_t launch_kv_append(const uint16_t *k, const uint16_t *v, const int32_t *slots, int ntok, int Hkv, int bits,
                            int64_t num_blocks, uint8_t *cache, int num_cus, hipStream_t stream) {
    if (ntok == 0) return hipSuccess;
    const int64_t quads = (ntok + kAppendQuad - 1) / kAppendQuad;
    const int64_t tasks = (quads + kAppendWaves - 1) / kAppendWaves * Hkv;
    const int64_t resident = (int64_t)num_cus * kAppendWgPerCu;
    const dim3 grid((unsigned)(tasks < resident ? tasks : resident));
    const dim3 block(64 * kAppendWaves);
    if (bits == 8)
        hipLaunchKernelGGL(kv_append_kernel<8>, grid, block, 0, stream, k, v, slots, ntok, Hkv, num_blocks, cache);
    else
        hipLaunchKernelGGL(kv_append_kernel<4>, grid, block, 0, stream, k, v, slots, ntok, Hkv, num_blocks, cache);
    return hipGetLastError();
}

KvPlan kv_plan(int B, int Hkv, int max_blocks, int num_cus, int bits) {
    KvPlan p;
    // split each (sequence, KV head) into as many chunks of whole blocks as
    // keep the work in one round of resident waves (4 SIMDs per CU)
    const long pairs = (long)B * Hkv;
    const long resident = (long)num_cus * 4 * (bits == 8 ? kv_waves_per_simd<8>() : kv_waves_per_simd<4>());
    int nchunks = (int)(resident / pairs);
    if (nchunks > max_blocks) nchunks = max_blocks;
    if (nchunks < 1) nchunks = 1;
    p.chunk_blocks = (max_blocks + nchunks - 1) / nchunks;
    p.nchunks = (max_blocks + p.chunk_blocks - 1) / p.chunk_blocks;
    return p;
}

size_t kv_workspace_bytes(int B, int Hkv, int max_blocks, int num_cus) {
    // sized for the larger of the two code widths' plans
    const KvPlan p8 = kv_plan(B, Hkv, max_blocks, num_cus, 8), p4 = kv_plan(B, Hkv, max_blocks, num_cus, 4);
    const size_t units = (size_t)B * Hkv * (p8.nchunks > p4.nchunks ? p8.nchunks : p4.nchunks);
    return units * 16 * kHD * sizeof(float) + units * 16 * sizeof(float2);
}

hipError_t launch_kv_attention(const uint16_t *q, const uint8_t *cache, const int32_t *block_table, int max_blocks,
                               const int32_t *lengths, int B, int Hq, int Hkv, int bits, int64_t num_blocks,
                               float sm_scale, uint16_t *out, void *workspace, int num_cus, hipStream_t stream) {
    const KvPlan p = kv_plan(B, Hkv, max_blocks, num_cus, bits);
    const size_t units = (size_t)B * Hkv * p.nchunks;
    float *part_o = static_cast<float *>(workspace);
    float2 *part_ml = reinterpret_cast<float2 *>(part_o + units * 16 * kHD);
    const unsigned wgs = (unsigned)((units + 3) / 4);
    const float score_scale = sm_scale * kLog2e;
    if (bits == 8)
        hipLaunchKernelGGL(kv_attention_kernel<8>, dim3(wgs), dim3(256), 0, stream, q, cache, block_table, max_blocks,
                           lengths, B, Hq, Hkv, num_blocks, score_scale, p.chunk_blocks, p.nchunks, part_o, part_ml);
    else
        hipLaunchKernelGGL(kv_attention_kernel<4>, dim3(wgs), dim3(256), 0, stream, q, cache, block_table, max_blocks,
                           lengths, B, Hq, Hkv, num_blocks, score_scale, p.chunk_blocks, p.nchunks, part_o, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kv_combine_kernel, dim3((unsigned)(B * Hq)), dim3(kHD), 0, stream, part_o, part_ml, Hq, Hkv,
                       p.nchunks, out);
    return hipGetLastError();
}

}  // namespace w4a16
