// Streaming read of a device buffer: the achievable-bandwidth yardstick the
// measurement uses beside the datasheet peak. A decode GEMM streams every
// weight byte once per call ("LMDeploy" interview notes, answer on why W4A16
// raises throughput although FLOPs do not change), so the plainest bound on
// its time at a given byte count is how fast one kernel launch can read that
// many bytes and do nothing else.
//
// Shape: one wave reads a contiguous run of 1 KiB chunks (one 16-byte load
// per lane per chunk, non-temporal, all of the wave's chunks in flight at
// once); a workgroup is WAVES such waves. The launch is sized so that the
// whole buffer is covered by one round of resident workgroups. A load's whole
// offset is its per-lane (vector) offset, and chunks past the end take an
// offset past the descriptor: they read zeros and make no memory request. The
// data are folded into one word per lane that is stored only if it equals a
// value the caller chooses not to expect, so nothing is written in practice
// and the loads cannot be dropped.
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

template <int U>
__global__ void __launch_bounds__(256)
stream_read_kernel(const uint8_t *__restrict__ buf, uint32_t bytes, int chunks_per_wave, uint32_t never,
                   uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint32_t gw = (uint32_t)blockIdx.x * (blockDim.x >> 6) + wave;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(buf, bytes);
    const uint32_t base = gw * (uint32_t)chunks_per_wave * 1024u;
    uint32_t acc = 0;
    for (int i = 0; i < chunks_per_wave; i += U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t c = base + (uint32_t)(i + u) * 1024u;  // wave-uniform chunk start
            v[u] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, c < bytes ? c + (uint32_t)lane * 16u : kOobOffset, 0, 2));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == never) sink[lane] = acc;
}

}  // namespace

// 4 waves per workgroup, each wave's chunks all in flight: 12 per wave up to
// 12 MiB (256 workgroups), fewer chunks per wave (more workgroups) above; the
// shapes measured fastest on MI355X for 12.6, 29 and 117-235 MB buffers.
hipError_t launch_stream_read(const uint8_t *buf, size_t bytes, uint32_t never, uint32_t *sink, hipStream_t stream) {
    const int64_t chunks = (int64_t)((bytes + 1023) / 1024);
    const int U = chunks <= 256 * 4 * 12 ? 12 : 4;
    const int64_t waves = (chunks + U - 1) / U;
    const unsigned grid = (unsigned)((waves + 3) / 4);
    if (U == 12)
        hipLaunchKernelGGL(stream_read_kernel<12>, dim3(grid), dim3(256), 0, stream, buf, (uint32_t)bytes, U, never,
                           sink);
    else
        hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(256), 0, stream, buf, (uint32_t)bytes, U, never,
                           sink);
    return hipGetLastError();
}

}  // namespace w4a16
