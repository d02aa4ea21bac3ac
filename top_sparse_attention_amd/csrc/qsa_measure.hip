// Measurement aid (gfx950): a plain streaming read, the ceiling of each level
// of the memory hierarchy that the attention's gathers are served from.  Run
// over a footprint that stays in the L2 of every XCD, one that fits the
// Infinity Cache but not the L2s, and one larger than the Infinity Cache, it
// gives the read bandwidth of the L2s, of the Infinity Cache and of HBM for
// fully coalesced 16-byte loads.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "qsa_device.h"
#include "qsa_kernels.h"
#include "qsa_measure.h"

namespace qsa {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;   // 16-byte loads in flight per thread

// Workgroup w reads chunks_per_wg consecutive 16-byte chunks of the footprint
// starting at chunk (w * chunks_per_wg) mod footprint_chunks, wrapping at the
// end (chunks_per_wg <= footprint_chunks, so one subtraction wraps), and
// writes the XOR of everything it read to sink[w].
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const StreamParams p) {
    const u32x4_t *buf = (const u32x4_t *)p.buf;
    const int64_t n = p.footprint_chunks;
    const int64_t start = (int64_t)blockIdx.x * p.chunks_per_wg % n;
    u32x4_t acc = {0, 0, 0, 0};
    for (int64_t i = threadIdx.x; i < p.chunks_per_wg; i += kStreamThreads * kStreamUnroll) {
        u32x4_t r[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const int64_t k = i + (int64_t)kStreamThreads * u;
            int64_t idx = start + k;
            idx = idx >= n ? idx - n : idx;
            r[u] = k < p.chunks_per_wg ? ldg16<u32x4_t>(buf + idx) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= r[u];
    }
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
    __shared__ uint32_t wave_x[kStreamThreads / 64];
    if ((threadIdx.x & 63) == 0) wave_x[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
        for (int w = 0; w < kStreamThreads / 64; ++w) y ^= wave_x[w];
        p.sink[blockIdx.x] = y;
    }
}

}  // namespace

hipError_t launch_stream_read(const StreamParams &p, int64_t workgroups, hipStream_t stream) {
    if (workgroups == 0) return hipSuccess;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kStreamThreads), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace qsa
