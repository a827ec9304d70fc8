// Attainable HBM read rate on gfx950: a plain streaming read of a buffer,
// every byte once, with the same load form the hot kernels use for their
// streams (16-byte non-temporal loads, several in flight per lane).
//
// The llama.cpp MTP article (section on the theoretical maximum of
// generation speed) bounds decoding by memory bandwidth: the rate is the
// memory speed over the bytes of the active weights, and it compares that
// bound with what is measured.  This kernel gives the measured side of that
// comparison on this GPU, so each hot kernel's rate can be stated both as a
// share of the published peak and as a share of what a plain read attains.
//
// The loads feed an XOR of 32-bit words, written per workgroup, so none is
// dead and the caller can check that every word was read.
#include "spec_internal.h"

namespace spec {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;   // 16-byte loads per lane per round

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

// Workgroup g reads rounds g, g + G, ... of kThreads * kInFlight 16-byte
// words (32 KB contiguous); lane t takes words t, t + 256, ... of a round,
// so each load instruction of a wave covers 1 KB of consecutive memory.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4v *__restrict__ src,
                                                               size_t n16,
                                                               uint32_t *__restrict__ sink) {
    constexpr size_t kRound = (size_t)kThreads * kInFlight;
    const size_t rounds = (n16 + kRound - 1) / kRound;
    unsigned acc = 0;
    for (size_t r = blockIdx.x; r < rounds; r += gridDim.x) {
        const size_t base = r * kRound + threadIdx.x;
        u32x4v v[kInFlight];
        if ((r + 1) * kRound <= n16) {
#pragma unroll
            for (int q = 0; q < kInFlight; ++q)
                v[q] = __builtin_nontemporal_load(&src[base + q * kThreads]);
        } else {   // the last, partial round
#pragma unroll
            for (int q = 0; q < kInFlight; ++q)
                v[q] = base + q * kThreads < n16 ? __builtin_nontemporal_load(&src[base + q * kThreads])
                                                 : u32x4v{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < kInFlight; ++q)
            acc ^= v[q].x ^ v[q].y ^ v[q].z ^ v[q].w;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        acc ^= (unsigned)__shfl_xor((int)acc, o);
    __shared__ unsigned part[kThreads / 64];
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0)
        sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

} // namespace

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, int groups,
                              hipStream_t stream) {
    stream_read_kernel<<<groups, kThreads, 0, stream>>>(
        static_cast<const u32x4v *>(src), bytes / 16, sink);
    return hipGetLastError();
}

} // namespace spec
