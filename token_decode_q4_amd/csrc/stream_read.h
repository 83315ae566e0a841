// stream_read.h -- the plain streaming read kernel that the q4_0 GEMV is
// measured against (a measurement utility, not a step of the decode path).
//
// Every workgroup reads its 16-byte chunks with non-temporal 128-bit loads,
// U chunks per thread per round, all of a round's loads issued before any is
// used, and XORs the 32-bit words it read (so no load is dead); the
// workgroup's XOR goes to sink[blockIdx.x].  Chunk i of round r of workgroup
// w: i = (r * gridDim.x + w) * 256 * U + u * 256 + threadIdx.x.
#pragma once

#include "qd_common.h"

namespace qd {

constexpr int SR_THREADS = 256;
constexpr int SR_U = 4;
constexpr int SR_MAX_GROUPS = 2048;

inline int stream_read_groups(size_t bytes)
{
    const size_t n16 = bytes / 16;
    const size_t per = (size_t)SR_THREADS * SR_U;
    const size_t g = (n16 + per - 1) / per;
    return (int)(g < (size_t)SR_MAX_GROUPS ? (g > 0 ? g : 1) : SR_MAX_GROUPS);
}

__global__ void __launch_bounds__(SR_THREADS)
k_stream_read(const uint4* __restrict__ src, size_t n16, uint32_t* __restrict__ sink)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4* s = reinterpret_cast<const u32x4*>(src);
    const size_t round = (size_t)gridDim.x * SR_THREADS * SR_U;
    uint32_t acc = 0;
    for (size_t base = (size_t)blockIdx.x * SR_THREADS * SR_U + threadIdx.x; base < n16;
         base += round) {
        u32x4 v[SR_U];
#pragma unroll
        for (int u = 0; u < SR_U; ++u) {
            const size_t i = base + (size_t)u * SR_THREADS;
            v[u] = __builtin_nontemporal_load(s + (i < n16 ? i : n16 - 1));   // clamped, never a branch
        }
#pragma unroll
        for (int u = 0; u < SR_U; ++u)
            if (base + (size_t)u * SR_THREADS < n16)
                acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // workgroup XOR: shuffles inside a wave, then the waves through LDS
    for (int m = WAVE / 2; m >= 1; m >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, m, WAVE);
    __shared__ uint32_t part[SR_THREADS / WAVE];
    if ((threadIdx.x & (WAVE - 1)) == 0)
        part[threadIdx.x / WAVE] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < SR_THREADS / WAVE; ++w)
            r ^= part[w];
        sink[blockIdx.x] = r;
    }
}

}  // namespace qd
