// qd_common.h -- device helpers shared by the decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#define QD_DEV __device__ __forceinline__

namespace qd {

constexpr int WAVE = 64;

QD_DEV float f16_to_f32(uint16_t h) { return __half2float(__ushort_as_half(h)); }
// round to nearest even
QD_DEV uint16_t f32_to_f16(float f) { return __half_as_ushort(__float2half_rn(f)); }

// butterfly sum over groups of `width` consecutive lanes (width a power of two <= 64);
// every lane of a group ends with the group's sum.  Fixed order, so deterministic.
template <int WIDTH>
QD_DEV float group_sum(float v)
{
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, WAVE);
    return v;
}

template <int WIDTH>
QD_DEV float group_max(float v)
{
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m >>= 1)
        v = fmaxf(v, __shfl_xor(v, m, WAVE));
    return v;
}

// Make this workgroup's global stores visible device-wide, then count it in
// `*counter`.  Returns true in every thread of the workgroup that completes
// the count of `target`; that workgroup resets the counter to zero before it
// returns, so the counter is ready for the next launch.  Any workgroup that
// does not complete the count returns false and must not touch the counter
// again.  Must be called by all threads of the workgroup.
QD_DEV bool arrive_last(unsigned int* counter, unsigned int target, bool* smem_flag)
{
    __threadfence();  // release this thread's stores (agent scope: other XCDs too)
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned int prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL,
                                                   __HIP_MEMORY_SCOPE_AGENT);
        *smem_flag = (prev == target - 1);
    }
    __syncthreads();
    bool last = *smem_flag;
    if (last)
        __threadfence();  // acquire: see the stores of every counted workgroup
    return last;
}

QD_DEV void reset_counter(unsigned int* counter)
{
    if (threadIdx.x == 0)
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qd
