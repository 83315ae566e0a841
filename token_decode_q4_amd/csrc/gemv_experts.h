// gemv_experts.h -- q4_0 GEMV over the experts a router picked (gfx950).
#pragma once

#include "gemv_q4_0.h"

namespace qd {

// y[j] = W[experts[j]] x for the experts picked by a router (the MoE expert
// GEMV of the inferencelayer cuda_llm.rs page): W is a stack of n_experts q4_0
// matrices of N x K, expert e at block offset e * N * nb; grid.y = j.  An index
// outside [0, n_experts) (device data, not checkable on the host) makes that
// output row NaN and reads nothing.
template <int LPR, int RPS, int NWAVES, int BG, int NBUF, int UNR, bool NTL>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_experts(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
               const int32_t* __restrict__ experts, int n_experts, const float* __restrict__ x,
               float* __restrict__ y, int N, int nb)
{
    extern __shared__ __align__(16) float smem[];   // 16-byte aligned: x is read as float4
    const int j = blockIdx.y;
    const int e = experts[j];
    float* yj = y + (size_t)j * N;
    if (e < 0 || e >= n_experts) {   // uniform over the workgroup
        for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < N; r += gridDim.x * blockDim.x)
            yj[r] = __builtin_nanf("");
        return;
    }
    const size_t off = (size_t)e * (size_t)N * (size_t)nb;
    EpiStore ep{yj, N};
    gemv_run<LPR, RPS, NWAVES, BG, NBUF, UNR, NTL>(D + off, Q + off * 16, x, N, nb, smem, smem + nb * XPAD, ep);
}

}  // namespace qd
