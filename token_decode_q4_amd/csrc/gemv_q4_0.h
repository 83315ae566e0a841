// gemv_q4_0.h -- q4_0 GEMV for gfx950 (batch 1) and its fused epilogues.
//
// y = W x with W in q4_0 (inferencelayer cuda_llm.rs page, Q4Dev and
// CudaQwen3::gemv: 32-weight blocks, one f16 scale, 16 bytes of nibbles;
// weight = (nibble - 8) * scale).
//
// Work mapping.  A workgroup of NWAVES wave64s owns a tile of rows.  Inside a
// wave, groups of LPR lanes share a row slot and split that row's blocks
// (lane i of the group takes blocks i, i+LPR, ...); each lane keeps RPS rows
// of its slot in flight, so one staged x chunk is reused RPS times.  A lane
// loads a whole block's 16 nibble bytes with one 128-bit load: consecutive
// lanes read consecutive blocks of a row, so a wave reads LPR*16 contiguous
// bytes per row.  x is staged once per workgroup into LDS (block b at float
// offset b*36: the 4-float pad keeps the per-lane 128-bit reads of 64 lanes
// on distinct banks) together with each block's sum of x.
//
// In-register dequant: for one 32-bit word of nibbles, (w & 0x0f0f0f0f) and
// ((w >> 4) & 0x0f0f0f0f) hold four codes each in byte lanes, which convert
// to f32 one instruction each; the offset -8 is applied once per block as
//   sum_j (c_j - 8) x_j = sum_j c_j x_j - 8 * sum_j x_j,
// with sum_j x_j precomputed per block.  Partial row sums are reduced across
// the LPR lanes with butterfly shuffles in a fixed order (deterministic).
#pragma once

#include "qd_common.h"

namespace qd {

constexpr int XPAD = 36;  // floats per staged x block (32 + pad)

// LDS floats needed to stage x of nb blocks
__host__ __device__ constexpr int gemv_lds_floats(int nb) { return nb * XPAD + nb; }

// Stage x[32*nb] (global f32) into LDS: xl[b*XPAD + j] = x[32b + j], xs[b] = sum_j x[32b+j].
template <int NT>
QD_DEV void stage_x(const float* __restrict__ x, int nb, float* xl, float* xs)
{
    // 8 float4 per block; 8 consecutive lanes hold one block, so the block sum
    // is a butterfly over those 8 lanes.  NT is a multiple of 64.
    const int n4 = nb * 8;
    for (int i0 = 0; i0 < n4; i0 += NT) {
        int i = i0 + (int)threadIdx.x;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < n4) {
            v = reinterpret_cast<const float4*>(x)[i];
            *reinterpret_cast<float4*>(xl + (i >> 3) * XPAD + (i & 7) * 4) = v;
        }
        float s = (v.x + v.y) + (v.z + v.w);
        s = group_sum<8>(s);
        if (i < n4 && (i & 7) == 0)
            xs[i >> 3] = s;
    }
    __syncthreads();
}

// sum_j c_j * x_j over one block (codes c_j in [0, 15]); xv = the block's 32 x values
QD_DEV float q4_block_dot(uint4 q, const float4 (&xv)[8])
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        // word k = bytes 4k..4k+3: low nibbles are elements 4k..4k+3,
        // high nibbles are elements 16+4k..16+4k+3
        const uint32_t lo = w[k] & 0x0f0f0f0fu;
        const uint32_t hi = (w[k] >> 4) & 0x0f0f0f0fu;
        s0 = fmaf((float)(lo & 0xffu), xv[k].x, s0);
        s0 = fmaf((float)((lo >> 8) & 0xffu), xv[k].y, s0);
        s0 = fmaf((float)((lo >> 16) & 0xffu), xv[k].z, s0);
        s0 = fmaf((float)(lo >> 24), xv[k].w, s0);
        s1 = fmaf((float)(hi & 0xffu), xv[4 + k].x, s1);
        s1 = fmaf((float)((hi >> 8) & 0xffu), xv[4 + k].y, s1);
        s1 = fmaf((float)((hi >> 16) & 0xffu), xv[4 + k].z, s1);
        s1 = fmaf((float)(hi >> 24), xv[4 + k].w, s1);
    }
    return s0 + s1;
}

template <int LPR, int RPS, int NWAVES>
struct GemvGeom {
    static constexpr int SLOTS = WAVE / LPR;        // row slots per wave
    static constexpr int RPW = SLOTS * RPS;         // rows per wave
    static constexpr int ROWS = NWAVES * RPW;       // rows per workgroup tile
    static constexpr int NT = NWAVES * WAVE;
};

// Dot products of the RPS rows of this lane's slot in tile `tile`, reduced over
// the slot's LPR lanes: every lane of the slot returns the same acc[] values.
// The slot's rows are row0 .. row0+RPS-1 (row0 returned); rows >= N give 0.
template <int LPR, int RPS, int NWAVES>
QD_DEV int gemv_tile(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q, int N,
                     int nb, const float* xl, const float* xs, int tile, float (&acc)[RPS])
{
    using G = GemvGeom<LPR, RPS, NWAVES>;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int slot = lane / LPR, lr = lane % LPR;
    const int row0 = tile * G::ROWS + wave * G::RPW + slot * RPS;
#pragma unroll
    for (int r = 0; r < RPS; ++r)
        acc[r] = 0.f;
    for (int b = lr; b < nb; b += LPR) {
        uint4 q[RPS];
        float d[RPS];
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            const int row = row0 + r;
            if (row < N) {
                const size_t blk = (size_t)row * nb + b;
                q[r] = *reinterpret_cast<const uint4*>(Q + blk * 16);
                d[r] = f16_to_f32(D[blk]);
            } else {
                q[r] = make_uint4(0, 0, 0, 0);
                d[r] = 0.f;
            }
        }
        float4 xv[8];
        const float4* xp = reinterpret_cast<const float4*>(xl + b * XPAD);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            xv[k] = xp[k];
        const float m8 = -8.f * xs[b];
#pragma unroll
        for (int r = 0; r < RPS; ++r)
            acc[r] = fmaf(d[r], q4_block_dot(q[r], xv) + m8, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < RPS; ++r)
        acc[r] = group_sum<LPR>(acc[r]);
    return row0;
}

// 1 / sqrt(mean(x^2) + eps) from per-workgroup partial sums of x^2 written by
// the producer of x (summed here in a fixed order).  All threads get the value.
QD_DEV float inv_rms_from_partials(const float* __restrict__ ss_part, int n_part, int n, float eps,
                                   float* smem_scalar)
{
    if (threadIdx.x < WAVE) {
        float s = 0.f;
        for (int i = threadIdx.x; i < n_part; i += WAVE)
            s += ss_part[i];
        s = group_sum<WAVE>(s);
        if (threadIdx.x == 0)
            *smem_scalar = 1.0f / sqrtf(s / (float)n + eps);
    }
    __syncthreads();
    return *smem_scalar;
}

// ----------------------------------------------------------------- plain GEMV

template <int LPR, int RPS, int NWAVES>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_plain(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
             const float* __restrict__ x, float* __restrict__ y, int N, int nb)
{
    using G = GemvGeom<LPR, RPS, NWAVES>;
    extern __shared__ float smem[];
    float* xl = smem;
    float* xs = smem + nb * XPAD;
    stage_x<G::NT>(x, nb, xl, xs);
    const int ntiles = (N + G::ROWS - 1) / G::ROWS;
    const int lr = (threadIdx.x & (WAVE - 1)) % LPR;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        float acc[RPS];
        const int row0 = gemv_tile<LPR, RPS, NWAVES>(D, Q, N, nb, xl, xs, tile, acc);
        if (lr == 0) {
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                if (row0 + r < N)
                    y[row0 + r] = acc[r];
        }
    }
}

}  // namespace qd
