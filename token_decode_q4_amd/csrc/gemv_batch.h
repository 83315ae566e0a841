// gemv_batch.h -- q4_0 GEMV over a batch of B <= 8 input vectors (gfx950):
// Y[b] = W X[b], every weight read from memory once for all B vectors.
//
// The batched decode of the inferencelayer cuda_llm.rs page (its q4 GEMV arm
// against the bf16 GEMM arm at M = 1 .. 16 tokens, section on the batched
// head-to-head): the weights are streamed once per step whatever the batch,
// so a step of B tokens costs about the bytes of one.
//
// Work mapping as the single-vector GEMV (gemv_q4_0.h): LPR lanes share a row
// and split its blocks, RPS rows per lane slot, persistent (tile, block group)
// items with NBUF-1 items of loads in flight.  Differences:
//   - the B input vectors are staged together into LDS (one XPAD-padded
//     layout per vector, upper half-blocks divided by 16, block sums beside);
//     every x load of the batch is issued in one round before the first
//     weight items, over a flat (vector, float4) index;
//   - each block's 32 codes of each of the RPS rows are converted to f32 once
//     (v_cvt_f32_ubyte on the masked nibble bytes) and reused for all B
//     vectors; products are exact in f32 as in the single-vector kernel.
#pragma once

#include "gemv_q4_0.h"

namespace qd {

constexpr int GB_MAXB = 8;           // vectors per launch
constexpr int GB_MAXKB = 32768;      // B * K bound (registers of the x staging)
constexpr int GB_MAXU = 16;          // float4 of x staged per thread (512 threads)

// LDS bytes of B staged vectors of nb blocks
__host__ __device__ constexpr size_t gemv_batch_lds_bytes(int nb, int B)
{
    return (size_t)B * gemv_lds_floats(nb) * sizeof(float);
}

template <int NC, int LPR, int RPS, int NWAVES, int BG, int NBUF, int UNR, bool NTL>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_batch(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
             const float* __restrict__ X, float* __restrict__ Y, int N, int nb)
{
    static_assert(NC >= 1 && NC <= GB_MAXB, "batch");
    static_assert(NBUF >= 1 && NBUF <= 6 && UNR >= NBUF, "buffers");
    using G = GemvGeom<LPR, RPS, NWAVES>;
    static_assert(G::NT * GB_MAXU * 4 >= GB_MAXKB, "x staging registers");
    extern __shared__ __align__(16) float smem[];   // 16-byte aligned: x is read as float4
    const int lds_col = gemv_lds_floats(nb);          // floats per staged vector
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int slot = lane / LPR, lr = lane % LPR;
    const int ntiles = (N + G::ROWS - 1) / G::ROWS;
    const int ngroups = (nb + LPR * BG - 1) / (LPR * BG);
    const int my_tiles = (int)blockIdx.x < ntiles ? (ntiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    const int nitems = my_tiles * ngroups;
    const int n4 = nb * 8;        // float4 per vector
    const int nf = NC * n4;       // float4 of the batch

    // ---- x loads of the whole batch (flat index f = vector * n4 + float4)
    float4 xv[GB_MAXU];
#pragma unroll
    for (int u = 0; u < GB_MAXU; ++u) {
        if (u * G::NT < nf) {   // uniform
            const int f = min((int)threadIdx.x + u * G::NT, nf - 1);
            xv[u] = reinterpret_cast<const float4*>(X)[f];   // X is [NC][K] contiguous
        }
    }

    auto load = [&](GemvBuf<RPS, BG>& bf, int i) {
        i = max(0, min(i, nitems - 1));
        const int tile = (int)blockIdx.x + (i / ngroups) * (int)gridDim.x;
        const int grp = i % ngroups;
        const int row0 = tile * G::ROWS + wave * G::RPW + slot * RPS;
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            const uint32_t rb = __umul24((uint32_t)min(row0 + r, N - 1), (uint32_t)nb);
#pragma unroll
            for (int g = 0; g < BG; ++g) {
                const uint32_t blk = rb + (uint32_t)min(grp * LPR * BG + g * LPR + lr, nb - 1);
                const uint4* qp = reinterpret_cast<const uint4*>(Q + blk * 16u);
                if (NTL) {
                    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qp));
                    bf.q[g][r] = make_uint4(t.x, t.y, t.z, t.w);
                } else {
                    bf.q[g][r] = *qp;
                }
                bf.d[g][r] = D[blk];
            }
        }
    };
    GemvBuf<RPS, BG> bufs[NBUF];
#pragma unroll
    for (int j = 0; j + 1 < NBUF; ++j)
        load(bufs[j], j);

    // ---- stage the batch: vector c at smem + c * lds_col (x blocks, then block sums)
#pragma unroll
    for (int u = 0; u < GB_MAXU; ++u) {
        if (u * G::NT < nf) {   // uniform
            const int f = (int)threadIdx.x + u * G::NT;
            const float4 w = xv[u];
            float s = (w.x + w.y) + (w.z + w.w);
            s = group_sum<8>(s);   // 8 consecutive lanes hold one block (n4 is a multiple of 8)
            if (f < nf) {
                const int c = f / n4, i = f % n4;
                float* xl = smem + (size_t)c * lds_col;
                const float fct = (i & 7) < 4 ? 1.f : 0.0625f;
                *reinterpret_cast<float4*>(xl + (i >> 3) * XPAD + (i & 7) * 4) =
                    make_float4(w.x * fct, w.y * fct, w.z * fct, w.w * fct);
                if ((i & 7) == 0)
                    xl[nb * XPAD + (i >> 3)] = s;
            }
        }
    }
    __syncthreads();

    float acc[RPS][NC];
#pragma unroll
    for (int r = 0; r < RPS; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            acc[r][c] = 0.f;

    auto compute = [&](const GemvBuf<RPS, BG>& bf, int i) {
        const int tile = (int)blockIdx.x + (i / ngroups) * (int)gridDim.x;
        const int grp = i % ngroups;
#pragma unroll
        for (int g = 0; g < BG; ++g) {
            const int b = grp * LPR * BG + g * LPR + lr;
            if (b < nb) {
                // codes of this block for every row: element j in cf[r][j], the
                // upper 16 as 16 x code (the staged x there is x / 16)
                float cf[RPS][32];
                float dd[RPS];
#pragma unroll
                for (int r = 0; r < RPS; ++r) {
                    const uint32_t w[4] = {bf.q[g][r].x, bf.q[g][r].y, bf.q[g][r].z, bf.q[g][r].w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t lo = and_opaque(w[k], 0x0f0f0f0fu);
                        const uint32_t hi = and_opaque(w[k], 0xf0f0f0f0u);
                        cf[r][4 * k + 0] = (float)(lo & 0xffu);
                        cf[r][4 * k + 1] = (float)((lo >> 8) & 0xffu);
                        cf[r][4 * k + 2] = (float)((lo >> 16) & 0xffu);
                        cf[r][4 * k + 3] = (float)(lo >> 24);
                        cf[r][16 + 4 * k + 0] = (float)(hi & 0xffu);
                        cf[r][16 + 4 * k + 1] = (float)((hi >> 8) & 0xffu);
                        cf[r][16 + 4 * k + 2] = (float)((hi >> 16) & 0xffu);
                        cf[r][16 + 4 * k + 3] = (float)(hi >> 24);
                    }
                    dd[r] = f16_to_f32((uint16_t)bf.d[g][r]);
                }
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const float* xl = smem + (size_t)c * lds_col;
                    const float4* xp = reinterpret_cast<const float4*>(xl + b * XPAD);
                    float4 x4[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        x4[k] = xp[k];
                    const float m8 = -8.f * xl[nb * XPAD + b];
#pragma unroll
                    for (int r = 0; r < RPS; ++r) {
                        float s0 = 0.f, s1 = 0.f;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            s0 = fmaf(cf[r][4 * k + 0], x4[k].x, s0);
                            s0 = fmaf(cf[r][4 * k + 1], x4[k].y, s0);
                            s0 = fmaf(cf[r][4 * k + 2], x4[k].z, s0);
                            s0 = fmaf(cf[r][4 * k + 3], x4[k].w, s0);
                            s1 = fmaf(cf[r][16 + 4 * k + 0], x4[4 + k].x, s1);
                            s1 = fmaf(cf[r][16 + 4 * k + 1], x4[4 + k].y, s1);
                            s1 = fmaf(cf[r][16 + 4 * k + 2], x4[4 + k].z, s1);
                            s1 = fmaf(cf[r][16 + 4 * k + 3], x4[4 + k].w, s1);
                        }
                        acc[r][c] = fmaf(dd[r], (s0 + s1) + m8, acc[r][c]);
                    }
                }
            }
        }
        if (grp == ngroups - 1) {
            const int row0 = tile * G::ROWS + wave * G::RPW + slot * RPS;
#pragma unroll
            for (int r = 0; r < RPS; ++r)
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const float v = group_sum<LPR>(acc[r][c]);
                    if (lr == 0 && row0 + r < N)
                        Y[(size_t)c * N + row0 + r] = v;
                    acc[r][c] = 0.f;
                }
        }
    };

    for (int base = 0; base < nitems; base += UNR) {
        if (base > 0) {
#pragma unroll
            for (int j = 0; j + 1 < NBUF; ++j)
                load(bufs[j], base + j);
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            if (u + NBUF - 1 < UNR)
                load(bufs[(u + NBUF - 1) % NBUF], base + u + NBUF - 1);
            if (base + u < nitems)
                compute(bufs[u % NBUF], base + u);
        }
    }
}

}  // namespace qd
