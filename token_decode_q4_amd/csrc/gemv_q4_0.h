// gemv_q4_0.h -- q4_0 GEMV for gfx950 (batch 1) and its fused epilogues.
//
// y = W x with W in q4_0 (inferencelayer cuda_llm.rs page, Q4Dev and
// CudaQwen3::gemv: 32-weight blocks, one f16 scale, 16 bytes of nibbles;
// weight = (nibble - 8) * scale).
//
// Work mapping.  A workgroup of NWAVES wave64s owns tiles of rows.  Inside a
// wave, groups of LPR lanes share a row slot and split that row's blocks
// (lane i of the group takes blocks i, i+LPR, ...); each lane keeps RPS rows
// of its slot in flight, so one staged x chunk serves RPS rows.  A lane loads
// a block's 16 nibble bytes with one 128-bit load: consecutive lanes read
// consecutive blocks of a row, so a wave reads LPR*16 contiguous bytes per
// row.  The grid is persistent: a workgroup walks its tiles in (tile, block
// group) work items, keeping NBUF-1 items of loads in flight ahead of the one
// it consumes; x is loaded first, then the first items, then x is staged.
//
// x is staged once per workgroup into LDS, block b at float offset b*36 (the
// 4-float pad keeps the per-lane 128-bit reads of 64 lanes on distinct banks):
// x[32b .. 32b+15] as is and x[32b+16 .. 32b+31] divided by 16 (exact), with
// the block's sum of x beside it.
//
// In-register dequant: a 16-bit field whose only set bits are among its low
// 8 is an f16 subnormal, value field * 2^-24 exactly.  For one 32-bit word w
// of nibbles (bytes 4k..4k+3 of a block) w & 0x000F000F holds the codes of
// elements 4k and 4k+2 as such a pair, w & 0x00F000F0 sixteen times those of
// 16+4k and 16+4k+2, and the same two masks of w >> 8 cover 4k+1, 4k+3,
// 16+4k+1 and 16+4k+3.  v_fma_mix_f32 takes one f16 half as a multiplicand
// of an f32 FMA (subnormal inputs kept, exactly), so the conversion costs
// nothing: 1 shift + 4 ANDs + 8 FMAs per 8 weights, exact products in f32.
// The factor 16 cancels against the staged x/16; the factor 2^-24 is carried
// through the row sums (every partial result is the exact-arithmetic one
// scaled by a power of two, so nothing changes unless a value leaves the
// normal f32 range) and removed once per row.  The -8 offset is applied once
// per block:
//   sum_j (c_j - 8) x_j = sum_j c_j x_j - 8 * sum_j x_j.
// Row sums are reduced across the LPR lanes with butterfly shuffles in a fixed
// order (deterministic).
#pragma once

#include "qd_common.h"

namespace qd {

constexpr int XPAD = 36;  // floats per staged x block (32 + pad)

// LDS floats needed to stage x of nb blocks
__host__ __device__ constexpr int gemv_lds_floats(int nb) { return nb * XPAD + nb; }

// x staging in two halves, so that the x loads fly together with the weight
// loads and with the epilogue's own prologue loads:
//   stage_x_load   issues every x load of this thread (K <= 64*NT floats)
//   stage_x_store  writes the LDS layout
template <int NT>
struct XStage {
    static constexpr int MAXU = 16384 / (4 * NT);
    float4 v[MAXU];
};

// Loads are never under a branch (an index past the end is clamped and its
// value discarded): a load inside a divergent block makes the compiler wait
// for every earlier load at the join, which serialises the whole batch.
template <int NT>
QD_DEV void stage_x_load(const float* __restrict__ x, int nb, XStage<NT>& st)
{
    const int n4 = nb * 8;
#pragma unroll
    for (int u = 0; u < XStage<NT>::MAXU; ++u) {
        if (u * NT < n4) {   // uniform
            const int i = (int)threadIdx.x + u * NT;
            st.v[u] = reinterpret_cast<const float4*>(x)[min(i, n4 - 1)];
        }
    }
}

// Block b at float offset b*XPAD: x[32b .. 32b+15] as is and x[32b+16 .. 32b+31]
// divided by 16 (exact); xs[b] = the block's sum of x.  Starts and ends with
// a barrier (the LDS may still be read by a previous use).
template <int NT>
QD_DEV void stage_x_store(int nb, const XStage<NT>& st, float* xl, float* xs)
{
    const int n4 = nb * 8;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < XStage<NT>::MAXU; ++u) {
        if (u * NT < n4) {   // uniform
            const int i = (int)threadIdx.x + u * NT;
            const float4 w = st.v[u];
            // 8 consecutive lanes hold one block: its sum is a butterfly over them
            float s = (w.x + w.y) + (w.z + w.w);
            s = group_sum<8>(s);
            if (i < n4) {
                const float f = (i & 7) < 4 ? 1.f : 0.0625f;
                *reinterpret_cast<float4*>(xl + (i >> 3) * XPAD + (i & 7) * 4) =
                    make_float4(w.x * f, w.y * f, w.z * f, w.w * f);
                if ((i & 7) == 0)
                    xs[i >> 3] = s;
            }
        }
    }
    __syncthreads();
}

// w & m through an opaque instruction, so that each mask stays one v_and_b32
// instead of being re-derived per field (bit-field extracts, per-half masks)
QD_DEV uint32_t and_opaque(uint32_t w, uint32_t m)
{
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(w), "v"(m));
    return r;
}

// Q4_SUB = 2^-24, the value of the f16 subnormal with field 1
constexpr float Q4_SUB = 0x1p-24f;
constexpr float Q4_UNSUB = 0x1p24f;

// Q4_SUB * sum_j c_j * x_j over one block (codes c_j in [0, 15]); xv = the
// staged block (x[16..31] divided by 16)
QD_DEV float q4_block_dot(uint4 q, const float4 (&xv)[8])
{
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t t = w[k] >> 8;
        const half2_t a = __builtin_bit_cast(half2_t, and_opaque(w[k], 0x000F000Fu));   // 4k, 4k+2
        const half2_t b = __builtin_bit_cast(half2_t, and_opaque(t, 0x000F000Fu));      // 4k+1, 4k+3
        const half2_t c = __builtin_bit_cast(half2_t, and_opaque(w[k], 0x00F000F0u));   // 16 x (16+4k, 16+4k+2)
        const half2_t e = __builtin_bit_cast(half2_t, and_opaque(t, 0x00F000F0u));      // 16 x (16+4k+1, 16+4k+3)
        s0 = fmaf((float)a[0], xv[k].x, s0);
        s0 = fmaf((float)b[0], xv[k].y, s0);
        s0 = fmaf((float)a[1], xv[k].z, s0);
        s0 = fmaf((float)b[1], xv[k].w, s0);
        s1 = fmaf((float)c[0], xv[4 + k].x, s1);
        s1 = fmaf((float)e[0], xv[4 + k].y, s1);
        s1 = fmaf((float)c[1], xv[4 + k].z, s1);
        s1 = fmaf((float)e[1], xv[4 + k].w, s1);
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

// Registers of one work item: BG blocks x RPS rows of this lane.
template <int RPS, int BG>
struct GemvBuf {
    uint4 q[BG][RPS];
    uint32_t d[BG][RPS];   // f16 scale bits
};

// Persistent GEMV driver.  Work items are (tile, block group) pairs, tiles
// strided by gridDim.x.  NBUF register buffers rotate: the loads of item
// i + NBUF - 1 are issued before item i is consumed.  `epi` receives every
// finished tile:
//   epi.issue(row0)             first of all: the epilogue's own loads (row0 =
//                               this lane's first row of its first tile)
//   epi.finish()                after x is staged: what needs those loads
//   epi.tile(row0, acc, lead)   acc[RPS] = dot products of rows row0 .. row0+RPS-1
template <int LPR, int RPS, int NWAVES, int BG, int NBUF, int UNR, bool NTL, class Epi>
QD_DEV void gemv_run(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
                     const float* __restrict__ x, int N, int nb, float* xl, float* xs, Epi& epi)
{
    static_assert(NBUF >= 1 && NBUF <= 6, "buffers");
    static_assert(UNR >= NBUF, "unroll");
    using G = GemvGeom<LPR, RPS, NWAVES>;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int slot = lane / LPR, lr = lane % LPR;
    const int ntiles = (N + G::ROWS - 1) / G::ROWS;
    const int ngroups = (nb + LPR * BG - 1) / (LPR * BG);
    const int my_tiles = (int)blockIdx.x < ntiles ? (ntiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    const int nitems = my_tiles * ngroups;
    QD_MARK(0);

    // issue the loads of item i (clamped: an item past the end reloads the last one)
    auto load = [&](GemvBuf<RPS, BG>& bf, int i) {
        i = max(0, min(i, nitems - 1));   // rows and blocks below are clamped too
        const int tile = (int)blockIdx.x + (i / ngroups) * (int)gridDim.x;
        const int grp = i % ngroups;
        const int row0 = tile * G::ROWS + wave * G::RPW + slot * RPS;
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            // 32-bit block index (the host keeps N * nb * 16 below 2^32)
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
    float acc[RPS];
#pragma unroll
    for (int r = 0; r < RPS; ++r)
        acc[r] = 0.f;
    // consume item i from buffer bf
    auto compute = [&](const GemvBuf<RPS, BG>& bf, int i) {
        const int tile = (int)blockIdx.x + (i / ngroups) * (int)gridDim.x;
        const int grp = i % ngroups;
#pragma unroll
        for (int g = 0; g < BG; ++g) {
            const int b = grp * LPR * BG + g * LPR + lr;
            if (b < nb) {
                float4 xv[8];
                const float4* xp = reinterpret_cast<const float4*>(xl + b * XPAD);
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    xv[k] = xp[k];
                const float m8 = (-8.f * Q4_SUB) * xs[b];
#pragma unroll
                for (int r = 0; r < RPS; ++r)
                    acc[r] = fmaf(f16_to_f32((uint16_t)bf.d[g][r]), q4_block_dot(bf.q[g][r], xv) + m8,
                                  acc[r]);
            }
        }
        if (grp == ngroups - 1) {
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                acc[r] = group_sum<LPR>(acc[r]) * Q4_UNSUB;
            const int row0 = tile * G::ROWS + wave * G::RPW + slot * RPS;
            epi.tile(row0, acc, lr == 0);
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                acc[r] = 0.f;
        }
    };

    // x (and the epilogue's inputs) first: loads return in order, so x can be
    // staged while the weight items behind it are still arriving
    epi.issue((int)blockIdx.x * G::ROWS + wave * G::RPW + slot * RPS);
    XStage<G::NT> xst;
    stage_x_load<G::NT>(x, nb, xst);
    GemvBuf<RPS, BG> bufs[NBUF];
#pragma unroll
    for (int j = 0; j + 1 < NBUF; ++j)
        load(bufs[j], j);
    stage_x_store<G::NT>(nb, xst, xl, xs);   // ends with a barrier
    epi.finish();
    QD_MARK(1);
    // Items in chunks of UNR, each chunk fully unrolled, so that no loaded
    // register is live across a loop back-edge (the compiler copies such a
    // register at the latch and waits for every load to do it) and no load
    // is issued past the chunk.  With UNR >= the items of a workgroup there is
    // a single chunk.
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
    QD_MARK(2);
}

// 1 / sqrt(mean(x^2) + eps) from the per-workgroup partial sums of x^2 written
// by the producer of x.  Every wave computes it on its own (no LDS, no
// barrier): issue() loads up to RMS_U * 64 partials into registers, finish()
// sums them -- then any further ones -- in a fixed order, so every wave of
// every workgroup gets the same value.
constexpr int RMS_U = 16;
struct RmsPartials {
    const float* ss_part;
    int n_part;
    float v[RMS_U];
    QD_DEV void issue()
    {
        const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
        for (int u = 0; u < RMS_U; ++u)
            v[u] = ss_part[min(lane + u * WAVE, n_part - 1)];   // n_part >= 1
    }
    QD_DEV float finish(int n, float eps) const
    {
        const int lane = threadIdx.x & (WAVE - 1);
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < RMS_U; ++u)
            s += (lane + u * WAVE < n_part) ? v[u] : 0.f;
        for (int i = lane + RMS_U * WAVE; i < n_part; i += WAVE)
            s += ss_part[i];
        s = group_sum<WAVE>(s);
        return 1.0f / sqrtf(s / (float)n + eps);
    }
};

// ----------------------------------------------------------------- epilogues

// y[row] = acc
struct EpiStore {
    float* y;
    int N;
    QD_DEV void issue(int) {}
    QD_DEV void finish() {}
    template <int RPS>
    QD_DEV void tile(int row0, const float (&acc)[RPS], bool lead)
    {
        if (lead) {
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                if (row0 + r < N)
                    y[row0 + r] = acc[r];
        }
    }
};

template <int LPR, int RPS, int NWAVES, int BG, int NBUF, int UNR, bool NTL>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_plain(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
             const float* __restrict__ x, float* __restrict__ y, int N, int nb)
{
    extern __shared__ __align__(16) float smem[];   // 16-byte aligned: x is read as float4
    EpiStore e{y, N};
    gemv_run<LPR, RPS, NWAVES, BG, NBUF, UNR, NTL>(D, Q, x, N, nb, smem, smem + nb * XPAD, e);
}

}  // namespace qd
