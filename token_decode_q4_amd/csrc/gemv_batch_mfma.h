// gemv_batch_mfma.h -- batched q4_0 GEMV on the matrix cores (gfx950):
// Y[b] = W X[b] for 1 <= B <= 16 vectors, every weight read once.
//
// The batched decode of the inferencelayer cuda_llm.rs page (its q4 GEMV arm
// against the bf16 GEMM arm at M = 1 .. 16 tokens, section on the batched
// head-to-head).  With B vectors the GEMV is a skinny matrix product; here it
// runs as one v_mfma_f32_16x16x32_f16 per q4_0 block and 16 weight rows.
//
// Operands.  The first operand (M = 16) is the vectors, the second (N = 16)
// the weight rows, K = 32 = one block.  Lane l = (r, kg), r = l % 16,
// kg = l / 16, supplies 8 values of vector r (first operand) and 8 codes of
// weight row r (second operand), both at the K slots of lane group kg, and
// receives the products of vectors 4kg .. 4kg+3 with row r.  A lane's outputs
// therefore share one weight row, and the block's scale d is one number per
// lane: each block's MFMA starts from zero and the lane adds d * P to its
// sums (v_fma_mix_f32 takes d as an f16 half, no conversion).
//
// Codes.  Lane group kg takes word kg (bytes 4kg .. 4kg+3) of the block: the
// low nibbles are elements 4kg .. 4kg+3, the high ones 16+4kg .. 16+4kg+3.
// (w & 0x000F000F) | 0x64006400 holds two codes as the f16 values 1024 + c,
// (w & 0x00F000F0) | 0x64006400 two as 1024 + 16c; packed f16 adds of -1032
// and -1152 leave c - 8 and 16(c - 8), exactly.  With t = w >> 8 the same two
// masks give the odd elements.  K slot order of a lane group: 4kg, 4kg+2,
// 4kg+1, 4kg+3, then the same four plus 16; x of the high four is staged
// divided by 16 (exact).  Each lane loads 16 bytes (one block of its row) per
// 4 blocks; a 4 x 4 transpose of words across the lane groups (v_permlane32
// and v_permlane16 swaps) gives every lane group its word of each of the
// four blocks.  The 8 f16 scales of a lane group's eighth of a 32-block chunk
// come with one 16-byte load and are shared by the same swaps.
//
// x enters as an f16 pair after a power of two s per (vector, chunk of 32
// blocks) that puts the chunk's largest |x| in [2^13, 2^14): hi = RN(x s),
// lo = RN(x s - hi), about 22 significant bits at any input scale, no f16
// overflow.  Both pairs meet the same codes (two MFMAs per block, products
// exact in f32); each chunk's sums are multiplied by 1/s, exactly.  x is
// staged per chunk in LDS in the first operand's layout
// [block][lane group][hi, lo][vector][8 halves].  All weight loads of a chunk
// (one 16-byte load per lane, row group and step of 4 blocks) are in flight
// before the chunk is staged; the next chunk's x, scales and weights are
// issued while the current one is computed.
//
// Grid (row tiles, K slices): slice y takes chunks [y * kch, (y + 1) * kch)
// and writes its partial products to Y + y * ystride.  A workgroup of 4 waves
// owns 64 * RG rows (RG groups of 16 per wave).  dvec: the scales may be
// loaded 16 bytes at a time (nb % 8 == 0 and D 16-byte aligned).
#pragma once

#include "qd_common.h"

namespace qd {

typedef _Float16 gbm_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 gbm_half2 __attribute__((ext_vector_type(2)));
typedef float gbm_floatx4 __attribute__((ext_vector_type(4)));

constexpr int GBM_MAXB = 16;              // vectors per launch
constexpr int GBM_KC = 32;                // blocks per staged chunk
constexpr int GBM_NW = 4;                 // waves per workgroup
constexpr int GBM_STEPS = GBM_KC / 4;     // 4-block steps per chunk

// rows per workgroup with RG row groups per wave
__host__ __device__ constexpr int gbm_rows(int rg) { return GBM_NW * 16 * rg; }

// LDS bytes of one staged chunk (16 vector slots)
__host__ __device__ constexpr size_t gemv_batch_mfma_lds_bytes()
{
    return (size_t)GBM_KC * 4 * 2 * 16 * 8 * sizeof(_Float16);
}

// 4 x 4 transpose of words across the lane groups: before, lane group g holds
// word w of block g in w[w]; after, lane group g holds word g of block b in w[b]
QD_DEV void gbm_transpose4(uint32_t (&w)[4])
{
    const auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto e = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    w[0] = c[0];
    w[1] = c[1];
    w[2] = e[0];
    w[3] = e[1];
}

// the word v of lane groups 0..3 (same r) into g[0..3], in every lane group
QD_DEV void gbm_allgather4(uint32_t v, uint32_t (&g)[4])
{
    const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);     // groups kg & 1, (kg & 1) | 2
    const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
    g[0] = b[0];
    g[1] = b[1];
    g[2] = c[0];
    g[3] = c[1];
}

// (a & m) | o in one instruction (the compiler would emit an AND and an OR:
// a VOP3 instruction takes no literal on gfx9, so m and o come in registers)
QD_DEV uint32_t gbm_and_or(uint32_t a, uint32_t m, uint32_t o)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
    return r;
}

// the second operand of one block from this lane group's word w of it
QD_DEV gbm_half8 gbm_codes(uint32_t w)
{
    const uint32_t bias = 0x64006400u, t = w >> 8;
    const gbm_half2 k8 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const gbm_half2 k128 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const gbm_half2 p0 = __builtin_bit_cast(gbm_half2, gbm_and_or(w, 0x000F000Fu, bias)) + k8;     // 4kg, 4kg+2
    const gbm_half2 p2 = __builtin_bit_cast(gbm_half2, gbm_and_or(t, 0x000F000Fu, bias)) + k8;     // 4kg+1, 4kg+3
    const gbm_half2 p1 = __builtin_bit_cast(gbm_half2, gbm_and_or(w, 0x00F000F0u, bias)) + k128;   // 16 x (16+4kg, ..+2)
    const gbm_half2 p3 = __builtin_bit_cast(gbm_half2, gbm_and_or(t, 0x00F000F0u, bias)) + k128;   // 16 x (..+1, ..+3)
    return gbm_half8{p0[0], p0[1], p2[0], p2[1], p1[0], p1[1], p3[0], p3[1]};
}

// s = 2^k with a * s in [2^13, 2^14) for the largest magnitude a of a chunk
// of a vector (k clamped to [-100, 100]; 1 when a is 0 or not finite)
QD_DEV float gbm_scale_for(float a)
{
    if (!(a > 0.f) || !(a <= 3.4e38f))
        return 1.f;
    int e;
    (void)frexpf(a, &e);   // a in [2^(e-1), 2^e)
    return ldexpf(1.f, max(-100, min(100, 14 - e)));
}

// staging items (block, lane group, vector) per thread per chunk
template <int NC>
struct GbmItems {
    static constexpr int N = (GBM_KC * 4 * NC + GBM_NW * WAVE - 1) / (GBM_NW * WAVE);
};
template <int NC>
struct GbmX {
    float4 xa[GbmItems<NC>::N];        // x of this thread's staging items: elements 4kg .. 4kg+3
    float4 xb[GbmItems<NC>::N];        //   and 16+4kg .. 16+4kg+3
};

template <int NC, int RG>
__global__ void __launch_bounds__(GBM_NW* WAVE)
k_gemv_batch_mfma(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
                  const float* __restrict__ X, float* __restrict__ Y, int N, int nb, int kch, size_t ystride,
                  int dvec)
{
    static_assert(NC >= 1 && NC <= 16, "batch");
    constexpr int NT = GBM_NW * WAVE;
    constexpr int NITEM = GBM_KC * 4 * NC;           // staging items of a chunk
    extern __shared__ __align__(16) _Float16 xs[];   // [KC][4][2][16][8]
    __shared__ unsigned xmax[2][GBM_MAXB];            // |x| maxima (f32 bits), by chunk parity
    __shared__ float xinv[2][GBM_MAXB];               // 1/s of a staged chunk, by parity
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r = lane & 15, kg = lane >> 4;
    const int K = nb * 32;
    const int nch = (nb + GBM_KC - 1) / GBM_KC;
    const int c0 = (int)blockIdx.y * kch, c1 = min(nch, c0 + kch);   // this slice's chunks
    Y += (size_t)blockIdx.y * ystride;
    const int row0 = (int)blockIdx.x * gbm_rows(RG) + wave * 16 * RG;
    size_t rb[RG];   // first block of this lane's row in each row group
#pragma unroll
    for (int g = 0; g < RG; ++g)
        rb[g] = (size_t)min(row0 + 16 * g + r, N - 1) * (size_t)nb;
    const int nsteps = (c1 - c0) * GBM_STEPS;
    if (nsteps <= 0) {   // an empty slice (the host never launches one): zeros
        for (int g = 0; g < RG; ++g) {
            const int row = row0 + 16 * g + r;
            for (int i = 0; i < 4; ++i)
                if (row < N && 4 * kg + i < NC)
                    Y[(size_t)(4 * kg + i) * N + row] = 0.f;
        }
        return;
    }

    if (threadIdx.x < 2 * GBM_MAXB) {   // ordered by the first stage's barriers
        xmax[threadIdx.x / GBM_MAXB][threadIdx.x % GBM_MAXB] = 0u;
        xinv[threadIdx.x / GBM_MAXB][threadIdx.x % GBM_MAXB] = 0.f;
    }
    if constexpr (NC < 16) {   // vector slots past the batch stay zero
        constexpr int NZ = GBM_KC * 4 * 2 * (16 - NC);
        for (int i = threadIdx.x; i < NZ; i += NT) {
            const int v = NC + i % (16 - NC), q = i / (16 - NC);
            *reinterpret_cast<uint4*>(xs + ((size_t)q * 16 + v) * 8) = make_uint4(0u, 0u, 0u, 0u);
        }
    }

    // weight loads of step s (blocks 4j .. 4j+3 of its chunk; this lane: 4j + kg;
    // clamped, never a branch around a load)
    struct Buf {
        uint4 q[RG];
    };
    auto load = [&](Buf& bf, int s) {
        s = min(s, nsteps - 1);
        const int blk = min((c0 + s / GBM_STEPS) * GBM_KC + (s % GBM_STEPS) * 4 + kg, nb - 1);
#pragma unroll
        for (int g = 0; g < RG; ++g)
            bf.q[g] = *reinterpret_cast<const uint4*>(Q + (rb[g] + (size_t)blk) * 16u);
    };
    // scales of chunk c: this lane group's eighth, blocks 32c + 8kg .. 8kg+7
    auto load_d = [&](uint4 (&dq)[RG], int c) {
        const int b0 = c * GBM_KC + 8 * kg;
        if (dvec) {   // uniform: nb % 8 == 0 and D 16-byte aligned
            const int bq = min(b0, nb - 8);
#pragma unroll
            for (int g = 0; g < RG; ++g)
                dq[g] = *reinterpret_cast<const uint4*>(D + rb[g] + (size_t)bq);
        } else {
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    h[e] = D[rb[g] + (size_t)min(b0 + e, nb - 1)];
                dq[g] = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
            }
        }
    };
    auto load_x = [&](GbmX<NC>& bf, int c) {
#pragma unroll
        for (int u = 0; u < GbmItems<NC>::N; ++u) {
            const int i = min((int)threadIdx.x + u * NT, NITEM - 1);
            const int v = i % NC, q = (i / NC) & 3, bl = i / (4 * NC);
            const int b = min(c * GBM_KC + bl, nb - 1);
            const float* xp = X + (size_t)v * K + (size_t)b * 32 + 4 * q;
            bf.xa[u] = *reinterpret_cast<const float4*>(xp);
            bf.xb[u] = *reinterpret_cast<const float4*>(xp + 16);
        }
    };
    // stage chunk c from the registers of its loads: the chunk's largest |x|
    // per vector (LDS atomic max of the f32 bits, which order like the values
    // for |x|), then the scaled split
    auto stage = [&](const GbmX<NC>& bf, int c, int par) {
        __syncthreads();   // the previous chunk's reads of x are done
#pragma unroll
        for (int u = 0; u < GbmItems<NC>::N; ++u) {
            const int i = (int)threadIdx.x + u * NT;
            if (i >= NITEM)   // uniform except in the last round of an odd batch
                continue;
            const bool in = c * GBM_KC + i / (4 * NC) < nb;
            const float4 a = bf.xa[u], h = bf.xb[u];
            const float mx = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                                   fmaxf(fmaxf(fabsf(h.x), fabsf(h.y)), fmaxf(fabsf(h.z), fabsf(h.w))));
            if (in)
                atomicMax(&xmax[par][i % NC], __float_as_uint(mx));
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < GbmItems<NC>::N; ++u) {
            const int i = (int)threadIdx.x + u * NT;
            if (i >= NITEM)
                continue;
            const int v = i % NC, q = (i / NC) & 3, bl = i / (4 * NC);
            const bool in = c * GBM_KC + bl < nb;
            const float sc = gbm_scale_for(__uint_as_float(xmax[par][v]));
            const float sh = sc * 0.0625f;
            const float4 a = bf.xa[u], h = bf.xb[u];
            float e[8] = {a.x * sc, a.z * sc, a.y * sc, a.w * sc, h.x * sh, h.z * sh, h.y * sh, h.w * sh};
            gbm_half8 xh, xl;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float f = in ? e[k] : 0.f;
                const _Float16 t = (_Float16)f;
                xh[k] = t;
                xl[k] = (_Float16)(f - (float)t);
            }
            _Float16* dst = xs + ((size_t)(bl * 4 + q) * 2 * 16 + v) * 8;
            *reinterpret_cast<gbm_half8*>(dst) = xh;
            *reinterpret_cast<gbm_half8*>(dst + 16 * 8) = xl;
        }
        if (threadIdx.x < NC) {
            xinv[par][threadIdx.x] = 1.0f / gbm_scale_for(__uint_as_float(xmax[par][threadIdx.x]));
            // the other parity was last read before this stage's first barrier
            // and is next written after the following stage's first barrier
            xmax[par ^ 1][threadIdx.x] = 0u;
        }
        __syncthreads();
    };

    float acc[RG][4];
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[g][i] = 0.f;
    // A whole chunk of weight loads is in flight before its x is staged: the
    // first chunk's are issued here, the next chunk's step by step as the
    // current chunk frees its buffers; its scales and x come with them.
    // x and scales first: loads return in order, so the chunk is staged while
    // its weight loads are still arriving
    GbmX<NC> xr;
    load_x(xr, c0);
    uint4 dq[RG];
    load_d(dq, c0);
    Buf bufs[GBM_STEPS];
#pragma unroll
    for (int u = 0; u < GBM_STEPS; ++u)
        load(bufs[u], u);
    const gbm_floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    int par = 0;
    for (int c = c0; c < c1; ++c, par ^= 1) {
        stage(xr, c, par);
        uint32_t dg[RG][4][4];   // [group][lane group q][dword]: halves = scales of blocks 8q ..
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const uint32_t dw[4] = {dq[g].x, dq[g].y, dq[g].z, dq[g].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint32_t t[4];
                gbm_allgather4(dw[k], t);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    dg[g][q][k] = t[q];
            }
        }
        if (c + 1 < c1) {   // uniform
            load_x(xr, c + 1);
            load_d(dq, c + 1);
        }
        float cacc[RG][4];
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                cacc[g][i] = 0.f;
        const int sbase = (c - c0) * GBM_STEPS;
#pragma unroll
        for (int j = 0; j < GBM_STEPS; ++j) {
            uint32_t w[RG][4];
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                w[g][0] = bufs[j].q[g].x;
                w[g][1] = bufs[j].q[g].y;
                w[g][2] = bufs[j].q[g].z;
                w[g][3] = bufs[j].q[g].w;
                gbm_transpose4(w[g]);
            }
            load(bufs[j], sbase + GBM_STEPS + j);   // the same step of the next chunk
            // the step's 4 blocks side by side: their x operands, codes, 8
            // independent MFMAs into 4 accumulators, then the scaled sums
            gbm_half8 xh[4], xl[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const _Float16* src = xs + ((size_t)((4 * j + b) * 4 + kg) * 2 * 16 + r) * 8;
                xh[b] = *reinterpret_cast<const gbm_half8*>(src);
                xl[b] = *reinterpret_cast<const gbm_half8*>(src + 16 * 8);
            }
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                gbm_floatx4 p[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const gbm_half8 wop = gbm_codes(w[g][b]);
                    p[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[b], wop, zero, 0, 0, 0);
                    p[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[b], wop, p[b], 0, 0, 0);
                }
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int bl = 4 * j + b;   // block within the chunk
                    const uint32_t dd = dg[g][bl >> 3][(bl & 7) >> 1];
                    const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)((bl & 1) ? dd >> 16 : dd));
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        cacc[g][i] = fmaf((float)dh, p[b][i], cacc[g][i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float inv = xinv[par][4 * kg + i];   // vector 4kg + i
#pragma unroll
            for (int g = 0; g < RG; ++g)
                acc[g][i] = fmaf(cacc[g][i], inv, acc[g][i]);
        }
        // keeps the next chunk's loads where they are issued (the compiler would
        // otherwise sink them to the top of the next iteration, next to their use)
        asm volatile("" ::: "memory");
    }
    // acc[g][i] = vector 4kg + i, row row0 + 16g + r
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int row = row0 + 16 * g + r;
        if (row < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * kg + i < NC)
                    Y[(size_t)(4 * kg + i) * N + row] = acc[g][i];
        }
    }
}

// ---------------------------------------------------------------------------
// x split once, outside the product (the batched decode step, prefill).  The
// producer of a product's input writes it already split, in the staged
// layout, one 64 KB chunk at a time: with NG groups of 16 vector slots
// (S = 16 NG slots) a chunk holds KCB = 32 / NG blocks,
//   XP[chunk][block][lane group][hi, lo][S slots][8 halves],
// and XS[chunk][S] = 1/s of each vector's chunk.  Slots past the batch and
// blocks past the end stay zero (the buffers are cleared once when
// allocated).  The product then copies a chunk into LDS, once per workgroup,
// with no arithmetic.
constexpr int GBM_XP_CHUNK = GBM_KC * 4 * 2 * 16 * 8;   // halves per chunk (any NG)

__host__ __device__ constexpr int gbm_kcb(int ng) { return GBM_KC / ng; }          // blocks per chunk
__host__ __device__ constexpr int gbm_nchunks(int nb, int ng) { return (nb + gbm_kcb(ng) - 1) / gbm_kcb(ng); }
// threads of a producer workgroup of one chunk (4 per block; at least a wave,
// the items past the chunk's blocks idle)
__host__ __device__ constexpr int gbm_chunk_threads(int ng) { return 4 * gbm_kcb(ng) > 64 ? 4 * gbm_kcb(ng) : 64; }

// largest |.| of the 8 elements in slot order (the high four undone)
QD_DEV float gbm_xp_absmax(const float (&e)[8])
{
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        m = fmaxf(m, fabsf(e[k]) * (k < 4 ? 1.f : 16.f));
    return m;
}

// writes the split pair of (chunk c, block bl, lane group kg, slot v), scale s
QD_DEV void gbm_xp_put(_Float16* __restrict__ XP, int ng, int c, int bl, int kg, int v, const float (&e)[8],
                       float s)
{
    gbm_half8 xh, xl;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float f = e[k] * s;
        const _Float16 t = (_Float16)f;
        xh[k] = t;
        xl[k] = (_Float16)(f - (float)t);
    }
    const int S = 16 * ng;
    _Float16* dst = XP + (size_t)c * GBM_XP_CHUNK + ((size_t)(bl * 4 + kg) * 2 * S + v) * 8;
    *reinterpret_cast<gbm_half8*>(dst) = xh;
    *reinterpret_cast<gbm_half8*>(dst + S * 8) = xl;
}

// largest value over a workgroup of 64 or 128 threads (a chunk's items); every
// thread gets it; red >= 2 floats
QD_DEV float gbm_chunk_max(float m, float* red)
{
    m = group_max<WAVE>(m);
    if ((threadIdx.x & (WAVE - 1)) == 0)
        red[threadIdx.x / WAVE] = m;
    __syncthreads();
    return blockDim.x > WAVE ? fmaxf(red[0], red[1]) : red[0];
}

// grid (chunks, B), gbm_chunk_threads(ng) threads (one per (block, lane group) item):
// vector b of X [B][nb * 32] into XP / XS with NG = ng slot groups.  With a
// gate (vector b's at gate + b * gstride, as ngslab partial products gslab
// floats apart, added in slab order) x is first multiplied by sigmoid(gate),
// as the decode step gates the merged attention output.
__global__ void __launch_bounds__(128)
k_xsplit_batch(const float* __restrict__ X, int nb, int ng, _Float16* __restrict__ XP, float* __restrict__ XS,
               const float* __restrict__ gate = nullptr, int gstride = 0, int ngslab = 1, size_t gslab = 0)
{
    __shared__ float red[2];
    const int c = blockIdx.x, b = blockIdx.y;
    const int bl = threadIdx.x >> 2, kg = threadIdx.x & 3, blk = c * gbm_kcb(ng) + bl;
    const bool in = bl < gbm_kcb(ng) && blk < nb;
    float e[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (in) {
        const size_t off = (size_t)blk * 32 + 4 * kg;
        float xv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const size_t i = off + (k < 4 ? k : 12 + k);   // elements 4kg.., then 16+4kg..
            float x = X[(size_t)b * nb * 32 + i];
            if (gate) {   // uniform
                const float* gp = gate + (size_t)b * gstride + i;
                float g = gp[0];
                for (int q = 1; q < ngslab; ++q)
                    g += gp[q * gslab];
                x *= 1.0f / (1.0f + expf(-g));
            }
            xv[k] = x;
        }
        const float q = 0.0625f;
        e[0] = xv[0];
        e[1] = xv[2];
        e[2] = xv[1];
        e[3] = xv[3];
        e[4] = xv[4] * q;
        e[5] = xv[6] * q;
        e[6] = xv[5] * q;
        e[7] = xv[7] * q;
    }
    const float s = gbm_scale_for(gbm_chunk_max(gbm_xp_absmax(e), red));
    if (in)
        gbm_xp_put(XP, ng, c, bl, kg, b, e, s);
    if (threadIdx.x == 0)
        XS[c * 16 * ng + b] = 1.0f / s;
}

// The product on a split x: grid (row tiles, K slices) as k_gemv_batch_mfma
// (K slices in units of KCB-block chunks), B <= 16 NG vectors at run time
// (slots past B are zero in XP); Y[b] for b < B.  With NG = 2 each block's
// codes, built once, meet two 16-vector groups: the code-building work per
// vector halves.  A chunk enters LDS in SUB stages of KCB / SUB blocks (32 KB
// each with SUB = 2), so that four workgroups fit a compute unit's LDS; each
// block's scaled products are folded into the stage's sums as soon as they
// are made (held otherwise, the 16 blocks' products would take 64 more
// registers per lane and halve the waves a SIMD holds).
constexpr int GBM_XP_SUB = 2;   // stages per chunk (one with NG = 4: 8 blocks)

__host__ __device__ constexpr int gbm_xp_sub(int ng) { return ng == 4 ? 1 : GBM_XP_SUB; }

__host__ __device__ constexpr size_t gbm_xp_lds_bytes(int sub = GBM_XP_SUB)
{
    return (size_t)GBM_XP_CHUNK * sizeof(_Float16) / sub;
}

template <int RG, int NG, int DV, int SUB = gbm_xp_sub(NG)>
__global__ void __launch_bounds__(GBM_NW* WAVE)
k_gemv_batch_xp(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
                const _Float16* __restrict__ XP, const float* __restrict__ XS, float* __restrict__ Y,
                int N, int nb, int B, int kch, size_t ystride, const float* __restrict__ SQ = nullptr,
                int nsq = 0, float hn = 1.f, float eps = 0.f)
{
    static_assert(NG == 1 || NG == 2 || NG == 4, "slot groups");
    constexpr int KCB = GBM_KC / NG;      // blocks per chunk
    constexpr int KS = KCB / SUB;         // blocks per stage
    static_assert(KS % 8 == 0 && KS * SUB == KCB, "a stage holds whole eighths of a chunk");
    constexpr int STEPS = KS / 4;         // 4-block steps per stage
    constexpr int S = 16 * NG;            // vector slots
    constexpr int QW = 16 / SUB;          // 1 KB copies per wave and stage
    extern __shared__ __align__(16) _Float16 xs[];   // one stage of XP
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r = lane & 15, kg = lane >> 4;
    const int nch = (nb + KCB - 1) / KCB, nst = (nb + KS - 1) / KS;
    const int c0 = (int)blockIdx.y * kch, c1 = min(nch, c0 + kch);
    const int s0 = c0 * SUB, s1 = min(nst, c1 * SUB);   // this slice's stages
    Y += (size_t)blockIdx.y * ystride;
    const int row0 = (int)blockIdx.x * gbm_rows(RG) + wave * 16 * RG;
    size_t rb[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g)
        rb[g] = (size_t)min(row0 + 16 * g + r, N - 1) * (size_t)nb;
    const int nsteps = (s1 - s0) * STEPS;
    if (nsteps <= 0) {   // an empty slice (the host never launches one): zeros
        for (int g = 0; g < RG; ++g) {
            const int row = row0 + 16 * g + r;
            for (int v = 4 * kg; v < S; v += 16)
                for (int i = 0; i < 4; ++i)
                    if (row < N && v + i < B)
                        Y[(size_t)(v + i) * N + row] = 0.f;
        }
        return;
    }
    struct Buf {
        uint4 q[RG];
    };
    auto load = [&](Buf& bf, int s) {
        s = min(s, nsteps - 1);
        const int blk = min((s0 + s / STEPS) * KS + (s % STEPS) * 4 + kg, nb - 1);
#pragma unroll
        for (int g = 0; g < RG; ++g)
            bf.q[g] = *reinterpret_cast<const uint4*>(Q + (rb[g] + (size_t)blk) * 16u);
    };
    // scales of stage st: lane group kg's eighth-of-32 blocks, st*KS + 8kg .. +7
    // (the lane groups past KS / 8 load scales no block of the stage uses)
    auto load_d = [&](uint4 (&dq)[RG], int st) {
        const int b0 = st * KS + 8 * kg;
        if constexpr (DV) {   // nb % 8 == 0 and D 16-byte aligned
            const int bq = min(b0, nb - 8);
#pragma unroll
            for (int g = 0; g < RG; ++g)
                dq[g] = *reinterpret_cast<const uint4*>(D + rb[g] + (size_t)bq);
        } else {
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    h[e] = D[rb[g] + (size_t)min(b0 + e, nb - 1)];
                dq[g] = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
            }
        }
    };
    // stage st of XP into LDS (its blocks are contiguous in the chunk): wave w
    // copies QW KB, 1 KB per instruction
    auto dma_x = [&](int st) {
        const _Float16* src = XP + (size_t)(st / SUB) * GBM_XP_CHUNK + (size_t)(st % SUB) * (GBM_XP_CHUNK / SUB) +
                              (size_t)wave * QW * 512 + lane * 8;
#pragma unroll
        for (int q = 0; q < QW; ++q)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(src + q * 512),
                (__attribute__((address_space(3))) void*)(xs + (wave * QW + q) * 512), 16, 0, 0);
    };
    auto load_inv = [&](float4 (&inv)[NG], int st) {
#pragma unroll
        for (int h = 0; h < NG; ++h)
            inv[h] = *reinterpret_cast<const float4*>(XS + (st / SUB) * S + 16 * h + 4 * kg);
    };

    float acc[NG][RG][4];
#pragma unroll
    for (int h = 0; h < NG; ++h)
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[h][g][i] = 0.f;
    // an input split without its RMSNorm (SQ: the chunk sums of x^2, nsq <=
    // 16 NQR chunks, hn = the row length): 1/rms of each of this lane's
    // vectors multiplies its sums at the end.  Lane r of a lane group loads
    // chunks r, r + 16, .. (clamped, zero past nsq) first; the 16 lanes'
    // values are added, in a fixed order, once the first stage's wait has
    // seen them land.
    constexpr int NQR = NG == 4 ? 4 : 2;
    const bool norm = SQ != nullptr;
    const int nq = norm ? nsq : 0;
    float4 sq4[NQR][NG];
    {
        const float* sqp = norm ? SQ : XS;
        const int last = max(nq - 1, 0);
#pragma unroll
        for (int u = 0; u < NQR; ++u)
#pragma unroll
            for (int h = 0; h < NG; ++h)
                sq4[u][h] = *reinterpret_cast<const float4*>(sqp + (size_t)min(r + 16 * u, last) * S + 16 * h + 4 * kg);
    }
    // x first (loads complete in order), then the scales, then every weight
    // load of the first stage; the next stage's weights are issued while the
    // current one is computed, its x and scales right after it
    dma_x(s0);
    uint4 dq[RG];
    load_d(dq, s0);
    float4 inv[NG];
    load_inv(inv, s0);
    Buf bufs[STEPS];
#pragma unroll
    for (int u = 0; u < STEPS; ++u)
        load(bufs[u], u);
    const gbm_floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    float rinv[NG][4];
    for (int st = s0; st < s1; ++st) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this stage's x (and everything before it) landed
        __syncthreads();
        if (st == s0) {   // uniform
#pragma unroll
            for (int h = 0; h < NG; ++h) {
                float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < NQR; ++u) {
                    const float on = r + 16 * u < nq ? 1.f : 0.f;
                    v[0] += sq4[u][h].x * on;
                    v[1] += sq4[u][h].y * on;
                    v[2] += sq4[u][h].z * on;
                    v[3] += sq4[u][h].w * on;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    rinv[h][i] = norm ? 1.0f / sqrtf(group_sum<16>(v[i]) / hn + eps) : 1.0f;
            }
        }
        uint32_t dg[RG][KS / 8][4];   // [group][lane group q][dword]: halves = scales of blocks 8q ..
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const uint32_t dw[4] = {dq[g].x, dq[g].y, dq[g].z, dq[g].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint32_t t[4];
                gbm_allgather4(dw[k], t);
#pragma unroll
                for (int q = 0; q < KS / 8; ++q)
                    dg[g][q][k] = t[q];
            }
        }
        float cacc[NG][RG][4];
#pragma unroll
        for (int h = 0; h < NG; ++h)
#pragma unroll
            for (int g = 0; g < RG; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    cacc[h][g][i] = 0.f;
        const int sbase = (st - s0) * STEPS;
        // x of block bl of the stage; each block's pair is read one block ahead
        auto read_x = [&](gbm_half8 (&xh)[NG], gbm_half8 (&xl)[NG], int bl) {
#pragma unroll
            for (int h = 0; h < NG; ++h) {
                const _Float16* src = xs + ((size_t)(bl * 4 + kg) * 2 * S + 16 * h + r) * 8;
                xh[h] = *reinterpret_cast<const gbm_half8*>(src);
                xl[h] = *reinterpret_cast<const gbm_half8*>(src + S * 8);
            }
        };
        gbm_half8 nxh[NG], nxl[NG];
        read_x(nxh, nxl, 0);
#pragma unroll
        for (int j = 0; j < STEPS; ++j) {
            uint32_t w[RG][4];
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                w[g][0] = bufs[j].q[g].x;
                w[g][1] = bufs[j].q[g].y;
                w[g][2] = bufs[j].q[g].z;
                w[g][3] = bufs[j].q[g].w;
                gbm_transpose4(w[g]);
            }
            load(bufs[j], sbase + STEPS + j);   // the same step of the next stage
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int bl = 4 * j + b;   // block within the stage
                gbm_half8 xh[NG], xl[NG];
#pragma unroll
                for (int h = 0; h < NG; ++h) {
                    xh[h] = nxh[h];
                    xl[h] = nxl[h];
                }
                if (bl + 1 < KS)   // compile-time
                    read_x(nxh, nxl, bl + 1);
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    const gbm_half8 wop = gbm_codes(w[g][b]);
                    const uint32_t dd = dg[g][bl >> 3][(bl & 7) >> 1];
                    const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)((bl & 1) ? dd >> 16 : dd));
#pragma unroll
                    for (int h = 0; h < NG; ++h) {
                        gbm_floatx4 pv = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[h], wop, zero, 0, 0, 0);
                        pv = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[h], wop, pv, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            cacc[h][g][i] = fmaf((float)dh, pv[i], cacc[h][g][i]);
                    }
                }
                // the block's sums are made here: its products die at once
#pragma unroll
                for (int h = 0; h < NG; ++h)
#pragma unroll
                    for (int g = 0; g < RG; ++g)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            asm volatile("" : "+v"(cacc[h][g][i]));
            }
        }
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            const float ci[4] = {inv[h].x, inv[h].y, inv[h].z, inv[h].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int g = 0; g < RG; ++g)
                    acc[h][g][i] = fmaf(cacc[h][g][i], ci[i], acc[h][g][i]);
        }
        if (st + 1 < s1) {   // uniform
            __syncthreads();   // every wave is done with this stage's x
            dma_x(st + 1);
            load_d(dq, st + 1);
            load_inv(inv, st + 1);
        }
        asm volatile("" ::: "memory");   // keeps the next stage's loads where they are issued
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int row = row0 + 16 * g + r;
        if (row < N) {
#pragma unroll
            for (int h = 0; h < NG; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * h + 4 * kg + i < B)
                        Y[(size_t)(16 * h + 4 * kg + i) * N + row] = acc[h][g][i] * rinv[h][i];
        }
    }
}

}  // namespace qd
