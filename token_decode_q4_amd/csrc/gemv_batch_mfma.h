// gemv_batch_mfma.h -- batched q4_0 GEMV on the matrix cores (gfx950):
// Y[b] = W X[b] for 2 <= B <= 16 vectors, every weight read once.
//
// The batched decode of the inferencelayer cuda_llm.rs page (its q4 GEMV arm
// against the bf16 GEMM arm at M = 1 .. 16 tokens, section on the batched
// head-to-head).  With B vectors the GEMV is a skinny matrix product, so it
// runs on v_mfma_f32_16x16x32_f16: M = 16 weight rows, N = 16 columns (the B
// vectors, the rest discarded), K = 32.
//
// Layout.  A workgroup of 4 waves owns a 64-row tile, a wave one 16-row
// slice of it.  Lane l = (r, kg), r = l % 16, kg = l / 16, loads block
// 4j + kg of row r whole (16 bytes; 4 lanes read 64 contiguous bytes of a
// row).  MFMA w (w = 0..3) of group j takes from every lane its block's word
// w: the 8 codes there (low nibbles: elements 4w..4w+3, high nibbles:
// 16+4w..16+4w+3), so one MFMA spans the four blocks 4j..4j+3, one per lane
// group.  Because the blocks differ in scale, the scale is part of the A
// operand: (code - 8) * d as an f16 pair hi + lo with hi = RN((code-8)*d)
// and lo = (code-8)*d - hi, both exact in f16 for |d| < 8192 ((code-8)*d has
// at most 15 significant bits).  x enters as an f16 pair too, after a power
// of two s per (vector, chunk of 32 blocks) that puts the chunk's largest
// |x| in [2^13, 2^14): hi = RN(x s), lo = RN(x s - hi), about 22 bits at any
// input scale and no f16 overflow.  The four products hi*hi, hi*lo, lo*hi,
// lo*lo accumulate in f32 (every product exact); each chunk's sum is
// multiplied by 1/s, exactly, into the result.
//
// Codes to f16: (w & 0x000F000F) | 0x64006400 holds two codes as the f16
// values 1024 + code; a packed f16 add of -1032 leaves code - 8, exactly.
//
// x is staged per chunk of 32 blocks in LDS, already in the B-operand
// layout: [block][word][vector][8 hi, 8 lo] halves.  The weight loads (two
// register buffers, the chunk loop unrolled by two) and the x loads (one
// buffer, refilled as soon as it is staged) of the next chunk are issued
// before the current one is computed, so staging a chunk is conversions and
// LDS writes only.
#pragma once

#include "qd_common.h"

namespace qd {

typedef _Float16 gbm_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 gbm_half2 __attribute__((ext_vector_type(2)));
typedef float gbm_floatx4 __attribute__((ext_vector_type(4)));

constexpr int GBM_MAXB = 16;   // vectors per launch
constexpr int GBM_KC = 32;     // blocks per staged chunk
constexpr int GBM_NW = 4;      // waves per workgroup
constexpr int GBM_ROWS = 64;   // rows per workgroup tile

// LDS bytes of one staged chunk of B vectors
__host__ __device__ constexpr size_t gemv_batch_mfma_lds_bytes(int B)
{
    return (size_t)GBM_KC * 4 * B * 16 * sizeof(_Float16);
}

// Element (within its block) of position e (0..7) of word w in both operands:
// e -> 16*(e/4) + 4w + (0, 2, 1, 3)[e%4]
QD_DEV int gbm_elem(int w, int e) { return 16 * (e >> 2) + 4 * w + ((e & 1) << 1) + ((e >> 1) & 1); }

// (code - 8) * d of word w as the f16 pair (hi, lo), in gbm_elem order
QD_DEV void gbm_a_operand(uint32_t w, gbm_half2 d2, gbm_half8& hi, gbm_half8& lo)
{
    const uint32_t m = 0x000F000Fu, bias = 0x64006400u;
    const uint32_t t[4] = {(w & m) | bias, ((w >> 8) & m) | bias, ((w >> 4) & m) | bias,
                           ((w >> 12) & m) | bias};
    const gbm_half2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const gbm_half2 c = __builtin_bit_cast(gbm_half2, t[k]) + off;   // code - 8, exact
        const gbm_half2 h = c * d2;
        const gbm_half2 l = __builtin_elementwise_fma(c, d2, -h);        // exact remainder
        hi[2 * k] = h[0];
        hi[2 * k + 1] = h[1];
        lo[2 * k] = l[0];
        lo[2 * k + 1] = l[1];
    }
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

// staging items (block, word, vector) per thread per chunk
template <int NC>
struct GbmItems {
    static constexpr int N = (GBM_KC * 4 * NC + GBM_NW * WAVE - 1) / (GBM_NW * WAVE);
};

struct GbmBuf {
    uint4 q[GBM_KC / 4];               // block 4j + kg of this lane's row, j = 0..7
    uint32_t d[GBM_KC / 4];            // its f16 scale
};
template <int NC>
struct GbmX {
    float4 xa[GbmItems<NC>::N];        // x of this thread's staging items: elements 4w .. 4w+3
    float4 xb[GbmItems<NC>::N];        //   and 16+4w .. 16+4w+3
};

// grid (row tiles, K slices): slice y takes chunks [y * kch, (y + 1) * kch)
// and writes its partial products to Y + y * ystride (one slice: Y itself)
template <int NC>
__global__ void __launch_bounds__(GBM_NW* WAVE)
k_gemv_batch_mfma(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
                  const float* __restrict__ X, float* __restrict__ Y, int N, int nb, int kch, size_t ystride)
{
    static_assert(NC >= 2 && NC <= 16, "batch");
    constexpr int NITEM = GBM_KC * 4 * NC;   // staging items of a chunk
    extern __shared__ __align__(16) _Float16 xs[];   // [KC][4][NC][16]
    __shared__ unsigned xmax[2][GBM_MAXB];            // |x| maxima (f32 bits), by chunk parity
    __shared__ float xinv[GBM_MAXB];                  // 1/s of the staged chunk, per vector
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r = lane & 15, kg = lane >> 4;
    const int col = min(lane & 15, NC - 1);          // columns past NC repeat the last vector
    const int K = nb * 32;
    const int nch = (nb + GBM_KC - 1) / GBM_KC;
    const int c0 = (int)blockIdx.y * kch, c1 = min(nch, c0 + kch);   // this slice's chunks
    Y += (size_t)blockIdx.y * ystride;
    const int ntiles = (N + GBM_ROWS - 1) / GBM_ROWS;
    if (threadIdx.x < 2 * GBM_MAXB)
        xmax[threadIdx.x / GBM_MAXB][threadIdx.x % GBM_MAXB] = 0u;   // ordered by the first stage's barrier
    int gc = 0;   // chunks staged so far by this workgroup (parity of xmax)

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {   // uniform per workgroup
        const int row0 = tile * GBM_ROWS + wave * 16;
        const uint32_t rb = (uint32_t)min(row0 + r, N - 1) * (uint32_t)nb;

        // weight and x loads of chunk c (clamped: never a branch around a
        // load; x of a block past nb is zeroed where it is staged).  Staging
        // item i = (block, word, vector) takes 8 values of x.
        auto load = [&](GbmBuf& bf, int c) {
#pragma unroll
            for (int j = 0; j < GBM_KC / 4; ++j) {
                const uint32_t blk = rb + (uint32_t)min(c * GBM_KC + 4 * j + kg, nb - 1);
                bf.q[j] = *reinterpret_cast<const uint4*>(Q + blk * 16u);
                bf.d[j] = D[blk];
            }
        };
        auto load_x = [&](GbmX<NC>& bf, int c) {
#pragma unroll
            for (int u = 0; u < GbmItems<NC>::N; ++u) {
                const int i = min((int)threadIdx.x + u * GBM_NW * WAVE, NITEM - 1);
                const int v = i % NC, w = (i / NC) & 3, bl = i / (4 * NC);
                const int b = min(c * GBM_KC + bl, nb - 1);
                const float* xp = X + (size_t)v * K + (size_t)b * 32 + 4 * w;
                bf.xa[u] = *reinterpret_cast<const float4*>(xp);
                bf.xb[u] = *reinterpret_cast<const float4*>(xp + 16);
            }
        };
        // stage x of chunk c from the registers of its loads: the chunk's
        // largest |x| per vector (LDS atomic max of the f32 bits, which order
        // like the values for |x|), then the scaled split
        auto stage = [&](const GbmX<NC>& bf, int c) {
            unsigned* xm = xmax[gc & 1];
            __syncthreads();   // the previous chunk's reads (x, 1/s) are done
#pragma unroll
            for (int u = 0; u < GbmItems<NC>::N; ++u) {
                const int i = (int)threadIdx.x + u * GBM_NW * WAVE;
                if (i >= NITEM)   // uniform except in the last round of an odd batch
                    continue;
                const bool in = c * GBM_KC + i / (4 * NC) < nb;
                const float4 a = bf.xa[u], h = bf.xb[u];
                const float mx = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                                       fmaxf(fmaxf(fabsf(h.x), fabsf(h.y)), fmaxf(fabsf(h.z), fabsf(h.w))));
                if (in)
                    atomicMax(&xm[i % NC], __float_as_uint(mx));
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < GbmItems<NC>::N; ++u) {
                const int i = (int)threadIdx.x + u * GBM_NW * WAVE;
                if (i >= NITEM)
                    continue;
                const int bl = i / (4 * NC);
                const bool in = c * GBM_KC + bl < nb;
                const float sc = gbm_scale_for(__uint_as_float(xm[i % NC]));
                const float4 a = bf.xa[u], h = bf.xb[u];
                float e[8] = {a.x, a.z, a.y, a.w, h.x, h.z, h.y, h.w};
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    e[k] = in ? e[k] * sc : 0.f;
                gbm_half8 xh, xl;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const _Float16 t = (_Float16)e[k];
                    xh[k] = t;
                    xl[k] = (_Float16)(e[k] - (float)t);
                }
                gbm_half8* dst = reinterpret_cast<gbm_half8*>(xs + (size_t)i * 16);
                dst[0] = xh;
                dst[1] = xl;
            }
            if (threadIdx.x < NC) {
                xinv[threadIdx.x] = 1.0f / gbm_scale_for(__uint_as_float(xm[threadIdx.x]));
                // the other parity was last read before this stage's first barrier
                // and is next written after the following stage's first barrier
                xmax[(gc + 1) & 1][threadIdx.x] = 0u;
            }
            ++gc;
            __syncthreads();
        };
        gbm_floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        auto compute = [&](const GbmBuf& bf) {
            gbm_floatx4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < GBM_KC / 4; ++j) {
                const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)bf.d[j]);
                const gbm_half2 d2 = {dh, dh};
                const uint32_t wd[4] = {bf.q[j].x, bf.q[j].y, bf.q[j].z, bf.q[j].w};
                const int bl = 4 * j + kg;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    gbm_half8 ahi, alo;
                    gbm_a_operand(wd[w], d2, ahi, alo);
                    const gbm_half8* src =
                        reinterpret_cast<const gbm_half8*>(xs + ((size_t)(bl * 4 + w) * NC + col) * 16);
                    const gbm_half8 bhi = src[0], blo = src[1];
                    part = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bhi, part, 0, 0, 0);
                    part = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, blo, part, 0, 0, 0);
                    part = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bhi, part, 0, 0, 0);
                    part = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, blo, part, 0, 0, 0);
                }
            }
            const float inv = xinv[col];   // column col = this lane's vector
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = fmaf(part[i], inv, acc[i]);
        };
        GbmBuf b0, b1;
        GbmX<NC> xr;
        load(b0, c0);
        load_x(xr, c0);
        for (int c = c0; c < c1; c += 2) {
            stage(xr, c);
            load(b1, min(c + 1, c1 - 1));
            load_x(xr, min(c + 1, c1 - 1));
            compute(b0);
            if (c + 1 < c1) {   // uniform
                stage(xr, c + 1);
                load(b0, min(c + 2, c1 - 1));
                load_x(xr, min(c + 2, c1 - 1));
                compute(b1);
            }
        }
        // acc[i] = row 4*kg + i of the slice, vector lane % 16
        if ((lane & 15) < NC) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = row0 + 4 * kg + i;
                if (row < N)
                    Y[(size_t)(lane & 15) * N + row] = acc[i];
            }
        }
    }
}

}  // namespace qd
