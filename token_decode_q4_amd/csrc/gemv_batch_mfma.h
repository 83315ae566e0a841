// gemv_batch_mfma.h -- batched q4_0 GEMV on the matrix cores (gfx950):
// Y[b] = W X[b] for 2 <= B <= 8 vectors, every weight read once.
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
// at most 15 significant bits).  x enters as an f16 pair too (hi = RN(x),
// lo = RN(x - hi), about 22 bits), and the four products hi*hi, hi*lo, lo*hi,
// lo*lo accumulate in f32: every product is exact in f32.
//
// Codes to f16: (w & 0x000F000F) | 0x64006400 holds two codes as the f16
// values 1024 + code; a packed f16 add of -1032 leaves code - 8, exactly.
//
// x is staged per chunk of 32 blocks in LDS, already in the B-operand
// layout: [block][word][vector][8 hi, 8 lo] halves.  The weight loads of the
// next chunk are issued before the current one is computed (two register
// buffers, the chunk loop unrolled by two).
#pragma once

#include "qd_common.h"

namespace qd {

typedef _Float16 gbm_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 gbm_half2 __attribute__((ext_vector_type(2)));
typedef float gbm_floatx4 __attribute__((ext_vector_type(4)));

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

template <int NC>
struct GbmBuf {
    uint4 q[GBM_KC / 4];       // block 4j + kg of this lane's row, j = 0..7
    uint32_t d[GBM_KC / 4];    // its f16 scale
};

template <int NC>
__global__ void __launch_bounds__(GBM_NW* WAVE)
k_gemv_batch_mfma(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
                  const float* __restrict__ X, float* __restrict__ Y, int N, int nb)
{
    static_assert(NC >= 2 && NC <= 8, "batch");
    extern __shared__ __align__(16) _Float16 xs[];   // [KC][4][NC][16]
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r = lane & 15, kg = lane >> 4;
    const int col = min(lane & 15, NC - 1);          // columns past NC repeat the last vector
    const int K = nb * 32;
    const int nch = (nb + GBM_KC - 1) / GBM_KC;
    const int ntiles = (N + GBM_ROWS - 1) / GBM_ROWS;

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {   // uniform per workgroup
        const int row0 = tile * GBM_ROWS + wave * 16;
        const uint32_t rb = (uint32_t)min(row0 + r, N - 1) * (uint32_t)nb;

        // weight loads of chunk c (clamped: never a branch around a load)
        auto load = [&](GbmBuf<NC>& bf, int c) {
#pragma unroll
            for (int j = 0; j < GBM_KC / 4; ++j) {
                const uint32_t blk = rb + (uint32_t)min(c * GBM_KC + 4 * j + kg, nb - 1);
                bf.q[j] = *reinterpret_cast<const uint4*>(Q + blk * 16u);
                bf.d[j] = D[blk];
            }
        };
        // stage x of chunk c: item i = (block, word, vector), 8 values each
        auto stage = [&](int c) {
            __syncthreads();   // the previous chunk's reads are done
            for (int i = threadIdx.x; i < GBM_KC * 4 * NC; i += GBM_NW * WAVE) {
                const int v = i % NC, w = (i / NC) & 3, bl = i / (4 * NC);
                const int b = c * GBM_KC + bl;
                float e[8];
                if (b < nb) {
                    const float* xp = X + (size_t)v * K + (size_t)b * 32 + 4 * w;
                    const float4 a = *reinterpret_cast<const float4*>(xp);
                    const float4 h = *reinterpret_cast<const float4*>(xp + 16);
                    e[0] = a.x; e[1] = a.z; e[2] = a.y; e[3] = a.w;
                    e[4] = h.x; e[5] = h.z; e[6] = h.y; e[7] = h.w;
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        e[k] = 0.f;
                }
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
            __syncthreads();
        };
        gbm_floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        auto compute = [&](const GbmBuf<NC>& bf) {
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
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bhi, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, blo, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bhi, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, blo, acc, 0, 0, 0);
                }
            }
        };
        GbmBuf<NC> b0, b1;
        load(b0, 0);
        for (int c = 0; c < nch; c += 2) {
            load(b1, min(c + 1, nch - 1));
            stage(c);
            compute(b0);
            if (c + 1 < nch) {   // uniform
                load(b0, min(c + 2, nch - 1));
                stage(c + 1);
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
