// prefill_gemm.h -- the q4_0 matrix product of a prefill chunk on the matrix
// cores (gfx950): Y[t] = W x[t] for the T <= 16 positions of a chunk, every
// weight read once per chunk (inferencelayer cuda_llm.rs page: prefill as the
// many-token form of the step, its q4 GEMV arm at M > 1).
//
// v_mfma_f32_16x16x32_f16 with the roles of the batched GEMV swapped: the A
// operand (M = 16) is the chunk's positions, the B operand (N = 16) sixteen
// weight rows, and K = 32 one q4_0 block.  With K inside one block the scale
// is one per lane (the lane's weight row) and is applied after the product:
//   part = x_hi . c + x_lo . c   (c = code - 8 exact in f16; every product
//                                 exact in f32, summed in f32)
//   acc  = fma(part, d, acc)
// The activations arrive already split (XP below) in the A-operand order, so
// a lane reads its 8 + 8 halves of a block with two 16-byte loads straight
// from memory.
//
// XP layout: [16 positions][nb blocks][hi, lo][4 lane groups][8 halves];
// lane group g of block j holds the elements of word g of the q4_0 block
// (low nibbles 4g..4g+3, high nibbles 16+4g..16+4g+3) in the order xp_pos
// gives.  hi = RN_f16(x s), lo = RN_f16(x s - hi), with s = 2^k a power of two
// per position chosen from the position's largest |x| so that |x s| lies in
// [2^13, 2^14): hi never overflows f16 and the pair keeps about 22
// significant bits at any input scale.  1/s (XS[t]) multiplies the position's
// sums in f32, exactly.  A position's hi halves of a block are 64 contiguous
// bytes, as are its lo halves.
//
// Weights are read coalesced: lane (r, g) loads block b0 + g of row r whole
// (16 bytes; four lanes read 64 contiguous bytes of a row) and its scale,
// and a per-wave LDS transpose hands lane (r, g) word g of each of the four
// blocks.
#pragma once

#include "qd_common.h"

namespace qd {

typedef _Float16 pg_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 pg_half2 __attribute__((ext_vector_type(2)));
typedef float pg_floatx4 __attribute__((ext_vector_type(4)));

constexpr int PG_T = 16;   // positions per chunk (the MFMA's M)

// Position (0..7) within its lane group of element e (0..31) of a block:
// word (e & 15) >> 2; low-nibble elements first; within each half the order
// (0, 2, 1, 3) of the word's bytes, which is how pg_codes unpacks them.
QD_DEV int xp_pos(int e) { return ((e >> 4) << 2) | ((e & 1) << 1) | ((e >> 1) & 1); }
QD_DEV size_t xp_index(int t, int k, int nb)   // half index of hi; lo is +32
{
    const int j = k >> 5, e = k & 31;
    return ((size_t)t * nb + j) * 64 + ((e & 15) >> 2) * 8 + xp_pos(e);
}
// s = 2^k with a * s in [2^13, 2^14) for the largest magnitude a of a
// vector (k clamped to [-100, 100]; 1 when a is 0 or not finite)
QD_DEV float xp_scale_for(float a)
{
    if (!(a > 0.f) || !(a <= 3.4e38f))
        return 1.f;
    int e;
    (void)frexpf(a, &e);   // a in [2^(e-1), 2^e)
    return ldexpf(1.f, max(-100, min(100, 14 - e)));
}

QD_DEV void xp_store(_Float16* XP, int t, int k, int nb, float x)
{
    const _Float16 h = (_Float16)x;
    const size_t i = xp_index(t, k, nb);
    XP[i] = h;
    XP[i + 32] = (_Float16)(x - (float)h);
}

// the 8 codes of one word as code - 8 in f16, in xp_pos order:
// (w & 0x000F000F) | 0x64006400 holds two codes as 1024 + code
QD_DEV pg_half8 pg_codes(uint32_t w)
{
    const uint32_t m = 0x000F000Fu, bias = 0x64006400u;
    const uint32_t t[4] = {(w & m) | bias, ((w >> 8) & m) | bias, ((w >> 4) & m) | bias,
                           ((w >> 12) & m) | bias};
    const pg_half2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    pg_half8 c;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const pg_half2 v = __builtin_bit_cast(pg_half2, t[k]) + off;
        c[2 * k] = v[0];
        c[2 * k + 1] = v[1];
    }
    return c;
}

enum PgMode { PG_STORE = 0, PG_RESID = 1, PG_SWIGLU = 2 };

// largest |value| over a workgroup (every thread gets it); red >= 16 floats
QD_DEV float pg_block_max(float v, float* red)
{
    v = group_max<WAVE>(v);
    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    __syncthreads();
    if (lane == 0)
        red[wv] = v;
    __syncthreads();
    float m = 0.f;
    for (int i = 0; i < (int)(blockDim.x / WAVE); ++i)
        m = fmaxf(m, red[i]);
    return m;
}

// One workgroup of NW waves owns 16*R weight rows; wave w takes the 4-block
// steps w, w + NW, ... of every row (the next step's loads issued before the
// current one is computed), and the NW partial sums are added in wave order
// through LDS.  Epilogue (T positions written):
// (sum = the product of position t's split input, times XS[t]):
//   PG_STORE : Y[t][row] = sum
//   PG_RESID : Y[t][row] += sum                     (residual add)
//   PG_SWIGLU: rows 2i, 2i+1 are gate and up of unit i; silu(gate) * up is
//              written to Y[t][i] (Y is [T][N/2]), split by k_pf_xsplit
template <int R, int NW, int MODE>
__global__ void __launch_bounds__(NW* WAVE)
k_pf_gemm(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q, const _Float16* __restrict__ XP,
          const float* __restrict__ XS, int N, int nb, int T, float* __restrict__ Y)
{
    constexpr int CB = 4;   // blocks per step
    __shared__ uint4 wl[NW][R][16][CB + 1];   // codes [row][block], one pad per row
    __shared__ __align__(8) uint16_t sl[NW][R][16][CB];
    __shared__ pg_floatx4 red[NW][R][WAVE];
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    const int r = lane & 15, g = lane >> 4;
    const int row0 = blockIdx.x * 16 * R;
    const int nstep = (nb + CB - 1) / CB;
    uint32_t rbase[R];
#pragma unroll
    for (int s = 0; s < R; ++s)
        rbase[s] = (uint32_t)min(row0 + 16 * s + r, N - 1) * (uint32_t)nb;
    const _Float16* xl = XP + (size_t)r * nb * 64 + g * 8;   // position r, lane group g

    struct Ld {
        uint4 q[R];
        uint16_t d[R];
        pg_half8 xh[CB], xo[CB];
    };
    // loads of step st (clamped: never a branch around a load)
    // every workgroup starts its walk over K at its own step, so that the
    // workgroups do not all read the same activations at the same moment
    const int rot = (int)((blockIdx.x * 5u) % (unsigned)nstep);
    auto phys = [&](int st) { return st + rot < nstep ? st + rot : st + rot - nstep; };
    auto load = [&](Ld& L, int st) {
        const int b0 = phys(min(st, nstep - 1)) * CB;
        const int bq = min(b0 + g, nb - 1);
#pragma unroll
        for (int s = 0; s < R; ++s) {
            // weights stream through once per chunk: non-temporal, so that
            // they do not push the chunk's activations out of L2
            typedef unsigned int pg_u32x4 __attribute__((ext_vector_type(4)));
            const pg_u32x4 qv =
                __builtin_nontemporal_load(reinterpret_cast<const pg_u32x4*>(Q + ((size_t)rbase[s] + bq) * 16));
            L.q[s] = make_uint4(qv.x, qv.y, qv.z, qv.w);
            L.d[s] = D[rbase[s] + bq];
        }
#pragma unroll
        for (int m = 0; m < CB; ++m) {
            const pg_half8* xp = reinterpret_cast<const pg_half8*>(xl + (size_t)min(b0 + m, nb - 1) * 64);
            L.xh[m] = xp[0];
            L.xo[m] = xp[4];
        }
    };
    pg_floatx4 acc[R];
#pragma unroll
    for (int s = 0; s < R; ++s)
        acc[s] = pg_floatx4{0.f, 0.f, 0.f, 0.f};
    // one step: transpose the codes and scales through this wave's LDS (its
    // DS operations run in order), then 2 MFMAs and 4 scaled adds per block
    auto compute = [&](const Ld& L, int st) {
        const int b0 = phys(st) * CB;
#pragma unroll
        for (int s = 0; s < R; ++s) {
            wl[wave][s][r][g] = L.q[s];
            sl[wave][s][r][g] = L.d[s];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int s = 0; s < R; ++s) {
            const uint2 sc2 = *reinterpret_cast<const uint2*>(&sl[wave][s][r][0]);
            const uint16_t scs[4] = {(uint16_t)(sc2.x & 0xffff), (uint16_t)(sc2.x >> 16),
                                     (uint16_t)(sc2.y & 0xffff), (uint16_t)(sc2.y >> 16)};
#pragma unroll
            for (int m = 0; m < CB; ++m) {
                const uint32_t w = reinterpret_cast<const uint32_t*>(&wl[wave][s][r][m])[g];
                const pg_half8 c = pg_codes(w);
                pg_floatx4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(L.xh[m], c,
                                                                      pg_floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                p = __builtin_amdgcn_mfma_f32_16x16x32_f16(L.xo[m], c, p, 0, 0, 0);
                const float sc = b0 + m < nb ? f16_to_f32(scs[m]) : 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[s][i] = fmaf(p[i], sc, acc[s][i]);
            }
        }
        __builtin_amdgcn_wave_barrier();
    };
    // two register buffers in turn (no copy between them, so no wait on the
    // loads just issued)
    Ld b0, b1;
    load(b0, wave);
    for (int st = wave; st < nstep; st += 2 * NW) {   // uniform per wave
        load(b1, st + NW);
        compute(b0, st);
        if (st + NW < nstep) {   // uniform per wave
            load(b0, st + 2 * NW);
            compute(b1, st + NW);
        }
    }
#pragma unroll
    for (int s = 0; s < R; ++s)
        red[wave][s][lane] = acc[s];
    __syncthreads();
    // wave s of the first R waves finishes slice s (R <= NW)
    if (wave < R) {
        const int s = wave;
        pg_floatx4 v = red[0][s][lane];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) {
            const pg_floatx4 o = red[w2][s][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] += o[i];
        }
        // v[i]: position 4g + i, row row0 + 16 s + r; undo the input scale
        const int row = row0 + 16 * s + r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] *= XS[min(4 * g + i, T - 1)];
        if (MODE == PG_SWIGLU) {
            const int K2 = N >> 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float up = __shfl_xor(v[i], 1, WAVE);
                const int t = 4 * g + i;
                if (!(r & 1) && row < N && t < T) {
                    const float gt = v[i];
                    Y[(size_t)t * K2 + (row >> 1)] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
                }
            }
        } else if (row < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * g + i;
                if (t < T) {
                    float* y = Y + (size_t)t * N + row;
                    *y = MODE == PG_RESID ? *y + v[i] : v[i];
                }
            }
        }
    }
}

// X [T][K] f32 -> XP (split, A-operand order) and XS[t] = 1/s; grid T, 1024
// threads.  With a gate (row t at gate + t * gstride), x is multiplied by
// sigmoid(gate) first, as the decode step gates the merged attention output.
__global__ void __launch_bounds__(1024)
k_pf_xsplit(const float* __restrict__ X, int K, const float* __restrict__ gate, int gstride,
            _Float16* __restrict__ XP, float* __restrict__ XS)
{
    __shared__ float red[16];
    const int t = blockIdx.x;
    auto val = [&](int k) {
        float x = X[(size_t)t * K + k];
        if (gate)   // uniform
            x *= 1.0f / (1.0f + expf(-gate[(size_t)t * gstride + k]));
        return x;
    };
    float a = 0.f;
    for (int k = threadIdx.x; k < K; k += blockDim.x)
        a = fmaxf(a, fabsf(val(k)));
    const float sc = xp_scale_for(pg_block_max(a, red));
    for (int k = threadIdx.x; k < K; k += blockDim.x)
        xp_store(XP, t, k, K >> 5, val(k) * sc);
    if (threadIdx.x == 0)
        XS[t] = 1.0f / sc;
}

// RMSNorm of X[t] (weight w) written split into XP, XS[t] = 1/s; grid T,
// 1024 threads, H a multiple of 32 (each thread 4 consecutive elements per
// round)
__global__ void __launch_bounds__(1024)
k_pf_rmsnorm_xp(const float* __restrict__ X, const float* __restrict__ w, int H, float eps,
                _Float16* __restrict__ XP, float* __restrict__ XS)
{
    __shared__ float red[16];
    const int t = blockIdx.x;
    const float4* x4 = reinterpret_cast<const float4*>(X + (size_t)t * H);
    const float4* w4 = reinterpret_cast<const float4*>(w);
    const int n4 = H >> 2;
    float ss = 0.f, a = 0.f;
    for (int i = threadIdx.x; i < n4; i += blockDim.x) {
        const float4 v = x4[i], g = w4[i];
        ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
        a = fmaxf(fmaxf(a, fmaxf(fabsf(v.x * g.x), fabsf(v.y * g.y))), fmaxf(fabsf(v.z * g.z), fabsf(v.w * g.w)));
    }
    ss = group_sum<WAVE>(ss);
    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    if (lane == 0)
        red[wv] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < (int)(blockDim.x / WAVE); ++i)   // fixed order
        tot += red[i];
    const float rs = 1.0f / sqrtf(tot / (float)H + eps);
    // largest |x w rs| up to rounding: the scale only has to keep it below 2^15
    const float sc = xp_scale_for(pg_block_max(a, red) * rs);
    const float f = rs * sc;
    for (int i = threadIdx.x; i < n4; i += blockDim.x) {
        const float4 v = x4[i], g = w4[i];
        xp_store(XP, t, 4 * i, H >> 5, v.x * f * g.x);
        xp_store(XP, t, 4 * i + 1, H >> 5, v.y * f * g.y);
        xp_store(XP, t, 4 * i + 2, H >> 5, v.z * f * g.z);
        xp_store(XP, t, 4 * i + 3, H >> 5, v.w * f * g.w);
    }
    if (threadIdx.x == 0)
        XS[t] = 1.0f / sc;
}

}  // namespace qd
