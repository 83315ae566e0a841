// step_kernels.h -- the kernels of one batch-1 decode step (gfx950).
//
// Step order (inferencelayer cuda_llm.rs page, CudaQwen3::step;
// ferrum-kernels cuda_decode.rs page, CudaDecodeRunner::decode_step with its
// fused add + RMSNorm chaining across layers):
//   k_embed                       x = E[token]; u = x * w_attn(0); ss = sum x^2
//   per layer:
//     k_gemv_qkv                  [q;k;v] = Wqkv u / rms; per-head q/k RMSNorm,
//                                 rotary, K/V written at pos (last workgroup of a head)
//     k_attn_decode               split-KV GQA attention + combine
//     k_gemv_residual (o)         x += Wo attn; u = x * w_ffn; ss partials
//     k_gemv_swiglu (gate|up)     a = silu(Wg u / rms) * (Wu u / rms)
//     k_gemv_residual (down)      x += Wd a; u = x * w_next; ss partials
//   k_gemv_lmhead                 logits = Wlm u / rms; argmax; advance position
//
// RMSNorm is split between producer and consumer: the kernel that writes x
// also writes u = x * w (elementwise, w = the next norm's weight) and per-
// workgroup partial sums of x^2; the consuming GEMV scales its dot products by
// 1/sqrt(mean(x^2) + eps), since W (x * w * r) = r * (W (x * w)) for the scalar r.
#pragma once

#include "gemv_q4_0.h"
#include "attn_decode.h"

namespace qd {

// device-resident step state
struct StepState {
    int32_t pos;       // position of the next step
    int32_t n_forced;  // positions < n_forced keep their stored token
    int32_t error;     // bit 0: token out of range, bit 1: position out of range
    int32_t pad;
};

QD_DEV float block_sum256(float v, float* red /* >= 4 floats */)
{
    v = group_sum<WAVE>(v);
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    __syncthreads();
    if (lane == 0)
        red[wave] = v;
    __syncthreads();
    const int nw = blockDim.x / WAVE;
    float s = 0.f;
    for (int i = 0; i < nw; ++i)
        s += red[i];
    return s;
}

// ----------------------------------------------------------------- embedding

__global__ void __launch_bounds__(256)
k_embed(const uint16_t* __restrict__ Ed, const uint8_t* __restrict__ Eq, int H, int vocab,
        StepState* __restrict__ st, const int32_t* __restrict__ ids, int max_seq,
        const float* __restrict__ w_norm, float* __restrict__ x, float* __restrict__ u,
        float* __restrict__ ss_part)
{
    __shared__ float red[8];
    int pos = st->pos;
    int tok = 0;
    if (pos < 0 || pos >= max_seq) {
        if (threadIdx.x == 0) st->error |= 2;
        pos = 0;
    }
    tok = ids[pos];
    if (tok < 0 || tok >= vocab) {
        if (threadIdx.x == 0) st->error |= 1;
        tok = 0;
    }
    const int nb = H / 32;
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += blockDim.x) {
        const int bk = i >> 5, j = i & 31;
        const size_t blk = (size_t)tok * nb + bk;
        const uint8_t byte = Eq[blk * 16 + (j & 15)];
        const int code = (j < 16) ? (byte & 15) : (byte >> 4);
        const float v = (float)(code - 8) * f16_to_f32(Ed[blk]);
        x[i] = v;
        u[i] = v * w_norm[i];
        ss = fmaf(v, v, ss);
    }
    ss = block_sum256(ss, red);
    if (threadIdx.x == 0)
        ss_part[0] = ss;
}

// ----------------------------------------------------------------- fused QKV

struct QkvEpi {
    float* raw;                 // [rows] f32: q | k | v before norm/rotary
    float* q_out;               // [nq*hd]
    int nq, nkv, hd, rot, qk_norm;
    float eps;
    const float* q_norm;        // [hd]
    const float* k_norm;        // [hd]
    const float* rope_cos;      // [max_seq][rot/2]
    const float* rope_sin;
    const StepState* st;
    int max_seq;
    uint16_t* kc;               // this layer's K cache
    uint16_t* vc;
    int paged;
    const int32_t* table;       // paged: logical -> physical block
    unsigned int* counters;     // [nq + 2*nkv]
};

// Per-head finish: q/k RMSNorm over head_dim, NeoX rotary on the first rot
// dims (pairs i, i + rot/2), q to q_out, K/V to the cache at pos as f16.
QD_DEV void qkv_head_finish(const QkvEpi& e, int hh, float* sv, float* red)
{
    const int t = threadIdx.x;
    const int hd = e.hd;
    const float val = (t < hd) ? e.raw[(size_t)hh * hd + t] : 0.f;
    const bool is_q = hh < e.nq, is_k = !is_q && hh < e.nq + e.nkv;
    float v = val;
    if ((is_q || is_k) && e.qk_norm) {
        const float ss = block_sum256(val * val, red);
        const float inv = 1.0f / sqrtf(ss / (float)hd + e.eps);
        if (t < hd)
            v = val * inv * (is_q ? e.q_norm[t] : e.k_norm[t]);
    }
    int pos = e.st->pos;
    pos = (pos < 0) ? 0 : (pos >= e.max_seq ? e.max_seq - 1 : pos);
    if (is_q || is_k) {
        if (t < hd)
            sv[t] = v;
        __syncthreads();
        const int half = e.rot / 2;
        if (t < e.rot) {
            const int i = (t < half) ? t : t - half;
            const float c = e.rope_cos[(size_t)pos * half + i];
            const float s = e.rope_sin[(size_t)pos * half + i];
            if (t < half)
                v = sv[t] * c - sv[t + half] * s;
            else
                v = sv[t - half] * s + sv[t] * c;
        }
    }
    if (t < hd) {
        if (is_q) {
            e.q_out[(size_t)hh * hd + t] = v;
        } else {
            const int g = is_k ? hh - e.nq : hh - e.nq - e.nkv;
            uint16_t* base = is_k ? e.kc : e.vc;
            size_t off;
            if (e.paged) {
                const int phys = e.table[pos / ATT_BS];
                off = (((size_t)phys * e.nkv + g) * ATT_BS + pos % ATT_BS) * hd + t;
            } else {
                off = ((size_t)g * e.max_seq + pos) * hd + t;
            }
            base[off] = f32_to_f16(v);
        }
    }
}

template <int LPR, int RPS, int NWAVES>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_qkv(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
           const float* __restrict__ u, int N, int nb, const float* __restrict__ ss_part,
           int n_part, int n_in, float eps_in, QkvEpi e)
{
    using G = GemvGeom<LPR, RPS, NWAVES>;
    extern __shared__ float smem[];
    __shared__ float scal, red[8], sv[128];
    __shared__ bool last;
    float* xl = smem;
    float* xs = smem + nb * XPAD;
    const float inv = inv_rms_from_partials(ss_part, n_part, n_in, eps_in, &scal);
    stage_x<G::NT>(u, nb, xl, xs);
    const int ntiles = N / G::ROWS;            // N is a multiple of hd, hd of ROWS
    const int tiles_per_head = e.hd / G::ROWS;
    const int lr = (threadIdx.x & (WAVE - 1)) % LPR;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        float acc[RPS];
        const int row0 = gemv_tile<LPR, RPS, NWAVES>(D, Q, N, nb, xl, xs, tile, acc);
        if (lr == 0) {
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                e.raw[row0 + r] = acc[r] * inv;
        }
        const int hh = tile / tiles_per_head;
        if (arrive_last(e.counters + hh, (unsigned)tiles_per_head, &last)) {
            qkv_head_finish(e, hh, sv, red);
            reset_counter(e.counters + hh);
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------------- residual

// x[row] += W row . a; u[row] = x[row] * w_next[row]; per-workgroup sum of x^2
template <int LPR, int RPS, int NWAVES>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_residual(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
                const float* __restrict__ a, int N, int nb, float* __restrict__ x,
                float* __restrict__ u, const float* __restrict__ w_next,
                float* __restrict__ ss_part)
{
    using G = GemvGeom<LPR, RPS, NWAVES>;
    extern __shared__ float smem[];
    __shared__ float red[8];
    float* xl = smem;
    float* xs = smem + nb * XPAD;
    stage_x<G::NT>(a, nb, xl, xs);
    const int ntiles = (N + G::ROWS - 1) / G::ROWS;
    const int lr = (threadIdx.x & (WAVE - 1)) % LPR;
    float ss = 0.f;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        float acc[RPS];
        const int row0 = gemv_tile<LPR, RPS, NWAVES>(D, Q, N, nb, xl, xs, tile, acc);
        if (lr == 0) {
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const int row = row0 + r;
                if (row < N) {
                    const float nx = x[row] + acc[r];
                    x[row] = nx;
                    u[row] = nx * w_next[row];
                    ss = fmaf(nx, nx, ss);
                }
            }
        }
    }
    ss = block_sum256(ss, red);
    if (threadIdx.x == 0)
        ss_part[blockIdx.x] = ss;
}

// ----------------------------------------------------------------- gate|up + SwiGLU

// rows interleaved: row 2i = gate_i, row 2i+1 = up_i; act[i] = silu(g) * up
template <int LPR, int RPS, int NWAVES>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_swiglu(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
              const float* __restrict__ u, int N, int nb, const float* __restrict__ ss_part,
              int n_part, int n_in, float eps_in, float* __restrict__ act)
{
    static_assert(RPS % 2 == 0, "gate/up pairs");
    using G = GemvGeom<LPR, RPS, NWAVES>;
    extern __shared__ float smem[];
    __shared__ float scal;
    float* xl = smem;
    float* xs = smem + nb * XPAD;
    const float inv = inv_rms_from_partials(ss_part, n_part, n_in, eps_in, &scal);
    stage_x<G::NT>(u, nb, xl, xs);
    const int ntiles = (N + G::ROWS - 1) / G::ROWS;
    const int lr = (threadIdx.x & (WAVE - 1)) % LPR;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        float acc[RPS];
        const int row0 = gemv_tile<LPR, RPS, NWAVES>(D, Q, N, nb, xl, xs, tile, acc);
        if (lr == 0) {
#pragma unroll
            for (int r = 0; r < RPS; r += 2) {
                if (row0 + r + 1 < N) {
                    const float gt = acc[r] * inv, up = acc[r + 1] * inv;
                    act[(row0 + r) >> 1] = gt / (1.0f + expf(-gt)) * up;
                }
            }
        }
    }
}

// ----------------------------------------------------------------- LM head + greedy

// logits = W u / rms; greedy argmax (lowest index among equal maxima); the
// last workgroup records the token and advances the position.
template <int LPR, int RPS, int NWAVES>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_lmhead(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
              const float* __restrict__ u, int N, int nb, const float* __restrict__ ss_part,
              int n_part, int n_in, float eps_in, float* __restrict__ logits,
              float* __restrict__ part_val, int32_t* __restrict__ part_idx,
              unsigned int* __restrict__ counter, StepState* __restrict__ st,
              int32_t* __restrict__ ids, int32_t* __restrict__ pred, int max_seq)
{
    using G = GemvGeom<LPR, RPS, NWAVES>;
    extern __shared__ float smem[];
    __shared__ float scal, bv[NWAVES];
    __shared__ int32_t bi[NWAVES];
    __shared__ bool last;
    float* xl = smem;
    float* xs = smem + nb * XPAD;
    const float inv = inv_rms_from_partials(ss_part, n_part, n_in, eps_in, &scal);
    stage_x<G::NT>(u, nb, xl, xs);
    const int ntiles = (N + G::ROWS - 1) / G::ROWS;
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    const int lr = lane % LPR;
    float best = -INFINITY;
    int32_t bidx = 0x7fffffff;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        float acc[RPS];
        const int row0 = gemv_tile<LPR, RPS, NWAVES>(D, Q, N, nb, xl, xs, tile, acc);
        if (lr == 0) {
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const int row = row0 + r;
                if (row < N) {
                    const float v = acc[r] * inv;
                    logits[row] = v;
                    if (v > best || (v == best && row < bidx)) {
                        best = v;
                        bidx = row;
                    }
                }
            }
        }
    }
    // workgroup argmax (lanes that hold no row keep -inf / INT_MAX)
    for (int m = WAVE / 2; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(best, m, WAVE);
        const int32_t oi = __shfl_xor(bidx, m, WAVE);
        if (ov > best || (ov == best && oi < bidx)) {
            best = ov;
            bidx = oi;
        }
    }
    if (lane == 0) {
        bv[wave] = best;
        bi[wave] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < NWAVES; ++w)
            if (bv[w] > best || (bv[w] == best && bi[w] < bidx)) {
                best = bv[w];
                bidx = bi[w];
            }
        part_val[blockIdx.x] = best;
        part_idx[blockIdx.x] = bidx;
    }
    if (!arrive_last(counter, gridDim.x, &last))
        return;
    // final argmax over the workgroups' candidates, in a fixed order
    best = -INFINITY;
    bidx = 0x7fffffff;
    for (int i = threadIdx.x; i < (int)gridDim.x; i += blockDim.x) {
        const float v = part_val[i];
        const int32_t ix = part_idx[i];
        if (v > best || (v == best && ix < bidx)) {
            best = v;
            bidx = ix;
        }
    }
    for (int m = WAVE / 2; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(best, m, WAVE);
        const int32_t oi = __shfl_xor(bidx, m, WAVE);
        if (ov > best || (ov == best && oi < bidx)) {
            best = ov;
            bidx = oi;
        }
    }
    __syncthreads();
    if (lane == 0) {
        bv[wave] = best;
        bi[wave] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < NWAVES; ++w)
            if (bv[w] > best || (bv[w] == best && bi[w] < bidx)) {
                best = bv[w];
                bidx = bi[w];
            }
        if (bidx < 0 || bidx >= N)
            bidx = 0;
        int p = st->pos;
        if (p >= 0 && p < max_seq) {
            pred[p] = bidx;
            if (p + 1 < max_seq && p + 1 >= st->n_forced)
                ids[p + 1] = bidx;
        }
        st->pos = p + 1;
        *counter = 0u;
    }
}

}  // namespace qd
