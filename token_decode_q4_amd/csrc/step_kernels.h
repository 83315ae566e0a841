// step_kernels.h -- the kernels of one batch-1 decode step (gfx950).
//
// Step order (inferencelayer cuda_llm.rs page, CudaQwen3::step;
// ferrum-kernels cuda_decode.rs page, CudaDecodeRunner::decode_step with its
// fused add + RMSNorm chaining across layers):
//   k_embed                       x = E[token]; u = x * w_attn(0); ss partials
//   per layer:
//     k_gemv_scaled (q|k|v)       raw = Wqkv u / rms
//     k_attn_split                per-head q/k RMSNorm + rotary, K/V of the token
//                                 written at pos, split-KV GQA partials
//     k_attn_combine              online-softmax merge of the partials
//     k_gemv_residual (o)         x += Wo attn; u = x * w_ffn; ss partials
//     k_gemv_swiglu (gate|up)     a = silu(Wg u / rms) * (Wu u / rms)
//     k_gemv_residual (down)      x += Wd a; u = x * w_next; ss partials
//   k_gemv_lmhead                 logits = Wlm u / rms; per-workgroup argmax
//   k_argmax_advance              greedy token, stored token, position + 1
//
// No kernel waits on another workgroup of its own launch: every global
// dependency is a kernel boundary (cross-workgroup fences are far more costly
// than a boundary on this part).
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

// grid ceil(H/256): one element per thread; per-workgroup sum of x^2.
// Workgroup 0 also copies the rotary factors of the step's position from the
// tables [max_seq][half] to rope_cur (cos [half] then sin [half]), and zeroes
// the n_zero words at zero_words (the persistent layer kernel's barrier
// counters; nothing when n_zero is 0).
__global__ void __launch_bounds__(256)
k_embed(const uint16_t* __restrict__ Ed, const uint8_t* __restrict__ Eq, int H, int vocab,
        StepState* __restrict__ st, const int32_t* __restrict__ ids, int max_seq,
        const float* __restrict__ w_norm, float* __restrict__ x, float* __restrict__ u,
        float* __restrict__ ss_part, const float* __restrict__ rope_cos,
        const float* __restrict__ rope_sin, int half, float* __restrict__ rope_cur,
        unsigned* __restrict__ zero_words, int n_zero)
{
    __shared__ float red[8];
    if (blockIdx.x == 0)
        for (int k = threadIdx.x; k < n_zero; k += blockDim.x)
            zero_words[k] = 0u;
    int pos = st->pos;
    if (pos < 0 || pos >= max_seq) {
        if (threadIdx.x == 0 && blockIdx.x == 0) st->error |= 2;
        pos = 0;
    }
    int tok = ids[pos];
    if (tok < 0 || tok >= vocab) {
        if (threadIdx.x == 0 && blockIdx.x == 0) st->error |= 1;
        tok = 0;
    }
    if (blockIdx.x == 0) {
        for (int k = threadIdx.x; k < half; k += blockDim.x) {
            rope_cur[k] = rope_cos[(size_t)pos * half + k];
            rope_cur[half + k] = rope_sin[(size_t)pos * half + k];
        }
    }
    const int nb = H / 32;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    float v = 0.f;
    if (i < H) {
        const int bk = i >> 5, j = i & 31;
        const size_t blk = (size_t)tok * nb + bk;
        const uint8_t byte = Eq[blk * 16 + (j & 15)];
        const int code = (j < 16) ? (byte & 15) : (byte >> 4);
        v = (float)(code - 8) * f16_to_f32(Ed[blk]);
        x[i] = v;
        u[i] = v * w_norm[i];
    }
    const float ss = block_sum256(v * v, red);
    if (threadIdx.x == 0)
        ss_part[blockIdx.x] = ss;
}

// ----------------------------------------------------------------- GEMV epilogues

// y[row] = (W u)[row] / rms, with 1/rms from the producer's partial sums
struct EpiScaled {
    float* y;
    int N;
    RmsPartials rp;
    int n_in;
    float eps;
    float inv;
    QD_DEV void issue(int) { rp.issue(); }
    QD_DEV void finish() { inv = rp.finish(n_in, eps); }
    template <int RPS>
    QD_DEV void tile(int row0, const float (&acc)[RPS], bool lead)
    {
        if (lead) {
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                if (row0 + r < N)
                    y[row0 + r] = acc[r] * inv;
        }
    }
};

// x[row] += acc; u[row] = x[row] * w_next[row]; running sum of the new x^2.
// Launched with one tile per workgroup: issue() loads the tile's x and w_next
// rows at kernel start, so the epilogue itself loads nothing.
template <int RPS>
struct EpiResidual {
    float* x;
    float* u;
    const float* w_next;
    int N;
    float ss;
    float px[RPS], pw[RPS];
    QD_DEV void issue(int row0)
    {
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            const int row = min(row0 + r, N - 1);
            px[r] = x[row];
            pw[r] = w_next[row];
        }
    }
    QD_DEV void finish() {}
    QD_DEV void tile(int row0, const float (&acc)[RPS], bool lead)
    {
        if (lead) {
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const int row = row0 + r;
                if (row < N) {
                    const float nx = px[r] + acc[r];
                    x[row] = nx;
                    u[row] = nx * pw[r];
                    ss = fmaf(nx, nx, ss);
                }
            }
        }
    }
};

// rows interleaved (2i = gate_i, 2i+1 = up_i): act[i] = silu(g) * up, with
// g = (Wg u)/rms and up = (Wu u)/rms
struct EpiSwiglu {
    float* act;
    int N;
    RmsPartials rp;
    int n_in;
    float eps;
    float inv;
    QD_DEV void issue(int) { rp.issue(); }
    QD_DEV void finish() { inv = rp.finish(n_in, eps); }
    template <int RPS>
    QD_DEV void tile(int row0, const float (&acc)[RPS], bool lead)
    {
        static_assert(RPS % 2 == 0, "gate/up pairs");
        if (lead) {
#pragma unroll
            for (int r = 0; r < RPS; r += 2) {
                if (row0 + r + 1 < N) {
                    const float gt = acc[r] * inv, up = acc[r + 1] * inv;
                    // silu(g) = g / (1 + e^-g); hardware reciprocal (about 1 ulp)
                    act[(row0 + r) >> 1] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
                }
            }
        }
    }
};

// logits[row] = (W u)[row] / rms; running best (value, lowest index among equals)
struct EpiLmHead {
    float* logits;
    int N;
    RmsPartials rp;
    int n_in;
    float eps;
    float inv;
    float best;
    int32_t bidx;
    QD_DEV void issue(int) { rp.issue(); }
    QD_DEV void finish() { inv = rp.finish(n_in, eps); }
    template <int RPS>
    QD_DEV void tile(int row0, const float (&acc)[RPS], bool lead)
    {
        if (lead) {
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
};

// ----------------------------------------------------------------- GEMV kernels

template <int LPR, int RPS, int NWAVES, int BG, int NBUF, int UNR, bool NTL>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_scaled(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
              const float* __restrict__ u, int N, int nb, const float* __restrict__ ss_part,
              int n_part, int n_in, float eps_in, float* __restrict__ y)
{
    extern __shared__ __align__(16) float smem[];   // 16-byte aligned: x is read as float4
    EpiScaled e{y, N, {ss_part, n_part}, n_in, eps_in};
    gemv_run<LPR, RPS, NWAVES, BG, NBUF, UNR, NTL>(D, Q, u, N, nb, smem, smem + nb * XPAD, e);
    QD_MARK(3);
}

template <int LPR, int RPS, int NWAVES, int BG, int NBUF, int UNR, bool NTL>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_residual(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
                const float* __restrict__ a, int N, int nb, float* __restrict__ x,
                float* __restrict__ u, const float* __restrict__ w_next,
                float* __restrict__ ss_part)
{
    extern __shared__ __align__(16) float smem[];   // 16-byte aligned: x is read as float4
    __shared__ float red[8];
    EpiResidual<RPS> e{x, u, w_next, N, 0.f};
    gemv_run<LPR, RPS, NWAVES, BG, NBUF, UNR, NTL>(D, Q, a, N, nb, smem, smem + nb * XPAD, e);
    const float ss = block_sum256(e.ss, red);
    if (threadIdx.x == 0)
        ss_part[blockIdx.x] = ss;
    QD_MARK(3);
}

template <int LPR, int RPS, int NWAVES, int BG, int NBUF, int UNR, bool NTL>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_swiglu(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
              const float* __restrict__ u, int N, int nb, const float* __restrict__ ss_part,
              int n_part, int n_in, float eps_in, float* __restrict__ act)
{
    extern __shared__ __align__(16) float smem[];   // 16-byte aligned: x is read as float4
    EpiSwiglu e{act, N, {ss_part, n_part}, n_in, eps_in};
    gemv_run<LPR, RPS, NWAVES, BG, NBUF, UNR, NTL>(D, Q, u, N, nb, smem, smem + nb * XPAD, e);
    QD_MARK(3);
}

// logits = W u / rms; each workgroup's best (value, lowest index among equals)
template <int LPR, int RPS, int NWAVES, int BG, int NBUF, int UNR, bool NTL>
__global__ void __launch_bounds__(NWAVES* WAVE)
k_gemv_lmhead(const uint16_t* __restrict__ D, const uint8_t* __restrict__ Q,
              const float* __restrict__ u, int N, int nb, const float* __restrict__ ss_part,
              int n_part, int n_in, float eps_in, float* __restrict__ logits,
              float* __restrict__ part_val, int32_t* __restrict__ part_idx)
{
    extern __shared__ __align__(16) float smem[];   // 16-byte aligned: x is read as float4
    __shared__ float bv[NWAVES];
    __shared__ int32_t bi[NWAVES];
    EpiLmHead e{logits, N, {ss_part, n_part}, n_in, eps_in, 0.f, -INFINITY, 0x7fffffff};
    gemv_run<LPR, RPS, NWAVES, BG, NBUF, UNR, NTL>(D, Q, u, N, nb, smem, smem + nb * XPAD, e);
    float best = e.best;
    int32_t bidx = e.bidx;
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
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
}

// one workgroup: greedy token from the LM head's per-workgroup candidates (a
// fixed-order reduction, lowest index among equal maxima), recorded as the
// step's prediction; it becomes the stored token of the next position unless
// that position is forced; the position advances.
QD_DEV void argmax_advance_body(const float* __restrict__ part_val, const int32_t* __restrict__ part_idx,
                                int n_part, int vocab, StepState* __restrict__ st, int32_t* __restrict__ ids,
                                int32_t* __restrict__ pred, int max_seq)
{
    __shared__ float bv[4];
    __shared__ int32_t bi[4];
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    float best = -INFINITY;
    int32_t bidx = 0x7fffffff;
    constexpr int U = 8;   // every load of a round issued before any compare
    for (int i0 = 0; i0 < n_part; i0 += U * 256) {
        float v[U];
        int32_t ix[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + (int)threadIdx.x + u * 256;
            const int ic = min(i, n_part - 1);   // loads never under a branch
            v[u] = part_val[ic];
            ix[u] = part_idx[ic];
            if (i >= n_part) {
                v[u] = -INFINITY;
                ix[u] = 0x7fffffff;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (v[u] > best || (v[u] == best && ix[u] < bidx)) {
                best = v[u];
                bidx = ix[u];
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
    if (lane == 0) {
        bv[wave] = best;
        bi[wave] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < (int)(blockDim.x / WAVE); ++w)
            if (bv[w] > best || (bv[w] == best && bi[w] < bidx)) {
                best = bv[w];
                bidx = bi[w];
            }
        if (bidx < 0 || bidx >= vocab)
            bidx = 0;
        const int p = st->pos;
        if (p >= 0 && p < max_seq) {
            pred[p] = bidx;
            if (p + 1 < max_seq && p + 1 >= st->n_forced)
                ids[p + 1] = bidx;
        }
        st->pos = p + 1;
    }
}

__global__ void __launch_bounds__(256)
k_argmax_advance(const float* __restrict__ part_val, const int32_t* __restrict__ part_idx,
                 int n_part, int vocab, StepState* __restrict__ st, int32_t* __restrict__ ids,
                 int32_t* __restrict__ pred, int max_seq)
{
    argmax_advance_body(part_val, part_idx, n_part, vocab, st, ids, pred, max_seq);
}

}  // namespace qd
