// prefill_kernels.h -- the kernels of a chunked prefill (gfx950) of its own:
// T <= 32 prompt positions at a time, every weight read once per chunk by the
// batched GEMV on split inputs (gemv_batch_mfma.h: the positions are its
// vectors), the norms, SwiGLU and splits of the batched decode step
// (step_batch.h), the same arithmetic per position as the decode step
// (inferencelayer cuda_llm.rs page: prefill as the M > 1 form of the step; the
// step's order of operations).  Here: the embedding rows, the per-head q/k
// norm + rotary + K/V store, and the index table of the greedy pick.
#pragma once

#include "step_kernels.h"

namespace qd {

constexpr int PF_NG = 4;          // 16-position groups per chunk
constexpr int PF_T = 16 * PF_NG;   // positions per chunk

// X[t][i] = dequant(E)[ids[p0 + t]][i]; grid (ceil(H/256), T)
__global__ void __launch_bounds__(256)
k_pf_embed(const uint16_t* __restrict__ Ed, const uint8_t* __restrict__ Eq, int H,
           const int32_t* __restrict__ ids, int p0, float* __restrict__ X)
{
    const int t = blockIdx.y, i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= H)
        return;
    // every stored token is in range: the buffer starts zeroed, host tokens
    // are checked when stored, and the greedy step stores a clamped argmax
    const int tok = ids[p0 + t];
    const int nb = H / 32, bk = i >> 5, j = i & 31;
    const size_t blk = (size_t)tok * nb + bk;
    const uint8_t byte = Eq[blk * 16 + (j & 15)];
    const int code = (j < 16) ? (byte & 15) : (byte >> 4);
    X[(size_t)t * H + i] = (float)(code - 8) * f16_to_f32(Ed[blk]);
}

// Per position t (grid.y) and head (grid.x: nq query heads, then nkv kv heads),
// one wave per head: q/k RMSNorm over the head (if qk_norm), NeoX rotary at
// position p0 + t from the tables, then q -> Qr[t][h], and for a kv head K and
// V into the cache at p0 + t (f16, or e4m3 of value / scale).  Also
// kv_lens[t] = p0 + t + 1.
template <int HD, bool KV8>
__global__ void __launch_bounds__(WAVE)
k_pf_qk(const float* __restrict__ QKV, int qkv_rows, int nq, int nkv, const float* __restrict__ q_norm,
        const float* __restrict__ k_norm, int qk_norm, float eps, int rot,
        const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, int p0,
        float* __restrict__ Qr, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
        const int32_t* __restrict__ table, int max_seq, float k_scale, float v_scale,
        int32_t* __restrict__ kv_lens, int nslab, size_t slab)
{
    constexpr int DPL = HD / WAVE;
    const int t = blockIdx.y, hh = blockIdx.x, lane = threadIdx.x;
    const int pos = p0 + t;
    const bool is_q = hh < nq;
    const int g = hh - nq;
    // QKV may come as nslab partial products slab floats apart: added in slab order
    auto ld = [&](const float* p) { return slab_sum<8>(p, nslab, slab); };
    const float* src = QKV + (size_t)t * qkv_rows + (size_t)(is_q ? hh : nq + g) * HD;
    const float* w = is_q ? q_norm : k_norm;
    float v[DPL];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        v[e] = ld(src + lane * DPL + e);
        ss = fmaf(v[e], v[e], ss);
    }
    ss = group_sum<WAVE>(ss);
    const float r = qk_norm ? 1.0f / sqrtf(ss / (float)HD + eps) : 1.f;
    __shared__ float row[HD];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        v[e] = v[e] * r * (qk_norm ? w[lane * DPL + e] : 1.f);
        row[lane * DPL + e] = v[e];
    }
    __syncthreads();
    const int half = rot / 2;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        const int d = lane * DPL + e;
        if (d < rot) {
            const int i = d < half ? d : d - half;
            const float c = rope_cos[(size_t)pos * half + i], s = rope_sin[(size_t)pos * half + i];
            const float partner = row[d < half ? d + half : d - half];
            v[e] = fmaf(partner, d < half ? -s : s, v[e] * c);
        }
    }
    if (is_q) {
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            Qr[((size_t)t * nq + hh) * HD + lane * DPL + e] = v[e];
    } else {
        size_t o;
        if (table)
            o = ((((size_t)table[pos / ATT_BS] * nkv + g) * ATT_BS) + pos % ATT_BS) * HD;
        else
            o = (((size_t)g * max_seq) + pos) * HD;
        const float* vsrc = QKV + (size_t)t * qkv_rows + (size_t)(nq + nkv + g) * HD;
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            const int d = lane * DPL + e;
            const float vv = ld(vsrc + d);
            if (KV8) {
                reinterpret_cast<uint8_t*>(kc)[o + d] = (uint8_t)f32_to_e4m3(v[e] / k_scale);
                reinterpret_cast<uint8_t*>(vc)[o + d] = (uint8_t)f32_to_e4m3(vv / v_scale);
            } else {
                kc[o + d] = f32_to_f16(v[e]);
                vc[o + d] = f32_to_f16(vv);
            }
        }
    }
    if (hh == 0 && lane == 0)
        kv_lens[t] = pos + 1;
}

// logit i -> candidate (value, index i): the argmax kernel's input form
__global__ void __launch_bounds__(256) k_pf_iota(int32_t* __restrict__ idx, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        idx[i] = i;
}

}  // namespace qd
