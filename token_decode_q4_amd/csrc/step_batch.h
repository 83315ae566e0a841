// step_batch.h -- the elementwise kernels of the decode step of B sequences
// at once (batched decode: the inferencelayer cuda_llm.rs page, its batched
// head-to-head of the q4 GEMV arm at M = 2 .. 16 tokens, and
// step_batch_inner; ferrum-kernels cuda_decode.rs page,
// batched_decode_attention).
//
// Each of the B sequences has its own position, stored tokens, K/V cache and
// greedy prediction; every weight is read once per step for all of them by
// the batched GEMVs (gemv_batch_mfma.h), which take their input already split
// (XP / XS).  So here, unlike the one-sequence step, the RMSNorm's weights are
// applied before the product, by one workgroup per (chunk, sequence); each
// chunk's sum of x^2 goes beside the split and the product applies 1/rms.
//   k_embed_xp_batch        x[b] = E[token_b]; split of x[b] * w; rotary factors
//   (batched q|k|v GEMV; split-KV attention over the B caches, whose merge
//    writes the o product's split input from 8 sequences, k_xsplit_batch
//    below that; batched o GEMV)
//   k_resid_norm_xp_batch   x[b] += y[b]; split of x[b] * w
//   (batched gate|up GEMV)  k_swiglu_xp_batch: a[b][i] = silu(g) * up
//   (batched down GEMV)     k_resid_norm_xp_batch (next layer's or the final norm)
//   (batched LM head)       k_argmax_batch, k_argmax_advance_batch
// k_resid_rmsnorm_batch, one workgroup per row, writes a normalised row in
// f32 (the prefill's final norm, whose last row feeds the one-vector LM head).
#pragma once

#include "gemv_batch_mfma.h"
#include "step_kernels.h"

namespace qd {

constexpr int SB_MAXB = 16;    // sequences of a batched model
constexpr int SB_THREADS = 1024;
constexpr int SB_MAXSLAB = 12;  // K slices of a batched step's product

// sum over a workgroup of SB_THREADS threads in a fixed order (every thread
// gets it); red >= 16 floats
QD_DEV float sb_block_sum(float v, float* red)
{
    v = group_sum<WAVE>(v);
    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    __syncthreads();
    if (lane == 0)
        red[wv] = v;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < (int)(blockDim.x / WAVE); ++i)
        s += red[i];
    return s;
}

// The batched RMSNorm works on items (chunk, block, lane group) of 8
// elements: 4kg .. 4kg+3 and 16+4kg .. 16+4kg+3 of the block, as the split
// for the product groups them (chunks of 32 / ng blocks for ng slot groups).  A thread holds at most SB_ITEMS items (item
// it = thread + u * SB_THREADS), so every load of a row is issued in one
// round and the values stay in registers between the two passes.
constexpr int SB_ITEMS = 2;   // H <= 16384

// items of a row with NG = ng slot groups: chunks of KCB = 32 / ng blocks,
// 4 KCB items each (a multiple of a wave)
QD_DEV int sb_nitems(int H, int ng) { return gbm_nchunks(H / 32, ng) * 4 * gbm_kcb(ng); }

// item it of a row: its chunk, block within the chunk, lane group, block
QD_DEV void sb_item(int it, int ng, int& c, int& bl, int& kg, int& blk)
{
    const int kcb = gbm_kcb(ng);
    c = it / (4 * kcb);
    bl = (it >> 2) % kcb;
    kg = it & 3;
    blk = c * kcb + bl;
}

// the second pass: v[u] (element order 4kg.., 16+4kg..) / rms * w of the
// thread's items, written as f32 to h (if not null) and split into XP / XS
// (if not null) for the product; cmax >= 32 floats
QD_DEV void sb_norm_items(const float (&v)[SB_ITEMS][8], const float (&wv)[SB_ITEMS][8], float inv, int H,
                          int b, float* __restrict__ h, _Float16* __restrict__ XP, float* __restrict__ XS,
                          int ng, float* cmax)
{
    const int nb = H / 32, nit = sb_nitems(H, ng), wpc = gbm_kcb(ng) * 4 / WAVE;   // waves per chunk
    float e[SB_ITEMS][8];
#pragma unroll
    for (int u = 0; u < SB_ITEMS; ++u) {
        const int it = (int)threadIdx.x + u * SB_THREADS;
        if (it < nit) {   // uniform per wave (nit is a multiple of 64)
            int c, bl, kg, blk;
            sb_item(it, ng, c, bl, kg, blk);
            float hv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                hv[k] = v[u][k] * inv * wv[u][k];
            if (h && blk < nb) {
                float* hp = h + (size_t)b * H + (size_t)blk * 32 + 4 * kg;
                *reinterpret_cast<float4*>(hp) = make_float4(hv[0], hv[1], hv[2], hv[3]);
                *reinterpret_cast<float4*>(hp + 16) = make_float4(hv[4], hv[5], hv[6], hv[7]);
            }
            const float q = 0.0625f;   // the split order (high four divided by 16)
            const float ev[8] = {hv[0], hv[2], hv[1], hv[3], hv[4] * q, hv[6] * q, hv[5] * q, hv[7] * q};
#pragma unroll
            for (int k = 0; k < 8; ++k)
                e[u][k] = ev[k];
            if (XP) {   // uniform
                const float m = group_max<WAVE>(gbm_xp_absmax(e[u]));
                if ((threadIdx.x & (WAVE - 1)) == 0)
                    cmax[it / WAVE] = m;
            }
        }
    }
    if (!XP)
        return;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < SB_ITEMS; ++u) {
        const int it = (int)threadIdx.x + u * SB_THREADS;
        if (it < nit) {
            int c, bl, kg, blk;
            sb_item(it, ng, c, bl, kg, blk);
            float cm = cmax[c * wpc];
            for (int q = 1; q < wpc; ++q)
                cm = fmaxf(cm, cmax[c * wpc + q]);
            const float s = gbm_scale_for(cm);
            if (blk < nb)
                gbm_xp_put(XP, ng, c, bl, kg, b, e[u], s);
            if (bl == 0 && kg == 0)
                XS[c * 16 * ng + b] = 1.0f / s;
        }
    }
}

// grid B: x[b] += y[b] (y may be null: no residual; y may come as nslab <=
// SB_MAXSLAB partial products slab floats apart, added in slab order);
// x[b] / rms * w to h and/or XP / XS (as sb_norm_items)
__global__ void __launch_bounds__(SB_THREADS)
k_resid_rmsnorm_batch(float* __restrict__ x, const float* __restrict__ y, int nslab, size_t slab, int H,
                      const float* __restrict__ w, float eps, float* __restrict__ h,
                      _Float16* __restrict__ XP, float* __restrict__ XS, int ng)
{
    __shared__ float red[16];
    __shared__ float cmax[32];
    const int b = blockIdx.x;
    const int nb = H / 32, nit = sb_nitems(H, ng);
    float* xb = x + (size_t)b * H;
    float v[SB_ITEMS][8], wv[SB_ITEMS][8];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < SB_ITEMS; ++u) {
        const int it = (int)threadIdx.x + u * SB_THREADS;
        int c, bl, kg, blk;
        sb_item(it, ng, c, bl, kg, blk);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[u][k] = wv[u][k] = 0.f;
        if (it < nit && blk < nb) {
            const size_t off = (size_t)blk * 32 + 4 * kg;
            float4 a = *reinterpret_cast<const float4*>(xb + off);
            float4 e = *reinterpret_cast<const float4*>(xb + off + 16);
            const float4 wa = *reinterpret_cast<const float4*>(w + off);
            const float4 wh = *reinterpret_cast<const float4*>(w + off + 16);
            if (y) {   // uniform
                const float* yb = y + (size_t)b * H + off;
                float4 ra = *reinterpret_cast<const float4*>(yb);
                float4 re = *reinterpret_cast<const float4*>(yb + 16);
#pragma unroll
                for (int k = 1; k < SB_MAXSLAB; ++k) {
                    if (k < nslab) {   // uniform
                        const float4 pa = *reinterpret_cast<const float4*>(yb + k * slab);
                        const float4 pe = *reinterpret_cast<const float4*>(yb + k * slab + 16);
                        ra = make_float4(ra.x + pa.x, ra.y + pa.y, ra.z + pa.z, ra.w + pa.w);
                        re = make_float4(re.x + pe.x, re.y + pe.y, re.z + pe.z, re.w + pe.w);
                    }
                }
                a = make_float4(a.x + ra.x, a.y + ra.y, a.z + ra.z, a.w + ra.w);
                e = make_float4(e.x + re.x, e.y + re.y, e.z + re.z, e.w + re.w);
                *reinterpret_cast<float4*>(xb + off) = a;
                *reinterpret_cast<float4*>(xb + off + 16) = e;
            }
            const float vl[8] = {a.x, a.y, a.z, a.w, e.x, e.y, e.z, e.w};
            const float wl[8] = {wa.x, wa.y, wa.z, wa.w, wh.x, wh.y, wh.z, wh.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                v[u][k] = vl[k];
                wv[u][k] = wl[k];
                ss = fmaf(vl[k], vl[k], ss);
            }
        }
    }
    const float inv = 1.0f / sqrtf(sb_block_sum(ss, red) / (float)H + eps);
    sb_norm_items(v, wv, inv, H, b, h, XP, XS, ng, cmax);
}

// sum over a workgroup of 64 or 128 threads (a chunk's items) in a fixed
// order; every thread gets it; red >= 2 floats
QD_DEV float sb_chunk_sum(float v, float* red)
{
    v = group_sum<WAVE>(v);
    if ((threadIdx.x & (WAVE - 1)) == 0)
        red[threadIdx.x / WAVE] = v;
    __syncthreads();
    return blockDim.x > WAVE ? red[0] + red[1] : red[0];
}

// The chunk-parallel form of the norm before a product: one workgroup per
// (chunk, sequence) holds v (elements 4kg.., 16+4kg.. of its item, zero past
// the row) and the norm weights wv, and writes v * w split (XP / XS with a
// scale of its own) and the chunk's sum of v^2 to SQ[c][slot].  The 1/rms
// factor is left to the product, which sums SQ over the chunks of its
// vectors (k_gemv_batch_xp): a row's norm needs no workgroup to wait for
// another.
QD_DEV void sb_norm_chunk(const float (&v)[8], const float (&wv)[8], int c, int bl, int kg, int b, bool in,
                          int ng, _Float16* __restrict__ XP, float* __restrict__ XS, float* __restrict__ SQ,
                          float* red_m, float* red_s)
{
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        ss = fmaf(v[k], v[k], ss);
    const float q = 0.0625f;   // the split order (high four divided by 16)
    const float e[8] = {v[0] * wv[0], v[2] * wv[2], v[1] * wv[1], v[3] * wv[3],
                        v[4] * wv[4] * q, v[6] * wv[6] * q, v[5] * wv[5] * q, v[7] * wv[7] * q};
    const float s = gbm_scale_for(gbm_chunk_max(gbm_xp_absmax(e), red_m));
    const float sq = sb_chunk_sum(ss, red_s);
    if (in)
        gbm_xp_put(XP, ng, c, bl, kg, b, e, s);
    if (threadIdx.x == 0) {
        XS[c * 16 * ng + b] = 1.0f / s;
        SQ[c * 16 * ng + b] = sq;
    }
}

// grid (chunks of H, B), gbm_chunk_threads(ng) threads: x[b] += y[b] (y may
// be null: no residual; y may come as nslab partial products slab floats
// apart, added in slab order), then x[b] * w split for the product with the
// chunk sums of x[b]^2 (sb_norm_chunk)
__global__ void __launch_bounds__(128)
k_resid_norm_xp_batch(float* __restrict__ x, const float* __restrict__ y, int nslab, size_t slab, int H,
                      const float* __restrict__ w, int ng, _Float16* __restrict__ XP, float* __restrict__ XS,
                      float* __restrict__ SQ)
{
    __shared__ float red_m[2], red_s[2];
    const int c = blockIdx.x, b = blockIdx.y;
    const int bl = threadIdx.x >> 2, kg = threadIdx.x & 3, blk = c * gbm_kcb(ng) + bl;
    const bool in = bl < gbm_kcb(ng) && blk < H / 32;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (in) {
        const size_t off = (size_t)blk * 32 + 4 * kg;
        float* xb = x + (size_t)b * H + off;
        float4 a = *reinterpret_cast<const float4*>(xb);
        float4 e = *reinterpret_cast<const float4*>(xb + 16);
        const float4 wa = *reinterpret_cast<const float4*>(w + off);
        const float4 wh = *reinterpret_cast<const float4*>(w + off + 16);
        if (y) {   // uniform
            const float* yb = y + (size_t)b * H + off;
            const float4 ra = slab_sum<SB_MAXSLAB>(reinterpret_cast<const float4*>(yb), nslab, slab / 4);
            const float4 re = slab_sum<SB_MAXSLAB>(reinterpret_cast<const float4*>(yb + 16), nslab, slab / 4);
            a = make_float4(a.x + ra.x, a.y + ra.y, a.z + ra.z, a.w + ra.w);
            e = make_float4(e.x + re.x, e.y + re.y, e.z + re.z, e.w + re.w);
            *reinterpret_cast<float4*>(xb) = a;
            *reinterpret_cast<float4*>(xb + 16) = e;
        }
        const float vl[8] = {a.x, a.y, a.z, a.w, e.x, e.y, e.z, e.w};
        const float wl[8] = {wa.x, wa.y, wa.z, wa.w, wh.x, wh.y, wh.z, wh.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            v[k] = vl[k];
            wv[k] = wl[k];
        }
    }
    sb_norm_chunk(v, wv, c, bl, kg, b, in, ng, XP, XS, SQ, red_m, red_s);
}

// grid (chunks of H, B), gbm_chunk_threads(ng) threads: sequence b at its position
// st[b].pos reads its stored token and writes x[b] (the embedding row), the
// split of x[b] * w with the chunk sums of x[b]^2 (as k_resid_norm_xp_batch)
// and, in the chunk 0 workgroup, the rotary factors of its position (cos
// [half] then sin [half]) at rope_cur + b * rstride.  A position or token out
// of range is recorded in st[b].error and replaced by 0 (reported by
// qd_check).
__global__ void __launch_bounds__(128)
k_embed_xp_batch(const uint16_t* __restrict__ Ed, const uint8_t* __restrict__ Eq, int H, int vocab,
                 StepState* __restrict__ st, const int32_t* __restrict__ ids, int max_seq,
                 const float* __restrict__ w, float* __restrict__ x, int ng, _Float16* __restrict__ XP,
                 float* __restrict__ XS, float* __restrict__ SQ, const float* __restrict__ rope_cos,
                 const float* __restrict__ rope_sin, int half, float* __restrict__ rope_cur, int rstride)
{
    __shared__ float red_m[2], red_s[2];
    const int c = blockIdx.x, b = blockIdx.y;
    StepState* sb = st + b;
    int pos = sb->pos;
    const bool pos_bad = pos < 0 || pos >= max_seq;
    if (pos_bad)
        pos = 0;
    int tok = ids[(size_t)b * max_seq + pos];
    const bool tok_bad = tok < 0 || tok >= vocab;
    if (tok_bad)
        tok = 0;
    if (c == 0) {
        if (threadIdx.x == 0 && (pos_bad || tok_bad))
            sb->error |= (pos_bad ? 2 : 0) | (tok_bad ? 1 : 0);
        for (int k = threadIdx.x; k < half; k += blockDim.x) {
            rope_cur[(size_t)b * rstride + k] = rope_cos[(size_t)pos * half + k];
            rope_cur[(size_t)b * rstride + half + k] = rope_sin[(size_t)pos * half + k];
        }
    }
    const int nb = H / 32;
    const int bl = threadIdx.x >> 2, kg = threadIdx.x & 3, blk = c * gbm_kcb(ng) + bl;
    const bool in = bl < gbm_kcb(ng) && blk < nb;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (in) {
        // word kg of the token's block: codes of elements 4kg.. (low nibbles) and 16+4kg.. (high)
        const size_t blkg = (size_t)tok * nb + blk;
        const uint32_t wd = *reinterpret_cast<const uint32_t*>(Eq + blkg * 16 + 4 * kg);
        const float d = f16_to_f32(Ed[blkg]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = (float)((int)((wd >> (8 * k)) & 15u) - 8) * d;
            v[4 + k] = (float)((int)((wd >> (8 * k + 4)) & 15u) - 8) * d;
        }
        float* xp = x + (size_t)b * H + (size_t)blk * 32 + 4 * kg;
        *reinterpret_cast<float4*>(xp) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(xp + 16) = make_float4(v[4], v[5], v[6], v[7]);
        const float4 wa = *reinterpret_cast<const float4*>(w + (size_t)blk * 32 + 4 * kg);
        const float4 wh = *reinterpret_cast<const float4*>(w + (size_t)blk * 32 + 16 + 4 * kg);
        const float wl[8] = {wa.x, wa.y, wa.z, wa.w, wh.x, wh.y, wh.z, wh.w};
#pragma unroll
        for (int k = 0; k < 8; ++k)
            wv[k] = wl[k];
    }
    sb_norm_chunk(v, wv, c, bl, kg, b, in, ng, XP, XS, SQ, red_m, red_s);
}

// grid (chunks of I, B), gbm_chunk_threads(ng) threads (KCB = 32 / ng blocks
// per chunk): a = silu(g) * up of
// sequence b, chunk by chunk, split for the down product into XP / XS with
// ng slot groups (gate and up rows
// interleaved; gu as nslab partial products slab floats apart, added in slab
// order)
__global__ void __launch_bounds__(128)
k_swiglu_xp_batch(const float* __restrict__ gu, int nslab, size_t slab, int I, int ng, _Float16* __restrict__ XP,
                  float* __restrict__ XS)
{
    __shared__ float red[2];
    const int c = blockIdx.x, b = blockIdx.y;
    const int bl = threadIdx.x >> 2, kg = threadIdx.x & 3, blk = c * gbm_kcb(ng) + bl;
    const bool in = bl < gbm_kcb(ng) && blk < I / 32;
    float e[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (in) {
        const float2* g2 = reinterpret_cast<const float2*>(gu + (size_t)b * 2 * I);
        float a[8];   // elements 4kg .. 4kg+3, then 16+4kg .. 16+4kg+3 of the block
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int i = blk * 32 + 4 * kg + (q < 4 ? q : 12 + q);
            const float2 v = slab_sum<4>(g2 + i, nslab, slab / 2);
            a[q] = v.x * __builtin_amdgcn_rcpf(1.0f + __expf(-v.x)) * v.y;
        }
        e[0] = a[0];
        e[1] = a[2];
        e[2] = a[1];
        e[3] = a[3];
        e[4] = a[4] * 0.0625f;
        e[5] = a[6] * 0.0625f;
        e[6] = a[5] * 0.0625f;
        e[7] = a[7] * 0.0625f;
    }
    const float s = gbm_scale_for(gbm_chunk_max(gbm_xp_absmax(e), red));
    if (in)
        gbm_xp_put(XP, ng, c, bl, kg, b, e, s);
    if (threadIdx.x == 0)
        XS[c * 16 * ng + b] = 1.0f / s;
}

// (value, index) better than (bv, bi): larger value, lowest index among equals
QD_DEV bool sb_better(float v, int32_t i, float bv, int32_t bi) { return v > bv || (v == bv && i < bi); }

// stage 1 of the greedy pick, grid (G, B), 256 threads: workgroup g of
// sequence b takes logits[b][g*chunk .. (g+1)*chunk) and writes its best
// (value, lowest index) to cand[b * G + g]
__global__ void __launch_bounds__(256)
k_argmax_batch(const float* __restrict__ logits, int V, int chunk, float* __restrict__ cval,
               int32_t* __restrict__ cidx)
{
    __shared__ float bv[4];
    __shared__ int32_t bi[4];
    const int g = blockIdx.x, b = blockIdx.y, G = gridDim.x;
    const float* lb = logits + (size_t)b * V;
    float best = -INFINITY;
    int32_t bidx = 0x7fffffff;
    const int i1 = min(V, (g + 1) * chunk);
    for (int i = g * chunk + (int)threadIdx.x; i < i1; i += blockDim.x) {
        const float v = lb[i];
        if (sb_better(v, i, best, bidx)) {
            best = v;
            bidx = i;
        }
    }
    for (int m = WAVE / 2; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(best, m, WAVE);
        const int32_t oi = __shfl_xor(bidx, m, WAVE);
        if (sb_better(ov, oi, best, bidx)) {
            best = ov;
            bidx = oi;
        }
    }
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    if (lane == 0) {
        bv[wave] = best;
        bi[wave] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w2 = 1; w2 < (int)(blockDim.x / WAVE); ++w2)
            if (sb_better(bv[w2], bi[w2], best, bidx)) {
                best = bv[w2];
                bidx = bi[w2];
            }
        cval[(size_t)b * G + g] = best;
        cidx[(size_t)b * G + g] = bidx;
    }
}

// stage 2, grid B: sequence b's greedy token from its G candidates, recorded
// and advanced as k_argmax_advance does for one sequence
__global__ void __launch_bounds__(256)
k_argmax_advance_batch(const float* __restrict__ cval, const int32_t* __restrict__ cidx, int G, int vocab,
                       StepState* __restrict__ st, int32_t* __restrict__ ids, int32_t* __restrict__ pred,
                       int max_seq)
{
    const int b = blockIdx.x;
    argmax_advance_body(cval + (size_t)b * G, cidx + (size_t)b * G, G, vocab, st + b,
                        ids + (size_t)b * max_seq, pred + (size_t)b * max_seq, max_seq);
}

}  // namespace qd
