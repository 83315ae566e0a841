// attn_decode.h -- split-KV GQA decode attention for gfx950.
//
// Computes, for every query head h of sequence b,
//   out = softmax(scale * q_h K^T) V   over keys t in [0, kv_len[b])
// with kv head g = h / (nq/nkv) (inferencelayer cuda_llm.rs page, attn_partial,
// attn_reduce and the flash-decoding arm that stages a K/V chunk once for the
// whole query group; ferrum-kernels cuda_decode.rs page, flash_decode_attention
// phase 1/2, paged_decode_attention, batched_decode_attention).
//
// k_attn_split: grid (nsplit, nkv, B).  A workgroup owns one (sequence, kv
// head, key range) and serves all GQ query heads of that kv head: each 64-key
// tile of K and V is copied to LDS once and read by the GQ heads from there.
// Per tile:
//   1. QK: 16 lanes per key (128 dims, 8 dims a lane, one 128-bit LDS read);
//      each lane holds its 8 dims of all GQ queries in registers.
//   2. online softmax: one wave per head over the 64 keys (running max m,
//      running sum l, rescale factor for the accumulators).
//   3. PV: lanes own 2 output dims, waves own 16 keys; each V element read
//      once from LDS and used by all GQ heads.
// It writes its partial (acc[hd], m, l) per head.  k_attn_combine (grid
// (nq, B)) merges a head's partials with the online-softmax rule
//   M = max_s m_s,  out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s.
//
// In the decode step the split kernel also finishes the projection: it reads
// the raw q|k|v of the token, applies the per-head q/k RMSNorm and the NeoX
// rotary at the position (ferrum-kernels cuda_decode.rs page, the q/k norm
// then rope order of decode_step), and the one workgroup whose key range holds
// the position stores the token's K and V (f16) in the cache and in its tile.
#pragma once

#include "qd_common.h"

namespace qd {

struct AttnParams {
    const float* q;            // [B][nq][HD] (standalone) or raw q|k|v of the step
    const uint16_t* k;         // paged pool [nblocks][nkv][BS][HD] or contiguous [B][nkv][max_kv][HD]
    const uint16_t* v;
    const int32_t* tables;     // [B][mbps] or nullptr (contiguous)
    int mbps;
    const int32_t* kv_lens;    // [B], or nullptr: kv_len = *pos + 1 (B == 1)
    const int32_t* pos;
    int max_kv;                // contiguous capacity per (b, g); bound on kv_len
    int nq, nkv;
    float scale;
    int chunk;                 // keys per split, a multiple of 64
    int nsplit;
    float* part;               // [B][nq][nsplit][HD + 2]
    float* out;                // [B][nq][HD] (combine)
    // decode-step prologue (QMODE 1)
    const float* q_norm;       // [HD] or nullptr (no q/k norm)
    const float* k_norm;
    float eps;
    int rot;
    const float* rope_cos;     // [max_kv][rot/2]
    const float* rope_sin;
    uint16_t* kc;              // cache written at pos (same buffers as k/v)
    uint16_t* vc;
};

constexpr int ATT_T = 64;      // keys per LDS tile
constexpr int ATT_BS = 16;     // paged block size
constexpr int ATT_NT = 256;    // threads per workgroup

template <int HD, int GQ>
struct AttnSmem {
    uint16_t kt[ATT_T * HD];
    uint16_t vt[ATT_T * HD];
    float sc[GQ][ATT_T];       // scores, then probabilities
    float m[GQ], l[GQ], alpha[GQ];
    float qv[GQ + 1][HD];      // prologue: q heads (+ the token's k)
    float red[4][GQ][HD];      // cross-wave reduction of the accumulators
    float ss[GQ + 1];
};

template <int HD, bool PAGED>
QD_DEV size_t kv_offset(const AttnParams& p, int phys_or_b, int g, int t)
{
    if (PAGED)
        return (((size_t)phys_or_b * p.nkv + g) * ATT_BS + (t % ATT_BS)) * HD;
    return (((size_t)phys_or_b * p.nkv + g) * p.max_kv + t) * HD;
}

// QMODE 0: q given (standalone); QMODE 1: decode-step prologue from raw q|k|v
template <int HD, int GQ, bool PAGED, int QMODE>
__global__ void __launch_bounds__(ATT_NT) k_attn_split(AttnParams p)
{
    static_assert(HD == 64 || HD == 128, "head_dim");
    static_assert(GQ >= 1 && GQ <= 8, "group");
    __shared__ AttnSmem<HD, GQ> sm;
    constexpr int LPK = HD / 8;          // lanes per key in QK (8 dims each)
    constexpr int KPP = WAVE / LPK;      // keys per wave pass
    constexpr int DPL = HD / WAVE;       // output dims per lane in PV (1 or 2)
    constexpr int PIECES = ATT_T * HD / 8;      // 16-byte pieces per K (or V) tile
    constexpr int PPT = PIECES / ATT_NT;        // pieces per thread (2 or 4)
    constexpr int MAXIT = ((GQ + 1) * HD + ATT_NT - 1) / ATT_NT;

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
    int kv_len = p.kv_lens ? p.kv_lens[b] : (*p.pos + 1);
    kv_len = max(0, min(kv_len, p.max_kv));
    const int t_begin = s * p.chunk;
    const int t_end = min(kv_len, t_begin + p.chunk);
    const int h0 = g * GQ;
    const int cur = kv_len - 1;                       // the step's own position (QMODE 1)
    const bool owner = QMODE == 1 && cur >= t_begin && cur < t_end;
    if (t_begin >= t_end)
        return;   // key range past kv_len: the combine reads only active splits

    // ---- every prologue load first: queries (and the token's k, v), rotary
    // factors and norm weights of this thread's elements
    const int nrows = owner ? GQ + 1 : GQ;
    const int half = p.rot / 2;
    float qe[MAXIT], ce[MAXIT], se[MAXIT], we[MAXIT];
    float vtok = 0.f;
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
        const int i = tid + it * ATT_NT;
        qe[it] = 0.f;
        ce[it] = 1.f;
        se[it] = 0.f;
        we[it] = 1.f;
        if (i < nrows * HD) {
            const int j = i / HD, d = i % HD;
            if (QMODE == 0) {
                qe[it] = p.q[((size_t)b * p.nq + h0) * HD + i];
            } else {
                qe[it] = (j < GQ) ? p.q[(size_t)(h0 + j) * HD + d] : p.q[((size_t)p.nq + g) * HD + d];
                if (d < p.rot) {
                    const int ii = d < half ? d : d - half;
                    ce[it] = p.rope_cos[(size_t)cur * half + ii];
                    se[it] = p.rope_sin[(size_t)cur * half + ii];
                }
                if (p.q_norm)
                    we[it] = (j == GQ) ? p.k_norm[d] : p.q_norm[d];
            }
        }
    }
    if (owner && tid < HD)
        vtok = p.q[((size_t)p.nq + p.nkv + g) * HD + tid];

    // ---- first tile's K/V loads
    uint4 kr[PPT], vr[PPT];
    auto load_tile = [&](int t0, int n) {
        int phys[ATT_T / ATT_BS];
#pragma unroll
        for (int k = 0; k < ATT_T / ATT_BS; ++k) {
            if (PAGED)
                phys[k] = (k * ATT_BS < n) ? p.tables[(size_t)b * p.mbps + t0 / ATT_BS + k] : 0;
            else
                phys[k] = b;
        }
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            const int i = tid + u * ATT_NT;
            const int tk = i / (HD / 8), off = (i % (HD / 8)) * 8;
            kr[u] = make_uint4(0, 0, 0, 0);
            vr[u] = make_uint4(0, 0, 0, 0);
            if (tk < n) {
                const size_t o = kv_offset<HD, PAGED>(p, phys[tk / ATT_BS], g, t0 + tk) + off;
                kr[u] = *reinterpret_cast<const uint4*>(p.k + o);
                vr[u] = *reinterpret_cast<const uint4*>(p.v + o);
            }
        }
    };
    load_tile(t_begin, min(ATT_T, t_end - t_begin));

    // ---- queries into LDS; per-head q/k RMSNorm and NeoX rotary (QMODE 1)
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
        const int i = tid + it * ATT_NT;
        if (i < nrows * HD)
            sm.qv[i / HD][i % HD] = qe[it];
    }
    __syncthreads();
    if (QMODE == 1) {
        if (p.q_norm) {
            for (int j = wave; j < nrows; j += ATT_NT / WAVE) {
                float ss = 0.f;
                for (int d = lane; d < HD; d += WAVE)
                    ss += sm.qv[j][d] * sm.qv[j][d];
                ss = group_sum<WAVE>(ss);
                if (lane == 0)
                    sm.ss[j] = 1.0f / sqrtf(ss / (float)HD + p.eps);
            }
            __syncthreads();
#pragma unroll
            for (int it = 0; it < MAXIT; ++it) {
                const int i = tid + it * ATT_NT;
                if (i < nrows * HD) {
                    qe[it] = qe[it] * sm.ss[i / HD] * we[it];
                    sm.qv[i / HD][i % HD] = qe[it];
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int it = 0; it < MAXIT; ++it) {
            const int i = tid + it * ATT_NT;
            if (i < nrows * HD) {
                const int j = i / HD, d = i % HD;
                if (d < p.rot)
                    qe[it] = d < half ? qe[it] * ce[it] - sm.qv[j][d + half] * se[it]
                                      : sm.qv[j][d - half] * se[it] + qe[it] * ce[it];
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < MAXIT; ++it) {
            const int i = tid + it * ATT_NT;
            if (i < nrows * HD)
                sm.qv[i / HD][i % HD] = qe[it];
        }
        __syncthreads();
        if (owner) {
            // the token's K and V, rounded to f16 once: cache and tile get the same values
            size_t o;
            if (PAGED) {
                const int phys = p.tables[(size_t)b * p.mbps + cur / ATT_BS];
                o = kv_offset<HD, PAGED>(p, phys, g, cur);
            } else {
                o = kv_offset<HD, PAGED>(p, b, g, cur);
            }
            if (tid < HD) {
                const uint16_t kh = f32_to_f16(sm.qv[GQ][tid]);
                const uint16_t vh = f32_to_f16(vtok);
                p.kc[o + tid] = kh;
                p.vc[o + tid] = vh;
                sm.qv[GQ][tid] = __uint_as_float(((uint32_t)vh << 16) | kh);   // stash for the tile
            }
        }
    }
    const int part = lane % LPK;
    float qr[GQ][8];
#pragma unroll
    for (int j = 0; j < GQ; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            qr[j][e] = sm.qv[j][part * 8 + e] * p.scale;
    if (tid < GQ) {
        sm.m[tid] = -INFINITY;
        sm.l[tid] = 0.f;
    }
    float acc[GQ][DPL];
#pragma unroll
    for (int j = 0; j < GQ; ++j)
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            acc[j][e] = 0.f;

    for (int t0 = t_begin; t0 < t_end; t0 += ATT_T) {
        const int n = min(ATT_T, t_end - t0);
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            const int i = tid + u * ATT_NT;
            const int tk = i / (HD / 8), off = (i % (HD / 8)) * 8;
            *reinterpret_cast<uint4*>(&sm.kt[tk * HD + off]) = kr[u];
            *reinterpret_cast<uint4*>(&sm.vt[tk * HD + off]) = vr[u];
        }
        __syncthreads();
        // the next tile's loads fly while this one is consumed
        if (t0 + ATT_T < t_end)
            load_tile(t0 + ATT_T, min(ATT_T, t_end - t0 - ATT_T));
        if (owner && cur >= t0 && cur < t0 + n) {
            const int slot = cur - t0;
            for (int d = tid; d < HD; d += ATT_NT) {
                const uint32_t kv = __float_as_uint(sm.qv[GQ][d]);
                sm.kt[slot * HD + d] = (uint16_t)(kv & 0xffffu);
                sm.vt[slot * HD + d] = (uint16_t)(kv >> 16);
            }
            __syncthreads();
        }
        // ---- QK
#pragma unroll
        for (int pass = 0; pass < (ATT_T / 4) / KPP; ++pass) {
            const int tk = wave * (ATT_T / 4) + pass * KPP + lane / LPK;
            const uint4 kraw = *reinterpret_cast<const uint4*>(&sm.kt[tk * HD + part * 8]);
            const uint32_t kw[4] = {kraw.x, kraw.y, kraw.z, kraw.w};
            float kf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[2 * e] = f16_to_f32((uint16_t)(kw[e] & 0xffffu));
                kf[2 * e + 1] = f16_to_f32((uint16_t)(kw[e] >> 16));
            }
#pragma unroll
            for (int j = 0; j < GQ; ++j) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    d = fmaf(qr[j][e], kf[e], d);
                d = group_sum<LPK>(d);
                if (part == 0)
                    sm.sc[j][tk] = tk < n ? d : -INFINITY;
            }
        }
        __syncthreads();
        // ---- online softmax, one wave per head
        for (int j = wave; j < GQ; j += ATT_NT / WAVE) {
            const float sv = sm.sc[j][lane];
            const float mold = sm.m[j];
            const float mnew = fmaxf(mold, group_max<WAVE>(sv));
            const float pr = (lane < n) ? expf(sv - mnew) : 0.f;
            const float ps = group_sum<WAVE>(pr);
            const float al = expf(mold - mnew);   // 0 on the first tile (mold = -inf)
            sm.sc[j][lane] = pr;
            __builtin_amdgcn_wave_barrier();
            if (lane == 0) {
                sm.m[j] = mnew;
                sm.l[j] = sm.l[j] * al + ps;
                sm.alpha[j] = al;
            }
        }
        __syncthreads();
        // ---- PV
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
            const float al = sm.alpha[j];
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                acc[j][e] *= al;
        }
        for (int i = 0; i < ATT_T / 4; ++i) {
            const int tk = wave * (ATT_T / 4) + i;
            float vf[2];
            if (DPL == 2) {
                const uint32_t w2 = *reinterpret_cast<const uint32_t*>(&sm.vt[tk * HD + lane * 2]);
                vf[0] = f16_to_f32((uint16_t)(w2 & 0xffffu));
                vf[1] = f16_to_f32((uint16_t)(w2 >> 16));
            } else {
                vf[0] = f16_to_f32(sm.vt[tk * HD + lane]);
                vf[1] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < GQ; ++j) {
                const float pj = sm.sc[j][tk];
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    acc[j][e] = fmaf(pj, vf[e], acc[j][e]);
            }
        }
        __syncthreads();
    }

    // ---- cross-wave reduction of the accumulators, partial write
#pragma unroll
    for (int j = 0; j < GQ; ++j)
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            sm.red[wave][j][lane * DPL + e] = acc[j][e];
    __syncthreads();
    const size_t pstride = HD + 2;
    for (int i = tid; i < GQ * HD; i += ATT_NT) {
        const int j = i / HD, d = i % HD;
        const float v = (sm.red[0][j][d] + sm.red[1][j][d]) + (sm.red[2][j][d] + sm.red[3][j][d]);
        float* pp = p.part + (((size_t)b * p.nq + h0 + j) * p.nsplit + s) * pstride;
        pp[d] = v;
        if (d == 0) {
            pp[HD] = sm.m[j];
            pp[HD + 1] = sm.l[j];
        }
    }
}

constexpr int ATT_CNT = 512;   // combine threads per head

QD_DEV float block_reduce_max512(float v, float* red)
{
    v = group_max<WAVE>(v);
    if ((threadIdx.x & (WAVE - 1)) == 0)
        red[threadIdx.x / WAVE] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < ATT_CNT / WAVE; ++i)
        r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

QD_DEV float block_reduce_sum512(float v, float* red)
{
    v = group_sum<WAVE>(v);
    if ((threadIdx.x & (WAVE - 1)) == 0)
        red[threadIdx.x / WAVE] = v;
    __syncthreads();
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < ATT_CNT / WAVE; ++i)
        r += red[i];
    __syncthreads();
    return r;
}

// Merge the partials of one (sequence, head): grid (nq, B), 512 threads.  Only
// the splits holding keys below kv_len were written; the others are skipped.
// Round 1 loads every split's (m, l); round 2 the accumulators, split among
// 512 / HD thread groups, each thread's loads issued together.
template <int HD>
__global__ void __launch_bounds__(ATT_CNT) k_attn_combine(const float* __restrict__ part,
                                                          int nsplit_all, int chunk,
                                                          const int32_t* __restrict__ kv_lens,
                                                          const int32_t* __restrict__ pos,
                                                          int max_kv, int nq, float* __restrict__ out)
{
    constexpr int SG = ATT_CNT / HD;
    extern __shared__ float wsh[];          // [nsplit] weights
    __shared__ float red[ATT_CNT / WAVE];
    __shared__ float numsh[SG][HD];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const size_t pstride = HD + 2;
    const float* pp = part + ((size_t)b * nq + h) * nsplit_all * pstride;
    int kv_len = kv_lens ? kv_lens[b] : (*pos + 1);
    kv_len = max(0, min(kv_len, max_kv));
    const int nsplit = min(nsplit_all, (kv_len + chunk - 1) / chunk);
    float mloc = -INFINITY;
    for (int s = tid; s < nsplit; s += ATT_CNT) {
        const float m = pp[s * pstride + HD];
        wsh[s] = m;
        mloc = fmaxf(mloc, m);
    }
    const float M = block_reduce_max512(mloc, red);
    float dloc = 0.f;
    for (int s = tid; s < nsplit; s += ATT_CNT) {
        const float m = wsh[s];
        const float e = (m == -INFINITY || M == -INFINITY) ? 0.f : expf(m - M);
        wsh[s] = e;
        dloc = fmaf(e, pp[s * pstride + HD + 1], dloc);
    }
    const float den = block_reduce_sum512(dloc, red);   // its barriers publish wsh
    const int d = tid % HD, sg = tid / HD;
    float num = 0.f;
    for (int s0 = sg; s0 < nsplit; s0 += 16 * SG) {
        float a[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int s = s0 + u * SG;
            a[u] = (s < nsplit) ? pp[s * pstride + d] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int s = s0 + u * SG;
            if (s < nsplit)
                num = fmaf(wsh[s], a[u], num);
        }
    }
    numsh[sg][d] = num;
    __syncthreads();
    if (sg == 0) {
        float t = numsh[0][d];
#pragma unroll
        for (int k = 1; k < SG; ++k)
            t += numsh[k][d];
        out[((size_t)b * nq + h) * HD + d] = (den > 0.f) ? t / den : 0.f;
    }
}

// Split policy of the standalone entry: about 4 workgroups per CU over all
// (sequence, kv head) pairs, at least one 64-key tile per split.
inline void attn_split(int B, int nkv, int max_kv, int* chunk, int* nsplit)
{
    const int tiles = max(1, (max_kv + ATT_T - 1) / ATT_T);
    int want = (1024 + B * nkv - 1) / (B * nkv);
    if (want < 1) want = 1;
    if (want > tiles) want = tiles;
    const int tiles_per = (tiles + want - 1) / want;
    *chunk = tiles_per * ATT_T;
    *nsplit = (max(1, max_kv) + *chunk - 1) / *chunk;
}

}  // namespace qd
