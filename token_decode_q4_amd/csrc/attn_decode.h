// attn_decode.h -- split-KV GQA decode attention for gfx950.
//
// Computes, for every query head h of sequence b,
//   out = softmax(scale * q_h K^T) V   over keys t in [0, kv_len[b])
// with kv head g = h / (nq/nkv) (inferencelayer cuda_llm.rs page, attn_partial,
// attn_reduce and the flash-decoding arm that stages a K/V chunk once for the
// whole query group; ferrum-kernels cuda_decode.rs page, flash_decode_attention
// phase 1/2, paged_decode_attention, batched_decode_attention).
//
// Grid (nsplit, nkv, B).  A workgroup owns one (sequence, kv head, key range)
// and serves all GQ query heads of that kv head: each 64-key tile of K and V
// is copied to LDS once and read by the GQ heads from there.  Per tile:
//   1. QK: 16 lanes per key (128 dims, 8 dims a lane, one 128-bit LDS read);
//      each lane holds its 8 dims of all GQ queries in registers.
//   2. online softmax: one wave per head over the 64 keys (running max m,
//      running sum l, rescale factor for the accumulators).
//   3. PV: lanes own 2 output dims, waves own 16 keys; each V element read
//      once from LDS and used by all GQ heads.
// The workgroup writes its partial (acc[hd], m, l) per head; the last
// workgroup of a (sequence, kv head) to finish merges the partials with the
// online-softmax rule
//   M = max_s m_s,  out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s
// and resets its completion counter.
#pragma once

#include "qd_common.h"

namespace qd {

struct AttnParams {
    const float* q;            // [B][nq][HD]
    const uint16_t* k;         // paged pool [nblocks][nkv][BS][HD] or contiguous [B][nkv][max_kv][HD]
    const uint16_t* v;
    const int32_t* tables;     // [B][mbps] or nullptr (contiguous)
    int mbps;
    const int32_t* kv_lens;    // [B], or nullptr: kv_len = *pos + 1 (B == 1)
    const int32_t* pos;
    int max_kv;                // contiguous capacity per (b, g)
    int nq, nkv;
    float scale;
    int chunk;                 // keys per split, a multiple of 64
    int nsplit;
    float* part;               // [B][nq][nsplit][HD + 2]
    unsigned int* counters;    // [B][nkv]
    float* out;                // [B][nq][HD]
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
    float red[4][GQ][HD];      // cross-wave reduction of the accumulators
    bool last;
};

template <int HD, bool PAGED>
QD_DEV const uint16_t* kv_row_ptr(const AttnParams& p, const uint16_t* base, int b, int g, int t)
{
    if (PAGED) {
        const int phys = p.tables[(size_t)b * p.mbps + t / ATT_BS];
        return base + (((size_t)phys * p.nkv + g) * ATT_BS + (t % ATT_BS)) * HD;
    }
    return base + (((size_t)b * p.nkv + g) * p.max_kv + t) * HD;
}

template <int HD, int GQ, bool PAGED>
__global__ void __launch_bounds__(ATT_NT) k_attn_decode(AttnParams p)
{
    static_assert(HD == 64 || HD == 128, "head_dim");
    static_assert(GQ >= 1 && GQ <= 8, "group");
    __shared__ AttnSmem<HD, GQ> sm;
    constexpr int LPK = HD / 8;          // lanes per key in QK (8 dims each)
    constexpr int KPP = WAVE / LPK;      // keys per wave pass
    constexpr int DPL = HD / WAVE;       // output dims per lane in PV (1 or 2)

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
    int kv_len = p.kv_lens ? p.kv_lens[b] : (*p.pos + 1);
    kv_len = max(0, min(kv_len, p.max_kv));
    const int t_begin = s * p.chunk;
    const int t_end = min(kv_len, t_begin + p.chunk);
    const int h0 = g * GQ;

    // this lane's 8 query dims of every head of the group, pre-scaled
    const int part = lane % LPK;
    float qr[GQ][8];
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
        const float* qh = p.q + ((size_t)b * p.nq + h0 + j) * HD + part * 8;
        const float4 a = reinterpret_cast<const float4*>(qh)[0];
        const float4 c = reinterpret_cast<const float4*>(qh)[1];
        qr[j][0] = a.x * p.scale; qr[j][1] = a.y * p.scale; qr[j][2] = a.z * p.scale; qr[j][3] = a.w * p.scale;
        qr[j][4] = c.x * p.scale; qr[j][5] = c.y * p.scale; qr[j][6] = c.z * p.scale; qr[j][7] = c.w * p.scale;
    }
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
        // ---- K/V tile -> LDS (keys past n are zero-filled, never loaded)
        constexpr int PIECES = ATT_T * HD / 8;     // 16-byte pieces per tile
#pragma unroll
        for (int i = tid; i < PIECES; i += ATT_NT) {
            const int tk = i / (HD / 8), off = (i % (HD / 8)) * 8;
            uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
            if (tk < n) {
                kv = *reinterpret_cast<const uint4*>(kv_row_ptr<HD, PAGED>(p, p.k, b, g, t0 + tk) + off);
                vv = *reinterpret_cast<const uint4*>(kv_row_ptr<HD, PAGED>(p, p.v, b, g, t0 + tk) + off);
            }
            *reinterpret_cast<uint4*>(&sm.kt[tk * HD + off]) = kv;
            *reinterpret_cast<uint4*>(&sm.vt[tk * HD + off]) = vv;
        }
        __syncthreads();
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
            float vf[DPL];
            if (DPL == 2) {
                const uint32_t w2 = *reinterpret_cast<const uint32_t*>(&sm.vt[tk * HD + lane * 2]);
                vf[0] = f16_to_f32((uint16_t)(w2 & 0xffffu));
                vf[DPL - 1] = f16_to_f32((uint16_t)(w2 >> 16));
            } else {
                vf[0] = f16_to_f32(sm.vt[tk * HD + lane]);
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
    // ---- the last workgroup of this (b, g) merges the partials
    if (!arrive_last(p.counters + (size_t)b * p.nkv + g, (unsigned)p.nsplit, &sm.last))
        return;
    for (int i = tid; i < GQ * HD; i += ATT_NT) {
        const int j = i / HD, d = i % HD;
        const float* pp = p.part + (((size_t)b * p.nq + h0 + j) * p.nsplit) * pstride;
        float M = -INFINITY;
        for (int ss = 0; ss < p.nsplit; ++ss)
            M = fmaxf(M, pp[ss * pstride + HD]);
        float num = 0.f, den = 0.f;
        if (M != -INFINITY) {
            for (int ss = 0; ss < p.nsplit; ++ss) {
                const float ms = pp[ss * pstride + HD];
                const float w = (ms == -INFINITY) ? 0.f : expf(ms - M);
                num = fmaf(w, pp[ss * pstride + d], num);
                den = fmaf(w, pp[ss * pstride + HD + 1], den);
            }
        }
        p.out[((size_t)b * p.nq + h0 + j) * HD + d] = (den > 0.f) ? num / den : 0.f;
    }
    reset_counter(p.counters + (size_t)b * p.nkv + g);
}

// Split policy: about 4 workgroups per CU over all (sequence, kv head) pairs,
// at least one 64-key tile per split.
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
