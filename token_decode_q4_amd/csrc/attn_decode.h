// attn_decode.h -- split-KV GQA decode attention for gfx950.
//
// Computes, for every query head h of sequence b,
//   out = softmax(scale * q_h K^T) V   over keys t in [0, kv_len[b])
// with kv head g = h / (nq/nkv) (inferencelayer cuda_llm.rs page, attn_partial,
// attn_reduce and the flash-decoding arm that reads a K/V chunk once for the
// whole query group; ferrum-kernels cuda_decode.rs page, flash_decode_attention
// phase 1/2, paged_decode_attention, batched_decode_attention).
//
// k_attn_split: grid (nsplit, nkv, B), 4 waves.  A workgroup owns one
// (sequence, kv head, key range) and serves all GQ query heads of that kv
// head.  Each wave works on its own 16-key steps (one paged block) with no
// workgroup barrier until the end:
//   QK   lane (key k = lane/4, quarter c = lane%4) holds 8 dims of K[k] in each
//        32-dim slice (dims 32i + 8c .. +7), reads the matching query dims from
//        LDS and reduces the 4 quarters with two shuffles;
//   softmax  per head over the 16 keys (shuffles across the key lanes), online
//        across the wave's steps (running max m, sum l, rescale of acc);
//   PV   lane owns HD/64 output dims; the step's probabilities go through a
//        small per-wave LDS table [key][head]; V is loaded in that layout.
// The four waves' (m, l, acc) are merged once through LDS and written as the
// workgroup's partial.  k_attn_combine (grid (nq, B)) merges a head's partials:
//   M = max_s m_s,  out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s.
//
// In the decode step (QMODE 1) the split kernel also finishes the projection:
// from the raw q|k|v of the token it applies the per-head q/k RMSNorm and the
// NeoX rotary at the position (ferrum-kernels cuda_decode.rs page, the q/k
// norm then rope order of decode_step), and the wave whose keys hold the
// position stores the token's K and V (f16) in the cache and uses the same f16
// values.  There the block table covers every position below max_kv, so the
// first step's table entry and K/V loads are issued before the position is
// known; keys at or past kv_len are masked (score -inf, V taken as 0).
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
    int chunk;                 // keys per split, a multiple of 16 * waves per workgroup
    int nsplit;
    float* part;               // [B][nq][nsplit][HD + 2]
    float* out;                // [B][nq][HD] (combine)
    // decode-step prologue (QMODE 1)
    int qk_norm;               // 1: per-head RMSNorm of q and k
    const float* q_norm;       // [HD] (valid even when qk_norm is 0)
    const float* k_norm;
    float eps;
    int rot;
    const float* rope_cur;     // cos [rot/2] then sin [rot/2] at the step's position
    uint16_t* kc;              // cache written at pos (same buffers as k/v)
    uint16_t* vc;
};

constexpr int ATT_WK = 16;                 // keys per wave step (one paged block)
constexpr int ATT_BS = 16;                 // paged block size

// Waves per workgroup: a launch parameter (blockDim.x / 64) up to ATT_MAXW;
// the host sizes the grid so that it fits the chip in one round.
template <int GQ>
struct AttnMaxWaves {
    static constexpr int value = GQ <= 4 ? 8 : 4;   // keeps the LDS below 64 KB
};

template <int HD, int GQ>
struct alignas(16) AttnSmem {
    static constexpr int W = AttnMaxWaves<GQ>::value;
    float q[W][GQ][HD];             // per wave: queries ready for QK (times scale)
    float krow[W][HD];              // per wave: the token's k during its rotary
    float p[W][ATT_WK][GQ];         // per wave: probabilities of the step, [key][head]
    uint16_t knew[W][HD];           // per wave: the token's k in f16
    float m[W][GQ], l[W][GQ];
    float acc[W][GQ][HD];
};

// LDS writes of this wave are seen by its later LDS reads (no workgroup barrier)
QD_DEV void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int HD, bool PAGED>
QD_DEV size_t kv_row(const AttnParams& p, int phys_or_b, int g, int t)
{
    if (PAGED)
        return (((size_t)phys_or_b * p.nkv + g) * ATT_BS + (t % ATT_BS)) * HD;
    return (((size_t)phys_or_b * p.nkv + g) * p.max_kv + t) * HD;
}

// registers of one wave step: K in the QK layout, V in the PV layout
template <int HD>
struct AttnStep {
    static constexpr int NI = HD / 32;     // 32-dim slices
    static constexpr int DPL = HD / WAVE;  // output dims per lane
    uint4 k[NI];
    uint32_t v[ATT_WK];                    // DPL f16 of key kk in the low (and high) half
};

// QMODE 0: q given (standalone); QMODE 1: decode-step prologue from raw q|k|v
template <int HD, int GQ, bool PAGED, int QMODE>
__global__ void __launch_bounds__(AttnMaxWaves<GQ>::value * WAVE) k_attn_split(AttnParams p)
{
    static_assert(HD == 64 || HD == 128, "head_dim");
    static_assert(GQ == 1 || GQ == 2 || GQ == 4 || GQ == 8, "group");
    __shared__ AttnSmem<HD, GQ> sm;
    using Step = AttnStep<HD>;
    constexpr int NI = Step::NI, DPL = Step::DPL;

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int nw = blockDim.x / WAVE;          // waves of this launch
    const int wstride = nw * ATT_WK;           // keys between a wave's steps
    const int kk = lane >> 2, cq = lane & 3;   // QK layout: key, quarter
    const int h0 = g * GQ;
    const int t_begin = s * p.chunk;
    QD_MARK(0);

    // loads of one wave step at key tw, any tw: rows and table entries are
    // clamped into range (never a branch around a load); rows past kv_len are
    // masked where they are used
    auto load_step = [&](Step& st, int tw) {
        const int twc = min(tw, p.max_kv - 1);
        const uint16_t *kp, *vp;
        if (PAGED) {
            const int phys = max(0, p.tables[(size_t)b * p.mbps + twc / ATT_BS]);
            const size_t base = kv_row<HD, PAGED>(p, phys, g, twc & ~(ATT_BS - 1));
            kp = p.k + base + (size_t)kk * HD;
            vp = p.v + base;
        } else {
            kp = p.k + kv_row<HD, PAGED>(p, b, g, min(tw + kk, p.max_kv - 1));
            vp = p.v + kv_row<HD, PAGED>(p, b, g, 0);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
            st.k[i] = *reinterpret_cast<const uint4*>(kp + 8 * cq + 32 * i);
#pragma unroll
        for (int j = 0; j < ATT_WK; ++j) {
            const uint16_t* r = PAGED ? vp + (size_t)j * HD
                                      : vp + (size_t)min(tw + j, p.max_kv - 1) * HD;
            if (DPL == 2)
                st.v[j] = *reinterpret_cast<const uint32_t*>(r + lane * DPL);
            else
                st.v[j] = r[lane * DPL];
        }
    };

    // kv_len first (vector loads return in order): the loads below do not need it
    int kv_len = p.kv_lens ? p.kv_lens[b] : (*p.pos + 1);

    // ---- loads that do not need kv_len: the token's q|k|v, norm weights,
    // rotary factors, and (decode step) the first step's K/V
    float qv[GQ][DPL], kv_[DPL], vv[DPL], wq[DPL], wk[DPL], cs[DPL], sn[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        const int d = lane * DPL + e;
#pragma unroll
        for (int j = 0; j < GQ; ++j)
            qv[j][e] = (QMODE == 0) ? p.q[((size_t)b * p.nq + h0 + j) * HD + d]
                                    : p.q[(size_t)(h0 + j) * HD + d];
        kv_[e] = vv[e] = 0.f;
        wq[e] = wk[e] = cs[e] = 1.f;
        sn[e] = 0.f;
        if (QMODE == 1) {
            // q_norm / k_norm / rope_cur always point at valid arrays here
            kv_[e] = p.q[((size_t)p.nq + g) * HD + d];
            vv[e] = p.q[((size_t)p.nq + p.nkv + g) * HD + d];
            wq[e] = p.q_norm[d];
            wk[e] = p.k_norm[d];
            const int half = p.rot / 2;
            const int ii = d < half ? d : (d < p.rot ? d - half : 0);
            const float c0 = p.rope_cur[ii], s0 = p.rope_cur[half + ii];
            cs[e] = d < p.rot ? c0 : 1.f;
            sn[e] = d < p.rot ? s0 : 0.f;
        }
    }
    Step cur_st;
    const int tw0 = t_begin + w * ATT_WK;
    load_step(cur_st, tw0);

    kv_len = max(0, min(kv_len, p.max_kv));
    if (kv_len >= 0)
        QD_MARK(1);
    const int t_end = min(kv_len, t_begin + p.chunk);
    if (t_begin >= t_end)
        return;   // key range past kv_len: the combine reads only active splits
    const int tcur = kv_len - 1;   // the step's own position (QMODE 1)

    // ---- queries: per-head RMSNorm and rotary (QMODE 1), times scale, into
    // this wave's LDS rows; the wave holding tcur also prepares the token's K/V
    // the owner: the wave whose step own_tw holds tcur, at row slot of it
    float vnew[DPL];
    const int rel = tcur - t_begin;
    const bool owner = QMODE == 1 && tcur >= t_begin && tcur < t_end && (rel / ATT_WK) % nw == w;
    const int own_tw = t_begin + (rel / ATT_WK) * ATT_WK;
    const int slot = tcur - own_tw;
    if (QMODE == 1) {
        const float* nq_w = wq;
        if (p.qk_norm) {
#pragma unroll
            for (int j = 0; j < GQ; ++j) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    ss = fmaf(qv[j][e], qv[j][e], ss);
                ss = group_sum<WAVE>(ss);
                const float r = 1.0f / sqrtf(ss / (float)HD + p.eps);
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    qv[j][e] = qv[j][e] * r * nq_w[e];
            }
            if (owner) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    ss = fmaf(kv_[e], kv_[e], ss);
                ss = group_sum<WAVE>(ss);
                const float r = 1.0f / sqrtf(ss / (float)HD + p.eps);
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    kv_[e] = kv_[e] * r * wk[e];
            }
        }
        // rotary: the partner of dim d is d +- rot/2, read from LDS
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
#pragma unroll
            for (int j = 0; j < GQ; ++j)
                sm.q[w][j][lane * DPL + e] = qv[j][e];
            sm.krow[w][lane * DPL + e] = kv_[e];
        }
        wave_lds_sync();
        const int half = p.rot / 2;
        float qpart[GQ][DPL], kpart[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            const int d = lane * DPL + e;
            const int pd = d < half ? d + half : d - half;
            const bool rd = d < p.rot;
#pragma unroll
            for (int j = 0; j < GQ; ++j)
                qpart[j][e] = rd ? sm.q[w][j][pd] : 0.f;
            kpart[e] = rd ? sm.krow[w][pd] : 0.f;
        }
        wave_lds_sync();   // every partner read done before the rows change
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            const int d = lane * DPL + e;
            if (d < p.rot) {
                const float sg = d < half ? -sn[e] : sn[e];
#pragma unroll
                for (int j = 0; j < GQ; ++j)
                    qv[j][e] = fmaf(qpart[j][e], sg, qv[j][e] * cs[e]);
                kv_[e] = fmaf(kpart[e], sg, kv_[e] * cs[e]);
            }
        }
        if (owner) {
            size_t o;
            if (PAGED)
                o = kv_row<HD, PAGED>(p, p.tables[(size_t)b * p.mbps + tcur / ATT_BS], g, tcur);
            else
                o = kv_row<HD, PAGED>(p, b, g, tcur);
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                const int d = lane * DPL + e;
                const uint16_t kh = f32_to_f16(kv_[e]);
                const uint16_t vh = f32_to_f16(vv[e]);
                p.kc[o + d] = kh;
                p.vc[o + d] = vh;
                sm.knew[w][d] = kh;
                vnew[e] = f16_to_f32(vh);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e)
#pragma unroll
        for (int j = 0; j < GQ; ++j)
            sm.q[w][j][lane * DPL + e] = qv[j][e] * p.scale;
    wave_lds_sync();
    QD_MARK(2);

    // ---- the wave's steps
    float m[GQ], l[GQ], acc[GQ][DPL];
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            acc[j][e] = 0.f;
    }
    for (int tw = tw0; tw < t_end; tw += wstride) {
        Step nxt;
        const bool more = tw + wstride < t_end;
        if (more)
            load_step(nxt, tw + wstride);
        const int nvalid = min(ATT_WK, t_end - tw);
        const bool own_here = owner && tw == own_tw;
        // QK: 8 dims x NI slices of key kk
        float kf[NI][8];
        uint4 kr[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i)
            kr[i] = cur_st.k[i];
        if (own_here && kk == slot) {
#pragma unroll
            for (int i = 0; i < NI; ++i)
                kr[i] = *reinterpret_cast<const uint4*>(&sm.knew[w][32 * i + 8 * cq]);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[i][2 * e] = f16_to_f32((uint16_t)(kw[e] & 0xffffu));
                kf[i][2 * e + 1] = f16_to_f32((uint16_t)(kw[e] >> 16));
            }
        }
        const bool kvalid = kk < nvalid;
        QD_MARK(4);
        float sc[GQ];
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const float4 qa = *reinterpret_cast<const float4*>(&sm.q[w][j][32 * i + 8 * cq]);
                const float4 qb = *reinterpret_cast<const float4*>(&sm.q[w][j][32 * i + 8 * cq + 4]);
                d = fmaf(qa.x, kf[i][0], d);
                d = fmaf(qa.y, kf[i][1], d);
                d = fmaf(qa.z, kf[i][2], d);
                d = fmaf(qa.w, kf[i][3], d);
                d = fmaf(qb.x, kf[i][4], d);
                d = fmaf(qb.y, kf[i][5], d);
                d = fmaf(qb.z, kf[i][6], d);
                d = fmaf(qb.w, kf[i][7], d);
            }
            d = group_sum<4>(d);   // the 4 quarters of key kk
            sc[j] = kvalid ? d : -INFINITY;
        }
        QD_MARK(5);
        // online softmax over the step's keys: the 4 lanes of a key hold the
        // same score, so the max runs over the whole wave and the sum over
        // the quarter-0 lanes (the others add zeros)
        float alpha[GQ];
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
            const float mnew = fmaxf(m[j], group_max<WAVE>(sc[j]));
            const float pr = expf(sc[j] - mnew);
            const float ps = group_sum<WAVE>(cq == 0 ? pr : 0.f);
            alpha[j] = expf(m[j] - mnew);   // 0 on the first step (m = -inf)
            l[j] = fmaf(l[j], alpha[j], ps);
            m[j] = mnew;
            if (cq == 0)
                sm.p[w][kk][j] = pr;
        }
        wave_lds_sync();
        QD_MARK(6);
        // PV: lane owns dims lane*DPL ..
#pragma unroll
        for (int j = 0; j < GQ; ++j)
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                acc[j][e] *= alpha[j];
#pragma unroll
        for (int t = 0; t < ATT_WK; ++t) {
            float vf[DPL];
            const uint32_t vw = cur_st.v[t];
            vf[0] = f16_to_f32((uint16_t)(vw & 0xffffu));
            if (DPL == 2)
                vf[DPL - 1] = f16_to_f32((uint16_t)(vw >> 16));
            if (own_here && t == slot) {
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    vf[e] = vnew[e];
            }
            const bool tv = t < nvalid;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                vf[e] = tv ? vf[e] : 0.f;
            float pt[GQ];
#pragma unroll
            for (int j = 0; j < GQ; ++j)
                pt[j] = sm.p[w][t][j];
#pragma unroll
            for (int j = 0; j < GQ; ++j)
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    acc[j][e] = fmaf(pt[j], vf[e], acc[j][e]);
        }
        wave_lds_sync();   // the p table is rewritten by the next step
        if (more)
            cur_st = nxt;
    }

    // ---- merge the waves, write the workgroup's partial
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
        if (lane == 0) {
            sm.m[w][j] = m[j];
            sm.l[w][j] = l[j];
        }
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            sm.acc[w][j][lane * DPL + e] = acc[j][e];
    }
    QD_MARK(7);
    __syncthreads();
    const size_t pstride = HD + 2;
    for (int i = tid; i < GQ * HD; i += nw * WAVE) {
        const int j = i / HD, d = i % HD;
        float M = sm.m[0][j];
        for (int u = 1; u < nw; ++u)
            M = fmaxf(M, sm.m[u][j]);
        float L = 0.f, A = 0.f;
        for (int u = 0; u < nw; ++u) {
            const float mu = sm.m[u][j];
            const float f = (mu == -INFINITY) ? 0.f : expf(mu - M);
            L = fmaf(f, sm.l[u][j], L);
            A = fmaf(f, sm.acc[u][j][d], A);
        }
        float* pp = p.part + (((size_t)b * p.nq + h0 + j) * p.nsplit + s) * pstride;
        pp[d] = A;
        if (d == 0) {
            pp[HD] = M;
            pp[HD + 1] = L;
        }
    }
    QD_MARK(3);
}

constexpr int ATT_CNT = 512;   // combine threads per head

// Merge the partials of one (sequence, head): grid (nq, B), 512 threads in
// groups of HD; group sg takes splits sg, sg + SG, ...  Each round issues all
// of its loads (acc, m, l of up to 16 splits) before using them; only splits
// holding keys below kv_len count.  The groups' (max, numerator, denominator)
// are merged through LDS in a fixed order.
template <int HD>
__global__ void __launch_bounds__(ATT_CNT) k_attn_combine(const float* __restrict__ part,
                                                          int nsplit_all, int chunk,
                                                          const int32_t* __restrict__ kv_lens,
                                                          const int32_t* __restrict__ pos,
                                                          int max_kv, int nq, float* __restrict__ out)
{
    constexpr int SG = ATT_CNT / HD;
    constexpr int U = 16;
    __shared__ float gm[SG][HD], gn[SG][HD], gd[SG][HD];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int d = tid % HD, sg = tid / HD;
    const size_t pstride = HD + 2;
    const float* pp = part + ((size_t)b * nq + h) * nsplit_all * pstride;
    QD_MARK(0);
    float mt = -INFINITY, num = 0.f, den = 0.f;
    int nact = -1;
    for (int s0 = sg; s0 < nsplit_all; s0 += U * SG) {
        float a[U], mm[U], ll[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t sp = (size_t)min(s0 + u * SG, nsplit_all - 1) * pstride;   // never a branch
            a[u] = pp[sp + d];
            mm[u] = pp[sp + HD];
            ll[u] = pp[sp + HD + 1];
        }
        if (nact < 0) {
            int kv_len = kv_lens ? kv_lens[b] : (*pos + 1);
            kv_len = max(0, min(kv_len, max_kv));
            nact = min(nsplit_all, (kv_len + chunk - 1) / chunk);
            QD_MARK(1);
        }
        float rm = mt;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (s0 + u * SG < nact)
                rm = fmaxf(rm, mm[u]);
        if (rm == -INFINITY)
            continue;
        const float sc = (mt == -INFINITY) ? 0.f : expf(mt - rm);
        num *= sc;
        den *= sc;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s0 + u * SG < nact) {
                const float f = expf(mm[u] - rm);
                num = fmaf(f, a[u], num);
                den = fmaf(f, ll[u], den);
            }
        }
        mt = rm;
    }
    gm[sg][d] = mt;
    gn[sg][d] = num;
    gd[sg][d] = den;
    __syncthreads();
    QD_MARK(2);
    if (sg == 0) {
        float M = gm[0][d];
#pragma unroll
        for (int k = 1; k < SG; ++k)
            M = fmaxf(M, gm[k][d]);
        float N = 0.f, D = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int k = 0; k < SG; ++k) {
                const float f = (gm[k][d] == -INFINITY) ? 0.f : expf(gm[k][d] - M);
                N = fmaf(f, gn[k][d], N);
                D = fmaf(f, gd[k][d], D);
            }
        }
        out[((size_t)b * nq + h) * HD + d] = (D > 0.f) ? N / D : 0.f;
    }
    QD_MARK(3);
}

// Split policy.  Waves per workgroup and keys per split for a grid of
// (nsplit, nkv, B): each wave step is 16 keys, a split is `waves` x 16 keys x
// steps.  The model path aims at one workgroup per CU (256 CUs): a second
// workgroup on a CU delays both.  The standalone path aims at about 1024
// workgroups of 4 waves, several 16-key steps each at long contexts.
struct AttnGeom {
    int waves, chunk, nsplit;
};
inline AttnGeom attn_geom(int B, int nkv, int max_kv, int target_wgs, int max_waves, int fixed_waves)
{
    AttnGeom a;
    const int steps16 = max(1, (max_kv + ATT_WK - 1) / ATT_WK);   // 16-key steps in max_kv
    int want = target_wgs / max(1, B * nkv);                         // splits per (b, g)
    want = max(1, min(want, steps16));
    const int per = (steps16 + want - 1) / want;                     // 16-key steps per split
    if (fixed_waves > 0) {
        a.waves = fixed_waves;
        const int st = (per + fixed_waves - 1) / fixed_waves;        // steps per wave
        a.chunk = st * fixed_waves * ATT_WK;
    } else {
        a.waves = min(per, max_waves);
        const int st = (per + a.waves - 1) / a.waves;
        a.chunk = st * a.waves * ATT_WK;
    }
    a.nsplit = (max(1, max_kv) + a.chunk - 1) / a.chunk;
    return a;
}

}  // namespace qd
