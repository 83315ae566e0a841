// prefill_attn.h -- causal attention of a prefill chunk with each K/V tile
// read once for all of the chunk's queries (gfx950 matrix cores).
//
// The T positions p0 .. p0+T-1 of a chunk attend over one cache: query
// t sees keys 0 .. p0+t (inferencelayer cuda_llm.rs page, fa_prefill: a tile
// of queries, K and V tiles staged once and shared, the causal mask inside
// the tile; the online-softmax partials merged as in attn_reduce).
//
// Workgroup (split s, kv head g, piece z) owns keys [s*chunk, (s+1)*chunk)
// of that kv head and every query row of its GQA group for the piece's tp
// positions: tp*GQ rows (t, j), row R = t*GQ + j (head g*GQ + j), 16 rows per
// wave (wave w: rows 16w .. 16w+15), so NWV = GQ * tp / 16 waves.  A piece's
// splits past its last key return at once.  Per 16-key step (one paged block) the K and
// V tiles are loaded once into LDS and every wave uses them:
//   S^T = K Q^T   v_mfma_f32_16x16x32_f16, M = the 16 keys, N = the wave's 16
//                 query rows, K = 32 dims per instruction; q enters as an f16
//                 hi + lo pair (about 22 bits), K is f16 already
//   mask          key > p0 + t (or t >= T): -inf
//   softmax       online per query column (max and sum over the 16 keys:
//                 4 registers, then the 4 lane groups)
//   O^T += V^T P  v_mfma_f32_16x16x16_f16, M = 16 dims of a tile, K = the 16
//                 keys, N = the queries; the B operand is the softmax's own
//                 accumulator layout (lane l: keys 4*(l/16) .. +3 of query
//                 l%16), as an f16 hi + lo pair; V^T from a transposed LDS tile
// The partial (m, l, acc) of every (position, head, split) goes to the
// partials layout of k_attn_combine, which merges the active splits of each
// query (kv_len = p0 + t + 1).
#pragma once

#include "attn_decode.h"

namespace qd {

typedef _Float16 fa_half4 __attribute__((ext_vector_type(4)));
typedef _Float16 fa_half8 __attribute__((ext_vector_type(8)));
typedef float fa_floatx4 __attribute__((ext_vector_type(4)));

constexpr int FA_KPAD = 8;   // halves of padding per K row in LDS
constexpr int FA_VPAD = 4;   // halves of padding per transposed V row

struct FaParams {
    const float* q;           // [T][nq][HD], normed and rotated
    const uint16_t* k;        // cache (paged [nblocks][nkv][16][HD] or contiguous [nkv][max_kv][HD])
    const uint16_t* v;
    const int32_t* table;     // sequence 0's block table, or nullptr (contiguous)
    int max_kv;
    int nq, nkv, T, p0;
    float scale;
    int chunk, nsplit;        // keys per split (a multiple of 16), splits
    float* part;              // [T][nq][nsplit][HD + 2]
    int tp;                   // positions per workgroup (blockIdx.z: the piece)
};

template <int HD, int GQ, int NWV>
__global__ void __launch_bounds__(NWV* WAVE) k_pf_attn(FaParams p)
{
    {   // this workgroup's piece of the chunk: positions z*tp .. z*tp+tp-1
        const int z = blockIdx.z, t0 = z * p.tp;
        p.p0 += t0;
        p.q += (size_t)t0 * p.nq * HD;
        p.part += (size_t)t0 * p.nq * p.nsplit * (HD + 2);
        p.T = min(p.tp, p.T - t0);
    }
    static_assert(NWV * WAVE <= 1024, "workgroup");
    constexpr int NI = HD / 32;     // 32-dim slices (QK)
    constexpr int NT = HD / 16;     // 16-dim tiles (PV)
    constexpr int NTH = NWV * WAVE;
    constexpr int KROW = HD + FA_KPAD, VROW = 16 + FA_VPAD;
    __shared__ __align__(16) _Float16 kt[16 * KROW];    // K tile [key][dim]
    __shared__ __align__(16) _Float16 vt[HD * VROW];    // V tile transposed [dim][key]
    const int s = blockIdx.x, g = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int c = lane & 15, kg = lane >> 4;            // query column, lane group
    const int kv_total = p.p0 + p.T;
    const int k_begin = s * p.chunk, k_end = min(kv_total, k_begin + p.chunk);
    if (k_begin >= k_end)
        return;   // uniform: no query reads this split

    // this lane's query row: R = 16 w + c -> (t, j)
    const int R = 16 * w + c, t = R / GQ, j = R % GQ, h = g * GQ + j;
    const bool qvalid = t < p.T;
    const int klim = qvalid ? p.p0 + t : -1;             // last key this query sees

    // q as f16 hi + lo in the B layout: dims 32i + 8kg .. +7 of query row R
    fa_half8 bhi[NI], blo[NI];
    {
        const float* qp = p.q + ((size_t)min(t, p.T - 1) * p.nq + h) * HD;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const float4 a = *reinterpret_cast<const float4*>(qp + 32 * i + 8 * kg);
            const float4 b = *reinterpret_cast<const float4*>(qp + 32 * i + 8 * kg + 4);
            const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = qvalid ? f[e] * p.scale : 0.f;
                const _Float16 hh = (_Float16)v;
                bhi[i][e] = hh;
                blo[i][e] = (_Float16)(v - (float)hh);
            }
        }
    }

    // global loads of one 16-key tile (clamped rows, never a branch around a load)
    constexpr int NU = (16 * HD / 8 + NTH - 1) / NTH;   // 8-half units per thread
    uint4 kr[NU], vr[NU];
    auto load_tile = [&](int k0) {
        const uint16_t *kb, *vb;
        if (p.table) {
            const int phys = max(0, p.table[min(k0, p.max_kv - 1) / ATT_BS]);
            const size_t base = ((size_t)phys * p.nkv + g) * ATT_BS * HD;
            kb = p.k + base;
            vb = p.v + base;
        } else {
            const size_t base = (size_t)g * p.max_kv * HD;
            kb = p.k + base;
            vb = p.v + base;
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int idx = min(tid + u * NTH, 16 * HD / 8 - 1);
            const int row = idx / (HD / 8), col = (idx % (HD / 8)) * 8;
            const size_t r = p.table ? (size_t)row : (size_t)min(k0 + row, p.max_kv - 1);
            kr[u] = *reinterpret_cast<const uint4*>(kb + r * HD + col);
            vr[u] = *reinterpret_cast<const uint4*>(vb + r * HD + col);
        }
    };
    auto store_tile = [&] {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int idx = tid + u * NTH;
            if (idx < 16 * HD / 8) {
                const int row = idx / (HD / 8), col = (idx % (HD / 8)) * 8;
                *reinterpret_cast<uint4*>(&kt[row * KROW + col]) = kr[u];
                const fa_half8 vv = __builtin_bit_cast(fa_half8, vr[u]);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    vt[(col + e) * VROW + row] = vv[e];
            }
        }
    };

    float m_c = -INFINITY, l_c = 0.f;
    fa_floatx4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n)
        acc[n] = fa_floatx4{0.f, 0.f, 0.f, 0.f};

    load_tile(k_begin);
    for (int k0 = k_begin; k0 < k_end; k0 += 16) {
        __syncthreads();   // the previous step's LDS reads are done
        store_tile();
        __syncthreads();
        if (k0 + 16 < k_end)   // uniform
            load_tile(k0 + 16);
        // S^T: keys 4kg + r of the step, query c
        fa_floatx4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const fa_half8 a = *reinterpret_cast<const fa_half8*>(&kt[c * KROW + 32 * i + 8 * kg]);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bhi[i], sc, 0, 0, 0);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, blo[i], sc, 0, 0, 0);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = k0 + 4 * kg + r;
            sc[r] = (key <= klim && key < k_end) ? sc[r] : -INFINITY;
            mx = fmaxf(mx, sc[r]);
        }
        {
            float lo, hi;
            lanes::swap16(mx, lo, hi);
            mx = fmaxf(lo, hi);
            lanes::swap32(mx, lo, hi);
            mx = fmaxf(lo, hi);
        }
        const float mnew = fmaxf(m_c, mx);
        // a query with no key in this step so far keeps everything at zero
        const bool none = mnew == -INFINITY;
        float pr[4], ps = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pr[r] = none ? 0.f : expf(sc[r] - mnew);   // 0 for a masked key
            ps += pr[r];
        }
        {
            float lo, hi;
            lanes::swap16(ps, lo, hi);
            ps = lo + hi;
            lanes::swap32(ps, lo, hi);
            ps = lo + hi;
        }
        const float alpha = (m_c == -INFINITY) ? 0.f : expf(m_c - mnew);
        l_c = fmaf(l_c, alpha, ps);
        m_c = mnew;
        fa_half4 phi, plo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const _Float16 hh = (_Float16)pr[r];
            phi[r] = hh;
            plo[r] = (_Float16)(pr[r] - (float)hh);
        }
        // O^T tile n: dims 16n + 4kg + i of query c
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const fa_half4 a = *reinterpret_cast<const fa_half4*>(&vt[(16 * n + c) * VROW + 4 * kg]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[n][i] *= alpha;
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, phi, acc[n], 0, 0, 0);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, plo, acc[n], 0, 0, 0);
        }
    }

    // the partial of (position t, head h, split s)
    if (qvalid) {
        const size_t pstride = HD + 2;
        float* pp = p.part + (((size_t)t * p.nq + h) * p.nsplit + s) * pstride;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pp[16 * n + 4 * kg + i] = acc[n][i];
        if (kg == 0) {
            pp[HD] = m_c;
            pp[HD + 1] = l_c;
        }
    }
}

// The split merge of a prefill chunk written straight as the o product's
// input: grid (chunks of 256 output elements, T positions), 512 threads
// (element i = tid % 256 of the chunk, split group tid / 256).  Each group
// merges splits sg, sg + 2, .. with every load of a round of U issued first
// (U * 2 >= nsplit on the host, so one round); the two groups are merged in
// LDS (M = max m_s, out = sum e^(m_s - M) acc_s / sum e^(m_s - M) l_s, as
// k_attn_combine), the output multiplied by sigmoid(gate) for a model with
// the attention output gate (gate rows of position t at gate + t * gstride,
// as ngslab partial products gslab floats apart), then split as
// k_xsplit_batch does with four slot groups: the chunk's largest |x| sets its
// power of two, position t is slot t.
constexpr int FA_CMB_THREADS = 512;
template <int HD, int U>
__global__ void __launch_bounds__(FA_CMB_THREADS)
k_attn_combine_xp(const float* __restrict__ part, int nsplit, int chunk, const int32_t* __restrict__ kv_lens,
                  int max_kv, int nq, _Float16* __restrict__ XP, float* __restrict__ XS,
                  const float* __restrict__ gate, int gstride, int ngslab, size_t gslab)
{
    constexpr int NG = 4, CE = 32 * gbm_kcb(NG), SG = FA_CMB_THREADS / CE;   // 256 elements, 2 groups
    __shared__ float gm[SG][CE], gn[SG][CE], gd[SG][CE];
    const int c = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
    const int i = tid % CE, sg = tid / CE;
    const int n = nq * HD, e = min(c * CE + i, n - 1);   // clamped: the results past n are dropped
    const int h = e / HD, d = e % HD;
    const size_t pstride = HD + 2;
    const float* pp = part + ((size_t)t * nq + h) * nsplit * pstride;
    int kv_len = kv_lens[t];
    kv_len = max(0, min(kv_len, max_kv));
    const int nact = min(nsplit, (kv_len + chunk - 1) / chunk);
    float mt = -INFINITY, num = 0.f, den = 0.f;
    for (int s0 = sg; s0 < nsplit; s0 += U * SG) {
        float a[U], mm[U], ll[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t sp = (size_t)min(s0 + u * SG, nsplit - 1) * pstride;   // never a branch
            a[u] = pp[sp + d];
            mm[u] = pp[sp + HD];
            ll[u] = pp[sp + HD + 1];
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
    gm[sg][i] = mt;
    gn[sg][i] = num;
    gd[sg][i] = den;
    __syncthreads();
    if (sg == 0) {
        float M = gm[0][i];
#pragma unroll
        for (int k = 1; k < SG; ++k)
            M = fmaxf(M, gm[k][i]);
        float N = 0.f, D = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int k = 0; k < SG; ++k) {
                const float f = (gm[k][i] == -INFINITY) ? 0.f : expf(gm[k][i] - M);
                N = fmaf(f, gn[k][i], N);
                D = fmaf(f, gd[k][i], D);
            }
        }
        float o = (D > 0.f) ? N / D : 0.f;
        if (gate) {   // uniform
            const float g = slab_sum<4>(gate + (size_t)t * gstride + e, ngslab, gslab);
            o *= 1.0f / (1.0f + expf(-g));
        }
        gm[1][i] = o;   // the merged chunk, read below by the split items
    }
    __syncthreads();
    // the chunk's 32 items (block bl = tid / 4, lane group kg = tid % 4): wave 0
    if (tid < WAVE) {
        const int bl = tid >> 2, kg = tid & 3;
        const bool in = tid < 4 * gbm_kcb(NG) && (c * CE + bl * 32) < n;
        float ev[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (in) {
            const float* x = &gm[1][bl * 32 + 4 * kg];
            // slot order of a lane group: 4kg, 4kg+2, 4kg+1, 4kg+3, then the
            // same four plus 16, divided by 16 (exact)
            ev[0] = x[0];
            ev[1] = x[2];
            ev[2] = x[1];
            ev[3] = x[3];
            ev[4] = x[16] * 0.0625f;
            ev[5] = x[18] * 0.0625f;
            ev[6] = x[17] * 0.0625f;
            ev[7] = x[19] * 0.0625f;
        }
        const float sc = gbm_scale_for(group_max<WAVE>(gbm_xp_absmax(ev)));
        if (in)
            gbm_xp_put(XP, NG, c, bl, kg, t, ev, sc);
        if (tid == 0)
            XS[c * 16 * NG + t] = 1.0f / sc;
    }
}

}  // namespace qd
