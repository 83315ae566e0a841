// attn_decode.h -- split-KV GQA decode attention for gfx950.
//
// Computes, for every query head h of sequence b,
//   out = softmax(scale * q_h K^T) V   over keys t in [0, kv_len[b])
// with kv head g = h / (nq/nkv) (inferencelayer cuda_llm.rs page, attn_partial,
// attn_reduce and the flash-decoding arm that reads a K/V chunk once for the
// whole query group; ferrum-kernels cuda_decode.rs page, flash_decode_attention
// phase 1/2, paged_decode_attention, batched_decode_attention).
//
// k_attn_split: grid (nsplit, nkv, B), up to 8 waves (4 with GQA 8).  A
// workgroup owns one (sequence, kv head, key range) and serves all GQ query
// heads of that kv head.  Each wave works on its own 16-key steps (one paged
// block), the next step's K/V in flight while it computes one, with no
// workgroup barrier until the end:
//   QK   v_mfma_f32_16x16x32_f16 with M = the step's 16 keys (straight from
//        the K loads), N = the query heads (columns past GQ zero), K = 32 dims
//        per instruction; q enters as an f16 hi + lo pair (about 22 bits);
//   softmax  per head over the 16 keys (4 accumulator registers, then shuffles
//        across the 4 lane groups), online across the wave's steps (running
//        max m, sum l, rescale of acc);
//   PV   lane owns HD/64 output dims; the step's probabilities go through a
//        small per-wave LDS table [key][head]; V is loaded in that layout.
// The waves' (m, l, acc) are merged once through LDS and written as the
// workgroup's partial.  The partials of a head are merged as
//   M = max_s m_s,  out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s
// by one of: k_attn_combine (grid (nq, B), a launch of its own); the last
// split workgroup of each (sequence, kv head) to finish (counters given); or,
// in the batched decode step, the last of each (sequence, 1024-element chunk
// of the output), which writes the chunk as the o product's split input.
//
// In the decode step (QMODE 1; QMODE 2 for B sequences whose raw q|k|v come
// as K-slice partial products) the split kernel also finishes the projection:
// from the raw q|k|v of the token it applies the per-head q/k RMSNorm and the
// NeoX rotary at the position (ferrum-kernels cuda_decode.rs page, the q/k
// norm then rope order of decode_step), and the wave whose keys hold the
// position stores the token's K and V (f16) in the cache and uses the same f16
// values.  There the block table covers every position below max_kv, so the
// first step's table entry and K/V loads are issued before the position is
// known; keys at or past kv_len are masked (score -inf, V taken as 0).
#pragma once

#include "qd_common.h"
#include "gemv_batch_mfma.h"

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
    unsigned* counters;        // [B][nkv], zero between launches: when given, the last
                               // workgroup of each (b, g) merges the partials itself
    // decode-step prologue (QMODE 1 and 2)
    int qk_norm;               // 1: per-head RMSNorm of q and k
    const float* q_norm;       // [HD] (valid even when qk_norm is 0)
    const float* k_norm;
    float eps;
    int rot;
    const float* rope_cur;     // cos [rot/2] then sin [rot/2] at the step's position
    uint16_t* kc;              // cache written at pos (same buffers as k/v)
    uint16_t* vc;
    // K/V in fp8 e4m3: element = e4m3 value * scale
    float k_scale, v_scale;
    // attention output gate (decode step): the merged output of head h, dim d
    // is multiplied by sigmoid(gate[h * HD + d]); nullptr = none
    const float* gate;
    // 1: every sequence b reads the cache of sequence 0 (the B queries of a
    // prefill chunk over one cache, each with its own kv_len)
    int shared_kv;
    // decode step of B sequences (QMODE 1 and 2): sequence b's raw q|k|v at
    // q + b * q_stride, its position at pos[b * pos_stride], its rotary
    // factors at rope_cur + b * rope_stride (all 0 for one sequence); with
    // QMODE 2 the raw q|k|v come as q_slabs partial products q_slab_stride
    // floats apart, summed here in slab order (QMODE 1: one, q_slabs unused)
    int q_stride, pos_stride, rope_stride;
    int q_slabs;
    size_t q_slab_stride;
    // QMODE 2 with counters: when xp is given, the merge writes sequence b's
    // output as the o product's split input instead of out: chunk c of 1024
    // elements (the kv heads whose query heads it holds) is merged by the
    // last workgroup of those kv heads to finish, which writes its f16 pairs
    // to xp and 1/scale to xs[c * 16 + b] (the layout of k_xsplit_batch with
    // one slot group); counters are then per (b, chunk)
    _Float16* xp;
    float* xs;
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
    int last;
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// f32 -> OCP fp8 e4m3 code (sign, 4 exponent bits with bias 7, 3 mantissa
// bits), rounded to nearest even and saturated at +-448: the decode step's
// store into an fp8 cache.  Written out rather than left to a conversion
// instruction, so that its rounding and saturation are the stated ones.
QD_DEV uint32_t f32_to_e4m3(float x)
{
    const uint32_t sgn = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = fminf(fabsf(x), 448.f);
    if (a < 0.015625f)                                   // subnormal: multiples of 2^-9
        return sgn | (uint32_t)rintf(a * 512.f);         // 0 .. 8 (8 is the smallest normal)
    int e;
    const float f = frexpf(a, &e);                       // a = (2f) 2^(e-1), 2f in [1, 2)
    int E = e - 1;
    int mant = (int)rintf((2.f * f - 1.f) * 8.f);        // exact argument, ties to even
    if (mant == 8) {                                     // rounded up to the next power of two
        mant = 0;
        E += 1;
    }
    return sgn | (uint32_t)(((E + 7) << 3) | mant);
}
typedef float floatx4 __attribute__((ext_vector_type(4)));

// float load: agent-scope (COH, a value another workgroup of the same launch
// stored agent-scope) or plain
template <bool COH>
QD_DEV float ld_f32(const float* p)
{
    if (COH)
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return *p;
}
template <bool COH>
QD_DEV void st_f32(float* p, float v)
{
    if (COH)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

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

// Online-softmax merge of the split partials of the GQ heads of (sequence b,
// kv head g), splits [0, nact), in rounds of U <= 64 splits:
//   M = max_s m_s,  out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s.
// A wave covers dims of one head (HD >= 64), so lane k loads (m, l) of split
// s0 + k once for the whole wave and the weights e^(m_s - M) are read across
// lanes; each lane loads its own dim of every split of the round.  All loads
// of a round are issued before any is used (indexes clamped, never a branch).
// Agent-scope loads: the partials come from other workgroups of this launch.
template <int HD, int GQ, int U, bool COH>
QD_DEV void attn_merge_heads(const AttnParams& p, int b, int g, int nact, float* lds_out = nullptr)
{
    static_assert(U <= WAVE, "one split per lane");
    const size_t pstride = HD + 2;
    const int lane = threadIdx.x & (WAVE - 1);
    // GQ * HD and blockDim.x are multiples of 64: a wave is wholly in or out
    for (int i = threadIdx.x; i < GQ * HD; i += blockDim.x) {
        const int j = i / HD, d = i % HD;
        const int h = g * GQ + j;
        const float* pp = p.part + ((size_t)b * p.nq + h) * p.nsplit * pstride;
        float mt = -INFINITY, num = 0.f, den = 0.f;
        for (int s0 = 0; s0 < nact; s0 += U) {
            const int sl = min(s0 + lane, nact - 1);
            const uint64_t ml = __hip_atomic_load(reinterpret_cast<const uint64_t*>(pp + sl * pstride + HD),
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            float a[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                a[u] = __hip_atomic_load(pp + (size_t)min(s0 + u, nact - 1) * pstride + d,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool act = s0 + lane < nact && lane < U;
            const float m = act ? __uint_as_float((uint32_t)ml) : -INFINITY;
            const float l = act ? __uint_as_float((uint32_t)(ml >> 32)) : 0.f;
            const float rm = fmaxf(mt, group_max<WAVE>(m));
            const float sc = (mt == -INFINITY) ? 0.f : expf(mt - rm);
            const float f = (m == -INFINITY) ? 0.f : expf(m - rm);
            den = fmaf(den, sc, group_sum<WAVE>(f * l));
            num *= sc;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (s0 + u < nact)   // uniform
                    num = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), u)), a[u], num);
            mt = rm;
        }
        float o = (den > 0.f) ? num / den : 0.f;
        if (lds_out) {   // uniform
            lds_out[i] = o;
            continue;
        }
        if (p.gate)   // uniform
            o *= 1.0f / (1.0f + expf(-ld_f32<COH>(p.gate + (size_t)h * HD + d)));
        st_f32<COH>(p.out + ((size_t)b * p.nq + h) * HD + d, o);
    }
}

// Merge of the split partials of one (sequence b, kv head g) by the last of
// its workgroups to finish.  Every workgroup's partial stores are
// agent-scope; each thread waits for its own, the workgroup counts itself once
// with a relaxed agent-scope add, and the one that completes the count reads
// all partials with agent-scope loads.  No fence is needed: no plain store is
// published this way.  The order rests on a gfx9 property, not on the memory
// model's release/acquire: stores count in vmcnt, so after s_waitcnt vmcnt(0)
// this thread's agent-scope stores are complete at the agent's coherence
// point, before the add is issued; and the merging workgroup's agent-scope
// loads are issued after it observed the count.  (A release add would write
// back the XCD's L2 in every workgroup: ~19 us against ~1.5 us per round trip.)
// The counter is returned to zero for the next launch.
template <int HD, int GQ, bool COH>
QD_DEV void attn_merge_last(const AttnParams& p, int b, int g, int kv_len, int* last)
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's partial stores are done
    __syncthreads();
    const int nact = (kv_len + p.chunk - 1) / p.chunk;
    unsigned* cnt = p.counters + (size_t)b * p.nkv + g;
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *last = (prev + 1 == (unsigned)nact);
    }
    __syncthreads();
    if (!*last)
        return;
    // the merge is on the critical path of the step: one round of loads
    // for up to 32 splits, sized to the active count
    if (nact <= 8)
        attn_merge_heads<HD, GQ, 8, COH>(p, b, g, nact);
    else if (nact <= 16)
        attn_merge_heads<HD, GQ, 16, COH>(p, b, g, nact);
    else
        attn_merge_heads<HD, GQ, 32, COH>(p, b, g, nact);
    if (threadIdx.x == 0)
        __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The merge of attn_merge_heads for n consecutive output elements of
// sequence b starting at kv head g0's first query head, EPT elements per
// thread (i = threadIdx.x + r * blockDim.x, n <= EPT * blockDim.x), into
// out[i]: every load of a round of U splits is issued for all of a thread's
// elements before any is used, so the merge costs one memory latency per
// round whatever EPT is.  Indexes past n are clamped (their results dropped).
template <int HD, int GQ, int U, int EPT>
QD_DEV void attn_merge_rows(const AttnParams& p, int b, int g0, int n, int nact, float* out)
{
    static_assert(U <= WAVE, "one split per lane");
    const size_t pstride = HD + 2;
    const int lane = threadIdx.x & (WAVE - 1);
    float mt[EPT], num[EPT], den[EPT];
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
        mt[r] = -INFINITY;
        num[r] = den[r] = 0.f;
    }
    for (int s0 = 0; s0 < nact; s0 += U) {
        uint64_t ml[EPT];
        float a[EPT][U];
#pragma unroll
        for (int r = 0; r < EPT; ++r) {
            // a wave's 64 elements lie in one head (HD and blockDim.x multiples of 64)
            const int i = min((int)threadIdx.x + r * (int)blockDim.x, n - 1);
            const float* pp = p.part + ((size_t)b * p.nq + g0 * GQ + i / HD) * p.nsplit * pstride;
            const int sl = min(s0 + lane, nact - 1);
            ml[r] = __hip_atomic_load(reinterpret_cast<const uint64_t*>(pp + sl * pstride + HD), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int u = 0; u < U; ++u)
                a[r][u] = __hip_atomic_load(pp + (size_t)min(s0 + u, nact - 1) * pstride + i % HD, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int r = 0; r < EPT; ++r) {
            const bool act = s0 + lane < nact;
            const float m = act ? __uint_as_float((uint32_t)ml[r]) : -INFINITY;
            const float l = act ? __uint_as_float((uint32_t)(ml[r] >> 32)) : 0.f;
            const float rm = fmaxf(mt[r], group_max<WAVE>(m));
            const float sc = (mt[r] == -INFINITY) ? 0.f : expf(mt[r] - rm);
            const float f = (m == -INFINITY) ? 0.f : expf(m - rm);
            den[r] = fmaf(den[r], sc, group_sum<WAVE>(f * l));
            num[r] *= sc;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (s0 + u < nact)   // uniform
                    num[r] = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), u)), a[r][u], num[r]);
            mt[r] = rm;
        }
    }
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
        const int i = threadIdx.x + r * blockDim.x;
        if (i < n)
            out[i] = (den[r] > 0.f) ? num[r] / den[r] : 0.f;
    }
}

// the chunk merge needs 1024 floats of LDS, taken from the workgroup's acc
// rows, and one float per wave (m rows)
__host__ __device__ constexpr bool attn_split_out_ok(int hd, int gq)
{
    return (gq <= 4 ? 8 : 4) * gq * hd >= 1024 && 1024 % (gq * hd) == 0;
}

// The merge as attn_merge_last, per chunk c of 1024 output elements of
// sequence b (KPC = 1024 / (GQ HD) kv heads, fewer in a ragged last chunk):
// the last of the chunk's workgroups to finish merges every head of the chunk
// into LDS (buf: 1024 floats; one round of loads with attn_merge_rows when a
// thread holds at most 4 elements, else kv head by kv head) and writes the
// chunk as the o product's split input, as k_xsplit_batch does: items
// (block, lane group) of 8 elements, the power of two that puts the chunk's
// largest |x| in [2^13, 2^14), the f16 pair of each element, 1/scale in xs.
template <int HD, int GQ>
QD_DEV void attn_merge_split(const AttnParams& p, int b, int g, int kv_len, int* last, float* buf, float* red)
{
    constexpr int KPC = 1024 / (GQ * HD);
    static_assert(attn_split_out_ok(HD, GQ) && AttnMaxWaves<GQ>::value == (GQ <= 4 ? 8 : 4),
                  "a kv head inside one chunk, 1024 floats of acc rows");
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's partial stores are done
    __syncthreads();
    const int nact = (kv_len + p.chunk - 1) / p.chunk;
    const int c = g / KPC, g0 = c * KPC, nkc = min(KPC, p.nkv - g0);
    const int nchunk = (p.nkv + KPC - 1) / KPC;
    unsigned* cnt = p.counters + (size_t)b * nchunk + c;
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *last = (prev + 1 == (unsigned)(nact * nkc));
    }
    __syncthreads();
    if (!*last)
        return;
    const int n = nkc * GQ * HD, ept = (n + (int)blockDim.x - 1) / (int)blockDim.x;
    if (ept <= 2 && nact <= 8)
        attn_merge_rows<HD, GQ, 8, 2>(p, b, g0, n, nact, buf);
    else if (ept <= 2)
        attn_merge_rows<HD, GQ, 32, 2>(p, b, g0, n, nact, buf);
    else if (ept <= 4 && nact <= 8)
        attn_merge_rows<HD, GQ, 8, 4>(p, b, g0, n, nact, buf);
    else if (ept <= 4)
        attn_merge_rows<HD, GQ, 32, 4>(p, b, g0, n, nact, buf);
    else   // small workgroups: kv head by kv head
        for (int k = 0; k < nkc; ++k) {
            float* dst = buf + k * GQ * HD;
            if (nact <= 8)
                attn_merge_heads<HD, GQ, 8, false>(p, b, g0 + k, nact, dst);
            else if (nact <= 16)
                attn_merge_heads<HD, GQ, 16, false>(p, b, g0 + k, nact, dst);
            else
                attn_merge_heads<HD, GQ, 32, false>(p, b, g0 + k, nact, dst);
        }
    __syncthreads();
    // the chunk's 128 items (block bl = it / 4, lane group kg = it % 4): item
    // t and t + blockDim.x of thread t (blockDim.x >= 64)
    const int nb = p.nq * HD / 32, nw = blockDim.x / WAVE;
    float e[2][8];
    float m = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int it = threadIdx.x + u * blockDim.x;
        const bool in = it < 128 && c * 32 + (it >> 2) < nb;
        const float* x = buf + min(it >> 2, 31) * 32 + 4 * (it & 3);
        // slot order of a lane group: 4kg, 4kg+2, 4kg+1, 4kg+3, then the same
        // four plus 16, divided by 16 (exact)
        e[u][0] = in ? x[0] : 0.f;
        e[u][1] = in ? x[2] : 0.f;
        e[u][2] = in ? x[1] : 0.f;
        e[u][3] = in ? x[3] : 0.f;
        e[u][4] = in ? x[16] * 0.0625f : 0.f;
        e[u][5] = in ? x[18] * 0.0625f : 0.f;
        e[u][6] = in ? x[17] * 0.0625f : 0.f;
        e[u][7] = in ? x[19] * 0.0625f : 0.f;
        m = fmaxf(m, gbm_xp_absmax(e[u]));
    }
    m = group_max<WAVE>(m);
    if ((threadIdx.x & (WAVE - 1)) == 0)
        red[threadIdx.x / WAVE] = m;
    __syncthreads();
    float cm = red[0];
    for (int u = 1; u < nw; ++u)
        cm = fmaxf(cm, red[u]);
    const float sc = gbm_scale_for(cm);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int it = threadIdx.x + u * blockDim.x;
        if (it < 128 && c * 32 + (it >> 2) < nb)
            gbm_xp_put(p.xp, 1, c, it >> 2, it & 3, b, e[u], sc);
    }
    if (threadIdx.x == 0) {
        p.xs[c * 16 + b] = 1.0f / sc;
        __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The work of one split workgroup: (split s, kv head g, sequence b).
// QMODE 0: q given (standalone); QMODE 1: decode-step prologue from raw q|k|v;
// QMODE 2: the same with q|k|v summed from q_slabs partial products.
// FUSED: inside the persistent layer kernel.  wait() runs after the first
// step's K/V loads are issued (they need nothing of this step) and before
// anything of this step's q|k|v is read; q|k|v are read and the merged output
// is stored agent-scope (other workgroups of the same launch wrote / read them).
template <int HD, int GQ, bool PAGED, int QMODE, bool FUSED, bool KV8, class Wait>
QD_DEV void attn_split_body(const AttnParams& p, int s, int g, int b, AttnSmem<HD, GQ>& sm, Wait&& wait)
{
    static_assert(HD == 64 || HD == 128, "head_dim");
    static_assert(!KV8 || !FUSED, "fp8 K/V: not in the persistent layer kernel");
    static_assert(GQ == 1 || GQ == 2 || GQ == 4 || GQ == 8, "group");
    static_assert(QMODE >= 0 && QMODE <= 2, "query mode");
    static_assert(QMODE != 2 || !FUSED, "q|k|v slabs: not in the persistent layer kernel");
    using Step = AttnStep<HD>;
    constexpr int NI = Step::NI, DPL = Step::DPL;

    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int nw = blockDim.x / WAVE;          // waves of this launch
    const int wstride = nw * ATT_WK;           // keys between a wave's steps
    const int kk = lane & 15;                  // QK: the key of this lane's A rows
    const int h0 = g * GQ;
    const int t_begin = s * p.chunk;
    const int bk = p.shared_kv ? 0 : b;        // the sequence whose cache is read
    QD_MARK(0);

    // loads of one wave step at key tw, any tw: rows and table entries are
    // clamped into range (never a branch around a load); rows past kv_len are
    // masked where they are used
    auto load_step = [&](Step& st, int tw) {
        const int twc = min(tw, p.max_kv - 1);
        if (KV8) {
            // e4m3 bytes.  K: this lane takes the 8*NI contiguous dims
            // kg*8*NI .. (the QK dim order of the fp8 path, matched by q).
            // V: the lane's DPL bytes of each key.
            const uint8_t* k8 = reinterpret_cast<const uint8_t*>(p.k);
            const uint8_t* v8 = reinterpret_cast<const uint8_t*>(p.v);
            size_t kb, vb;
            if (PAGED) {
                const int phys = max(0, p.tables[(size_t)bk * p.mbps + twc / ATT_BS]);
                const size_t base = kv_row<HD, PAGED>(p, phys, g, twc & ~(ATT_BS - 1));
                kb = base + (size_t)kk * HD;
                vb = base;
            } else {
                kb = kv_row<HD, PAGED>(p, bk, g, min(tw + kk, p.max_kv - 1));
                vb = kv_row<HD, PAGED>(p, bk, g, 0);
            }
#pragma unroll
            for (int i = 0; i < NI / 2; ++i)
                st.k[i] = *reinterpret_cast<const uint4*>(k8 + kb + 8 * NI * (lane >> 4) + 16 * i);
#pragma unroll
            for (int j = 0; j < ATT_WK; ++j) {
                const size_t r = PAGED ? vb + (size_t)j * HD
                                       : vb + (size_t)min(tw + j, p.max_kv - 1) * HD;
                if (DPL == 2)
                    st.v[j] = *reinterpret_cast<const uint16_t*>(v8 + r + lane * DPL);
                else
                    st.v[j] = v8[r + lane * DPL];
            }
            return;
        }
        const uint16_t *kp, *vp;
        if (PAGED) {
            const int phys = max(0, p.tables[(size_t)bk * p.mbps + twc / ATT_BS]);
            const size_t base = kv_row<HD, PAGED>(p, phys, g, twc & ~(ATT_BS - 1));
            kp = p.k + base + (size_t)kk * HD;
            vp = p.v + base;
        } else {
            kp = p.k + kv_row<HD, PAGED>(p, bk, g, min(tw + kk, p.max_kv - 1));
            vp = p.v + kv_row<HD, PAGED>(p, bk, g, 0);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
            st.k[i] = *reinterpret_cast<const uint4*>(kp + 8 * (lane >> 4) + 32 * i);
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

    Step cur_st;
    const int tw0 = t_begin + w * ATT_WK;
    if (FUSED) {
        // K/V of the wave's first step before the wait: the cache rows below
        // the position were written by earlier launches
        load_step(cur_st, tw0);
        asm volatile("" ::: "memory");   // keep these loads ahead of the wait
        wait();
    }

    // kv_len first (vector loads return in order): the loads below do not need
    // it.  One load from a selected address, so nothing waits for it here.
    const int32_t* kvp = p.kv_lens ? p.kv_lens + b : p.pos + (size_t)b * p.pos_stride;
    const int kv_raw = *kvp;

    // ---- loads that do not need kv_len: the token's q|k|v, norm weights,
    // rotary factors, and (decode step) the first step's K/V.  Lane values
    // raw[i][e] at dim lane*DPL + e: query heads h0 .. h0+GQ-1, then the kv
    // head's k and v (QMODE >= 1).
    constexpr int NE = GQ + 2;
    const float* qb = p.q + (size_t)b * p.q_stride;              // QMODE >= 1: this sequence's q|k|v
    auto qkv_off = [&](int i, int e) -> size_t {
        const int row = i < GQ ? h0 + i : (i == GQ ? p.nq + g : p.nq + p.nkv + g);
        return (size_t)row * HD + lane * DPL + e;
    };
    float raw[NE][DPL];
    if (QMODE == 2) {
        // q|k|v as q_slabs partial products, added in slab order.  Every load
        // of a group of QSG slabs is issued before any is used (slab indexes
        // clamped, never a branch): adding each slab as its load arrived would
        // wait out one memory latency per slab.
        constexpr int QSG = 4;
        const int nsl = max(1, p.q_slabs);
#pragma unroll
        for (int i = 0; i < NE; ++i)
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                raw[i][e] = 0.f;
        for (int s0 = 0; s0 < nsl; s0 += QSG) {
            float t[QSG][NE][DPL];
#pragma unroll
            for (int u = 0; u < QSG; ++u) {
                const float* src = qb + (size_t)min(s0 + u, nsl - 1) * p.q_slab_stride;
#pragma unroll
                for (int i = 0; i < NE; ++i)
#pragma unroll
                    for (int e = 0; e < DPL; ++e)
                        t[u][i][e] = ld_f32<FUSED>(src + qkv_off(i, e));
            }
#pragma unroll
            for (int u = 0; u < QSG; ++u) {
                const bool on = s0 + u < nsl;
#pragma unroll
                for (int i = 0; i < NE; ++i)
#pragma unroll
                    for (int e = 0; e < DPL; ++e)
                        raw[i][e] += on ? t[u][i][e] : 0.f;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NE; ++i)
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                raw[i][e] = (QMODE == 0) ? (i < GQ ? ld_f32<FUSED>(p.q + ((size_t)b * p.nq + h0 + i) * HD + lane * DPL + e) : 0.f)
                                         : ld_f32<FUSED>(qb + qkv_off(i, e));
    }
    const float* rc = p.rope_cur + (size_t)b * p.rope_stride;    // QMODE >= 1: its rotary factors
    float qv[GQ][DPL], kv_[DPL], vv[DPL], wq[DPL], wk[DPL], cs[DPL], sn[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        const int d = lane * DPL + e;
#pragma unroll
        for (int j = 0; j < GQ; ++j)
            qv[j][e] = raw[j][e];
        kv_[e] = raw[GQ][e];
        vv[e] = raw[GQ + 1][e];
        wq[e] = wk[e] = cs[e] = 1.f;
        sn[e] = 0.f;
        if (QMODE >= 1) {
            // q_norm / k_norm / rope_cur always point at valid arrays here
            wq[e] = p.q_norm[d];
            wk[e] = p.k_norm[d];
            const int half = p.rot / 2;
            const int ii = d < half ? d : (d < p.rot ? d - half : 0);
            const float c0 = rc[ii], s0 = rc[half + ii];
            cs[e] = d < p.rot ? c0 : 1.f;
            sn[e] = d < p.rot ? s0 : 0.f;
        }
    }
    if (!FUSED)
        load_step(cur_st, tw0);

    // ---- queries (and the token's k): per-head RMSNorm and rotary (QMODE >= 1),
    // times scale, into this wave's LDS rows.  None of it needs kv_len, so it
    // runs while the position is still in flight.
    if (QMODE >= 1) {
        // no branch around the uses of the norm weights: a load used only in
        // a branch is sunk into it, behind the K/V loads, and then waits for them
        const bool qkn = p.qk_norm != 0;
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                ss = fmaf(qv[j][e], qv[j][e], ss);
            ss = group_sum<WAVE>(ss);
            const float r = qkn ? 1.0f / sqrtf(ss / (float)HD + p.eps) : 1.f;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                qv[j][e] = qv[j][e] * r * (qkn ? wq[e] : 1.f);
        }
        {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                ss = fmaf(kv_[e], kv_[e], ss);
            ss = group_sum<WAVE>(ss);
            const float r = qkn ? 1.0f / sqrtf(ss / (float)HD + p.eps) : 1.f;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                kv_[e] = kv_[e] * r * (qkn ? wk[e] : 1.f);
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
        // (dims at or past rot have cos 1 and sin 0: the same formula keeps them)
        const int half = p.rot / 2;
        float qpart[GQ][DPL], kpart[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            const int d = lane * DPL + e;
            const int pd = d < half ? d + half : d - half;   // in [0, HD)
#pragma unroll
            for (int j = 0; j < GQ; ++j)
                qpart[j][e] = sm.q[w][j][pd];
            kpart[e] = sm.krow[w][pd];
        }
        wave_lds_sync();   // every partner read done before the rows change
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            const int d = lane * DPL + e;
            const float sg = d < half ? -sn[e] : sn[e];
#pragma unroll
            for (int j = 0; j < GQ; ++j)
                qv[j][e] = fmaf(qpart[j][e], sg, qv[j][e] * cs[e]);
            kv_[e] = fmaf(kpart[e], sg, kv_[e] * cs[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e)
#pragma unroll
        for (int j = 0; j < GQ; ++j)
            sm.q[w][j][lane * DPL + e] = qv[j][e] * (KV8 ? p.scale * p.k_scale : p.scale);

    // ---- now the position: the key range, and the wave whose step own_tw
    // holds the token's own position stores its K and V (f16) and uses them
    const int kv_len = max(0, min(p.kv_lens ? kv_raw : kv_raw + 1, p.max_kv));
    if (kv_len >= 0)
        QD_MARK(1);
    const int t_end = min(kv_len, t_begin + p.chunk);
    if (t_begin >= t_end)
        return;   // key range past kv_len: the combine reads only active splits
    const int tcur = kv_len - 1;
    float vnew[DPL];
    const int rel = tcur - t_begin;
    const bool owner = QMODE >= 1 && tcur >= t_begin && tcur < t_end && (rel / ATT_WK) % nw == w;
    const int own_tw = t_begin + (rel / ATT_WK) * ATT_WK;
    const int slot = tcur - own_tw;
    if (owner) {
        size_t o;
        if (PAGED)
            o = kv_row<HD, PAGED>(p, p.tables[(size_t)b * p.mbps + tcur / ATT_BS], g, tcur);
        else
            o = kv_row<HD, PAGED>(p, b, g, tcur);
        if (KV8) {
            // e4m3 of value / scale; the wave's own row keeps the bytes in the
            // order of the fp8 QK operand (plain dim order: a lane loads
            // contiguous dims)
            uint8_t* kc8 = reinterpret_cast<uint8_t*>(p.kc);
            uint8_t* vc8 = reinterpret_cast<uint8_t*>(p.vc);
            uint8_t* kn8 = reinterpret_cast<uint8_t*>(&sm.knew[w][0]);
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                const int d = lane * DPL + e;
                const uint32_t k8 = f32_to_e4m3(kv_[e] / p.k_scale);
                const uint32_t v8 = f32_to_e4m3(vv[e] / p.v_scale);
                kc8[o + d] = (uint8_t)k8;
                vc8[o + d] = (uint8_t)v8;
                kn8[d] = (uint8_t)k8;
                vnew[e] = __builtin_amdgcn_cvt_pk_f32_fp8((int)v8, false)[0];
            }
        } else {
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
    wave_lds_sync();
    QD_MARK(2);

    // ---- QK operands of the matrix core: v_mfma_f32_16x16x32_f16 with
    // M = the step's 16 keys, N = query heads (columns >= GQ are zero), K = 32
    // dims per instruction.  Lane l holds dims 8*(l/16) .. +7 of each 32-dim
    // slice: of key l%16 for A (straight from the K loads) and of head l%16 for
    // B.  q enters as a pair of f16 (hi + lo, about 22 significant bits); the
    // two products accumulate in one f32 result, and K is f16 already.
    half8 bhi[NI], blo[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int col = lane & 15;
        float qf[8];
        // dims of slice i in this lane group: 32i + 8kg .. (f16 K, the loads'
        // order), or kg*8*NI + 8i .. (fp8 K: a lane loads contiguous dims)
        const float* src = &sm.q[w][col < GQ ? col : 0][KV8 ? 8 * NI * (lane >> 4) + 8 * i
                                                            : 32 * i + 8 * (lane >> 4)];
        const float4 q0 = *reinterpret_cast<const float4*>(src);
        const float4 q1 = *reinterpret_cast<const float4*>(src + 4);
        qf[0] = q0.x; qf[1] = q0.y; qf[2] = q0.z; qf[3] = q0.w;
        qf[4] = q1.x; qf[5] = q1.y; qf[6] = q1.z; qf[7] = q1.w;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = col < GQ ? qf[e] : 0.f;
            const _Float16 h = (_Float16)v;
            bhi[i][e] = h;
            blo[i][e] = (_Float16)(v - (float)h);
        }
    }

    // ---- the wave's steps.  m_c, l_c: running max and sum of head
    // c = lane % 16 (meaningful for c < GQ), the same in the lanes c + 16 k.
    float m_c = -INFINITY, l_c = 0.f, acc[GQ][DPL];
#pragma unroll
    for (int j = 0; j < GQ; ++j)
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            acc[j][e] = 0.f;
    const int col = lane & 15, kg = lane >> 4;
    for (int tw = tw0; tw < t_end; tw += wstride) {
        Step nxt;
        const bool more = tw + wstride < t_end;
        if (more)
            load_step(nxt, tw + wstride);
        const int nvalid = min(ATT_WK, t_end - tw);
        const bool own_here = owner && tw == own_tw;
        uint4 kr[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i)
            kr[i] = cur_st.k[i];
        if (own_here && kk == slot) {
            if (KV8) {
                const uint8_t* kn8 = reinterpret_cast<const uint8_t*>(&sm.knew[w][0]);
#pragma unroll
                for (int u = 0; u < NI / 2; ++u)
                    kr[u] = *reinterpret_cast<const uint4*>(kn8 + 8 * NI * kg + 16 * u);
            } else {
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    kr[i] = *reinterpret_cast<const uint4*>(&sm.knew[w][32 * i + 8 * kg]);
            }
        }
        QD_MARK(4);
        floatx4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            half8 a;
            if (KV8) {
                // 8 e4m3 bytes of slice i -> f16 (exact: every e4m3 value is an f16 value)
                const uint4 kq = kr[i / 2];
                const uint32_t w0 = (i & 1) ? kq.z : kq.x, w1 = (i & 1) ? kq.w : kq.y;
                const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
                const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
                const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
                const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
                a[0] = (_Float16)f0[0]; a[1] = (_Float16)f0[1];
                a[2] = (_Float16)f1[0]; a[3] = (_Float16)f1[1];
                a[4] = (_Float16)f2[0]; a[5] = (_Float16)f2[1];
                a[6] = (_Float16)f3[0]; a[7] = (_Float16)f3[1];
            } else {
                a = __builtin_bit_cast(half8, kr[i]);
            }
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bhi[i], sc, 0, 0, 0);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, blo[i], sc, 0, 0, 0);
        }
        QD_MARK(5);
        // sc[r] = score of key 4*kg + r for head col; online softmax per head
        // over the 16 keys: 4 registers, then the 4 lane groups kg
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sc[r] = (4 * kg + r < nvalid) ? sc[r] : -INFINITY;
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
        float pr[4], ps = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pr[r] = expf(sc[r] - mnew);   // 0 for a masked key
            ps += pr[r];
        }
        {
            float lo, hi;
            lanes::swap16(ps, lo, hi);
            ps = lo + hi;
            lanes::swap32(ps, lo, hi);
            ps = lo + hi;
        }
        const float alpha_c = expf(m_c - mnew);   // 0 on the first step (m = -inf)
        l_c = fmaf(l_c, alpha_c, ps);
        m_c = mnew;
        if (col < GQ) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sm.p[w][4 * kg + r][col] = pr[r];
        }
        float alpha[GQ];
#pragma unroll
        for (int j = 0; j < GQ; ++j)
            alpha[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha_c), j));
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
            if (KV8) {
                const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw, false);
                vf[0] = f[0];
                if (DPL == 2)
                    vf[DPL - 1] = f[1];
            } else {
                vf[0] = f16_to_f32((uint16_t)(vw & 0xffffu));
                if (DPL == 2)
                    vf[DPL - 1] = f16_to_f32((uint16_t)(vw >> 16));
            }
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
    if (lane < GQ) {
        sm.m[w][lane] = m_c;
        sm.l[w][lane] = l_c;
    }
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            sm.acc[w][j][lane * DPL + e] = KV8 ? acc[j][e] * p.v_scale : acc[j][e];
    }
    QD_MARK(7);
    __syncthreads();
    const size_t pstride = HD + 2;
    const bool merge_here = p.counters != nullptr;
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
        if (merge_here) {
            // agent-scope stores: seen by the merging workgroup on any XCD
            __hip_atomic_store(&pp[d], A, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (d == 0) {
                __hip_atomic_store(&pp[HD], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&pp[HD + 1], L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            pp[d] = A;
            if (d == 0) {
                pp[HD] = M;
                pp[HD + 1] = L;
            }
        }
    }
    if constexpr (QMODE == 2 && attn_split_out_ok(HD, GQ)) {
        if (merge_here && p.xp) {   // uniform
            // the LDS rows of acc and m were all read above, before the partial stores
            attn_merge_split<HD, GQ>(p, b, g, kv_len, &sm.last, &sm.acc[0][0][0], &sm.m[0][0]);
            QD_MARK(3);
            return;
        }
    }
    if (merge_here)
        attn_merge_last<HD, GQ, FUSED>(p, b, g, kv_len, &sm.last);
    QD_MARK(3);
}

template <int HD, int GQ, bool PAGED, int QMODE, bool KV8 = false>
__global__ void __launch_bounds__(AttnMaxWaves<GQ>::value * WAVE) k_attn_split(AttnParams p)
{
    __shared__ AttnSmem<HD, GQ> sm;
    attn_split_body<HD, GQ, PAGED, QMODE, false, KV8>(p, (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z, sm,
                                                 [] {});
}

constexpr int ATT_CNT = 512;   // combine threads per head

// Merge the partials of one (sequence, head): grid (nq, B), 512 threads in
// groups of HD; group sg takes splits sg, sg + SG, ...  Each round issues all
// of its loads (acc, m, l of U splits, U * SG >= the split count on the host
// so that one round does, and no more loads than the splits need) before
// using them; only splits holding keys below kv_len count.  The groups' (max, numerator, denominator)
// are merged through LDS in a fixed order.
template <int HD, int U = 16>
__global__ void __launch_bounds__(ATT_CNT) k_attn_combine(const float* __restrict__ part,
                                                          int nsplit_all, int chunk,
                                                          const int32_t* __restrict__ kv_lens,
                                                          const int32_t* __restrict__ pos,
                                                          int max_kv, int nq, float* __restrict__ out)
{
    constexpr int SG = ATT_CNT / HD;
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
