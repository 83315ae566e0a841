// fused_layers.h -- every layer of a decode step in one persistent kernel (gfx950).
//
// The same steps as the per-layer kernels of step_kernels.h (inferencelayer
// cuda_llm.rs page, CudaQwen3::step; ferrum-kernels cuda_decode.rs page,
// CudaDecodeRunner::decode_step): per layer q|k|v GEMV, attention (per-head
// q/k norm + rotary, K/V write, split-KV partials, merge), o GEMV + residual,
// gate|up GEMV + SwiGLU, down GEMV + residual.  Here one workgroup per CU runs
// all of them, phase after phase, one launch per layer, and a device-wide
// barrier separates the phases inside a layer instead of a kernel boundary.
// What that buys: before a workgroup waits for the previous phase it has
// already issued the loads of its first weight items of the next phase (the
// small q|k|v and o tiles fit in registers whole), and an attention workgroup
// its first K/V rows, so the wait overlaps HBM traffic instead of idling it.
//
// Coherence inside the launch.  Every value a phase produces for other
// workgroups is stored agent-scope (write-through to memory) and read
// agent-scope; each thread waits for its own stores before its workgroup
// arrives at the barrier.  Every layer has its own activation buffers.  The
// relaxed arrival adds are ordered after those stores by a gfx9 property:
// stores count in vmcnt, so s_waitcnt vmcnt(0) means they are complete at the
// agent's coherence point (a release add would write back the XCD's L2 in
// every workgroup).
//
// Barrier: 16 arrival counters 256 B apart (workgroup w adds 1 to counter
// w % 16, one relaxed agent-scope add per workgroup); a waiter polls all 16
// with one load per lane.  Counters only grow within a step (k_embed zeroes
// them before the first layer); after n barriers counter k holds n times its
// group size.
// Every wait is bounded: past the spin limit the workgroup records bit 2 of
// StepState::error and stops waiting (the step's results are then invalid, the
// launch still ends).
#pragma once

#include "step_kernels.h"

namespace qd {

constexpr int FUSED_WAVES = 8;
constexpr int FUSED_THREADS = FUSED_WAVES * WAVE;
constexpr int FB_GROUPS = 16;
constexpr int FB_STRIDE = 64;   // uints between counters
constexpr int FB_WORDS = FB_GROUPS * FB_STRIDE;
constexpr int FB_SPIN_LIMIT = 1 << 16;

// Timeline marks of the persistent kernel in profiling builds only (like
// QD_MARK): 16 per workgroup and layer, at qd_ftl[(l * gridDim.x + w) * 16 + k].
#ifdef QD_TIMELINE
__constant__ uint64_t* qd_ftl;
#define QD_FMARK(l, k)                                                                   \
    do {                                                                                 \
        if (threadIdx.x == 0 && qd_ftl)                                                  \
            qd_ftl[((size_t)(l) * gridDim.x + blockIdx.x) * 16 + (k)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#else
#define QD_FMARK(l, k) \
    do {               \
    } while (0)
#endif

template <class T>
QD_DEV const __attribute__((address_space(1))) T* gptr(const T* p)
{
    return (const __attribute__((address_space(1))) T*)p;
}

struct FusedBarrier {
    unsigned* ctr;
    int32_t* err;
    int* broken;   // LDS flag of this workgroup
    int spin_limit;
    QD_DEV void arrive() const
    {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's stores are done
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(ctr + (blockIdx.x % FB_GROUPS) * FB_STRIDE, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    // wait until n barriers are complete
    QD_DEV void wait(unsigned n) const
    {
        if (threadIdx.x < WAVE && !*broken) {
            const int k = threadIdx.x < FB_GROUPS ? (int)threadIdx.x : 0;
            const unsigned G = gridDim.x;
            const unsigned per = G / FB_GROUPS + ((unsigned)k < G % FB_GROUPS ? 1u : 0u);
            const unsigned target = n * per;
            const unsigned* c = ctr + k * FB_STRIDE;
            for (int spins = 0;; ++spins) {
                const unsigned v = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (__all(v >= target))
                    break;
                if (spins >= spin_limit) {
                    if (threadIdx.x == 0) {
                        *broken = 1;
                        __hip_atomic_fetch_or(err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        __syncthreads();
    }
};

// x staging from a vector other workgroups of this launch wrote: 64-bit
// agent-scope loads (then the usual LDS layout)
template <int NT>
QD_DEV void stage_x_load_agent(const float* __restrict__ x, int nb, XStage<NT>& st)
{
    const int n4 = nb * 8;
#pragma unroll
    for (int u = 0; u < XStage<NT>::MAXU; ++u) {
        if (u * NT < n4) {   // uniform
            const int i = min((int)threadIdx.x + u * NT, n4 - 1);
            const uint64_t* p = reinterpret_cast<const uint64_t*>(x) + 2 * i;
            const uint64_t lo = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t hi = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            st.v[u] = make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                                  __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
        }
    }
}

// RmsPartials with agent-scope loads
struct RmsAgent {
    const float* ss_part;
    int n_part;
    float v[RMS_U];
    QD_DEV void issue()
    {
        const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
        for (int u = 0; u < RMS_U; ++u)
            v[u] = ld_f32<true>(ss_part + min(lane + u * WAVE, n_part - 1));
    }
    QD_DEV float finish(int n, float eps) const
    {
        const int lane = threadIdx.x & (WAVE - 1);
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < RMS_U; ++u)
            s += (lane + u * WAVE < n_part) ? v[u] : 0.f;
        for (int i = lane + RMS_U * WAVE; i < n_part; i += WAVE)
            s += ld_f32<true>(ss_part + i);
        s = group_sum<WAVE>(s);
        return 1.0f / sqrtf(s / (float)n + eps);
    }
};

// ----------------------------------------------------------------- epilogues

struct FEpiScaled {   // y = acc / rms
    float* y;
    int N;
    RmsAgent rp;
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
                    st_f32<true>(y + row0 + r, acc[r] * inv);
        }
    }
};

// x_out = x_in + acc; u_out = x_out * w_next; running sum of x_out^2.  The
// rows of the first tile are loaded by issue(); a later tile of the same
// workgroup loads its own.
template <int RPS>
struct FEpiResidual {
    const float* x_in;
    float* x_out;
    float* u_out;
    const float* w_next;
    int N;
    float ss;
    int row_pre;
    float px[RPS], pw[RPS];
    QD_DEV void load_rows(int row0)
    {
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            const int row = min(row0 + r, N - 1);
            px[r] = ld_f32<true>(x_in + row);
            pw[r] = w_next[row];
        }
        row_pre = row0;
    }
    QD_DEV void issue(int row0) { load_rows(row0); }
    QD_DEV void finish() {}
    QD_DEV void tile(int row0, const float (&acc)[RPS], bool lead)
    {
        if (row0 != row_pre)
            load_rows(row0);
        if (lead) {
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const int row = row0 + r;
                if (row < N) {
                    const float nx = px[r] + acc[r];
                    st_f32<true>(x_out + row, nx);
                    st_f32<true>(u_out + row, nx * pw[r]);
                    ss = fmaf(nx, nx, ss);
                }
            }
        }
    }
};

// rows interleaved (2i = gate_i, 2i+1 = up_i): act[i] = silu(g) * up
struct FEpiSwiglu {
    float* act;
    int N;
    RmsAgent rp;
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
                    st_f32<true>(act + ((row0 + r) >> 1), gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up);
                }
            }
        }
    }
};

// ----------------------------------------------------------------- GEMV phase

// One GEMV phase of the persistent kernel: the gemv_run work mapping (tiles
// strided by gridDim.x, NBUF register buffers, unrolled chunks) with the
// phase order: first weight items -> wait() -> the epilogue's loads and x
// (agent-scope) -> the stream.
template <int LPR, int RPS, int BG, int NBUF, int UNR, class Epi, class Wait>
QD_DEV void fused_gemv(const uint16_t* D, const uint8_t* Q, const float* x, int N, int nb, float* xl,
                       float* xs, Epi& epi, Wait&& wait)
{
    static_assert(NBUF >= 1 && NBUF <= 6 && UNR >= NBUF, "buffers");
    using G = GemvGeom<LPR, RPS, FUSED_WAVES>;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int slot = lane / LPR, lr = lane % LPR;
    const int ntiles = (N + G::ROWS - 1) / G::ROWS;
    const int ngroups = (nb + LPR * BG - 1) / (LPR * BG);
    const int my_tiles = (int)blockIdx.x < ntiles ? (ntiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    const int nitems = my_tiles * ngroups;

    auto load = [&](GemvBuf<RPS, BG>& bf, int i) {
        i = max(0, min(i, nitems - 1));   // clamped: never a branch around a load
        const int tile = (int)blockIdx.x + (i / ngroups) * (int)gridDim.x;
        const int grp = i % ngroups;
        const int row0 = tile * G::ROWS + wave * G::RPW + slot * RPS;
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            const uint32_t rb = __umul24((uint32_t)min(row0 + r, N - 1), (uint32_t)nb);
#pragma unroll
            for (int g = 0; g < BG; ++g) {
                const uint32_t blk = rb + (uint32_t)min(grp * LPR * BG + g * LPR + lr, nb - 1);
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 t = *gptr(reinterpret_cast<const u32x4*>(Q + blk * 16u));
                bf.q[g][r] = make_uint4(t.x, t.y, t.z, t.w);
                bf.d[g][r] = *gptr(D + blk);
            }
        }
    };
    float acc[RPS];
#pragma unroll
    for (int r = 0; r < RPS; ++r)
        acc[r] = 0.f;
    auto compute = [&](const GemvBuf<RPS, BG>& bf, int i) {
        const int tile = (int)blockIdx.x + (i / ngroups) * (int)gridDim.x;
        const int grp = i % ngroups;
#pragma unroll
        for (int g = 0; g < BG; ++g) {
            const int b = grp * LPR * BG + g * LPR + lr;
            if (b < nb) {
                float4 xv[8];
                const float4* xp = reinterpret_cast<const float4*>(xl + b * XPAD);
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    xv[k] = xp[k];
                const float m8 = (-8.f * Q4_SUB) * xs[b];
#pragma unroll
                for (int r = 0; r < RPS; ++r)
                    acc[r] = fmaf(f16_to_f32((uint16_t)bf.d[g][r]), q4_block_dot(bf.q[g][r], xv) + m8,
                                  acc[r]);
            }
        }
        if (grp == ngroups - 1) {
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                acc[r] = group_sum<LPR>(acc[r]) * Q4_UNSUB;
            const int row0 = tile * G::ROWS + wave * G::RPW + slot * RPS;
            epi.tile(row0, acc, lr == 0);
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                acc[r] = 0.f;
        }
    };

    GemvBuf<RPS, BG> bufs[NBUF];
#pragma unroll
    for (int j = 0; j + 1 < NBUF; ++j)
        load(bufs[j], j);
    // a compiler barrier keeps these loads ahead of the wait (else they are
    // sunk next to their first use, after it)
    asm volatile("" ::: "memory");
    wait();
    epi.issue((int)blockIdx.x * G::ROWS + wave * G::RPW + slot * RPS);
    XStage<G::NT> xst;
    stage_x_load_agent<G::NT>(x, nb, xst);
    stage_x_store<G::NT>(nb, xst, xl, xs);   // ends with a barrier
    epi.finish();
    for (int base = 0; base < nitems; base += UNR) {
        if (base > 0) {
#pragma unroll
            for (int j = 0; j + 1 < NBUF; ++j)
                load(bufs[j], base + j);
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            if (u + NBUF - 1 < UNR)
                load(bufs[(u + NBUF - 1) % NBUF], base + u + NBUF - 1);
            asm volatile("" ::: "memory");
            if (base + u < nitems)
                compute(bufs[u % NBUF], base + u);
        }
    }
}

// ----------------------------------------------------------------- the kernel

// One layer's weights and its activation buffers (device table, one entry per
// layer).  x_in/u_in/ss_in are the previous layer's x_out/u_out/ss_out (or
// the embedding's); every other buffer belongs to this layer only.
struct FusedLayer {
    const uint16_t *qkv_d, *o_d, *gu_d, *down_d;
    const uint8_t *qkv_q, *o_q, *gu_q, *down_q;
    const float *ffn_norm, *w_next, *q_norm, *k_norm;
    uint16_t *kc, *vc;
    const float *x_in, *u_in, *ss_in;
    int n_in;
    float *qkv, *part, *att, *xm, *um, *ssa, *act, *x_out, *u_out, *ss_out;
    unsigned* cnt;
};

struct FusedArgs {
    const FusedLayer* layers;
    int L, H, nq, nkv, hd, I, qkv_rows;
    float eps;
    const int32_t* tables;   // paged block table or nullptr
    int mbps;
    const int32_t* pos;
    int max_kv;
    float scale;
    int chunk, nsplit, qk_norm, rot;
    const float* rope_cur;
    unsigned* bar;
    int32_t* err;
    int spin_limit;   // polls before a wait gives up (FB_SPIN_LIMIT)
};

// GEMV configurations of the phases (LPR, RPS, block group, buffers, unroll):
// every workgroup prefetches NBUF-1 items of its next phase before it waits
#define QD_FCFG_QKV 64, 3, 1, 3, 4
#define QD_FCFG_O 64, 2, 1, 3, 4
#define QD_FCFG_GU 32, 2, 1, 3, 12
#define QD_FCFG_DOWN 64, 2, 1, 4, 6

template <int HD, int GQ>
constexpr size_t fused_lds_bytes(int nb_max)
{
    const size_t g = (size_t)gemv_lds_floats(nb_max) * sizeof(float);
    const size_t a = sizeof(AttnSmem<HD, GQ>);
    return g > a ? g : a;
}

// One layer per launch (a loop over the layers inside the kernel lets the
// compiler hoist every layer-invariant address out of it and spill).  The
// barrier counters run on across the layers of a step: layer l starts after
// 4 l barriers.
template <int HD, int GQ, bool PAGED>
__global__ void __launch_bounds__(FUSED_THREADS) k_layer_fused(FusedArgs a, int l)
{
    static_assert(AttnMaxWaves<GQ>::value == FUSED_WAVES, "attention workgroups of 8 waves");
    extern __shared__ __align__(16) float smem[];   // x staging | attention, one at a time
    __shared__ float red[FUSED_WAVES];
    __shared__ int broken;
    if (threadIdx.x == 0)
        broken = 0;
    __syncthreads();
    const FusedBarrier bar{a.bar, a.err, &broken, a.spin_limit};
    const unsigned nbar0 = 4u * (unsigned)l;
    unsigned nbar = nbar0;   // barriers completed before the phase to come
    [[maybe_unused]] int phase = 0;   // marks 3 phase (entry), 3 phase + 1 (after the wait), 3 phase + 2 (end)
    auto wait = [&] {
        if (nbar > nbar0)   // the layer's first phase follows a kernel boundary
            bar.wait(nbar);
        QD_FMARK(l, 3 * phase + 1);
    };
    const int nbH = a.H / 32, nbA = a.nq * a.hd / 32, nbI = a.I / 32;
    float* xl = smem;
    auto xs_of = [&](int nb) { return smem + nb * XPAD; };
    auto block_ss = [&](float v, float* out) {
        v = block_sum256(v, red);
        if (threadIdx.x == 0)
            st_f32<true>(out + blockIdx.x, v);
    };
    AttnSmem<HD, GQ>& asm_ = *reinterpret_cast<AttnSmem<HD, GQ>*>(smem);

    {
        const FusedLayer& Lw = a.layers[l];
        // q | k | v
        QD_FMARK(l, 0);
        {
            FEpiScaled e{Lw.qkv, a.qkv_rows, {Lw.ss_in, Lw.n_in}, a.H, a.eps};
            fused_gemv<QD_FCFG_QKV>(Lw.qkv_d, Lw.qkv_q, Lw.u_in, a.qkv_rows, nbH, xl, xs_of(nbH), e, wait);
        }
        QD_FMARK(l, 2);
        bar.arrive();
        ++nbar;
        phase = 1;
        QD_FMARK(l, 3);
        // attention: workgroup w < nsplit * nkv takes split w % nsplit of kv head w / nsplit
        {
            AttnParams p = AttnParams{};
            p.q = Lw.qkv;
            p.k = Lw.kc;
            p.v = Lw.vc;
            p.tables = a.tables;
            p.mbps = a.mbps;
            p.kv_lens = nullptr;
            p.pos = a.pos;
            p.max_kv = a.max_kv;
            p.nq = a.nq;
            p.nkv = a.nkv;
            p.scale = a.scale;
            p.chunk = a.chunk;
            p.nsplit = a.nsplit;
            p.part = Lw.part;
            p.out = Lw.att;
            p.counters = Lw.cnt;
            p.qk_norm = a.qk_norm;
            p.q_norm = Lw.q_norm;
            p.k_norm = Lw.k_norm;
            p.eps = a.eps;
            p.rot = a.rot;
            p.rope_cur = a.rope_cur;
            p.kc = Lw.kc;
            p.vc = Lw.vc;
            const int w = blockIdx.x;
            if (w < a.nsplit * a.nkv)
                attn_split_body<HD, GQ, PAGED, 1, true, false>(p, w % a.nsplit, w / a.nsplit, 0, asm_, wait);
            else
                wait();
        }
        QD_FMARK(l, 5);
        bar.arrive();
        ++nbar;
        phase = 2;
        QD_FMARK(l, 6);
        // o + residual
        {
            FEpiResidual<2> e{Lw.x_in, Lw.xm, Lw.um, Lw.ffn_norm, a.H, 0.f, -1};
            fused_gemv<QD_FCFG_O>(Lw.o_d, Lw.o_q, Lw.att, a.H, nbA, xl, xs_of(nbA), e, wait);
            block_ss(e.ss, Lw.ssa);
        }
        QD_FMARK(l, 8);
        bar.arrive();
        ++nbar;
        phase = 3;
        QD_FMARK(l, 9);
        // gate | up + SwiGLU
        {
            FEpiSwiglu e{Lw.act, 2 * a.I, {Lw.ssa, (int)gridDim.x}, a.H, a.eps};
            fused_gemv<QD_FCFG_GU>(Lw.gu_d, Lw.gu_q, Lw.um, 2 * a.I, nbH, xl, xs_of(nbH), e, wait);
        }
        QD_FMARK(l, 11);
        bar.arrive();
        ++nbar;
        phase = 4;
        QD_FMARK(l, 12);
        // down + residual
        {
            FEpiResidual<2> e{Lw.xm, Lw.x_out, Lw.u_out, Lw.w_next, a.H, 0.f, -1};
            fused_gemv<QD_FCFG_DOWN>(Lw.down_d, Lw.down_q, Lw.act, a.H, nbI, xl, xs_of(nbI), e, wait);
            block_ss(e.ss, Lw.ss_out);
        }
        QD_FMARK(l, 14);
    }
}

}  // namespace qd
