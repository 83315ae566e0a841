// qd_api.hip -- C ABI and runtime of the batch-1 q4_0 decode library (gfx950).
//
// The runtime owns: device copies of the weights (q|k|v rows concatenated,
// gate/up rows interleaved), the f16 KV cache (contiguous, or a paged pool
// with a block table fixed at create time), every step buffer (allocated
// once in qd_create: nothing is allocated per step), host-built rotary
// cos/sin tables, the device-resident step state (position, stored token per
// position, forced-prefix length) and an optional hipGraph of one step.
// (inferencelayer cuda_llm.rs page, CudaQwen3 fields, step, seed, capture,
// run_graph, tokens; ferrum-kernels cuda_decode.rs page, GpuPagedKvPool use
// and init_kv_cache_paged.)
#include "qd.h"

#include "fused_layers.h"
#include "gemv_cfg.h"
#include "gemv_batch.h"
#include "gemv_batch_mfma.h"
#include "gemv_experts.h"
#include "prefill_kernels.h"
#include "prefill_attn.h"
#include "step_batch.h"
#include "stream_read.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

using namespace qd;

// ------------------------------------------------------------------ errors

static thread_local std::string g_err;

static int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

#define HIP_TRY(expr)                                                                     \
    do {                                                                                  \
        hipError_t e_ = (expr);                                                           \
        if (e_ != hipSuccess)                                                             \
            return fail(QD_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));          \
    } while (0)

extern "C" const char* qd_last_error(void) { return g_err.c_str(); }

// ------------------------------------------------------------------ GEMV launch

// attention workgroups of a decode step and the most waves per workgroup
// (measured best on MI355X; compile-time overridable for tuning builds)
#ifndef QD_ATT_MODEL_WGS
#define QD_ATT_MODEL_WGS 160
#endif
#ifndef QD_ATT_MODEL_WAVES
#define QD_ATT_MODEL_WAVES 8
#endif
static constexpr int ATT_MODEL_WGS = QD_ATT_MODEL_WGS;

static hipError_t launch_gemv_plain(const uint16_t* d, const uint8_t* q, const float* x, float* y,
                                    int N, int K, hipStream_t s)
{
    const int nb = K / 32, lpr = pick_lpr(nb);
    const size_t lds = gemv_lds_bytes(nb);
    if (N <= 8192) {
        QD_GEMV(k_gemv_plain, (QD_CFG_O), lpr, gemv_grid(CFG_O, lpr, N), lds, s, d, q, x, y, N, nb);
    } else if (N <= 65536) {
        const int l = pick_lpr(nb, CFG_GU.lpr_max);
        QD_GEMV(k_gemv_plain, (QD_CFG_GU), l, gemv_grid(CFG_GU, l, N), lds, s, d, q, x, y, N, nb);
    } else {
        QD_GEMV(k_gemv_plain, (QD_CFG_HEAD), lpr, gemv_grid(CFG_HEAD, lpr, N), lds, s, d, q, x, y, N, nb);
    }
    return hipGetLastError();
}

// Y[b] = W X[b] for b < B (1 <= B <= 16) through the batched GEMV kernels
// (defined with qd_gemv_q4_0_batch below)
static hipError_t gemv_batch_launch(const uint16_t* d, const uint8_t* q, const float* x, float* y, int N, int K,
                                    int B, hipStream_t s);
// the matrix-core batched GEMV, K in ks slices (defined below)
template <int NC>
static hipError_t launch_gemv_batch_mfma(const uint16_t* d, const uint8_t* q, const float* x, float* y,
                                         int N, int nb, hipStream_t s, int ks = 1);

// workgroups of the attention of a batched decode step over all its sequences
// (measured at the Qwen3-8B shape, 16 / 8 / 4 sequences at kv_len ~550:
// 256 against 64 .. 2048 is the fastest for each)
#ifndef QD_ATT_BATCH_WGS
#define QD_ATT_BATCH_WGS 256
#endif
// sequences from which a batched step's attention writes the o product's split
// input itself (Qwen3-8B shape, one box: 2.94 -> 2.88 ms per step at 8, 3.10
// -> 3.06 at 16, 2.797 -> 2.813 at 4)
static constexpr int ATT_SPLIT_OUT_MIN_B = 8;

// ------------------------------------------------------------------ model

struct DevQ4 {
    uint16_t* d = nullptr;
    uint8_t* qs = nullptr;
    int rows = 0, cols = 0, nb = 0;
};

struct DevLayer {
    DevQ4 qkv, o, gu, down;
    float *attn_norm = nullptr, *ffn_norm = nullptr, *q_norm = nullptr, *k_norm = nullptr;
    uint16_t *kc = nullptr, *vc = nullptr;
};

struct qd_model {
    int H, L, nq, nkv, hd, I, V, rot, qkv_rows, max_seq, qk_norm, paged, nblocks;
    float eps;
    // sequences stepped together (qd_create_batch; 1 for qd_create) and the
    // written prefix of each (see hw below)
    int B = 1;
    std::vector<int> hwb;
    int rstride = 2;                  // floats of rotary factors per sequence
    // buffers of the batched step ([B] rows each)
    float *bx = nullptr, *bh = nullptr, *bqkv = nullptr, *battn = nullptr, *bo = nullptr;
    float *bgu = nullptr, *bact = nullptr, *blog = nullptr, *bcval = nullptr;
    // the batched products' inputs, split (gemv_batch_mfma.h): hidden-sized
    // (q|k|v, gate|up, LM head), attention output (o), SwiGLU output (down)
    _Float16 *xp_h = nullptr, *xp_o = nullptr, *xp_i = nullptr;
    float *xs_h = nullptr, *xs_o = nullptr, *xs_i = nullptr;
    float* sq_h = nullptr;   // chunk sums of x^2 of the hidden-sized split (its norm's 1/rms)
    int32_t* bcidx = nullptr;
    int bG = 1, bchunk = 1;
    int ks_qkv = 1, ks_o = 1, ks_gu = 1, ks_down = 1;   // K slices of the batched products
    // the written prefix of the KV cache: positions 0 .. hw hold K/V of the
    // current sequence (-1: none).  A step at p writes p and makes [0, p] the
    // prefix; a step may start at most one position past it.
    int hw = -1;
    // chunked prefill buffers (allocated by the first qd_prefill)
    struct {
        float *X = nullptr, *Q = nullptr, *O = nullptr, *HF = nullptr;
        // the products' outputs as K-slice partial slabs: q|k|v, o and down, gate|up
        float *QKV = nullptr, *OD = nullptr, *GU = nullptr;
        int ks_qkv = 1, ks_o = 1, ks_gu = 1, ks_down = 1;
        // the products' inputs split (gemv_batch_mfma.h), one vector slot per
        // position: hidden-sized, attention output, SwiGLU output
        _Float16 *xp_h = nullptr, *xp_o = nullptr, *xp_i = nullptr;
        float *xs_h = nullptr, *xs_o = nullptr, *xs_i = nullptr;
        float* sq_h = nullptr;   // chunk sums of x^2 of the hidden-sized split
        float* fa = nullptr;                       // k_pf_attn partials [T][nq][FA_MAXS][hd + 2]
        int32_t *lens = nullptr, *iota = nullptr;
        float* ws = nullptr;
        AttnGeom geo;
        bool ready = false;
    } pf;
    int kv_fp8 = 0;                 // fp8 e4m3 K/V cache (1 byte per element)
    int attn_gate = 0;              // attention output gate rows after q | k | v
    float k_scale = 1.f, v_scale = 1.f;
    std::vector<DevLayer> layers;
    DevQ4 embed, lm;
    float* final_norm = nullptr;
    float *rope_cos = nullptr, *rope_sin = nullptr;   // [max_seq][rot/2]
    float* rope_cur = nullptr;                        // cos, sin at the step's position
    float* ones_hd = nullptr;                         // [head_dim] of 1 (no q/k norm)
    unsigned* attn_cnt = nullptr;                     // [n_kv] split counters, zero between steps
    int32_t* table = nullptr;
    // step buffers
    float *x = nullptr, *u = nullptr, *ss_part = nullptr, *qkv_raw = nullptr;
    float *attn = nullptr, *act = nullptr, *logits = nullptr, *arg_val = nullptr;
    int32_t* arg_idx = nullptr;
    float* attn_part = nullptr;
    int attn_waves = 0, attn_chunk = 0, attn_nsplit = 0;
    StepState* st = nullptr;
    int32_t *ids = nullptr, *pred = nullptr;
    // launch geometry
    int lpr_qkv, grid_qkv, lpr_o, grid_o, lpr_gu, grid_gu, lpr_down, grid_down;
    bool small_qkv = false, small_o = false, small_down = false;   // one-row configurations
    int lpr_lm, grid_lm, grid_embed;
    // graph
    int use_graph = 0;
    hipStream_t cap_stream = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    std::vector<void*> allocs;
    StepState* h_state = nullptr;  // pinned host staging
    // persistent layer kernel (fused = 1): one workgroup per CU runs every layer
    int fused = 0, fused_grid = 0, fused_nsplit = 0, fused_chunk = 0;
    size_t fused_lds = 0;
    FusedLayer* flayers = nullptr;   // device table [L]
    unsigned* fbar = nullptr;        // barrier counters [FB_WORDS]
    float *fX = nullptr, *fU = nullptr, *fSS = nullptr;   // [L+1] chains: x, u, sum-of-squares partials
    int fss_stride = 0;
    int fused_spin = FB_SPIN_LIMIT;
};

static int dev_alloc(qd_model* m, void** p, size_t bytes)
{
    if (bytes == 0)
        bytes = 16;
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        return fail(e == hipErrorOutOfMemory ? QD_ENOMEM : QD_EHIP, "hipMalloc(%zu): %s", bytes,
                    hipGetErrorString(e));
    }
    m->allocs.push_back(*p);
    return QD_OK;
}

#define QD_TRY(expr)                  \
    do {                              \
        int r_ = (expr);              \
        if (r_ != QD_OK)              \
            return r_;                \
    } while (0)

template <class T>
static int dev_alloc_t(qd_model* m, T** p, size_t count)
{
    return dev_alloc(m, reinterpret_cast<void**>(p), count * sizeof(T));
}

static int check_q4(const qd_q4_0& w, int rows, int cols, const char* name)
{
    if (!w.d || !w.qs)
        return fail(QD_EINVAL, "%s: null pointer", name);
    if (w.rows != rows || w.cols != cols)
        return fail(QD_EINVAL, "%s: shape [%d, %d], expected [%d, %d]", name, w.rows, w.cols, rows,
                    cols);
    return QD_OK;
}

// Upload row blocks of several host q4_0 matrices into one device matrix.
// `order` lists (source index, source row) for every destination row.
struct RowSrc {
    const qd_q4_0* w;
    int row;
};

static int upload_rows(qd_model* m, DevQ4* dst, const std::vector<RowSrc>& rows, int cols,
                       hipStream_t s)
{
    const int nb = cols / 32;
    dst->rows = (int)rows.size();
    dst->cols = cols;
    dst->nb = nb;
    QD_TRY(dev_alloc_t(m, &dst->d, (size_t)dst->rows * nb));
    QD_TRY(dev_alloc_t(m, &dst->qs, (size_t)dst->rows * nb * 16));
    std::vector<uint16_t> hd((size_t)dst->rows * nb);
    std::vector<uint8_t> hq((size_t)dst->rows * nb * 16);
    for (size_t r = 0; r < rows.size(); ++r) {
        const qd_q4_0* w = rows[r].w;
        const size_t sr = (size_t)rows[r].row;
        memcpy(&hd[r * nb], w->d + sr * nb, sizeof(uint16_t) * nb);
        memcpy(&hq[r * nb * 16], w->qs + sr * nb * 16, (size_t)nb * 16);
    }
    HIP_TRY(hipMemcpyAsync(dst->d, hd.data(), hd.size() * sizeof(uint16_t), hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(dst->qs, hq.data(), hq.size(), hipMemcpyHostToDevice, s));
    HIP_TRY(hipStreamSynchronize(s));
    return QD_OK;
}

static int upload_whole(qd_model* m, DevQ4* dst, const qd_q4_0& w, hipStream_t s)
{
    const int nb = w.cols / 32;
    dst->rows = w.rows;
    dst->cols = w.cols;
    dst->nb = nb;
    QD_TRY(dev_alloc_t(m, &dst->d, (size_t)w.rows * nb));
    QD_TRY(dev_alloc_t(m, &dst->qs, (size_t)w.rows * nb * 16));
    HIP_TRY(hipMemcpyAsync(dst->d, w.d, (size_t)w.rows * nb * sizeof(uint16_t), hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(dst->qs, w.qs, (size_t)w.rows * nb * 16, hipMemcpyHostToDevice, s));
    HIP_TRY(hipStreamSynchronize(s));
    return QD_OK;
}

static int upload_f32(qd_model* m, float** dst, const float* src, size_t n, hipStream_t s)
{
    QD_TRY(dev_alloc_t(m, dst, n));
    HIP_TRY(hipMemcpyAsync(*dst, src, n * sizeof(float), hipMemcpyHostToDevice, s));
    HIP_TRY(hipStreamSynchronize(s));
    return QD_OK;
}

static void free_model(qd_model* m)
{
    if (!m)
        return;
    if (m->exec)
        (void)hipGraphExecDestroy(m->exec);
    if (m->graph)
        (void)hipGraphDestroy(m->graph);
    if (m->cap_stream)
        (void)hipStreamDestroy(m->cap_stream);
    for (void* p : m->allocs)
        (void)hipFree(p);
    if (m->h_state)
        (void)hipHostFree(m->h_state);
    delete m;
}

static int validate_config(const qd_config* c, const qd_weights* w, int B)
{
    if (!c || !w)
        return fail(QD_EINVAL, "null config or weights");
    if (c->hidden <= 0 || c->layers <= 0 || c->n_heads <= 0 || c->n_kv <= 0 || c->head_dim <= 0 ||
        c->intermediate <= 0 || c->vocab <= 0 || c->max_seq <= 0)
        return fail(QD_EINVAL, "sizes must be positive");
    if (c->n_heads % c->n_kv)
        return fail(QD_EINVAL, "n_heads %% n_kv != 0");
    const int gq = c->n_heads / c->n_kv;
    if (gq != 1 && gq != 2 && gq != 4 && gq != 8)
        return fail(QD_EUNSUPPORTED, "GQA group %d not in {1,2,4,8}", gq);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(QD_EUNSUPPORTED, "head_dim %d not in {64,128}", c->head_dim);
    if (c->hidden % 32 || c->intermediate % 32 || (c->n_heads * c->head_dim) % 32)
        return fail(QD_EUNSUPPORTED, "hidden, intermediate and n_heads*head_dim must be multiples of 32");
    if (c->rot_dim < 0 || c->rot_dim > c->head_dim || (c->rot_dim & 1))
        return fail(QD_EINVAL, "rot_dim must be even and <= head_dim");
    if (c->rot_dim > 0 && !c->inv_freq)
        return fail(QD_EINVAL, "inv_freq is null");
    if (!(c->eps >= 0.f))
        return fail(QD_EINVAL, "eps must be >= 0");
    const size_t kmax = (size_t)GEMV_MAX_LDS / (sizeof(float) * (XPAD + 1)) * 32;
    if ((size_t)c->hidden > kmax || (size_t)c->intermediate > kmax ||
        (size_t)c->n_heads * c->head_dim > kmax)
        return fail(QD_EUNSUPPORTED, "GEMV input length above %zu", kmax);
    // the GEMV addresses a matrix's nibbles with 32-bit offsets
    const uint64_t big = std::max<uint64_t>({(uint64_t)c->vocab * c->hidden,
                                             (uint64_t)2 * c->intermediate * c->hidden,
                                             (uint64_t)(c->n_heads + 2 * c->n_kv) * c->head_dim * c->hidden});
    if (big / 2 >= (uint64_t)1 << 32 || c->vocab >= (1 << 24) || 2 * c->intermediate >= (1 << 24))
        return fail(QD_EUNSUPPORTED, "a matrix above 2^32 bytes of nibbles or 2^24 rows");
    if (c->kv_paged) {
        if (c->kv_block_size != ATT_BS)
            return fail(QD_EUNSUPPORTED, "kv_block_size %d (only %d)", c->kv_block_size, ATT_BS);
        // B sequences: B tables of `need` entries, all distinct
        const int need = (c->max_seq + ATT_BS - 1) / ATT_BS;
        if ((int64_t)c->num_kv_blocks < (int64_t)need * B)
            return fail(QD_EINVAL, "num_kv_blocks %d < %d blocks for max_seq x %d sequences", c->num_kv_blocks,
                        need * B, B);
        if (c->block_table) {
            std::vector<char> seen(c->num_kv_blocks, 0);
            for (int i = 0; i < need * B; ++i) {
                const int p = c->block_table[i];
                if (p < 0 || p >= c->num_kv_blocks)
                    return fail(QD_EINVAL, "block_table[%d] = %d out of range", i, p);
                if (seen[p])
                    return fail(QD_EINVAL, "block_table maps two logical blocks to physical %d", p);
                seen[p] = 1;
            }
        }
    }
    const int H = c->hidden, hd = c->head_dim, nqd = c->n_heads * hd, nkd = c->n_kv * hd;
    QD_TRY(check_q4(w->embed, c->vocab, H, "embed"));
    if (!c->tied)
        QD_TRY(check_q4(w->lm_head, c->vocab, H, "lm_head"));
    if (!w->final_norm || !w->layers)
        return fail(QD_EINVAL, "final_norm or layers is null");
    for (int l = 0; l < c->layers; ++l) {
        const qd_layer_weights& L = w->layers[l];
        char nm[64];
        if (!L.attn_norm || !L.ffn_norm || (c->qk_norm && (!L.q_norm || !L.k_norm)))
            return fail(QD_EINVAL, "layer %d: null norm weight", l);
        snprintf(nm, sizeof nm, "layer %d wq", l);
        QD_TRY(check_q4(L.wq, nqd, H, nm));
        snprintf(nm, sizeof nm, "layer %d wk", l);
        QD_TRY(check_q4(L.wk, nkd, H, nm));
        snprintf(nm, sizeof nm, "layer %d wv", l);
        QD_TRY(check_q4(L.wv, nkd, H, nm));
        snprintf(nm, sizeof nm, "layer %d wo", l);
        QD_TRY(check_q4(L.wo, H, nqd, nm));
        if (c->attn_out_gate) {
            snprintf(nm, sizeof nm, "layer %d attn_gate", l);
            QD_TRY(check_q4(L.attn_gate, nqd, H, nm));
        }
        snprintf(nm, sizeof nm, "layer %d wgate", l);
        QD_TRY(check_q4(L.wgate, c->intermediate, H, nm));
        snprintf(nm, sizeof nm, "layer %d wup", l);
        QD_TRY(check_q4(L.wup, c->intermediate, H, nm));
        snprintf(nm, sizeof nm, "layer %d wdown", l);
        QD_TRY(check_q4(L.wdown, H, c->intermediate, nm));
    }
    if (c->kv_fp8 != 0 && c->kv_fp8 != 1)
        return fail(QD_EINVAL, "kv_fp8 %d (0 or 1)", c->kv_fp8);
    if (c->attn_out_gate != 0 && c->attn_out_gate != 1)
        return fail(QD_EINVAL, "attn_out_gate %d (0 or 1)", c->attn_out_gate);
    if (c->attn_out_gate && c->layer_kernel)
        return fail(QD_EUNSUPPORTED, "attn_out_gate with layer_kernel = 1");
    if (B > 1 && (c->layer_kernel || c->attn_out_gate))
        return fail(QD_EUNSUPPORTED, "a batched model supports neither layer_kernel nor attn_out_gate");
    if (B > 1 && c->hidden > 16384)   // the batched RMSNorm splits at most 2 items per thread
        return fail(QD_EUNSUPPORTED, "a batched model supports hidden <= 16384 (got %d)", c->hidden);
    if (c->kv_fp8) {
        if (!(c->k_scale > 0.f) || !(c->v_scale > 0.f) || !std::isfinite(c->k_scale) ||
            !std::isfinite(c->v_scale))
            return fail(QD_EINVAL, "kv_fp8: k_scale and v_scale must be finite and positive");
        if (c->layer_kernel)
            return fail(QD_EUNSUPPORTED, "kv_fp8 with layer_kernel = 1");
    }
    if (c->layer_kernel) {
        const int nqd = c->n_heads * c->head_dim;
        if (c->head_dim != 128 || c->n_heads != 4 * c->n_kv || c->hidden % 2048 || nqd % 2048 ||
            c->intermediate % 2048)
            return fail(QD_EUNSUPPORTED, "layer_kernel needs head_dim 128, n_heads = 4 n_kv and "
                                         "hidden, intermediate, n_heads*head_dim multiples of 2048");
        const int k_max = std::max(c->hidden, std::max(nqd, c->intermediate));
        if (gemv_lds_bytes(k_max / 32) > (size_t)GEMV_MAX_LDS)
            return fail(QD_EUNSUPPORTED, "layer_kernel: a GEMV's K (%d) is above 14 144", k_max);
    }
    return QD_OK;
}

// Launch the split-KV attention (split + combine).
template <int QMODE, bool KV8 = false>
static hipError_t launch_attention(const AttnParams& p, int waves, int hd, int gq, bool paged, int B,
                                   int nq, hipStream_t s)
{
    // the split kernel's LDS rows and launch bound hold AttnMaxWaves<GQ> waves;
    // the split output (xp) is written by the counted merge of the batched
    // step's query mode only
    if (waves < 1 || waves > (gq <= 4 ? 8 : 4))
        return hipErrorInvalidConfiguration;
    if (p.xp && (QMODE != 2 || !p.counters || !p.xs || !attn_split_out_ok(hd, gq)))
        return hipErrorInvalidValue;
    const dim3 grid(p.nsplit, p.nkv, B), block(waves * WAVE);
    // with max_kv == 0 every kv_len is 0: no split runs and the combine writes zeros
#define QD_ATT(HD_, GQ_)                                                                          \
    if (p.max_kv <= 0) {                                                                          \
    } else if (paged)                                                                             \
        hipLaunchKernelGGL((k_attn_split<HD_, GQ_, true, QMODE, KV8>), grid, block, 0, s, p);     \
    else                                                                                          \
        hipLaunchKernelGGL((k_attn_split<HD_, GQ_, false, QMODE, KV8>), grid, block, 0, s, p);
    if (hd == 128) {
        if (gq == 1) { QD_ATT(128, 1) } else if (gq == 2) { QD_ATT(128, 2) }
        else if (gq == 4) { QD_ATT(128, 4) } else { QD_ATT(128, 8) }
    } else {
        if (gq == 1) { QD_ATT(64, 1) } else if (gq == 2) { QD_ATT(64, 2) }
        else if (gq == 4) { QD_ATT(64, 4) } else { QD_ATT(64, 8) }
    }
#undef QD_ATT
    if (p.counters)
        return hipGetLastError();   // the split kernel merged the partials itself
    // one round of loads: U splits per group of HD threads, U * (ATT_CNT / HD) >= nsplit
    const int per = (p.nsplit + ATT_CNT / hd - 1) / (ATT_CNT / hd);
#define QD_CMB(HD_, U_)                                                                             \
    hipLaunchKernelGGL((k_attn_combine<HD_, U_>), dim3(nq, B), dim3(ATT_CNT), 0, s, p.part, p.nsplit, \
                       p.chunk, p.kv_lens, p.pos, p.max_kv, nq, p.out)
    if (hd == 128) {
        if (per <= 2) QD_CMB(128, 2); else if (per <= 4) QD_CMB(128, 4); else if (per <= 8) QD_CMB(128, 8);
        else QD_CMB(128, 16);
    } else {
        if (per <= 2) QD_CMB(64, 2); else if (per <= 4) QD_CMB(64, 4); else if (per <= 8) QD_CMB(64, 8);
        else QD_CMB(64, 16);
    }
#undef QD_CMB
    return hipGetLastError();
}

// Enqueue one decode step (position and token come from the device state).
static int enqueue_step_fused(qd_model* m, hipStream_t s)
{
    const int H = m->H;
    hipLaunchKernelGGL(k_embed, dim3(m->grid_embed), dim3(256), 0, s, m->embed.d, m->embed.qs, H,
                       m->V, m->st, m->ids, m->max_seq, m->layers[0].attn_norm, m->fX, m->fU,
                       m->fSS, m->rope_cos, m->rope_sin, m->rot / 2, m->rope_cur, m->fbar, FB_WORDS);
    FusedArgs a;
    a.layers = m->flayers;
    a.L = m->L;
    a.H = H;
    a.nq = m->nq;
    a.nkv = m->nkv;
    a.hd = m->hd;
    a.I = m->I;
    a.qkv_rows = m->qkv_rows;
    a.eps = m->eps;
    a.tables = m->paged ? m->table : nullptr;
    a.mbps = (m->max_seq + ATT_BS - 1) / ATT_BS;
    a.pos = &m->st->pos;
    a.max_kv = m->max_seq;
    a.scale = 1.0f / sqrtf((float)m->hd);
    a.chunk = m->fused_chunk;
    a.nsplit = m->fused_nsplit;
    a.qk_norm = m->qk_norm;
    a.rot = m->rot;
    a.rope_cur = m->rope_cur;
    a.bar = m->fbar;
    a.err = &m->st->error;
    a.spin_limit = m->fused_spin;
    for (int l = 0; l < m->L; ++l) {
        if (m->paged)
            hipLaunchKernelGGL((k_layer_fused<128, 4, true>), dim3(m->fused_grid), dim3(FUSED_THREADS),
                               m->fused_lds, s, a, l);
        else
            hipLaunchKernelGGL((k_layer_fused<128, 4, false>), dim3(m->fused_grid), dim3(FUSED_THREADS),
                               m->fused_lds, s, a, l);
    }
    const float* uL = m->fU + (size_t)m->L * H;
    const float* ssL = m->fSS + (size_t)m->L * m->fss_stride;
    QD_GEMV(k_gemv_lmhead, (QD_CFG_HEAD), m->lpr_lm, m->grid_lm, gemv_lds_bytes(m->lm.nb), s,
                   m->lm.d, m->lm.qs, uL, m->lm.rows, m->lm.nb, ssL, m->fused_grid, H, m->eps,
                   m->logits, m->arg_val, m->arg_idx);
    hipLaunchKernelGGL(k_argmax_advance, dim3(1), dim3(256), 0, s, m->arg_val, m->arg_idx,
                       m->grid_lm, m->V, m->st, m->ids, m->pred, m->max_seq);
    HIP_TRY(hipGetLastError());
    return QD_OK;
}

// K slices of a batched step's product of N rows and nb blocks: the row tiles
// of the matrix-core GEMV alone give too few workgroups for short matrices,
// so K is cut into slices (whole 32-block chunks) up to about 768 workgroups
// (measured at the Qwen3-8B shapes: gate|up 2 slices, q|k|v and o 4, down 6)
// Row groups per wave of each split-input product (measured best at the
// Qwen3-8B shape: with 16 vectors one row group except the LM head, whose
// grid is large anyway; with the prefill's 32 two, except o)
constexpr int STEP_RG_QKV = 1, STEP_RG_O = 1, STEP_RG_GU = 1, STEP_RG_DOWN = 1, STEP_RG_LM = 2;
constexpr int PF_RG_QKV = 2, PF_RG_O = 1, PF_RG_GU = 2, PF_RG_DOWN = 2;

// K slices of a split-input product: about 768 workgroups, at most one per
// chunk and SB_MAXSLAB in all (Qwen3-8B shape, one box: prefill 11 988
// positions/s against 11 659 and 11 414 with 384 and 512 (gate|up in 2 and 3
// slices instead of 4); the 16-sequence step 3.08 ms against 3.30 with 512
// (gate|up 1 slice, down 6))
#ifndef QD_STEP_KS_WGS
#define QD_STEP_KS_WGS 768
#endif
#ifndef QD_PF_KS_WGS
#define QD_PF_KS_WGS 768
#endif
static int step_kslices(int N, int nb, int ng, int rg, int target = 768)
{
    const int tiles = (N + gbm_rows(rg) - 1) / gbm_rows(rg);
    const int nch = gbm_nchunks(nb, ng);
    int ks = std::min({nch, SB_MAXSLAB, std::max(1, (target + tiles / 2) / tiles)});
    if (ks > 1) {
        const int kch = (nch + ks - 1) / ks;
        ks = (nch + kch - 1) / kch;
    }
    return ks;
}

// Y = W X on the matrix cores from x split in XP / XS with NG slot groups
// (nv <= 16 NG vectors), rg row groups per wave, in ks K slices (partial
// slabs of nv*N floats, summed by the consumer).  With SQ (the chunk sums of
// x^2 of a split written without its RMSNorm, nsq chunks) the product applies
// 1/rms = 1/sqrt(sum / hn + eps) of each vector itself.
template <int NG>
static hipError_t xp_gemv(const DevQ4& W, const _Float16* XP, const float* XS, float* Y, int nv, int ks, int rg,
                          hipStream_t s, const float* SQ = nullptr, int nsq = 0, float hn = 1.f, float eps = 0.f)
{
    const int N = W.rows, nb = W.nb;
    const int nch = gbm_nchunks(nb, NG);
    const int kch = (nch + ks - 1) / ks;
    if (ks < 1 || (int64_t)(ks - 1) * kch >= nch || (rg != 1 && rg != 2) || nsq < 0 || nsq > (NG == 4 ? 64 : 32))
        return hipErrorInvalidValue;   // every slice holds a chunk; the chunk sums the product reads
    const bool dvec = nb % 8 == 0 && reinterpret_cast<uintptr_t>(W.d) % 16 == 0;
    const dim3 grid((N + gbm_rows(rg) - 1) / gbm_rows(rg), ks), block(GBM_NW * WAVE);
    const size_t lds = gbm_xp_lds_bytes(gbm_xp_sub(NG)), ys = (size_t)nv * N;
    if (rg == 1 && dvec)
        hipLaunchKernelGGL((k_gemv_batch_xp<1, NG, 1>), grid, block, lds, s, W.d, W.qs, XP, XS, Y, N, nb, nv, kch, ys, SQ, nsq,
                           hn, eps);
    else if (rg == 1)
        hipLaunchKernelGGL((k_gemv_batch_xp<1, NG, 0>), grid, block, lds, s, W.d, W.qs, XP, XS, Y, N, nb, nv, kch, ys, SQ, nsq,
                           hn, eps);
    else if (dvec)
        hipLaunchKernelGGL((k_gemv_batch_xp<2, NG, 1>), grid, block, lds, s, W.d, W.qs, XP, XS, Y, N, nb, nv, kch, ys, SQ, nsq,
                           hn, eps);
    else
        hipLaunchKernelGGL((k_gemv_batch_xp<2, NG, 0>), grid, block, lds, s, W.d, W.qs, XP, XS, Y, N, nb, nv, kch, ys, SQ, nsq,
                           hn, eps);
    return hipGetLastError();
}

// the batched step's product over its B sequences; normed: the input is the
// hidden-sized split written by a norm (k_resid_norm_xp_batch, k_embed_xp_batch)
static hipError_t step_gemv(const qd_model* m, const DevQ4& W, const _Float16* XP, const float* XS, float* Y,
                            int ks, int rg, hipStream_t s, bool normed = false)
{
    if (normed)
        return xp_gemv<1>(W, XP, XS, Y, m->B, ks, rg, s, m->sq_h, gbm_nchunks(m->H / 32, 1), (float)m->H, m->eps);
    return xp_gemv<1>(W, XP, XS, Y, m->B, ks, rg, s);
}

// One step of the B sequences of a batched model: every weight read once for
// all of them (gemv_batch_launch), the attention over the B caches with each
// sequence's own position, the norms and SwiGLU as small kernels per sequence
// (step_batch.h), the greedy pick per sequence.
static int enqueue_step_batch(qd_model* m, hipStream_t s)
{
    const int B = m->B, H = m->H, I = m->I;
    const int nqd = m->nq * m->hd;
    const dim3 ngrid(gbm_nchunks(H / 32, 1), B), nblock(gbm_chunk_threads(1));
    hipLaunchKernelGGL(k_embed_xp_batch, ngrid, nblock, 0, s, m->embed.d, m->embed.qs, H, m->V, m->st, m->ids,
                       m->max_seq, m->layers[0].attn_norm, m->bx, 1, m->xp_h, m->xs_h, m->sq_h, m->rope_cos,
                       m->rope_sin, m->rot / 2, m->rope_cur, m->rstride);
    for (int l = 0; l < m->L; ++l) {
        DevLayer& Ly = m->layers[l];
        HIP_TRY(step_gemv(m, Ly.qkv, m->xp_h, m->xs_h, m->bqkv, m->ks_qkv, STEP_RG_QKV, s, true));
        AttnParams p;
        memset(&p, 0, sizeof p);
        p.q = m->bqkv;
        p.q_stride = m->qkv_rows;
        p.q_slabs = m->ks_qkv;
        p.q_slab_stride = (size_t)B * m->qkv_rows;
        p.k = Ly.kc;
        p.v = Ly.vc;
        p.tables = m->paged ? m->table : nullptr;
        p.mbps = (m->max_seq + ATT_BS - 1) / ATT_BS;
        p.kv_lens = nullptr;
        p.pos = &m->st->pos;
        p.pos_stride = sizeof(StepState) / sizeof(int32_t);
        p.max_kv = m->max_seq;
        p.nq = m->nq;
        p.nkv = m->nkv;
        p.scale = 1.0f / sqrtf((float)m->hd);
        p.chunk = m->attn_chunk;
        p.nsplit = m->attn_nsplit;
        p.part = m->attn_part;
        p.out = m->battn;
        p.qk_norm = m->qk_norm;
        p.q_norm = m->qk_norm ? Ly.q_norm : m->ones_hd;   // read either way
        p.k_norm = m->qk_norm ? Ly.k_norm : m->ones_hd;
        p.eps = m->eps;
        p.rot = m->rot;
        p.rope_cur = m->rope_cur;
        p.rope_stride = m->rstride;
        p.counters = m->attn_cnt;
        p.kc = Ly.kc;
        p.vc = Ly.vc;
        p.k_scale = m->k_scale;
        p.v_scale = m->v_scale;
        // from 8 sequences the attention's merge writes the o product's split
        // input itself (per 1024-element chunk; where its LDS allows): one
        // launch less per layer.  With fewer sequences each chunk's merge
        // waits for more split workgroups than the separate split costs.
        const bool split_out = B >= ATT_SPLIT_OUT_MIN_B && attn_split_out_ok(m->hd, m->nq / m->nkv);
        p.xp = split_out ? m->xp_o : nullptr;
        p.xs = split_out ? m->xs_o : nullptr;
        if (m->kv_fp8)
            HIP_TRY((launch_attention<2, true>(p, m->attn_waves, m->hd, m->nq / m->nkv, m->paged, B, m->nq, s)));
        else
            HIP_TRY((launch_attention<2>(p, m->attn_waves, m->hd, m->nq / m->nkv, m->paged, B, m->nq, s)));
        const size_t slab_h = (size_t)B * H;
        if (!split_out)
            hipLaunchKernelGGL(k_xsplit_batch, dim3(gbm_nchunks(nqd / 32, 1), B), dim3(128), 0, s, m->battn,
                               nqd / 32, 1, m->xp_o, m->xs_o, nullptr, 0, 1, (size_t)0);
        HIP_TRY(step_gemv(m, Ly.o, m->xp_o, m->xs_o, m->bo, m->ks_o, STEP_RG_O, s));
        hipLaunchKernelGGL(k_resid_norm_xp_batch, ngrid, nblock, 0, s, m->bx, m->bo, m->ks_o, slab_h, H,
                           Ly.ffn_norm, 1, m->xp_h, m->xs_h, m->sq_h);
        HIP_TRY(step_gemv(m, Ly.gu, m->xp_h, m->xs_h, m->bgu, m->ks_gu, STEP_RG_GU, s, true));
        hipLaunchKernelGGL(k_swiglu_xp_batch, dim3(gbm_nchunks(I / 32, 1), B), dim3(128), 0, s, m->bgu,
                           m->ks_gu, (size_t)B * 2 * I, I, 1, m->xp_i, m->xs_i);
        HIP_TRY(step_gemv(m, Ly.down, m->xp_i, m->xs_i, m->bo, m->ks_down, STEP_RG_DOWN, s));
        const float* wn = (l + 1 < m->L) ? m->layers[l + 1].attn_norm : m->final_norm;
        hipLaunchKernelGGL(k_resid_norm_xp_batch, ngrid, nblock, 0, s, m->bx, m->bo, m->ks_down, slab_h, H, wn,
                           1, m->xp_h, m->xs_h, m->sq_h);
    }
    HIP_TRY(step_gemv(m, m->lm, m->xp_h, m->xs_h, m->blog, 1, STEP_RG_LM, s, true));
    hipLaunchKernelGGL(k_argmax_batch, dim3(m->bG, B), dim3(256), 0, s, m->blog, m->V, m->bchunk, m->bcval,
                       m->bcidx);
    hipLaunchKernelGGL(k_argmax_advance_batch, dim3(B), dim3(256), 0, s, m->bcval, m->bcidx, m->bG, m->V, m->st,
                       m->ids, m->pred, m->max_seq);
    HIP_TRY(hipGetLastError());
    return QD_OK;
}

static int enqueue_step(qd_model* m, hipStream_t s)
{
    if (m->B > 1)
        return enqueue_step_batch(m, s);
    if (m->fused)
        return enqueue_step_fused(m, s);
    const int H = m->H;
    hipLaunchKernelGGL(k_embed, dim3(m->grid_embed), dim3(256), 0, s, m->embed.d, m->embed.qs, H,
                       m->V, m->st, m->ids, m->max_seq, m->layers[0].attn_norm, m->x, m->u,
                       m->ss_part, m->rope_cos, m->rope_sin, m->rot / 2, m->rope_cur,
                       (unsigned*)nullptr, 0);
    int n_part = m->grid_embed;
    for (int l = 0; l < m->L; ++l) {
        DevLayer& Ly = m->layers[l];
        // q | k | v (raw, before the per-head norm and rotary)
        if (m->small_qkv) {
            QD_GEMV(k_gemv_scaled, (QD_CFG_QKV_S), m->lpr_qkv, m->grid_qkv, gemv_lds_bytes(Ly.qkv.nb), s,
                    Ly.qkv.d, Ly.qkv.qs, m->u, Ly.qkv.rows, Ly.qkv.nb, m->ss_part, n_part, H, m->eps,
                    m->qkv_raw);
        } else {
            QD_GEMV(k_gemv_scaled, (QD_CFG_QKV), m->lpr_qkv, m->grid_qkv, gemv_lds_bytes(Ly.qkv.nb), s,
                    Ly.qkv.d, Ly.qkv.qs, m->u, Ly.qkv.rows, Ly.qkv.nb, m->ss_part, n_part, H, m->eps,
                    m->qkv_raw);
        }
        // per-head norm + rotary, K/V write, split-KV attention, combine
        {
            AttnParams p;
            memset(&p, 0, sizeof p);
            p.q = m->qkv_raw;
            p.k = Ly.kc;
            p.v = Ly.vc;
            p.tables = m->paged ? m->table : nullptr;
            p.mbps = (m->max_seq + ATT_BS - 1) / ATT_BS;
            p.kv_lens = nullptr;
            p.pos = &m->st->pos;
            p.max_kv = m->max_seq;
            p.nq = m->nq;
            p.nkv = m->nkv;
            p.scale = 1.0f / sqrtf((float)m->hd);
            p.chunk = m->attn_chunk;
            p.nsplit = m->attn_nsplit;
            p.part = m->attn_part;
            p.out = m->attn;
            p.qk_norm = m->qk_norm;
            p.q_norm = m->qk_norm ? Ly.q_norm : m->ones_hd;   // read either way
            p.k_norm = m->qk_norm ? Ly.k_norm : m->ones_hd;
            p.eps = m->eps;
            p.rot = m->rot;
            p.rope_cur = m->rope_cur;
            p.counters = m->attn_cnt;
            p.kc = Ly.kc;
            p.vc = Ly.vc;
            p.k_scale = m->k_scale;
            p.v_scale = m->v_scale;
            p.gate = m->attn_gate ? m->qkv_raw + (size_t)(m->nq + 2 * m->nkv) * m->hd : nullptr;
            if (m->kv_fp8)
                HIP_TRY((launch_attention<1, true>(p, m->attn_waves, m->hd, m->nq / m->nkv, m->paged, 1, m->nq, s)));
            else
                HIP_TRY((launch_attention<1>(p, m->attn_waves, m->hd, m->nq / m->nkv, m->paged, 1, m->nq, s)));
        }
        // o-proj + residual, u = x * ffn_norm
        if (m->small_o) {
            QD_GEMV(k_gemv_residual, (QD_CFG_O_S), m->lpr_o, m->grid_o, gemv_lds_bytes(Ly.o.nb), s,
                    Ly.o.d, Ly.o.qs, m->attn, Ly.o.rows, Ly.o.nb, m->x, m->u, Ly.ffn_norm, m->ss_part);
        } else {
            QD_GEMV(k_gemv_residual, (QD_CFG_O), m->lpr_o, m->grid_o, gemv_lds_bytes(Ly.o.nb), s,
                    Ly.o.d, Ly.o.qs, m->attn, Ly.o.rows, Ly.o.nb, m->x, m->u, Ly.ffn_norm, m->ss_part);
        }
        n_part = m->grid_o;
        // gate|up + SwiGLU
        QD_GEMV(k_gemv_swiglu, (QD_CFG_GU), m->lpr_gu, m->grid_gu, gemv_lds_bytes(Ly.gu.nb), s,
                       Ly.gu.d, Ly.gu.qs, m->u, Ly.gu.rows, Ly.gu.nb, m->ss_part, n_part, H, m->eps,
                       m->act);
        // down + residual, u = x * (next attn_norm | final_norm)
        const float* wn = (l + 1 < m->L) ? m->layers[l + 1].attn_norm : m->final_norm;
        if (m->small_down) {
            QD_GEMV(k_gemv_residual, (QD_CFG_DOWN_S), m->lpr_down, m->grid_down, gemv_lds_bytes(Ly.down.nb), s,
                    Ly.down.d, Ly.down.qs, m->act, Ly.down.rows, Ly.down.nb, m->x, m->u, wn, m->ss_part);
        } else {
            QD_GEMV(k_gemv_residual, (QD_CFG_DOWN), m->lpr_down, m->grid_down, gemv_lds_bytes(Ly.down.nb), s,
                    Ly.down.d, Ly.down.qs, m->act, Ly.down.rows, Ly.down.nb, m->x, m->u, wn, m->ss_part);
        }
        n_part = m->grid_down;
    }
    QD_GEMV(k_gemv_lmhead, (QD_CFG_HEAD), m->lpr_lm, m->grid_lm, gemv_lds_bytes(m->lm.nb), s,
                   m->lm.d, m->lm.qs, m->u, m->lm.rows, m->lm.nb, m->ss_part, n_part, H, m->eps,
                   m->logits, m->arg_val, m->arg_idx);
    hipLaunchKernelGGL(k_argmax_advance, dim3(1), dim3(256), 0, s, m->arg_val, m->arg_idx,
                       m->grid_lm, m->V, m->st, m->ids, m->pred, m->max_seq);
    HIP_TRY(hipGetLastError());
    return QD_OK;
}

static int run_steps(qd_model* m, int n, hipStream_t s)
{
    for (int i = 0; i < n; ++i) {
        if (m->use_graph) {
            HIP_TRY(hipGraphLaunch(m->exec, s));
        } else {
            QD_TRY(enqueue_step(m, s));
        }
    }
    return QD_OK;
}

// tiny kernel: set position / forced prefix / a stored token (so that setting
// state is an ordinary stream operation, never a host-synchronous copy)
__global__ void k_set_state(StepState* st, int32_t* ids, int pos, int n_forced, int tok_pos,
                            int tok)
{
    if (threadIdx.x == 0) {
        st->pos = pos;
        if (n_forced >= 0)
            st->n_forced = n_forced;
        if (tok_pos >= 0)
            ids[tok_pos] = tok;
    }
}

// The persistent layer kernel (layer_kernel = 1) needs a model that fits its
// instantiation: head_dim 128, 4 query heads per kv head, every GEMV's K a
// multiple of 2048 and at most 14 144, one workgroup per CU resident, and the
// attention splits (8 waves x 16 keys each, over max_seq) at most one per
// workgroup.
static int setup_fused(qd_model* m, hipStream_t s, int want)
{
    m->fused = 0;
    if (!want)
        return QD_OK;
    const int H = m->H, nqd = m->nq * m->hd;   // shapes checked by validate_config
    const int nb_max = std::max(H, std::max(nqd, m->I)) / 32;
    int dev = 0, cus = 0;
    HIP_TRY(hipGetDevice(&dev));
    HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    const size_t lds = fused_lds_bytes<128, 4>(nb_max);
    int per_cu = 0;
    const void* kfn = m->paged ? (const void*)k_layer_fused<128, 4, true> : (const void*)k_layer_fused<128, 4, false>;
    HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, FUSED_THREADS, lds));
    if (per_cu < 1 || cus < 1)
        return fail(QD_EUNSUPPORTED, "layer_kernel: a workgroup does not fit a CU");
    const int G = cus;
    const AttnGeom ag = attn_geom(1, m->nkv, m->max_seq, G, FUSED_WAVES, FUSED_WAVES);
    if (ag.nsplit * m->nkv > G)
        return fail(QD_EUNSUPPORTED, "layer_kernel: %d attention splits for %d workgroups",
                    ag.nsplit * m->nkv, G);
    m->fused_grid = G;
    m->fused_lds = lds;
    // testing only: a smaller bound on the barrier polls (forces the timeout path)
    if (const char* e = getenv("QD_LAYER_KERNEL_SPIN_LIMIT"))
        m->fused_spin = std::max(0, atoi(e));
    m->fused_nsplit = ag.nsplit;
    m->fused_chunk = ag.chunk;
    m->fss_stride = std::max(G, m->grid_embed);
    const int L = m->L;
    int rc;
    if ((rc = dev_alloc_t(m, &m->fbar, FB_WORDS)) || (rc = dev_alloc_t(m, &m->fX, (size_t)(L + 1) * H)) ||
        (rc = dev_alloc_t(m, &m->fU, (size_t)(L + 1) * H)) ||
        (rc = dev_alloc_t(m, &m->fSS, (size_t)(L + 1) * m->fss_stride)) ||
        (rc = dev_alloc_t(m, &m->flayers, (size_t)L)))
        return rc;
    std::vector<FusedLayer> t(L);
    for (int l = 0; l < L; ++l) {
        DevLayer& D = m->layers[l];
        FusedLayer& F = t[l];
        F.qkv_d = D.qkv.d; F.qkv_q = D.qkv.qs;
        F.o_d = D.o.d; F.o_q = D.o.qs;
        F.gu_d = D.gu.d; F.gu_q = D.gu.qs;
        F.down_d = D.down.d; F.down_q = D.down.qs;
        F.ffn_norm = D.ffn_norm;
        F.w_next = (l + 1 < L) ? m->layers[l + 1].attn_norm : m->final_norm;
        F.q_norm = m->qk_norm ? D.q_norm : m->ones_hd;
        F.k_norm = m->qk_norm ? D.k_norm : m->ones_hd;
        F.kc = D.kc;
        F.vc = D.vc;
        F.x_in = m->fX + (size_t)l * H;
        F.u_in = m->fU + (size_t)l * H;
        F.ss_in = m->fSS + (size_t)l * m->fss_stride;
        F.n_in = l == 0 ? m->grid_embed : G;
        F.x_out = m->fX + (size_t)(l + 1) * H;
        F.u_out = m->fU + (size_t)(l + 1) * H;
        F.ss_out = m->fSS + (size_t)(l + 1) * m->fss_stride;
        if ((rc = dev_alloc_t(m, &F.qkv, m->qkv_rows)) ||
            (rc = dev_alloc_t(m, &F.part, (size_t)m->nq * ag.nsplit * (m->hd + 2))) ||
            (rc = dev_alloc_t(m, &F.att, nqd)) || (rc = dev_alloc_t(m, &F.xm, H)) ||
            (rc = dev_alloc_t(m, &F.um, H)) || (rc = dev_alloc_t(m, &F.ssa, G)) ||
            (rc = dev_alloc_t(m, &F.act, m->I)) || (rc = dev_alloc_t(m, &F.cnt, m->nkv)))
            return rc;
        if (hipMemsetAsync(F.cnt, 0, sizeof(unsigned) * m->nkv, s) != hipSuccess)
            return fail(QD_EHIP, "fused counter clear failed");
    }
    if (hipMemcpyAsync(m->flayers, t.data(), sizeof(FusedLayer) * L, hipMemcpyHostToDevice, s) != hipSuccess ||
        hipMemsetAsync(m->fbar, 0, sizeof(unsigned) * FB_WORDS, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return fail(QD_EHIP, "fused layer table upload failed");
    m->fused = 1;
    return QD_OK;
}

static int create_model(const qd_config* cfg, const qd_weights* w, int B, qd_stream stream, qd_model** out)
{
    if (!out)
        return fail(QD_EINVAL, "out is null");
    *out = nullptr;
    QD_TRY(validate_config(cfg, w, B));
    hipStream_t s = (hipStream_t)stream;
    qd_model* m = new qd_model();
    m->B = B;
    m->hwb.assign(B, -1);
    auto bail = [&](int rc) {
        free_model(m);
        return rc;
    };
    const qd_config& c = *cfg;
    m->H = c.hidden;
    m->L = c.layers;
    m->nq = c.n_heads;
    m->nkv = c.n_kv;
    m->hd = c.head_dim;
    m->I = c.intermediate;
    m->V = c.vocab;
    m->rot = c.rot_dim;
    m->eps = c.eps;
    m->max_seq = c.max_seq;
    m->qk_norm = c.qk_norm ? 1 : 0;
    m->paged = c.kv_paged ? 1 : 0;
    m->kv_fp8 = c.kv_fp8;
    m->k_scale = c.kv_fp8 ? c.k_scale : 1.f;
    m->v_scale = c.kv_fp8 ? c.v_scale : 1.f;
    m->nblocks = c.kv_paged ? c.num_kv_blocks : 0;
    m->attn_gate = c.attn_out_gate;
    // q | k | v (| gate): the gate rows project the same normed input
    m->qkv_rows = (m->nq + 2 * m->nkv + (m->attn_gate ? m->nq : 0)) * m->hd;
    m->use_graph = c.use_graph ? 1 : 0;
    const int H = m->H, hd = m->hd, nqd = m->nq * hd, nkd = m->nkv * hd;

    int rc;
    // weights
    m->layers.resize(m->L);
    for (int l = 0; l < m->L; ++l) {
        const qd_layer_weights& S = w->layers[l];
        DevLayer& D = m->layers[l];
        std::vector<RowSrc> rows;
        rows.reserve(m->qkv_rows);
        for (int r = 0; r < nqd; ++r) rows.push_back({&S.wq, r});
        for (int r = 0; r < nkd; ++r) rows.push_back({&S.wk, r});
        for (int r = 0; r < nkd; ++r) rows.push_back({&S.wv, r});
        if (m->attn_gate)
            for (int r = 0; r < nqd; ++r) rows.push_back({&S.attn_gate, r});
        if ((rc = upload_rows(m, &D.qkv, rows, H, s))) return bail(rc);
        rows.clear();
        for (int r = 0; r < m->I; ++r) {
            rows.push_back({&S.wgate, r});
            rows.push_back({&S.wup, r});
        }
        if ((rc = upload_rows(m, &D.gu, rows, H, s))) return bail(rc);
        if ((rc = upload_whole(m, &D.o, S.wo, s))) return bail(rc);
        if ((rc = upload_whole(m, &D.down, S.wdown, s))) return bail(rc);
        if ((rc = upload_f32(m, &D.attn_norm, S.attn_norm, H, s))) return bail(rc);
        if ((rc = upload_f32(m, &D.ffn_norm, S.ffn_norm, H, s))) return bail(rc);
        if (m->qk_norm) {
            if ((rc = upload_f32(m, &D.q_norm, S.q_norm, hd, s))) return bail(rc);
            if ((rc = upload_f32(m, &D.k_norm, S.k_norm, hd, s))) return bail(rc);
        }
    }
    if ((rc = upload_whole(m, &m->embed, w->embed, s))) return bail(rc);
    if (c.tied)
        m->lm = m->embed;
    else if ((rc = upload_whole(m, &m->lm, w->lm_head, s)))
        return bail(rc);
    if ((rc = upload_f32(m, &m->final_norm, w->final_norm, H, s))) return bail(rc);

    // rotary tables: cos/sin of pos * inv_freq[i], evaluated in f64 on the host
    {
        const int half = m->rot / 2;
        const size_t n = (size_t)m->max_seq * (half > 0 ? half : 1);
        std::vector<float> hc(n, 1.f), hs(n, 0.f);
        for (int p = 0; p < m->max_seq; ++p)
            for (int i = 0; i < half; ++i) {
                const double th = (double)p * (double)c.inv_freq[i];
                hc[(size_t)p * half + i] = (float)std::cos(th);
                hs[(size_t)p * half + i] = (float)std::sin(th);
            }
        if ((rc = upload_f32(m, &m->rope_cos, hc.data(), n, s))) return bail(rc);
        if ((rc = upload_f32(m, &m->rope_sin, hs.data(), n, s))) return bail(rc);
        m->rstride = 2 * (half > 0 ? half : 1);
        if ((rc = dev_alloc_t(m, &m->rope_cur, (size_t)B * m->rstride))) return bail(rc);
        const std::vector<float> ones((size_t)m->hd, 1.f);
        if ((rc = upload_f32(m, &m->ones_hd, ones.data(), (size_t)m->hd, s))) return bail(rc);
        if ((rc = dev_alloc_t(m, &m->attn_cnt, (size_t)B * m->nkv))) return bail(rc);
        if (hipMemsetAsync(m->attn_cnt, 0, sizeof(unsigned) * B * m->nkv, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return bail(fail(QD_EHIP, "attention counter clear failed"));
    }

    // KV cache
    for (int l = 0; l < m->L; ++l) {
        DevLayer& D = m->layers[l];
        const size_t n = m->paged ? (size_t)m->nblocks * m->nkv * ATT_BS * hd
                                  : (size_t)B * m->nkv * m->max_seq * hd;
        // n elements of 2 bytes (f16) or 1 byte (fp8; hd is even, so n / 2 halves)
        const size_t nh = m->kv_fp8 ? n / 2 : n;
        if ((rc = dev_alloc_t(m, &D.kc, nh))) return bail(rc);
        if ((rc = dev_alloc_t(m, &D.vc, nh))) return bail(rc);
        if (hipMemsetAsync(D.kc, 0, nh * 2, s) != hipSuccess || hipMemsetAsync(D.vc, 0, nh * 2, s) != hipSuccess)
            return bail(fail(QD_EHIP, "KV cache clear failed"));
    }
    if (m->paged) {
        // one table per sequence: [B][need]
        const int need = (m->max_seq + ATT_BS - 1) / ATT_BS;
        std::vector<int32_t> t((size_t)B * need);
        for (int i = 0; i < B * need; ++i)
            t[i] = c.block_table ? c.block_table[i] : i;
        if ((rc = dev_alloc_t(m, &m->table, (size_t)B * need))) return bail(rc);
        if (hipMemcpyAsync(m->table, t.data(), t.size() * sizeof(int32_t), hipMemcpyHostToDevice, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return bail(fail(QD_EHIP, "block table upload failed"));
    }

    // launch geometry
    {
        const int nbH = H / 32;
        m->grid_embed = (H + 255) / 256;
        m->lpr_qkv = pick_lpr(nbH);
        m->grid_qkv = gemv_grid(CFG_QKV, m->lpr_qkv, m->qkv_rows);
        if ((m->small_qkv = m->grid_qkv < QD_GEMV_SMALL_GRID))
            m->grid_qkv = gemv_grid(CFG_QKV_S, m->lpr_qkv, m->qkv_rows);
        m->lpr_o = pick_lpr(nqd / 32);
        m->grid_o = gemv_grid(CFG_O, m->lpr_o, H);   // one tile per workgroup (residual epilogue)
        if ((m->small_o = m->grid_o < QD_GEMV_SMALL_GRID))
            m->grid_o = gemv_grid(CFG_O_S, m->lpr_o, H);
        m->lpr_gu = pick_lpr(nbH, CFG_GU.lpr_max);
        m->grid_gu = gemv_grid(CFG_GU, m->lpr_gu, 2 * m->I);
        m->lpr_down = pick_lpr(m->I / 32);
        m->grid_down = gemv_grid(CFG_DOWN, m->lpr_down, H);   // one tile per workgroup
        if ((m->small_down = m->grid_down < QD_GEMV_SMALL_GRID))
            m->grid_down = gemv_grid(CFG_DOWN_S, m->lpr_down, H);
        m->lpr_lm = pick_lpr(nbH);
        m->grid_lm = gemv_grid(CFG_HEAD, m->lpr_lm, m->V);
        // attention: splits over max_seq (the grid does not depend on the position),
        // about one workgroup per CU (B sequences: as many over all of them)
        const int gq = m->nq / m->nkv;
        const AttnGeom ag = attn_geom(B, m->nkv, m->max_seq, B == 1 ? ATT_MODEL_WGS : QD_ATT_BATCH_WGS,
                                      gq <= 4 ? QD_ATT_MODEL_WAVES : 4, 0);
        m->attn_waves = ag.waves;
        m->attn_chunk = ag.chunk;
        m->attn_nsplit = ag.nsplit;
    }

    // step buffers
    const int maxp = 4096;
    if ((rc = dev_alloc_t(m, &m->x, H)) || (rc = dev_alloc_t(m, &m->u, H)) ||
        (rc = dev_alloc_t(m, &m->ss_part, maxp)) || (rc = dev_alloc_t(m, &m->qkv_raw, m->qkv_rows)) ||
        (rc = dev_alloc_t(m, &m->attn, nqd)) || (rc = dev_alloc_t(m, &m->act, m->I)) ||
        (rc = dev_alloc_t(m, &m->logits, m->V)) || (rc = dev_alloc_t(m, &m->arg_val, maxp)) ||
        (rc = dev_alloc_t(m, &m->arg_idx, maxp)) ||
        (rc = dev_alloc_t(m, &m->attn_part, (size_t)B * m->nq * m->attn_nsplit * (hd + 2))) ||
        (rc = dev_alloc_t(m, &m->st, B)) || (rc = dev_alloc_t(m, &m->ids, (size_t)B * m->max_seq)) ||
        (rc = dev_alloc_t(m, &m->pred, (size_t)B * m->max_seq)))
        return bail(rc);
    if (B > 1) {
        m->bchunk = 4096;
        m->bG = (m->V + m->bchunk - 1) / m->bchunk;
        m->ks_qkv = step_kslices(m->qkv_rows, H / 32, 1, STEP_RG_QKV, QD_STEP_KS_WGS);
        m->ks_o = step_kslices(H, nqd / 32, 1, STEP_RG_O, QD_STEP_KS_WGS);
        m->ks_gu = step_kslices(2 * m->I, H / 32, 1, STEP_RG_GU, QD_STEP_KS_WGS);
        m->ks_down = step_kslices(H, m->I / 32, 1, STEP_RG_DOWN, QD_STEP_KS_WGS);
        const size_t Bz = B;
        if ((rc = dev_alloc_t(m, &m->bx, Bz * H)) || (rc = dev_alloc_t(m, &m->bh, Bz * H)) ||
            (rc = dev_alloc_t(m, &m->bqkv, Bz * m->ks_qkv * m->qkv_rows)) ||
            (rc = dev_alloc_t(m, &m->battn, Bz * nqd)) ||
            (rc = dev_alloc_t(m, &m->bo, Bz * std::max(m->ks_o, m->ks_down) * H)) ||
            (rc = dev_alloc_t(m, &m->bgu, Bz * m->ks_gu * 2 * m->I)) ||
            (rc = dev_alloc_t(m, &m->bact, Bz * m->I)) || (rc = dev_alloc_t(m, &m->blog, Bz * m->V)) ||
            (rc = dev_alloc_t(m, &m->bcval, Bz * m->bG)) || (rc = dev_alloc_t(m, &m->bcidx, Bz * m->bG)))
            return bail(rc);
        const size_t ch_h = gbm_nchunks(H / 32, 1), ch_o = gbm_nchunks(nqd / 32, 1),
                     ch_i = gbm_nchunks(m->I / 32, 1);
        if ((rc = dev_alloc_t(m, &m->xp_h, ch_h * GBM_XP_CHUNK)) ||
            (rc = dev_alloc_t(m, &m->xp_o, ch_o * GBM_XP_CHUNK)) ||
            (rc = dev_alloc_t(m, &m->xp_i, ch_i * GBM_XP_CHUNK)) || (rc = dev_alloc_t(m, &m->xs_h, ch_h * 16)) ||
            (rc = dev_alloc_t(m, &m->xs_o, ch_o * 16)) || (rc = dev_alloc_t(m, &m->xs_i, ch_i * 16)) ||
            (rc = dev_alloc_t(m, &m->sq_h, ch_h * 16)))
            return bail(rc);
        // slots past the batch and blocks past the end are read as zeros forever
        if (hipMemsetAsync(m->xp_h, 0, ch_h * GBM_XP_CHUNK * sizeof(_Float16), s) != hipSuccess ||
            hipMemsetAsync(m->xp_o, 0, ch_o * GBM_XP_CHUNK * sizeof(_Float16), s) != hipSuccess ||
            hipMemsetAsync(m->xp_i, 0, ch_i * GBM_XP_CHUNK * sizeof(_Float16), s) != hipSuccess ||
            hipMemsetAsync(m->xs_h, 0, ch_h * 16 * sizeof(float), s) != hipSuccess ||
            hipMemsetAsync(m->xs_o, 0, ch_o * 16 * sizeof(float), s) != hipSuccess ||
            hipMemsetAsync(m->xs_i, 0, ch_i * 16 * sizeof(float), s) != hipSuccess ||
            hipMemsetAsync(m->sq_h, 0, ch_h * 16 * sizeof(float), s) != hipSuccess)
            return bail(fail(QD_EHIP, "batch buffer clear failed"));
    }
    if (hipMemsetAsync(m->st, 0, sizeof(StepState) * B, s) != hipSuccess ||
        hipMemsetAsync(m->ids, 0, sizeof(int32_t) * B * m->max_seq, s) != hipSuccess ||
        hipMemsetAsync(m->pred, 0, sizeof(int32_t) * B * m->max_seq, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return bail(fail(QD_EHIP, "step buffer clear failed"));
    if ((rc = setup_fused(m, s, c.layer_kernel)))
        return bail(rc);

    // graph of one step
    if (m->use_graph) {
        if (hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking) != hipSuccess)
            return bail(fail(QD_EHIP, "stream create failed"));
        if (hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal) != hipSuccess)
            return bail(fail(QD_EHIP, "begin capture failed"));
        int src = enqueue_step(m, m->cap_stream);
        hipError_t ee = hipStreamEndCapture(m->cap_stream, &m->graph);
        if (src != QD_OK)
            return bail(src);
        if (ee != hipSuccess)
            return bail(fail(QD_EHIP, "end capture: %s", hipGetErrorString(ee)));
        ee = hipGraphInstantiate(&m->exec, m->graph, nullptr, nullptr, 0);
        if (ee != hipSuccess)
            return bail(fail(QD_EHIP, "graph instantiate: %s", hipGetErrorString(ee)));
    }
    *out = m;
    return QD_OK;
}

extern "C" int qd_create(const qd_config* cfg, const qd_weights* w, qd_stream stream, qd_model** out)
{
    return create_model(cfg, w, 1, stream, out);
}

extern "C" int qd_create_batch(const qd_config* cfg, const qd_weights* w, int32_t batch, qd_stream stream,
                               qd_model** out)
{
    if (out)
        *out = nullptr;
    if (batch < 2 || batch > SB_MAXB)
        return fail(QD_EINVAL, "batch %d not in [2, %d]", batch, SB_MAXB);
    return create_model(cfg, w, batch, stream, out);
}

extern "C" int qd_destroy(qd_model* m)
{
    if (!m)
        return fail(QD_EINVAL, "null model");
    (void)hipDeviceSynchronize();
    free_model(m);
    return QD_OK;
}

// entry points of one sequence refuse a batched model, and the reverse
#define QD_ONE_SEQUENCE(m)                                                                         \
    if ((m)->B != 1)                                                                               \
        return fail(QD_EINVAL, "a model of %d sequences (qd_create_batch): use the batch entry points", (m)->B)
#define QD_BATCHED(m)                                                                              \
    if ((m)->B == 1)                                                                               \
        return fail(QD_EINVAL, "a model of one sequence (qd_create): use the one-sequence entry points")

extern "C" int qd_decode_step(qd_model* m, int32_t token, int32_t pos, float* d_logits,
                              int32_t* d_next, qd_stream stream)
{
    if (!m)
        return fail(QD_EINVAL, "null model");
    QD_ONE_SEQUENCE(m);
    if (token < 0 || token >= m->V)
        return fail(QD_ERANGE, "token %d not in [0, %d)", token, m->V);
    if (pos < 0 || pos >= m->max_seq)
        return fail(QD_ERANGE, "pos %d not in [0, %d)", pos, m->max_seq);
    if (pos > m->hw + 1)
        return fail(QD_ERANGE, "pos %d past the written prefix: positions 0..%d hold K/V, so the "
                               "next step is at most at %d", pos, m->hw, m->hw + 1);
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(k_set_state, dim3(1), dim3(64), 0, s, m->st, m->ids, pos, pos + 1, pos, token);
    HIP_TRY(hipGetLastError());
    QD_TRY(run_steps(m, 1, s));
    m->hw = pos;
    if (d_logits)
        HIP_TRY(hipMemcpyAsync(d_logits, m->logits, sizeof(float) * m->V, hipMemcpyDeviceToDevice, s));
    if (d_next)
        HIP_TRY(hipMemcpyAsync(d_next, m->pred + pos, sizeof(int32_t), hipMemcpyDeviceToDevice, s));
    return QD_OK;
}

extern "C" int qd_set_prompt(qd_model* m, const int32_t* tokens, int32_t n, qd_stream stream)
{
    if (!m)
        return fail(QD_EINVAL, "null model");
    QD_ONE_SEQUENCE(m);
    if (n < 0 || n > m->max_seq)
        return fail(QD_ERANGE, "prompt length %d not in [0, %d]", n, m->max_seq);
    if (n > 0 && !tokens)
        return fail(QD_EINVAL, "null tokens");
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= m->V)
            return fail(QD_ERANGE, "token[%d] = %d not in [0, %d)", i, tokens[i], m->V);
    hipStream_t s = (hipStream_t)stream;
    if (n > 0) {
        HIP_TRY(hipMemcpyAsync(m->ids, tokens, sizeof(int32_t) * n, hipMemcpyHostToDevice, s));
        HIP_TRY(hipStreamSynchronize(s));  // the host array may go away on return
    }
    hipLaunchKernelGGL(k_set_state, dim3(1), dim3(64), 0, s, m->st, m->ids, 0, n, -1, 0);
    HIP_TRY(hipGetLastError());
    return QD_OK;
}

extern "C" int qd_generate(qd_model* m, int32_t pos0, int32_t n_steps, int32_t* d_tokens,
                           float* d_logits_last, qd_stream stream)
{
    if (!m)
        return fail(QD_EINVAL, "null model");
    QD_ONE_SEQUENCE(m);
    if (pos0 < 0 || n_steps < 0 || (int64_t)pos0 + n_steps > m->max_seq)
        return fail(QD_ERANGE, "positions [%d, %d) not within max_seq %d", pos0, pos0 + n_steps,
                    m->max_seq);
    if (n_steps > 0 && pos0 > m->hw + 1)
        return fail(QD_ERANGE, "pos0 %d past the written prefix: positions 0..%d hold K/V, so the "
                               "next step is at most at %d", pos0, m->hw, m->hw + 1);
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(k_set_state, dim3(1), dim3(64), 0, s, m->st, m->ids, pos0, -1, -1, 0);
    HIP_TRY(hipGetLastError());
    QD_TRY(run_steps(m, n_steps, s));
    if (n_steps > 0)
        m->hw = pos0 + n_steps - 1;
    if (d_tokens && n_steps > 0)
        HIP_TRY(hipMemcpyAsync(d_tokens, m->pred + pos0, sizeof(int32_t) * n_steps,
                               hipMemcpyDeviceToDevice, s));
    if (d_logits_last && n_steps > 0)
        HIP_TRY(hipMemcpyAsync(d_logits_last, m->logits, sizeof(float) * m->V,
                               hipMemcpyDeviceToDevice, s));
    return QD_OK;
}

// ------------------------------------------------------------------ batched decode entry points

extern "C" int qd_set_prompt_seq(qd_model* m, int32_t seq, const int32_t* tokens, int32_t n, qd_stream stream)
{
    if (!m)
        return fail(QD_EINVAL, "null model");
    QD_BATCHED(m);
    if (seq < 0 || seq >= m->B)
        return fail(QD_EINVAL, "sequence %d not in [0, %d)", seq, m->B);
    if (n < 0 || n > m->max_seq)
        return fail(QD_ERANGE, "prompt length %d not in [0, %d]", n, m->max_seq);
    if (n > 0 && !tokens)
        return fail(QD_EINVAL, "null tokens");
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= m->V)
            return fail(QD_ERANGE, "token[%d] = %d not in [0, %d)", i, tokens[i], m->V);
    hipStream_t s = (hipStream_t)stream;
    int32_t* ids = m->ids + (size_t)seq * m->max_seq;
    if (n > 0) {
        HIP_TRY(hipMemcpyAsync(ids, tokens, sizeof(int32_t) * n, hipMemcpyHostToDevice, s));
        HIP_TRY(hipStreamSynchronize(s));  // the host array may go away on return
    }
    hipLaunchKernelGGL(k_set_state, dim3(1), dim3(64), 0, s, m->st + seq, ids, 0, n, -1, 0);
    HIP_TRY(hipGetLastError());
    return QD_OK;
}

// host checks of per-sequence start positions of n steps
static int check_batch_positions(qd_model* m, const int32_t* pos, int32_t n_steps)
{
    if (!pos)
        return fail(QD_EINVAL, "null positions");
    for (int b = 0; b < m->B; ++b) {
        if (pos[b] < 0 || (int64_t)pos[b] + n_steps > m->max_seq)
            return fail(QD_ERANGE, "sequence %d: positions [%d, %d) not within max_seq %d", b, pos[b],
                        pos[b] + n_steps, m->max_seq);
        if (n_steps > 0 && pos[b] > m->hwb[b] + 1)
            return fail(QD_ERANGE, "sequence %d: position %d past the written prefix: positions 0..%d hold "
                                   "K/V, so the next step is at most at %d", b, pos[b], m->hwb[b], m->hwb[b] + 1);
    }
    return QD_OK;
}

extern "C" int qd_generate_batch(qd_model* m, const int32_t* pos0, int32_t n_steps, int32_t* d_tokens,
                                 float* d_logits_last, qd_stream stream)
{
    if (!m)
        return fail(QD_EINVAL, "null model");
    QD_BATCHED(m);
    if (n_steps < 0)
        return fail(QD_ERANGE, "n_steps %d < 0", n_steps);
    QD_TRY(check_batch_positions(m, pos0, n_steps));
    hipStream_t s = (hipStream_t)stream;
    for (int b = 0; b < m->B; ++b)
        hipLaunchKernelGGL(k_set_state, dim3(1), dim3(64), 0, s, m->st + b, m->ids + (size_t)b * m->max_seq,
                           pos0[b], -1, -1, 0);
    HIP_TRY(hipGetLastError());
    QD_TRY(run_steps(m, n_steps, s));
    if (n_steps > 0) {
        for (int b = 0; b < m->B; ++b)
            m->hwb[b] = pos0[b] + n_steps - 1;
        if (d_tokens)
            for (int b = 0; b < m->B; ++b)
                HIP_TRY(hipMemcpyAsync(d_tokens + (size_t)b * n_steps, m->pred + (size_t)b * m->max_seq + pos0[b],
                                       sizeof(int32_t) * n_steps, hipMemcpyDeviceToDevice, s));
        if (d_logits_last)
            HIP_TRY(hipMemcpyAsync(d_logits_last, m->blog, sizeof(float) * m->B * m->V, hipMemcpyDeviceToDevice,
                                   s));
    }
    return QD_OK;
}

extern "C" int qd_decode_step_batch(qd_model* m, const int32_t* tokens, const int32_t* pos, float* d_logits,
                                    int32_t* d_next, qd_stream stream)
{
    if (!m)
        return fail(QD_EINVAL, "null model");
    QD_BATCHED(m);
    if (!tokens)
        return fail(QD_EINVAL, "null tokens");
    for (int b = 0; b < m->B; ++b)
        if (tokens[b] < 0 || tokens[b] >= m->V)
            return fail(QD_ERANGE, "sequence %d: token %d not in [0, %d)", b, tokens[b], m->V);
    QD_TRY(check_batch_positions(m, pos, 1));
    hipStream_t s = (hipStream_t)stream;
    for (int b = 0; b < m->B; ++b)
        hipLaunchKernelGGL(k_set_state, dim3(1), dim3(64), 0, s, m->st + b, m->ids + (size_t)b * m->max_seq,
                           pos[b], pos[b] + 1, pos[b], tokens[b]);
    HIP_TRY(hipGetLastError());
    QD_TRY(run_steps(m, 1, s));
    for (int b = 0; b < m->B; ++b)
        m->hwb[b] = pos[b];
    if (d_logits)
        HIP_TRY(hipMemcpyAsync(d_logits, m->blog, sizeof(float) * m->B * m->V, hipMemcpyDeviceToDevice, s));
    if (d_next)
        for (int b = 0; b < m->B; ++b)
            HIP_TRY(hipMemcpyAsync(d_next + b, m->pred + (size_t)b * m->max_seq + pos[b], sizeof(int32_t),
                                   hipMemcpyDeviceToDevice, s));
    return QD_OK;
}

// ------------------------------------------------------------------ standalone kernels

__global__ void k_fill_f32(float* __restrict__ y, int n, float v)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        y[i] = v;
}

extern "C" int qd_gemv_q4_0(const uint16_t* d_scales, const uint8_t* d_qs, const float* d_x,
                            float* d_y, int32_t N, int32_t K, qd_stream stream)
{
    if (!d_scales || !d_qs || !d_x || !d_y)
        return fail(QD_EINVAL, "null pointer");
    if (N < 0 || K < 0 || K % 32)
        return fail(QD_EINVAL, "bad shape N=%d K=%d (K %% 32 must be 0)", N, K);
    if (gemv_lds_bytes(K / 32) > (size_t)GEMV_MAX_LDS)
        return fail(QD_EUNSUPPORTED, "K=%d above the staged-x limit", K);
    if ((uint64_t)N * (uint64_t)K / 2 >= (uint64_t)1 << 32 || N >= (1 << 24))
        return fail(QD_EUNSUPPORTED, "N=%d K=%d: above 2^32 bytes of nibbles or 2^24 rows", N, K);
    if ((reinterpret_cast<uintptr_t>(d_qs) | reinterpret_cast<uintptr_t>(d_x)) & 15)
        return fail(QD_EINVAL, "qs and x must be 16-byte aligned");
    if (N == 0)
        return QD_OK;
    if (K == 0) {   // y = 0 by a fill kernel (no memset node inside a captured graph)
        hipLaunchKernelGGL(k_fill_f32, dim3((N + 255) / 256), dim3(256), 0, (hipStream_t)stream, d_y, N,
                           0.f);
        HIP_TRY(hipGetLastError());
        return QD_OK;
    }
    HIP_TRY(launch_gemv_plain(d_scales, d_qs, d_x, d_y, N, K, (hipStream_t)stream));
    return QD_OK;
}

// ------------------------------------------------------------------ rotary frequencies

// inv_freq for qd_config (host only): theta^(-2i/rot_dim) for i < rot_dim/2,
// evaluated in f64 and rounded to f32 once, with the rotary-scaling rules of
// the inferencelayer cuda_llm.rs page (Cfg::rope_inv_freq): linear divides
// every frequency by `factor`; llama3 divides the frequencies whose wavelength
// 2*pi/f is above original_max_pos/low_freq_factor by `factor`, keeps those
// below original_max_pos/high_freq_factor, and between the two blends
// (1 - s) * f/factor + s * f with s = (original_max_pos/wavelength -
// low_freq_factor) / (high_freq_factor - low_freq_factor).  Any other type is
// refused, as on the page.
extern "C" int qd_rope_inv_freq(float theta, int32_t rot_dim, int32_t scaling, float factor,
                                float low_freq_factor, float high_freq_factor,
                                float original_max_pos, float* out)
{
    if (!out)
        return fail(QD_EINVAL, "null output");
    if (rot_dim <= 0 || rot_dim % 2)
        return fail(QD_EINVAL, "rot_dim %d must be positive and even", rot_dim);
    if (!(theta > 1.0f) || !std::isfinite(theta))
        return fail(QD_EINVAL, "theta %g must be finite and above 1", (double)theta);
    if (scaling < QD_ROPE_DEFAULT || scaling > QD_ROPE_LLAMA3)
        return fail(QD_EUNSUPPORTED, "rotary scaling type %d is not implemented", scaling);
    const double fac = factor, lo = low_freq_factor, hi = high_freq_factor, orig = original_max_pos;
    if (scaling != QD_ROPE_DEFAULT && !(fac > 0.0 && std::isfinite(fac)))
        return fail(QD_EINVAL, "scaling factor %g must be finite and positive", fac);
    if (scaling == QD_ROPE_LLAMA3 &&
        !(lo > 0.0 && hi > lo && std::isfinite(hi) && orig > 0.0 && std::isfinite(orig)))
        return fail(QD_EINVAL, "llama3 scaling needs 0 < low_freq_factor < high_freq_factor and "
                    "original_max_pos > 0 (got %g, %g, %g)", lo, hi, orig);
    const double pi = 3.14159265358979323846;
    for (int i = 0; i < rot_dim / 2; ++i) {
        double f = std::pow((double)theta, -2.0 * i / (double)rot_dim);
        if (scaling == QD_ROPE_LINEAR) {
            f /= fac;
        } else if (scaling == QD_ROPE_LLAMA3) {
            const double wl = 2.0 * pi / f;
            if (wl > orig / lo) {
                f /= fac;
            } else if (wl >= orig / hi) {
                const double sm = (orig / wl - lo) / (hi - lo);
                f = (1.0 - sm) * (f / fac) + sm * f;
            }
        }
        out[i] = (float)f;
    }
    return QD_OK;
}

// ------------------------------------------------------------------ batched GEMV

// launch configuration of the batched GEMV: rows per slot, waves, block
// groups per item, register buffers, items per unrolled chunk, non-temporal
// weight loads (lanes per row: 16 or 8, following K)
// (rows per slot: 4 up to 4 vectors, 2 above, where the registers of 4 rows of
// decoded codes and 8 accumulators per row cost more than the shared LDS reads)
#ifndef QD_CFG_BATCH
#define QD_CFG_BATCH 8, 1, 2, 8   // waves, block groups, buffers, unroll; tunable at compile time
#endif
constexpr int GB_CFG[4] = {QD_CFG_BATCH};
constexpr int GB_NW = GB_CFG[0], GB_BG = GB_CFG[1], GB_NBUF = GB_CFG[2], GB_UNR = GB_CFG[3];
constexpr bool GB_NTL = true;
__host__ __device__ constexpr int gb_rps(int nc) { return nc <= 4 ? 4 : 2; }
constexpr int GB_GRID_CAP = 512;

template <int NC, int L>
static hipError_t launch_gemv_batch_l(const uint16_t* d, const uint8_t* q, const float* x, float* y,
                                      int N, int nb, hipStream_t s)
{
    const size_t lds = gemv_batch_lds_bytes(nb, NC);
    if (lds > 64 * 1024) {
        // dynamic LDS above 64 KB is opted into per kernel (160 KB per CU on gfx950)
        static size_t allowed = 0;
        if (lds > allowed) {
            const hipError_t e = hipFuncSetAttribute(
                reinterpret_cast<const void*>(&k_gemv_batch<NC, L, gb_rps(NC), GB_NW, GB_BG, GB_NBUF, GB_UNR, GB_NTL>),
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess)
                return e;
            allowed = lds;
        }
    }
    const int rows = GB_NW * (WAVE / L) * gb_rps(NC);
    const int grid = std::max(1, std::min((N + rows - 1) / rows, GB_GRID_CAP));
    hipLaunchKernelGGL((k_gemv_batch<NC, L, gb_rps(NC), GB_NW, GB_BG, GB_NBUF, GB_UNR, GB_NTL>), dim3(grid),
                       dim3(GB_NW * WAVE), lds, s, d, q, x, y, N, nb);
    return hipGetLastError();
}

// the matrix-core kernel from QD_BATCH_MFMA_MIN vectors on (measured faster at
// 6 and more at 24576 x 4096; below that the vector kernel is faster)
#ifndef QD_BATCH_MFMA_MIN
#define QD_BATCH_MFMA_MIN 6
#endif

// K in ks slices of whole chunks, partial products to y + k * NC * N; two row
// groups per wave once one would give 768 workgroups or more
template <int NC>
static hipError_t launch_gemv_batch_mfma(const uint16_t* d, const uint8_t* q, const float* x, float* y,
                                         int N, int nb, hipStream_t s, int ks)
{
    const int nch = (nb + GBM_KC - 1) / GBM_KC;
    const int kch = (nch + ks - 1) / ks;
    if (ks < 1 || (int64_t)(ks - 1) * kch >= nch)   // every slice holds at least one chunk
        return hipErrorInvalidValue;
    const int dvec = (nb % 8 == 0 && reinterpret_cast<uintptr_t>(d) % 16 == 0) ? 1 : 0;
    const int t1 = (N + gbm_rows(1) - 1) / gbm_rows(1);
    if ((int64_t)t1 * ks >= 768) {
        hipLaunchKernelGGL((k_gemv_batch_mfma<NC, 2>), dim3((N + gbm_rows(2) - 1) / gbm_rows(2), ks),
                           dim3(GBM_NW * WAVE), gemv_batch_mfma_lds_bytes(), s, d, q, x, y, N, nb, kch,
                           (size_t)NC * N, dvec);
    } else {
        hipLaunchKernelGGL((k_gemv_batch_mfma<NC, 1>), dim3(t1, ks), dim3(GBM_NW * WAVE),
                           gemv_batch_mfma_lds_bytes(), s, d, q, x, y, N, nb, kch, (size_t)NC * N, dvec);
    }
    return hipGetLastError();
}

template <int NC>
static hipError_t launch_gemv_batch(const uint16_t* d, const uint8_t* q, const float* x, float* y,
                                    int N, int K, hipStream_t s)
{
    const int nb = K / 32;
    static_assert(QD_BATCH_MFMA_MIN >= 2 && QD_BATCH_MFMA_MIN <= GB_MAXB + 1, "kernel switch");
    if constexpr (NC >= QD_BATCH_MFMA_MIN) {
        return launch_gemv_batch_mfma<NC>(d, q, x, y, N, nb, s);
    } else {
        if ((int64_t)NC * K > GB_MAXKB)   // the batch does not fit the vector kernel's LDS
            return launch_gemv_batch_mfma<NC>(d, q, x, y, N, nb, s);
        if (pick_lpr(nb, 16) == 16)
            return launch_gemv_batch_l<NC, 16>(d, q, x, y, N, nb, s);
        return launch_gemv_batch_l<NC, 8>(d, q, x, y, N, nb, s);
    }
}

extern "C" int qd_gemv_q4_0_batch(const uint16_t* d_scales, const uint8_t* d_qs, const float* d_x,
                                  float* d_y, int32_t N, int32_t K, int32_t B, qd_stream stream)
{
    if (!d_scales || !d_qs || !d_x || !d_y)
        return fail(QD_EINVAL, "null pointer");
    if (N < 0 || K < 0 || K % 32)
        return fail(QD_EINVAL, "bad shape N=%d K=%d (K %% 32 must be 0)", N, K);
    if (B < 1 || B > GBM_MAXB)
        return fail(QD_EINVAL, "batch B=%d outside [1, %d]", B, GBM_MAXB);
    if (B == 1 && gemv_lds_bytes(K / 32) > (size_t)GEMV_MAX_LDS)
        return fail(QD_EUNSUPPORTED, "K=%d above the staged-x limit", K);
    if ((uint64_t)N * (uint64_t)K / 2 >= (uint64_t)1 << 32 || N >= (1 << 24))
        return fail(QD_EUNSUPPORTED, "N=%d K=%d: above 2^32 bytes of nibbles or 2^24 rows", N, K);
    if ((reinterpret_cast<uintptr_t>(d_qs) | reinterpret_cast<uintptr_t>(d_x)) & 15)
        return fail(QD_EINVAL, "qs and x must be 16-byte aligned");
    if (N == 0)
        return QD_OK;
    const hipStream_t s = (hipStream_t)stream;
    if (K == 0) {   // Y = 0 by a fill kernel (no memset node inside a captured graph)
        const int n = N * B;
        hipLaunchKernelGGL(k_fill_f32, dim3((n + 255) / 256), dim3(256), 0, s, d_y, n, 0.f);
        HIP_TRY(hipGetLastError());
        return QD_OK;
    }
    HIP_TRY(gemv_batch_launch(d_scales, d_qs, d_x, d_y, N, K, B, s));
    return QD_OK;
}

static hipError_t gemv_batch_launch(const uint16_t* d, const uint8_t* q, const float* x, float* y, int N, int K,
                                    int B, hipStream_t s)
{
    switch (B) {
    case 1: return launch_gemv_plain(d, q, x, y, N, K, s);
    case 2: return launch_gemv_batch<2>(d, q, x, y, N, K, s);
    case 3: return launch_gemv_batch<3>(d, q, x, y, N, K, s);
    case 4: return launch_gemv_batch<4>(d, q, x, y, N, K, s);
    case 5: return launch_gemv_batch<5>(d, q, x, y, N, K, s);
    case 6: return launch_gemv_batch<6>(d, q, x, y, N, K, s);
    case 7: return launch_gemv_batch<7>(d, q, x, y, N, K, s);
    case 8: return launch_gemv_batch<8>(d, q, x, y, N, K, s);
    case 9: return launch_gemv_batch<9>(d, q, x, y, N, K, s);
    case 10: return launch_gemv_batch<10>(d, q, x, y, N, K, s);
    case 11: return launch_gemv_batch<11>(d, q, x, y, N, K, s);
    case 12: return launch_gemv_batch<12>(d, q, x, y, N, K, s);
    case 13: return launch_gemv_batch<13>(d, q, x, y, N, K, s);
    case 14: return launch_gemv_batch<14>(d, q, x, y, N, K, s);
    case 15: return launch_gemv_batch<15>(d, q, x, y, N, K, s);
    default: return launch_gemv_batch<16>(d, q, x, y, N, K, s);
    }
}

// ------------------------------------------------------------------ expert GEMV

extern "C" int qd_gemv_q4_0_experts(const uint16_t* d_scales, const uint8_t* d_qs,
                                    const int32_t* d_experts, int32_t n_experts, int32_t k,
                                    const float* d_x, float* d_y, int32_t N, int32_t K,
                                    qd_stream stream)
{
    if (!d_scales || !d_qs || !d_experts || !d_x || !d_y)
        return fail(QD_EINVAL, "null pointer");
    if (N < 0 || K < 0 || K % 32 || n_experts <= 0 || k < 0)
        return fail(QD_EINVAL, "bad shape N=%d K=%d n_experts=%d k=%d", N, K, n_experts, k);
    if (k > 65535 || (int64_t)N * k >= ((int64_t)1 << 31))
        return fail(QD_EUNSUPPORTED, "k=%d experts per call (above 65535, or N*k >= 2^31)", k);
    if (gemv_lds_bytes(K / 32) > (size_t)GEMV_MAX_LDS)
        return fail(QD_EUNSUPPORTED, "K=%d above the staged-x limit", K);
    if ((uint64_t)N * (uint64_t)K / 2 >= (uint64_t)1 << 32 || N >= (1 << 24))
        return fail(QD_EUNSUPPORTED, "N=%d K=%d: above 2^32 bytes of nibbles or 2^24 rows", N, K);
    if ((reinterpret_cast<uintptr_t>(d_qs) | reinterpret_cast<uintptr_t>(d_x)) & 15)
        return fail(QD_EINVAL, "qs and x must be 16-byte aligned");
    if (N == 0 || k == 0)
        return QD_OK;
    const hipStream_t s = (hipStream_t)stream;
    if (K == 0) {
        hipLaunchKernelGGL(k_fill_f32, dim3((N * k + 255) / 256), dim3(256), 0, s, d_y, N * k, 0.f);
        HIP_TRY(hipGetLastError());
        return QD_OK;
    }
    const int nb = K / 32, lpr = pick_lpr(nb);
    const dim3 grid(gemv_grid(CFG_O, lpr, N), k);
    switch (lpr) {
#define QD_EXP(L)                                                                                  \
    case L:                                                                                        \
        hipLaunchKernelGGL((k_gemv_experts<L, QD_CFG_O>), grid, dim3(QD_NW(QD_CFG_O) * WAVE),        \
                           gemv_lds_bytes(nb), s, d_scales, d_qs, d_experts, n_experts, d_x, d_y, N, nb); \
        break;
    QD_EXP(64) QD_EXP(32) QD_EXP(16)
    default:
        hipLaunchKernelGGL((k_gemv_experts<8, QD_CFG_O>), grid, dim3(QD_NW(QD_CFG_O) * WAVE),
                           gemv_lds_bytes(nb), s, d_scales, d_qs, d_experts, n_experts, d_x, d_y, N, nb);
        break;
#undef QD_EXP
    }
    HIP_TRY(hipGetLastError());
    return QD_OK;
}

// Grid of qd_attn_decode.  The split kernel holds 212 VGPRs, so a compute
// unit runs 8 of its waves.  One sequence: 256 workgroups of 8 waves, one
// resident round.  Several: 2048 workgroups of 4 waves, so that the longest
// sequences' splits hold fewer keys (a split past a sequence's kv_len returns
// at once).  Measured (graph of 100 launches over rotated pools, f16 / fp8):
// one sequence at kv_len 32768 32.4 / 24.0 us against 40.1 / 29.4 with 1024
// x 4 waves for every B, 4096 11.2 / 10.6 against 12.7 / 12.1, 512 8.7 / 8.5
// against 8.1 / 8.1; 8 sequences of mixed lengths up to 16384 70.4 / 49.0
// against 89.1 / 65.1.
#ifndef QD_ATT_SA1_WGS
#define QD_ATT_SA1_WGS 256
#endif
#ifndef QD_ATT_SA_WGS
#define QD_ATT_SA_WGS 2048
#endif
static AttnGeom standalone_geom(int32_t B, int32_t nq, int32_t nkv, int32_t max_kv)
{
    // the kernel's LDS rows and launch bound hold 8 waves up to GQA 4, 4 beyond
    const int wmax = nq / nkv <= 4 ? 8 : 4;
    if (B == 1)
        return attn_geom(B, nkv, max_kv, QD_ATT_SA1_WGS * 8 / wmax, wmax, wmax);
    return attn_geom(B, nkv, max_kv, QD_ATT_SA_WGS, 4, 4);
}

static size_t attn_ws_layout(int32_t B, int32_t nq, int32_t nkv, int32_t hd, int32_t max_kv,
                             AttnGeom* g)
{
    *g = standalone_geom(B, nq, nkv, max_kv);
    return (size_t)B * nq * g->nsplit * (hd + 2) * sizeof(float);
}

extern "C" size_t qd_attn_workspace_bytes(int32_t B, int32_t nq, int32_t nkv, int32_t head_dim,
                                          int32_t max_kv_len)
{
    if (B <= 0 || nq <= 0 || nkv <= 0 || head_dim <= 0 || max_kv_len < 0)
        return 0;
    AttnGeom g;
    return attn_ws_layout(B, nq, nkv, head_dim, max_kv_len, &g);
}

// Argument checks of the standalone attention (no HIP call).
template <bool KV8>
static int attn_validate(const qd_attn_args* a, float k_scale, float v_scale)
{
    if (!a)
        return fail(QD_EINVAL, "null args");
    if (!a->q || !a->k || !a->v || !a->kv_lens || !a->out)
        return fail(QD_EINVAL, "null pointer");
    if (a->B < 0 || a->nq <= 0 || a->nkv <= 0 || a->max_kv_len < 0)
        return fail(QD_EINVAL, "bad sizes");
    if (a->nq % a->nkv)
        return fail(QD_EINVAL, "nq %% nkv != 0");
    const int gq = a->nq / a->nkv;
    if (gq != 1 && gq != 2 && gq != 4 && gq != 8)
        return fail(QD_EUNSUPPORTED, "GQA group %d not in {1,2,4,8}", gq);
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(QD_EUNSUPPORTED, "head_dim %d not in {64,128}", a->head_dim);
    if (a->block_tables) {
        if (a->block_size != ATT_BS)
            return fail(QD_EUNSUPPORTED, "block_size %d (only %d)", a->block_size, ATT_BS);
        if ((int64_t)a->max_blocks_per_seq * ATT_BS < a->max_kv_len)
            return fail(QD_EINVAL, "max_blocks_per_seq too small for max_kv_len");
    }
    if (KV8) {
        if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
            return fail(QD_EINVAL, "fp8 K/V scales must be finite and positive");
        if ((reinterpret_cast<uintptr_t>(a->k) | reinterpret_cast<uintptr_t>(a->v)) & 15)
            return fail(QD_EINVAL, "fp8 K/V pools must be 16-byte aligned");
    }
    return QD_OK;
}

template <bool KV8>
static int attn_decode_impl(const qd_attn_args* a, float k_scale, float v_scale, void* d_workspace,
                            size_t workspace_bytes, qd_stream stream)
{
    QD_TRY(attn_validate<KV8>(a, k_scale, v_scale));
    if (!d_workspace)
        return fail(QD_EINVAL, "null workspace");
    if (a->B == 0)
        return QD_OK;
    AttnGeom geo;
    const size_t need = attn_ws_layout(a->B, a->nq, a->nkv, a->head_dim, a->max_kv_len, &geo);
    if (workspace_bytes < need)
        return fail(QD_EINVAL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    AttnParams p;
    memset(&p, 0, sizeof p);
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.tables = a->block_tables;
    p.mbps = a->max_blocks_per_seq;
    p.kv_lens = a->kv_lens;
    p.pos = nullptr;
    p.max_kv = a->max_kv_len;
    p.nq = a->nq;
    p.nkv = a->nkv;
    p.scale = a->scale;
    p.chunk = geo.chunk;
    p.nsplit = geo.nsplit;
    p.part = reinterpret_cast<float*>(d_workspace);
    p.out = a->out;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    HIP_TRY((launch_attention<0, KV8>(p, geo.waves, a->head_dim, a->nq / a->nkv, a->block_tables != nullptr, a->B, a->nq,
                             (hipStream_t)stream)));
    HIP_TRY(hipGetLastError());
    return QD_OK;
}

extern "C" int qd_attn_decode(const qd_attn_args* a, void* d_workspace, size_t workspace_bytes,
                              qd_stream stream)
{
    return attn_decode_impl<false>(a, 1.f, 1.f, d_workspace, workspace_bytes, stream);
}

extern "C" int qd_attn_decode_kv8(const qd_attn_args* a, float k_scale, float v_scale,
                                  void* d_workspace, size_t workspace_bytes, qd_stream stream)
{
    return attn_decode_impl<true>(a, k_scale, v_scale, d_workspace, workspace_bytes, stream);
}

// ------------------------------------------------------------------ attention without allocation

// The split-KV partials of qd_attn_decode_noalloc: a file-scope device array,
// one copy per GPU the library runs on, held until the process ends.  On the
// host its name is only a stand-in for the symbol: the device address of each
// GPU's copy comes from hipGetSymbolAddress (looked up once per device, with
// that device current, on the entry point's first call there) and only that
// address is handed to kernels.
constexpr size_t QD_NOALLOC_SCRATCH_BYTES = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[QD_NOALLOC_SCRATCH_BYTES];

constexpr int QD_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[QD_MAX_DEVICES];

// device address of the current device's scratch array
static int noalloc_scratch(void** out)
{
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= QD_MAX_DEVICES)
        return fail(QD_EUNSUPPORTED, "device %d: the no-allocation entry point keeps scratch for "
                                     "devices 0..%d", dev, QD_MAX_DEVICES - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(QD_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QD_OK;
}

extern "C" size_t qd_attn_noalloc_max_bytes(void) { return QD_NOALLOC_SCRATCH_BYTES; }

extern "C" int qd_attn_decode_noalloc(const qd_attn_args* a, qd_stream stream)
{
    QD_TRY(attn_validate<false>(a, 1.f, 1.f));
    if (a->B == 0)
        return QD_OK;
    AttnGeom geo;
    const size_t need = attn_ws_layout(a->B, a->nq, a->nkv, a->head_dim, a->max_kv_len, &geo);
    if (need > QD_NOALLOC_SCRATCH_BYTES)
        return fail(QD_EUNSUPPORTED, "these sizes need %zu bytes of split partials, above the %zu bytes "
                                     "of the no-allocation entry point's scratch (use qd_attn_decode "
                                     "with a workspace)", need, QD_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    QD_TRY(noalloc_scratch(&ws));
    return attn_decode_impl<false>(a, 1.f, 1.f, ws, QD_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" int qd_check(qd_model* m, qd_stream stream)
{
    if (!m)
        return fail(QD_EINVAL, "null model");
    HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
    std::vector<StepState> hs(m->B);
    HIP_TRY(hipMemcpy(hs.data(), m->st, sizeof(StepState) * m->B, hipMemcpyDeviceToHost));
    int32_t err = 0;
    for (const StepState& x : hs)
        err |= x.error;
    if (err == 0)
        return QD_OK;
    const int32_t zero = 0;
    for (int b = 0; b < m->B; ++b)
        HIP_TRY(hipMemcpy(&m->st[b].error, &zero, sizeof zero, hipMemcpyHostToDevice));
    if (err & 4)
        return fail(QD_EHIP, "a device-wide barrier of the layer kernel timed out: the steps since "
                             "the last check are invalid");
    return fail(QD_ERANGE, "a step saw a %s out of range", (err & 1) ? "token" : "position");
}

extern "C" size_t qd_stream_read_groups(size_t bytes)
{
    return (bytes < 16 || bytes % 16) ? 0 : (size_t)stream_read_groups(bytes);
}

extern "C" int qd_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink, qd_stream stream)
{
    if (!d_src || !d_sink)
        return fail(QD_EINVAL, "null pointer");
    if (bytes == 0 || bytes % 16)
        return fail(QD_EINVAL, "bytes=%zu must be a positive multiple of 16", bytes);
    if (reinterpret_cast<uintptr_t>(d_src) & 15)
        return fail(QD_EINVAL, "src must be 16-byte aligned");
    hipLaunchKernelGGL(k_stream_read, dim3(stream_read_groups(bytes)), dim3(SR_THREADS), 0,
                       (hipStream_t)stream, reinterpret_cast<const uint4*>(d_src), bytes / 16, d_sink);
    HIP_TRY(hipGetLastError());
    return QD_OK;
}

// ------------------------------------------------------------------ chunked prefill

// Chunk attention with each K/V tile read once for the chunk's queries
// (k_pf_attn, f16 caches): the chunk's positions in pieces of tp (a
// workgroup's query rows, tp * gq <= QD_PF_ATT_ROWS), about QD_PF_ATT_WGS
// workgroups over (key split, kv head, piece), at most PF_FA_MAXS splits of a
// multiple of 16 keys, then the combine.
#ifndef QD_PF_ATT_WGS
#define QD_PF_ATT_WGS 256
#endif
#ifndef QD_PF_ATT_ROWS
#define QD_PF_ATT_ROWS 128
#endif
constexpr int PF_FA_MAXS = 64;
template <int GQ>
constexpr int pf_att_tp() { return PF_T < QD_PF_ATT_ROWS / GQ ? PF_T : QD_PF_ATT_ROWS / GQ; }
// the split merge of the prefill's chunk attention, one round of loads per
// split group (U * 2 >= nsplit splits)
template <int HD>
static void pf_combine_xp(qd_model* m, int nsplit, int chunk, int T, const float* gate, size_t gslab,
                          hipStream_t s)
{
    auto& P = m->pf;
    const dim3 grid(gbm_nchunks(m->nq * HD / 32, PF_NG), T), block(FA_CMB_THREADS);
    const int half = (nsplit + 1) / 2;
#define QD_CMB(U_)                                                                                  \
    hipLaunchKernelGGL((k_attn_combine_xp<HD, U_>), grid, block, 0, s, P.fa, nsplit, chunk, P.lens,  \
                       m->max_seq, m->nq, P.xp_o, P.xs_o, gate, m->qkv_rows, P.ks_qkv, gslab)
    if (half <= 2)
        QD_CMB(2);
    else if (half <= 4)
        QD_CMB(4);
    else if (half <= 8)
        QD_CMB(8);
    else if (half <= 16)
        QD_CMB(16);
    else
        QD_CMB(32);
#undef QD_CMB
}

// the prefill's chunk attention (f16 cache), its split merge writing the o
// product's input (P.xp_o, P.xs_o; times sigmoid(gate) when gate is given)
static void pf_attention(qd_model* m, DevLayer& Ly, int p0, int T, const float* gate, size_t gslab, hipStream_t s)
{
    auto& P = m->pf;
    const int kv_total = p0 + T, gq = m->nq / m->nkv;
    const int tp = std::min(PF_T, QD_PF_ATT_ROWS / gq), npiece = (T + tp - 1) / tp;
    const int target = std::max(1, QD_PF_ATT_WGS / (m->nkv * npiece));
    int chunk = (kv_total + target - 1) / target;
    chunk = std::max(chunk, (kv_total + PF_FA_MAXS - 1) / PF_FA_MAXS);
    chunk = std::max(16, (chunk + 15) / 16 * 16);
    const int nsplit = (kv_total + chunk - 1) / chunk;
    FaParams f;
    f.q = P.Q;
    f.k = Ly.kc;
    f.v = Ly.vc;
    f.table = m->paged ? m->table : nullptr;
    f.max_kv = m->max_seq;
    f.nq = m->nq;
    f.nkv = m->nkv;
    f.T = T;
    f.p0 = p0;
    f.scale = 1.0f / sqrtf((float)m->hd);
    f.chunk = chunk;
    f.nsplit = nsplit;
    f.part = P.fa;
    f.tp = tp;
    const dim3 grid(nsplit, m->nkv, npiece);
#define QD_FA_GQ(HD_, GQ_)                                                                          \
    hipLaunchKernelGGL((k_pf_attn<HD_, GQ_, GQ_ * pf_att_tp<GQ_>() / 16>), grid,                    \
                       dim3(GQ_ * pf_att_tp<GQ_>() / 16 * WAVE), 0, s, f)
#define QD_FA(HD_)                                                                                 \
    switch (gq) {                                                                                  \
    case 1: QD_FA_GQ(HD_, 1); break;                                                               \
    case 2: QD_FA_GQ(HD_, 2); break;                                                               \
    case 4: QD_FA_GQ(HD_, 4); break;                                                               \
    default: QD_FA_GQ(HD_, 8); break;                                                              \
    }                                                                                              \
    pf_combine_xp<HD_>(m, nsplit, chunk, T, gate, gslab, s);
    if (m->hd == 128) {
        QD_FA(128)
    } else {
        QD_FA(64)
    }
#undef QD_FA
#undef QD_FA_GQ
}

static int pf_setup(qd_model* m)
{
    if (m->pf.ready)
        return QD_OK;
    auto& P = m->pf;
    const size_t T = PF_T, nqd = (size_t)m->nq * m->hd, H = m->H, I = m->I;
    const size_t ws = attn_ws_layout(PF_T, m->nq, m->nkv, m->hd, m->max_seq, &P.geo);
    if (m->H > 16384)   // the batched RMSNorm splits at most 2 items per thread
        return fail(QD_EUNSUPPORTED, "qd_prefill supports hidden <= 16384 (got %d)", m->H);
    P.ks_qkv = step_kslices(m->qkv_rows, m->H / 32, PF_NG, PF_RG_QKV, QD_PF_KS_WGS);
    P.ks_o = step_kslices(m->H, (int)nqd / 32, PF_NG, PF_RG_O, QD_PF_KS_WGS);
    P.ks_gu = step_kslices(2 * m->I, m->H / 32, PF_NG, PF_RG_GU, QD_PF_KS_WGS);
    P.ks_down = step_kslices(m->H, m->I / 32, PF_NG, PF_RG_DOWN, QD_PF_KS_WGS);
    const size_t ch_h = gbm_nchunks(m->H / 32, PF_NG), ch_o = gbm_nchunks((int)nqd / 32, PF_NG),
                 ch_i = gbm_nchunks(m->I / 32, PF_NG), S = 16 * PF_NG;
    int rc;
    if ((rc = dev_alloc_t(m, &P.X, T * H)) || (rc = dev_alloc_t(m, &P.Q, T * nqd)) ||
        (rc = dev_alloc_t(m, &P.O, T * nqd)) || (rc = dev_alloc_t(m, &P.HF, T * H)) ||
        (rc = dev_alloc_t(m, &P.QKV, (size_t)P.ks_qkv * T * m->qkv_rows)) ||
        (rc = dev_alloc_t(m, &P.OD, (size_t)std::max(P.ks_o, P.ks_down) * T * H)) ||
        (rc = dev_alloc_t(m, &P.GU, (size_t)P.ks_gu * T * 2 * I)) ||
        (rc = dev_alloc_t(m, &P.xp_h, ch_h * GBM_XP_CHUNK)) || (rc = dev_alloc_t(m, &P.xp_o, ch_o * GBM_XP_CHUNK)) ||
        (rc = dev_alloc_t(m, &P.xp_i, ch_i * GBM_XP_CHUNK)) || (rc = dev_alloc_t(m, &P.xs_h, ch_h * S)) ||
        (rc = dev_alloc_t(m, &P.xs_o, ch_o * S)) || (rc = dev_alloc_t(m, &P.xs_i, ch_i * S)) ||
        (rc = dev_alloc_t(m, &P.sq_h, ch_h * S)) ||
        (rc = dev_alloc_t(m, &P.fa, T * nqd / m->hd * PF_FA_MAXS * (m->hd + 2))) ||
        (rc = dev_alloc_t(m, &P.lens, T)) || (rc = dev_alloc_t(m, &P.iota, (size_t)m->V)) ||
        (rc = dev_alloc_t(m, &P.ws, ws / sizeof(float) + 1)))
        return rc;
    hipLaunchKernelGGL(k_pf_iota, dim3((m->V + 255) / 256), dim3(256), 0, 0, P.iota, m->V);
    // the split inputs are read for all 16 slots: slots past a short chunk
    // (stale from an earlier chunk, or zero) only feed outputs never written
    if (hipMemset(P.xp_h, 0, ch_h * GBM_XP_CHUNK * sizeof(_Float16)) != hipSuccess ||
        hipMemset(P.xp_o, 0, ch_o * GBM_XP_CHUNK * sizeof(_Float16)) != hipSuccess ||
        hipMemset(P.xp_i, 0, ch_i * GBM_XP_CHUNK * sizeof(_Float16)) != hipSuccess ||
        hipMemset(P.xs_h, 0, ch_h * S * sizeof(float)) != hipSuccess ||
        hipMemset(P.xs_o, 0, ch_o * S * sizeof(float)) != hipSuccess ||
        hipMemset(P.xs_i, 0, ch_i * S * sizeof(float)) != hipSuccess ||
        hipMemset(P.sq_h, 0, ch_h * S * sizeof(float)) != hipSuccess)
        return fail(QD_EHIP, "prefill buffer set-up failed");
    if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess)
        return fail(QD_EHIP, "prefill buffer set-up failed");
    P.ready = true;
    return QD_OK;
}

// the chunk's product over its T positions (vector slots in PF_NG groups of
// 16); SQ: the input is a hidden-sized split written by k_resid_norm_xp_batch
static hipError_t pf_gemv(const qd_model* m, const DevQ4& W, const _Float16* XP, const float* XS, int T, float* Y,
                          int ks, int rg, hipStream_t s, const float* SQ = nullptr)
{
    if (SQ)
        return xp_gemv<PF_NG>(W, XP, XS, Y, T, ks, rg, s, SQ, gbm_nchunks(m->H / 32, PF_NG), (float)m->H, m->eps);
    return xp_gemv<PF_NG>(W, XP, XS, Y, T, ks, rg, s);
}

extern "C" int32_t qd_prefill_chunk(void) { return PF_T; }

extern "C" int qd_prefill(qd_model* m, int32_t pos0, int32_t n, float* d_logits_last, qd_stream stream)
{
    if (!m)
        return fail(QD_EINVAL, "null model");
    QD_ONE_SEQUENCE(m);
    if (n <= 0 || pos0 < 0 || (int64_t)pos0 + n > m->max_seq)
        return fail(QD_ERANGE, "positions [%d, %d) not in [0, %d)", pos0, pos0 + n, m->max_seq);
    if (pos0 > m->hw + 1)
        return fail(QD_ERANGE, "pos0 %d past the written prefix: positions 0..%d hold K/V, so the "
                               "next position is at most %d", pos0, m->hw, m->hw + 1);
    QD_TRY(pf_setup(m));
    auto& P = m->pf;
    const hipStream_t s = (hipStream_t)stream;
    const int H = m->H, hd = m->hd, gq = m->nq / m->nkv;
    const int mbps = (m->max_seq + ATT_BS - 1) / ATT_BS;
    const int nqd = m->nq * hd, I = m->I;
    int T = 0;
    for (int c0 = 0; c0 < n; c0 += PF_T) {
        T = std::min(PF_T, n - c0);
        const int p0 = pos0 + c0;
        const size_t slab_h = (size_t)T * H;
        hipLaunchKernelGGL(k_pf_embed, dim3((H + 255) / 256, T), dim3(256), 0, s, m->embed.d, m->embed.qs,
                           H, m->ids, p0, P.X);
        const dim3 ngrid(gbm_nchunks(H / 32, PF_NG), T), nblock(gbm_chunk_threads(PF_NG));
        hipLaunchKernelGGL(k_resid_norm_xp_batch, ngrid, nblock, 0, s, P.X, nullptr, 0, (size_t)0, H,
                           m->layers[0].attn_norm, PF_NG, P.xp_h, P.xs_h, P.sq_h);
        for (int l = 0; l < m->L; ++l) {
            DevLayer& Ly = m->layers[l];
            HIP_TRY(pf_gemv(m, Ly.qkv, P.xp_h, P.xs_h, T, P.QKV, P.ks_qkv, PF_RG_QKV, s, P.sq_h));
            const size_t slab_qkv = (size_t)T * m->qkv_rows;
            const float* qn = m->qk_norm ? Ly.q_norm : m->ones_hd;
            const float* kn = m->qk_norm ? Ly.k_norm : m->ones_hd;
            const int32_t* tbl = m->paged ? m->table : nullptr;
            const dim3 g(m->nq + m->nkv, T);
#define QD_PFQK(HD_, K8_)                                                                            \
    hipLaunchKernelGGL((k_pf_qk<HD_, K8_>), g, dim3(WAVE), 0, s, P.QKV, m->qkv_rows, m->nq, m->nkv, qn,  \
                       kn, m->qk_norm, m->eps, m->rot, m->rope_cos, m->rope_sin, p0, P.Q, Ly.kc, Ly.vc, \
                       tbl, m->max_seq, m->k_scale, m->v_scale, P.lens, P.ks_qkv, slab_qkv)
            if (hd == 128) {
                if (m->kv_fp8) QD_PFQK(128, true); else QD_PFQK(128, false);
            } else {
                if (m->kv_fp8) QD_PFQK(64, true); else QD_PFQK(64, false);
            }
#undef QD_PFQK
            if (m->kv_fp8) {
                // fp8 cache: the decode attention, each query of the chunk as a sequence
                AttnParams p;
                memset(&p, 0, sizeof p);
                p.q = P.Q;
                p.k = Ly.kc;
                p.v = Ly.vc;
                p.tables = tbl;
                p.mbps = mbps;
                p.kv_lens = P.lens;
                p.max_kv = m->max_seq;
                p.nq = m->nq;
                p.nkv = m->nkv;
                p.scale = 1.0f / sqrtf((float)hd);
                p.chunk = P.geo.chunk;
                p.nsplit = P.geo.nsplit;
                p.part = P.ws;
                p.out = P.O;
                p.k_scale = m->k_scale;
                p.v_scale = m->v_scale;
                p.shared_kv = 1;
                HIP_TRY((launch_attention<0, true>(p, P.geo.waves, hd, gq, m->paged, T, m->nq, s)));
            }
            // the gate rows follow q|k|v in the fused product
            const float* gate = m->attn_gate ? P.QKV + (size_t)(m->nq + 2 * m->nkv) * hd : nullptr;
            if (m->kv_fp8)
                hipLaunchKernelGGL(k_xsplit_batch, dim3(gbm_nchunks(nqd / 32, PF_NG), T),
                                   dim3(gbm_chunk_threads(PF_NG)), 0, s, P.O, nqd / 32, PF_NG, P.xp_o, P.xs_o, gate,
                                   m->qkv_rows, P.ks_qkv, slab_qkv);
            else
                pf_attention(m, Ly, p0, T, gate, slab_qkv, s);   // writes the split itself
            HIP_TRY(pf_gemv(m, Ly.o, P.xp_o, P.xs_o, T, P.OD, P.ks_o, PF_RG_O, s));
            hipLaunchKernelGGL(k_resid_norm_xp_batch, ngrid, nblock, 0, s, P.X, P.OD, P.ks_o, slab_h, H,
                               Ly.ffn_norm, PF_NG, P.xp_h, P.xs_h, P.sq_h);
            HIP_TRY(pf_gemv(m, Ly.gu, P.xp_h, P.xs_h, T, P.GU, P.ks_gu, PF_RG_GU, s, P.sq_h));
            hipLaunchKernelGGL(k_swiglu_xp_batch, dim3(gbm_nchunks(I / 32, PF_NG), T), dim3(gbm_chunk_threads(PF_NG)), 0,
                               s, P.GU, P.ks_gu, (size_t)T * 2 * I, I, PF_NG, P.xp_i, P.xs_i);
            HIP_TRY(pf_gemv(m, Ly.down, P.xp_i, P.xs_i, T, P.OD, P.ks_down, PF_RG_DOWN, s));
            // the residual, then the next layer's norm (split for its q|k|v), or
            // the final norm of every position (f32, the last one feeds the LM head)
            if (l + 1 < m->L)
                hipLaunchKernelGGL(k_resid_norm_xp_batch, ngrid, nblock, 0, s, P.X, P.OD, P.ks_down, slab_h, H,
                                   m->layers[l + 1].attn_norm, PF_NG, P.xp_h, P.xs_h, P.sq_h);
            else
                hipLaunchKernelGGL(k_resid_rmsnorm_batch, dim3(T), dim3(SB_THREADS), 0, s, P.X, P.OD, P.ks_down,
                                   slab_h, H, m->final_norm, m->eps, P.HF, nullptr, P.xs_h, PF_NG);
        }
    }
    // the last position: LM head, greedy token as a decode step records it
    HIP_TRY(launch_gemv_plain(m->lm.d, m->lm.qs, P.HF + (size_t)(T - 1) * H, m->logits, m->V, H, s));
    hipLaunchKernelGGL(k_set_state, dim3(1), dim3(64), 0, s, m->st, m->ids, pos0 + n - 1, -1, -1, 0);
    hipLaunchKernelGGL(k_argmax_advance, dim3(1), dim3(256), 0, s, m->logits, P.iota, m->V, m->V, m->st,
                       m->ids, m->pred, m->max_seq);
    HIP_TRY(hipGetLastError());
    m->hw = pos0 + n - 1;
    if (d_logits_last)
        HIP_TRY(hipMemcpyAsync(d_logits_last, m->logits, sizeof(float) * m->V, hipMemcpyDeviceToDevice, s));
    return QD_OK;
}
