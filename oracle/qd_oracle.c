/*
 * qd_oracle.c -- plain f64 CPU oracle of the batch-1 q4_0 decode step.
 *
 * TEST INFRASTRUCTURE ONLY (see qd_oracle.h): used by the tests, the smoke
 * check and the benchmark's CPU baseline, never by the product path.
 *
 * Each function is the textbook definition written out, citing the passage
 * of the source pages it follows.  No blocking, fusion, splitting or
 * reordering beyond what the definition states.
 */
#include "qd_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* ------------------------------------------------------------ binary16 */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Subnormal value = fraction * 2^-24; normal = (1024 + fraction) * 2^(e-25). */
static inline double f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

double or_f16_to_f64(uint16_t h)
{
    return f16_value(h);
}

/* Round to the nearest binary16, ties to even.  The value is scaled by a power
 * of two to an integer-quantum grid (exact), rounded with nearbyint (the
 * default rounding mode is round-to-nearest-even), and re-encoded. */
uint16_t or_f64_to_f16(double v)
{
    if (isnan(v))
        return 0x7e00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; a rounded result of 1024 is the
         * smallest normal, whose encoding is also 1024 */
        double m = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)m);
    }
    int ex;
    frexp(a, &ex);             /* a = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;            /* a in [2^E, 2^(E+1)) */
    double m = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        E += 1;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)m - 1024));
}

/* ------------------------------------------------------------ q4_0 */

/* q4_0 (inferencelayer cuda_llm.rs page, Q4Dev: 32-weight blocks, an f16
 * scale and 16 bytes of nibbles; value = (nibble - 8) * d).  Element j of a
 * block is the low nibble of byte j for j < 16 and the high nibble of byte
 * j - 16 otherwise. */
static inline int q4_code(const uint8_t* blockq, int j)
{
    return j < 16 ? (blockq[j] & 0x0f) : (blockq[j - 16] >> 4);
}

void or_dequant_q4_0(const or_q4* w, double* out)
{
    int64_t nb = w->cols / 32;
    for (int64_t r = 0; r < w->rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            double d = f16_value(w->d[r * nb + b]);
            const uint8_t* q = w->qs + (r * nb + b) * 16;
            for (int j = 0; j < 32; j++)
                out[r * w->cols + b * 32 + j] = (double)(q4_code(q, j) - 8) * d;
        }
}

/* y = W x with W dequantised, one dot product per row, columns ascending
 * (inferencelayer cuda_llm.rs page, CudaQwen3::gemv). */
void or_gemv_q4_0(const or_q4* w, const double* x, double* y, int nthreads)
{
    const int64_t nb = w->cols / 32, rows = w->rows;
    const uint16_t* D = w->d;
    const uint8_t* Q = w->qs;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < rows; r++) {
        double acc = 0.0;
        for (int64_t b = 0; b < nb; b++) {
            /* dequantise the block (exact in f64), then accumulate in column order */
            double d = f16_value(D[r * nb + b]);
            const uint8_t* q = Q + (r * nb + b) * 16;
            double wb[32];
            for (int j = 0; j < 32; j++)
                wb[j] = (double)(q4_code(q, j) - 8) * d;
            for (int j = 0; j < 32; j++)
                acc += wb[j] * x[b * 32 + j];
        }
        y[r] = acc;
    }
}

/* ------------------------------------------------------------ norm, rotary */

/* RMSNorm with eps inside the square root (memra-engine qwen4exp_gpu.rs page,
 * host twin host_rms_norm; inferencelayer cuda_llm.rs page, Cfg eps). */
void or_rmsnorm(const double* x, const float* w, int64_t n, double eps, double* out)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; i++)
        ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; i++)
        out[i] = x[i] * inv * (double)w[i];
}

/* NeoX split-half rotary (memra-engine qwen4exp_gpu.rs page, host twin
 * host_rope_at; inferencelayer cuda_llm.rs page, Cfg rot_dim for partial
 * rotary).  The frequencies are an input (host-precomputed inv_freq). */
void or_rope_neox(double* v, int32_t hd, int32_t rot, const float* inv_freq, int64_t pos)
{
    int32_t half = rot / 2;
    (void)hd;
    for (int32_t i = 0; i < half; i++) {
        double th = (double)pos * (double)inv_freq[i];
        double c = cos(th), s = sin(th);
        double a = v[i], b = v[i + half];
        v[i] = a * c - b * s;
        v[i + half] = a * s + b * c;
    }
}

/* ------------------------------------------------------------ attention */

static const uint16_t* kv_row(const uint16_t* base, const int32_t* tables, int32_t mbps,
                              int32_t bs, int32_t cmax, int32_t nkv, int32_t hd, int32_t b,
                              int32_t g, int32_t t)
{
    if (tables) {
        int32_t p = tables[(int64_t)b * mbps + t / bs];
        return base + (((int64_t)p * nkv + g) * bs + t % bs) * hd;
    }
    return base + (((int64_t)b * nkv + g) * cmax + t) * hd;
}

/* Decode attention for one query over its sequence's keys (ferrum-kernels
 * cuda_decode.rs page, attention_paged: logical block t/16, slot t%16 through
 * the block table; scale 1/sqrt(hd)).  Softmax subtracts the row maximum
 * (memra-engine qwen4exp_gpu.rs page, host_softmax). */
int or_attn_decode(const float* q, const uint16_t* k, const uint16_t* v,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   int32_t block_size, int32_t contig_max_kv, const int32_t* kv_lens,
                   int32_t B, int32_t nq, int32_t nkv, int32_t hd, double scale,
                   double* out, int nthreads)
{
    if (B < 0 || nq <= 0 || nkv <= 0 || nq % nkv || hd <= 0)
        return -1;
    if (block_tables && block_size <= 0)
        return -1;
    int32_t grp = nq / nkv;
    int64_t nunits = (int64_t)B * nq;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : bad)
    for (int64_t u = 0; u < nunits; u++) {
        int32_t b = (int32_t)(u / nq), h = (int32_t)(u % nq), g = h / grp;
        int32_t n = kv_lens[b];
        double* o = out + u * hd;
        for (int32_t d = 0; d < hd; d++)
            o[d] = 0.0;
        if (n <= 0)
            continue;
        if (block_tables && (n + block_size - 1) / block_size > max_blocks_per_seq) {
            bad = 1;
            continue;
        }
        if (!block_tables && n > contig_max_kv) {
            bad = 1;
            continue;
        }
        const float* qh = q + u * hd;
        double* s = (double*)malloc(sizeof(double) * (size_t)n);
        double mx = -INFINITY;
        for (int32_t t = 0; t < n; t++) {
            const uint16_t* kr = kv_row(k, block_tables, max_blocks_per_seq, block_size,
                                        contig_max_kv, nkv, hd, b, g, t);
            double dot = 0.0;
            for (int32_t d = 0; d < hd; d++)
                dot += (double)qh[d] * or_f16_to_f64(kr[d]);
            s[t] = dot * scale;
            if (s[t] > mx)
                mx = s[t];
        }
        double l = 0.0;
        for (int32_t t = 0; t < n; t++) {
            s[t] = exp(s[t] - mx);
            l += s[t];
        }
        for (int32_t t = 0; t < n; t++) {
            const uint16_t* vr = kv_row(v, block_tables, max_blocks_per_seq, block_size,
                                        contig_max_kv, nkv, hd, b, g, t);
            double p = s[t] / l;
            for (int32_t d = 0; d < hd; d++)
                o[d] += p * or_f16_to_f64(vr[d]);
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------ decode step */

struct or_model {
    or_config cfg;
    or_q4 embed, lm_head;
    const or_layer* layers;
    const float* final_norm;
    int nthreads;
    double* kc; /* [layers][max_seq][n_kv*hd] */
    double* vc;
    /* scratch */
    double *x, *h, *q, *k, *v, *att, *o, *g, *u, *a, *tmp, *s;
};

or_model* or_model_create(const or_config* cfg, const or_q4* embed, const or_layer* layers,
                          const float* final_norm, const or_q4* lm_head, int nthreads)
{
    const or_config* c = cfg;
    if (c->hidden <= 0 || c->layers <= 0 || c->n_heads <= 0 || c->n_kv <= 0 ||
        c->n_heads % c->n_kv || c->head_dim <= 0 || c->intermediate <= 0 || c->vocab <= 0 ||
        c->rot_dim < 0 || c->rot_dim > c->head_dim || (c->rot_dim & 1) || c->max_seq <= 0 ||
        c->hidden % 32 || c->intermediate % 32 || ((int64_t)c->n_heads * c->head_dim) % 32)
        return NULL;
    int64_t qd0 = (int64_t)c->n_heads * c->head_dim, kv0 = (int64_t)c->n_kv * c->head_dim;
    if (embed->rows != c->vocab || embed->cols != c->hidden || lm_head->rows != c->vocab ||
        lm_head->cols != c->hidden)
        return NULL;
    for (int32_t li = 0; li < c->layers; li++) {
        const or_layer* L = &layers[li];
        if (L->wq.rows != qd0 || L->wq.cols != c->hidden || L->wk.rows != kv0 ||
            L->wk.cols != c->hidden || L->wv.rows != kv0 || L->wv.cols != c->hidden ||
            L->wo.rows != c->hidden || L->wo.cols != qd0 || L->wgate.rows != c->intermediate ||
            L->wgate.cols != c->hidden || L->wup.rows != c->intermediate ||
            L->wup.cols != c->hidden || L->wdown.rows != c->hidden ||
            L->wdown.cols != c->intermediate)
            return NULL;
        if (c->attn_out_gate && (L->wag.rows != qd0 || L->wag.cols != c->hidden || !L->wag.d))
            return NULL;
    }
    or_model* m = (or_model*)calloc(1, sizeof(or_model));
    m->cfg = *c;
    m->embed = *embed;
    m->lm_head = *lm_head;
    m->layers = layers;
    m->final_norm = final_norm;
    m->nthreads = nthreads > 0 ? nthreads : 1;
    int64_t kvd = (int64_t)c->n_kv * c->head_dim;
    size_t kvn = (size_t)c->layers * (size_t)c->max_seq * (size_t)kvd;
    m->kc = (double*)calloc(kvn, sizeof(double));
    m->vc = (double*)calloc(kvn, sizeof(double));
    int64_t qd = (int64_t)c->n_heads * c->head_dim;
    int64_t wide = c->hidden > qd ? c->hidden : qd;
    m->x = (double*)calloc((size_t)c->hidden, sizeof(double));
    m->h = (double*)calloc((size_t)c->hidden, sizeof(double));
    m->q = (double*)calloc((size_t)qd, sizeof(double));
    m->k = (double*)calloc((size_t)kvd, sizeof(double));
    m->v = (double*)calloc((size_t)kvd, sizeof(double));
    m->att = (double*)calloc((size_t)qd, sizeof(double));
    m->o = (double*)calloc((size_t)wide, sizeof(double));
    m->g = (double*)calloc((size_t)c->intermediate, sizeof(double));
    m->u = (double*)calloc((size_t)c->intermediate, sizeof(double));
    m->a = (double*)calloc((size_t)c->intermediate, sizeof(double));
    m->tmp = (double*)calloc((size_t)(c->head_dim > c->hidden ? c->head_dim : c->hidden),
                             sizeof(double));
    m->s = (double*)calloc((size_t)c->max_seq, sizeof(double));
    if (!m->kc || !m->vc || !m->x || !m->s) {
        or_model_destroy(m);
        return NULL;
    }
    return m;
}

void or_model_destroy(or_model* m)
{
    if (!m)
        return;
    free(m->kc); free(m->vc); free(m->x); free(m->h); free(m->q); free(m->k); free(m->v);
    free(m->att); free(m->o); free(m->g); free(m->u); free(m->a); free(m->tmp); free(m->s);
    free(m);
}

double or_e4m3_to_f64(uint8_t c)
{
    const int e = (c >> 3) & 15, mant = c & 7;
    if ((c & 0x7F) == 0x7F)
        return NAN;
    const double mag = e == 0 ? ldexp((double)mant, -9) : ldexp(1.0 + mant / 8.0, e - 7);
    return (c & 0x80) ? -mag : mag;
}

uint8_t or_f64_to_e4m3(double v)
{
    if (isnan(v))
        return 0x7F;
    const uint8_t sgn = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a > 448.0)
        a = 448.0;                                   /* saturate */
    if (a < ldexp(1.0, -6)) {                        /* subnormal: multiples of 2^-9 */
        const int mant = (int)nearbyint(ldexp(a, 9)); /* 0 .. 8; 8 is the smallest normal */
        return (uint8_t)(sgn | mant);
    }
    int e;
    const double f = frexp(a, &e);                   /* a = (2f) * 2^(e-1), 2f in [1, 2) */
    int E = e - 1;
    int mant = (int)nearbyint((2.0 * f - 1.0) * 8.0);
    if (mant == 8) {                                 /* rounded up to the next power of two */
        mant = 0;
        E += 1;
    }
    return (uint8_t)(sgn | ((E + 7) << 3) | mant);
}

static double kv_store(const or_model* m, double val, int which_v)
{
    if (m->cfg.kv_round == 2) {
        const double sc = which_v ? m->cfg.v_scale : m->cfg.k_scale;
        return or_e4m3_to_f64(or_f64_to_e4m3(val / sc)) * sc;
    }
    return m->cfg.kv_round ? or_f16_to_f64(or_f64_to_f16(val)) : val;
}

/* One decode step, in the order of the pages' batch-1 step (inferencelayer
 * cuda_llm.rs page, CudaQwen3::step; ferrum-kernels cuda_decode.rs page,
 * CudaDecodeRunner::decode_step):
 *   x = embedding row of the token;
 *   per layer: h = rms(x); q,k,v = W h; per-head rms of q and k; rotary of q
 *   and k at pos; K/V stored at pos; attention of every q head over positions
 *   0..pos of its kv head; x += Wo attn; h = rms(x); x += Wdown (silu(Wg h) * Wu h);
 *   logits = Wlm rms(x). */
int or_model_step(or_model* m, int32_t token, int32_t pos, double* logits)
{
    const or_config* c = &m->cfg;
    if (token < 0 || token >= c->vocab || pos < 0 || pos >= c->max_seq)
        return -1;
    const int64_t H = c->hidden, hd = c->head_dim, nq = c->n_heads, nkv = c->n_kv;
    const int64_t kvd = nkv * hd, grp = nq / nkv, I = c->intermediate;
    const double scale = 1.0 / sqrt((double)hd);
    const int nt = m->nthreads;

    /* embedding: the token's row of the (q4_0) embedding table */
    {
        int64_t nb = H / 32;
        for (int64_t b = 0; b < nb; b++) {
            double d = or_f16_to_f64(m->embed.d[(int64_t)token * nb + b]);
            const uint8_t* q = m->embed.qs + ((int64_t)token * nb + b) * 16;
            for (int j = 0; j < 32; j++)
                m->x[b * 32 + j] = (double)(q4_code(q, j) - 8) * d;
        }
    }

    for (int32_t li = 0; li < c->layers; li++) {
        const or_layer* L = &m->layers[li];
        double* kc = m->kc + ((int64_t)li * c->max_seq) * kvd;
        double* vc = m->vc + ((int64_t)li * c->max_seq) * kvd;

        or_rmsnorm(m->x, L->attn_norm, H, c->eps, m->h);
        or_gemv_q4_0(&L->wq, m->h, m->q, nt);
        or_gemv_q4_0(&L->wk, m->h, m->k, nt);
        or_gemv_q4_0(&L->wv, m->h, m->v, nt);
        if (c->qk_norm) {
            for (int64_t hh = 0; hh < nq; hh++) {
                or_rmsnorm(m->q + hh * hd, L->q_norm, hd, c->eps, m->tmp);
                memcpy(m->q + hh * hd, m->tmp, sizeof(double) * (size_t)hd);
            }
            for (int64_t gg = 0; gg < nkv; gg++) {
                or_rmsnorm(m->k + gg * hd, L->k_norm, hd, c->eps, m->tmp);
                memcpy(m->k + gg * hd, m->tmp, sizeof(double) * (size_t)hd);
            }
        }
        for (int64_t hh = 0; hh < nq; hh++)
            or_rope_neox(m->q + hh * hd, (int32_t)hd, c->rot_dim, c->inv_freq, pos);
        for (int64_t gg = 0; gg < nkv; gg++)
            or_rope_neox(m->k + gg * hd, (int32_t)hd, c->rot_dim, c->inv_freq, pos);
        for (int64_t i = 0; i < kvd; i++) {
            kc[(int64_t)pos * kvd + i] = kv_store(m, m->k[i], 0);
            vc[(int64_t)pos * kvd + i] = kv_store(m, m->v[i], 1);
        }
        /* attention over positions 0..pos (the new token's K/V included) */
        for (int64_t hh = 0; hh < nq; hh++) {
            int64_t gg = hh / grp;
            const double* qh = m->q + hh * hd;
            double mx = -INFINITY;
            for (int64_t t = 0; t <= pos; t++) {
                const double* kr = kc + t * kvd + gg * hd;
                double dot = 0.0;
                for (int64_t d = 0; d < hd; d++)
                    dot += qh[d] * kr[d];
                m->s[t] = dot * scale;
                if (m->s[t] > mx)
                    mx = m->s[t];
            }
            double l = 0.0;
            for (int64_t t = 0; t <= pos; t++) {
                m->s[t] = exp(m->s[t] - mx);
                l += m->s[t];
            }
            double* oh = m->att + hh * hd;
            for (int64_t d = 0; d < hd; d++)
                oh[d] = 0.0;
            for (int64_t t = 0; t <= pos; t++) {
                const double* vr = vc + t * kvd + gg * hd;
                double p = m->s[t] / l;
                for (int64_t d = 0; d < hd; d++)
                    oh[d] += p * vr[d];
            }
        }
        /* attention output gate (inferencelayer cuda_llm.rs page, Cfg::attn_out_gate:
         * a second projection of the same normed input, sigmoid, elementwise on the
         * attention result before the o-projection) */
        if (c->attn_out_gate) {
            or_gemv_q4_0(&L->wag, m->h, m->o, nt);
            for (int64_t i = 0; i < nq * hd; i++)
                m->att[i] *= 1.0 / (1.0 + exp(-m->o[i]));
        }
        or_gemv_q4_0(&L->wo, m->att, m->o, nt);
        for (int64_t i = 0; i < H; i++)
            m->x[i] += m->o[i];

        or_rmsnorm(m->x, L->ffn_norm, H, c->eps, m->h);
        or_gemv_q4_0(&L->wgate, m->h, m->g, nt);
        or_gemv_q4_0(&L->wup, m->h, m->u, nt);
        for (int64_t i = 0; i < I; i++)
            m->a[i] = m->g[i] / (1.0 + exp(-m->g[i])) * m->u[i];
        or_gemv_q4_0(&L->wdown, m->a, m->o, nt);
        for (int64_t i = 0; i < H; i++)
            m->x[i] += m->o[i];
    }
    or_rmsnorm(m->x, m->final_norm, H, c->eps, m->h);
    or_gemv_q4_0(&m->lm_head, m->h, logits, nt);
    return 0;
}

int or_model_kv(const or_model* m, int32_t layer, int32_t pos, int32_t kv_head, int32_t which_v,
                double* out)
{
    const or_config* c = &m->cfg;
    if (layer < 0 || layer >= c->layers || pos < 0 || pos >= c->max_seq || kv_head < 0 ||
        kv_head >= c->n_kv)
        return -1;
    int64_t kvd = (int64_t)c->n_kv * c->head_dim;
    const double* base = which_v ? m->vc : m->kc;
    memcpy(out, base + ((int64_t)layer * c->max_seq + pos) * kvd + (int64_t)kv_head * c->head_dim,
           sizeof(double) * (size_t)c->head_dim);
    return 0;
}

int or_model_load_kv(or_model* m, int32_t layer, int32_t pos0, int32_t n, const double* k,
                     const double* v)
{
    const or_config* c = &m->cfg;
    if (layer < 0 || layer >= c->layers || pos0 < 0 || n < 0 || (int64_t)pos0 + n > c->max_seq)
        return -1;
    int64_t kvd = (int64_t)c->n_kv * c->head_dim;
    int64_t off = ((int64_t)layer * c->max_seq + pos0) * kvd;
    memcpy(m->kc + off, k, sizeof(double) * (size_t)(n * kvd));
    memcpy(m->vc + off, v, sizeof(double) * (size_t)(n * kvd));
    return 0;
}
