/*
 * qd_oracle.h -- plain, slow, f64 CPU oracle of the batch-1 q4_0 decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no source with the HIP
 * library and knows nothing of its layouts, tiles or fusions.
 *
 * What it computes is the plain definition of a dense Qwen3-style decoder
 * step (inferencelayer cuda_llm.rs page, module doc and CudaQwen3::step;
 * ferrum-kernels cuda_decode.rs page, CudaDecodeRunner::decode_step), with
 *   - weights given as q4_0 blocks (value = (code - 8) * d, f16 d),
 *   - K and V stored as binary16 (round to nearest even),
 *   - every other quantity in f64.
 * Threads split output rows only; each row is summed in ascending column
 * order, so results do not depend on the thread count.
 */
#ifndef QD_ORACLE_H
#define QD_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* binary16 bit pattern -> exact f64 value (subnormals, inf and nan included) */
double or_f16_to_f64(uint16_t h);
/* f64 -> binary16 bit pattern, round to nearest, ties to even; overflow -> inf */
uint16_t or_f64_to_f16(double v);
/* OCP fp8 e4m3 (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
 * subnormal; 0x7f / 0xff NaN; no infinity; largest 448): exact decode, and
 * round to nearest even with saturation at +-448 (NaN input -> 0x7f). */
double or_e4m3_to_f64(uint8_t c);
uint8_t or_f64_to_e4m3(double v);

/* q4_0 matrix [rows, cols], row-major: d[rows][cols/32] f16 bits,
 * qs[rows][cols/32][16]: byte j = code of element j (low nibble) and of
 * element j+16 (high nibble). */
typedef struct {
    const uint16_t* d;
    const uint8_t* qs;
    int64_t rows, cols;
} or_q4;

/* out[r*cols + c] = (code(r,c) - 8) * d(r, c/32) */
void or_dequant_q4_0(const or_q4* w, double* out);
/* y[r] = sum_c w(r,c) * x[c], c ascending, f64 */
void or_gemv_q4_0(const or_q4* w, const double* x, double* y, int nthreads);

/* out_i = x_i / sqrt(mean(x^2) + eps) * w_i */
void or_rmsnorm(const double* x, const float* w, int64_t n, double eps, double* out);
/* NeoX split-half rotary on one head of hd values: for i < rot/2 the pair
 * (v_i, v_{i+rot/2}) turns by angle pos * inv_freq[i]; dims >= rot untouched */
void or_rope_neox(double* v, int32_t hd, int32_t rot, const float* inv_freq, int64_t pos);

/* GQA decode attention.  q f32 [B][nq][hd]; K/V f16 bits either paged
 * (block_tables != NULL): pool [num_blocks][nkv][block_size][hd] with
 * block_tables[B][max_blocks_per_seq] mapping logical to physical blocks, or
 * contiguous (block_tables == NULL): [B][nkv][contig_max_kv][hd].  Query head
 * h reads kv head h / (nq/nkv).  out f64 [B][nq][hd];
 * out = softmax(scale * q K^T) V over t in [0, kv_len[b]); kv_len 0 -> zeros.
 * Returns 0, or -1 on bad arguments. */
int or_attn_decode(const float* q, const uint16_t* k, const uint16_t* v,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   int32_t block_size, int32_t contig_max_kv, const int32_t* kv_lens,
                   int32_t B, int32_t nq, int32_t nkv, int32_t hd, double scale,
                   double* out, int nthreads);

typedef struct {
    const float *attn_norm, *ffn_norm, *q_norm, *k_norm; /* [H], [H], [hd], [hd] */
    or_q4 wq, wk, wv, wo, wgate, wup, wdown;
    or_q4 wag;             /* attention output gate [n_heads*hd, H] (attn_out_gate only) */
} or_layer;

typedef struct {
    int32_t hidden, layers, n_heads, n_kv, head_dim, intermediate, vocab;
    int32_t rot_dim;       /* even, <= head_dim */
    int32_t qk_norm;       /* per-head RMSNorm of q and k before the rotary */
    int32_t max_seq;
    int32_t kv_round;      /* 1: K/V stored as binary16 (the method); 0: kept f64;
                              2: stored as fp8 e4m3 of value / k_scale (K) or / v_scale (V) */
    double eps;
    const float* inv_freq; /* [rot_dim/2] */
    double k_scale, v_scale; /* kv_round 2 only */
    int32_t attn_out_gate;   /* 1: attention output *= sigmoid(wag h) before o-proj */
} or_config;

typedef struct or_model or_model;

/* Borrows every pointer (weights must outlive the model); allocates the KV cache. */
or_model* or_model_create(const or_config* cfg, const or_q4* embed, const or_layer* layers,
                          const float* final_norm, const or_q4* lm_head, int nthreads);
/* One decode step: token at position pos; attends over positions [0, pos].
 * logits f64 [vocab]. Returns 0, or -1 on bad token/pos. */
int or_model_step(or_model* m, int32_t token, int32_t pos, double* logits);
/* The K or V the model stored for (layer, pos, kv head), as f64 [hd]. */
int or_model_kv(const or_model* m, int32_t layer, int32_t pos, int32_t kv_head, int32_t which_v,
                double* out);
/* Overwrite the stored K and V of one layer at positions pos0 .. pos0+n-1
 * with k, v [n][n_kv*head_dim] (stored as given; no arithmetic).  For timing
 * steps at a long context without running the steps before it.  0 or -1. */
int or_model_load_kv(or_model* m, int32_t layer, int32_t pos0, int32_t n, const double* k,
                     const double* v);
void or_model_destroy(or_model* m);

#ifdef __cplusplus
}
#endif
#endif
