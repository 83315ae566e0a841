/*
 * qd.h -- C ABI of the MI355X (gfx950) batch-1 q4_0 decode library.
 *
 * The library computes the batch-1 greedy decode step of a dense Qwen3-style
 * decoder whose matrices are q4_0 (inferencelayer cuda_llm.rs page, module
 * doc and CudaQwen3::step; ferrum-kernels cuda_decode.rs page,
 * CudaDecodeRunner::decode_step), and exposes its two hot kernels on their
 * own: the q4_0 GEMV and the GQA decode attention.
 *
 * Conventions for every entry point:
 *   - return QD_OK (0) or a negative QD_E* code; qd_last_error() then returns
 *     a message (thread-local, valid until the next call on that thread);
 *   - arguments are validated before any HIP call: on a validation error
 *     nothing is enqueued and nothing is allocated;
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream);
 *     work is enqueued asynchronously on it unless stated otherwise;
 *   - "host" pointers are read during the call only; "device" pointers must
 *     stay valid until the enqueued work has finished;
 *   - no C++ exception crosses this interface.
 */
#ifndef QD_H
#define QD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QD_OK 0
#define QD_EINVAL (-1)       /* null pointer, bad shape or inconsistent config */
#define QD_ERANGE (-2)       /* token or position out of range */
#define QD_ENOMEM (-3)       /* device allocation failed */
#define QD_EUNSUPPORTED (-4) /* valid but not built: head_dim, GQA group, block size */
#define QD_EHIP (-5)         /* HIP runtime error (message has hipGetErrorString) */

typedef void* qd_stream; /* hipStream_t */

/* ------------------------------------------------------------------ q4_0
 * A q4_0 matrix [rows, cols], row-major, in blocks of 32 weights along a row
 * (inferencelayer cuda_llm.rs page, Q4Dev and LayerDev: one f16 scale and 16
 * bytes of nibbles per 32 weights; value = (nibble - 8) * scale):
 *   d  [rows][cols/32]      binary16 bit patterns of the block scales
 *   qs [rows][cols/32][16]  byte j of a block: element j in the low nibble,
 *                           element j+16 in the high nibble
 * cols must be a multiple of 32.                                           */
typedef struct {
    const uint16_t* d;
    const uint8_t* qs;
    int32_t rows, cols;
} qd_q4_0;

/* One decoder layer, host memory.  Norm vectors are f32: attn_norm and
 * ffn_norm [hidden], q_norm and k_norm [head_dim] (ignored when qk_norm = 0).
 * wq [n_heads*head_dim, hidden], wk and wv [n_kv*head_dim, hidden],
 * wo [hidden, n_heads*head_dim], wgate and wup [intermediate, hidden],
 * wdown [hidden, intermediate]. */
typedef struct {
    const float *attn_norm, *ffn_norm, *q_norm, *k_norm;
    qd_q4_0 wq, wk, wv, wo, wgate, wup, wdown;
    qd_q4_0 attn_gate;   /* [n_heads*head_dim, hidden], read only with attn_out_gate */
} qd_layer_weights;

/* embed [vocab, hidden] q4_0: a token's embedding is its dequantised row.
 * lm_head [vocab, hidden] q4_0, ignored when the config says tied (the
 * embedding table is then the head).  final_norm f32 [hidden].
 * layers: [config.layers]. */
typedef struct {
    qd_q4_0 embed;
    qd_q4_0 lm_head;
    const float* final_norm;
    const qd_layer_weights* layers;
} qd_weights;

/* Model configuration (inferencelayer cuda_llm.rs page, Cfg).
 *   rot_dim: even, <= head_dim; the first rot_dim dims of every q and k head
 *            turn NeoX split-half style (pairs i, i + rot_dim/2); the rest
 *            pass through (partial rotary).
 *   inv_freq: host f32 [rot_dim/2], the host-precomputed rotary frequencies
 *            (Cfg::rope_inv_freq); angle of pair i at position p = p*inv_freq[i].
 *   qk_norm: 1 = per-head RMSNorm of q and k (over head_dim) before rotary.
 *   max_seq: positions 0 .. max_seq-1 exist in the KV cache.
 *   kv_paged: 0 = contiguous f16 KV cache; 1 = paged (ferrum-kernels
 *            cuda_decode.rs page, PagedSequenceKvState / attention_paged):
 *            a pool of num_kv_blocks blocks of kv_block_size tokens per layer,
 *            and block_table [ceil(max_seq/kv_block_size)] (host, int32) mapping
 *            logical block -> physical block (distinct entries in
 *            [0, num_kv_blocks)); NULL = identity.  The whole table is fixed
 *            at create time, so a captured step never needs a table update.
 *   use_graph: 1 = one decode step is captured in a hipGraph at create time
 *            and replayed; 0 = the step's kernels are launched one by one.
 *   layer_kernel: 0 = five kernels per layer (every model above);
 *            1 = one persistent kernel launch per layer, one workgroup per
 *            CU, device-wide barriers between the layer's phases.  It needs
 *            head_dim 128, n_heads = 4 n_kv, hidden, intermediate and
 *            n_heads*head_dim multiples of 2048 (at most 14 144), and a
 *            device that keeps one 512-thread workgroup per CU resident;
 *            QD_EUNSUPPORTED otherwise.  Same results up to f32 rounding
 *            order (the RMSNorm partial sums are grouped differently).
 *   kv_fp8:  0 = f16 K/V cache; 1 = fp8 e4m3 cache (OCP e4m3, 1 byte per
 *            element): the step stores e4m3(k / k_scale) and e4m3(v /
 *            v_scale), rounded to nearest even and saturated at +-448, and the
 *            attention reads value * scale (as qd_attn_decode_kv8).  k_scale
 *            and v_scale finite and positive; not with layer_kernel = 1
 *            (QD_EUNSUPPORTED).  Fields past layer_kernel: a caller that
 *            zero-fills the struct gets the f16 cache.
 *   attn_out_gate: 1 = attention output gate (inferencelayer cuda_llm.rs
 *            page, Cfg::attn_out_gate): each layer's attn_gate rows project
 *            the same normed input as q|k|v (fused after them), and the
 *            attention result is multiplied elementwise by their sigmoid
 *            before the o-projection.  Not with layer_kernel = 1
 *            (QD_EUNSUPPORTED).
 * Supported: head_dim 64 or 128; n_heads / n_kv in {1, 2, 4, 8};
 * kv_block_size 16; hidden, intermediate and n_heads*head_dim multiples of 32. */
typedef struct {
    int32_t hidden, layers, n_heads, n_kv, head_dim, intermediate, vocab;
    float eps;
    int32_t rot_dim;
    const float* inv_freq;
    int32_t tied;
    int32_t qk_norm;
    int32_t max_seq;
    int32_t kv_paged, kv_block_size, num_kv_blocks;
    const int32_t* block_table;
    int32_t use_graph;
    int32_t layer_kernel;
    int32_t kv_fp8;
    float k_scale, v_scale;
    int32_t attn_out_gate;
} qd_config;

typedef struct qd_model qd_model;

/* Create a model on the current HIP device.  Copies every host array it is
 * given (weights, inv_freq, block_table) into library-owned device memory
 * (the layout there is the library's own); the caller's buffers may be freed
 * on return.  Synchronous.  *out receives the handle. */
int qd_create(const qd_config* cfg, const qd_weights* w, qd_stream stream, qd_model** out);

/* Free all device memory of the model (after synchronising its work). */
int qd_destroy(qd_model* m);

/* One decode step (inferencelayer cuda_llm.rs page, CudaQwen3::step): embed
 * `token` at position `pos`, write its K/V at `pos`, attend over positions
 * 0..pos, produce f32 logits [vocab].  Positions 0..pos-1 must have been
 * written by earlier steps (prefill is sequential decode): the library keeps
 * the written prefix on the host (none after qd_create; a step at p makes
 * it 0..p, so a step may also go back and rewrite) and refuses a pos more
 * than one past it with QD_ERANGE, as for a token outside [0, vocab) or a pos
 * outside [0, max_seq).  d_logits (device f32 [vocab]) and d_next (device
 * int32, greedy argmax, lowest index on ties) may each be NULL.  Asynchronous
 * on `stream`. */
int qd_decode_step(qd_model* m, int32_t token, int32_t pos, float* d_logits, int32_t* d_next,
                   qd_stream stream);

/* Greedy generation driven on the device (inferencelayer cuda_llm.rs page,
 * CudaQwen3::seed / capture / run_graph / tokens): the model keeps a token
 * per position.  qd_set_prompt stores host tokens [n] at positions 0..n-1
 * and marks them forced.  qd_generate runs n_steps steps at positions
 * pos0 .. pos0+n_steps-1 with no host synchronisation: the step at p reads
 * the token stored at p and computes the argmax of its logits; if p+1 is not
 * a forced position that argmax becomes the token at p+1.  d_tokens (device
 * int32 [n_steps] or NULL) receives the argmax of every step; d_logits_last
 * (device f32 [vocab] or NULL) the logits of the last step.  Prompt prefill
 * plus G greedy tokens is qd_set_prompt(prompt, P) then
 * qd_generate(0, P+G-1, ...): entries P-1 .. P+G-2 of d_tokens are the
 * greedy tokens.  Requires pos0 + n_steps <= max_seq and, for n_steps > 0,
 * pos0 at most one past the written prefix (QD_ERANGE otherwise); afterwards
 * the prefix is 0 .. pos0+n_steps-1. */
int qd_set_prompt(qd_model* m, const int32_t* tokens, int32_t n, qd_stream stream);
int qd_generate(qd_model* m, int32_t pos0, int32_t n_steps, int32_t* d_tokens,
                float* d_logits_last, qd_stream stream);

/* Chunked prompt prefill (inferencelayer cuda_llm.rs page: prefill as the
 * many-token form of the decode step, its q4 GEMV arm at M > 1): runs the
 * positions pos0 .. pos0+n-1 in chunks of up to qd_prefill_chunk() (64),
 * each chunk one batched product per matrix (every weight read once per
 * chunk), with the tokens
 * stored by qd_set_prompt (or an earlier step).  It writes the K/V cache of
 * every position as n decode steps would, and at the last position p =
 * pos0+n-1 it records what a decode step at p records: the argmax of its
 * logits as the prediction at p and, if p+1 is not forced, the token at
 * p+1.  d_logits_last (device f32 [vocab] or NULL) receives the logits at p.
 * Each position's values equal the decode step's up to f32 rounding order.
 * Continue with qd_generate(pos0 + n, ...).  Buffers (about 64 positions of
 * activations plus an attention workspace) are allocated by the first call,
 * which synchronises; later calls allocate nothing.  The matrix products
 * are those of the batched decode step with the chunk's positions as its
 * vectors: each position's activations enter as an f16 pair (hi + lo, about
 * 22 significant bits) after scaling each 256-element chunk of the position's
 * vector by a power of two that puts its largest magnitude in [2^13, 2^14),
 * undone exactly in f32, so any finite activation scale is handled; the block
 * scales d and each position's 1/rms are applied in f32.  A model with attn_out_gate gates each
 * position's attention output as the decode step does.  hidden <= 16384
 * (QD_EUNSUPPORTED otherwise).  QD_ERANGE unless 0 <= pos0, n >= 1,
 * pos0 + n <= max_seq and pos0 is at most one past the written prefix;
 * afterwards the prefix is 0 .. pos0+n-1. */
int qd_prefill(qd_model* m, int32_t pos0, int32_t n, float* d_logits_last, qd_stream stream);
/* Prompt positions per qd_prefill chunk (every weight is read once per
 * chunk); a constant of the library build.  Host only. */
int32_t qd_prefill_chunk(void);

/* Batched decode (inferencelayer cuda_llm.rs page, step_batch_inner and its
 * batched head-to-head of the q4 GEMV arm at M = 2 .. 16 tokens;
 * ferrum-kernels cuda_decode.rs page, batched_decode_attention): a model of
 * `batch` sequences (2 .. 16) stepped together, every weight read once per
 * step for all of them.  Each sequence has its own tokens, position, written
 * prefix, greedy predictions and K/V cache: contiguous (batch copies of
 * max_seq positions) or paged, where cfg->block_table (NULL = identity) holds
 * batch tables of ceil(max_seq/16) entries, sequence b's at
 * [b * ceil(max_seq/16)], all distinct and below num_kv_blocks.  Each
 * sequence's step computes what qd_decode_step computes for it (up to f32
 * rounding order: the RMSNorm is applied to the activations before the
 * batched GEMV instead of after it).  Not with layer_kernel or attn_out_gate,
 * and hidden <= 16384 (QD_EUNSUPPORTED otherwise).
 * The one-sequence entry points (qd_decode_step, qd_set_prompt, qd_generate,
 * qd_prefill) refuse a batched model and the batch entry points below refuse
 * a one-sequence model (QD_EINVAL).  Synchronous; *out receives the handle. */
int qd_create_batch(const qd_config* cfg, const qd_weights* w, int32_t batch, qd_stream stream,
                    qd_model** out);

/* qd_set_prompt for sequence `seq` of a batched model (host tokens [n] at
 * positions 0 .. n-1, marked forced). */
int qd_set_prompt_seq(qd_model* m, int32_t seq, const int32_t* tokens, int32_t n, qd_stream stream);

/* qd_generate for all sequences of a batched model at once: sequence b runs
 * positions pos0[b] .. pos0[b]+n_steps-1 (pos0: host int32 [batch]), each
 * start at most one past that sequence's written prefix, with no host
 * synchronisation.  d_tokens (device int32 [batch][n_steps] or NULL) receives
 * every step's argmax per sequence; d_logits_last (device f32 [batch][vocab]
 * or NULL) the logits of the last step.  QD_ERANGE for a position out of
 * range, nothing enqueued. */
int qd_generate_batch(qd_model* m, const int32_t* pos0, int32_t n_steps, int32_t* d_tokens,
                      float* d_logits_last, qd_stream stream);

/* qd_decode_step for all sequences of a batched model: sequence b embeds
 * tokens[b] at position pos[b] (host int32 [batch] each).  d_logits (device
 * f32 [batch][vocab]) and d_next (device int32 [batch]) may be NULL. */
int qd_decode_step_batch(qd_model* m, const int32_t* tokens, const int32_t* pos, float* d_logits,
                         int32_t* d_next, qd_stream stream);

/* Standalone q4_0 GEMV (inferencelayer cuda_llm.rs page, CudaQwen3::gemv):
 * y[N] = W[N, K] x[K], W in the q4_0 layout above (device d_scales
 * [N][K/32], d_qs [N][K/32][16]), x and y device f32.  K % 32 == 0; qs and x
 * 16-byte aligned.  Supported: K up to 14 144 (x is staged in LDS), N < 2^24,
 * N*K/2 < 2^32 (QD_EUNSUPPORTED otherwise).  No allocation; capturable. */
int qd_gemv_q4_0(const uint16_t* d_scales, const uint8_t* d_qs, const float* d_x, float* d_y,
                 int32_t N, int32_t K, qd_stream stream);

/* Batched q4_0 GEMV (inferencelayer cuda_llm.rs page, the batched decode
 * head-to-head of its q4 GEMV arm at M = 1 .. 16 tokens): Y[b] = W X[b] for
 * b < B, every weight read once for the whole batch.  W as for qd_gemv_q4_0;
 * d_x device f32 [B][K] and d_y device f32 [B][N], both contiguous; qs and x
 * 16-byte aligned.  1 <= B <= 16; B == 1 runs the single-vector kernel,
 * 2 <= B <= 5 a vector kernel that stages the whole batch in LDS when
 * B*K <= 32 768, otherwise (and always for B >= 6) the matrix cores: any K,
 * one product per q4_0 block with the codes as exact f16 values and the
 * block's scale applied to the product in f32, and x as an f16 pair (about
 * 22 significant bits) after a power-of-two scaling per vector and
 * 1024-element chunk, undone exactly in f32, so any finite input scale is
 * handled.  N < 2^24, N*K/2 < 2^32.
 * QD_EINVAL / QD_EUNSUPPORTED otherwise, with nothing enqueued.  The
 * summation order differs from the single-vector GEMV.  No allocation;
 * capturable. */
int qd_gemv_q4_0_batch(const uint16_t* d_scales, const uint8_t* d_qs, const float* d_x, float* d_y,
                       int32_t N, int32_t K, int32_t B, qd_stream stream);

/* Expert GEMV for mixture-of-experts decode (inferencelayer cuda_llm.rs page,
 * its MoE expert matrices): y[j] = W[experts[j]] x for j < k.  W is a stack
 * of n_experts q4_0 matrices [N, K] (d_scales [n_experts][N][K/32], d_qs
 * [n_experts][N][K/32][16], device); d_experts device int32 [k], the indices
 * a router picked (not read by the host); d_x device f32 [K]; d_y device f32
 * [k][N].  Each selected matrix is read once per call (an expert picked twice
 * is read twice).  An index outside [0, n_experts) gives a NaN row and reads
 * nothing.  K % 32 == 0, qs and x 16-byte aligned, K up to 14 144, N < 2^24,
 * N*K/2 < 2^32 per expert, k <= 65535 and N*k < 2^31 (QD_EINVAL /
 * QD_EUNSUPPORTED otherwise).  Routing itself is the caller's.  No
 * allocation; capturable. */
int qd_gemv_q4_0_experts(const uint16_t* d_scales, const uint8_t* d_qs, const int32_t* d_experts,
                         int32_t n_experts, int32_t k, const float* d_x, float* d_y, int32_t N,
                         int32_t K, qd_stream stream);

/* Rotary frequencies for qd_config.inv_freq (host only, no device work):
 * out[i] = theta^(-2i/rot_dim) for i < rot_dim/2, evaluated in f64 and rounded
 * to f32, with the rotary scaling of the inferencelayer cuda_llm.rs page
 * (Cfg::rope_inv_freq): QD_ROPE_DEFAULT none; QD_ROPE_LINEAR every frequency
 * divided by `factor`; QD_ROPE_LLAMA3 with wavelength wl = 2*pi/f: wl above
 * original_max_pos/low_freq_factor -> f/factor, wl below
 * original_max_pos/high_freq_factor -> f, between them (1-s)*f/factor + s*f
 * with s = (original_max_pos/wl - low_freq_factor) / (high_freq_factor -
 * low_freq_factor).  The last three arguments are read for LLAMA3 only.
 * `out` is a host float array [rot_dim/2] owned by the caller.  Errors:
 * QD_EINVAL (null out, odd or non-positive rot_dim, theta <= 1, factor <= 0,
 * llama3 factors out of order), QD_EUNSUPPORTED (any other scaling type:
 * refused, never ignored). */
enum { QD_ROPE_DEFAULT = 0, QD_ROPE_LINEAR = 1, QD_ROPE_LLAMA3 = 2 };
int qd_rope_inv_freq(float theta, int32_t rot_dim, int32_t scaling, float factor,
                     float low_freq_factor, float high_freq_factor, float original_max_pos,
                     float* out);

/* Standalone GQA decode attention with split-KV partials and an
 * online-softmax combine (inferencelayer cuda_llm.rs page, attn_partial /
 * attn_reduce and the flash-decoding arm; ferrum-kernels cuda_decode.rs page,
 * flash_decode_attention, paged_decode_attention, batched_decode_attention).
 *   q        device f32 [B][nq][head_dim]
 *   k, v     device f16 bits.  Paged (block_tables != NULL): pools
 *            [num_blocks][nkv][block_size][head_dim]; block_tables device
 *            int32 [B][max_blocks_per_seq], logical block -> physical block.
 *            Contiguous (block_tables == NULL): [B][nkv][max_kv_len][head_dim].
 *   kv_lens  device int32 [B]; each in [0, max_kv_len]; 0 -> output zeros
 *   max_kv_len host bound on kv_lens (sizes the grid)
 *   scale    softmax scale (usually 1/sqrt(head_dim))
 *   out      device f32 [B][nq][head_dim]
 * Query head h reads kv head h / (nq/nkv).  Supported: head_dim 64 or 128,
 * nq/nkv in {1, 2, 4, 8}, block_size 16. */
typedef struct {
    const float* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    int32_t block_size;
    const int32_t* kv_lens;
    int32_t max_kv_len;
    int32_t B, nq, nkv, head_dim;
    float scale;
    float* out;
} qd_attn_args;

/* Bytes of device workspace qd_attn_decode needs for these sizes (the
 * split-KV partials); no initialisation is needed.  A workspace must not be
 * shared by two calls in flight at the same time. */
size_t qd_attn_workspace_bytes(int32_t B, int32_t nq, int32_t nkv, int32_t head_dim,
                               int32_t max_kv_len);
int qd_attn_decode(const qd_attn_args* a, void* d_workspace, size_t workspace_bytes,
                   qd_stream stream);

/* The same attention over an fp8 KV cache (reduced-precision KV, the
 * inferencelayer cuda_llm.rs page's KV-format discussion; OCP e4m3, 1 byte
 * per element): a->k and a->v point at e4m3 bytes in the layouts above
 * (element counts unchanged), 16-byte aligned; element value = e4m3 value *
 * k_scale (K) or * v_scale (V), both finite and positive.  Arithmetic as
 * qd_attn_decode (f16 matrix-core QK with q as an f16 hi + lo pair, f32
 * softmax and PV).  Workspace as qd_attn_workspace_bytes.  Same errors;
 * QD_EINVAL also for a bad scale or alignment.  No allocation; capturable. */
int qd_attn_decode_kv8(const qd_attn_args* a, float k_scale, float v_scale, void* d_workspace,
                       size_t workspace_bytes, qd_stream stream);

/* The attention of qd_attn_decode without a workspace argument and without
 * any allocation, for callers that cannot allocate (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * split-KV partials live in a library scratch array of
 * qd_attn_noalloc_max_bytes() bytes (8 MiB) in each GPU's memory, kept until
 * the process ends.  Arguments and results as qd_attn_decode (f16 K/V);
 * sizes whose partials exceed the scratch
 * (qd_attn_workspace_bytes(B, nq, nkv, head_dim, max_kv_len) > the maximum)
 * are refused with QD_EUNSUPPORTED, nothing enqueued.  Every call on one GPU
 * uses that GPU's one scratch array: calls that overlap on a GPU (two
 * streams, or two threads) race and must be serialised by the caller.  The
 * scratch needs no initialisation (every partial read was written by the same
 * call).  No allocation; capturable. */
size_t qd_attn_noalloc_max_bytes(void);
int qd_attn_decode_noalloc(const qd_attn_args* a, qd_stream stream);

/* Synchronises `stream` and reports what the device recorded since the last
 * check, then clears it: QD_ERANGE if a step saw a token or a position out of
 * range (a stored token or position the host did not validate), QD_EHIP if a
 * device-wide barrier of the layer kernel (layer_kernel = 1) gave up waiting,
 * in which case the steps since the last check are invalid; QD_OK otherwise.
 * Blocks the host; not capturable. */
int qd_check(qd_model* m, qd_stream stream);

/* Measurement utility, not a step of the decode path: the plain streaming
 * read that the GEMV's bandwidth is compared with (its measured ceiling on
 * the same part).  Reads d_src[0, bytes) once with 128-bit non-temporal
 * loads; workgroup w writes the XOR of the 32-bit words it read to
 * d_sink[w], so the XOR of all qd_stream_read_groups(bytes) sink words is the
 * XOR of every word of the buffer.  bytes a positive multiple of 16, d_src
 * 16-byte aligned (QD_EINVAL otherwise); d_sink holds
 * qd_stream_read_groups(bytes) words (0 for an invalid size).  No
 * allocation; capturable. */
size_t qd_stream_read_groups(size_t bytes);
int qd_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink, qd_stream stream);

/* Message of the last failed call on this thread ("" if none). */
const char* qd_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* QD_H */
