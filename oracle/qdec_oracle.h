/*
 * CPU oracle for the batch-1 quantized GQA decode step.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark may load or call this code.  The GPU library never links it, and it
 * shares no header, kernel, helper or table with the GPU library.
 *
 * Every function computes the plain definition of its step: fp64 accumulation for
 * dot products, sums of squares and softmax, fp32 storage between steps, and bf16
 * rounding (round to nearest even) only where the KV cache stores bf16.
 */
#ifndef QDEC_ORACLE_H
#define QDEC_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_W_Q8 = 1, ORC_W_Q4 = 2 };
enum { ORC_KV_F32 = 1, ORC_KV_BF16 = 2 };

/* number formats */
float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float f);
float orc_bf16_to_f32(uint16_t b);

/* one weight row dequantised to fp32 */
void orc_dequant_row(int fmt, const void *W, const void *S, int group, int64_t row, int K, float *w);

/* y[n] = fp32( sum_k w[n][k] x[k]  (+ bias[n]) (+ residual[n]) ), sum in fp64 */
void orc_gemv(int fmt, const void *W, const void *S, int group, const float *x, const float *bias,
              const float *residual, float *y, int N, int K, int nthreads);

/* INT8 activations: q[k] in [-127, 127], one binary32 scale per group of `group` k */
void orc_quantize_act_i8(const float *x, int K, int group, int8_t *q, float *sx);
/* y[n] = fp32( sum_g wscale * sx[g] * sum_{k in g} level[n][k] q[k]  (+ bias) (+ residual) ) */
void orc_gemv_a8(int fmt, const void *W, const void *S, int group, const int8_t *q, const float *sx,
                 const float *bias, const float *residual, float *y, int N, int K, int nthreads);

/* per row of `dim`: y = gamma * x / sqrt(mean(x^2) + eps)  (gamma may be NULL: all ones) */
void orc_rmsnorm(const float *x, const float *gamma, float *y, int rows, int dim, double eps);

/* in place, per row of `dim`: rotate pairs (i, i + dim/2) by pos * base^(-2i/dim) */
void orc_rope(float *x, int rows, int dim, int pos, double base);

/* m[i] = silu(g[i]) * u[i], silu(z) = z / (1 + exp(-z)) */
void orc_swiglu(const float *g, const float *u, float *m, int n);

/* store one token's [n_kv_heads][head_dim] fp32 values into the paged pool */
void orc_kv_store(void *pool, int kv_fmt, const int32_t *page_table, int page_size, int n_kv_heads,
                  int head_dim, int t, const float *kv);
float orc_kv_load(const void *pool, int kv_fmt, const int32_t *page_table, int page_size,
                  int n_kv_heads, int head_dim, int t, int j, int d);

/* out[h][:] = softmax_t(q_h . k_{j,t} * scale) v_{j,t}, t in [0, T), j = h / (Hq / Hkv) */
void orc_attention(const float *q, const void *k_pool, const void *v_pool, int kv_fmt,
                   const int32_t *page_table, int page_size, int T, int Hq, int Hkv, int D,
                   double scale, float *out, float *probs /* [Hq][T] or NULL */);

/* smallest index among the maxima */
int orc_argmax(const float *v, int n);

/* Philox4x64-10; the uniform (0, 1) draw of token i at a step; temperature / top-k / top-p
   sampling with a Gumbel-max draw (greedy when temperature <= 0) */
void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);
double orc_sample_uniform(uint64_t seed, int64_t step, int64_t i);
int orc_sample(const float *logits, int V, double temperature, int top_k, double top_p, uint64_t seed,
               int64_t step);

typedef struct {
  int n_layers, hidden, n_heads, n_kv_heads, head_dim, inter, vocab;
  int wfmt, group, kv_fmt, page_size;
  int has_bias, has_qk_norm, has_embedding, has_lm_head;
  double eps, rope_base;
} orc_config;

typedef struct {
  const void *wq, *sq, *wk, *sk, *wv, *sv, *wo, *so, *wg, *sg, *wu, *su, *wd, *sd;
  const float *bq, *bk, *bv;
  const float *g_attn, *g_ffn, *g_q, *g_k;
  void *k_pool, *v_pool;
} orc_layer;

typedef struct {
  const uint16_t *embed; /* bf16 [V][H] */
  const float *g_out;
  const void *w_lm, *s_lm;
} orc_head;

/*
 * One decode step at position `pos` (0-based; keys 0..pos are attended).
 * h: in/out [H] residual stream; with has_embedding it is overwritten by the
 * embedding row of `token` first.  KV pools are updated at `pos`.
 * trace: optional [L + 1][H], h after the embedding and after each layer.
 * logits: optional [V].  Returns the greedy token (or -1 without an lm_head).
 */
int orc_decode_step(const orc_config *cfg, const orc_layer *layers, const orc_head *head,
                    const int32_t *page_table, int pos, int token, float *h, float *trace,
                    float *logits, int nthreads);

/*
 * The same step with the new token's cache entries exposed, for comparisons in which the
 * rounding of a stored value is a tie (both neighbouring codes are correct roundings within
 * fp32 accumulation error):
 *   kv_pre: optional out [L][2][Hkv * D], the fp32 k (after q/k norm and RoPE) and v of the new
 *           token at each layer, before they are rounded into the cache;
 *   kv_force, force_mask: optional (bf16 pools only): for every layer l with force_mask[l] != 0
 *           the new token's entries are stored as the given codes kv_force[l][0] (k) and
 *           kv_force[l][1] (v), [Hkv * D] each, instead of the rounding of kv_pre; the layer
 *           then attends over the cache as always.  Everything else is unchanged.
 */
int orc_decode_step_kv(const orc_config *cfg, const orc_layer *layers, const orc_head *head,
                       const int32_t *page_table, int pos, int token, float *h, float *trace,
                       float *logits, int nthreads, float *kv_pre, const uint16_t *kv_force,
                       const uint8_t *force_mask);

/* Batched decode: the single-sequence step for every slot b with pos[b] >= 0, with block table
   row b ([B][max_blocks]), token tokens[b] and residual stream h[b] ([B][H]); logits [B][V] or
   NULL; next[b] gets the greedy token (idle slots untouched). */
void orc_decode_batch(const orc_config *c, const orc_layer *layers, const orc_head *head, int B,
                      const int32_t *block_tables, int max_blocks, const int32_t *pos, const int32_t *tokens,
                      float *h, float *logits, int32_t *next, int nthreads);

/* Prefill: the single-token step for tokens[t] at position pos0 + t, t = 0 .. T-1, in order;
   h and logits (optional) are the last position's; returns its greedy token. */
int orc_prefill(const orc_config *c, const orc_layer *layers, const orc_head *head, const int32_t *page_table,
                int pos0, const int32_t *tokens, int T, float *h, float *logits, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
