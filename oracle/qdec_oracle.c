/*
 * CPU oracle for the batch-1 quantized GQA decode step (plain definitions, fp64).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark load this library.  It shares no code, header or table with the GPU
 * library; it reads the packed weight and KV layouts from their written description.
 *
 * Sources (page title, then section):
 *  [RT]  "How To Construct Your Personal LLM Runtime From Scratch" (newsaiworld post on the
 *        annotated H100 runtime): section 3 (dims, GQA 28:4, 16-token KV pages),
 *        section 6 (region order qkv_gemv -> append_tail_kv -> paged_attention -> o_proj ->
 *        gate_up_gemv -> swiglu_down), section 7 (per-weight INT4 decode contract).
 *  [H100] "Bare-Metal LLM Inference on NVIDIA H100 ..." (whatvis): "Architectural Blueprint"
 *        (group-wise INT4 with one fp16 scale per group per output row; GQA 7:1).
 *  [FQ]  FlashQwen README: "Local benchmark" (INT8 per-row weights, fp32 activations, bf16 KV),
 *        "Optimization study" stages 5 (greedy argmax), 7 (split-K decode attention),
 *        8 (INT8 per-output-row dequant in the GEMV).
 *  [PA]  "Chapter 2 Systems Foundations for LLMs": "PagedAttention - Virtual Memory for KV
 *        Caches" (page table from logical token block to physical block).
 *  [H100] also "Challenge 3" (Path A: INT8 activations with a per-group scale and dp4a).
 *  [NQ]  "Naive CUDA Kernel Qwen engine, part 1" (eduardoqian): sections RMSNorm, Rope,
 *        SwiGLU, Sampler; the GGUF tensor list of a Qwen2 block.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - INT4 codes: byte j of a row holds k = 2j in bits 0-3 and k = 2j+1 in bits 4-7; the code
 *    is unsigned with zero point 8, so the integer level is nibble - 8 in [-8, 7].
 *  - RoPE: theta_i = base^(-2i/D), pairs (i, i + D/2) ("rotate half"), angles in fp64.
 *  - Attention scale 1/sqrt(D), causal over every cached token plus the current one.
 *  - SwiGLU: SiLU (beta = 1) on the gate projection, the up projection linear.
 *  - Residual wiring: pre-norm, h += o_proj(attn(...)), h += down(swiglu(...)).
 *  - Greedy tie-break: smallest index.
 *  - INT8 activations: symmetric per group, s = max|x|/127, round half to even in binary32.
 *  - Sampling: temperature, then top-k, then top-p, then a Gumbel-max draw keyed by Philox.
 */
#include "qdec_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- number formats */

/* IEEE binary16 -> binary32 by fields; every binary16 value is exact in binary32. */
float orc_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1Fu;
  uint32_t m = h & 0x3FFu;
  uint32_t bits;
  float f;
  if (e == 0) {
    /* zero or subnormal: m * 2^-24 */
    f = (float)m * 5.9604644775390625e-08f;
    return sign ? -f : f;
  }
  if (e == 31)
    bits = sign | 0x7F800000u | (m << 13); /* inf / nan */
  else
    bits = sign | ((e + 112u) << 23) | (m << 13); /* rebias 15 -> 127 */
  memcpy(&f, &bits, 4);
  return f;
}

/* binary32 -> bf16 (upper 16 bits) rounded to nearest, ties to even. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x7FFFFFu)) return (uint16_t)((b >> 16) | 0x40u);
  uint32_t lsb = (b >> 16) & 1u;
  b += 0x7FFFu + lsb;
  return (uint16_t)(b >> 16);
}

float orc_bf16_to_f32(uint16_t v) {
  uint32_t b = (uint32_t)v << 16;
  float f;
  memcpy(&f, &b, 4);
  return f;
}

/* ---------------------------------------------------------------- dequantisation */

/*
 * INT8 per output row [FQ stage 8]: w = fp32(q) * s[row], one fp32 multiply.
 * INT4 [RT section 7; H100 "Architectural Blueprint"]: level = nibble - 8 (zero point 8),
 * times the fp16 scale of its group of `group` consecutive k in the row.  The product of a
 * 4-bit level and an 11-bit fp16 significand is exact in fp32.
 */
void orc_dequant_row(int fmt, const void *W, const void *S, int group, int64_t row, int K, float *w) {
  if (fmt == ORC_W_Q8) {
    const int8_t *q = (const int8_t *)W + row * (int64_t)K;
    float s = ((const float *)S)[row];
    for (int k = 0; k < K; ++k) w[k] = (float)q[k] * s;
  } else {
    const uint8_t *b = (const uint8_t *)W + row * (int64_t)(K / 2);
    const uint16_t *sc = (const uint16_t *)S + row * (int64_t)(K / group);
    for (int g = 0; g < K / group; ++g) {
      float s = orc_f16_to_f32(sc[g]); /* the scale of k in [g*group, (g+1)*group) */
      for (int k = g * group; k < (g + 1) * group; ++k) {
        uint8_t byte = b[k / 2];
        int nib = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
        w[k] = (float)(nib - 8) * s;
      }
    }
  }
}

/* ---------------------------------------------------------------- GEMV */

/* y = W x (+ bias) (+ residual), fp64 sum rounded once to fp32 [RT section 7: FP32 accumulate] */
void orc_gemv(int fmt, const void *W, const void *S, int group, const float *x, const float *bias,
              const float *residual, float *y, int N, int K, int nthreads) {
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
    float *w = (float *)malloc(sizeof(float) * (size_t)K);
#pragma omp for schedule(static)
    for (int n = 0; n < N; ++n) {
      orc_dequant_row(fmt, W, S, group, n, K, w);
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += (double)w[k] * (double)x[k];
      if (bias) acc += (double)bias[n];
      if (residual) acc += (double)residual[n];
      y[n] = (float)acc;
    }
    free(w);
  }
}

/* ---------------------------------------------------------------- INT8 activations (Path A)
 *
 * [H100 "Challenge 3", Path A; RT section 7, "Bug #3"]: before the GEMV the activations are
 * quantised to INT8 with one scale per group of consecutive k, the dot product of the integer
 * weight levels with the INT8 activations is taken in integers, and the group scales undo the
 * quantisation on the integer sum.  The pages do not fix the scale or the rounding; the reading:
 * symmetric per group of `group` k, s = max|x| / 127, q = round-half-even(x * (127 / max|x|)),
 * every operation in binary32 (so the integer decision is the one the GPU takes), q in
 * [-127, 127]; a group of zeros has s = 0 and q = 0.  Inputs are finite.
 */
void orc_quantize_act_i8(const float *x, int K, int group, int8_t *q, float *sx) {
  for (int g = 0; g < K / group; ++g) {
    const float *xg = x + (int64_t)g * group;
    int8_t *qg = q + (int64_t)g * group;
    float amax = 0.0f;
    for (int i = 0; i < group; ++i) {
      const float a = fabsf(xg[i]);
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
      sx[g] = 0.0f;
      memset(qg, 0, (size_t)group);
      continue;
    }
    const float inv = 127.0f / amax; /* binary32 division, correctly rounded */
    sx[g] = amax / 127.0f;
    for (int i = 0; i < group; ++i) {
      const float t = xg[i] * inv;   /* binary32 product */
      float r = rintf(t);            /* nearest, ties to even */
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      qg[i] = (int8_t)r;
    }
  }
}

/* y[n] = sum over groups g of (weight scale) * sx[g] * sum_{k in g} level[n][k] * q[k] (+ bias)
 * (+ residual): integer sums are exact (int64), the scaling is fp64, rounded once to fp32.
 * INT8 weights: level = the int8 code, one scale per row (applied per group).  INT4 weights:
 * level = nibble - 8 and the fp16 scale of the weight group; the activation groups are the
 * weight groups. */
void orc_gemv_a8(int fmt, const void *W, const void *S, int group, const int8_t *q, const float *sx,
                 const float *bias, const float *residual, float *y, int N, int K, int nthreads) {
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int n = 0; n < N; ++n) {
    double acc = 0.0;
    for (int g = 0; g < K / group; ++g) {
      int64_t isum = 0;
      double ws;
      if (fmt == ORC_W_Q8) {
        const int8_t *w = (const int8_t *)W + (int64_t)n * K;
        for (int k = g * group; k < (g + 1) * group; ++k) isum += (int64_t)w[k] * q[k];
        ws = (double)((const float *)S)[n];
      } else {
        const uint8_t *b = (const uint8_t *)W + (int64_t)n * (K / 2);
        for (int k = g * group; k < (g + 1) * group; ++k) {
          const int nib = (k % 2 == 0) ? (b[k / 2] & 0x0F) : (b[k / 2] >> 4);
          isum += (int64_t)(nib - 8) * q[k];
        }
        ws = (double)orc_f16_to_f32(((const uint16_t *)S)[(int64_t)n * (K / group) + g]);
      }
      acc += ws * (double)sx[g] * (double)isum;
    }
    if (bias != NULL) acc += (double)bias[n];
    if (residual != NULL) acc += (double)residual[n];
    y[n] = (float)acc;
  }
}

/* ---------------------------------------------------------------- RMSNorm [NQ RMSNorm] */

void orc_rmsnorm(const float *x, const float *gamma, float *y, int rows, int dim, double eps) {
  for (int r = 0; r < rows; ++r) {
    const float *xr = x + (int64_t)r * dim;
    double ss = 0.0;
    for (int i = 0; i < dim; ++i) ss += (double)xr[i] * (double)xr[i];
    double inv = 1.0 / sqrt(ss / dim + eps);
    for (int i = 0; i < dim; ++i) {
      double g = gamma ? (double)gamma[i] : 1.0;
      y[(int64_t)r * dim + i] = (float)(g * (double)xr[i] * inv);
    }
  }
}

/* ---------------------------------------------------------------- RoPE [NQ Rope] */

/* Position as a 2-D rotation of coordinate pairs; angle of pair i is pos * base^(-2i/dim). */
void orc_rope(float *x, int rows, int dim, int pos, double base) {
  int half = dim / 2;
  for (int i = 0; i < half; ++i) {
    double theta = pow(base, -2.0 * (double)i / (double)dim);
    double phi = (double)pos * theta;
    double c = cos(phi), s = sin(phi);
    for (int r = 0; r < rows; ++r) {
      float *xr = x + (int64_t)r * dim;
      double a = xr[i], b = xr[i + half];
      xr[i] = (float)(a * c - b * s);
      xr[i + half] = (float)(b * c + a * s);
    }
  }
}

/* ---------------------------------------------------------------- SwiGLU [NQ SwiGLU] */

void orc_swiglu(const float *g, const float *u, float *m, int n) {
  for (int i = 0; i < n; ++i) {
    double z = g[i];
    double silu = z / (1.0 + exp(-z));
    m[i] = (float)(silu * (double)u[i]);
  }
}

/* ---------------------------------------------------------------- paged KV [PA; RT section 3] */

static inline int64_t kv_index(const int32_t *page_table, int page_size, int n_kv_heads, int head_dim,
                               int t, int j, int d) {
  int64_t page = page_table[t / page_size];
  return ((page * n_kv_heads + j) * page_size + (t % page_size)) * (int64_t)head_dim + d;
}

void orc_kv_store(void *pool, int kv_fmt, const int32_t *page_table, int page_size, int n_kv_heads,
                  int head_dim, int t, const float *kv) {
  for (int j = 0; j < n_kv_heads; ++j)
    for (int d = 0; d < head_dim; ++d) {
      int64_t i = kv_index(page_table, page_size, n_kv_heads, head_dim, t, j, d);
      float v = kv[j * head_dim + d];
      if (kv_fmt == ORC_KV_F32)
        ((float *)pool)[i] = v;
      else
        ((uint16_t *)pool)[i] = orc_f32_to_bf16(v);
    }
}

float orc_kv_load(const void *pool, int kv_fmt, const int32_t *page_table, int page_size,
                  int n_kv_heads, int head_dim, int t, int j, int d) {
  int64_t i = kv_index(page_table, page_size, n_kv_heads, head_dim, t, j, d);
  return kv_fmt == ORC_KV_F32 ? ((const float *)pool)[i] : orc_bf16_to_f32(((const uint16_t *)pool)[i]);
}

/* ---------------------------------------------------------------- GQA decode attention */

/*
 * Query head h reads KV head h / (Hq / Hkv) [RT section 3: 28 query heads share 4 KV heads].
 * Plain two-pass softmax in fp64 (max, exp, sum, divide), no split: the split-K form of the
 * FlashQwen stage-7 kernel is an exact reformulation of this.
 */
void orc_attention(const float *q, const void *k_pool, const void *v_pool, int kv_fmt,
                   const int32_t *page_table, int page_size, int T, int Hq, int Hkv, int D,
                   double scale, float *out, float *probs) {
  int G = Hq / Hkv;
#pragma omp parallel for schedule(static)
  for (int h = 0; h < Hq; ++h) {
    int j = h / G;
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
    double mx = -INFINITY;
    for (int t = 0; t < T; ++t) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d)
        acc += (double)q[h * D + d] *
               (double)orc_kv_load(k_pool, kv_fmt, page_table, page_size, Hkv, D, t, j, d);
      s[t] = acc * scale;
      if (s[t] > mx) mx = s[t];
    }
    double z = 0.0;
    for (int t = 0; t < T; ++t) {
      s[t] = exp(s[t] - mx);
      z += s[t];
    }
    for (int t = 0; t < T; ++t) {
      s[t] /= z;
      if (probs) probs[(int64_t)h * T + t] = (float)s[t];
    }
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int t = 0; t < T; ++t)
        acc += s[t] * (double)orc_kv_load(v_pool, kv_fmt, page_table, page_size, Hkv, D, t, j, d);
      out[h * D + d] = (float)acc;
    }
    free(s);
  }
}

/* ---------------------------------------------------------------- greedy [FQ stage 5; NQ Sampler] */

int orc_argmax(const float *v, int n) {
  int best = -1;
  for (int i = 0; i < n; ++i)
    if (v[i] == v[i] && (best < 0 || v[i] > v[best])) best = i;
  return best;
}

/* ---------------------------------------------------------------- sampling
 *
 * [FQ "Local benchmark": the chat flags --temperature, --top-p, --top-k, --seed and the Qwen3
 * recommended 0.6 / 0.95 / 20; FQ "Optimization study" stage 5 (greedy on the GPU, sampling
 * still copied the logits out); NQ "Sampler" (greedy takes the largest, top-k draws at random
 * among the k most probable tokens).]  The pages fix neither the order of the filters nor the
 * random source.  The reading:
 *   - temperature <= 0: greedy (orc_argmax);
 *   - z_i = l_i / T in fp64;
 *   - top-k (0 < k < V): the k largest logits, equal logits ordered by smaller index first;
 *   - top-p (p < 1): within that set in the same order, the shortest prefix whose softmax mass
 *     (fp64, exp(z - z_max) summed in that order) reaches p of the set's total;
 *   - the draw: Gumbel-max over the kept set, token = argmax of fp32(z_i + g_i) with
 *     g_i = -ln(-ln u_i), smallest index on equal keys.  u_i is uniform in (0, 1): the 64-bit
 *     word (i mod 4) of Philox4x64-10 with key (seed, 0) and counter (floor(i / 4), step, 0, 0),
 *     as ((word >> 11) + 0.5) * 2^-53.  Gumbel-max draws token i with probability
 *     exp(z_i) / sum over the kept set of exp(z_j).
 * Logits are finite. */

/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
 * SC'11): ten rounds of two 64x64 -> 128-bit multiplications with the published multipliers
 * and Weyl key increments. */
void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    const unsigned __int128 p0 = (unsigned __int128)0xD2E7470EE14C6C93ull * c0;
    const unsigned __int128 p1 = (unsigned __int128)0xCA5A826395121157ull * c2;
    const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    const uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += 0x9E3779B97F4A7C15ull;
    k1 += 0xBB67AE8584CAA73Bull;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

double orc_sample_uniform(uint64_t seed, int64_t step, int64_t i) {
  const uint64_t ctr[4] = {(uint64_t)i >> 2, (uint64_t)step, 0, 0}, key[2] = {seed, 0};
  uint64_t w[4];
  orc_philox4x64_10(ctr, key, w);
  return ((double)(w[i & 3] >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

typedef struct {
  float l;
  int i;
} orc_li;

static int orc_li_desc(const void *a, const void *b) {
  const orc_li *x = (const orc_li *)a, *y = (const orc_li *)b;
  if (x->l != y->l) return x->l > y->l ? -1 : 1;
  return x->i - y->i;
}

int orc_sample(const float *logits, int V, double temperature, int top_k, double top_p, uint64_t seed,
               int64_t step) {
  if (!(temperature > 0.0)) return orc_argmax(logits, V);
  const int filt_k = top_k > 0 && top_k < V;
  const int filt_p = top_p < 1.0;
  int n = V;
  orc_li *ord = NULL;
  if (filt_k || filt_p) {
    ord = (orc_li *)malloc(sizeof(orc_li) * (size_t)V);
    for (int i = 0; i < V; ++i) {
      ord[i].l = logits[i];
      ord[i].i = i;
    }
    qsort(ord, (size_t)V, sizeof(orc_li), orc_li_desc);
    if (filt_k) n = top_k;
    if (filt_p) {
      const double zmax = (double)ord[0].l / temperature;
      double tot = 0.0;
      for (int j = 0; j < n; ++j) tot += exp((double)ord[j].l / temperature - zmax);
      double cum = 0.0;
      for (int j = 0; j < n; ++j) {
        cum += exp((double)ord[j].l / temperature - zmax);
        if (cum >= top_p * tot) {
          n = j + 1;
          break;
        }
      }
    }
  }
  float best = 0.0f;
  int best_i = -1;
  for (int j = 0; j < n; ++j) {
    const int i = ord ? ord[j].i : j;
    const double g = -log(-log(orc_sample_uniform(seed, step, i)));
    const float key = (float)((double)logits[i] / temperature + g);
    if (best_i < 0 || key > best || (key == best && i < best_i)) {
      best = key;
      best_i = i;
    }
  }
  free(ord);
  return best_i;
}

/* ---------------------------------------------------------------- one decode step */

int orc_decode_step(const orc_config *c, const orc_layer *layers, const orc_head *head,
                    const int32_t *page_table, int pos, int token, float *h, float *trace,
                    float *logits, int nthreads) {
  return orc_decode_step_kv(c, layers, head, page_table, pos, token, h, trace, logits, nthreads, NULL, NULL, NULL);
}

/* Stores given bf16 codes as token t's entries of one layer's pool (the layout of orc_kv_store). */
static void kv_store_codes(void *pool, const int32_t *page_table, int page_size, int n_kv_heads, int head_dim,
                           int t, const uint16_t *codes) {
  for (int j = 0; j < n_kv_heads; ++j)
    for (int d = 0; d < head_dim; ++d)
      ((uint16_t *)pool)[kv_index(page_table, page_size, n_kv_heads, head_dim, t, j, d)] = codes[j * head_dim + d];
}

int orc_decode_step_kv(const orc_config *c, const orc_layer *layers, const orc_head *head,
                       const int32_t *page_table, int pos, int token, float *h, float *trace,
                       float *logits, int nthreads, float *kv_pre, const uint16_t *kv_force,
                       const uint8_t *force_mask) {
  const int H = c->hidden, Hq = c->n_heads, Hkv = c->n_kv_heads, D = c->head_dim, I = c->inter;
  const int qd = Hq * D, kvd = Hkv * D, T = pos + 1;
  const double scale = 1.0 / sqrt((double)D);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  float *a = (float *)malloc(sizeof(float) * (size_t)(H > qd ? H : qd));
  float *q = (float *)malloc(sizeof(float) * (size_t)qd);
  float *k = (float *)malloc(sizeof(float) * (size_t)kvd);
  float *v = (float *)malloc(sizeof(float) * (size_t)kvd);
  float *att = (float *)malloc(sizeof(float) * (size_t)qd);
  float *g = (float *)malloc(sizeof(float) * (size_t)I);
  float *u = (float *)malloc(sizeof(float) * (size_t)I);
  float *m = (float *)malloc(sizeof(float) * (size_t)I);

  /* embedding: the bf16 row of the token, widened exactly to fp32 */
  if (c->has_embedding)
    for (int i = 0; i < H; ++i) h[i] = orc_bf16_to_f32(head->embed[(int64_t)token * H + i]);
  if (trace) memcpy(trace, h, sizeof(float) * (size_t)H);

  for (int l = 0; l < c->n_layers; ++l) {
    const orc_layer *L = &layers[l];
    /* attention block: pre-norm, q/k/v projections with bias (Qwen2) */
    orc_rmsnorm(h, L->g_attn, a, 1, H, c->eps);
    orc_gemv(c->wfmt, L->wq, L->sq, c->group, a, c->has_bias ? L->bq : NULL, NULL, q, qd, H, nthreads);
    orc_gemv(c->wfmt, L->wk, L->sk, c->group, a, c->has_bias ? L->bk : NULL, NULL, k, kvd, H, nthreads);
    orc_gemv(c->wfmt, L->wv, L->sv, c->group, a, c->has_bias ? L->bv : NULL, NULL, v, kvd, H, nthreads);
    if (c->has_qk_norm) { /* per-head RMSNorm of q and k (Qwen3), before RoPE */
      orc_rmsnorm(q, L->g_q, q, Hq, D, c->eps);
      orc_rmsnorm(k, L->g_k, k, Hkv, D, c->eps);
    }
    orc_rope(q, Hq, D, pos, c->rope_base);
    orc_rope(k, Hkv, D, pos, c->rope_base);
    /* append the new token, then attend over keys 0..pos read back from the cache */
    if (kv_pre) {
      memcpy(kv_pre + (int64_t)(2 * l) * kvd, k, sizeof(float) * (size_t)kvd);
      memcpy(kv_pre + (int64_t)(2 * l + 1) * kvd, v, sizeof(float) * (size_t)kvd);
    }
    if (kv_force && force_mask && force_mask[l] && c->kv_fmt == ORC_KV_BF16) {
      kv_store_codes(L->k_pool, page_table, c->page_size, Hkv, D, pos, kv_force + (int64_t)(2 * l) * kvd);
      kv_store_codes(L->v_pool, page_table, c->page_size, Hkv, D, pos, kv_force + (int64_t)(2 * l + 1) * kvd);
    } else {
      orc_kv_store(L->k_pool, c->kv_fmt, page_table, c->page_size, Hkv, D, pos, k);
      orc_kv_store(L->v_pool, c->kv_fmt, page_table, c->page_size, Hkv, D, pos, v);
    }
    orc_attention(q, L->k_pool, L->v_pool, c->kv_fmt, page_table, c->page_size, T, Hq, Hkv, D, scale,
                  att, NULL);
    orc_gemv(c->wfmt, L->wo, L->so, c->group, att, NULL, h, h, H, qd, nthreads);
    /* MLP block: pre-norm, SwiGLU, down projection */
    orc_rmsnorm(h, L->g_ffn, a, 1, H, c->eps);
    orc_gemv(c->wfmt, L->wg, L->sg, c->group, a, NULL, NULL, g, I, H, nthreads);
    orc_gemv(c->wfmt, L->wu, L->su, c->group, a, NULL, NULL, u, I, H, nthreads);
    orc_swiglu(g, u, m, I);
    orc_gemv(c->wfmt, L->wd, L->sd, c->group, m, NULL, h, h, H, I, nthreads);
    if (trace) memcpy(trace + (int64_t)(l + 1) * H, h, sizeof(float) * (size_t)H);
  }

  int next = -1;
  if (c->has_lm_head) {
    orc_rmsnorm(h, head->g_out, a, 1, H, c->eps);
    float *lg = logits ? logits : (float *)malloc(sizeof(float) * (size_t)c->vocab);
    orc_gemv(c->wfmt, head->w_lm, head->s_lm, c->group, a, NULL, NULL, lg, c->vocab, H, nthreads);
    next = orc_argmax(lg, c->vocab);
    if (!logits) free(lg);
  }
  free(a); free(q); free(k); free(v); free(att); free(g); free(u); free(m);
  return next;
}

/* ---------------------------------------------------------------- batched decode
 * [Systems "PagedAttention - Virtual Memory for KV Caches", "Continuous Batching", "Request
 * Lifecycle" (decode: one new token per running sequence per step, all running sequences batched
 * together; each sequence's block table maps its logical blocks to physical blocks of one shared
 * pool, allocated on demand).]  Sequences in a batch do not interact: the batched step is the
 * single-sequence step applied to every running slot with that slot's block table, position and
 * token.  A slot with pos < 0 is idle and left untouched. */
void orc_decode_batch(const orc_config *c, const orc_layer *layers, const orc_head *head, int B,
                      const int32_t *block_tables, int max_blocks, const int32_t *pos, const int32_t *tokens,
                      float *h, float *logits, int32_t *next, int nthreads) {
  for (int b = 0; b < B; ++b) {
    if (pos[b] < 0) continue;
    next[b] = orc_decode_step(c, layers, head, block_tables + (int64_t)b * max_blocks, pos[b], tokens[b],
                              h + (int64_t)b * c->hidden, NULL,
                              logits ? logits + (int64_t)b * c->vocab : NULL, nthreads);
  }
}

/* ---------------------------------------------------------------- prefill
 * [RT section 6 and FQ "Local benchmark": prefill runs the whole prompt through the model, writing
 * its KV, and the first token comes from the last position's logits.]  A causal decoder's prefill
 * of tokens t_0 .. t_{T-1} at positions pos0 .. pos0 + T - 1 is, by definition, the single-token
 * step applied to each position in order: position p attends to keys 0 .. p.  Returns the greedy
 * token of the last position; h and logits are those of the last position. */
int orc_prefill(const orc_config *c, const orc_layer *layers, const orc_head *head, const int32_t *page_table,
                int pos0, const int32_t *tokens, int T, float *h, float *logits, int nthreads) {
  /* positions before the last need no logits: their steps skip the lm head */
  orc_config body = *c;
  body.has_lm_head = 0;
  int next = -1;
  for (int t = 0; t < T; ++t)
    next = orc_decode_step(t == T - 1 ? c : &body, layers, head, page_table, pos0 + t, tokens[t], h, NULL,
                           t == T - 1 ? logits : NULL, nthreads);
  return next;
}

