/*
 * Seeded synthetic inputs for the batch-1 quantized decode step.
 *
 * This file only draws random numbers and stores them in the storage types the
 * decode step reads (int8, packed nibbles, IEEE fp16, bf16, fp32).  It holds no
 * step of the decode method itself: no dequantisation, no dot product, no
 * normalisation, no attention.  Both the CPU oracle and the GPU path read the
 * bytes written here, and neither of them links this file.
 *
 * Generator: a counter-based splitmix64.  splitmix64 is the generator of
 * Steele, Lea and Flood ("Fast splittable pseudorandom number generators",
 * OOPSLA 2014): the state advances by the golden-ratio increment and each
 * output is the state passed through the variant-13 64-bit finaliser.  Used as
 * a counter-based generator, element i of stream (seed, tensor id) is the
 * finaliser applied to key + (i + 1) * increment, where key is itself the
 * finaliser of seed and tensor id.  Every element can therefore be
 * regenerated on its own, and the output does not depend on thread count.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC synth.c -o libsynth.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t fin64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return fin64(fin64(seed + GOLDEN) ^ (stream * 0xD1B54A32D192ED03ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return fin64(key + (i + 1) * GOLDEN); }

/* uniform double in [0, 1) from the top 53 bits */
static inline double unif(uint64_t r) { return (double)(r >> 11) * (1.0 / 9007199254740992.0); }

uint64_t synth_draw(uint64_t seed, uint64_t stream, uint64_t i) {
  return draw(stream_key(seed, stream), i);
}

/* fp32 -> bf16, round to nearest even (finite inputs only: the generator never makes NaN/Inf) */
static inline uint16_t to_bf16(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* double -> IEEE binary16, round to nearest even, for finite values of magnitude
   in the normal fp16 range [2^-14, 65504]; zero maps to +0.  Returns 0xFFFF on
   out-of-range input so a bad recipe is visible. */
static inline uint16_t to_f16(double x) {
  if (x == 0.0) return 0;
  uint16_t sign = 0;
  if (x < 0) { sign = 0x8000; x = -x; }
  int e;
  double m = frexp(x, &e);          /* x = m * 2^e, m in [0.5, 1) */
  e -= 1;                            /* x = (2m) * 2^e, 2m in [1, 2) */
  if (e < -14 || e > 15) return 0xFFFF;
  double sig = nearbyint(ldexp(x, 10 - e)); /* 11-bit significand, RNE */
  if (sig >= 2048.0) { sig = 1024.0; e += 1; if (e > 15) return 0xFFFF; }
  return (uint16_t)(sign | ((uint16_t)(e + 15) << 10) | ((uint16_t)sig - 1024));
}

/* standard normal for element i: Box-Muller on the pair (i/2); even i takes the
   cosine branch, odd i the sine branch */
static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = unif(draw(key, 2 * p));
  double u2 = unif(draw(key, 2 * p + 1));
  double r = sqrt(-2.0 * log(1.0 - u1)); /* 1-u1 in (0, 1] */
  double a = 6.283185307179586476925 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

/* uniform bytes 0..255: both nibbles of a byte are then uniform on 0..15 and independent */
void synth_fill_u8(uint8_t *out, int64_t n, uint64_t seed, uint64_t stream) {
  uint64_t key = stream_key(seed, stream);
  int64_t nw = n / 8;
#pragma omp parallel for schedule(static)
  for (int64_t w = 0; w < nw; ++w) {
    uint64_t r = draw(key, (uint64_t)w);
    memcpy(out + 8 * w, &r, 8); /* little-endian host: byte b = bits 8b..8b+7 */
  }
  if (n % 8) {
    uint64_t r = draw(key, (uint64_t)nw);
    for (int64_t b = 0; b < n % 8; ++b) out[8 * nw + b] = (uint8_t)(r >> (8 * b));
  }
}

/* uniform integers on [lo, hi] as int8 (multiply-shift reduction of 32 random bits) */
void synth_fill_i8(int8_t *out, int64_t n, uint64_t seed, uint64_t stream, int lo, int hi) {
  uint64_t key = stream_key(seed, stream);
  uint64_t span = (uint64_t)(hi - lo + 1);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t r = draw(key, (uint64_t)i) >> 32;
    out[i] = (int8_t)(lo + (int)((r * span) >> 32));
  }
}

void synth_fill_f32_normal(float *out, int64_t n, uint64_t seed, uint64_t stream, double mean,
                           double std) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + std * normal_at(key, (uint64_t)i));
}

void synth_fill_f32_uniform(float *out, int64_t n, uint64_t seed, uint64_t stream, double lo,
                            double hi) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(lo + (hi - lo) * unif(draw(key, (uint64_t)i)));
}

void synth_fill_f16_uniform(uint16_t *out, int64_t n, uint64_t seed, uint64_t stream, double lo,
                            double hi) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = to_f16(lo + (hi - lo) * unif(draw(key, (uint64_t)i)));
}

void synth_fill_bf16_normal(uint16_t *out, int64_t n, uint64_t seed, uint64_t stream, double mean,
                            double std) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = to_bf16((float)(mean + std * normal_at(key, (uint64_t)i)));
}

/* Fisher-Yates shuffle of 0..n-1, driven by the counter stream (sequential by nature) */
void synth_permutation(int32_t *out, int64_t n, uint64_t seed, uint64_t stream) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)i;
  for (int64_t i = n - 1; i > 0; --i) {
    uint64_t r = draw(key, (uint64_t)i) >> 32;
    int64_t j = (int64_t)((r * (uint64_t)(i + 1)) >> 32);
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/*
 * Prior-context KV values, drawn by LOGICAL index (token t, kv head j, dim d) so the
 * value at a token does not depend on where its page lives, then stored at the
 * physical slot pool[page_table[t / page_size]][j][t % page_size][d].
 * kv_fmt 1: fp32 pool, kv_fmt 2: bf16 pool.  Slots of tokens >= ctx are left untouched.
 */
void synth_fill_kv(void *pool, int kv_fmt, const int32_t *page_table, int page_size, int64_t ctx,
                   int n_kv_heads, int head_dim, uint64_t seed, uint64_t stream, double std) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < ctx; ++t) {
    int64_t page = page_table[t / page_size];
    int64_t slot = t % page_size;
    for (int j = 0; j < n_kv_heads; ++j) {
      int64_t dst = ((page * n_kv_heads + j) * page_size + slot) * head_dim;
      int64_t src = (t * n_kv_heads + j) * (int64_t)head_dim;
      for (int d = 0; d < head_dim; ++d) {
        float v = (float)(std * normal_at(key, (uint64_t)(src + d)));
        if (kv_fmt == 1)
          ((float *)pool)[dst + d] = v;
        else
          ((uint16_t *)pool)[dst + d] = to_bf16(v);
      }
    }
  }
}

/*
 * Input recipe for a tied embedding next to an INT8 per-row lm_head: the embedding
 * table is the same matrix stored in bf16, E[r][c] = bf16(fp32(q[r][c]) * s[r]).
 * This builds an input table; the decode step only ever reads E as given.
 */
void synth_tied_embedding(uint16_t *E, const int8_t *q, const float *s, int64_t rows, int64_t cols) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) E[r * cols + c] = to_bf16((float)q[r * cols + c] * s[r]);
}
