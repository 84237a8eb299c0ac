// Small per-step kernels: q/k RMSNorm + RoPE + KV append, RMSNorm/RoPE rows, SwiGLU, embedding
// gather, greedy argmax.  Each is a few KB of traffic per step; they are written for latency
// (one wave per head or row, wave64 shuffles) rather than bandwidth.
//
// Definitions (naive-CUDA Qwen engine post, part 1): RMSNorm y = g * x / sqrt(mean(x^2) + eps)
// (section RMSNorm); RoPE rotates coordinate pairs as 2-D rotations by position-proportional
// angles (section Rope) with the rotate-half pairing (i, i + D/2) and theta_i = base^(-2i/D);
// SwiGLU multiplies the Swish of one projection by the other (section SwiGLU), Swish taken with
// beta = 1 on the gate projection; greedy sampling picks the largest logit (section Sampler),
// the smallest index on ties, done on the GPU so one int leaves the device (FlashQwen README,
// "Optimization study", stage 5).
#include <hip/hip_runtime.h>

#include <climits>

#include "qdec_batch.h"

namespace qdec {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x7FFFFFu)) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// One wave normalises (optional) and rotates (optional) one row of `dim` <= 256 values.
// src and dst may alias.  On return the final row is also in `buf` (LDS, >= dim floats, private
// to the single-wave workgroup) and visible to every lane.
__device__ void norm_rope_row(const float *src, float *dst, int dim, const float *gamma, float eps,
                              float base, int pos, float *buf) {
  const int lane = threadIdx.x & 63;
  float v[4];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < dim) ? src[e] : 0.f;
    ss += v[i] * v[i];
  }
  if (gamma) {
    const float r = rsqrtf(wave_sum(ss) / (float)dim + eps);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < dim) v[i] = gamma[e] * (v[i] * r);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    if (e < dim) buf[e] = v[i];
  }
  __syncthreads();
  if (base > 0.f) {
    const int half = dim / 2;
    double ra[2], rb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int i = lane + 64 * c;
      if (i < half) {
        const double theta = pow((double)base, -2.0 * (double)i / (double)dim);
        const double phi = (double)pos * theta;
        double sn, cs;
        sincos(phi, &sn, &cs);
        const double a = buf[i], b = buf[i + half];
        ra[c] = a * cs - b * sn;
        rb[c] = b * cs + a * sn;
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int i = lane + 64 * c;
      if (i < half) {
        buf[i] = (float)ra[c];
        buf[i + half] = (float)rb[c];
      }
    }
    __syncthreads();
  }
  for (int e = lane; e < dim; e += 64) dst[e] = buf[e];
}

__device__ __forceinline__ void store_kv(void *pool, int kv_fmt, size_t e, float v) {
  if (kv_fmt == QDEC_KV_BF16)
    reinterpret_cast<uint16_t *>(pool)[e] = float_to_bf16_rne(v);
  else
    reinterpret_cast<float *>(pool)[e] = v;
}

// grid: Hq + 2 Hkv waves, one per q head, k head, v head (in that order)
__global__ void __launch_bounds__(64) qkv_post(QkvPostArgs a) {
  __shared__ float buf[256];
  const int hh = blockIdx.x;
  const int D = a.D;
  const int t = *a.pos;
  float *x;
  int kind, j;
  if (hh < a.Hq) {
    kind = 0; j = hh; x = a.qkv + (size_t)hh * D;
  } else if (hh < a.Hq + a.Hkv) {
    kind = 1; j = hh - a.Hq; x = a.qkv + (size_t)(a.Hq + j) * D;
  } else {
    kind = 2; j = hh - a.Hq - a.Hkv; x = a.qkv + (size_t)(a.Hq + a.Hkv + j) * D;
  }
  if (kind < 2) {
    norm_rope_row(x, x, D, kind == 0 ? a.g_q : a.g_k, a.eps, a.rope_base, t, buf);
  }
  if (kind == 0 || !a.k_pool) return;
  const int phys = a.page_table[t >> 4];
  if (phys < 0 || phys >= a.n_pages) return;
  void *pool = (kind == 1) ? a.k_pool : a.v_pool;
  const size_t e0 = (((size_t)phys * a.Hkv + j) * 16 + (t & 15)) * D;
  for (int d = threadIdx.x; d < D; d += 64) store_kv(pool, a.kv_fmt, e0 + d, kind == 1 ? buf[d] : x[d]);
}

__global__ void __launch_bounds__(64) rmsnorm_rope_rows(const float *x, const float *gamma, float *y,
                                                        int dim, float eps, float base,
                                                        const int32_t *pos) {
  __shared__ float buf[256];
  const int row = blockIdx.x;
  const int t = pos ? *pos : 0;
  norm_rope_row(x + (size_t)row * dim, y + (size_t)row * dim, dim, gamma, eps, base, t, buf);
}

__global__ void swiglu_k(const float *__restrict__ g, const float *__restrict__ u, float *__restrict__ m, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const float z = g[i];
    m[i] = (z / (1.0f + expf(-z))) * u[i];
  }
}

// grid: ceil(H/64) waves.  E == null: h is given, only the per-tile sums of squares are written.
__global__ void __launch_bounds__(64) embed_k(const uint16_t *__restrict__ E, const int32_t *__restrict__ token,
                                              int H, int V, float *h, float *__restrict__ ssq,
                                              const int32_t *__restrict__ pos, float base, int D,
                                              double *__restrict__ cs, unsigned *epoch) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (epoch && blockIdx.x == 0 && threadIdx.x == 0) *epoch += 1u;
  if (cs && blockIdx.x == 0) {
    // same angle as the per-row rotation above: theta_i = base^(-2i/D), phi = pos * theta_i
    const int t = *pos;
    for (int k = threadIdx.x; k < D / 2; k += 64) {
      const double theta = pow((double)base, -2.0 * (double)k / (double)D);
      double sn, c;
      sincos((double)t * theta, &sn, &c);
      cs[2 * k] = c;
      cs[2 * k + 1] = sn;
    }
  }
  float v = 0.f;
  if (E) {
    int tok = *token;
    if (tok < 0 || tok >= V) tok = 0;  // documented precondition; never read outside the table
    if (i < H) {
      v = __builtin_bit_cast(float, (uint32_t)E[(size_t)tok * H + i] << 16);
      h[i] = v;
    }
  } else if (i < H) {
    v = h[i];
  }
  const float s = wave_sum(v * v);
  if (threadIdx.x == 0) ssq[blockIdx.x] = s;
}

__global__ void __launch_bounds__(1024) argmax_finish_k(const float *__restrict__ logits, int n,
                                                        int32_t *token, int32_t *pos, int32_t *log,
                                                        int32_t *step, int log_len) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const int tid = threadIdx.x;
  int bi = INT_MAX;
  float bv = -INFINITY;
  if (logits) {
    for (int i = tid; i < n; i += 1024) {
      const float v = logits[i];
      if (v == v && (bi == INT_MAX || v > bv)) {  // strict: the first index of a maximum wins
        bv = v;
        bi = i;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float v2 = __shfl_xor(bv, o, 64);
      const int i2 = __shfl_xor(bi, o, 64);
      if (i2 != INT_MAX && (bi == INT_MAX || v2 > bv || (v2 == bv && i2 < bi))) {
        bv = v2;
        bi = i2;
      }
    }
    if ((tid & 63) == 0) {
      sv[tid >> 6] = bv;
      si[tid >> 6] = bi;
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (logits) {
      bv = sv[0];
      bi = si[0];
      for (int w = 1; w < 16; ++w) {
        const int i2 = si[w];
        const float v2 = sv[w];
        if (i2 != INT_MAX && (bi == INT_MAX || v2 > bv || (v2 == bv && i2 < bi))) {
          bv = v2;
          bi = i2;
        }
      }
      if (bi == INT_MAX) bi = 0;  // all NaN: token 0
      *token = bi;
      if (log && step) {
        const int s = *step;
        if (s >= 0 && s < log_len) log[s] = bi;
      }
    }
    if (step) *step += 1;
    if (pos) *pos += 1;
  }
}

// ------------------------------------------------------------------ rows of the batched step
// grid (ceil(H / 256), B): h[b] = E[tokens[b]] for running rows; block (0, b) also writes row b's
// RoPE table (the same angles as embed_k)
__global__ void __launch_bounds__(256) embed_rows_k(const uint16_t *__restrict__ E, const int32_t *__restrict__ tokens,
                                                    const int32_t *__restrict__ pos, int H, int V, float *h,
                                                    float *__restrict__ ssq, float base, int D, double *__restrict__ cs) {
  const int b = blockIdx.y;
  const int t = pos[b];
  if (t < 0) return;
  if (blockIdx.x == 0) {
    double *c = cs + (size_t)b * D;
    for (int k = threadIdx.x; k < D / 2; k += 256) {
      const double theta = pow((double)base, -2.0 * (double)k / (double)D);
      double sn, co;
      sincos((double)t * theta, &sn, &co);
      c[2 * k] = co;
      c[2 * k + 1] = sn;
    }
  }
  int tok = tokens[b];
  if (tok < 0 || tok >= V) tok = 0;  // documented precondition; never read outside the table
  const int i = blockIdx.x * 256 + threadIdx.x;
  const float v = i < H ? __builtin_bit_cast(float, (uint32_t)E[(size_t)tok * H + i] << 16) : 0.f;
  if (i < H) h[(size_t)b * H + i] = v;
  // wave w of the block covers the 64-value tile 4 blockIdx.x + w
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (ssq && tile * 64 < H) {
    const float sq = wave_sum(v * v);
    if ((threadIdx.x & 63) == 0) ssq[(size_t)b * ((H + 63) / 64) + tile] = sq;
  }
}

// one workgroup of 1024 threads per row: y = gamma * x / sqrt(mean(x^2) + eps); rows of a
// multiple of 4 values are read and written as float4, each element loaded once into registers
__global__ void __launch_bounds__(1024) rmsnorm_rows_k(const float *__restrict__ x, const float *__restrict__ gamma,
                                                       float *__restrict__ y, int dim, float eps) {
  __shared__ float part[16];
  const float4 *xr = reinterpret_cast<const float4 *>(x + (size_t)blockIdx.x * dim);
  float4 *yr = reinterpret_cast<float4 *>(y + (size_t)blockIdx.x * dim);
  const float4 *g4 = reinterpret_cast<const float4 *>(gamma);
  const int n4 = dim / 4;
  constexpr int kMaxPer = 4;  // float4 per thread held in registers (rows up to 16384 values)
  float4 v[kMaxPer];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    const int i = threadIdx.x + 1024 * k;
    v[k] = i < n4 ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    ss += (v[k].x * v[k].x + v[k].y * v[k].y) + (v[k].z * v[k].z + v[k].w * v[k].w);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < 16; ++w) tot += part[w];
  const float r = rsqrtf(tot / (float)dim + eps);
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    const int i = threadIdx.x + 1024 * k;
    if (i < n4) {
      const float4 g = g4[i];
      yr[i] = make_float4(g.x * (v[k].x * r), g.y * (v[k].y * r), g.z * (v[k].z * r), g.w * (v[k].w * r));
    }
  }
}

// (value, index) reduction of one workgroup of 1024 threads: larger value, then smaller index
__device__ __forceinline__ void block_argmax_1024(float &bv, int &bi, float *sv, int *si) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v2 = __shfl_xor(bv, o, 64);
    const int i2 = __shfl_xor(bi, o, 64);
    if (i2 != INT_MAX && (bi == INT_MAX || v2 > bv || (v2 == bv && i2 < bi))) {
      bv = v2;
      bi = i2;
    }
  }
  if ((tid & 63) == 0) {
    sv[tid >> 6] = bv;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  bv = sv[0];
  bi = si[0];
  for (int w = 1; w < 16; ++w) {
    const int i2 = si[w];
    const float v2 = sv[w];
    if (i2 != INT_MAX && (bi == INT_MAX || v2 > bv || (v2 == bv && i2 < bi))) {
      bv = v2;
      bi = i2;
    }
  }
}

constexpr int kArgChunks = 64;  // workgroups per row in the first argmax pass

// grid (kArgChunks, B): candidate (value, index) of chunk c of row b
__global__ void __launch_bounds__(1024) argmax_rows_part_k(const float *__restrict__ logits, int V,
                                                           const int32_t *__restrict__ pos, float *cv, int *ci) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const int b = blockIdx.y;
  if (pos[b] < 0) return;
  const int chunk = (V + kArgChunks - 1) / kArgChunks;
  const int i0 = blockIdx.x * chunk, i1 = min(V, i0 + chunk);
  const float *lg = logits + (size_t)b * V;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int i = i0 + (int)threadIdx.x; i < i1; i += 1024) {
    const float v = lg[i];
    if (v == v && (bi == INT_MAX || v > bv)) {
      bv = v;
      bi = i;
    }
  }
  block_argmax_1024(bv, bi, sv, si);
  if (threadIdx.x == 0) {
    cv[b * kArgChunks + blockIdx.x] = bv;
    ci[b * kArgChunks + blockIdx.x] = bi;
  }
}

// one wave per row: tokens[b] = smallest index of the largest logit over the chunk candidates,
// pos[b] += 1
__global__ void __launch_bounds__(64) argmax_rows_k(const float *__restrict__ cv, const int *__restrict__ ci,
                                                    int32_t *tokens, int32_t *pos) {
  const int b = blockIdx.x;
  if (pos[b] < 0) return;
  const int tid = threadIdx.x;
  float bv = cv[b * kArgChunks + tid];
  int bi = ci[b * kArgChunks + tid];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v2 = __shfl_xor(bv, o, 64);
    const int i2 = __shfl_xor(bi, o, 64);
    if (i2 != INT_MAX && (bi == INT_MAX || v2 > bv || (v2 == bv && i2 < bi))) {
      bv = v2;
      bi = i2;
    }
  }
  if (tid == 0) {
    tokens[b] = (bi == INT_MAX) ? 0 : bi;
    pos[b] += 1;
  }
}

// ------------------------------------------------------------------ prefill rows
__global__ void prefill_positions_k(const int32_t *__restrict__ pos, int T, int32_t *__restrict__ rows) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < T) rows[t] = *pos + t;
}

__global__ void add_pos_k(int32_t *pos, int delta) {
  if (threadIdx.x == 0) *pos += delta;
}

// grid (ceil(H / 256), T)
__global__ void __launch_bounds__(256) embed_tokens_k(const uint16_t *__restrict__ E, const int32_t *__restrict__ tokens,
                                                      int H, int V, float *__restrict__ x) {
  int tok = tokens[blockIdx.y];
  if (tok < 0 || tok >= V) tok = 0;  // documented precondition; never read outside the table
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < H) x[(size_t)blockIdx.y * H + i] = __builtin_bit_cast(float, (uint32_t)E[(size_t)tok * H + i] << 16);
}

// fp32 -> fp16 pair: h = fp16(v) (nearest even), l = fp16(v - h); h + l carries 22 bits of v
__device__ __forceinline__ void split_h(float v, uint32_t &h, uint32_t &l) {
  const _Float16 hi = (_Float16)v;
  h = __builtin_bit_cast(uint16_t, hi);
  l = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)hi));
}

// as rmsnorm_rows_k, the output as an fp16 pair
__global__ void __launch_bounds__(1024) rmsnorm_rows_h_k(const float *__restrict__ x, const float *__restrict__ gamma,
                                                         uint16_t *__restrict__ yh, uint16_t *__restrict__ yl, int dim,
                                                         float eps) {
  __shared__ float part[16];
  const float4 *xr = reinterpret_cast<const float4 *>(x + (size_t)blockIdx.x * dim);
  uint2 *yrh = reinterpret_cast<uint2 *>(yh + (size_t)blockIdx.x * dim);
  uint2 *yrl = reinterpret_cast<uint2 *>(yl + (size_t)blockIdx.x * dim);
  const float4 *g4 = reinterpret_cast<const float4 *>(gamma);
  const int n4 = dim / 4;
  constexpr int kMaxPer = 4;
  float4 v[kMaxPer];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    const int i = threadIdx.x + 1024 * k;
    v[k] = i < n4 ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    ss += (v[k].x * v[k].x + v[k].y * v[k].y) + (v[k].z * v[k].z + v[k].w * v[k].w);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < 16; ++w) tot += part[w];
  const float r = rsqrtf(tot / (float)dim + eps);
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    const int i = threadIdx.x + 1024 * k;
    if (i < n4) {
      const float4 g = g4[i];
      uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
      split_h(g.x * (v[k].x * r), h0, l0);
      split_h(g.y * (v[k].y * r), h1, l1);
      split_h(g.z * (v[k].z * r), h2, l2);
      split_h(g.w * (v[k].w * r), h3, l3);
      yrh[i] = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
      yrl[i] = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
    }
  }
}

__global__ void to_half_k(const float *__restrict__ x, uint16_t *__restrict__ yh, uint16_t *__restrict__ yl, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    uint32_t h, l;
    split_h(x[i], h, l);
    yh[i] = (uint16_t)h;
    yl[i] = (uint16_t)l;
  }
}

// grid (Hq + 2 Hkv, T): as qkv_post for token t at position pos_rows[t]
__global__ void __launch_bounds__(64) qkv_post_rows_k(QkvRows r) {
  __shared__ float buf[256];
  const QkvPostArgs &a = r.a;
  const int hh = blockIdx.x, row = blockIdx.y;
  const int D = a.D;
  const int t = r.pos_rows[row];
  float *qkv = r.qkv + (size_t)row * (a.Hq + 2 * a.Hkv) * D;
  float *x;
  int kind, j;
  if (hh < a.Hq) {
    kind = 0; j = hh; x = qkv + (size_t)hh * D;
  } else if (hh < a.Hq + a.Hkv) {
    kind = 1; j = hh - a.Hq; x = qkv + (size_t)(a.Hq + j) * D;
  } else {
    kind = 2; j = hh - a.Hq - a.Hkv; x = qkv + (size_t)(a.Hq + a.Hkv + j) * D;
  }
  if (kind < 2) norm_rope_row(x, x, D, kind == 0 ? a.g_q : a.g_k, a.eps, a.rope_base, t, buf);
  if (kind == 0 || !a.k_pool) return;
  const int phys = a.page_table[t >> 4];
  if (phys < 0 || phys >= a.n_pages) return;
  void *pool = (kind == 1) ? a.k_pool : a.v_pool;
  const size_t e0 = (((size_t)phys * a.Hkv + j) * 16 + (t & 15)) * D;
  for (int d = threadIdx.x; d < D; d += 64) store_kv(pool, a.kv_fmt, e0 + d, kind == 1 ? buf[d] : x[d]);
}

__global__ void copy_k(const float *__restrict__ s, float *__restrict__ d, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) d[i] = s[i];
}

}  // namespace

hipError_t launch_qkv_post(const QkvPostArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(qkv_post, dim3(a.Hq + 2 * a.Hkv), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rope(const float *x, const float *gamma, float *y, int rows, int dim,
                               float eps, float rope_base, const int32_t *pos, hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_rope_rows, dim3(rows), dim3(64), 0, st, x, gamma, y, dim, eps, rope_base,
                     pos);
  return hipGetLastError();
}

hipError_t launch_swiglu(const float *g, const float *u, float *m, int n, hipStream_t st) {
  int blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(swiglu_k, dim3(blocks), dim3(256), 0, st, g, u, m, n);
  return hipGetLastError();
}

hipError_t launch_embed(const uint16_t *E, const int32_t *token, int H, int V, float *h, float *ssq,
                        const int32_t *pos, float rope_base, int D, double *rope_cs, unsigned *epoch,
                        hipStream_t st) {
  hipLaunchKernelGGL(embed_k, dim3((H + 63) / 64), dim3(64), 0, st, E, token, H, V, h, ssq, pos, rope_base,
                     D, rope_cs, epoch);
  return hipGetLastError();
}

hipError_t launch_argmax_finish(const float *logits, int n, int32_t *token, int32_t *pos,
                                int32_t *token_log, int32_t *step_count, int log_len,
                                hipStream_t st) {
  hipLaunchKernelGGL(argmax_finish_k, dim3(1), dim3(1024), 0, st, logits, n, token, pos, token_log,
                     step_count, log_len);
  return hipGetLastError();
}

hipError_t launch_embed_rows(const uint16_t *E, const int32_t *tokens, const int32_t *pos, int B, int H, int V,
                             float *h, float *ssq, float rope_base, int D, double *rope_cs, hipStream_t st) {
  hipLaunchKernelGGL(embed_rows_k, dim3((H + 255) / 256, B), dim3(256), 0, st, E, tokens, pos, H, V, h, ssq, rope_base,
                     D, rope_cs);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const float *x, const float *gamma, float *y, int B, int dim, float eps, hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_rows_k, dim3(B), dim3(1024), 0, st, x, gamma, y, dim, eps);
  return hipGetLastError();
}

size_t argmax_rows_workspace_bytes(int B) { return (size_t)B * kArgChunks * 8; }

hipError_t launch_argmax_rows(const float *logits, int B, int V, int32_t *tokens, int32_t *pos, void *ws,
                              hipStream_t st) {
  float *cv = reinterpret_cast<float *>(ws);
  int *ci = reinterpret_cast<int *>(cv + (size_t)B * kArgChunks);
  hipLaunchKernelGGL(argmax_rows_part_k, dim3(kArgChunks, B), dim3(1024), 0, st, logits, V, pos, cv, ci);
  hipLaunchKernelGGL(argmax_rows_k, dim3(B), dim3(64), 0, st, cv, ci, tokens, pos);
  return hipGetLastError();
}

hipError_t launch_prefill_positions(const int32_t *pos, int T, int32_t *pos_rows, hipStream_t st) {
  hipLaunchKernelGGL(prefill_positions_k, dim3((T + 255) / 256), dim3(256), 0, st, pos, T, pos_rows);
  return hipGetLastError();
}

hipError_t launch_add_pos(int32_t *pos, int delta, hipStream_t st) {
  hipLaunchKernelGGL(add_pos_k, dim3(1), dim3(64), 0, st, pos, delta);
  return hipGetLastError();
}

hipError_t launch_embed_tokens(const uint16_t *E, const int32_t *tokens, int T, int H, int V, float *x, hipStream_t st) {
  hipLaunchKernelGGL(embed_tokens_k, dim3((H + 255) / 256, T), dim3(256), 0, st, E, tokens, H, V, x);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows_h(const float *x, const float *gamma, uint16_t *yh, uint16_t *yl, int B, int dim,
                                 float eps, hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_rows_h_k, dim3(B), dim3(1024), 0, st, x, gamma, yh, yl, dim, eps);
  return hipGetLastError();
}

hipError_t launch_to_half(const float *x, uint16_t *yh, uint16_t *yl, size_t n, hipStream_t st) {
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(to_half_k, dim3((unsigned)blocks), dim3(256), 0, st, x, yh, yl, n);
  return hipGetLastError();
}

hipError_t launch_qkv_post_rows(const QkvRows &r, hipStream_t st) {
  hipLaunchKernelGGL(qkv_post_rows_k, dim3(r.a.Hq + 2 * r.a.Hkv, r.T), dim3(64), 0, st, r);
  return hipGetLastError();
}

hipError_t launch_copy(const float *src, float *dst, int n, hipStream_t st) {
  hipLaunchKernelGGL(copy_k, dim3((n + 255) / 256), dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}


// ------------------------------------------------------------------------------ streaming read
// Reference read for bandwidth measurements: every byte of [src, src + bytes) is loaded once with
// 16-byte non-temporal loads, four in flight per thread, and folded into an XOR that is stored
// only if it equals an unlikely value (so the loads cannot be dropped and nearly nothing is
// written).
namespace {
typedef unsigned int rd_u32x4 __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) stream_read_k(const rd_u32x4 *__restrict__ src, size_t n16, uint32_t *sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const rd_u32x4 a = __builtin_nontemporal_load(src + i);
    const rd_u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const rd_u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const rd_u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const rd_u32x4 a = __builtin_nontemporal_load(src + i);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (x == 0x9E3779B9u) sink[0] = x;
}
}  // namespace

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st) {
  int dev_id = 0, cus = 256;
  if (hipGetDevice(&dev_id) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev_id);
  const size_t n16 = bytes / 16;
  size_t blocks = (size_t)cus * 8;
  const size_t need = (n16 + 255) / 256;
  if (need < blocks) blocks = need > 0 ? need : 1;
  hipLaunchKernelGGL(stream_read_k, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const rd_u32x4 *>(src), n16, sink);
  return hipGetLastError();
}
}  // namespace qdec
