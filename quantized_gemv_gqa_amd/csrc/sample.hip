// On-GPU sampling of the next token from the logits: temperature, top-k, top-p, seeded.
//
// What it computes (FlashQwen README, "Local benchmark": the chat flags temperature / top-p /
// top-k / seed; "Optimization study" stage 5: the token is chosen on the GPU, so only one int
// leaves the device; the Naive Qwen engine, "Sampler": greedy takes the largest logit, top-k draws
// among the k most probable tokens).  The pages fix neither the filter order nor the random source;
// the reading (the same in the CPU oracle):
//   temperature <= 0: greedy (largest logit, smallest index on ties);
//   z_i = l_i / T (fp64); top-k (0 < k < V) keeps the k largest logits, smaller index first on
//   equal logits; top-p (p < 1) keeps, in that order, the shortest prefix whose softmax mass
//   (fp64, summed in that order) reaches p of the kept total; the token is the Gumbel-max draw
//   argmax over the kept set of fp32(z_i - ln(-ln u_i)), smallest index on equal keys, with u_i
//   the word i mod 4 of Philox4x64-10 (key (seed, 0), counter (i / 4, step, 0, 0)) mapped to
//   ((word >> 11) + 0.5) 2^-53.
//
// How: two launches.
//   S1, many workgroups over contiguous ranges of the vocabulary: without top-k, each workgroup
//     reduces its range to one (key, index) candidate (greedy: the logit; sampling: the Gumbel
//     key); with top-k, each workgroup selects the exact top-k of its range (8-bit radix select
//     on order-preserving keys, equal keys ranked by index) and writes them in index order.
//   S2, one workgroup: the candidates hold the global answer (the global top-k lies in the union
//     of the ranges' top-k).  It selects the global top-k the same way, sorts it (bitonic, logit
//     descending then index ascending), takes the top-p prefix with one thread summing in order in
//     fp64 (the summation order is the reading's, so the cut is the oracle's), draws the Gumbel
//     keys of the kept tokens and reduces them; then it writes the token and, in the decode step,
//     the token log, step count and position.
// Every decision is a comparison of integers or of values computed as the reading states, so the
// result does not depend on the launch shape or on timing.
#include <hip/hip_runtime.h>

#include <climits>

#include "qdec_device.h"

namespace qdec {

namespace {

using namespace dev;

constexpr int kS1Threads = 256;
constexpr int kS1BlocksFull = 256;  // greedy / full-vocabulary draw: one candidate per block
constexpr int kS1BlocksTopK = 64;   // top-k: k candidates per block
constexpr int kS2Threads = 1024;

struct SampleArgs {
  const float *logits;
  int V;
  float temperature;
  int top_k;  // 0: no top-k filter (then top_p must be 1)
  float top_p;
  uint64_t seed;
  const int32_t *step;  // draw counter (device), null: 0
  int32_t *token;
  // decode-step bookkeeping (null outside the step): token_log[*step_count] = token,
  // *step_count += 1, *pos += 1
  int32_t *token_log, *step_count, *pos;
  int log_len;
  // workspace: candidates (logit or key, index) [blocks][slots], per-block counts
  float *cand_v;
  int32_t *cand_i;
  int32_t *cand_n;
  int blocks, slots;
};

// ------------------------------------------------------------------ Philox4x64-10 and the draw
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t a = c[0], b = c[2];
    const uint64_t hi0 = __umul64hi(0xD2E7470EE14C6C93ull, a), lo0 = 0xD2E7470EE14C6C93ull * a;
    const uint64_t hi1 = __umul64hi(0xCA5A826395121157ull, b), lo1 = 0xCA5A826395121157ull * b;
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += 0x9E3779B97F4A7C15ull;
    k1 += 0xBB67AE8584CAA73Bull;
  }
}

// Gumbel noise -ln(-ln u) for a 64-bit Philox word
__device__ __forceinline__ double gumbel(uint64_t w) {
  const double u = ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0);
  return -log(-log(u));
}

__device__ __forceinline__ float gumbel_key(float l, float T, uint64_t w) {
  return (float)((double)l / (double)T + gumbel(w));
}

// order-preserving 32-bit key of a finite float (-0 and +0 equal; NaN lowest)
__device__ __forceinline__ uint32_t okey(float f) {
  if (f != f) return 0u;
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  if (b == 0x80000000u) b = 0u;  // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// larger value wins, smaller index on equal values; index INT_MAX: none
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  if (i == INT_MAX) return false;
  if (bi == INT_MAX) return true;
  return v > bv || (v == bv && i < bi);
}

template <int NT>
struct RedSmem {
  float v[NT / 64];
  int i[NT / 64];
};

// block (value, index) reduction; every thread returns the result
template <int NT>
__device__ __forceinline__ void block_best(float &v, int &i, RedSmem<NT> &sm) {
  wave_argmax(v, i);  // (treats INT_MAX as "no candidate", same order)
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm.v[w] = v;
    sm.i[w] = i;
  }
  __syncthreads();
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int k = 0; k < NT / 64; ++k)
    if (better(sm.v[k], sm.i[k], bv, bi)) {
      bv = sm.v[k];
      bi = sm.i[k];
    }
  __syncthreads();
  v = bv;
  i = bi;
}

// ------------------------------------------------------------------ block top-k selection
template <int NT>
struct SelSmem {
  unsigned hist[256];
  unsigned wave_cnt[2][NT / 64];
  unsigned bin, above;
};

// The k-th largest key among n elements (key_at(j), j < n; k <= n): tau, and how many of the
// elements equal to tau belong to the top k (krem) out of how many there are (ceq).
template <int NT, class KeyAt>
__device__ void radix_kth(const KeyAt &key_at, int n, int k, SelSmem<NT> &sm, uint32_t &tau, int &krem, int &ceq) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0, mask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += NT) sm.hist[b] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += NT) {
      const uint32_t key = key_at(j);
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane L owns bins 4L .. 4L+3; counts above a bin come from the higher lanes
      const unsigned h0 = sm.hist[4 * lane], h1 = sm.hist[4 * lane + 1], h2 = sm.hist[4 * lane + 2],
                     h3 = sm.hist[4 * lane + 3];
      const unsigned own = h0 + h1 + h2 + h3;
      unsigned suf = own;  // sum over lanes >= this lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned t = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += t;
      }
      const uint64_t bal = __ballot(suf >= (unsigned)need);
      const int L = 63 - __builtin_clzll(bal);  // highest lane whose suffix reaches need
      if (lane == L) {
        unsigned above = suf - own;
        const unsigned hs[4] = {h0, h1, h2, h3};
        int b = 3;
        for (; b > 0; --b) {
          if (above + hs[b] >= (unsigned)need) break;
          above += hs[b];
        }
        sm.bin = 4u * lane + b;
        sm.above = above;
      }
    }
    __syncthreads();
    const uint32_t bin = sm.bin;
    need -= (int)sm.above;
    prefix |= bin << shift;
    mask |= 255u << shift;
    if (shift == 0) ceq = (int)sm.hist[bin];
    __syncthreads();
  }
  tau = prefix;
  krem = need;
}

// Write the selected elements (key > tau, or key == tau among the first krem such elements in
// index order) in index order through emit(position, j); returns the count.
template <int NT, class KeyAt, class Emit>
__device__ int select_ordered(const KeyAt &key_at, int n, uint32_t tau, int krem, SelSmem<NT> &sm, const Emit &emit) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int ties_before = 0, out_before = 0;
  for (int base = 0; base < n; base += NT) {
    const int j = base + tid;
    uint32_t key = 0;
    bool gt = false, eq = false;
    if (j < n) {
      key = key_at(j);
      gt = key > tau;
      eq = key == tau;
    }
    const uint64_t beq = __ballot(eq);
    if (lane == 0) sm.wave_cnt[0][w] = (unsigned)__popcll(beq);
    __syncthreads();
    int tb = ties_before;
    int ties_chunk = 0;
    for (int k = 0; k < NT / 64; ++k) {
      if (k < w) tb += (int)sm.wave_cnt[0][k];
      ties_chunk += (int)sm.wave_cnt[0][k];
    }
    const int rank = tb + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(beq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)beq, 0u));
    const bool sel = gt || (eq && rank < krem);
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) sm.wave_cnt[1][w] = (unsigned)__popcll(bsel);
    __syncthreads();
    int ob = out_before, out_chunk = 0;
    for (int k = 0; k < NT / 64; ++k) {
      if (k < w) ob += (int)sm.wave_cnt[1][k];
      out_chunk += (int)sm.wave_cnt[1][k];
    }
    if (sel) emit(ob + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bsel >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bsel, 0u)), j);
    ties_before += ties_chunk;
    out_before += out_chunk;
    __syncthreads();
  }
  return out_before;
}

// ------------------------------------------------------------------ S1
__global__ void __launch_bounds__(kS1Threads) sample_s1(const SampleArgs a) {
  __shared__ RedSmem<kS1Threads> red;
  __shared__ SelSmem<kS1Threads> sel;
  const int chunk = ((a.V + a.blocks - 1) / a.blocks + 3) & ~3;
  const int start = blockIdx.x * chunk;
  const int n = max(0, min(chunk, a.V - start));
  const float *lg = a.logits + start;
  if (a.top_k > 0) {
    const int k = min(a.top_k, n);
    auto key_at = [&](int j) { return okey(lg[j]); };
    float *cv = a.cand_v + (size_t)blockIdx.x * a.slots;
    int32_t *ci = a.cand_i + (size_t)blockIdx.x * a.slots;
    auto emit = [&](int p, int j) {
      cv[p] = lg[j];
      ci[p] = start + j;
    };
    int cnt = 0;
    if (k > 0) {
      uint32_t tau = 0;
      int krem = 0, ceq = 0;
      if (k < n) {
        radix_kth<kS1Threads>(key_at, n, k, sel, tau, krem, ceq);
      } else {
        krem = n;  // all of them: tau = 0 keeps every key (finite logits have keys > 0)
      }
      cnt = select_ordered<kS1Threads>(key_at, n, tau, krem, sel, emit);
    }
    if (threadIdx.x == 0) a.cand_n[blockIdx.x] = cnt;
    return;
  }
  // one candidate per block: greedy (logit) or Gumbel key
  const bool greedy = !(a.temperature > 0.f);
  const uint64_t step = a.step ? (uint64_t)(int64_t)*a.step : 0ull;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int q = threadIdx.x * 4; q < n; q += kS1Threads * 4) {
    const int i0 = start + q;  // multiple of 4
    uint64_t c[4] = {(uint64_t)(i0 >> 2), step, 0ull, 0ull};
    if (!greedy) philox4x64_10(c, a.seed, 0ull);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (q + e >= n) break;
      const float l = lg[q + e];
      if (l != l) continue;
      const float v = greedy ? l : gumbel_key(l, a.temperature, c[e]);
      if (better(v, i0 + e, bv, bi)) {
        bv = v;
        bi = i0 + e;
      }
    }
  }
  block_best<kS1Threads>(bv, bi, red);
  if (threadIdx.x == 0) {
    a.cand_v[blockIdx.x] = bv;
    a.cand_i[blockIdx.x] = bi;
  }
}

// ------------------------------------------------------------------ S2
struct S2Smem {
  SelSmem<kS2Threads> sel;
  RedSmem<kS2Threads> red;
  float lv[kSampleMaxTopK];
  int li[kSampleMaxTopK];
  int n_keep;
};

__device__ __forceinline__ void finish(const SampleArgs &a, int tok) {
  *a.token = tok;
  if (a.step_count) {
    const int stc = *a.step_count;
    if (a.token_log && stc >= 0 && stc < a.log_len) a.token_log[stc] = tok;
    *a.step_count = stc + 1;
  }
  if (a.pos) *a.pos += 1;
}

__global__ void __launch_bounds__(kS2Threads) sample_s2(const SampleArgs a) {
  __shared__ S2Smem sm;
  const int tid = threadIdx.x;
  if (a.top_k <= 0) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int b = tid; b < a.blocks; b += kS2Threads)
      if (better(a.cand_v[b], a.cand_i[b], bv, bi)) {
        bv = a.cand_v[b];
        bi = a.cand_i[b];
      }
    block_best<kS2Threads>(bv, bi, sm.red);
    if (tid == 0) finish(a, bi == INT_MAX ? 0 : bi);
    return;
  }
  // candidates: block b's count at cand_n[b], slots b * slots .. ; ordered by token index
  const int slots = a.slots;
  const int total = a.blocks * slots;
  auto valid = [&](int c) { return (c % slots) < a.cand_n[c / slots]; };
  auto key_at = [&](int c) { return valid(c) ? okey(a.cand_v[c]) : 0u; };
  int nvalid = 0;
  for (int b = 0; b < a.blocks; ++b) nvalid += a.cand_n[b];
  const int k = min(a.top_k, nvalid);
  uint32_t tau = 0;
  int krem = nvalid, ceq = 0;
  if (k < nvalid) radix_kth<kS2Threads>(key_at, total, k, sm.sel, tau, krem, ceq);
  auto emit = [&](int p, int c) {
    sm.lv[p] = a.cand_v[c];
    sm.li[p] = a.cand_i[c];
  };
  // invalid slots have key 0, below every finite logit's, so tau > 0 never selects them
  int n = 0;
  if (k < nvalid) {
    n = select_ordered<kS2Threads>(key_at, total, tau, krem, sm.sel, emit);
  } else {
    // every valid candidate is kept
    auto all_at = [&](int c) { return valid(c) ? 1u : 0u; };
    n = select_ordered<kS2Threads>(all_at, total, 0u, 0, sm.sel, emit);
  }
  // bitonic sort of the n <= kSampleMaxTopK selected: logit descending, index ascending
  int np = 1;
  while (np < n) np <<= 1;
  for (int p = n + tid; p < np; p += kS2Threads) {
    sm.lv[p] = -INFINITY;
    sm.li[p] = INT_MAX;
  }
  __syncthreads();
  for (int size = 2; size <= np; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < np / 2; t += kS2Threads) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;  // this half sorts "best first"
        const float va = sm.lv[lo], vb = sm.lv[hi];
        const int ia = sm.li[lo], ib = sm.li[hi];
        const bool b_first = better(vb, ib, va, ia);
        if (b_first == up) {
          sm.lv[lo] = vb;
          sm.li[lo] = ib;
          sm.lv[hi] = va;
          sm.li[hi] = ia;
        }
      }
      __syncthreads();
    }
  }
  // top-p: the shortest prefix whose mass reaches p of the total, summed in order in fp64
  if (tid == 0) {
    int keep = n;
    if (a.top_p < 1.0f && n > 0) {
      const double T = (double)a.temperature, zmax = (double)sm.lv[0] / T;
      double tot = 0.0;
      for (int j = 0; j < n; ++j) tot += exp((double)sm.lv[j] / T - zmax);
      double cum = 0.0;
      for (int j = 0; j < n; ++j) {
        cum += exp((double)sm.lv[j] / T - zmax);
        if (cum >= (double)a.top_p * tot) {
          keep = j + 1;
          break;
        }
      }
    }
    sm.n_keep = keep;
  }
  __syncthreads();
  const int keep = sm.n_keep;
  const uint64_t step = a.step ? (uint64_t)(int64_t)*a.step : 0ull;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int j = tid; j < keep; j += kS2Threads) {
    const int i = sm.li[j];
    uint64_t c[4] = {(uint64_t)(i >> 2), step, 0ull, 0ull};
    philox4x64_10(c, a.seed, 0ull);
    const float v = gumbel_key(sm.lv[j], a.temperature, c[i & 3]);
    if (better(v, i, bv, bi)) {
      bv = v;
      bi = i;
    }
  }
  block_best<kS2Threads>(bv, bi, sm.red);
  if (tid == 0) finish(a, bi == INT_MAX ? 0 : bi);
}

}  // namespace

size_t sample_workspace_bytes() {
  return (size_t)kS1BlocksFull * kSampleMaxTopK * 8 + (size_t)kS1BlocksFull * 4 + 256;
}

hipError_t launch_sample(const float *logits, int V, float temperature, int top_k, float top_p, uint64_t seed,
                         const int32_t *step, int32_t *token, int32_t *token_log, int32_t *step_count, int32_t *pos,
                         int log_len, void *ws, hipStream_t st) {
  SampleArgs a{};
  a.logits = logits;
  a.V = V;
  a.temperature = temperature;
  // top-k path when it filters, or when top-p needs the sorted set (then top_k >= V keeps all V)
  const bool sampling = temperature > 0.f;
  a.top_k = 0;
  if (sampling && top_k > 0 && (top_k < V || top_p < 1.0f)) a.top_k = top_k < V ? top_k : V;
  a.top_p = top_p;
  a.seed = seed;
  a.step = step;
  a.token = token;
  a.token_log = token_log;
  a.step_count = step_count;
  a.pos = pos;
  a.log_len = log_len;
  a.blocks = a.top_k > 0 ? kS1BlocksTopK : kS1BlocksFull;
  a.slots = a.top_k > 0 ? a.top_k : 1;
  // workspace: values [blocks * slots] floats, indices, counts
  char *w = reinterpret_cast<char *>(ws);
  a.cand_v = reinterpret_cast<float *>(w);
  a.cand_i = reinterpret_cast<int32_t *>(w + (size_t)kS1BlocksFull * kSampleMaxTopK * 4);
  a.cand_n = reinterpret_cast<int32_t *>(w + (size_t)kS1BlocksFull * kSampleMaxTopK * 8);
  hipLaunchKernelGGL(sample_s1, dim3(a.blocks), dim3(kS1Threads), 0, st, a);
  hipLaunchKernelGGL(sample_s2, dim3(1), dim3(kS2Threads), 0, st, a);
  return hipGetLastError();
}

}  // namespace qdec
