// Split-K (flash-decoding) paged GQA decode attention for gfx950.
//
// What it computes (one new token): for query head h and its KV head j = h / G, G = Hq / Hkv,
//   out[h] = sum_t softmax_t(q_h . k_{j,t} * scale) v_{j,t},  t = 0 .. pos,
// with token t stored in 16-token pages found through a page table ("Chapter 2 Systems
// Foundations for LLMs", "PagedAttention - Virtual Memory for KV Caches"; 16-token pages with a
// contiguous per-KV-head slice: "How To Construct Your Personal LLM Runtime From Scratch",
// section 3).  The key range is cut into splits, each reduced with an online softmax by its own
// workgroup, and a second pass merges the partial (max, sum, output) triples (FlashQwen README,
// "Optimization study", stage 7).
//
// How, on CDNA4: a workgroup (4 waves) owns one (KV head, split) pair and serves all G query
// heads of that KV head from registers, so each KV byte is read from HBM once per KV head.  In a
// wave, lane = (slot g = lane / 16, part i = lane % 16): the 16 lanes of a slot read one token's
// row (16 B each for bf16 at D = 128), four slots cover four tokens per load instruction, and a
// 16-lane butterfly finishes each q.k.  Every wave keeps its own online-softmax state; states
// are merged across slots with lane shuffles and across waves in LDS.  There is no barrier
// inside a divergent branch, and the partial last page is masked per token, which is the case
// the H100 runtime's tail-page race corrupted ("Bare-Metal LLM Inference on NVIDIA H100",
// "Challenge 1").
#include <hip/hip_runtime.h>

#include "qdec_internal.h"

namespace qdec {

namespace {

constexpr float kNegBig = -1e30f;  // finite "minus infinity" for running maxima
constexpr int kAuxSc1 = 16;        // sc1: device-coherent load (bypasses non-coherent L2 copies)

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x7FFFFFu)) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

template <int D, int KVF>
struct RowLoad {
  static constexpr int DPL = D / 16;  // elements per lane
  // load DPL elements of a token row starting at element e0
  __device__ __forceinline__ static void load(const void *pool, size_t e0, float (&r)[DPL]) {
    if constexpr (KVF == QDEC_KV_BF16) {
      const uint16_t *p = reinterpret_cast<const uint16_t *>(pool) + e0;
      if constexpr (DPL == 8) {
        const uint4 v = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          r[2 * i] = __builtin_bit_cast(float, w[i] << 16);
          r[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
        }
      } else {
        static_assert(DPL == 4, "head_dim 64 or 128");
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        const uint32_t w[2] = {v.x, v.y};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          r[2 * i] = __builtin_bit_cast(float, w[i] << 16);
          r[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
        }
      }
    } else {
      const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(pool) + e0);
#pragma unroll
      for (int i = 0; i < DPL / 4; ++i) {
        const float4 v = p[i];
        r[4 * i] = v.x; r[4 * i + 1] = v.y; r[4 * i + 2] = v.z; r[4 * i + 3] = v.w;
      }
    }
  }
};

__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

template <int D, int G, int KVF>
__global__ void __launch_bounds__(256) attn_split(AttnArgs a) {
  constexpr int DPL = D / 16;
  __shared__ float sm_m[4][G], sm_l[4][G], sm_o[4][G][D];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = lane >> 4;
  const int part = lane & 15;
  const int j = blockIdx.x;
  const int s = blockIdx.y;
  const int T = *a.pos + 1;
  const int P = min((T + 15) >> 4, a.n_pages);  // never index past the page table
  const int pps = (P + a.splits - 1) / a.splits;
  const int p0 = s * pps;
  const int p1 = min(P, p0 + pps);

  float q[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) q[h][e] = a.q[(size_t)(j * G + h) * D + part * DPL + e] * a.scale_log2;

  float m[G], l[G], o[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] = 0.f;
  }

  const size_t head_stride = (size_t)16 * D;  // elements of one head's slice of a page
  for (int p = p0 + wave; p < p1; p += 4) {
    const int phys = a.page_table[p];
    if (phys < 0 || phys >= a.n_pages) continue;  // documented precondition; never read outside
    const size_t base = ((size_t)phys * a.Hkv + j) * head_stride;
    // all K and V rows this lane needs from the page, issued before any is used
    float kr[4][DPL], vr[4][DPL];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const size_t e = base + (size_t)(sub * 4 + slot) * D + part * DPL;
      RowLoad<D, KVF>::load(a.k_pool, e, kr[sub]);
      RowLoad<D, KVF>::load(a.v_pool, e, vr[sub]);
    }
    float sc[4][G];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const bool valid = p * 16 + sub * 4 + slot < T;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) d = fmaf(q[h][e], kr[sub][e], d);
        d = sum16(d);
        sc[sub][h] = valid ? d : -INFINITY;
      }
      // slots past the newest token may hold stale bits (even NaN): select them away, never
      // multiply them by a zero weight
#pragma unroll
      for (int e = 0; e < DPL; ++e) vr[sub][e] = valid ? vr[sub][e] : 0.f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mx = fmaxf(fmaxf(m[h], fmaxf(sc[0][h], sc[1][h])), fmaxf(sc[2][h], sc[3][h]));
      const float alpha = exp2f(m[h] - mx);
      m[h] = mx;
      float pr[4];
      float ls = 0.f;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        pr[sub] = exp2f(sc[sub][h] - mx);
        ls += pr[sub];
      }
      l[h] = fmaf(l[h], alpha, ls);
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        float acc = o[h][e] * alpha;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) acc = fmaf(pr[sub], vr[sub][e], acc);
        o[h][e] = acc;
      }
    }
  }

  // merge the four token slots of this wave (lanes part, part+16, part+32, part+48)
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float m2 = __shfl_xor(m[h], off, 64);
      const float l2 = __shfl_xor(l[h], off, 64);
      const float mx = fmaxf(m[h], m2);
      const float a1 = exp2f(m[h] - mx), a2 = exp2f(m2 - mx);
      l[h] = l[h] * a1 + l2 * a2;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float o2 = __shfl_xor(o[h][e], off, 64);
        o[h][e] = o[h][e] * a1 + o2 * a2;
      }
      m[h] = mx;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) sm_o[wave][h][part * DPL + e] = o[h][e];
      if (part == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  // merge the four waves and publish the split's partial (o, m, l) for each query head through
  // device-coherent stores (the merging block may sit on another XCD)
  float *wsj = a.ws + (size_t)j * G * (D + 2);  // head h of split s at wsj + s * Hq * (D+2) + h * (D+2)
  const size_t sstride = (size_t)a.Hq * (D + 2);
  for (int idx = threadIdx.x; idx < G * (D + 2); idx += 256) {
    const int h = idx / (D + 2);
    const int d = idx - h * (D + 2);
    float mx = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, sm_m[w][h]);
    float val = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = exp2f(sm_m[w][h] - mx);
      val += f * (d < D ? sm_o[w][h][d] : (d == D + 1 ? sm_l[w][h] : 0.f));
    }
    if (d == D) val = mx;
    __hip_atomic_store(wsj + s * sstride + idx, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are acknowledged
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  __shared__ unsigned last;
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&a.counters[j], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (unsigned)(a.splits - 1);
  __syncthreads();
  if (!last) return;

  // The last split block of KV head j merges all splits of its G query heads:
  //   out[h][d] = sum_s 2^(m_s - M) o_s[d] / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
  // Splits without keys carry m = -1e30, l = 0, o = 0 and get weight 0.
  __shared__ float sw[kMaxMergeSplits][G];
  __shared__ float sM[G], sL[G];
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc(wsj, (short)0, (int)(a.splits * sstride * 4), 0x00020000);
  for (int idx = threadIdx.x; idx < a.splits * G; idx += 256) {
    const int ss = idx / G, h = idx - ss * G;
    sw[ss][h] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    wr, (h * (D + 2) + D) * 4, (int)(ss * sstride * 4), kAuxSc1));
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = kNegBig;
    for (int ss = 0; ss < a.splits; ++ss) M = fmaxf(M, sw[ss][h]);
    sM[h] = M;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.splits * G; idx += 256) {
    const int ss = idx / G, h = idx - ss * G;
    sw[ss][h] = exp2f(sw[ss][h] - sM[h]);
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float L = 0.f;
    for (int ss = 0; ss < a.splits; ++ss)
      L = fmaf(sw[ss][h], __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                              wr, (h * (D + 2) + D + 1) * 4, (int)(ss * sstride * 4), kAuxSc1)), L);
    sL[h] = L;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx - h * D;
    float O = 0.f;
    int ss = 0;
    for (; ss + 8 <= a.splits; ss += 8) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        t[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                   wr, (h * (D + 2) + d) * 4, (int)((ss + u) * sstride * 4), kAuxSc1));
#pragma unroll
      for (int u = 0; u < 8; ++u) O = fmaf(sw[ss + u][h], t[u], O);
    }
    for (; ss < a.splits; ++ss)
      O = fmaf(sw[ss][h], __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                              wr, (h * (D + 2) + d) * 4, (int)(ss * sstride * 4), kAuxSc1)), O);
    a.out[(size_t)(j * G + h) * D + d] = O / sL[h];
  }
  if (threadIdx.x == 0) __hip_atomic_store(&a.counters[j], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void kv_append(const float *__restrict__ k, const float *__restrict__ v, void *k_pool,
                          void *v_pool, int kv_fmt, const int32_t *__restrict__ page_table,
                          int n_pages, const int32_t *__restrict__ pos, int Hkv, int D) {
  const int t = *pos;
  const int phys = page_table[t >> 4];
  if (phys < 0 || phys >= n_pages) return;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < Hkv * D; i += gridDim.x * blockDim.x) {
    const int j = i / D, d = i - j * D;
    const size_t e = (((size_t)phys * Hkv + j) * 16 + (t & 15)) * D + d;
    if (kv_fmt == QDEC_KV_BF16) {
      reinterpret_cast<uint16_t *>(k_pool)[e] = float_to_bf16_rne(k[i]);
      reinterpret_cast<uint16_t *>(v_pool)[e] = float_to_bf16_rne(v[i]);
    } else {
      reinterpret_cast<float *>(k_pool)[e] = k[i];
      reinterpret_cast<float *>(v_pool)[e] = v[i];
    }
  }
}

template <int D, int KVF>
hipError_t launch_g(const AttnArgs &a, int G, hipStream_t st) {
  dim3 grid(a.Hkv, a.splits);
  switch (G) {
#define QDEC_G(g) \
  case g: hipLaunchKernelGGL((attn_split<D, g, KVF>), grid, dim3(256), 0, st, a); break;
    QDEC_G(1) QDEC_G(2) QDEC_G(3) QDEC_G(4) QDEC_G(5) QDEC_G(6) QDEC_G(7) QDEC_G(8)
#undef QDEC_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// [256 B of per-KV-head arrival counters, zero between launches][splits][Hq][D + 2] partials
size_t attn_workspace_bytes(int Hq, int D, int splits) {
  return kAttnCounterBytes + (size_t)splits * Hq * (D + 2) * sizeof(float);
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  hipError_t e;
  if (a.D == 128)
    e = a.kv_fmt == QDEC_KV_BF16 ? launch_g<128, QDEC_KV_BF16>(a, G, st) : launch_g<128, QDEC_KV_F32>(a, G, st);
  else
    e = a.kv_fmt == QDEC_KV_BF16 ? launch_g<64, QDEC_KV_BF16>(a, G, st) : launch_g<64, QDEC_KV_F32>(a, G, st);
  return e;
}

hipError_t launch_kv_append(const float *k, const float *v, void *k_pool, void *v_pool, int kv_fmt,
                            const int32_t *page_table, int n_pages, const int32_t *pos, int Hkv,
                            int D, hipStream_t st) {
  const int n = Hkv * D;
  hipLaunchKernelGGL(kv_append, dim3((n + 255) / 256), dim3(256), 0, st, k, v, k_pool, v_pool, kv_fmt,
                     page_table, n_pages, pos, Hkv, D);
  return hipGetLastError();
}

}  // namespace qdec
