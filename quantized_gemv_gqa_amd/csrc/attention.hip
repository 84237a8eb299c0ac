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
// How, on CDNA4: a workgroup (8 waves) owns one (KV head, split) pair and serves all G query
// heads of that KV head from registers, so each KV byte is read from HBM once per KV head.  In a
// wave, lane = (slot g = lane / 16, part i = lane % 16): the 16 lanes of a slot read one token's
// row (16 B each for bf16 at D = 128), four slots cover four tokens per load instruction, and a
// 16-lane butterfly finishes each q.k.  Every wave keeps its own online-softmax state; states
// are merged across slots with lane shuffles and across waves in LDS.  There is no barrier
// inside a divergent branch, and the partial last page is masked per token, which is the case
// the H100 runtime's tail-page race corrupted ("Bare-Metal LLM Inference on NVIDIA H100",
// "Challenge 1").
#include <hip/hip_runtime.h>

#include <cmath>

#include "qdec_attention.h"
#include "qdec_batch.h"

namespace qdec {

namespace {

using namespace dev;

template <int D, int G, int KVF, bool ROPE>
__global__ void __launch_bounds__(attn::kAttnThreads) attn_split(AttnArgs a) {
  __shared__ attn::AttnSmem<D, G, ROPE> sm;
  attn::attn_unit<D, G, KVF, ROPE, false>(a, blockIdx.x, blockIdx.y, sm);
}

// grid (Hkv, splits, B): the step form of the unit for sequence b, its pointers offset by b
template <int D, int G, int KVF>
__global__ void __launch_bounds__(attn::kAttnThreads) attn_split_batch(const AttnBatch ab) {
  __shared__ attn::AttnSmem<D, G, true> sm;
  const int b = blockIdx.z;
  const int t = ab.pos[b];
  if (t < 0 || t >= ab.max_blocks * 16) return;  // idle slot, or past its block table: skipped
  AttnArgs a = ab.a;
  a.qkv = ab.qkv + (size_t)b * (a.Hq + 2 * a.Hkv) * D;
  a.rope_cs = ab.rope_cs + (size_t)b * D;
  a.pos = ab.pos + b;
  a.page_table = ab.tables + (size_t)b * ab.max_blocks;
  a.counters = reinterpret_cast<unsigned *>(ab.ws + (size_t)b * ab.ws_stride);
  a.ws = reinterpret_cast<float *>(ab.ws + (size_t)b * ab.ws_stride + kAttnCounterBytes);
  a.out = ab.out + (size_t)b * a.Hq * D;
  attn::attn_unit<D, G, KVF, true, false>(a, blockIdx.x, blockIdx.y, sm);
}

// grid (Hkv, 1, T): query t of a prompt over keys 0 .. pos_rows[t] (one split)
template <int D, int G, int KVF>
__global__ void __launch_bounds__(attn::kAttnThreads) attn_split_rows(const AttnRows r) {
  __shared__ attn::AttnSmem<D, G, false> sm;
  const int t = blockIdx.z;
  AttnArgs a = r.a;
  a.q = r.q + (size_t)t * r.q_stride;
  a.pos = r.pos_rows + t;
  a.counters = reinterpret_cast<unsigned *>(r.ws + (size_t)t * r.ws_stride);
  a.ws = reinterpret_cast<float *>(r.ws + (size_t)t * r.ws_stride + kAttnCounterBytes);
  a.out = r.out + (size_t)t * a.Hq * D;
  attn::attn_unit<D, G, KVF, false, false>(a, blockIdx.x, blockIdx.y, sm);
}

__global__ void kv_append(const float *__restrict__ k, const float *__restrict__ v, void *k_pool,
                          void *v_pool, int kv_fmt, const int32_t *__restrict__ page_table,
                          int n_pages, const int32_t *__restrict__ pos, int Hkv, int D) {
  const int t = *pos;
  if (t < 0 || (t >> 4) >= n_pages) return;
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
  constexpr int kT = attn::kAttnThreads;
  switch (G) {
#define QDEC_G(g)                                                                         \
  case g:                                                                                 \
    if (a.qkv)                                                                            \
      hipLaunchKernelGGL((attn_split<D, g, KVF, true>), grid, dim3(kT), 0, st, a);       \
    else                                                                                  \
      hipLaunchKernelGGL((attn_split<D, g, KVF, false>), grid, dim3(kT), 0, st, a);      \
    break;
    QDEC_G(1) QDEC_G(2) QDEC_G(3) QDEC_G(4) QDEC_G(5) QDEC_G(6) QDEC_G(7) QDEC_G(8)
#undef QDEC_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int KVF>
hipError_t launch_batch_g(const AttnBatch &ab, int G, hipStream_t st) {
  dim3 grid(ab.a.Hkv, ab.a.splits, ab.B);
  constexpr int kT = attn::kAttnThreads;
  switch (G) {
#define QDEC_G(g)                                                                            \
  case g:                                                                                    \
    hipLaunchKernelGGL((attn_split_batch<D, g, KVF>), grid, dim3(kT), 0, st, ab);            \
    break;
    QDEC_G(1) QDEC_G(2) QDEC_G(3) QDEC_G(4) QDEC_G(5) QDEC_G(6) QDEC_G(7) QDEC_G(8)
#undef QDEC_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int KVF>
hipError_t launch_rows_g(const AttnRows &r, int G, hipStream_t st) {
  dim3 grid(r.a.Hkv, r.a.splits, r.T);
  constexpr int kT = attn::kAttnThreads;
  switch (G) {
#define QDEC_G(g)                                                                            \
  case g:                                                                                    \
    hipLaunchKernelGGL((attn_split_rows<D, g, KVF>), grid, dim3(kT), 0, st, r);              \
    break;
    QDEC_G(1) QDEC_G(2) QDEC_G(3) QDEC_G(4) QDEC_G(5) QDEC_G(6) QDEC_G(7) QDEC_G(8)
#undef QDEC_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_rows(const AttnRows &r, hipStream_t st) {
  const int G = r.a.Hq / r.a.Hkv;
  if (r.a.D == 128)
    return r.a.kv_fmt == QDEC_KV_BF16 ? launch_rows_g<128, QDEC_KV_BF16>(r, G, st) : launch_rows_g<128, QDEC_KV_F32>(r, G, st);
  return r.a.kv_fmt == QDEC_KV_BF16 ? launch_rows_g<64, QDEC_KV_BF16>(r, G, st) : launch_rows_g<64, QDEC_KV_F32>(r, G, st);
}

hipError_t launch_attention_batch(const AttnBatch &ab, hipStream_t st) {
  const int G = ab.a.Hq / ab.a.Hkv;
  if (ab.a.D == 128)
    return ab.a.kv_fmt == QDEC_KV_BF16 ? launch_batch_g<128, QDEC_KV_BF16>(ab, G, st)
                                       : launch_batch_g<128, QDEC_KV_F32>(ab, G, st);
  return ab.a.kv_fmt == QDEC_KV_BF16 ? launch_batch_g<64, QDEC_KV_BF16>(ab, G, st)
                                     : launch_batch_g<64, QDEC_KV_F32>(ab, G, st);
}

// [per-KV-head arrival counters, one 128-byte line each, zero between launches]
// [splits][Hq][D] partial outputs, then [splits][Hq][2] partial (max, sum)
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
