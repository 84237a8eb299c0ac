// Persistent decode-step kernel: the whole batch-1 decode step of a Qwen-style GQA decoder in one
// launch of co-resident workgroups on gfx950.
//
// Why: at batch 1 every weight byte is read once per token, so the step is an HBM stream of a
// few GB split into ~140 dependent phases (per layer: fused qkv GEMV -> paged attention -> o GEMV
// -> gate/up GEMV + SwiGLU -> down GEMV; then the lm head and greedy argmax).  Launched as one
// kernel per phase, each launch pays a fixed dispatch/drain cost comparable to a small GEMV's
// whole HBM time (FlashQwen README, "Optimization study", stage 6, and the H100 runtime post,
// section 6, make the same point about per-kernel launch cost; there a captured graph was the
// answer).  Here the phases run back to back inside one kernel:
//   * work is statically assigned: GEMV units (64-row tile, k-split) go to waves round-robin,
//     attention units (KV head, split) go to workgroups round-robin;
//   * phase order is enforced with per-phase "done" counters in device-coherent memory: the
//     finishing wave of each GEMV tile (and the merging workgroup of each KV head) counts it,
//     consumers poll the producer's counter (bounded spin, error flag on timeout);
//   * before it polls, a wave already requests its first batch of weights (or KV pages) for the
//     next unit, so the dependency latency overlaps the HBM stream;
//   * data that crosses workgroups (activations, residual stream, KV of the new token, split
//     partials) moves through sc1 (device-coherent) stores and loads; weights stream with nt.
// Co-residency of all workgroups is guaranteed by a cooperative launch.
#include <hip/hip_runtime.h>

#include <cmath>

#include "qdec_device.h"
#include "qdec_fused.h"

namespace qdec {
namespace {

using namespace dev;

template <int D, int G>
struct AttnSmem {
  float m[4][G], l[4][G], o[4][G][D];
  float w[kMaxMergeSplits][G];
  float M[G], L[G];
  unsigned last;
};

// Separate regions, not a union: the waves of a workgroup run GEMV units independently and
// may be in different phases at the same time.
template <int CK, int D, int G>
struct FusedSmem {
  Stage<CK> st[4];
  AttnSmem<D, G> at;
};

// bf16 KV row piece of one lane: 8 values (D = 128) at byte offset `off` of the pool;
// coherent: sc1 load (rows written earlier in this kernel by another workgroup)
__device__ __forceinline__ void load_row8(__amdgpu_buffer_rsrc_t pool, uint32_t off, float (&r)[8], bool coherent) {
  const u32x4 v = coherent ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(pool, off, 0, kAuxSc1))
                           : __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(pool, off, 0, 0));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = __builtin_bit_cast(float, v[i] << 16);
    r[2 * i + 1] = __builtin_bit_cast(float, v[i] & 0xFFFF0000u);
  }
}

// 8 consecutive fp32 values written earlier in this kernel (sc1 buffer loads, pipelined)
__device__ __forceinline__ void load8_coh(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[8]) {
  const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxSc1));
  const f32x4 b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kAuxSc1));
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

typedef double f64x2 __attribute__((ext_vector_type(2)));

// Normalise (optional) and rotate one head vector held 8 dims per lane (lanes `part` of a 16-lane
// slot group hold dims part*8 .. part*8+7).  `own` are the lane's dims, `mate` the dims D/2 away.
// cs: fp64 (cos, sin) of the lane's 8 rotation pairs (computed once per step).
__device__ __forceinline__ void norm_rope8(float (&own)[8], float (&mate)[8], int part, const float *gamma,
                                           float eps, const double (&cs)[16]) {
  constexpr int D = 128, HALF = 64;
  const int d0 = part * 8;
  const bool lo = d0 < HALF;
  if (gamma) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(own[e], own[e], ss);
    ss = sum16(ss);
    const float r = rsqrtf(ss / (float)D + eps);
    const int dm = lo ? d0 + HALF : d0 - HALF;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      own[e] = gamma[d0 + e] * (own[e] * r);
      mate[e] = gamma[dm + e] * (mate[e] * r);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double c = cs[2 * e], s = cs[2 * e + 1];
    const double a = own[e], b = mate[e];
    // low half: a' = a c - b s (b = x[i + D/2]); high half: a' = a c + b s (b = x[i - D/2])
    own[e] = (float)(lo ? (a * c - b * s) : (a * c + b * s));
  }
}

// Attention work unit (KV head j, split s) executed by a whole workgroup (4 waves).
template <int G>
__device__ void attn_unit(const FusedArgs &a, const FusedLayer &Lw, int j, int s, int pos,
                          AttnSmem<128, G> &sm, const unsigned *prog, unsigned prog_target,
                          unsigned *done_att, unsigned att_phase) {
  constexpr int D = 128, DPL = 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = lane >> 4;
  const int part = lane & 15;
  const int T = pos + 1;
  const int P = (T + 15) >> 4;
  const int pps = (P + a.splits - 1) / a.splits;
  const int p0 = s * pps;
  const int p1 = min(P, p0 + pps);
  const int last_page = P - 1;
  const uint32_t pool_bytes = (uint32_t)((size_t)a.n_pages * a.Hkv * 16 * D * 2);
  const __amdgpu_buffer_rsrc_t kpool = rsrc(Lw.k_pool, pool_bytes);
  const __amdgpu_buffer_rsrc_t vpool = rsrc(Lw.v_pool, pool_bytes);
  const __amdgpu_buffer_rsrc_t qkvr = rsrc(a.qkv, (uint32_t)((a.Hq + 2 * a.Hkv) * D * 4));
  const size_t head_stride = (size_t)16 * D;

  // prefetch the wave's first page unless it is the one the new token lands in
  float kr[4][DPL], vr[4][DPL];
  int pf = p0 + wave;
  bool have = false;
  int phys_pf = -1;
  if (pf < p1 && pf != last_page) {
    phys_pf = a.page_table[pf];
    if (phys_pf >= 0 && phys_pf < a.n_pages) {
      const size_t base = ((size_t)phys_pf * a.Hkv + j) * head_stride;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const uint32_t e = (uint32_t)((base + (size_t)(sub * 4 + slot) * D + part * DPL) * 2);
        load_row8(kpool, e, kr[sub], false);
        load_row8(vpool, e, vr[sub], false);
      }
      have = true;
    }
  }

  const bool ok = wait_counter(prog, prog_target, a.err);

  // q of the G query heads: normalised (Qwen3), rotated, scaled into the log2 domain
  float q[G][DPL];
  // the step's (cos, sin) table was written by another workgroup of this kernel: the lane's 8
  // rotation pairs come through device-coherent loads
  double cs[16];
  {
    const __amdgpu_buffer_rsrc_t cr = rsrc(a.rope_cs, 64 * 16);
    const int i0 = part * DPL < 64 ? part * DPL : part * DPL - 64;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f64x2 v = __builtin_bit_cast(f64x2, __builtin_amdgcn_raw_buffer_load_b128(cr, (i0 + e) * 16, 0, kAuxSc1));
      cs[2 * e] = v.x;
      cs[2 * e + 1] = v.y;
    }
  }
  const int dmate = part * DPL < 64 ? part * DPL + 64 : part * DPL - 64;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float own[8], mate[8];
    const uint32_t qoff = (uint32_t)((j * G + h) * D) * 4;
    load8_coh(qkvr, qoff + part * DPL * 4, own);
    load8_coh(qkvr, qoff + dmate * 4, mate);
    norm_rope8(own, mate, part, Lw.g_q, a.eps, cs);
#pragma unroll
    for (int e = 0; e < DPL; ++e) q[h][e] = own[e] * a.scale_log2;
  }

  // the split that owns the last page appends the new token's k (normalised, rotated) and v
  const bool mine_last = p0 <= last_page && last_page < p1;
  if (mine_last && ok && wave == 0 && slot == 0) {
    float own[8], mate[8], vv[8];
    const uint32_t koff = (uint32_t)((a.Hq + j) * D) * 4, voff = (uint32_t)((a.Hq + a.Hkv + j) * D) * 4;
    load8_coh(qkvr, koff + part * DPL * 4, own);
    load8_coh(qkvr, koff + dmate * 4, mate);
    load8_coh(qkvr, voff + part * DPL * 4, vv);
    norm_rope8(own, mate, part, Lw.g_k, a.eps, cs);
    const int phys = a.page_table[last_page];
    if (phys >= 0 && phys < a.n_pages) {
      const size_t e0 = (((size_t)phys * a.Hkv + j) * 16 + (pos & 15)) * D + part * DPL;
      uint32_t *kd = reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(Lw.k_pool) + e0);
      uint32_t *vd = reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(Lw.v_pool) + e0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kw = (uint32_t)float_to_bf16_rne(own[2 * e]) | ((uint32_t)float_to_bf16_rne(own[2 * e + 1]) << 16);
        const uint32_t vw = (uint32_t)float_to_bf16_rne(vv[2 * e]) | ((uint32_t)float_to_bf16_rne(vv[2 * e + 1]) << 16);
        __hip_atomic_store(kd + e, kw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(vd + e, vw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    drain_stores();
  }
  __syncthreads();  // the appended row is acknowledged before any wave reads the last page

  float m[G], l[G], o[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] = 0.f;
  }
  for (int p = p0 + wave; p < p1 && ok; p += 4) {
    if (!(have && p == pf)) {
      const int phys = a.page_table[p];
      if (phys < 0 || phys >= a.n_pages) continue;  // documented precondition; never read outside
      const size_t base = ((size_t)phys * a.Hkv + j) * head_stride;
      const bool coh = p == last_page;  // rows written by this step must bypass stale L2 copies
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const uint32_t e = (uint32_t)((base + (size_t)(sub * 4 + slot) * D + part * DPL) * 2);
        load_row8(kpool, e, kr[sub], coh);
        load_row8(vpool, e, vr[sub], coh);
      }
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
  // merge the four token slots of the wave
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
      for (int e = 0; e < DPL; ++e) sm.o[wave][h][part * DPL + e] = o[h][e];
      if (part == 0) {
        sm.m[wave][h] = m[h];
        sm.l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  // publish the split's (o, m, l) per query head
  float *wsj = a.attn_ws + (size_t)j * G * (D + 2);
  const size_t sstride = (size_t)a.Hq * (D + 2);
  for (int idx = threadIdx.x; idx < G * (D + 2); idx += 256) {
    const int h = idx / (D + 2);
    const int d = idx - h * (D + 2);
    float mx = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, sm.m[w][h]);
    float val = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = exp2f(sm.m[w][h] - mx);
      val += f * (d < D ? sm.o[w][h][d] : (d == D + 1 ? sm.l[w][h] : 0.f));
    }
    if (d == D) val = mx;
    __hip_atomic_store(wsj + s * sstride + idx, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    sm.last = __hip_atomic_fetch_add(&a.attn_cnt[j], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(a.splits - 1);
  __syncthreads();
  if (!sm.last) return;

  // the last split of KV head j merges the splits of its G query heads
  const __amdgpu_buffer_rsrc_t wr = rsrc(wsj, (uint32_t)(a.splits * sstride * 4));
  for (int idx = threadIdx.x; idx < a.splits * G; idx += 256) {
    const int ss = idx / G, h = idx - ss * G;
    sm.w[ss][h] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                      wr, (h * (D + 2) + D) * 4, (int)(ss * sstride * 4), kAuxSc1));
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = kNegBig;
    for (int ss = 0; ss < a.splits; ++ss) M = fmaxf(M, sm.w[ss][h]);
    sm.M[h] = M;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.splits * G; idx += 256) {
    const int ss = idx / G, h = idx - ss * G;
    sm.w[ss][h] = exp2f(sm.w[ss][h] - sm.M[h]);
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float Lsum = 0.f;
    for (int ss = 0; ss < a.splits; ++ss)
      Lsum = fmaf(sm.w[ss][h], __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                   wr, (h * (D + 2) + D + 1) * 4, (int)(ss * sstride * 4), kAuxSc1)), Lsum);
    sm.L[h] = Lsum;
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
      for (int u = 0; u < 8; ++u) O = fmaf(sm.w[ss + u][h], t[u], O);
    }
    for (; ss < a.splits; ++ss)
      O = fmaf(sm.w[ss][h], __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                wr, (h * (D + 2) + d) * 4, (int)(ss * sstride * 4), kAuxSc1)), O);
    st_f<true>(a.attn + (size_t)(j * G + h) * D + d, O / sm.L[h]);
  }
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(&a.attn_cnt[j], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x < 64) count_done(done_att, (unsigned)a.Hkv, att_phase, a.progress, threadIdx.x, a.phase_ts);
}

template <int FMT, int G>
__global__ void __launch_bounds__(256, 2) decode_step_fused(const FusedArgs a) {
  constexpr int CK = (FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16;
  __shared__ FusedSmem<CK, 128, G> sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * 4 + wave;
  const int NW = gridDim.x * 4;
  const int L = a.L;
  const int pos = __builtin_amdgcn_readfirstlane(*a.pos);
  if (pos < 0 || pos >= a.n_pages * 16) {  // no page for the new token: report, touch nothing
    if (threadIdx.x == 0) __hip_atomic_store(a.err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  unsigned *const done = a.done;  // [0]: embed, [1 + 5l + k]: layer l phase k, [1 + 5L]: lm head
  if (a.phase_ts && gw == 0 && lane == 0) a.phase_ts[0] = wall_clock64();

  // ---------------------------------------------------------------- embedding + RoPE table
  const int ntiles_h = (a.H + 63) / 64;
  if (gw < ntiles_h) {
    const int tok = (int)__builtin_bit_cast(unsigned, ld_f<true>(reinterpret_cast<const float *>(a.token)));
    const int t = (tok < 0 || tok >= a.V) ? 0 : tok;
    const int i = gw * 64 + lane;
    float v = 0.f;
    if (i < a.H) {
      v = __builtin_bit_cast(float, (uint32_t)a.embed[(size_t)t * a.H + i] << 16);
      st_f<true>(a.hidden + i, v);
      if (a.trace) a.trace[i] = v;
    }
    const float sq = wave_sum(v * v);
    if (lane == 0) st_f<true>(a.ssq + gw, sq);
    count_done(&done[0], (unsigned)ntiles_h + 1, 0u, a.progress, lane, a.phase_ts);
  } else if (gw == ntiles_h) {
    // fp64 (cos, sin) of pos * base^(-2i/D) for the D/2 rotation pairs of this step
    if (lane < 64) {
      const double theta = pow((double)a.rope_base, -2.0 * (double)lane / 128.0);
      double sn, cs;
      sincos((double)pos * theta, &sn, &cs);
      __hip_atomic_store(&a.rope_cs[2 * lane], cs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.rope_cs[2 * lane + 1], sn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    count_done(&done[0], (unsigned)ntiles_h + 1, 0u, a.progress, lane, a.phase_ts);
  }

  // this workgroup's replica of the "phases completed" value; phase k is done when it is > k
  const unsigned *prog = a.progress + (blockIdx.x % kProgressReplicas) * 32;
  for (int l = 0; l < L; ++l) {
    const FusedLayer &Lw = a.layers[l];
    const unsigned ph = 1 + 5 * l;  // phase index of this layer's qkv GEMV
    unsigned *d_qkv = &done[ph];
    // qkv GEMV (RMSNorm prologue, bias)
    {
      GemvArgs g = a.g_qkv;
      g.W = Lw.w_qkv; g.S = Lw.s_qkv; g.gamma = Lw.g_attn; g.bias = Lw.b_qkv;
      g.done = d_qkv; g.done_target = a.p_qkv.tiles; g.done_phase = ph; g.progress = a.progress; g.phase_ts = a.phase_ts;
      const int units = a.p_qkv.tiles * a.p_qkv.ks;
      for (int u = gw; u < units; u += NW)
        gemv_unit<FMT, true, EPI_STORE, true>(g, u, sm.st[wave], lane, prog, ph, a.err);
    }
    // attention (q/k norm, RoPE, KV append, split partials, merge)
    {
      const int units = a.Hkv * a.splits;
      for (int u = blockIdx.x; u < units; u += gridDim.x) {
        const int j = u / a.splits, s = u - j * a.splits;
        attn_unit<G>(a, Lw, j, s, pos, sm.at, prog, ph + 1, &done[ph + 1], ph + 1);
        __syncthreads();  // the attention scratch is reused by the next unit
      }
    }
    // o GEMV + residual (updates the residual stream and its per-tile sums of squares)
    {
      GemvArgs g = a.g_o;
      g.W = Lw.w_o; g.S = Lw.s_o;
      g.done = &done[ph + 2]; g.done_target = a.p_o.tiles; g.done_phase = ph + 2; g.progress = a.progress; g.phase_ts = a.phase_ts;
      const int units = a.p_o.tiles * a.p_o.ks;
      for (int u = gw; u < units; u += NW)
        gemv_unit<FMT, false, EPI_STORE, true>(g, u, sm.st[wave], lane, prog, ph + 2, a.err);
    }
    // gate/up GEMV (RMSNorm prologue) + SwiGLU
    {
      GemvArgs g = a.g_gu;
      g.W = Lw.w_gu; g.S = Lw.s_gu; g.gamma = Lw.g_ffn;
      g.done = &done[ph + 3]; g.done_target = a.p_gu.tiles; g.done_phase = ph + 3; g.progress = a.progress; g.phase_ts = a.phase_ts;
      const int units = a.p_gu.tiles * a.p_gu.ks;
      for (int u = gw; u < units; u += NW)
        gemv_unit<FMT, true, EPI_SWIGLU, true>(g, u, sm.st[wave], lane, prog, ph + 3, a.err);
    }
    // down GEMV + residual
    {
      GemvArgs g = a.g_down;
      g.W = Lw.w_down; g.S = Lw.s_down;
      g.done = &done[ph + 4]; g.done_target = a.p_down.tiles; g.done_phase = ph + 4; g.progress = a.progress; g.phase_ts = a.phase_ts;
      g.y2 = a.trace ? a.trace + (size_t)(l + 1) * a.H : nullptr;
      const int units = a.p_down.tiles * a.p_down.ks;
      for (int u = gw; u < units; u += NW)
        gemv_unit<FMT, false, EPI_STORE, true>(g, u, sm.st[wave], lane, prog, ph + 4, a.err);
    }
  }
  // lm head (final RMSNorm prologue) + greedy argmax; its finisher writes the token, advances
  // pos and clears every phase counter and the progress replicas of the step
  {
    GemvArgs g = a.g_lm;
    g.progress = a.progress;
    g.phase_ts = a.phase_ts;
    g.done_phase = 1 + 5 * L; g.phase_ts = a.phase_ts;
    const int units = a.p_lm.tiles * a.p_lm.ks;
    for (int u = gw; u < units; u += NW)
      gemv_unit<FMT, true, EPI_ARGMAX, true>(g, u, sm.st[wave], lane, prog, 1 + 5 * L, a.err);
  }
}

template <int FMT, int G>
hipError_t launch_fused_t(const FusedArgs &a, int blocks, hipStream_t st) {
  void *args[] = {const_cast<FusedArgs *>(&a)};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&decode_step_fused<FMT, G>), dim3(blocks),
                                    dim3(256), args, 0, st);
}

template <int FMT, int G>
int occupancy_t() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_step_fused<FMT, G>, 256, 0) != hipSuccess) return 0;
  return nb;
}

}  // namespace

bool fused_supported(int wfmt, int G, int D, int kv_fmt) {
  if (D != 128 || kv_fmt != QDEC_KV_BF16) return false;
  if (wfmt == QDEC_W_Q4_G_ZP8) return G == 7;
  if (wfmt == QDEC_W_Q8_ROW) return G == 6 || G == 4;
  return false;
}

int fused_blocks_per_cu(int wfmt, int G) {
  if (wfmt == QDEC_W_Q4_G_ZP8 && G == 7) return occupancy_t<QDEC_W_Q4_G_ZP8, 7>();
  if (wfmt == QDEC_W_Q8_ROW && G == 6) return occupancy_t<QDEC_W_Q8_ROW, 6>();
  if (wfmt == QDEC_W_Q8_ROW && G == 4) return occupancy_t<QDEC_W_Q8_ROW, 4>();
  return 0;
}

hipError_t launch_fused(const FusedArgs &a, int wfmt, int G, int blocks, hipStream_t st) {
  if (wfmt == QDEC_W_Q4_G_ZP8 && G == 7) return launch_fused_t<QDEC_W_Q4_G_ZP8, 7>(a, blocks, st);
  if (wfmt == QDEC_W_Q8_ROW && G == 6) return launch_fused_t<QDEC_W_Q8_ROW, 6>(a, blocks, st);
  if (wfmt == QDEC_W_Q8_ROW && G == 4) return launch_fused_t<QDEC_W_Q8_ROW, 4>(a, blocks, st);
  return hipErrorInvalidValue;
}

}  // namespace qdec
