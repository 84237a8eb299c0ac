// INT8-activation GEMV ("Path A") for gfx950: per-group INT8 quantisation of the activations,
// then integer dot products of the weight codes with the INT8 activations.
//
// What it computes ("Building a Tiny LLM Runtime on H100", Challenge 3, Path A; "How To Construct
// Your Personal LLM Runtime From Scratch", section 7, the INT4 code convention):
//   activations: for each group of `group` consecutive k, amax = max |x|, s = amax / 127 and
//     q[k] = round-half-even(x[k] * (127 / amax)) clamped to [-127, 127], every step in binary32;
//     a group of zeros has s = 0 and q = 0;
//   GEMV: y[n] = sum_g wscale * s_g * sum_{k in g} level[n][k] q[k]  (+ bias[n]) (+ residual[n]),
//     level = the INT8 code (one scale per row) or the INT4 code minus 8 (fp16 scale per group;
//     the activation groups are then the weight groups).
//
// How, on CDNA4: the same tile64 weight layout and work split as the fp32-activation GEMV (a
// wave owns 64 output rows, one per lane, and streams 1 KiB runs; k is split across waves for
// small N, partials added in a fixed order by the last wave of a tile).  The difference is the
// inner loop: four codes times four INT8 activations per v_dot4_i32_i8 instead of one fp32 FMA
// per code.  INT4 codes sit in natural k order (low nibble even k, high nibble odd k), so a run's
// activations are staged de-interleaved in LDS: the 16 even-k bytes, then the 16 odd-k bytes; a
// word masked with 0x0F0F0F0F (codes of even k) meets an even-k word, the word shifted right by
// four and masked meets an odd-k word.  The zero point leaves the inner loop as
//   sum_k (c_k - 8) q_k = sum_k c_k q_k - 8 sum_k q_k,
// with -8 sum_k q_k (the same for all rows) staged once per run and used as the dot chain's start.
// Each run's integer sum (|sum| < 2^24, exact in fp32) is scaled once per run by the weight scale
// times the activation scale of its group, so split boundaries need not align with groups.
#include <hip/hip_runtime.h>

#include "qdec_device.h"

namespace qdec {

namespace {

using namespace dev;

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kA8Waves = 4;

struct A8Args {
  const uint8_t *W;   // packed tile64 weights
  const void *S;      // packed scales (q8: fp32 [Npad], q4: fp16 [tiles][K/group][64])
  const int8_t *q;    // INT8 activations [K], k order
  const float *sx;    // activation scales [K / group]
  const float *bias, *residual;
  float *y;
  float *part;
  unsigned *counters;
  int N, K;
  int gshift;         // q4: log2(group / 32), the weight-scale group in runs
  int ashift;         // log2(group): the activation group in k
  int ks, cps;
};

// A batch's staged activations, per run: Q4 words 0-3 even k, 4-7 odd k; Q8 words 0-3 in k
// order.  zp: the run's dot-chain start (-8 sum q for Q4, 0 for Q8); sx: its group's scale.
template <int CK>
struct StageA8 {
  uint32_t q[kBatch * CK / 4];
  int zp[kBatch];
  float sx[kBatch];
};

template <int FMT>
struct BatchA8 {
  u32x4 w[kBatch];
  uint16_t s[kBatch];
  uint32_t q;  // this lane's four activation bytes of the batch (k order)
  float sx;    // lanes < kBatch: activation scale of run `lane` of the batch
};

template <int FMT>
__device__ __forceinline__ void a8_load(BatchA8<FMT> &B, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                        __amdgpu_buffer_rsrc_t qr, __amdgpu_buffer_rsrc_t xr, int r, int c0, int g0,
                                        int a0, const A8Args &a, int lane) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  const uint32_t base = (uint32_t)r * (kTile * 16) + lane * 16;
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    B.w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, base + i * (kTile * 16), 0, kAuxStream));
    if constexpr (Q4) {
      const int g = ((c0 + r + i) >> a.gshift) - g0;
      B.s[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, (uint32_t)g * (kTile * 2) + lane * 2, 0, 0);
    }
  }
  // activation bytes: kBatch * CK of them, four per lane (past the wave's runs: zero)
  const uint32_t qo = (lane * 4 < kBatch * CK) ? (uint32_t)(r * CK + lane * 4) : 0x80000000u;
  B.q = __builtin_amdgcn_raw_buffer_load_b32(qr, qo, 0, 0);
  const int ga = (((c0 + r + lane) * CK) >> a.ashift) - a0;
  const uint32_t so = (lane < kBatch) ? (uint32_t)ga * 4u : 0x80000000u;
  B.sx = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, so, 0, 0));
}

template <int FMT>
__device__ __forceinline__ void a8_compute(float &acc, const BatchA8<FMT> &B, StageA8<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16> &sm,
                                           int lane) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  if constexpr (Q4) {
    // lane l holds k = 4l .. 4l+3 of the batch: run l / 8, word j = (l % 8) / 2, half h = l % 2
    const int run = lane >> 3, j = (lane >> 1) & 3, h = lane & 1;
    const uint32_t ev = __builtin_amdgcn_perm(0u, B.q, 0x0c0c0200u);  // bytes 0, 2 (even k)
    const uint32_t od = __builtin_amdgcn_perm(0u, B.q, 0x0c0c0301u);  // bytes 1, 3 (odd k)
    // sum of the run's 32 codes (8 lanes), exact in fp32 (every lane takes part in the DPP sum;
    // only the lanes that hold the batch's runs store)
    const float part = sum8((float)__builtin_amdgcn_sdot4((int)B.q, 0x01010101, 0, false));
    if (lane * 4 < kBatch * CK) {
      uint16_t *q16 = reinterpret_cast<uint16_t *>(sm.q);
      q16[run * 16 + j * 2 + h] = (uint16_t)ev;
      q16[run * 16 + 8 + j * 2 + h] = (uint16_t)od;
      if ((lane & 7) == 0) sm.zp[run] = -8 * (int)part;
    }
  } else {
    if (lane * 4 < kBatch * CK) sm.q[lane] = B.q;
    if (lane < kBatch) sm.zp[lane] = 0;
  }
  if (lane < kBatch) sm.sx[lane] = B.sx;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const uint32_t wd[4] = {B.w[i].x, B.w[i].y, B.w[i].z, B.w[i].w};
    int d = sm.zp[i];
    if constexpr (Q4) {
      const i32x4 qe = *reinterpret_cast<const i32x4 *>(&sm.q[i * 8]);
      const i32x4 qd = *reinterpret_cast<const i32x4 *>(&sm.q[i * 8 + 4]);
      const int qev[4] = {qe.x, qe.y, qe.z, qe.w}, qdv[4] = {qd.x, qd.y, qd.z, qd.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        d = __builtin_amdgcn_sdot4((int)(wd[w] & 0x0F0F0F0Fu), qev[w], d, false);
        d = __builtin_amdgcn_sdot4((int)((wd[w] >> 4) & 0x0F0F0F0Fu), qdv[w], d, false);
      }
      acc = fmaf(half_bits_to_float(B.s[i]) * sm.sx[i], (float)d, acc);
    } else {
      const i32x4 qv = *reinterpret_cast<const i32x4 *>(&sm.q[i * 4]);
      const int qa[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) d = __builtin_amdgcn_sdot4((int)wd[w], qa[w], d, false);
      acc = fmaf(sm.sx[i], (float)d, acc);
    }
  }
  __builtin_amdgcn_wave_barrier();  // the batch after next overwrites this slot
}

template <int FMT>
__global__ void __launch_bounds__(kA8Waves * 64) gemv_a8_tile64(const A8Args a) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  __shared__ StageA8<CK> stage_all[kA8Waves][2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * kA8Waves + wave;
  const int ks = a.ks, K = a.K, N = a.N;
  if (unit >= ((N + kTile - 1) / kTile) * ks) return;  // whole wave
  StageA8<CK>(&sm)[2] = stage_all[wave];
  const int tile = unit / ks;
  const int ksi = unit - tile * ks;
  const int nch = K / CK;
  const int c0 = ksi * a.cps;
  const int c1 = min(nch, c0 + a.cps);
  const int nrun = c1 - c0;
  const size_t tile_bytes = (size_t)nch * kTile * 16;
  const __amdgpu_buffer_rsrc_t wr = rsrc(a.W + (size_t)tile * tile_bytes + (size_t)c0 * kTile * 16, (uint32_t)nrun * kTile * 16);
  __amdgpu_buffer_rsrc_t sr = wr;
  int g0 = 0;
  if constexpr (Q4) {
    g0 = c0 >> a.gshift;
    const int g1 = (c1 - 1) >> a.gshift;
    sr = rsrc(reinterpret_cast<const uint8_t *>(a.S) + (size_t)tile * ((size_t)(nch >> a.gshift) * kTile * 2) + (size_t)g0 * kTile * 2,
              (uint32_t)(g1 - g0 + 1) * kTile * 2);
  }
  const __amdgpu_buffer_rsrc_t qr = rsrc(a.q + (size_t)c0 * CK, (uint32_t)nrun * CK);
  const int a0 = (c0 * CK) >> a.ashift;
  const int a1 = (c1 * CK - 1) >> a.ashift;
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.sx + a0, (uint32_t)(a1 - a0 + 1) * 4);

  float acc = 0.f;
  BatchA8<FMT> A, B;
  a8_load<FMT>(A, wr, sr, qr, xr, 0, c0, g0, a0, a, lane);
  const int n = tile * kTile + lane;
  const bool valid = n < N;
  float pre_bias = 0.f, pre_res = 0.f, pre_scale = 1.f;
  if (valid) {
    if (a.bias) pre_bias = a.bias[n];
    if (a.residual) pre_res = a.residual[n];  // (y may alias it: only this tile's epilogue writes y[n])
  }
  if constexpr (!Q4) pre_scale = reinterpret_cast<const float *>(a.S)[n];  // padded to tiles
  const int nb = (nrun + kBatch - 1) / kBatch;
  for (int b = 0; b < nb; b += 2) {
    a8_load<FMT>(B, wr, sr, qr, xr, (b + 1) * kBatch, c0, g0, a0, a, lane);
    a8_compute<FMT>(acc, A, sm[0], lane);
    if (b + 1 >= nb) break;
    a8_load<FMT>(A, wr, sr, qr, xr, (b + 2) * kBatch, c0, g0, a0, a, lane);
    a8_compute<FMT>(acc, B, sm[1], lane);
  }

  if (ks > 1 && !splitk_combine(acc, a.part, a.counters, tile, ks, ksi, lane)) return;
  if (valid) {
    float v = acc * pre_scale;
    if (a.bias) v += pre_bias;
    if (a.residual) v += pre_res;
    a.y[n] = v;
  }
}

// One wave per group of `group` activations (group a power of two in [32, 4096]).
__global__ void __launch_bounds__(256) quantize_act_i8_k(const float *__restrict__ x, int K, int group,
                                                         int8_t *__restrict__ q, float *__restrict__ sx) {
  const int lane = threadIdx.x & 63;
  const int ng = K / group;
  for (int g = blockIdx.x * 4 + (int)(threadIdx.x >> 6); g < ng; g += gridDim.x * 4) {
    const float *xg = x + (size_t)g * group;
    float m = 0.f;
    for (int i = lane; i < group; i += 64) m = fmaxf(m, fabsf(xg[i]));
    const float amax = wave_max(m);
    int8_t *qg = q + (size_t)g * group;
    if (amax == 0.f) {
      for (int i = lane; i < group; i += 64) qg[i] = 0;
      if (lane == 0) sx[g] = 0.f;
      continue;
    }
    const float inv = 127.0f / amax;  // binary32 division, correctly rounded
    for (int i = lane; i < group; i += 64) {
      const float r = fminf(fmaxf(rintf(xg[i] * inv), -127.0f), 127.0f);
      qg[i] = (int8_t)(int)r;
    }
    if (lane == 0) sx[g] = amax / 127.0f;
  }
}

}  // namespace

hipError_t launch_quantize_act_i8(const float *x, int K, int group, int8_t *q, float *sx, hipStream_t st) {
  const int ng = K / group;
  const int blocks = (ng + 3) / 4 < 1024 ? (ng + 3) / 4 : 1024;
  hipLaunchKernelGGL(quantize_act_i8_k, dim3(blocks), dim3(256), 0, st, x, K, group, q, sx);
  return hipGetLastError();
}

hipError_t launch_gemv_a8(int wfmt, const uint8_t *W, const void *S, const int8_t *q, const float *sx, int group,
                          const float *bias, const float *residual, float *y, int N, int K, void *ws, hipStream_t st) {
  const GemvPlan p = gemv_plan(wfmt, N, K, ws != nullptr);
  GemvArgs g{};
  gemv_bind_workspace(g, p, ws);
  A8Args a{};
  a.W = W;
  a.S = S;
  a.q = q;
  a.sx = sx;
  a.bias = bias;
  a.residual = residual;
  a.y = y;
  a.part = g.part;
  a.counters = g.counters;
  a.N = N;
  a.K = K;
  a.ks = p.ks;
  a.cps = p.cps;
  int ashift = 0;
  while ((1 << ashift) < group) ++ashift;
  a.ashift = ashift;
  a.gshift = ashift - 5;  // q4: group / 32 runs per weight-scale group
  const int blocks = (p.units + kA8Waves - 1) / kA8Waves;
  if (wfmt == QDEC_W_Q4_G_ZP8)
    hipLaunchKernelGGL(gemv_a8_tile64<QDEC_W_Q4_G_ZP8>, dim3(blocks), dim3(kA8Waves * 64), 0, st, a);
  else
    hipLaunchKernelGGL(gemv_a8_tile64<QDEC_W_Q8_ROW>, dim3(blocks), dim3(kA8Waves * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace qdec
