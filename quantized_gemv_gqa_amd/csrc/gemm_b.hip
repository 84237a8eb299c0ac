// Skinny GEMM for batched decode: Y[b] = W X[b] for up to NB activation columns (one per running
// sequence), with the same weight-only-quantized formats and fused dequant as the GEMV.
//
// What it computes: for every column b < nb, y_b[n] = sum_k w[n][k] x_b[k] (+ bias[n])
// (+ residual_b[n]), or the SwiGLU of the gate/up row pairs; INT8 per-row or INT4 group-scaled
// weights ("How To Construct Your Personal LLM Runtime From Scratch", section 7; FlashQwen README,
// "Optimization study" stage 8), fp32 activations and accumulation.  Batching the running
// sequences turns the decode GEMV into this skinny GEMM ("Chapter 2 Systems Foundations for LLMs",
// "Continuous Batching": all running sequences are decoded together, one token each).
//
// How: the GEMV's tile64 layout and work split (a wave owns 64 rows, one per lane; k split across
// waves with a deterministic combine).  Each 16-byte weight run is loaded once and converted to
// fp32 once (v_cvt_f32_ubyte on masked bytes), then used by every column: one FMA per code and
// column, with the zero point (INT4) and the byte bias (INT8) folded out as
// sum_k (c_k - z) x_k = sum_k c_k x_k - z sum_k x_k, sum_k x_k staged per run and column.  The
// columns' activation chunks are staged once per wave in LDS and read back as broadcasts.  fp32
// matrix cores would not help: on gfx950 their fp32 rate equals the vector rate, and 16-bit inputs
// would change the fp32 activations.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qdec_batch.h"
#include "qdec_device.h"

namespace qdec {

namespace {

using namespace dev;

constexpr int kRunsB = 4;  // weight runs per pipeline batch
constexpr int kWavesB = 4;

// f32x4 slots per lane that hold the NB columns' activation chunks of one batch of runs
template <int CK, int NB>
constexpr int x_slots() { return (NB * kRunsB * CK / 4 + 63) / 64; }

template <int FMT, int NB>
struct BatchB {
  u32x4 w[kRunsB];
  uint16_t s[kRunsB];
  f32x4 x[x_slots<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16, NB>()];  // this lane's share of the activations
};

template <int CK, int NB>
struct StageB {
  float x[NB][kRunsB * CK];
  float zp[NB][kRunsB];
};

template <int FMT, int NB>
__device__ __forceinline__ void b_load(BatchB<FMT, NB> &B, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                       __amdgpu_buffer_rsrc_t xr, int ldx, int r, int c0, int nrun, int g0, int gshift,
                                       int lane) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  const uint32_t base = (uint32_t)r * (kTile * 16) + lane * 16;
#pragma unroll
  for (int i = 0; i < kRunsB; ++i) {
    B.w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, base + i * (kTile * 16), 0, kAuxStream));
    if constexpr (Q4) {
      const int g = ((c0 + r + i) >> gshift) - g0;
      B.s[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, (uint32_t)g * (kTile * 2) + lane * 2, 0, 0);
    }
  }
  // column b, 4 values at chunk offset q: flat f = lane + 64 i, b = f / PER_COL, q = 4 (f % PER_COL);
  // runs past the wave's last one read zero (as their weights and scales do)
  constexpr int PER_COL = kRunsB * CK / 4;  // f32x4 per column per batch
#pragma unroll
  for (int i = 0; i < x_slots<CK, NB>(); ++i) {
    const int f = lane + 64 * i;
    const int b = f / PER_COL, q = (f % PER_COL) * 4;
    const bool in = b < NB && r + q / CK < nrun;
    const uint32_t off = in ? (uint32_t)(((size_t)b * ldx + (size_t)(c0 + r) * CK + q) * 4) : 0x80000000u;
    B.x[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
  }
}

template <int FMT, int NB>
__device__ __forceinline__ void b_compute(float (&acc)[NB], const BatchB<FMT, NB> &B,
                                          StageB<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16, NB> &sm, int lane) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  constexpr int PER_COL = kRunsB * CK / 4;
  constexpr int LPR = CK / 4;  // lanes (f32x4 slots) per run
  // stage the activations and each (column, run)'s sum of x
#pragma unroll
  for (int i = 0; i < x_slots<CK, NB>(); ++i) {
    const int f = lane + 64 * i;
    const int b = f / PER_COL, q = (f % PER_COL) * 4;
    const f32x4 v = B.x[i];
    float part = (v.x + v.y) + (v.z + v.w);
    if constexpr (LPR == 8) {
      part = sum8(part);
    } else {
      part += dpp<0xB1>(part);
      part += dpp<0x4E>(part);
    }
    if (b < NB) {
      *reinterpret_cast<f32x4 *>(&sm.x[b][q]) = v;
      if ((f % LPR) == 0) sm.zp[b][q / CK] = part * (Q4 ? 8.0f : 128.0f);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < kRunsB; ++i) {
    // the run's codes as floats, in k order
    float c[CK];
    const uint32_t wd[4] = {B.w[i].x, B.w[i].y, B.w[i].z, B.w[i].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (Q4) {
        const uint32_t lo = and_opaque(wd[q], 0x0F0F0F0Fu), hi = and_opaque(wd[q] >> 4, 0x0F0F0F0Fu);
        c[8 * q + 0] = ub0(lo); c[8 * q + 1] = ub0(hi);
        c[8 * q + 2] = ub1(lo); c[8 * q + 3] = ub1(hi);
        c[8 * q + 4] = ub2(lo); c[8 * q + 5] = ub2(hi);
        c[8 * q + 6] = ub3(lo); c[8 * q + 7] = ub3(hi);
      } else {
        const uint32_t u = wd[q] ^ 0x80808080u;  // c + 128 as an unsigned byte
        c[4 * q + 0] = ub0(u); c[4 * q + 1] = ub1(u);
        c[4 * q + 2] = ub2(u); c[4 * q + 3] = ub3(u);
      }
    }
    const float s = Q4 ? half_bits_to_float(B.s[i]) : 1.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int q = 0; q < CK / 4; ++q) {
        const f32x4 xv = *reinterpret_cast<const f32x4 *>(&sm.x[b][i * CK + 4 * q]);
        d0 = fmaf(c[4 * q + 0], xv.x, d0);
        d1 = fmaf(c[4 * q + 1], xv.y, d1);
        d0 = fmaf(c[4 * q + 2], xv.z, d0);
        d1 = fmaf(c[4 * q + 3], xv.w, d1);
      }
      const float dot = (d0 + d1) - sm.zp[b][i];
      if constexpr (Q4)
        acc[b] = fmaf(s, dot, acc[b]);
      else
        acc[b] += dot;
    }
  }
  __builtin_amdgcn_wave_barrier();  // the batch after next overwrites this slot
}

template <int FMT, int NB, int EPI>
__global__ void __launch_bounds__(kWavesB * 64) gemm_b_tile64(const GemmBArgs a) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  __shared__ StageB<CK, NB> stage_all[kWavesB][2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * kWavesB + wave;
  const int ks = a.ks, K = a.K, N = a.N;
  const int tiles = (N + kTile - 1) / kTile;
  if (unit >= tiles * ks) return;  // whole wave
  StageB<CK, NB>(&sm)[2] = stage_all[wave];
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
  // the nb columns' rows (each column reads only its own runs of the wave's k-range)
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.X, (uint32_t)((size_t)a.nb * a.ldx * 4));

  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
  BatchB<FMT, NB> A, B;
  b_load<FMT, NB>(A, wr, sr, xr, a.ldx, 0, c0, nrun, g0, a.gshift, lane);
  const int n = tile * kTile + lane;
  const bool valid = n < N;
  const float pre_scale = Q4 ? 1.f : reinterpret_cast<const float *>(a.S)[n];  // padded to tiles
  const int nb = (nrun + kRunsB - 1) / kRunsB;
  for (int bt = 0; bt < nb; bt += 2) {
    b_load<FMT, NB>(B, wr, sr, xr, a.ldx, (bt + 1) * kRunsB, c0, nrun, g0, a.gshift, lane);
    b_compute<FMT, NB>(acc, A, sm[0], lane);
    if (bt + 1 >= nb) break;
    b_load<FMT, NB>(A, wr, sr, xr, a.ldx, (bt + 2) * kRunsB, c0, nrun, g0, a.gshift, lane);
    b_compute<FMT, NB>(acc, B, sm[1], lane);
  }

  if (ks > 1) {
    // split-K: the NB partials of this wave as device-coherent stores, counted after they are
    // acknowledged; the last wave of the tile adds all splits in split order, per column
    float *pp = a.part + ((size_t)tile * ks + ksi) * NB * kTile + lane;
#pragma unroll
    for (int b = 0; b < NB; ++b) __hip_atomic_store(pp + b * kTile, acc[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    drain_stores();
    unsigned *ctr = a.counters + tile * kLine;
    unsigned prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (unsigned)(ks - 1)) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const __amdgpu_buffer_rsrc_t pr = rsrc(a.part + (size_t)tile * ks * NB * kTile, (uint32_t)ks * NB * kTile * 4);
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.f;
    for (int i = 0; i < ks; ++i) {
      float t[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        t[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, lane * 4, (i * NB + b) * kTile * 4, kAuxSc1));
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] += t[b];
    }
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b >= a.nb) break;
    if (a.pos && a.pos[b] < 0) continue;  // idle column: its outputs stay as they are
    float v = acc[b];
    if constexpr (!Q4) v *= pre_scale;
    if constexpr (EPI == EPI_SWIGLU) {
      // lanes 0..31: gate rows 32 tile + lane; lanes 32..63: the matching up rows
      const float u = __shfl(v, lane + 32, 64);
      const int i = tile * 32 + lane;
      if (lane < 32 && i < N / 2) a.Y[(size_t)b * a.ldy + i] = silu(v) * u;
    } else if (valid) {
      if (a.bias) v += a.bias[n];
      if (a.residual) v += a.residual[(size_t)b * a.ldy + n];
      a.Y[(size_t)b * a.ldy + n] = v;
    }
  }
}

template <int FMT, int NB>
hipError_t launch_nb(const GemmBArgs &a, int blocks, hipStream_t st) {
  if (a.epi == EPI_SWIGLU)
    hipLaunchKernelGGL((gemm_b_tile64<FMT, NB, EPI_SWIGLU>), dim3(blocks), dim3(kWavesB * 64), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_b_tile64<FMT, NB, EPI_STORE>), dim3(blocks), dim3(kWavesB * 64), 0, st, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const GemmBArgs &a, int blocks, hipStream_t st) {
  switch (a.nb_max) {
    case 2: return launch_nb<FMT, 2>(a, blocks, st);
    case 4: return launch_nb<FMT, 4>(a, blocks, st);
    case 8: return launch_nb<FMT, 8>(a, blocks, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gemm_b_columns(int batch) { return batch <= 2 ? 2 : (batch <= 4 ? 4 : 8); }

// The k-split plan is the GEMV's (measured: splitting further for the batch only adds partial
// sums; the waves are limited by staging the columns' activations, not by their number).
GemvPlan gemm_b_plan(int wfmt, int N, int K, int nb_max, bool allow_split) {
  (void)nb_max;
  return gemv_plan(wfmt, N, K, allow_split);
}

size_t gemm_b_workspace_bytes(int wfmt, int N, int K, int nb_max) {
  const GemvPlan p = gemm_b_plan(wfmt, N, K, nb_max, true);
  size_t b = kCounterBytes;
  if (p.ks > 1) b += (size_t)p.tiles * p.ks * nb_max * kTile * sizeof(float);
  return b;
}

hipError_t launch_gemm_b(int wfmt, GemmBArgs a, void *ws, hipStream_t st) {
  const GemvPlan p = gemm_b_plan(wfmt, a.N, a.K, a.nb_max, ws != nullptr);
  a.ks = p.ks;
  a.cps = p.cps;
  int gshift = 0;
  if (wfmt == QDEC_W_Q4_G_ZP8)
    while ((32 << gshift) < a.group) ++gshift;
  a.gshift = gshift;
  a.counters = reinterpret_cast<unsigned *>(ws);
  a.part = ws ? reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + kCounterBytes) : nullptr;
  const int blocks = (p.units + kWavesB - 1) / kWavesB;
  return wfmt == QDEC_W_Q4_G_ZP8 ? launch_fmt<QDEC_W_Q4_G_ZP8>(a, blocks, st) : launch_fmt<QDEC_W_Q8_ROW>(a, blocks, st);
}

}  // namespace qdec
