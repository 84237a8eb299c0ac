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
// columns' activation chunks are staged once per wave in LDS and read back as broadcasts.
//
// INT4 with 4 or 8 columns runs on the matrix cores instead (v_mfma_f32_16x16x32_f16): one FMA per
// code and column is VALU-bound there (8 columns: gate/up at about 1.4 TB/s).  Each lane keeps its
// own row's codes as the A operand, as fp16 c - 8 (exact), for one 8-code word at a time; lane
// group g = lane / 16 thus feeds rows 16 g .. 16 g + 15 of the 64-row tile into the instruction's
// 16 rows.  The B operand is block-diagonal: lane (group g, column j) holds the activations of
// batch column 4 bg + j % 4 only when j / 4 == g, so output column j gets exactly the products of
// tile row i + 16 (j / 4) — each instruction computes four independent 16-row x 4-column blocks,
// and the codes need no exchange between lanes.  Activations go in as fp16 pairs x = xh + xl
// (22 significant bits; two instructions), products are exact in fp32, the run's sum is scaled
// by the group scale in fp32.  A final LDS transpose returns to one row per lane for the shared
// split-K combine and epilogues.
//
// RMSNorm in front of the GEMM is folded in: with gamma set, column b is normalised while it is
// staged, x_b[k] -> gamma[k] (x_b[k] r_b) with r_b = 1 / sqrt(mean_k x_b[k]^2 + eps) (FlashQwen
// README, "Optimization study": norms fused into the neighbouring kernels), r_b taken from the
// per-64-row-tile sums of squares that the producing GEMM (or the embedding) wrote in its
// epilogue; so the staged values are exactly the normalised activations and no launch of its own
// is needed.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qdec_batch.h"
#include "qdec_device.h"

namespace qdec {

namespace {

using namespace dev;

// weight runs per pipeline batch: shorter batches keep more waves resident; at 8 columns the
// staged activations of one run already fill the wave (measured on MI355X, 7B shapes: 2 runs at
// 2 and 4 columns, 1 run at 8)
template <int NB>
constexpr int kRuns = NB >= 8 ? 1 : 2;
constexpr int kWavesB = 4;

// f32x4 slots per lane that hold the NB columns' activation chunks of one batch of runs
template <int CK, int NB>
constexpr int x_slots() { return (NB * kRuns<NB> * CK / 4 + 63) / 64; }

template <int FMT, int NB>
struct BatchB {
  u32x4 w[kRuns<NB>];
  uint16_t s[kRuns<NB>];
  f32x4 x[x_slots<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16, NB>()];  // this lane's share of the activations
  f32x4 g;  // RMSNorm gains of those activations (the same k in every slot)
};

template <int CK, int NB>
struct StageB {
  float x[NB][kRuns<NB> * CK];
  float zp[NB][kRuns<NB>];
};

// RMSNorm factors of the columns from the producer's per-tile sums of squares ([nb][ssq_n]),
// in two halves so that the first batch of weights is requested in between: norm_issue loads the
// first 64 tiles of every column, norm_finish adds the rest and reduces.  rl[i] = r_b of the column
// b that activation slot i of this lane belongs to (0 past nb); every wave reduces in the same
// order.
template <int NB>
__device__ __forceinline__ void norm_issue(float (&v)[NB], const GemmBArgs &a, int lane) {
  const int n = a.ssq_n;
  const __amdgpu_buffer_rsrc_t qr = rsrc(a.ssq, (uint32_t)((size_t)a.nb * n * 4));
#pragma unroll
  for (int b = 0; b < NB; ++b)
    v[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qr, lane < n ? (uint32_t)((b * n + lane) * 4) : 0x80000000u, 0, 0));
}

template <int CK, int NB, int XS>
__device__ __forceinline__ void norm_finish(float (&rl)[XS], float (&s)[NB], const GemmBArgs &a, int lane) {
  constexpr int PER_COL = kRuns<NB> * CK / 4;
  const int n = a.ssq_n;
  const __amdgpu_buffer_rsrc_t qr = rsrc(a.ssq, (uint32_t)((size_t)a.nb * n * 4));
  for (int t0 = 64; t0 < n; t0 += 64) {
    const int t = t0 + lane;
    float v[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
      v[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qr, t < n ? (uint32_t)((b * n + t) * 4) : 0x80000000u, 0, 0));
#pragma unroll
    for (int b = 0; b < NB; ++b) s[b] += v[b];
  }
#pragma unroll
  for (int i = 0; i < XS; ++i) rl[i] = 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b >= a.nb) break;
    const float r = rsqrtf(wave_sum(s[b]) / (float)a.K + a.eps);
#pragma unroll
    for (int i = 0; i < XS; ++i)
      if ((lane + 64 * i) / PER_COL == b) rl[i] = r;
  }
}

// the gains of this lane's activation slots for the batch of runs at r (zero past the k-range)
template <int CK, int NB>
__device__ __forceinline__ f32x4 gain_load(__amdgpu_buffer_rsrc_t gr, int r, int c0, int nrun, int lane) {
  constexpr int PER_COL = kRuns<NB> * CK / 4;
  const int q = (lane % PER_COL) * 4;
  const uint32_t off = r + q / CK < nrun ? (uint32_t)(((size_t)(c0 + r) * CK + q) * 4) : 0x80000000u;
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(gr, off, 0, 0));
}

// x_b[k] -> gamma[k] (x_b[k] r_b), the order of operations of a separate RMSNorm
__device__ __forceinline__ f32x4 normed(f32x4 v, f32x4 g, float r) {
  return f32x4{g.x * (v.x * r), g.y * (v.y * r), g.z * (v.z * r), g.w * (v.w * r)};
}

template <int FMT, int NB, bool NORM>
__device__ __forceinline__ void b_load(BatchB<FMT, NB> &B, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                       __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t gr, int ldx, int r, int c0,
                                       int nrun, int g0, int gshift, int lane) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  if constexpr (NORM) B.g = gain_load<CK, NB>(gr, r, c0, nrun, lane);
  const uint32_t base = (uint32_t)r * (kTile * 16) + lane * 16;
#pragma unroll
  for (int i = 0; i < kRuns<NB>; ++i) {
    B.w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, base + i * (kTile * 16), 0, kAuxStream));
    if constexpr (Q4) {
      const int g = ((c0 + r + i) >> gshift) - g0;
      B.s[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, (uint32_t)g * (kTile * 2) + lane * 2, 0, 0);
    }
  }
  // column b, 4 values at chunk offset q: flat f = lane + 64 i, b = f / PER_COL, q = 4 (f % PER_COL);
  // runs past the wave's last one read zero (as their weights and scales do)
  constexpr int PER_COL = kRuns<NB> * CK / 4;  // f32x4 per column per batch
#pragma unroll
  for (int i = 0; i < x_slots<CK, NB>(); ++i) {
    const int f = lane + 64 * i;
    const int b = f / PER_COL, q = (f % PER_COL) * 4;
    const bool in = b < NB && r + q / CK < nrun;
    const uint32_t off = in ? (uint32_t)(((size_t)b * ldx + (size_t)(c0 + r) * CK + q) * 4) : 0x80000000u;
    B.x[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
  }
}

template <int FMT, int NB, bool NORM>
__device__ __forceinline__ void b_compute(float (&acc)[NB], const BatchB<FMT, NB> &B,
                                          StageB<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16, NB> &sm,
                                          const float (&rl)[x_slots<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16, NB>()], int lane) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  constexpr int PER_COL = kRuns<NB> * CK / 4;
  constexpr int LPR = CK / 4;  // lanes (f32x4 slots) per run
  // stage the activations and each (column, run)'s sum of x
#pragma unroll
  for (int i = 0; i < x_slots<CK, NB>(); ++i) {
    const int f = lane + 64 * i;
    const int b = f / PER_COL, q = (f % PER_COL) * 4;
    f32x4 v = B.x[i];
    if constexpr (NORM) v = normed(v, B.g, rl[i]);
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
  for (int i = 0; i < kRuns<NB>; ++i) {
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

// ------------------------------------------------------------------ matrix-core path (INT4)
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4m __attribute__((ext_vector_type(4)));

// fp16 pairs of the columns' activations for one batch of runs; within each group of 8 k the
// order is k0, k4, k1, k5, k2, k6, k3, k7, the order in which a 32-bit word's nibbles come out of
// the masks (so the codes need no permutes)
template <int NB>
struct StageM {
  _Float16 xh[NB][kRuns<NB> * 32], xl[NB][kRuns<NB> * 32];
};

template <int NB>
struct BatchM {
  u32x4 w[kRuns<NB>];
  uint64_t s4[kRuns<NB>];  // fp16 scales of the four rows whose results this lane accumulates
  f32x4 x[x_slots<32, NB>()];
  f32x4 g;
};

// first of the four consecutive tile rows whose results lane holds (MFMA output element
// (4 (lane / 16) + r, lane % 16), column block lane % 16 / 4)
__device__ __forceinline__ int m_row0(int lane) { return 4 * (lane >> 4) + 16 * ((lane & 15) >> 2); }

template <int NB, bool NORM>
__device__ __forceinline__ void m_load(BatchM<NB> &B, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                       __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t gr, int ldx, int r, int c0,
                                       int nrun, int g0, int gshift, int lane) {
  constexpr int CK = 32;
  if constexpr (NORM) B.g = gain_load<CK, NB>(gr, r, c0, nrun, lane);
  const uint32_t base = (uint32_t)r * (kTile * 16) + lane * 16;
  const uint32_t r0 = (uint32_t)m_row0(lane);
#pragma unroll
  for (int i = 0; i < kRuns<NB>; ++i) {
    B.w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, base + i * (kTile * 16), 0, kAuxStream));
    const int g = ((c0 + r + i) >> gshift) - g0;
    B.s4[i] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(sr, (uint32_t)g * (kTile * 2) + r0 * 2, 0, 0));
  }
  constexpr int PER_COL = kRuns<NB> * CK / 4;
#pragma unroll
  for (int i = 0; i < x_slots<CK, NB>(); ++i) {
    const int f = lane + 64 * i;
    const int b = f / PER_COL, q = (f % PER_COL) * 4;
    const bool in = b < NB && r + q / CK < nrun;
    const uint32_t off = in ? (uint32_t)(((size_t)b * ldx + (size_t)(c0 + r) * CK + q) * 4) : 0x80000000u;
    B.x[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
  }
}

template <int NB, bool NORM>
__device__ __forceinline__ void m_compute(float (&acc)[NB / 4][4], const BatchM<NB> &B, StageM<NB> &sm,
                                          const float (&rl)[x_slots<32, NB>()], int lane) {
  constexpr int CK = 32, PER_COL = kRuns<NB> * CK / 4;
  // stage the activations as fp16 pairs
#pragma unroll
  for (int i = 0; i < x_slots<CK, NB>(); ++i) {
    const int f = lane + 64 * i;
    const int b = f / PER_COL, q = (f % PER_COL) * 4;
    if (b < NB) {
      f32x4 v = B.x[i];
      if constexpr (NORM) v = normed(v, B.g, rl[i]);
      const _Float16 h0 = (_Float16)v.x, h1 = (_Float16)v.y, h2 = (_Float16)v.z, h3 = (_Float16)v.w;
      const _Float16 l0 = (_Float16)(v.x - (float)h0), l1 = (_Float16)(v.y - (float)h1);
      const _Float16 l2 = (_Float16)(v.z - (float)h2), l3 = (_Float16)(v.w - (float)h3);
      // k = q .. q + 3 go to positions 2 j + (q mod 8) / 4 of their group of 8
      _Float16 *ph = &sm.xh[b][(q & ~7) + ((q >> 2) & 1)];
      _Float16 *pl = &sm.xl[b][(q & ~7) + ((q >> 2) & 1)];
      ph[0] = h0; ph[2] = h1; ph[4] = h2; ph[6] = h3;
      pl[0] = l0; pl[2] = l1; pl[4] = l2; pl[6] = l3;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const bool act = ((lane & 15) >> 2) == (lane >> 4);  // this lane's B block is on the diagonal
  const int bsub = lane & 3;
  // B operands: loaded in the diagonal lanes only; the other lanes keep the zeros they start with
  h8 xh = {}, xl = {};
  const h2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
  for (int i = 0; i < kRuns<NB>; ++i) {
    const uint32_t wd[4] = {B.w[i].x, B.w[i].y, B.w[i].z, B.w[i].w};
    f4m c[NB / 4];
#pragma unroll
    for (int bg = 0; bg < NB / 4; ++bg) c[bg] = f4m{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // the lane's codes k = 8 q .. 8 q + 7 of the run (byte b: k = 2 b low nibble, 2 b + 1 high
      // nibble) in the staged order: 0x6400 | c is the fp16 1024 + c, minus 1032 gives c - 8
      // exactly
      const uint32_t w = wd[q];
      const h2v c04 = __builtin_bit_cast(h2v, (w & 0x000F000Fu) | 0x64006400u) - off;
      const h2v c15 = __builtin_bit_cast(h2v, ((w >> 4) & 0x000F000Fu) | 0x64006400u) - off;
      const h2v c26 = __builtin_bit_cast(h2v, ((w >> 8) & 0x000F000Fu) | 0x64006400u) - off;
      const h2v c37 = __builtin_bit_cast(h2v, ((w >> 12) & 0x000F000Fu) | 0x64006400u) - off;
      const h8 av = {c04.x, c04.y, c15.x, c15.y, c26.x, c26.y, c37.x, c37.y};
#pragma unroll
      for (int bg = 0; bg < NB / 4; ++bg) {
        const int b = 4 * bg + bsub;
        if (act) {
          xh = *reinterpret_cast<const h8 *>(&sm.xh[b][i * CK + 8 * q]);
          xl = *reinterpret_cast<const h8 *>(&sm.xl[b][i * CK + 8 * q]);
        }
        c[bg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, xl, c[bg], 0, 0, 0);
        c[bg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, xh, c[bg], 0, 0, 0);
      }
    }
    // the run's sums times the group scales of the lane's four rows
    const uint64_t sv = B.s4[i];
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = half_bits_to_float((uint16_t)(sv >> (16 * r)));
#pragma unroll
    for (int bg = 0; bg < NB / 4; ++bg)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[bg][r] = fmaf(sc[r], c[bg][r], acc[bg][r]);
  }
  __builtin_amdgcn_wave_barrier();  // the batch after next overwrites this slot
}

// Split-K combine and epilogue of a tile, shared by both paths: acc[b] is this lane's row, column b.
template <int FMT, int NB, int EPI>
__device__ __forceinline__ void b_finish(const GemmBArgs &a, float (&acc)[NB], int tile, int ksi, int lane) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  const int ks = a.ks, N = a.N;
  const int n = tile * kTile + lane;
  const bool valid = n < N;
  const float pre_scale = Q4 ? 1.f : reinterpret_cast<const float *>(a.S)[n];  // padded to tiles
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
    } else {
      if (valid) {
        if (a.bias) v += a.bias[n];
        if (a.residual) v += a.residual[(size_t)b * a.ldy + n];
        a.Y[(size_t)b * a.ldy + n] = v;
      }
      // the sum of squares of the tile's stored outputs, for an RMSNorm folded into the next GEMM
      if (a.ssq_out) {
        const float sq = wave_sum(valid ? v * v : 0.f);
        if (lane == 0) a.ssq_out[(size_t)b * ((N + kTile - 1) / kTile) + tile] = sq;
      }
    }
  }
}

template <int NB, int EPI, bool NORM>
__global__ void __launch_bounds__(kWavesB * 64) gemm_b_mfma(const GemmBArgs a) {
  constexpr int CK = 32;
  // per wave: the two stage slots, reused at the end for the [64][NB + 1] transpose (which is
  // larger than the slots when a batch holds one run)
  union WaveLds {
    StageM<NB> st[2];
    float tr[64 * (NB + 1)];
  };
  __shared__ WaveLds lds_all[kWavesB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * kWavesB + wave;
  const int ks = a.ks, K = a.K, N = a.N;
  const int tiles = (N + kTile - 1) / kTile;
  if (unit >= tiles * ks) return;  // whole wave
  StageM<NB>(&sm)[2] = lds_all[wave].st;
  const int tile = unit / ks;
  const int ksi = unit - tile * ks;
  const int nch = K / CK;
  const int c0 = ksi * a.cps;
  const int c1 = min(nch, c0 + a.cps);
  const int nrun = c1 - c0;
  const size_t tile_bytes = (size_t)nch * kTile * 16;
  const __amdgpu_buffer_rsrc_t wr = rsrc(a.W + (size_t)tile * tile_bytes + (size_t)c0 * kTile * 16, (uint32_t)nrun * kTile * 16);
  const int g0 = c0 >> a.gshift, g1 = (c1 - 1) >> a.gshift;
  const __amdgpu_buffer_rsrc_t sr =
      rsrc(reinterpret_cast<const uint8_t *>(a.S) + (size_t)tile * ((size_t)(nch >> a.gshift) * kTile * 2) + (size_t)g0 * kTile * 2,
           (uint32_t)(g1 - g0 + 1) * kTile * 2);
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.X, (uint32_t)((size_t)a.nb * a.ldx * 4));
  const __amdgpu_buffer_rsrc_t gr = rsrc(a.gamma, (uint32_t)K * 4);
  float rl[x_slots<CK, NB>()], ss[NB];
  if constexpr (NORM) norm_issue<NB>(ss, a, lane);

  float acc4[NB / 4][4];
#pragma unroll
  for (int bg = 0; bg < NB / 4; ++bg)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc4[bg][r] = 0.f;
  BatchM<NB> A, B;
  m_load<NB, NORM>(A, wr, sr, xr, gr, a.ldx, 0, c0, nrun, g0, a.gshift, lane);
  if constexpr (NORM) norm_finish<CK, NB>(rl, ss, a, lane);
  const int nb = (nrun + kRuns<NB> - 1) / kRuns<NB>;
  for (int bt = 0; bt < nb; bt += 2) {
    m_load<NB, NORM>(B, wr, sr, xr, gr, a.ldx, (bt + 1) * kRuns<NB>, c0, nrun, g0, a.gshift, lane);
    m_compute<NB, NORM>(acc4, A, sm[0], rl, lane);
    if (bt + 1 >= nb) break;
    m_load<NB, NORM>(A, wr, sr, xr, gr, a.ldx, (bt + 2) * kRuns<NB>, c0, nrun, g0, a.gshift, lane);
    m_compute<NB, NORM>(acc4, B, sm[1], rl, lane);
  }
  // back to one row per lane: lane holds rows m_row0 + r of columns 4 bg + lane % 4
  float *tr = lds_all[wave].tr;  // [64][NB + 1]
  const int r0 = m_row0(lane);
#pragma unroll
  for (int bg = 0; bg < NB / 4; ++bg)
#pragma unroll
    for (int r = 0; r < 4; ++r) tr[(r0 + r) * (NB + 1) + 4 * bg + (lane & 3)] = acc4[bg][r];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = tr[lane * (NB + 1) + b];
  b_finish<QDEC_W_Q4_G_ZP8, NB, EPI>(a, acc, tile, ksi, lane);
}

template <int FMT, int NB, int EPI, bool NORM>
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
  const __amdgpu_buffer_rsrc_t gr = rsrc(a.gamma, (uint32_t)K * 4);
  float rl[x_slots<CK, NB>()], ss[NB];
  if constexpr (NORM) norm_issue<NB>(ss, a, lane);

  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
  BatchB<FMT, NB> A, B;
  b_load<FMT, NB, NORM>(A, wr, sr, xr, gr, a.ldx, 0, c0, nrun, g0, a.gshift, lane);
  if constexpr (NORM) norm_finish<CK, NB>(rl, ss, a, lane);
  const int nb = (nrun + kRuns<NB> - 1) / kRuns<NB>;
  for (int bt = 0; bt < nb; bt += 2) {
    b_load<FMT, NB, NORM>(B, wr, sr, xr, gr, a.ldx, (bt + 1) * kRuns<NB>, c0, nrun, g0, a.gshift, lane);
    b_compute<FMT, NB, NORM>(acc, A, sm[0], rl, lane);
    if (bt + 1 >= nb) break;
    b_load<FMT, NB, NORM>(A, wr, sr, xr, gr, a.ldx, (bt + 2) * kRuns<NB>, c0, nrun, g0, a.gshift, lane);
    b_compute<FMT, NB, NORM>(acc, B, sm[1], rl, lane);
  }
  b_finish<FMT, NB, EPI>(a, acc, tile, ksi, lane);
}

template <int FMT, int NB, int EPI, bool NORM>
void launch_k(const GemmBArgs &a, int blocks, hipStream_t st) {
  if constexpr (FMT == QDEC_W_Q4_G_ZP8 && NB >= 4)
    hipLaunchKernelGGL((gemm_b_mfma<NB, EPI, NORM>), dim3(blocks), dim3(kWavesB * 64), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_b_tile64<FMT, NB, EPI, NORM>), dim3(blocks), dim3(kWavesB * 64), 0, st, a);
}

template <int FMT, int NB>
hipError_t launch_nb(const GemmBArgs &a, int blocks, hipStream_t st) {
  const bool norm = a.gamma != nullptr;
  if (a.epi == EPI_SWIGLU)
    norm ? launch_k<FMT, NB, EPI_SWIGLU, true>(a, blocks, st) : launch_k<FMT, NB, EPI_SWIGLU, false>(a, blocks, st);
  else
    norm ? launch_k<FMT, NB, EPI_STORE, true>(a, blocks, st) : launch_k<FMT, NB, EPI_STORE, false>(a, blocks, st);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const GemmBArgs &a, int blocks, hipStream_t st) {
  switch (a.nb_max) {
    case 1: return launch_nb<FMT, 1>(a, blocks, st);
    case 2: return launch_nb<FMT, 2>(a, blocks, st);
    case 4: return launch_nb<FMT, 4>(a, blocks, st);
    case 8: return launch_nb<FMT, 8>(a, blocks, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// (one column alone: staging and multiplying a second, empty one cost a third of the time)
int gemm_b_columns(int batch) { return batch <= 1 ? 1 : (batch <= 2 ? 2 : (batch <= 4 ? 4 : 8)); }

// The k-split plan is the GEMV's (measured: splitting further for the batch only adds partial
// sums; the waves are limited by staging the columns' activations, not by their number).
GemvPlan gemm_b_plan(int wfmt, int N, int K, int nb_max, bool allow_split) {
  (void)nb_max;
  // (the skinny GEMMs keep about four waves per compute unit on the small matrices: more k-splits
  // made the batched step slower at every batch size)
  return gemv_plan(wfmt, N, K, allow_split, 1024);
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
