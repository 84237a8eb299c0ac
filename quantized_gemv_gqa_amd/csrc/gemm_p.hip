// Prefill GEMM on the matrix cores: Y[m][n] = sum_k X[m][k] w[n][k] for the M tokens of a prompt,
// with the weight-only-quantized formats of the decode GEMV dequantized inside the kernel.
//
// What it computes: the projections of a prompt's tokens (qkv + bias, o + residual, gate/up with
// the SwiGLU epilogue, down + residual), the same matrices and fp32 arithmetic as decode ("How To
// Construct Your Personal LLM Runtime From Scratch", section 7, for the INT4 codes; FlashQwen
// README, "Optimization study" stage 8, for INT8 rows).  Prefill is the one place of the step that
// is a dense contraction (M = prompt length), so it runs on the matrix cores.
//
// How (gfx950): 16-bit matrix inputs with fp32 accumulation, made as accurate as fp32 inputs by
// splitting each operand into an fp16 pair: the activations arrive as x = xh + xl (22 significant
// bits, split once by the kernel that produces them); an INT4 weight w = (c - 8) s has at most 15
// significant bits, so w 2^8 = wh + wl exactly (wh = fp16(w 2^8) by one packed multiply, wl by one
// packed fused multiply-add; the exact 2^8 keeps wl a normal fp16 and is undone on the result); INT8 codes are exact in fp16 (wl = 0, the row scale
// multiplies the fp32 result).  Each fragment takes wh xh + wl xh + wh xl (the dropped wl xl is
// below 2^-22 of the product).  A plain fp16 GEMM (only xh, only wh) was measured first: its 2^-11
// input rounding, through the sharp softmax of some prompt positions, moved their attention
// outputs and later keys by percents.
//
// A workgroup of 4 waves computes a 128 (n) x 128 (m) tile over k-tiles of 32.  Per k-tile the
// workgroup dequantizes its 128 weight rows once into LDS (half a 16-byte INT4 run, or one INT8
// run, per thread, read from the packed tile64 layout; codes become fp16 through the
// 0x6400 | c = 1024 + c bit pattern, byte permutes and packed fp16 arithmetic) and copies its 128
// rows of xh and xl; each wave then runs 4 x 4 fragments of v_mfma_f32_16x16x32_f16 (three per
// fragment for INT4, two for INT8) on its 64 x 64 quarter.  The next k-tile's global loads are
// issued before the current tile's MFMAs.  LDS rows are padded by 8 halves so the 16 lanes of a
// fragment read hit different banks.  Workgroups that share weight rows are adjacent in launch
// order (m fastest), so a weight tile read from HBM is reused from L2 by the other m-tiles.  GEMMs
// whose tiles do not fill the GPU (few output rows: o, down, qkv) also split k; the splits' fp32
// partials are added in split order by a second launch, so results do not depend on timing.
#include <hip/hip_runtime.h>

#include "qdec_batch.h"
#include "qdec_device.h"

namespace qdec {

namespace {

using namespace dev;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int BN = 128, BM = 128, BK = 32, LDP = BK + 8;  // tile sizes; padded LDS row (halves)

template <int FMT>
struct PrefetchP {
  uint32_t w[4];  // INT4: 8 bytes (16 codes) of a run; INT8: 16 bytes (one run)
  uint16_t s;     // INT4 group scale
  u32x4 x[4];     // 32 halves of one activation row (high or low part)
};

template <int FMT, bool LO>
__device__ __forceinline__ void p_load(PrefetchP<FMT> &P, const GemmPArgs &a, int n0, int m0, int kt, int tid) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  const int nch = a.K / CK;
  const int npad = ((a.N + kTile - 1) / kTile) * kTile;
  // weights: row tid % 128; INT4: bytes 8 (tid / 128) .. + 8 of the k-tile's run; INT8: run tid / 128
  const int row = tid & 127, n = n0 + row;
  const int half = tid >> 7;
  if (n < npad) {
    const size_t tile = (size_t)(n >> 6), r = (size_t)(n & 63);
    if constexpr (Q4) {
      const int c = kt;
      const uint2 v = *reinterpret_cast<const uint2 *>(a.W + ((tile * nch + c) * kTile + r) * 16 + 8 * half);
      P.w[0] = v.x;
      P.w[1] = v.y;
      const int ng = a.K / a.group;
      P.s = reinterpret_cast<const uint16_t *>(a.S)[(tile * ng + (c * CK) / a.group) * kTile + r];
    } else {
      const int c = 2 * kt + half;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(a.W + ((tile * nch + c) * kTile + r) * 16);
      P.w[0] = v.x;
      P.w[1] = v.y;
      P.w[2] = v.z;
      P.w[3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) P.w[i] = 0u;
    P.s = 0;
  }
  // activations: row m0 + tid / 2, the high part (tid even) or the low part (tid odd)
  const int m = m0 + (tid >> 1);
  const uint16_t *base = (tid & 1) ? a.Xl : a.X;
  const bool in = m < a.M && (LO || !(tid & 1));
  const uint16_t *xp = base + (size_t)m * a.ldx + (size_t)kt * BK;
#pragma unroll
  for (int i = 0; i < 4; ++i) P.x[i] = in ? *reinterpret_cast<const u32x4 *>(xp + 8 * i) : u32x4{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u(h2 v) { return __builtin_bit_cast(uint32_t, v); }

struct SmemP {
  _Float16 wh[BN][LDP], wl[BN][LDP], xh[BM][LDP], xl[BM][LDP];
};

template <int FMT>
__device__ __forceinline__ void p_stage(const PrefetchP<FMT> &P, SmemP &sm, int tid) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  const int row = tid & 127, half = tid >> 7;
  if constexpr (Q4) {
    // 8 codes of a word (byte b: k = 2b low nibble, 2b + 1 high nibble): 0x6400 | c is the fp16
    // 1024 + c, so subtracting 1032 gives c - 8 exactly; wh = (c - 8) s 2^8 rounded, wl = the rest.
    // The exact 2^8 (undone on the fp32 result) keeps wl out of the fp16 subnormals for weights
    // down to about 1e-3, so the pair stays exact there.
    const _Float16 sc = __builtin_bit_cast(_Float16, P.s) * (_Float16)256.0f;
    const h2 s2 = {sc, sc};
    const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t w = P.w[q];
      const uint32_t p0 = (w & 0x000F000Fu) | 0x64006400u;          // (k0, k4)
      const uint32_t p1 = ((w >> 4) & 0x000F000Fu) | 0x64006400u;   // (k1, k5)
      const uint32_t p2 = ((w >> 8) & 0x000F000Fu) | 0x64006400u;   // (k2, k6)
      const uint32_t p3 = ((w >> 12) & 0x000F000Fu) | 0x64006400u;  // (k3, k7)
      const h2 c01 = as_h2(__builtin_amdgcn_perm(p1, p0, 0x05040100u)) - off;
      const h2 c23 = as_h2(__builtin_amdgcn_perm(p3, p2, 0x05040100u)) - off;
      const h2 c45 = as_h2(__builtin_amdgcn_perm(p1, p0, 0x07060302u)) - off;
      const h2 c67 = as_h2(__builtin_amdgcn_perm(p3, p2, 0x07060302u)) - off;
      const h2 h01 = c01 * s2, h23 = c23 * s2, h45 = c45 * s2, h67 = c67 * s2;
      u32x4 vh, vl;
      vh.x = as_u(h01); vh.y = as_u(h23); vh.z = as_u(h45); vh.w = as_u(h67);
      vl.x = as_u(__builtin_elementwise_fma(c01, s2, -h01));
      vl.y = as_u(__builtin_elementwise_fma(c23, s2, -h23));
      vl.z = as_u(__builtin_elementwise_fma(c45, s2, -h45));
      vl.w = as_u(__builtin_elementwise_fma(c67, s2, -h67));
      *reinterpret_cast<u32x4 *>(&sm.wh[row][16 * half + 8 * q]) = vh;
      *reinterpret_cast<u32x4 *>(&sm.wl[row][16 * half + 8 * q]) = vl;
    }
  } else {
    // INT8 codes exactly: byte ^ 0x80 = c + 128, placed under 0x64 it is the fp16 1024 + c + 128
    const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t w0 = P.w[2 * q] ^ 0x80808080u, w1 = P.w[2 * q + 1] ^ 0x80808080u;
      u32x4 v;
      v.x = as_u(as_h2(__builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u)) - off);  // (c0, c1)
      v.y = as_u(as_h2(__builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u)) - off);  // (c2, c3)
      v.z = as_u(as_h2(__builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u)) - off);  // (c4, c5)
      v.w = as_u(as_h2(__builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u)) - off);  // (c6, c7)
      *reinterpret_cast<u32x4 *>(&sm.wh[row][16 * half + 8 * q]) = v;
    }
  }
  const int xr = tid >> 1;
  _Float16(*xs)[LDP] = (tid & 1) ? sm.xl : sm.xh;
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4 *>(&xs[xr][8 * i]) = P.x[i];
}

template <int FMT, int EPI, bool LO>
__global__ void __launch_bounds__(256) gemm_p_k(const GemmPArgs a) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  __shared__ SmemP sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int z = blockIdx.z;  // k-split
  const int wn = wave >> 1, wm = wave & 1;  // this wave's 64 x 64 quarter
  const int i16 = lane & 15, g = lane >> 4;
  f4 acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int h = 0; h < 4; ++h) acc[f][h] = f4{0.f, 0.f, 0.f, 0.f};
  const int nkt_all = a.K / BK;
  const int per = (nkt_all + a.ks - 1) / a.ks;
  const int kt0 = z * per, kt1 = min(nkt_all, kt0 + per);
  PrefetchP<FMT> P;
  if (kt0 < kt1) p_load<FMT, LO>(P, a, n0, m0, kt0, tid);
  for (int kt = kt0; kt < kt1; ++kt) {
    __syncthreads();  // the previous tile's fragments have been read
    p_stage<FMT>(P, sm, tid);
    __syncthreads();
    if (kt + 1 < kt1) p_load<FMT, LO>(P, a, n0, m0, kt + 1, tid);
    h8 wh[4], wl[4], xh[4], xl[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      wh[f] = *reinterpret_cast<const h8 *>(&sm.wh[wn * 64 + f * 16 + i16][g * 8]);
      if constexpr (Q4) wl[f] = *reinterpret_cast<const h8 *>(&sm.wl[wn * 64 + f * 16 + i16][g * 8]);
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      xh[h] = *reinterpret_cast<const h8 *>(&sm.xh[wm * 64 + h * 16 + i16][g * 8]);
      if constexpr (LO) xl[h] = *reinterpret_cast<const h8 *>(&sm.xl[wm * 64 + h * 16 + i16][g * 8]);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if constexpr (Q4) acc[f][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wl[f], xh[h], acc[f][h], 0, 0, 0);
        if constexpr (LO) acc[f][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh[f], xl[h], acc[f][h], 0, 0, 0);
        acc[f][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh[f], xh[h], acc[f][h], 0, 0, 0);
      }
  }
  // acc[f][h][r] = Y[m = m0 + 64 wm + 16 h + i16][n = n0 + 64 wn + 16 f + 4 g + r] (times 2^8 for INT4)
  constexpr float kUnscale = Q4 ? 0.00390625f : 1.0f;  // 2^-8, exact
  if constexpr (EPI == EPI_SWIGLU) {
    // the wave's 64 rows are one packed tile: rows 0..31 gate, 32..63 up of outputs 32 t + j
    const int t = (n0 >> 6) + wn;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int m = m0 + 64 * wm + 16 * h + i16;
      if (m >= a.M) continue;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 32 * t + 16 * f + 4 * g + r;
          if (i < a.N / 2) {
            float gv = acc[f][h][r] * kUnscale, uv = acc[f + 2][h][r] * kUnscale;
            if constexpr (!Q4) {  // INT8: the row scales of the packed gate and up rows
              const int ng = n0 + 64 * wn + 16 * f + 4 * g + r;
              gv *= reinterpret_cast<const float *>(a.S)[ng];
              uv *= reinterpret_cast<const float *>(a.S)[ng + 32];
            }
            const float v = silu(gv) * uv;
            if (a.Yh) {
              const _Float16 hi = (_Float16)v;
              a.Yh[(size_t)m * a.ldy + i] = __builtin_bit_cast(uint16_t, hi);
              a.Yl[(size_t)m * a.ldy + i] = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)hi));
            } else {
              a.Y[(size_t)m * a.ldy + i] = v;
            }
          }
        }
      }
    }
  } else if (a.ks > 1) {
    // this split's partial (unscaled for INT4's 2^8 already removed; the INT8 row scale, bias and
    // residual come in the reduce)
    float *pz = a.part + (size_t)z * a.M * a.N;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int m = m0 + 64 * wm + 16 * h + i16;
      if (m >= a.M) continue;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int nb = n0 + 64 * wn + 16 * f + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb + r < a.N) pz[(size_t)m * a.N + nb + r] = acc[f][h][r] * kUnscale;
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int m = m0 + 64 * wm + 16 * h + i16;
      if (m >= a.M) continue;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int nb = n0 + 64 * wn + 16 * f + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = nb + r;
          if (n >= a.N) continue;
          float v = acc[f][h][r] * kUnscale;
          if constexpr (FMT == QDEC_W_Q8_ROW) v *= reinterpret_cast<const float *>(a.S)[n];
          if (a.bias) v += a.bias[n];
          if (a.residual) v += a.residual[(size_t)m * a.ldy + n];
          a.Y[(size_t)m * a.ldy + n] = v;
        }
      }
    }
  }
}

// Y[m][n] = (sum over splits z in order of part[z][m][n]) (* INT8 row scale) (+ bias) (+ residual)
template <int FMT>
__global__ void __launch_bounds__(256) gemm_p_reduce_k(const GemmPArgs a) {
  const size_t total = (size_t)a.M * a.N;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / a.N), n = (int)(i % a.N);
    float v = 0.f;
    for (int z = 0; z < a.ks; ++z) v += a.part[(size_t)z * total + i];
    if constexpr (FMT == QDEC_W_Q8_ROW) v *= reinterpret_cast<const float *>(a.S)[n];
    if (a.bias) v += a.bias[n];
    if (a.residual) v += a.residual[(size_t)m * a.ldy + n];
    a.Y[(size_t)m * a.ldy + n] = v;
  }
}

template <int FMT, int EPI>
hipError_t launch_lo_p(const GemmPArgs &a, dim3 grid, hipStream_t st) {
  if (a.Xl)
    hipLaunchKernelGGL((gemm_p_k<FMT, EPI, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_p_k<FMT, EPI, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt_p(const GemmPArgs &a0, hipStream_t st) {
  GemmPArgs a = a0;
  if (a.ks < 1 || a.epi == EPI_SWIGLU || !a.part) a.ks = 1;
  const int npad = ((a.N + kTile - 1) / kTile) * kTile;
  dim3 grid((a.M + BM - 1) / BM, (npad + BN - 1) / BN, a.ks);
  hipError_t e = a.epi == EPI_SWIGLU ? launch_lo_p<FMT, EPI_SWIGLU>(a, grid, st) : launch_lo_p<FMT, EPI_STORE>(a, grid, st);
  if (e != hipSuccess || a.ks == 1) return e;
  const size_t total = (size_t)a.M * a.N;
  size_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(gemm_p_reduce_k<FMT>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int gemm_p_splits(int M, int N, int K, int epi) {
  if (epi == EPI_SWIGLU) return 1;
  const int npad = ((N + kTile - 1) / kTile) * kTile;
  const int tiles = ((M + BM - 1) / BM) * ((npad + BN - 1) / BN);
  int ks = 1;
  while (ks < 8 && tiles * ks < 512 && (K / BK) / (2 * ks) >= 16) ks *= 2;  // >= 16 k-tiles per split
  return ks;
}

hipError_t launch_gemm_p(int wfmt, const GemmPArgs &a, hipStream_t st) {
  return wfmt == QDEC_W_Q4_G_ZP8 ? launch_fmt_p<QDEC_W_Q4_G_ZP8>(a, st) : launch_fmt_p<QDEC_W_Q8_ROW>(a, st);
}

}  // namespace qdec
