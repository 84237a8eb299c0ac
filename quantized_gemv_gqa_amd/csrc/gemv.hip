// Weight-only-quantized GEMV with fused dequant for gfx950 (wave64).
//
// What it computes: y[n] = sum_k w[n][k] x[k] with INT8 per-row or INT4 group-scaled weights,
// fp32 activations and fp32 accumulation ("How To Construct Your Personal LLM Runtime From
// Scratch", section 7: mask a 4-bit code, apply the zero point, scale by the group's fp16 scale,
// accumulate in fp32; FlashQwen README, "Optimization study" stage 8: INT8 codes with one scale
// per output row dequantized inside the GEMV).
//
// How, on CDNA4: the pages' GEMVs give each output row to a warp and reduce across lanes.  Here a
// wave owns a tile of 64 output rows, one row per lane, so
//   * every weight load is one coalesced 1 KiB wave access (the packed "tile64" layout puts the
//     16-byte runs of 64 rows side by side),
//   * the activation chunk is the same for all lanes and is broadcast through scalar registers
//     (v_readlane), so there is no LDS staging and no cross-lane reduction of the dot product,
//   * the K dimension is split across waves to fill the 256 CUs when N is small; partial sums
//     go to a workspace and the last wave to arrive at a tile adds them in a fixed order
//     (deterministic, no float atomics) and runs the epilogue.
// INT4 codes are unpacked with one AND (low nibbles) and one shift+AND (high nibbles) per 8
// codes, then v_cvt_f32_ubyte{0..3}; the zero point is folded out of the inner loop:
//   sum_k (c_k - 8) x_k = sum_k c_k x_k - 8 sum_k x_k,  with sum_k x_k computed once per chunk.
// INT8 codes are biased to unsigned by XOR 0x80 (c + 128) and folded the same way.
#include <hip/hip_runtime.h>

#include <climits>

#include "qdec_internal.h"

namespace qdec {

namespace {

constexpr int kTargetUnits = 2048;  // ~8 waves per CU on 256 CUs
constexpr int kMinChunks = 4;       // at least 4 KiB of weights per wave
constexpr int kBatch = 8;           // 16-byte runs loaded per lane before computing
constexpr size_t kCounterBytes = 64 * 1024;                       // arrival counters region
constexpr int kArgmaxCounter = (int)(kCounterBytes / sizeof(unsigned)) - 1;  // last slot
constexpr int kMaxSplitTiles = kArgmaxCounter;                    // larger N: no split

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// DPP lane permutation of a float (gfx9 dpp_ctrl encodings)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// sum over aligned groups of 8 lanes; every lane of the group gets the same value
__device__ __forceinline__ float sum8(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror: lane i <-> 7 - i within each 8
  return v;
}

// The AND masks are kept opaque so the backend cannot fold them into per-nibble bit-field
// extracts: with the masks in place, each byte converts with one v_cvt_f32_ubyteN.
__device__ __forceinline__ uint32_t and_opaque(uint32_t v, uint32_t m) {
  uint32_t r;
  asm volatile("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(m), "v"(v));
  return r;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// (value, index) wave reduction: larger value wins, the smaller index on equal values;
// index INT_MAX marks "no candidate"
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v2 = __shfl_xor(v, o, 64);
    const int i2 = __shfl_xor(i, o, 64);
    if (i2 != INT_MAX && (i == INT_MAX || v2 > v || (v2 == v && i2 < i))) {
      v = v2;
      i = i2;
    }
  }
}

__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xFFu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xFFu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xFFu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }

// INT4: sum_k c_k x_k over the 32 codes of one 16-byte run.  xs holds the run's activations in
// k order with odd k pre-divided by 16: high nibbles are masked in place (value 16 c), so
// 16 c * (x / 16) = c x exactly.
__device__ __forceinline__ float dot_q4_run(u32x4 w, const f32x4 (&xs)[8]) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = and_opaque(wd[q], 0x0F0F0F0Fu);  // k = 8q + 0, 2, 4, 6
    const uint32_t hi = and_opaque(wd[q], 0xF0F0F0F0u);  // k = 8q + 1, 3, 5, 7 (times 16)
    const f32x4 xa = xs[2 * q], xb = xs[2 * q + 1];      // k = 8q .. 8q+3, 8q+4 .. 8q+7
    a0 = fmaf(ub0(lo), xa.x, a0);
    a1 = fmaf(ub0(hi), xa.y, a1);
    a0 = fmaf(ub1(lo), xa.z, a0);
    a1 = fmaf(ub1(hi), xa.w, a1);
    a0 = fmaf(ub2(lo), xb.x, a0);
    a1 = fmaf(ub2(hi), xb.y, a1);
    a0 = fmaf(ub3(lo), xb.z, a0);
    a1 = fmaf(ub3(hi), xb.w, a1);
  }
  return a0 + a1;
}

// INT8: sum_k (c_k + 128) x_k over the 16 codes of one 16-byte run
__device__ __forceinline__ float dot_q8_run(u32x4 w, const f32x4 (&xs)[4]) {
  const uint32_t wd[4] = {w.x ^ 0x80808080u, w.y ^ 0x80808080u, w.z ^ 0x80808080u,
                          w.w ^ 0x80808080u};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 xa = xs[q];
    a0 = fmaf(ub0(wd[q]), xa.x, a0);
    a1 = fmaf(ub1(wd[q]), xa.y, a1);
    a0 = fmaf(ub2(wd[q]), xa.z, a0);
    a1 = fmaf(ub3(wd[q]), xa.w, a1);
  }
  return a0 + a1;
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3: 32-bit data format).
// Loads through it take an SGPR base and a 32-bit VGPR offset (no per-lane 64-bit address math)
// and return zero instead of faulting outside [0, bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kAuxStream = 2;  // nt: weights are read once per step, do not keep them in L2
constexpr int kAuxSc1 = 16;    // sc1: device-coherent access (bypasses non-coherent L2 copies)

// Per-wave LDS staging of one batch of activations: up to kBatch runs of CK values (odd k / 16
// for INT4) followed by the runs' sums of the true values.
template <int CK>
struct Stage {
  float x[kBatch * CK];
  float sum[kBatch];
};

// Stage NB runs starting at run c.  Lane l covers values 4l .. 4l+3 of the batch; CK/4 lanes
// cover one run.
template <int CK, int NB, bool NORM>
__device__ __forceinline__ void stage_batch(Stage<CK> &sm, __amdgpu_buffer_rsrc_t xr,
                                            __amdgpu_buffer_rsrc_t gr, int c, int lane) {
  constexpr int LPR = CK / 4;  // lanes per run
  const bool active = lane < NB * LPR;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    const int soff = c * CK * 4;
    v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, lane * 16, soff, 0));
    if constexpr (NORM)
      v *= __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(gr, lane * 16, soff, 0));
  }
  float part = (v.x + v.y) + (v.z + v.w);
  if constexpr (LPR == 8) {
    part = sum8(part);
  } else {
    static_assert(LPR == 4, "runs of 16 or 32 values");
    part += dpp<0xB1>(part);
    part += dpp<0x4E>(part);
  }
  if constexpr (CK == 32) {  // odd k carry 1/16 (exact power-of-two scaling)
    v.y *= 0.0625f;
    v.w *= 0.0625f;
  }
  if (active) {
    *reinterpret_cast<f32x4 *>(&sm.x[4 * lane]) = v;
    if (lane % LPR == 0) sm.sum[lane / LPR] = part;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One batch of NB 16-byte runs starting at run cb: all weight and scale loads are issued first,
// then the activations are staged, then the dot products run.
template <int FMT, bool NORM, int NB>
__device__ __forceinline__ void run_batch(float &acc, Stage<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16> &sm,
                                          __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                          __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t gr,
                                          int cb, int gshift, int lane) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  constexpr int RV = CK / 4;
  constexpr float ZP = Q4 ? 8.0f : 128.0f;
  u32x4 wv[NB];
  uint16_t sraw[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    wv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, lane * 16, (cb + i) * (kTile * 16), kAuxStream));
    if constexpr (Q4)
      sraw[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, lane * 2, ((cb + i) >> gshift) * (kTile * 2), 0);
  }
  stage_batch<CK, NB, NORM>(sm, xr, gr, cb, lane);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    f32x4 xs[RV];
#pragma unroll
    for (int r = 0; r < RV; ++r) xs[r] = *reinterpret_cast<const f32x4 *>(&sm.x[i * CK + 4 * r]);
    const float xsum = sm.sum[i];
    if constexpr (Q4) {
      const float d = dot_q4_run(wv[i], xs);
      acc = fmaf(half_bits_to_float(sraw[i]), d - ZP * xsum, acc);
    } else {
      acc += dot_q8_run(wv[i], xs) - ZP * xsum;
    }
  }
  __builtin_amdgcn_wave_barrier();  // the next batch overwrites this wave's stage
}

template <int FMT, bool NORM, int EPI>
__global__ void __launch_bounds__(256) gemv_tile64(const GemvArgs a) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;  // k per 16-byte run
  __shared__ Stage<CK> stage_all[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Stage<CK> &sm = stage_all[wave];
  const int ks = a.ks, K = a.K, N = a.N;
  const int unit = blockIdx.x * 4 + wave;
  if (unit >= ((N + kTile - 1) / kTile) * ks) return;  // whole wave
  const int tile = unit / ks;
  const int ksi = unit - tile * ks;
  const int nch = K / CK;
  const int c0 = ksi * a.cps;
  const int c1 = min(nch, c0 + a.cps);
  const int gshift = a.group;  // Q4: log2(group / 32), set by the launcher
  const uint32_t tile_bytes = (uint32_t)nch * kTile * 16;
  const __amdgpu_buffer_rsrc_t wr = rsrc(a.W + (size_t)tile * tile_bytes, tile_bytes);
  __amdgpu_buffer_rsrc_t sr = wr;
  if constexpr (Q4) {
    const uint32_t sbytes = (uint32_t)((nch >> gshift) * kTile * 2);
    sr = rsrc(reinterpret_cast<const uint8_t *>(a.S) + (size_t)tile * sbytes, sbytes);
  }
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.x, (uint32_t)K * 4);
  const __amdgpu_buffer_rsrc_t gr = NORM ? rsrc(a.gamma, (uint32_t)K * 4) : xr;
  float *const part = a.part;
  unsigned *const counters = a.counters;

  float acc = 0.f;
  int cb = c0;
  for (; cb + kBatch <= c1; cb += kBatch) run_batch<FMT, NORM, kBatch>(acc, sm, wr, sr, xr, gr, cb, gshift, lane);
  const int rem = c1 - cb;
  if (rem & 4) { run_batch<FMT, NORM, 4>(acc, sm, wr, sr, xr, gr, cb, gshift, lane); cb += 4; }
  if (rem & 2) { run_batch<FMT, NORM, 2>(acc, sm, wr, sr, xr, gr, cb, gshift, lane); cb += 2; }
  if (rem & 1) { run_batch<FMT, NORM, 1>(acc, sm, wr, sr, xr, gr, cb, gshift, lane); }

  if (ks > 1) {
    // Split-K hand-off between waves that may sit on different XCDs.  Partials travel as
    // device-coherent (sc1) stores and loads, which bypass the per-XCD L2's non-coherent copies,
    // so no L2 write-back / invalidate is needed.  The wave waits for its partial store to be
    // acknowledged before it counts its arrival; the wave that completes the count therefore
    // finds every partial of the tile in coherent memory.
    float *pp = part + (size_t)tile * ks * kTile + lane;
    __hip_atomic_store(pp + (size_t)ksi * kTile, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    unsigned prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (unsigned)(ks - 1)) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // sc1 buffer loads (not atomics, so they pipeline); summed in a fixed order so the result
    // does not depend on which wave arrived last
    const __amdgpu_buffer_rsrc_t pr = rsrc(part + (size_t)tile * ks * kTile, (uint32_t)ks * kTile * 4);
    acc = 0.f;
    int i = 0;
    for (; i + 8 <= ks; i += 8) {
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        t[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, lane * 4, (i + j) * kTile * 4, kAuxSc1));
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += t[j];
    }
    for (; i < ks; ++i)
      acc += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, lane * 4, i * kTile * 4, kAuxSc1));
    if (lane == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ------------------------------------------------------------------ epilogue (one tile)
  float v = acc;
  if constexpr (NORM) {
    float t = 0.f;
    for (int i = lane; i < a.ssq_n; i += 64) t += a.ssq[i];
    const float ms = wave_sum(t) / (float)K;
    v *= rsqrtf(ms + a.eps);
  }
  const int n = tile * kTile + lane;
  if constexpr (FMT == QDEC_W_Q8_ROW) v *= reinterpret_cast<const float *>(a.S)[n];  // padded to tiles
  if constexpr (EPI == EPI_STORE || EPI == EPI_ARGMAX) {
    const bool valid = n < N;
    if (valid) {
      if (a.bias) v += a.bias[n];
      if (a.residual) v += a.residual[n];
      a.y[n] = v;
    }
    if (EPI == EPI_STORE && a.ssq_out) {
      const float sq = wave_sum(valid ? v * v : 0.f);
      if (lane == 0) a.ssq_out[tile] = sq;
    }
    if constexpr (EPI == EPI_ARGMAX) {
      // tile candidate: largest value, smallest row on ties (NaN never wins)
      float bv = (valid && v == v) ? v : -INFINITY;
      int bi = (valid && v == v) ? n : INT_MAX;
      wave_argmax(bv, bi);
      if (lane == 0) {
        __hip_atomic_store(&a.cand[2 * tile], bv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.cand[2 * tile + 1], __builtin_bit_cast(float, bi), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      const int tiles = (N + kTile - 1) / kTile;
      unsigned prev = 0;
      if (lane == 0)
        prev = __hip_atomic_fetch_add(&a.counters[kArgmaxCounter], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prev = __builtin_amdgcn_readfirstlane(prev);
      if (prev != (unsigned)(tiles - 1)) return;
      // last tile: reduce every tile's candidate
      const __amdgpu_buffer_rsrc_t cr = rsrc(a.cand, (uint32_t)tiles * 8);
      float gv = -INFINITY;
      int gi = INT_MAX;
      for (int t = lane; t < tiles; t += 64) {
        const float cv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(cr, t * 8, 0, kAuxSc1));
        const int ci = (int)__builtin_amdgcn_raw_buffer_load_b32(cr, t * 8 + 4, 0, kAuxSc1);
        if (ci != INT_MAX && (gi == INT_MAX || cv > gv || (cv == gv && ci < gi))) {
          gv = cv;
          gi = ci;
        }
      }
      wave_argmax(gv, gi);
      if (lane == 0) {
        const int tok = (gi == INT_MAX) ? 0 : gi;
        *a.token = tok;
        if (a.token_log && a.step_count) {
          const int st = *a.step_count;
          if (st >= 0 && st < a.log_len) a.token_log[st] = tok;
        }
        if (a.step_count) *a.step_count += 1;
        if (a.pos) *a.pos += 1;
        __hip_atomic_store(&a.counters[kArgmaxCounter], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  } else {
    // lanes 0..31: gate rows 32 tile + lane; lanes 32..63: the matching up rows
    const float u = __shfl(v, lane + 32, 64);
    const int i = tile * 32 + lane;
    if (lane < 32 && i < N / 2) a.y[i] = silu(v) * u;
  }
}

template <int FMT>
__global__ void pack_tile64(const uint4 *__restrict__ W, int N, int K, uint4 *__restrict__ Wp) {
  constexpr int CK = (FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16;
  const int nch = K / CK;
  const int tiles = (N + kTile - 1) / kTile;
  const size_t total = (size_t)tiles * nch * kTile;
  const size_t row16 = (size_t)nch;  // 16-byte runs per source row
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(idx % kTile);
    const size_t tc = idx / kTile;
    const int c = (int)(tc % nch);
    const int t = (int)(tc / nch);
    const int n = t * kTile + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n < N) v = W[(size_t)n * row16 + c];
    Wp[idx] = v;
  }
}

__global__ void pack_scales_q4(const uint16_t *__restrict__ S, int N, int ng, uint16_t *__restrict__ Sp) {
  const int tiles = (N + kTile - 1) / kTile;
  const size_t total = (size_t)tiles * ng * kTile;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(idx % kTile);
    const size_t tg = idx / kTile;
    const int g = (int)(tg % ng);
    const int t = (int)(tg / ng);
    const int n = t * kTile + r;
    Sp[idx] = (n < N) ? S[(size_t)n * ng + g] : (uint16_t)0;
  }
}

__global__ void pack_scales_q8(const float *__restrict__ S, int N, int Npad, float *__restrict__ Sp) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < Npad; i += gridDim.x * blockDim.x)
    Sp[i] = (i < N) ? S[i] : 0.f;
}

template <int FMT, bool NORM, int EPI>
hipError_t launch_t(const GemvArgs &a0, const GemvPlan &p, hipStream_t st) {
  GemvArgs a = a0;
  a.ks = p.ks;
  a.cps = p.cps;
  int gshift = 0;
  if (FMT == QDEC_W_Q4_G_ZP8)
    while ((32 << gshift) < a0.group) ++gshift;  // group = 32 << gshift (checked by the callers)
  a.group = gshift;
  hipLaunchKernelGGL((gemv_tile64<FMT, NORM, EPI>), dim3(p.blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int FMT, bool NORM>
hipError_t launch_e(const GemvArgs &a, const GemvPlan &p, hipStream_t st) {
  switch (a.epi) {
    case EPI_SWIGLU: return launch_t<FMT, NORM, EPI_SWIGLU>(a, p, st);
    case EPI_ARGMAX: return launch_t<FMT, NORM, EPI_ARGMAX>(a, p, st);
    default: return launch_t<FMT, NORM, EPI_STORE>(a, p, st);
  }
}

}  // namespace

GemvPlan gemv_plan(int wfmt, int N, int K, bool allow_split) {
  GemvPlan p;
  const int ck = (wfmt == QDEC_W_Q4_G_ZP8) ? 32 : 16;
  p.tiles = (N + kTile - 1) / kTile;
  p.nch = K / ck;
  int ks = 1;
  if (allow_split && p.tiles <= kMaxSplitTiles) {
    ks = (kTargetUnits + p.tiles / 2) / p.tiles;
    ks = max(1, min(ks, p.nch / kMinChunks));
  }
  p.cps = (p.nch + ks - 1) / ks;
  p.ks = (p.nch + p.cps - 1) / p.cps;
  p.units = p.tiles * p.ks;
  p.blocks = (p.units + 3) / 4;
  return p;
}

// Workspace layout, shared by every GEMV that runs on it one after another: the tile arrival
// counters sit in a fixed region at the start (each launch leaves the ones it used at zero, so
// the region stays zero between launches whatever the shape), the split-K partials follow.
size_t gemv_workspace_bytes(int wfmt, int N, int K, bool argmax) {
  GemvPlan p = gemv_plan(wfmt, N, K, true);
  size_t b = kCounterBytes;
  if (p.ks > 1) b += (size_t)p.tiles * p.ks * kTile * sizeof(float);
  if (argmax) b += (size_t)p.tiles * 2 * sizeof(float);
  return b;
}

void gemv_bind_workspace(GemvArgs &a, const GemvPlan &p, void *ws) {
  a.counters = reinterpret_cast<unsigned *>(ws);
  a.part = ws ? reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + kCounterBytes) : nullptr;
  a.cand = ws ? a.part + (p.ks > 1 ? (size_t)p.tiles * p.ks * kTile : 0) : nullptr;
}

hipError_t launch_gemv(int wfmt, const GemvArgs &a, const GemvPlan &p, hipStream_t st) {
  const bool norm = a.gamma != nullptr;
  if (wfmt == QDEC_W_Q4_G_ZP8)
    return norm ? launch_e<QDEC_W_Q4_G_ZP8, true>(a, p, st) : launch_e<QDEC_W_Q4_G_ZP8, false>(a, p, st);
  return norm ? launch_e<QDEC_W_Q8_ROW, true>(a, p, st) : launch_e<QDEC_W_Q8_ROW, false>(a, p, st);
}

hipError_t launch_pack_q8(const int8_t *W, const float *S, int N, int K, uint8_t *Wp, float *Sp,
                          hipStream_t st) {
  hipLaunchKernelGGL(pack_tile64<QDEC_W_Q8_ROW>, dim3(2048), dim3(256), 0, st,
                     reinterpret_cast<const uint4 *>(W), N, K, reinterpret_cast<uint4 *>(Wp));
  const int npad = ((N + kTile - 1) / kTile) * kTile;
  hipLaunchKernelGGL(pack_scales_q8, dim3((npad + 255) / 256), dim3(256), 0, st, S, N, npad, Sp);
  return hipGetLastError();
}

hipError_t launch_pack_q4(const uint8_t *W, const uint16_t *S, int N, int K, int group, uint8_t *Wp,
                          uint16_t *Sp, hipStream_t st) {
  hipLaunchKernelGGL(pack_tile64<QDEC_W_Q4_G_ZP8>, dim3(2048), dim3(256), 0, st,
                     reinterpret_cast<const uint4 *>(W), N, K, reinterpret_cast<uint4 *>(Wp));
  hipLaunchKernelGGL(pack_scales_q4, dim3(1024), dim3(256), 0, st, S, N, K / group, Sp);
  return hipGetLastError();
}

}  // namespace qdec
