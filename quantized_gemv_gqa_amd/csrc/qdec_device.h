// Device-side building blocks shared by the per-op kernels and the fused layer kernels (gfx950,
// wave64).  Everything here runs inside one wave unless a comment says otherwise.
#pragma once
#include <hip/hip_runtime.h>

#include <climits>

#include "qdec_internal.h"

namespace qdec {
namespace dev {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte weight runs a lane loads before computing.  Four (with the next four in flight) keep
// the INT4 GEMV under 100 VGPRs, four or five waves per SIMD; eight ran at three waves per SIMD
// and made the 7B decode step 5 % slower, two or three left too few bytes in flight.
constexpr int kBatch = 4;
constexpr int kAuxStream = 2;   // nt: weights are read once per step, do not keep them in L2
constexpr int kAuxSc1 = 16;     // sc1: device-coherent access (bypasses non-coherent L2 copies)
constexpr unsigned kSpinLimit = 1u << 24;  // bounded waits: ~1 s of polling, then give up
constexpr unsigned kLayerSpinLimit = 1u << 22;  // backed-off polls of the layer kernels: ~3.5 s
constexpr float kNegBig = -1e30f;          // finite "minus infinity" for running maxima
#ifndef QDEC_COMBINE_BURST
#define QDEC_COMBINE_BURST 32
#endif
constexpr int kCombineBurst = QDEC_COMBINE_BURST;  // split-K partials a combining wave requests at once

// ------------------------------------------------------------------------------ small helpers
// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3: 32-bit data format).
// Loads through it take an SGPR base and a 32-bit VGPR offset and return zero outside
// [0, bytes) instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Workgroup barrier for data that waves exchange through LDS with ordinary LDS instructions: the
// wave's own LDS accesses are complete (lgkmcnt 0) before it arrives, and the compiler moves no
// memory access across it.  Unlike __syncthreads() it does not wait for the wave's LDS DMA copies
// (a workgroup fence counts them as LDS writes): a wave whose DMA copies into a buffer that only it
// reads does not hold the others for them (its own later LDS reads still wait for them).
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
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
// sum over aligned groups of 16 lanes
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  v += dpp<0x140>(v);  // row_mirror: lane i <-> 15 - i within each 16
  return v;
}

// Whole-wave reductions without LDS: finish each 16-lane row with DPP, then fold rows with the
// row broadcasts (lane 15 into row 1 and lane 47 into row 3, then lane 31 into rows 2 and 3), so
// lane 63 holds the result; it is read back as a wave-uniform value.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_rows(float v, float old) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  v += dpp_rows<0x142, 0xA>(v, 0.f);  // row_bcast:15
  v += dpp_rows<0x143, 0xC>(v, 0.f);  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  v = fmaxf(v, dpp_rows<0x142, 0xA>(v, -INFINITY));
  v = fmaxf(v, dpp_rows<0x143, 0xC>(v, -INFINITY));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Exchange with the lane 16 (32) apart: every lane gets the pair (even-row value, odd-row value)
// ((lower-half value, upper-half value)), in the same order on both lanes of a pair.
__device__ __forceinline__ void pair16(float v, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v), false, false);
  // (elements are copied out before the cast: a cast of r[1] itself reads element 0)
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void pair32(float v, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v), false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
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

__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x7FFFFFu)) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

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

// Cross-workgroup data: device-coherent stores/loads (sc1) when COH, plain otherwise.
template <bool COH>
__device__ __forceinline__ void st_f(float *p, float v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool COH>
__device__ __forceinline__ float ld_f(const float *p) {
  if constexpr (COH)
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

// Wait until every store this wave issued is acknowledged (so a later counter update cannot be
// seen before them), with compiler fences so no memory access moves across.
__device__ __forceinline__ void drain_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Bounded device-coherent polls for the step-synchronised kernels.  A wait that exceeds
// kLayerSpinLimit polls (about 3.5 s) sets *err and gives up; once *err is set every other wait gives up within 1024
// polls, so a failed step ends (with wrong values and the error word set) instead of hanging.
__device__ __forceinline__ bool ge_u32(unsigned v, unsigned target) { return (int)(v - target) >= 0; }

// Polls back off from ~25 ns to ~0.85 us between reads: a waiting wave's device-coherent reads
// go past the L2, and hundreds of waves polling at full rate take memory bandwidth from the
// producers they wait for.
__device__ __forceinline__ void poll_pause(unsigned spins) {
  if (spins < 8)
    __builtin_amdgcn_s_sleep(1);
  else
    __builtin_amdgcn_s_sleep(8);
}

// One step of a poll loop: pause, then give up (false) once the step's error word is set (checked
// every 1024 polls) or after kLayerSpinLimit polls (setting it).
__device__ inline bool poll_step(unsigned &spins, unsigned *err) {
  poll_pause(spins);
  ++spins;
  if ((spins & 1023u) == 0 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return false;
  if (spins > kLayerSpinLimit) {
    __hip_atomic_store(err, kErrWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  return true;
}

// one thread: *p >= target
__device__ inline bool poll_count(const unsigned *p, unsigned target, unsigned *err) {
  unsigned spins = 0;
  while (!ge_u32(__hip_atomic_load(const_cast<unsigned *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), target)) {
    poll_pause(spins);
    ++spins;
    if ((spins & 1023u) == 0 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return false;
    if (spins > kLayerSpinLimit) {
      __hip_atomic_store(err, kErrWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return true;
}

// whole wave: flags[f] >= target for every f in [f0, f1] (the lanes poll 64 flags at a time)
__device__ inline bool poll_flags(const unsigned *flags, int f0, int f1, unsigned target, unsigned *err, int lane) {
  for (int base = f0; base <= f1; base += 64) {
    const int f = base + lane;
    unsigned spins = 0;
    for (;;) {
      const bool ok = f > f1 ||
                      ge_u32(__hip_atomic_load(const_cast<unsigned *>(flags + f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), target);
      if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
      poll_pause(spins);
      ++spins;
      if ((spins & 1023u) == 0 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return false;
      if (spins > kLayerSpinLimit) {
        if (lane == 0) __hip_atomic_store(err, kErrWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return true;
}

// Timeline marks (diagnostics): lane 0 stores the 100 MHz device clock at slot i of a wave's
// record when the record pointer is set.
__device__ __forceinline__ void mark(unsigned long long *rec, int i) {
  if (rec && (threadIdx.x & 63) == 0) rec[i] = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xFFu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xFFu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xFFu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }

// ------------------------------------------------------------------------------ GEMV pieces
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

// INT4 with mixed-precision FMAs: 2^-24 sum_k c_k x_k over the 32 codes of one 16-byte run, xs
// holding the run's true activations in k order.  Masking a word with 0x000F000F leaves two codes
// in the low bits of its 16-bit halves; read as fp16 bit patterns these are exact subnormals
// c * 2^-24, and with 0x00F000F0 they are 16 c * 2^-24.  v_fma_mix_f32 multiplies such a half by
// an fp32 activation in fp32, so eight codes cost four masks, one shift and eight FMAs (instead
// of two masks, eight conversions and eight FMAs).  fp16 subnormals are kept: the kernels run in
// the IEEE denormal mode for 16-bit values.
__device__ __forceinline__ float lo_half(uint32_t m) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(m & 0xFFFFu)); }
__device__ __forceinline__ float hi_half(uint32_t m) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(m >> 16)); }
__device__ __forceinline__ float dot_q4_mix(u32x4 w, const f32x4 (&xs)[8]) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float a0 = 0.f, a1 = 0.f;  // a0: codes of even k (times 2^-24); a1: odd k (times 16 * 2^-24)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // byte b of word q holds k = 8q + 2b (low nibble) and 8q + 2b + 1 (high nibble)
    const uint32_t v = wd[q], s = v >> 8;
    const uint32_t e02 = and_opaque(v, 0x000F000Fu);  // k = 8q, 8q + 4
    const uint32_t o02 = and_opaque(v, 0x00F000F0u);  // k = 8q + 1, 8q + 5
    const uint32_t e13 = and_opaque(s, 0x000F000Fu);  // k = 8q + 2, 8q + 6
    const uint32_t o13 = and_opaque(s, 0x00F000F0u);  // k = 8q + 3, 8q + 7
    const f32x4 xa = xs[2 * q], xb = xs[2 * q + 1];   // k = 8q .. 8q+3, 8q+4 .. 8q+7
    a0 = __builtin_fmaf(lo_half(e02), xa.x, a0);
    a1 = __builtin_fmaf(lo_half(o02), xa.y, a1);
    a0 = __builtin_fmaf(lo_half(e13), xa.z, a0);
    a1 = __builtin_fmaf(lo_half(o13), xa.w, a1);
    a0 = __builtin_fmaf(hi_half(e02), xb.x, a0);
    a1 = __builtin_fmaf(hi_half(o02), xb.y, a1);
    a0 = __builtin_fmaf(hi_half(e13), xb.z, a0);
    a1 = __builtin_fmaf(hi_half(o13), xb.w, a1);
  }
  return __builtin_fmaf(a1, 0.0625f, a0);
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

// One batch of a wave's work: kBatch 16-byte weight runs per lane, their scales (INT4), and the
// batch's activations (kBatch * CK values, four per lane) with the RMSNorm gain.
template <int FMT, bool NORM>
struct GemvBatch {
  u32x4 w[kBatch];
  uint16_t s[kBatch];
  f32x4 x, g;
};

// Per-wave LDS copy of a batch's activations and the runs' zero-point terms: 128 times the run's
// sum for INT8, 8 * 2^-24 times it for INT4 (the scale of dot_q4_mix).
template <int CK>
struct Stage {
  float x[kBatch * CK];
  float zp[kBatch];
};

// Issue the loads of runs r .. r + kBatch - 1 (relative to the wave's first run): weights and
// scales (load_weights), activations and gain (load_acts).  The resources cover exactly the wave's
// runs, scale groups and activations, so loads past its end read zero (and contribute nothing);
// the whole offset is in the VGPR operand, which the range check uses.  XCOH: the activations
// were written earlier in the same kernel by other workgroups (device-coherent loads).
template <int FMT, bool NORM>
__device__ __forceinline__ void load_weights(GemvBatch<FMT, NORM> &B, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                             int r, int c0, int g0, int gshift, int lane) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  const uint32_t base = (uint32_t)r * (kTile * 16) + lane * 16;
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    B.w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, base + i * (kTile * 16), 0, kAuxStream));
    if constexpr (Q4) {
      const int g = ((c0 + r + i) >> gshift) - g0;
      B.s[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, (uint32_t)g * (kTile * 2) + lane * 2, 0, 0);
    }
  }
}
template <int FMT, bool NORM, bool XCOH>
__device__ __forceinline__ void load_acts(GemvBatch<FMT, NORM> &B, __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t gr,
                                          int r, int lane) {
  constexpr int CK = (FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16;
  const uint32_t xo = (lane * 4 < kBatch * CK) ? (uint32_t)(r * CK + lane * 4) * 4u : 0x80000000u;
  B.x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xo, 0, XCOH ? kAuxSc1 : 0));
  if constexpr (NORM) B.g = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(gr, xo, 0, 0));
}
template <int FMT, bool NORM, bool XCOH>
__device__ __forceinline__ void load_batch(GemvBatch<FMT, NORM> &B, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                           __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t gr, int r, int c0, int g0,
                                           int gshift, int lane) {
  load_weights<FMT, NORM>(B, wr, sr, r, c0, g0, gshift, lane);
  load_acts<FMT, NORM, XCOH>(B, xr, gr, r, lane);
}

// Stage a batch's activations in the wave's LDS slot, then accumulate its runs into acc (INT4:
// times 2^-24).
template <int FMT, bool NORM>
__device__ __forceinline__ void compute_batch(float &acc, const GemvBatch<FMT, NORM> &B,
                                              Stage<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16> &sm, int lane) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  constexpr int LPR = CK / 4;  // lanes per run
  constexpr int RV = CK / 4;
  f32x4 v = B.x;
  if constexpr (NORM) v *= B.g;
  float part = (v.x + v.y) + (v.z + v.w);
  if constexpr (LPR == 8) {
    part = sum8(part);
  } else {
    static_assert(LPR == 4, "runs of 16 or 32 values");
    part += dpp<0xB1>(part);
    part += dpp<0x4E>(part);
  }
  if (lane * 4 < kBatch * CK) {
    *reinterpret_cast<f32x4 *>(&sm.x[4 * lane]) = v;
    if (lane % LPR == 0) sm.zp[lane / LPR] = part * (Q4 ? 4.76837158203125e-07f : 128.0f);  // 2^-21 (exact)
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    f32x4 xs[RV];
#pragma unroll
    for (int q = 0; q < RV; ++q) xs[q] = *reinterpret_cast<const f32x4 *>(&sm.x[i * CK + 4 * q]);
    const float zp = sm.zp[i];
    if constexpr (Q4)
      acc = fmaf(half_bits_to_float(B.s[i]), dot_q4_mix(B.w[i], xs) - zp, acc);
    else
      acc += dot_q8_run(B.w[i], xs) - zp;
  }
  __builtin_amdgcn_wave_barrier();  // the batch after next overwrites this slot
}

// Split-K hand-off between waves that may sit on different XCDs: partials travel as sc1
// stores/loads (no L2 write-back or invalidate needed); a wave counts its arrival only after its
// partial store is acknowledged, so the wave completing the count finds every partial.  Returns
// false on every wave but the last of the tile; the last gets the tile's sum in acc, added in
// split order (sc1 buffer loads, not atomics, so they pipeline), and resets the counter.
__device__ __forceinline__ bool splitk_combine(float &acc, float *part, unsigned *counters, int tile, int ks, int ksi,
                                               int lane) {
  float *pp = part + (size_t)tile * ks * kTile + lane;
  __hip_atomic_store(pp + (size_t)ksi * kTile, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  drain_stores();
  unsigned *ctr = counters + tile * kLine;
  unsigned prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev != (unsigned)(ks - 1)) return false;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const __amdgpu_buffer_rsrc_t pr = rsrc(part + (size_t)tile * ks * kTile, (uint32_t)ks * kTile * 4);
  // every partial of a burst is requested at once (one round trip per 32 splits; loads past the
  // last split read zero), then added in split order
  acc = 0.f;
  for (int i = 0; i < ks; i += kCombineBurst) {
    float t[kCombineBurst];
#pragma unroll
    for (int j = 0; j < kCombineBurst; ++j) {
      t[j] = 0.f;
      if (i + (j & ~7) < ks)  // whole groups of 8 (wave-uniform)
        t[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, (uint32_t)((i + j) * kTile + lane) * 4u, 0, kAuxSc1));
    }
#pragma unroll
    for (int j = 0; j < kCombineBurst; ++j)
      if (i + j < ks) acc += t[j];
  }
  if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Greedy token over the tiles of an lm-head GEMV: every tile posts its (max, row) candidate; the
// last tile of each group (tile mod kArgGroups) reduces its group, the last group reduces the
// groups, writes the token and advances the step scalars.  Two levels, because same-line
// atomics serialize: one counter for thousands of tiles would take tens of microseconds.
__device__ __forceinline__ void argmax_tiles(const GemvArgs &a, int tile, int tiles, float bv, int bi, int lane) {
  if (lane == 0) {
    __hip_atomic_store(&a.cand[2 * tile], bv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.cand[2 * tile + 1], __builtin_bit_cast(float, bi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  drain_stores();
  const int g = tile % kArgGroups;
  const int in_g = (tiles - 1 - g) / kArgGroups + 1;  // tiles of this group
  unsigned *gc = a.counters + (kArgGroupLine0 + g) * kLine;
  unsigned prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev + 1 != (unsigned)in_g) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (lane == 0) __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const __amdgpu_buffer_rsrc_t cr = rsrc(a.cand, (uint32_t)(tiles + kArgGroups) * 8);
  float gv = -INFINITY;
  int gi = INT_MAX;
  for (int i = lane; i < in_g; i += 64) {
    const int t = g + kArgGroups * i;
    const float cv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(cr, t * 8, 0, kAuxSc1));
    const int ci = (int)__builtin_amdgcn_raw_buffer_load_b32(cr, t * 8 + 4, 0, kAuxSc1);
    if (ci != INT_MAX && (gi == INT_MAX || cv > gv || (cv == gv && ci < gi))) {
      gv = cv;
      gi = ci;
    }
  }
  wave_argmax(gv, gi);
  float *gcand = a.cand + 2 * tiles;
  if (lane == 0) {
    __hip_atomic_store(&gcand[2 * g], gv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&gcand[2 * g + 1], __builtin_bit_cast(float, gi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  drain_stores();
  const int groups = tiles < kArgGroups ? tiles : kArgGroups;
  unsigned *tc = a.counters + kArgTopLine * kLine;
  prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(tc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev + 1 != (unsigned)groups) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  gv = -INFINITY;
  gi = INT_MAX;
  if (lane < groups) {
    const float cv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(cr, (tiles + lane) * 8, 0, kAuxSc1));
    const int ci = (int)__builtin_amdgcn_raw_buffer_load_b32(cr, (tiles + lane) * 8 + 4, 0, kAuxSc1);
    if (ci != INT_MAX) {
      gv = cv;
      gi = ci;
    }
  }
  wave_argmax(gv, gi);
  if (lane == 0) {
    __hip_atomic_store(tc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int tok = (gi == INT_MAX) ? 0 : gi;
    *a.token = tok;
    if (a.token_log && a.step_count) {
      const int stc = *a.step_count;
      if (stc >= 0 && stc < a.log_len) a.token_log[stc] = tok;
    }
    if (a.step_count) *a.step_count += 1;
    if (a.pos) *a.pos += 1;
  }
}

// The epilogue of one 64-row tile once its k-splits are summed into acc (the wave that finished
// the tile): 1/rms of an RMSNorm prologue, INT8 row scale, bias, residual, then the store (and a
// count for the qkv tile's KV head when COUNT), the tile's sum of squares for the next RMSNorm,
// or SwiGLU, or the greedy argmax candidate.  pre_*: the epilogue's inputs fetched earlier.
template <int FMT, bool NORM, int EPI, bool COUNT>
__device__ __forceinline__ void gemv_tile_epilogue(const GemvArgs &a, float acc, int tile, int n, bool valid, float pre_ssq,
                                                   float pre_bias, float pre_res, float pre_scale, int lane) {
  float v = acc;
  if constexpr (NORM) v *= rsqrtf(wave_sum(pre_ssq) / (float)a.K + a.eps);
  if constexpr (FMT == QDEC_W_Q8_ROW) v *= pre_scale;
  if constexpr (EPI == EPI_STORE || EPI == EPI_ARGMAX) {
    if (valid) {
      if (a.bias) v += pre_bias;
      if (a.residual) v += pre_res;
      st_f<COUNT>(a.y + n, v);
    }
    if constexpr (COUNT) {
      // qkv: count this tile for the KV head its rows belong to (tiles never straddle heads)
      drain_stores();
      const int row0 = tile * kTile, qd = a.Hq * a.hd, kd = a.Hkv * a.hd;
      const int j = row0 < qd ? (row0 / a.hd) / (a.Hq / a.Hkv) : (row0 < qd + kd ? (row0 - qd) / a.hd : (row0 - qd - kd) / a.hd);
      if (lane == 0) (void)__hip_atomic_fetch_add(a.done + j * kLine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      argmax_tiles(a, tile, (a.N + kTile - 1) / kTile, bv, bi, lane);
    }
  } else {
    // lanes 0..31: gate rows 32 tile + lane; lanes 32..63: the matching up rows
    const float u = __shfl(v, lane + 32, 64);
    const int i = tile * 32 + lane;
    if (lane < 32 && i < a.N / 2) a.y[i] = silu(v) * u;
  }
}

// One GEMV work unit (64-row tile t, k-split s) executed by one wave.
//   * the wave streams its runs in batches of kBatch, one batch in flight while the previous
//     one is computed;
//   * split-K partials travel through device-coherent memory and the last wave of a tile adds
//     them in a fixed order, then runs the epilogue.
// SYNC selects the unit's role in the fused attention kernels: kSyncNone (standalone),
// kSyncProducer (the qkv GEMV: device-coherent output stores, then a count for the KV head of
// its rows), kSyncConsumer (the o GEMV: weights requested, then a wait on the producers of its
// k-range, then device-coherent activation loads).
// start() issues the unit's first weight loads and fetches the epilogue's inputs; finish() does
// the rest, so a kernel can issue the loads of several roles before computing any of them.
// With WLDS the unit's runs (at most kStashRuns) are copied by start() straight from HBM into
// the wave's LDS stash (no registers held; the copy lands while the wave does other work), and
// finish() reads them from there.
constexpr int kSyncNone = 0, kSyncProducer = 1, kSyncConsumer = 2;
constexpr int kStashRuns = 8;  // 1 KiB runs of one unit an LDS stash holds

__device__ __forceinline__ void lds_dma_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, const void *lds_slot) {
  // each lane's 16 bytes land at lds_slot + 16 * lane
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void *)(const_cast<void *>(lds_slot)), 16, voff, 0, 0, kAuxStream);
}

template <int FMT, bool NORM, int EPI, int SYNC = kSyncNone, bool WLDS = false, int PF = 2>
struct GemvUnit {
  static constexpr bool XCOH = SYNC == kSyncConsumer;
  static constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  static constexpr int CK = Q4 ? 32 : 16;  // k per 16-byte run
  static_assert(PF >= 2 && PF % 2 == 0, "an even number of batches in flight (the two stage slots alternate)");
  int tile, ksi, c0, nrun, g0, gshift, n;
  bool valid;
  __amdgpu_buffer_rsrc_t wr, sr, xr, gr;
  GemvBatch<FMT, NORM> A;            // the stash path's first batch
  GemvBatch<FMT, NORM> buf[WLDS ? 1 : PF];
  uint16_t s_all[WLDS ? kStashRuns : 1];
  float pre_ssq, pre_bias, pre_res, pre_scale;

  __device__ __forceinline__ void start(const GemvArgs &a, int unit, int lane, const u32x4 *stash = nullptr) {
    const int ks = a.ks, K = a.K;
    tile = unit / ks;
    ksi = unit - tile * ks;
    const int nch = K / CK;
    c0 = ksi * a.cps;
    const int c1 = min(nch, c0 + a.cps);
    nrun = c1 - c0;
    gshift = a.group;  // Q4: log2(group / 32), set by the launcher
    const size_t tile_bytes = (size_t)nch * kTile * 16;
    wr = rsrc(a.W + (size_t)tile * tile_bytes + (size_t)c0 * kTile * 16, (uint32_t)nrun * kTile * 16);
    sr = wr;
    g0 = 0;
    if constexpr (Q4) {
      g0 = c0 >> gshift;
      const int g1 = (c1 - 1) >> gshift;
      sr = rsrc(reinterpret_cast<const uint8_t *>(a.S) + (size_t)tile * ((size_t)(nch >> gshift) * kTile * 2) + (size_t)g0 * kTile * 2,
                (uint32_t)(g1 - g0 + 1) * kTile * 2);
    }
    xr = rsrc(a.x + (size_t)c0 * CK, (uint32_t)nrun * CK * 4);
    gr = NORM ? rsrc(a.gamma + (size_t)c0 * CK, (uint32_t)nrun * CK * 4) : xr;
    // The epilogue's inputs (sums of squares, bias, residual, INT8 row scale) are fetched first,
    // so the wave that finishes a tile does not wait on memory for them; then the batches, each
    // as weights + activations, in the order the loop reissues them (so the loop's waits count
    // exactly the loads of the batch being computed).
    n = tile * kTile + lane;
    valid = n < a.N;
    pre_ssq = 0.f;
    pre_bias = 0.f;
    pre_res = 0.f;
    pre_scale = 1.f;
    if constexpr (NORM) {
      // one plain load per lane (a sum here would make the wave wait for the weights above too)
      if (lane < a.ssq_n) pre_ssq = a.ssq[lane];
      for (int i = lane + 64; i < a.ssq_n; i += 64) pre_ssq += a.ssq[i];
    }
    if (EPI != EPI_SWIGLU && valid) {
      if (a.bias) pre_bias = a.bias[n];
      if (a.residual) pre_res = a.residual[n];  // (y may alias it: only this tile's epilogue writes y[n])
    }
    if constexpr (FMT == QDEC_W_Q8_ROW) pre_scale = reinterpret_cast<const float *>(a.S)[n];  // padded to tiles
    if constexpr (WLDS) {
#pragma unroll
      for (int r = 0; r < kStashRuns; ++r)
        if (r < nrun) lds_dma_b128(wr, (uint32_t)r * (kTile * 16) + lane * 16, stash + r * kTile);
    } else {
      static_assert(SYNC != kSyncConsumer, "a consumer's activations are loaded after its wait");
#pragma unroll
      for (int i = 0; i + 1 < PF; ++i) load_batch<FMT, NORM, XCOH>(buf[i], wr, sr, xr, gr, i * kBatch, c0, g0, gshift, lane);
    }
  }

  // The activations of the stash's two batches from (value, tag) pairs, polled until every tag
  // of the unit's k-range equals this launch's tag (past the range: zeros).  False if the poll
  // gave up (the error word is then set).
  __device__ __forceinline__ bool load_tagged_acts(const GemvArgs &a, GemvBatch<FMT, NORM> &A, GemvBatch<FMT, NORM> &B, unsigned e,
                                                   int lane) {
    const unsigned tag = e * a.xt_tag_mul + a.xt_tag_add;
    const __amdgpu_buffer_rsrc_t tr = rsrc(a.xt + (size_t)c0 * CK * 2, (uint32_t)nrun * CK * 8);
    const bool in_a = lane * 4 < kBatch * CK && lane * 4 < nrun * CK;
    const bool in_b = lane * 4 < kBatch * CK && kBatch * CK + lane * 4 < nrun * CK;
    const uint32_t oa = in_a ? (uint32_t)(lane * 4) * 8u : 0x80000000u;
    const uint32_t ob = in_b ? (uint32_t)(kBatch * CK + lane * 4) * 8u : 0x80000000u;
    u32x4 a0, a1, b0, b1;
    unsigned spins = 0;
    for (;;) {
      a0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, oa, 0, kAuxSc1));
      a1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, oa + 16, 0, kAuxSc1));
      b0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, ob, 0, kAuxSc1));
      b1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, ob + 16, 0, kAuxSc1));
      const bool ok = (!in_a || (a0.y == tag && a0.w == tag && a1.y == tag && a1.w == tag)) &&
                      (!in_b || (b0.y == tag && b0.w == tag && b1.y == tag && b1.w == tag));
      if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
      if (!poll_step(spins, a.err)) return false;
    }
    // (whole-vector bit casts: a bit cast of one element of a vector compiles to element 0)
    const f32x4 fa0 = __builtin_bit_cast(f32x4, a0), fa1 = __builtin_bit_cast(f32x4, a1);
    const f32x4 fb0 = __builtin_bit_cast(f32x4, b0), fb1 = __builtin_bit_cast(f32x4, b1);
    A.x = f32x4{fa0.x, fa0.z, fa1.x, fa1.z};
    B.x = f32x4{fb0.x, fb0.z, fb1.x, fb1.z};
    if constexpr (NORM) {
      A.g = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(gr, in_a ? (uint32_t)(lane * 4) * 4u : 0x80000000u, 0, 0));
      B.g = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(gr, in_b ? (uint32_t)(kBatch * CK + lane * 4) * 4u : 0x80000000u, 0, 0));
    }
    return true;
  }

  __device__ __forceinline__ void finish(const GemvArgs &a, Stage<CK> (&sm)[2], int lane, const u32x4 *stash = nullptr,
                                        unsigned long long *rec = nullptr) {
    unsigned e = 0;
    if constexpr (SYNC != kSyncNone) e = __builtin_amdgcn_readfirstlane(*a.epoch);
    if constexpr (SYNC == kSyncConsumer) {
      // the producers of activations k = c0 CK .. (c0 + nrun) CK - 1 (the weights are already
      // on their way)
      // (tagged activations carry their own readiness: polled below, when they are loaded)
      if (!a.xt) {
        if (!poll_flags(a.wait_flags, (c0 * CK) / a.wait_div, ((c0 + nrun) * CK - 1) / a.wait_div, e, a.err, lane)) return;
        mark(rec, 0);
      }
    }
    float acc = 0.f;
    const int nb = (nrun + kBatch - 1) / kBatch;
    if constexpr (WLDS) {
      static_assert(kStashRuns == 2 * kBatch, "two batches per stash");
      GemvBatch<FMT, NORM> B;
      // The stash's scales are requested here, not in start(): held from there, the compiler
      // converts them at once, so start() would wait for the whole stash copy.
      if constexpr (Q4) {
#pragma unroll
        for (int r = 0; r < kStashRuns; ++r)
          s_all[r] = __builtin_amdgcn_raw_buffer_load_b16(sr, (uint32_t)(((c0 + r) >> gshift) - g0) * (kTile * 2) + lane * 2, 0, 0);
      }
      if (XCOH && a.xt) {
        if (!load_tagged_acts(a, A, B, e, lane)) return;
        mark(rec, 0);
      } else {
        load_acts<FMT, NORM, XCOH>(A, xr, gr, 0, lane);
        load_acts<FMT, NORM, XCOH>(B, xr, gr, kBatch, lane);
      }
      __builtin_amdgcn_s_waitcnt(0);  // the stash copies (not tracked by the compiler) have landed
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        A.w[i] = (i < nrun) ? stash[i * kTile + lane] : u32x4{0u, 0u, 0u, 0u};
        A.s[i] = (i < nrun) ? s_all[i] : (uint16_t)0;
      }
      compute_batch<FMT, NORM>(acc, A, sm[0], lane);
      if (nb > 1) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          B.w[i] = (kBatch + i < nrun) ? stash[(kBatch + i) * kTile + lane] : u32x4{0u, 0u, 0u, 0u};
          B.s[i] = (kBatch + i < nrun) ? s_all[kBatch + i] : (uint16_t)0;
        }
        compute_batch<FMT, NORM>(acc, B, sm[1], lane);
      }
    } else {
      // Software pipeline over PF batch slots: batches 0 .. PF - 2 were requested by start();
      // each step requests the batch PF - 1 ahead into the slot computed last, then stages and
      // computes the current one, so PF - 1 batches are in flight meanwhile.  The loop is entered
      // (from start() and from its own end) with the same loads pending, in the same order, so
      // the wait before each compute counts exactly the loads issued after that batch's.  Past
      // the last run the loads read zeros.
      for (int b = 0; b < nb; b += PF) {
#pragma unroll
        for (int k = 0; k < PF; ++k) {
          load_batch<FMT, NORM, XCOH>(buf[(k + PF - 1) % PF], wr, sr, xr, gr, (b + k + PF - 1) * kBatch, c0, g0, gshift,
                                      lane);
          compute_batch<FMT, NORM>(acc, buf[k], sm[k & 1], lane);
          if (b + k + 1 >= nb) break;
        }
      }
    }
    if constexpr (Q4) acc *= 16777216.0f;  // 2^24, exact
    mark(rec, 1);

    if (a.ks > 1 && !splitk_combine(acc, a.part, a.counters, tile, a.ks, ksi, lane)) return;
    mark(rec, 2);
    gemv_tile_epilogue<FMT, NORM, EPI, SYNC == kSyncProducer>(a, acc, tile, n, valid, pre_ssq, pre_bias, pre_res, pre_scale,
                                                             lane);
  }
};

}  // namespace dev
}  // namespace qdec
