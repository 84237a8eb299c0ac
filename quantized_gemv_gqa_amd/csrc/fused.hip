// Persistent decode-step kernel: the whole batch-1 decode step of a Qwen-style GQA decoder in one
// launch of co-resident workgroups on gfx950.
//
// Why: at batch 1 every weight byte is read once per token, so the step is an HBM stream of a
// few GB cut into ~140 dependent pieces (per layer: fused qkv GEMV -> paged attention -> o GEMV
// -> gate/up GEMV + SwiGLU -> down GEMV; then the lm head and greedy argmax).  Launched as one
// kernel per piece, each launch pays a fixed dispatch/drain cost comparable to a small GEMV's
// whole HBM time (FlashQwen README, "Optimization study", stage 6, and the H100 runtime post,
// section 6, make the same point about per-kernel launch cost; there a captured graph was the
// answer).  Here the pieces run inside one kernel and hand data over through device-coherent
// memory:
//   * GEMVs are split stream-K style: the packed weights of a GEMV are one contiguous run of
//     1 KiB chunks, and every wave of the grid takes an equal contiguous share, so no wave gets
//     twice the work of another; a tile split over several waves is summed by its last
//     contributor from per-wave partials in wave order (deterministic);
//   * a wave requests the first weights of its share before it waits for the activation, so
//     the wait overlaps the HBM stream, and it double-buffers weights while computing;
//   * dependencies are as narrow as the data flow allows: attention for KV head j waits only
//     for the qkv tiles of head j, a down-projection wave only for the gate/up tiles that
//     produce its slice of the MLP activation; only the RMSNorms (which need a whole vector)
//     wait for a whole GEMV, through a progress value replicated over 64 cache lines;
//   * the residual stream alternates between two buffers so that no wave overwrites a vector
//     another wave may still be reading, and counters that are polled only ever grow (a step
//     with epoch e waits for (e + 1) times the per-step arrivals), so nothing needs clearing;
//   * counters that many finishers hit are split (the argmax over the vocabulary counts per
//     group of tiles, then per group), because same-address atomics serialize.
// Co-residency of all workgroups is guaranteed by a cooperative launch.
#include <hip/hip_runtime.h>

#include <cmath>

#include "qdec_device.h"
#include "qdec_fused.h"

namespace qdec {
namespace {

using namespace dev;

constexpr int kStep = 8;    // 1 KiB runs per pipeline step: 8 KiB of weights per wave in flight
constexpr int kRound = 32;  // runs whose activations are staged in LDS at a time (more spills registers)

template <int CK>
struct XStage {
  float x[kRound * CK];
  float sum[kRound];
};

template <int D, int G>
struct AttnSmem {
  float m[4][G], l[4][G], o[4][G][D];
  float wm[kMaxMergeSplits][G];  // split maxima, then their weights
  float wl[kMaxMergeSplits][G];  // split sums
  float M[G], L[G];
  float qkv[(G + 2) * D];        // this KV head's q heads, then its new k and v (pre-RoPE)
  unsigned last;
};

// Separate regions, not a union: the waves of a workgroup run GEMV shares independently and
// may be in different phases at the same time.
template <int CK, int D, int G>
struct FusedSmem {
  XStage<CK> xs[4];
  AttnSmem<D, G> at;
  double cs[64][2];  // this step's RoPE (cos, sin) per rotation pair, computed by the workgroup
};

__device__ __forceinline__ bool reached(unsigned v, unsigned target) { return (int)(v - target) >= 0; }

__device__ __forceinline__ bool failed(unsigned *err) {
  return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}
__device__ __forceinline__ void fail(unsigned *err) {
  __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded waits (device-coherent polls).  On timeout they set *err; once *err is set every wait
// gives up within 1024 polls, so a failed step ends within one timeout.
__device__ bool wait_count(const unsigned *p, unsigned target, unsigned *err) {
  unsigned spins = 0;
  while (!reached(__hip_atomic_load(const_cast<unsigned *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), target)) {
    __builtin_amdgcn_s_sleep(2);
    if ((++spins & 1023u) == 0 && failed(err)) return false;
    if (spins > kSpinLimit) {
      fail(err);
      return false;
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return true;
}

__device__ bool wait_progress(const unsigned long long *p, unsigned long long target, unsigned *err) {
  unsigned spins = 0;
  while (__hip_atomic_load(const_cast<unsigned long long *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(2);
    if ((++spins & 1023u) == 0 && failed(err)) return false;
    if (spins > kSpinLimit) {
      fail(err);
      return false;
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return true;
}

// Wait until flags[f] has reached `target` for every f in [f0, f1] (lanes poll 64 at a time).
__device__ bool wait_flags(const unsigned *flags, int f0, int f1, unsigned target, unsigned *err, int lane) {
  for (int base = f0; base <= f1; base += 64) {
    const int f = base + lane;
    unsigned spins = 0;
    for (;;) {
      const bool ok = f > f1 ||
                      reached(__hip_atomic_load(const_cast<unsigned *>(flags + f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), target);
      if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
      __builtin_amdgcn_s_sleep(2);
      if ((++spins & 1023u) == 0 && failed(err)) return false;
      if (spins > kSpinLimit) {
        fail(err);
        return false;
      }
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return true;
}

// Publish "phase `value` reached" to every progress replica (one line per lane).  A maximum, not
// a store, so a late store of an older value can never move a replica backwards.
__device__ __forceinline__ void publish(unsigned long long *progress, unsigned long long value, int lane) {
  if (lane < kProgressReplicas)
    (void)__hip_atomic_fetch_max(progress + lane * 16, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void mark_time(unsigned long long *ts, int idx, int lane) {
  if (ts && lane == 0) (void)__hip_atomic_fetch_max(ts + idx, (unsigned long long)wall_clock64(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float bf16_to_float(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// Per-wave diagnostic marks: slot [phase][wave][mark] = low 32 bits of the 100 MHz clock.
__device__ __forceinline__ void wave_mark(unsigned *ts, int phase, int waves, int w, int mark, int lane) {
  if (ts && lane == 0) ts[((size_t)phase * waves + w) * 4 + mark] = (unsigned)wall_clock64();
}

// A pointer every lane holds the same value of (read from the layer table in memory), moved to
// scalar registers so buffer descriptors built from it stay scalar.
template <typename T>
__device__ __forceinline__ T *uniform(T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T *>(((uint64_t)hi << 32) | lo);
}

// ------------------------------------------------------------------------------ stream-K GEMV
__device__ __forceinline__ int sk_wave(const SkPhase &p, int r) {
  const int big = p.rem * (p.q + 1);
  return r < big ? r / (p.q + 1) : p.rem + (r - big) / p.q;
}

template <int FMT>
struct StepRegs {
  u32x4 w[kStep];
  uint16_t s[kStep];
};

template <int FMT>
__device__ __forceinline__ void load_step(StepRegs<FMT> &R, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                          int r, int n, int gshift, int lane) {
#pragma unroll
  for (int i = 0; i < kStep; ++i) {
    if (i < n) {
      R.w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, lane * 16, (r + i) * (kTile * 16), kAuxStream));
      if constexpr (FMT == QDEC_W_Q4_G_ZP8)
        R.s[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, lane * 2, ((r + i) >> gshift) * (kTile * 2), 0);
    }
  }
}

template <int FMT>
__device__ __forceinline__ void compute_step(float &acc, const StepRegs<FMT> &R, int n,
                                             const XStage<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16> &sm, int ri) {
  constexpr bool Q4 = FMT == QDEC_W_Q4_G_ZP8;
  constexpr int CK = Q4 ? 32 : 16;
  constexpr int RV = CK / 4;
#pragma unroll
  for (int i = 0; i < kStep; ++i) {
    if (i < n) {
      f32x4 xs[RV];
#pragma unroll
      for (int v = 0; v < RV; ++v) xs[v] = *reinterpret_cast<const f32x4 *>(&sm.x[(ri + i) * CK + 4 * v]);
      const float xsum = sm.sum[ri + i];
      if constexpr (Q4) {
        const float d = dot_q4_run(R.w[i], xs);
        acc = fmaf(half_bits_to_float(R.s[i]), d - 8.0f * xsum, acc);
      } else {
        acc += dot_q8_run(R.w[i], xs) - 128.0f * xsum;
      }
    }
  }
}

// Stage the activations of runs [rr, rr + nr) of a GEMV share (chunk index wraps at nch) into
// the wave's LDS region: odd k of INT4 pre-divided by 16, plus the per-run sums of the true
// values.  The source is an fp32 vector written earlier in this kernel (device-coherent loads;
// producers already applied the RMSNorm gain of the consuming GEMV) or, with EMB, a bf16
// embedding row times `gamma`.  All loads are in flight at once.
template <int FMT, bool EMB>
__device__ __forceinline__ void stage_round(XStage<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16> &sm, const float *x,
                                            const uint16_t *xe, const float *gamma, int K, int nch,
                                            int rr, int nr, int lane) {
  constexpr int CK = (FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16;
  constexpr int PER = kRound * CK / 256;  // 16-byte pieces per lane
  constexpr int LPR = CK / 4;             // lanes per run
  static_assert(PER * 256 == kRound * CK, "a round is a whole number of wave-wide pieces");
  const int c0 = rr % nch;
  const __amdgpu_buffer_rsrc_t xr = EMB ? rsrc(xe, (uint32_t)K * 2) : rsrc(x, (uint32_t)K * 4);
  const __amdgpu_buffer_rsrc_t gr = rsrc(EMB ? gamma : x, (uint32_t)K * 4);
  f32x4 v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int val = j * 256 + 4 * lane;
    const int i = val / CK;
    v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < nr) {
      const int k = ((c0 + i) % nch) * CK + (val % CK);
      if constexpr (EMB) {
        const uint64_t b = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(xr, k * 2, 0, 0));
        v[j] = f32x4{bf16_to_float((uint16_t)b), bf16_to_float((uint16_t)(b >> 16)),
                     bf16_to_float((uint16_t)(b >> 32)), bf16_to_float((uint16_t)(b >> 48))};
        v[j] *= __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(gr, k * 4, 0, 0));
      } else {
        v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, k * 4, 0, kAuxSc1));
      }
    }
  }
  __builtin_amdgcn_wave_barrier();  // earlier LDS reads of this wave are done before the overwrite
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int val = j * 256 + 4 * lane;
    float part = (v[j].x + v[j].y) + (v[j].z + v[j].w);
    if constexpr (LPR == 8) {
      part = sum8(part);
    } else {
      part += dpp<0xB1>(part);
      part += dpp<0x4E>(part);
    }
    f32x4 t = v[j];
    if constexpr (CK == 32) {  // odd k carry 1/16 (exact power-of-two scaling)
      t.y *= 0.0625f;
      t.w *= 0.0625f;
    }
    *reinterpret_cast<f32x4 *>(&sm.x[val]) = t;
    if (lane % LPR == 0) sm.sum[val / CK] = part;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int NL>
__device__ __forceinline__ float sum_slots_n(__amdgpu_buffer_rsrc_t pr, int lane) {
  float t[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i)
    t[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, lane * 4, i * 256, kAuxSc1));
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NL; ++i) s += t[i];
  return s;
}

// Sum the ns partials of a tile in slot order; slots past ns lie outside the resource and read 0.
__device__ __forceinline__ float sum_slots(const float *pt, int ns, int lane) {
  const __amdgpu_buffer_rsrc_t pr = rsrc(pt, (uint32_t)ns * 256);
  if (ns <= 4) return sum_slots_n<4>(pr, lane);
  if (ns <= 8) return sum_slots_n<8>(pr, lane);
  if (ns <= 16) return sum_slots_n<16>(pr, lane);
  if (ns <= 32) return sum_slots_n<32>(pr, lane);
  return sum_slots_n<64>(pr, lane);
}

enum FusedEpi : int { FE_QKV, FE_O, FE_GU, FE_DOWN, FE_LM };

struct StepCtx {
  int l;                   // layer
  unsigned e;              // epoch of this step
  unsigned long long pps;  // progress values per step
  int tok;                 // input token of this step
  int G;
};

__device__ __forceinline__ float q8_scale(const void *S, int n) { return reinterpret_cast<const float *>(S)[n]; }

// Greedy token over the lm-head tiles: every tile finisher posts (max, row); the last finisher
// of each group of tiles (t mod 64) reduces its group, the last group reduces the groups and
// completes the step (token, log, position, epoch).
__device__ __forceinline__ void lm_argmax(const FusedArgs &a, const StepCtx &c, int t, int tiles, float bv, int bi, int lane) {
  if (lane == 0) {
    __hip_atomic_store(&a.cand[2 * t], bv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.cand[2 * t + 1], __builtin_bit_cast(float, bi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  drain_stores();
  const int sub = t & 63;
  const int nsub_t = (tiles - 1 - sub) / 64 + 1;  // tiles in this group
  unsigned prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(a.lm_sub + sub * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev + 1 != (unsigned)nsub_t) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (lane == 0) __hip_atomic_store(a.lm_sub + sub * 32, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const __amdgpu_buffer_rsrc_t cr = rsrc(a.cand, (uint32_t)tiles * 8);
  float gv = -INFINITY;
  int gi = INT_MAX;
  for (int i = lane; i < nsub_t; i += 64) {
    const int tt = sub + 64 * i;
    const float cv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(cr, tt * 8, 0, kAuxSc1));
    const int ci = (int)__builtin_amdgcn_raw_buffer_load_b32(cr, tt * 8 + 4, 0, kAuxSc1);
    if (ci != INT_MAX && (gi == INT_MAX || cv > gv || (cv == gv && ci < gi))) {
      gv = cv;
      gi = ci;
    }
  }
  wave_argmax(gv, gi);
  if (lane == 0) {
    __hip_atomic_store(&a.sub_cand[2 * sub], gv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.sub_cand[2 * sub + 1], __builtin_bit_cast(float, gi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  drain_stores();
  const int ngroups = tiles < 64 ? tiles : 64;
  prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(a.lm_top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev + 1 != (unsigned)ngroups) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  gv = -INFINITY;
  gi = INT_MAX;
  if (lane < ngroups) {
    const __amdgpu_buffer_rsrc_t sr = rsrc(a.sub_cand, 64 * 8);
    const float cv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, lane * 8, 0, kAuxSc1));
    const int ci = (int)__builtin_amdgcn_raw_buffer_load_b32(sr, lane * 8 + 4, 0, kAuxSc1);
    if (ci != INT_MAX) {
      gv = cv;
      gi = ci;
    }
  }
  wave_argmax(gv, gi);
  if (lane == 0) {
    __hip_atomic_store(a.lm_top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int tok = (gi == INT_MAX) ? 0 : gi;
    st_f<true>(reinterpret_cast<float *>(a.token), __builtin_bit_cast(float, tok));
    if (a.token_log && a.step_count) {
      const int stc = *a.step_count;
      if (stc >= 0 && stc < a.log_len) a.token_log[stc] = tok;
    }
    if (a.step_count) *a.step_count += 1;
    *a.pos += 1;
    __hip_atomic_store(a.epoch, c.e + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.phase_ts) a.phase_ts[1 + 5 * a.L] = wall_clock64();
  }
}

// Finish tile t of a GEMV share: hand the partial over if the tile is split, and if this wave is
// the tile's last contributor, sum the partials and run the phase's epilogue.
template <int FMT, int E>
__device__ __forceinline__ void finish_tile(const FusedArgs &a, const SkPhase &p, const StepCtx &c, const FusedLayer &Lw,
                            const void *S, int w, int t, float acc, float rn, int lane) {
  const int nch = p.nch;
  const int wf = sk_wave(p, t * nch);
  const int ns = sk_wave(p, t * nch + nch - 1) - wf + 1;
  float v = acc;
  if (ns > 1) {
    float *pt = p.part + (size_t)t * p.slots * kTile;
    __hip_atomic_store(pt + (w - wf) * kTile + lane, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    drain_stores();
    unsigned prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(p.tile_cnt + t * kLine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (unsigned)(ns - 1)) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_store(p.tile_cnt + t * kLine, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    v = sum_slots(pt, ns, lane);
  }
  v *= rn;
  const int n = t * kTile + lane;
  if constexpr (FMT == QDEC_W_Q8_ROW) v *= q8_scale(S, n);  // scales are padded to whole tiles
  const int H = a.H;
  if constexpr (E == FE_QKV) {
    if (Lw.b_qkv) v += Lw.b_qkv[n];
    st_f<true>(a.qkv + n, v);
    // KV head whose attention needs this tile (tiles never straddle heads: D is a multiple of 64)
    const int qd = a.Hq * 128, kd = a.Hkv * 128;
    const int row0 = t * kTile;
    const int j = row0 < qd ? (row0 >> 7) / c.G : (row0 < qd + kd ? (row0 - qd) >> 7 : (row0 - qd - kd) >> 7);
    drain_stores();
    if (lane == 0) (void)__hip_atomic_fetch_add(a.qkv_done + (c.l * a.Hkv + j) * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    mark_time(a.phase_ts, 1 + 5 * c.l + 0, lane);
  } else if constexpr (E == FE_O || E == FE_DOWN) {
    float res;
    if (E == FE_O && c.l == 0) {
      res = bf16_to_float(a.embed[(size_t)c.tok * H + n]);
      if (a.trace) a.trace[n] = res;
    } else {
      res = ld_f<true>((E == FE_O ? a.hA : a.hB) + n);
    }
    v += res;
    st_f<true>((E == FE_O ? a.hB : a.hA) + n, v);
    // the consumer's RMSNorm gain, applied once here: gate/up after o, the next layer's qkv (or
    // the lm head) after down
    const float *gn = E == FE_O ? Lw.g_ffn : (c.l + 1 < a.L ? a.layers[c.l + 1].g_attn : a.g_out);
    st_f<true>((E == FE_O ? a.xb : a.xa) + n, v * gn[n]);
    if (E == FE_DOWN && a.trace) a.trace[(size_t)(c.l + 1) * H + n] = v;
    const float sq = wave_sum(v * v);
    if (lane == 0) st_f<true>((E == FE_O ? a.ssqB : a.ssqA) + t, sq);
    drain_stores();
    unsigned *ctr = (E == FE_O ? a.o_done : a.down_done) + c.l * 32;
    unsigned prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev + 1 == (c.e + 1u) * (unsigned)p.tiles)
      publish(reinterpret_cast<unsigned long long *>(a.progress), c.e * c.pps + 3ull * c.l + (E == FE_O ? 2 : 3), lane);
    mark_time(a.phase_ts, 1 + 5 * c.l + (E == FE_O ? 2 : 4), lane);
  } else if constexpr (E == FE_GU) {
    // lanes 0..31: gate rows 32 t + lane; lanes 32..63: the matching up rows
    const float u = __shfl(v, lane + 32, 64);
    if (lane < 32) st_f<true>(a.mlp + t * 32 + lane, silu(v) * u);
    drain_stores();
    if (lane == 0)
      __hip_atomic_store(a.gu_flag + (size_t)c.l * p.tiles + t, c.e + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    mark_time(a.phase_ts, 1 + 5 * c.l + 3, lane);
  } else {  // FE_LM
    const bool valid = n < a.V;
    if (valid) a.logits[n] = v;
    float bv = (valid && v == v) ? v : -INFINITY;  // NaN never wins
    int bi = (valid && v == v) ? n : INT_MAX;
    wave_argmax(bv, bi);
    lm_argmax(a, c, t, p.tiles, bv, bi, lane);
  }
}

// One wave's share of a GEMV phase.  The phase (E) fixes the input normalisation, the epilogue
// and the dependency: qkv, o, gate/up and the lm head wait for a progress value (layer 0's qkv,
// which reads the embedding row itself, waits for nothing); down waits per gate/up tile.
template <int FMT, int E, bool EMB>
__device__ __forceinline__ void sk_gemv(const FusedArgs &a, const SkPhase &p, const StepCtx &c, const FusedLayer &Lw,
                                        const uint8_t *W, const void *S, const float *x, const float *ssq, int K,
                                        int w, XStage<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16> &sm, int lane,
                                        const unsigned long long *prog, unsigned long long dep, int slot) {
  constexpr int CK = (FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16;
  constexpr bool NORM = E == FE_QKV || E == FE_GU || E == FE_LM;
  const int NWall = gridDim.x * 4;
  wave_mark(a.wave_ts, slot, NWall, w, 0, lane);
  if (w >= p.nw) return;
  const int r0 = w * p.q + min(w, p.rem);
  const int r1 = r0 + p.q + (w < p.rem ? 1 : 0);
  if (r0 >= r1) return;
  const int nch = p.nch;
  const int R = p.tiles * nch;
  W = uniform(W);
  S = uniform(S);
  const __amdgpu_buffer_rsrc_t wr = rsrc(W, (uint32_t)R * (kTile * 16));
  const __amdgpu_buffer_rsrc_t sr =
      (FMT == QDEC_W_Q4_G_ZP8) ? rsrc(S, (uint32_t)(R >> a.gshift) * (kTile * 2)) : wr;
  const int gshift = a.gshift;
  const uint16_t *xe = a.embed + (size_t)c.tok * a.H;

  int r = r0;
  int rr = r0, rend = min(r1, r0 + kRound);
  int tend = (r0 / nch + 1) * nch;  // end of the current tile's runs
  int n = min(kStep, min(rend, tend) - r);
  StepRegs<FMT> A, B;
  load_step<FMT>(A, wr, sr, r, n, gshift, lane);

  bool ok = true;
  if constexpr (E == FE_DOWN) {
    // activation k = c CK .. c CK + CK - 1 comes from gate/up tile k / 32
    const int c0 = r0 % nch, c1 = (r1 - 1) % nch;
    const unsigned tgt = c.e + 1u;
    const unsigned *flags = a.gu_flag + (size_t)c.l * a.p_gu.tiles;
    const int last = (nch * CK - 1) / 32;
    if (r1 - r0 >= nch) {
      ok = wait_flags(flags, 0, last, tgt, a.err, lane);
    } else if (c1 < c0) {  // the share wraps around the chunk range
      ok = wait_flags(flags, (c0 * CK) / 32, last, tgt, a.err, lane) &&
           wait_flags(flags, 0, (c1 * CK + CK - 1) / 32, tgt, a.err, lane);
    } else {
      ok = wait_flags(flags, (c0 * CK) / 32, (c1 * CK + CK - 1) / 32, tgt, a.err, lane);
    }
  } else if constexpr (!EMB) {
    ok = wait_progress(prog, dep, a.err);
  }
  if (!ok) return;
  wave_mark(a.wave_ts, slot, NWall, w, 1, lane);

  float rn = 1.f;
  if constexpr (NORM) {
    float ss = 0.f;
    if constexpr (EMB) {
      const __amdgpu_buffer_rsrc_t er = rsrc(xe, (uint32_t)K * 2);
      for (int i = lane; i < K / 8; i += 64) {
        const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(er, i * 16, 0, 0));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __builtin_bit_cast(float, b[q] << 16), hi = __builtin_bit_cast(float, b[q] & 0xFFFF0000u);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
      }
    } else {
      const int nt = (K + kTile - 1) / kTile;  // per-64-row sums of squares of x (nt <= 64)
      if (lane < nt) ss = ld_f<true>(ssq + lane);
    }
    rn = rsqrtf(wave_sum(ss) / (float)K + a.eps);
  }
  const float *const g_emb = EMB ? uniform(Lw.g_attn) : nullptr;
  stage_round<FMT, EMB>(sm, x, xe, g_emb, K, nch, rr, rend - rr, lane);
  wave_mark(a.wave_ts, slot, NWall, w, 2, lane);

  float acc = 0.f;
  // two copies of the loop body with the buffers' roles swapped (no register moves)
  auto body = [&](StepRegs<FMT> &cur, StepRegs<FMT> &nxt, int &ncur) -> bool {
    const int rb = r + ncur;
    int nb = 0, rbend = rend, tbend = tend;
    if (rb < r1) {
      if (rb == rend) rbend = min(r1, rb + kRound);
      if (rb == tend) tbend = tend + nch;
      nb = min(kStep, min(rbend, tbend) - rb);
      load_step<FMT>(nxt, wr, sr, rb, nb, gshift, lane);
    }
    compute_step<FMT>(acc, cur, ncur, sm, r - rr);
    if (rb == tend || rb == r1) {
      finish_tile<FMT, E>(a, p, c, Lw, S, w, (tend / nch) - 1, acc, rn, lane);
      acc = 0.f;
    }
    if (rb >= r1) return false;
    if (rb == rend) {
      rr = rb;
      rend = rbend;
      stage_round<FMT, EMB>(sm, x, xe, g_emb, K, nch, rr, rend - rr, lane);
    }
    tend = tbend;
    r = rb;
    ncur = nb;
    return true;
  };
  for (;;) {
    if (!body(A, B, n)) break;
    if (!body(B, A, n)) break;
  }
  wave_mark(a.wave_ts, slot, NWall, w, 3, lane);
}

// ------------------------------------------------------------------------------ attention
// bf16 KV row piece of one lane: 8 values (D = 128) at byte offset `off` of the pool, packed
__device__ __forceinline__ u32x4 load_row8_raw(__amdgpu_buffer_rsrc_t pool, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(pool, off, 0, 0));
}
__device__ __forceinline__ float bf16_at(u32x4 v, int e) {
  const uint32_t w = v[e >> 1];
  return __builtin_bit_cast(float, (e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}
// pack 8 floats to bf16 (round to nearest even), the layout of a row piece
__device__ __forceinline__ u32x4 pack_bf16x8(const float (&v)[8]) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = (uint32_t)float_to_bf16_rne(v[2 * i]) | ((uint32_t)float_to_bf16_rne(v[2 * i + 1]) << 16);
  return r;
}

// Normalise (optional) and rotate one head vector held 8 dims per lane (lanes `part` of a 16-lane
// slot group hold dims part*8 .. part*8+7).  `own` are the lane's dims, `mate` the dims D/2 away.
__device__ __forceinline__ void norm_rope8(float (&own)[8], float (&mate)[8], int part, const float *gamma,
                                           float eps, const double (*cs)[2]) {
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
  const int i0 = lo ? d0 : d0 - HALF;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double cc = cs[i0 + e][0], s = cs[i0 + e][1];
    const double x = own[e], y = mate[e];
    // low half: x' = x c - y s (y = x[i + D/2]); high half: x' = x c + y s (y = x[i - D/2])
    own[e] = (float)(lo ? (x * cc - y * s) : (x * cc + y * s));
  }
}

// One wave, one 16-token page: token slot sub*4 + slot sits in this lane's kp[sub] / vp[sub];
// tokens at or past T are masked.
template <int G>
__device__ __forceinline__ void attend_page8(u32x4 (&kp)[4], u32x4 (&vp)[4], int p, int T, int slot,
                                             const float (&q)[G][8], float (&m)[G], float (&l)[G],
                                             float (&o)[G][8]) {
  float sc[4][G];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    const bool valid = p * 16 + sub * 4 + slot < T;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(q[h][e], bf16_at(kp[sub], e), d);
      d = sum16(d);
      sc[sub][h] = valid ? d : -INFINITY;
    }
    if (!valid) vp[sub] = u32x4{0u, 0u, 0u, 0u};  // masked slots add 0 * 0
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mx = fmaxf(fmaxf(m[h], fmaxf(sc[0][h], sc[1][h])), fmaxf(sc[2][h], sc[3][h]));
    const float alpha = exp2f(m[h] - mx);
    m[h] = mx;
    float ls = 0.f;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      sc[sub][h] = exp2f(sc[sub][h] - mx);
      ls += sc[sub][h];
    }
    l[h] = fmaf(l[h], alpha, ls);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
  }
#pragma unroll
  for (int sub = 0; sub < 4; ++sub)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float vv = bf16_at(vp[sub], e);
#pragma unroll
      for (int h = 0; h < G; ++h) o[h][e] = fmaf(sc[sub][h], vv, o[h][e]);
    }
}

constexpr int kMergeChunk = 32;  // splits whose partial outputs one merge pass loads at once

// Attention work unit (KV head j, split s) executed by a whole workgroup (4 waves).
template <int G>
__device__ __forceinline__ void attn_unit(const FusedArgs &a, const StepCtx &c, const FusedLayer &Lw, int j, int s, int pos,
                          AttnSmem<128, G> &sm, const double (*cs)[2]) {
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
  void *const k_pool = uniform(Lw.k_pool), *const v_pool = uniform(Lw.v_pool);
  const uint32_t pool_bytes = (uint32_t)((size_t)a.n_pages * a.Hkv * 16 * D * 2);
  const __amdgpu_buffer_rsrc_t kpool = rsrc(k_pool, pool_bytes);
  const __amdgpu_buffer_rsrc_t vpool = rsrc(v_pool, pool_bytes);
  const __amdgpu_buffer_rsrc_t qkvr = rsrc(a.qkv, (uint32_t)((a.Hq + 2 * a.Hkv) * D * 4));
  const size_t head_stride = (size_t)16 * D;

  // the wave's first two pages are requested before the wait (the newest token's row of the last
  // page is replaced by the freshly computed k and v below, so no page depends on this step)
  u32x4 kp[2][4], vp[2][4];
  bool have[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = p0 + wave + 4 * i;
    have[i] = false;
    if (p < p1) {
      const int phys = a.page_table[p];
      if (phys >= 0 && phys < a.n_pages) {  // documented precondition; never read outside
        have[i] = true;
        const size_t base = ((size_t)phys * a.Hkv + j) * head_stride;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
          const uint32_t e = (uint32_t)((base + (size_t)(sub * 4 + slot) * D + part * DPL) * 2);
          kp[i][sub] = load_row8_raw(kpool, e);
          vp[i][sub] = load_row8_raw(vpool, e);
        }
      }
    }
  }

  const int gwv = blockIdx.x * 4 + wave, NWall = gridDim.x * 4;
  wave_mark(a.wave_ts, 5 * c.l + 1, NWall, gwv, 0, lane);
  // the qkv tiles of KV head j: G q heads plus one k and one v head, D / 64 tiles each
  const unsigned tiles_j = (unsigned)((G + 2) * (D / kTile));
  const bool ok = wait_count(a.qkv_done + (c.l * a.Hkv + j) * 32, (c.e + 1u) * tiles_j, a.err);
  wave_mark(a.wave_ts, 5 * c.l + 1, NWall, gwv, 1, lane);

  // stage this KV head's q heads and its new k, v in LDS (device-coherent loads, one round trip)
  for (int i = threadIdx.x; i < (G + 2) * D / 4; i += 256) {
    const int h = (i * 4) / D, d = i * 4 - h * D;
    const int row = h < G ? (j * G + h) : (h == G ? a.Hq + j : a.Hq + a.Hkv + j);
    *reinterpret_cast<f32x4 *>(&sm.qkv[h * D + d]) =
        __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(qkvr, (uint32_t)((row * D + d) * 4), 0, kAuxSc1));
  }
  __syncthreads();

  // q of the G query heads: normalised (Qwen3), rotated, scaled into the log2 domain
  float q[G][DPL];
  const int dmate = part * DPL < 64 ? part * DPL + 64 : part * DPL - 64;
  const float *gq = uniform(Lw.g_q), *gk = uniform(Lw.g_k);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float own[8], mate[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      own[e] = sm.qkv[h * D + part * DPL + e];
      mate[e] = sm.qkv[h * D + dmate + e];
    }
    norm_rope8(own, mate, part, gq, a.eps, cs);
#pragma unroll
    for (int e = 0; e < DPL; ++e) q[h][e] = own[e] * a.scale_log2;
  }
  // the new token's k (normalised, rotated) and v, rounded to bf16 like every cached key
  u32x4 knew, vnew;
  {
    float own[8], mate[8], vv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      own[e] = sm.qkv[G * D + part * DPL + e];
      mate[e] = sm.qkv[G * D + dmate + e];
      vv[e] = sm.qkv[(G + 1) * D + part * DPL + e];
    }
    norm_rope8(own, mate, part, gk, a.eps, cs);
    knew = pack_bf16x8(own);
    vnew = pack_bf16x8(vv);
  }
  // the split that owns the last page appends them for later steps (nothing reads them in this
  // step: the newest row is taken from registers below)
  const bool mine_last = p0 <= last_page && last_page < p1;
  if (mine_last && ok && wave == 0 && slot == 0) {
    const int phys = a.page_table[last_page];
    if (phys >= 0 && phys < a.n_pages) {
      const size_t e0 = (((size_t)phys * a.Hkv + j) * 16 + (pos & 15)) * D + part * DPL;
      *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(k_pool) + e0) = knew;
      *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(v_pool) + e0) = vnew;
    }
  }
  const int new_sub = (pos & 15) >> 2, new_slot = pos & 3;

  float m[G], l[G], o[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] = 0.f;
  }
  auto page = [&](u32x4 (&kq)[4], u32x4 (&vq)[4], int p) {
    if (p == last_page) {  // the newest token's row comes from registers
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
        if (sub == new_sub && slot == new_slot) {
          kq[sub] = knew;
          vq[sub] = vnew;
        }
    }
    attend_page8<G>(kq, vq, p, T, slot, q, m, l, o);
  };
  if (ok) {
    if (have[0]) page(kp[0], vp[0], p0 + wave);
    if (have[1]) page(kp[1], vp[1], p0 + wave + 4);
    for (int p = p0 + wave + 8; p < p1; p += 4) {
      const int phys = a.page_table[p];
      if (phys < 0 || phys >= a.n_pages) continue;
      const size_t base = ((size_t)phys * a.Hkv + j) * head_stride;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const uint32_t e = (uint32_t)((base + (size_t)(sub * 4 + slot) * D + part * DPL) * 2);
        kp[0][sub] = load_row8_raw(kpool, e);
        vp[0][sub] = load_row8_raw(vpool, e);
      }
      page(kp[0], vp[0], p);
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
  // publish the split's partial: o at [s][head][D], (m, l) at [s][head][2]
  float *wso = a.attn_ws;
  float *wsml = a.attn_ws + (size_t)a.splits * a.Hq * D;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx - h * D;
    float mx = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, sm.m[w][h]);
    float val = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) val += exp2f(sm.m[w][h] - mx) * sm.o[w][h][d];
    __hip_atomic_store(wso + ((size_t)s * a.Hq + j * G + h) * D + d, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float mx = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, sm.m[w][h]);
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) lsum += exp2f(sm.m[w][h] - mx) * sm.l[w][h];
    float *dst = wsml + ((size_t)s * a.Hq + j * G + h) * 2;
    __hip_atomic_store(dst, mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(dst + 1, lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  drain_stores();
  wave_mark(a.wave_ts, 5 * c.l + 1, NWall, gwv, 2, lane);
  __syncthreads();
  if (threadIdx.x == 0)
    sm.last = __hip_atomic_fetch_add(&a.attn_cnt[j * kLine], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(a.splits - 1);
  __syncthreads();
  if (!sm.last) return;

  // the last split of KV head j merges the splits of its G query heads; every pass issues all of
  // its loads before using them (one memory round trip per pass)
  const __amdgpu_buffer_rsrc_t mlr = rsrc(wsml, (uint32_t)((size_t)a.splits * a.Hq * 2 * 4));
  for (int idx = threadIdx.x; idx < a.splits * G; idx += 256) {
    const int ss = idx / G, h = idx - ss * G;
    const uint64_t v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(
                           mlr, (uint32_t)(((size_t)ss * a.Hq + j * G + h) * 2 * 4), 0, kAuxSc1));
    sm.wm[ss][h] = __builtin_bit_cast(float, (uint32_t)v);
    sm.wl[ss][h] = __builtin_bit_cast(float, (uint32_t)(v >> 32));
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = kNegBig;
    for (int ss = 0; ss < a.splits; ++ss) M = fmaxf(M, sm.wm[ss][h]);
    float Lsum = 0.f;
    for (int ss = 0; ss < a.splits; ++ss) Lsum = fmaf(exp2f(sm.wm[ss][h] - M), sm.wl[ss][h], Lsum);
    sm.M[h] = M;
    sm.L[h] = Lsum;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.splits * G; idx += 256) {
    const int ss = idx / G, h = idx - ss * G;
    sm.wm[ss][h] = exp2f(sm.wm[ss][h] - sm.M[h]) / sm.L[h];
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t orr = rsrc(wso, (uint32_t)((size_t)a.splits * a.Hq * D * 4));
  for (int t = threadIdx.x; t < G * D / 4; t += 256) {
    const int h = t / (D / 4), d4 = (t - h * (D / 4)) * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.splits; s0 += kMergeChunk) {
      f32x4 v[kMergeChunk];
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u)  // splits past the last lie outside the resource: 0
        v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                   orr, (uint32_t)((((size_t)(s0 + u) * a.Hq + j * G + h) * D + d4) * 4), 0, kAuxSc1));
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u)
        if (s0 + u < a.splits) acc += sm.wm[s0 + u][h] * v[u];
    }
    float *dst = a.attn + (size_t)(j * G + h) * D + d4;
#pragma unroll
    for (int e = 0; e < 4; ++e) st_f<true>(dst + e, acc[e]);
  }
  drain_stores();
  __syncthreads();
  if (threadIdx.x < 64) {
    const int ln = threadIdx.x;
    unsigned prev = 0;
    if (ln == 0) {
      __hip_atomic_store(&a.attn_cnt[j * kLine], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prev = __hip_atomic_fetch_add(a.attn_all + c.l * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev + 1 == (c.e + 1u) * (unsigned)a.Hkv)
      publish(reinterpret_cast<unsigned long long *>(a.progress), c.e * c.pps + 3ull * c.l + 1, ln);
    mark_time(a.phase_ts, 1 + 5 * c.l + 1, ln);
    wave_mark(a.wave_ts, 5 * c.l + 1, NWall, gwv, 3, ln);
  }
}

template <int FMT, int G>
__global__ void __launch_bounds__(256, 2) decode_step_fused(const FusedArgs a) {
  constexpr int CK = (FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16;
  __shared__ FusedSmem<CK, 128, G> sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * 4 + wave;
  const int L = a.L;
  const int pos = __builtin_amdgcn_readfirstlane(*a.pos);
  if (pos < 0 || pos >= a.n_pages * 16) {  // no page for the new token: report, touch nothing
    if (threadIdx.x == 0) __hip_atomic_store(a.err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  StepCtx c;
  c.e = __builtin_amdgcn_readfirstlane(__hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  c.pps = 3ull * (unsigned)L + 1ull;
  {
    const int tk = __builtin_amdgcn_readfirstlane(__hip_atomic_load(a.token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    c.tok = (tk < 0 || tk >= a.V) ? 0 : tk;
  }
  c.G = G;
  if (a.phase_ts && gw == 0 && lane == 0) a.phase_ts[0] = wall_clock64();

  // this workgroup's RoPE table for the step's position (fp64 angles)
  if (wave == 0) {
    const double theta = pow((double)a.rope_base, -2.0 * (double)lane / 128.0);
    double sn, cs;
    sincos((double)pos * theta, &sn, &cs);
    sm.cs[lane][0] = cs;
    sm.cs[lane][1] = sn;
  }
  __syncthreads();

  const unsigned long long *prog =
      reinterpret_cast<const unsigned long long *>(a.progress) + (blockIdx.x % kProgressReplicas) * 16;
  const unsigned long long base = c.e * c.pps;
  XStage<CK> &xs = sm.xs[wave];
  for (int l = 0; l < L; ++l) {
    c.l = l;
    const FusedLayer &Lw = a.layers[l];
    // qkv GEMV: RMSNorm prologue (layer 0 reads the embedding row itself), bias
    if (l == 0)
      sk_gemv<FMT, FE_QKV, true>(a, a.p_qkv, c, Lw, Lw.w_qkv, Lw.s_qkv, nullptr, nullptr, a.H, gw, xs, lane, prog, 0,
                                 5 * l);
    else
      sk_gemv<FMT, FE_QKV, false>(a, a.p_qkv, c, Lw, Lw.w_qkv, Lw.s_qkv, a.xa, a.ssqA, a.H, gw, xs, lane, prog,
                                  base + 3ull * l, 5 * l);
    // attention: q/k norm, RoPE, KV append, split partials, merge
    for (int u = blockIdx.x; u < a.Hkv * a.splits; u += gridDim.x) {
      const int jh = u / a.splits, s = u - jh * a.splits;
      attn_unit<G>(a, c, Lw, jh, s, pos, sm.at, sm.cs);
      __syncthreads();  // the attention scratch is reused by the next unit
    }
    // o GEMV + residual (writes hB, its sums of squares and hB * g_ffn)
    sk_gemv<FMT, FE_O, false>(a, a.p_o, c, Lw, Lw.w_o, Lw.s_o, a.attn, nullptr, a.Hq * 128, gw, xs, lane, prog,
                              base + 3ull * l + 1, 5 * l + 2);
    // gate/up GEMV (RMSNorm prologue) + SwiGLU
    sk_gemv<FMT, FE_GU, false>(a, a.p_gu, c, Lw, Lw.w_gu, Lw.s_gu, a.xb, a.ssqB, a.H, gw, xs, lane, prog,
                               base + 3ull * l + 2, 5 * l + 3);
    // down GEMV + residual (writes hA); waits per gate/up tile
    sk_gemv<FMT, FE_DOWN, false>(a, a.p_down, c, Lw, Lw.w_down, Lw.s_down, a.mlp, nullptr, a.I, gw, xs, lane,
                                 prog, 0, 5 * l + 4);
  }
  // lm head (final RMSNorm prologue) + greedy argmax; its last finisher completes the step
  c.l = L;
  sk_gemv<FMT, FE_LM, false>(a, a.p_lm, c, a.layers[0], a.w_lm, a.s_lm, a.xa, a.ssqA, a.H, gw, xs, lane, prog,
                             base + 3ull * L, 5 * L);
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
