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
//   * the activation chunk is the same for all lanes: it is staged once per batch of runs in LDS
//     and read back as a broadcast, so the dot product needs no cross-lane reduction,
//   * the K dimension is split across waves to fill the 256 CUs when N is small; partial sums
//     go to a workspace and the last wave to arrive at a tile adds them in a fixed order
//     (deterministic, no float atomics) and runs the epilogue.
// INT4 codes are unpacked with two AND masks per 8 codes (low nibbles in place, high nibbles in
// place as 16 c, met by activations pre-divided by 16), then v_cvt_f32_ubyte{0..3}; the zero
// point is folded out of the inner loop:
//   sum_k (c_k - 8) x_k = sum_k c_k x_k - 8 sum_k x_k,  with sum_k x_k computed once per chunk.
// INT8 codes are biased to unsigned by XOR 0x80 (c + 128) and folded the same way.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>

#include "qdec_device.h"

namespace qdec {

namespace {

using namespace dev;

// Waves a launch aims for: few k-splits keep the split-K tail short on small matrices (up to 128
// tiles), more waves stream the large ones (measured on MI355X: for the down projections about
// seven waves per compute unit, the most whose k-splits still fit one burst of partial loads in
// the combine, beat four and six; one wave per SIMD hides too little latency, and 35 k-splits
// need a second burst).
constexpr int kTargetUnitsSmall = 1792;
constexpr int kTargetUnitsLarge = 2048;
constexpr int kMinChunks = 4;       // at least 4 KiB of weights per wave

// Standalone launch: one wave per (tile, k-split) unit, no cross-phase dependency.
template <int FMT, bool NORM, int EPI>
__global__ void __launch_bounds__(64 * kMaxGemvWaves) gemv_tile64(const GemvArgs a) {
  __shared__ Stage<(FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16> stage_all[kMaxGemvWaves][2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = wave * gridDim.x + blockIdx.x;
  if (unit >= ((a.N + kTile - 1) / kTile) * a.ks) return;  // whole wave
  // optional timeline, per unit: entry, loads issued, computed, combined (the tile's last wave),
  // exit (slots 0, 1, 3, 4, 5)
  unsigned long long *rec = a.timeline ? a.timeline + (size_t)unit * 8 : nullptr;
  mark(rec, 0);
  GemvUnit<FMT, NORM, EPI, kSyncNone> u;
  u.start(a, unit, lane);
  mark(rec, 1);
  u.finish(a, stage_all[wave], lane, nullptr, rec ? rec + 2 : nullptr);
  mark(rec, 5);
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
  gemv_apply_plan(a, p, FMT);
  hipLaunchKernelGGL((gemv_tile64<FMT, NORM, EPI>), dim3(p.blocks), dim3(64 * p.wpb), 0, st, a);
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

void gemv_apply_plan(GemvArgs &a, const GemvPlan &p, int wfmt) {
  a.ks = p.ks;
  a.cps = p.cps;
  int gshift = 0;
  if (wfmt == QDEC_W_Q4_G_ZP8)
    while ((32 << gshift) < a.group) ++gshift;  // group = 32 << gshift (checked by the callers)
  a.group = gshift;
}

GemvPlan gemv_plan(int wfmt, int N, int K, bool allow_split, int target_small) {
  GemvPlan p;
  const int ck = (wfmt == QDEC_W_Q4_G_ZP8) ? 32 : 16;
  p.tiles = (N + kTile - 1) / kTile;
  p.nch = K / ck;
  int ks = 1;
  if (allow_split && p.tiles <= kMaxSplitTiles) {
    const int target = p.tiles <= 128 ? (target_small > 0 ? target_small : kTargetUnitsSmall) : kTargetUnitsLarge;
    ks = (target + p.tiles / 2) / p.tiles;
    // (at most one burst of partial loads in the combine: a second costs a round trip)
    ks = max(1, min(min(ks, kCombineBurst), p.nch / kMinChunks));
  }
  p.cps = (p.nch + ks - 1) / ks;
  p.ks = (p.nch + p.cps - 1) / p.cps;
  p.units = p.tiles * p.ks;
  gemv_set_grid(p);
  return p;
}

void gemv_set_grid(GemvPlan &p) {
  p.wpb = std::max(1, std::min(kMaxGemvWaves, (p.units + kComputeUnits - 1) / kComputeUnits));
  p.blocks = (p.units + p.wpb - 1) / p.wpb;
}

// Workspace layout, shared by every GEMV that runs on it one after another: the arrival counters
// (one per 128-byte line: tile counters from line 0, then the argmax top and group counters at
// the end of the region) sit in a fixed region at the start; each launch leaves the ones it used
// at zero, so the region stays zero between launches whatever the shape.  Split-K partials
// follow, then the argmax candidates (per tile, then per group).
size_t gemv_workspace_bytes(int wfmt, int N, int K, bool argmax) {
  GemvPlan p = gemv_plan(wfmt, N, K, true);
  size_t b = kCounterBytes;
  if (p.ks > 1) b += (size_t)p.tiles * p.ks * kTile * sizeof(float);
  if (argmax) b += (size_t)(p.tiles + kArgGroups) * 2 * sizeof(float);
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
