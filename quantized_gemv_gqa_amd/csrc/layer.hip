// Fused attention kernel: the attention half of a decoder layer (qkv GEMV, split attention with
// its merge, o GEMV) in one launch.
//
// What it computes is exactly what the per-op kernels compute (the same device code runs, with
// the same split of the work, so results are equal bit for bit); what changes is when.
//
// One workgroup of 8 waves per compute unit, and every workgroup takes part in every phase:
//   wave w of workgroup b holds qkv GEMV unit w nblk + b and o GEMV unit (7 - w) nblk + b (units
//   dealt over the workgroups first, so each compute unit streams an equal share), and the
//   workgroup as a whole holds attention unit (KV head b / splits, split b % splits) if b is
//   below Hkv * splits.
// A wave first streams and computes its qkv unit; then it requests its first KV quarters
// (registers), and once the attention has its pages, its o weights, which are copied straight
// from HBM into an LDS stash and need no registers while the attention publishes and merges.  So
// the qkv weights stream alone, the later phases' bytes land during the waits, and what remains
// are the hand-offs:
//   * attention unit (j, s) waits until the 2G + 4 qkv tiles of KV head j (its G q heads, its k
//     and v) are stored, counted per head;
//   * the splits publish their partials as (value, tag) pairs, one 8-byte store each, which a
//     reader sees whole or not at all; query head j G + i is merged by split i of KV head j (all
//     G heads in parallel), which polls the tags of every split's partial, so the splits neither
//     wait for their stores to be acknowledged nor count themselves in;
//   * the merged outputs go out as tagged pairs too, and an o GEMV unit polls the pairs of its
//     k-range directly (no flag).  The tag is the step number times the layer count plus the
//     layer, so a pair left by another layer or step never matches.
// Producers never wait for consumers, and the grid is one workgroup per compute unit of a
// kernel that fits once per unit, so all workgroups are resident together and every wait is
// for a workgroup that is running.  Waits are bounded polls: a step whose producers do not
// arrive in time sets the step's error word instead of hanging.
//
// Counters and tags are monotonic: the step number e (advanced by the embedding kernel at the
// start of each step) sets the target, so nothing has to be cleared between steps.  Data crossing
// workgroups inside a launch uses device-coherent stores and loads (sc1), and a producer's
// counter moves only after its stores are acknowledged.  The residual stream alternates between
// two buffers (hA, read by the qkv GEMV and as o's residual, written by down; hB, written by o
// and read by gate/up and down), so no unit overwrites a vector that a unit of the same launch
// may still read.
#include <hip/hip_runtime.h>

#include "qdec_attention.h"

namespace qdec {

namespace {

using namespace dev;

constexpr int kAttnLayerWaves = attn::kAttnWaves;  // 8 waves: attention units need a whole workgroup
// o units go to the waves that do not stage the attention's inputs when they fit there
constexpr int kOWaves = kAttnLayerWaves - attn::AttnUnit<128, 4, QDEC_KV_BF16, true, true>::kRopeWaves;

__device__ __forceinline__ int gemv_units(const GemvArgs &g) { return ((g.N + kTile - 1) / kTile) * g.ks; }

template <int FMT, int G, int KVF>
__global__ void __launch_bounds__(attn::kAttnThreads) attn_layer_k(const LayerArgs a) {
  constexpr int CK = (FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16;
  union Smem {
    Stage<CK> st[kAttnLayerWaves][2];
    attn::AttnSmem<128, G, true> at;
  };
  __shared__ Smem sm;
  __shared__ u32x4 stash[kAttnLayerWaves][kStashRuns * kTile];  // o weights, 8 KiB per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  // GEMV units are dealt over the workgroups first: qkv unit w nblk + b to wave w, o unit
  // w nblk + b to wave 7 - w, o on the last o_waves waves (4 when they suffice: then the
  // attention's staging waves keep no stash copies in flight)
  const int nq = gemv_units(a.qkv), no = gemv_units(a.o);
  const int uq = wave * a.nblk + b;
  const int uo = (kAttnLayerWaves - 1 - wave) * a.nblk + b;
  const bool q_role = uq < nq;
  const bool o_role = wave >= kAttnLayerWaves - a.o_waves && uo < no;
  const bool at_role = b < a.at.Hkv * a.at.splits;  // the same for the whole workgroup
  const int j = b / a.at.splits, s = b - j * a.at.splits;

  GemvUnit<FMT, true, EPI_STORE, kSyncProducer> gq;
  attn::AttnUnit<128, G, KVF, true, true> at;
  GemvUnit<FMT, false, EPI_STORE, kSyncConsumer, true> go;
  // optional timeline: per wave 16 marks (clock at entry, loads issued, qkv computed / combined /
  // stored, attention wait done / pages done / published / merged, o wait done / computed /
  // combined, exit, attention q staged / heads rotated)
  unsigned long long *rec = a.timeline ? a.timeline + ((size_t)b * kAttnLayerWaves + wave) * 16 : nullptr;
  mark(rec, 0);
  if (q_role) {
    gq.start(a.qkv, uq, lane);
    mark(rec, 1);
    gq.finish(a.qkv, sm.st[wave], lane, nullptr, rec ? rec + 2 : nullptr);
  }
  mark(rec, 5);
  // The later phases' bytes are requested once the wave's qkv unit is done, so the qkv weights,
  // on the critical path, do not share HBM with them: the first KV quarters then, the o weights
  // once the attention has its pages (they land while it publishes and merges; requested
  // earlier, they compete with the qkv split-K hand-off).
  if (at_role) at.start(a.at, j, s);
  // (the attention's first LDS write follows a workgroup barrier, so every wave is past its
  // qkv unit's use of the union by then)
  bool at_ok = true;
  if (at_role) at_ok = at.pages(a.at, j, s, sm.at, rec ? rec + 6 : nullptr);
  if (o_role) go.start(a.o, uo, lane, stash[wave]);
  if (at_role && at_ok) at.publish(a.at, j, s, sm.at, rec ? rec + 6 : nullptr);
  if (o_role) go.finish(a.o, sm.st[wave], lane, stash[wave], rec ? rec + 10 : nullptr);
  mark(rec, 13);
}

template <int FMT, int G, int KVF>
const void *kernel_ptr() {
  return reinterpret_cast<const void *>(&attn_layer_k<FMT, G, KVF>);
}

template <int FMT, int KVF>
const void *kernel_g(int G) {
  switch (G) {
    case 4: return kernel_ptr<FMT, 4, KVF>();
    case 6: return kernel_ptr<FMT, 6, KVF>();
    case 7: return kernel_ptr<FMT, 7, KVF>();
    case 8: return kernel_ptr<FMT, 8, KVF>();
    default: return nullptr;
  }
}

const void *layer_kernel(int wfmt, int kv_fmt, int G) {
  if (wfmt == QDEC_W_Q4_G_ZP8)
    return kv_fmt == QDEC_KV_BF16 ? kernel_g<QDEC_W_Q4_G_ZP8, QDEC_KV_BF16>(G) : kernel_g<QDEC_W_Q4_G_ZP8, QDEC_KV_F32>(G);
  return kv_fmt == QDEC_KV_BF16 ? kernel_g<QDEC_W_Q8_ROW, QDEC_KV_BF16>(G) : kernel_g<QDEC_W_Q8_ROW, QDEC_KV_F32>(G);
}

}  // namespace

bool layer_fusion_supported(int G, int D) { return D == 128 && (G == 4 || G == 6 || G == 7 || G == 8); }

int attn_layer_waves() { return kAttnLayerWaves; }

int attn_layer_o_waves() { return kOWaves; }  // preferred; all waves when the o plan needs them

int attn_layer_stash_runs() { return kStashRuns; }

int attn_layer_blocks_per_cu(int wfmt, int kv_fmt, int G) {
  const void *k = layer_kernel(wfmt, kv_fmt, G);
  int nb = 0;
  if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, attn::kAttnThreads, 0) != hipSuccess) return 0;
  return nb;
}

hipError_t launch_attn_layer(const LayerArgs &a, int wfmt, hipStream_t st) {
  const void *k = layer_kernel(wfmt, a.at.kv_fmt, a.at.Hq / a.at.Hkv);
  if (!k) return hipErrorInvalidValue;
  void *args[] = {const_cast<LayerArgs *>(&a)};
  return hipLaunchKernel(k, dim3(a.nblk), dim3(attn::kAttnThreads), args, 0, st);
}

}  // namespace qdec
