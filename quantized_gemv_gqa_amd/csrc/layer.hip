// Fused attention kernel: the attention half of a decoder layer (qkv GEMV, split attention, o
// GEMV) in one launch instead of three.
//
// What they compute is exactly what the per-op kernels compute (the same device code runs); what
// changes is when.  Launched one after another, each piece pays its own ramp-up and drain, which
// for the small pieces (the qkv and o GEMVs, attention) is most of their time.  Here pieces with
// a narrow data dependency share one launch, as workgroup roles ordered by block index:
//
//   [qkv GEMV units] [attention units (KV head j, split s)] [o GEMV units]
//
// and a consumer waits only for the producers of its own inputs:
//   * attention unit (j, s) requests its first KV pages, then waits until the 2G + 4 qkv tiles of
//     KV head j (its G q heads, its k and v) are stored, counted per head;
//   * an o GEMV unit requests its first weights, then waits for the attention outputs of the KV
//     heads whose query heads cover its k-range (a flag per KV head, set by the split merge).
// The MLP half stays two plain launches: the RMSNorm before gate/up needs the whole o output, and
// all gate/up tiles finish at about the same time, so a down GEMV sharing their launch could
// only wait (measured: one launch for both was slower than two).  The residual stream alternates
// between two buffers (hA, read by the qkv GEMV and as o's residual, written by down; hB, written
// by o and read by gate/up and down), so no unit overwrites a vector that a unit of the same
// launch may still read.
//
// Ordering and progress: workgroups are dispatched in block-index order, so every producer a
// unit waits for was dispatched before it; producers never wait.  Waits are bounded polls: a step
// whose producers do not arrive in time sets the step's error word instead of hanging.
//
// Flags and counters are monotonic: the step number e (advanced by the embedding kernel at the
// start of each step) is the target, so nothing has to be cleared between steps.  Data crossing
// workgroups inside a launch uses device-coherent stores and loads (sc1), and a producer's
// counter moves only after its stores are acknowledged.
#include <hip/hip_runtime.h>

#include "qdec_attention.h"

namespace qdec {

namespace {

using namespace dev;

constexpr int kAttnLayerWaves = attn::kAttnWaves;  // 8 waves: attention units need a whole workgroup

__device__ __forceinline__ int gemv_units(const GemvArgs &g) { return ((g.N + kTile - 1) / kTile) * g.ks; }

template <int FMT, int G, int KVF>
__global__ void __launch_bounds__(attn::kAttnThreads) attn_layer_k(const LayerArgs a) {
  constexpr int CK = (FMT == QDEC_W_Q4_G_ZP8) ? 32 : 16;
  union Smem {
    Stage<CK> st[kAttnLayerWaves][2];
    attn::AttnSmem<128, G, true> at;
  };
  __shared__ Smem sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int b = blockIdx.x;
  if (b < a.nb_qkv) {
    const int unit = b * kAttnLayerWaves + wave;
    if (unit < gemv_units(a.qkv)) gemv_unit<FMT, true, EPI_STORE, kSyncProducer>(a.qkv, unit, sm.st[wave], lane);
    return;
  }
  b -= a.nb_qkv;
  const int natt = a.at.Hkv * a.at.splits;
  if (b < natt) {
    attn::attn_unit<128, G, KVF, true, true>(a.at, b / a.at.splits, b % a.at.splits, sm.at);
    return;
  }
  b -= natt;
  const int unit = b * kAttnLayerWaves + wave;
  if (unit < gemv_units(a.o)) gemv_unit<FMT, false, EPI_STORE, kSyncConsumer>(a.o, unit, sm.st[wave], lane);
}

template <int FMT, int KVF>
hipError_t launch_attn_g(const LayerArgs &a, int G, hipStream_t st) {
  const int blocks = a.nb_qkv + a.at.Hkv * a.at.splits + a.nb_o;
  switch (G) {
    case 4: hipLaunchKernelGGL((attn_layer_k<FMT, 4, KVF>), dim3(blocks), dim3(attn::kAttnThreads), 0, st, a); break;
    case 6: hipLaunchKernelGGL((attn_layer_k<FMT, 6, KVF>), dim3(blocks), dim3(attn::kAttnThreads), 0, st, a); break;
    case 7: hipLaunchKernelGGL((attn_layer_k<FMT, 7, KVF>), dim3(blocks), dim3(attn::kAttnThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL((attn_layer_k<FMT, 8, KVF>), dim3(blocks), dim3(attn::kAttnThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool layer_fusion_supported(int G, int D) { return D == 128 && (G == 4 || G == 6 || G == 7 || G == 8); }

int attn_layer_waves() { return kAttnLayerWaves; }

hipError_t launch_attn_layer(const LayerArgs &a, int wfmt, hipStream_t st) {
  const int G = a.at.Hq / a.at.Hkv;
  if (wfmt == QDEC_W_Q4_G_ZP8)
    return a.at.kv_fmt == QDEC_KV_BF16 ? launch_attn_g<QDEC_W_Q4_G_ZP8, QDEC_KV_BF16>(a, G, st)
                                       : launch_attn_g<QDEC_W_Q4_G_ZP8, QDEC_KV_F32>(a, G, st);
  return a.at.kv_fmt == QDEC_KV_BF16 ? launch_attn_g<QDEC_W_Q8_ROW, QDEC_KV_BF16>(a, G, st)
                                     : launch_attn_g<QDEC_W_Q8_ROW, QDEC_KV_F32>(a, G, st);
}

}  // namespace qdec
