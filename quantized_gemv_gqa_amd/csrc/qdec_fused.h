// Host/device interface of the persistent decode-step kernel.
#pragma once
#include "qdec_internal.h"

namespace qdec {

// Per-layer device pointers, stored in device memory (a table in the step workspace).
struct FusedLayer {
  const uint8_t *w_qkv, *w_o, *w_gu, *w_down;
  const void *s_qkv, *s_o, *s_gu, *s_down;
  const float *b_qkv, *g_attn, *g_ffn, *g_q, *g_k;
  void *k_pool, *v_pool;
};

// Stream-K partition of one GEMV over the waves of the persistent grid.  The packed weights of a
// GEMV are R = tiles * nch 1 KiB runs laid out back to back (run r = tile r / nch, chunk r % nch);
// wave w < nw takes the contiguous runs [w q + min(w, rem), ... + q + (w < rem)).  A tile whose
// runs are split over several waves is summed by its last contributor from `part`, in wave
// order, so the result does not depend on arrival order.
constexpr int kMaxSlots = 64;  // contributors of one tile at most
struct SkPhase {
  int tiles, nch, nw, q, rem;
  int slots;                   // partial slots per tile (>= max contributors)
  float *part;                 // [tiles][slots][64] partial sums
  unsigned *tile_cnt;          // arrival counter of tile t at [t * kLine], zero between uses
};

struct FusedArgs {
  const FusedLayer *layers;    // device [L]
  int L, H, Hq, Hkv, V, I, splits, n_pages, gshift;
  float eps, scale_log2, rope_base;
  const uint16_t *embed;       // bf16 [V][H]
  const uint8_t *w_lm;
  const void *s_lm;
  const float *g_out;
  const int32_t *page_table;
  int32_t *pos, *token, *token_log, *step_count;
  int log_len;
  // activations: hA = residual stream entering a layer (written by down), hB = after the
  // attention block (written by o); ssqA / ssqB are their per-64-row sums of squares
  float *hA, *hB, *ssqA, *ssqB, *trace, *logits, *qkv, *attn, *mlp, *attn_ws;
  // inputs of the RMSNorm-prologue GEMVs with the gain applied by their producer:
  // xa = hA * (next layer's attention gain, or the final gain), xb = hB * (MLP gain)
  float *xa, *xb;
  // synchronisation (device-coherent, every counter on its own 128-byte line unless noted).
  // Counters that consumers poll are monotonic across steps: a step with epoch e waits for
  // (e + 1) * arrivals, compared modulo 2^32.
  unsigned *epoch;             // fused steps completed
  unsigned *qkv_done;          // [L][Hkv]: qkv tiles of KV head j finished
  unsigned *attn_all;          // [L]: KV heads merged (last one publishes progress)
  unsigned *o_done;            // [L]: o tiles finished
  unsigned *down_done;         // [L]: down tiles finished
  unsigned *gu_flag;           // [L][tiles_gu] (packed): e + 1 once gate/up tile t is stored
  unsigned *progress;          // [kProgressReplicas lines]: e * (3L + 1) + phases completed
  unsigned *attn_cnt;          // split arrivals of KV head j at [j * kLine] (reset by the merger)
  unsigned *lm_sub;            // [64 lines] argmax arrivals per tile group (reset by the last)
  unsigned *lm_top;            // argmax groups finished (reset by the last)
  float *cand;                 // [tiles_lm][2] per-tile (value, index)
  float *sub_cand;             // [64][2] per-group (value, index)
  unsigned *err;               // set when a bounded wait gives up
  unsigned long long *phase_ts;  // optional [2 + 5 L]: start, per-phase last finish, lm finish
  unsigned *wave_ts;           // optional [5 L + 1][waves][4]: per-wave marks (low 32 bits of the clock)
  SkPhase p_qkv, p_o, p_gu, p_down, p_lm;
};

bool fused_supported(int wfmt, int G, int D, int kv_fmt);
int fused_blocks_per_cu(int wfmt, int G);
hipError_t launch_fused(const FusedArgs &a, int wfmt, int G, int blocks, hipStream_t st);

}  // namespace qdec
