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

struct FusedArgs {
  const FusedLayer *layers;  // device [L]
  int L, H, Hq, Hkv, V, splits, n_pages;
  float eps, scale_log2, rope_base;
  const uint16_t *embed;
  const int32_t *page_table;
  int32_t *pos, *token;
  float *hidden, *trace, *qkv, *attn, *ssq, *attn_ws;
  double *rope_cs;           // [64][2] (cos, sin) of this step's position
  unsigned *attn_cnt;        // [Hkv]
  unsigned *done;            // [2 + 5 L] phase counters, zero between steps
  unsigned *progress;        // [kProgressReplicas * 32]: phases completed, one replica per line
  unsigned *err;             // set when a bounded wait gives up
  unsigned long long *phase_ts;  // optional [3 + 5 L]: [0] kernel start, [1 + k] phase k done
  GemvPlan p_qkv, p_o, p_gu, p_down, p_lm;
  GemvArgs g_qkv, g_o, g_gu, g_down, g_lm;  // per-phase templates; per-layer pointers filled in-kernel
};

bool fused_supported(int wfmt, int G, int D, int kv_fmt);
int fused_blocks_per_cu(int wfmt, int G);
hipError_t launch_fused(const FusedArgs &a, int wfmt, int G, int blocks, hipStream_t st);

}  // namespace qdec
