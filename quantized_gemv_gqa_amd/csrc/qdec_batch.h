// Internal declarations of the batched decode path (several sequences, one token each).
#pragma once
#include "qdec_internal.h"

namespace qdec {

// Skinny GEMM (gemm_b.hip): Y[b] = W X[b] for b < nb columns, nb <= nb_max in {2, 4, 8}.
struct GemmBArgs {
  const uint8_t *W;        // packed tile64 weights
  const void *S;           // packed scales
  const float *X;          // activations [nb][ldx]
  int ldx;
  const float *bias;       // [N] or null
  const float *residual;   // [nb][ldy] or null (may alias Y)
  float *Y;                // [nb][ldy]; EPI_SWIGLU: [nb][ldy] with N / 2 outputs per column
  int ldy;
  float *part;             // set by the launcher from the workspace
  unsigned *counters;
  int N, K, group;
  int gshift, ks, cps;     // set by the launcher
  int nb, nb_max;
  int epi;                 // EPI_STORE or EPI_SWIGLU
  const int32_t *pos;      // [nb] or null: columns with pos[b] < 0 are computed but not stored
};
int gemm_b_columns(int batch);  // nb_max for a batch size (2, 4 or 8)
size_t gemm_b_workspace_bytes(int wfmt, int N, int K, int nb_max);
hipError_t launch_gemm_b(int wfmt, GemmBArgs a, void *ws, hipStream_t st);

// Row kernels of the batched step (elementwise.hip).  A row b with pos[b] < 0 is idle.
// h[b] = bf16 -> fp32 E[tokens[b]]; rope_cs[b] = the fp64 (cos, sin) table of pos[b] (D/2 pairs)
hipError_t launch_embed_rows(const uint16_t *E, const int32_t *tokens, const int32_t *pos, int B, int H, int V,
                             float *h, float rope_base, int D, double *rope_cs, hipStream_t st);
// y[b] = gamma * x[b] / sqrt(mean(x[b]^2) + eps); dim a multiple of 4, at most 16384; x, y, gamma
// 16-byte aligned
hipError_t launch_rmsnorm_rows(const float *x, const float *gamma, float *y, int B, int dim, float eps, hipStream_t st);
// tokens[b] = argmax of logits[b] (smallest index among equal maxima), pos[b] += 1, for running
// rows; two launches (chunk candidates in ws, then one wave per row)
size_t argmax_rows_workspace_bytes(int B);
hipError_t launch_argmax_rows(const float *logits, int B, int V, int32_t *tokens, int32_t *pos, void *ws,
                              hipStream_t st);

// Batched attention (attention.hip): the step form of the attention unit (raw qkv, q/k norm, RoPE
// from rope_cs, KV append by split 0) for every running sequence b, with q/k/v, rope table,
// position, block table row, workspace and output offset by b.  Sequences whose position is
// negative or reaches max_blocks * 16 are skipped.
struct AttnBatch {
  AttnArgs a;              // fields of sequence 0; per-sequence pointers below
  const float *qkv;        // [B][(Hq + 2 Hkv) D]
  const double *rope_cs;   // [B][D]
  const int32_t *pos;      // [B]
  const int32_t *tables;   // [B][max_blocks]
  int max_blocks;
  char *ws;                // [B][ws_stride] bytes: each sequence's attention workspace
  size_t ws_stride;
  float *out;              // [B][Hq D]
  int B;
};
hipError_t launch_attention_batch(const AttnBatch &ab, hipStream_t st);

}  // namespace qdec
