// Internal declarations of the batched decode path (several sequences, one token each).
#pragma once
#include "qdec_internal.h"

namespace qdec {

// Skinny GEMM (gemm_b.hip): Y[b] = W X[b] for b < nb columns, nb <= nb_max in {1, 2, 4, 8}.
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
  // Folded RMSNorm (gamma non-null): column b is used as gamma * x_b / sqrt(mean(x_b^2) + eps),
  // with sum(x_b^2) the sum of ssq[b * ssq_n + t] over t < ssq_n (per-64-row-tile sums, written
  // by the producer of X).
  const float *gamma;
  const float *ssq;
  int ssq_n;
  float eps;
  // EPI_STORE: if non-null, ssq_out[b * ceil(N / 64) + t] = sum of the squares of column b's
  // stored outputs in rows 64 t .. 64 t + 63 (stored columns only)
  float *ssq_out;
};
int gemm_b_columns(int batch);  // nb_max for a batch size (1, 2, 4 or 8)
size_t gemm_b_workspace_bytes(int wfmt, int N, int K, int nb_max);
hipError_t launch_gemm_b(int wfmt, GemmBArgs a, void *ws, hipStream_t st);

// Prefill GEMM on the matrix cores (gemm_p.hip): Y[m][n] = sum_k X[m][k] w[n][k] for m < M, with
// activations given as fp16 pairs X = Xh + Xl ([M][ldx] each, ldx % 8 == 0; Xl null: Xh alone),
// K % 32 == 0; fp32 output, + bias[n], + residual[m][n] (same layout as Y, may alias it), or the
// SwiGLU of the gate/up row pairs with EPI_SWIGLU, written as an fp16 pair (Yh, Yl) [M][ldy]
// (N / 2 outputs) when Yh is set.
struct GemmPArgs {
  const uint8_t *W;
  const void *S;
  const uint16_t *X, *Xl;  // fp16 bits: high and low parts
  int ldx;
  const float *bias, *residual;
  float *Y;
  uint16_t *Yh, *Yl;       // EPI_SWIGLU: fp16 pair output [M][ldy] instead of Y
  int ldy;
  int M, N, K, group;
  int epi;
  // k-split (EPI_STORE only): split z writes its fp32 partial to part[z][M][N], and a reduce
  // launch adds the splits in order (deterministic) and applies scale, bias and residual
  int ks;
  float *part;
};
// k-splits a prefill GEMM uses (1 when its tiles already fill the GPU); part needs
// ks * M * N floats
int gemm_p_splits(int M, int N, int K, int epi);
hipError_t launch_gemm_p(int wfmt, const GemmPArgs &a, hipStream_t st);

// Prefill row kernels (elementwise.hip)
// pos_rows[t] = *pos + t for t < T
hipError_t launch_prefill_positions(const int32_t *pos, int T, int32_t *pos_rows, hipStream_t st);
// *pos += delta
hipError_t launch_add_pos(int32_t *pos, int delta, hipStream_t st);
// x[t] = E[tokens[t]] (bf16 -> fp32), t < T
hipError_t launch_embed_tokens(const uint16_t *E, const int32_t *tokens, int T, int H, int V, float *x, hipStream_t st);
// fp16 pair rows: v = gamma * x[b] / sqrt(mean(x[b]^2) + eps) as yh = fp16(v), yl = fp16(v - yh);
// and the same split of plain fp32 values
hipError_t launch_rmsnorm_rows_h(const float *x, const float *gamma, uint16_t *yh, uint16_t *yl, int B, int dim,
                                 float eps, hipStream_t st);
hipError_t launch_to_half(const float *x, uint16_t *yh, uint16_t *yl, size_t n, hipStream_t st);
// per token t and head: q/k RMSNorm (optional), RoPE at pos_rows[t], k and v stored into the pools
// at the page of pos_rows[t]; qkv [T][(Hq + 2 Hkv) D] rewritten in place (q, k rotated)
struct QkvRows {
  QkvPostArgs a;            // per-sequence fields (qkv, pos unused)
  float *qkv;
  const int32_t *pos_rows;
  int T;
};
hipError_t launch_qkv_post_rows(const QkvRows &r, hipStream_t st);

// Prefill attention (attention.hip): query t of the prompt (rotated q at q + t * q_stride) over
// keys 0 .. pos_rows[t] of the sequence's pages, one split; out [T][Hq D].
struct AttnRows {
  AttnArgs a;               // pools, page table, heads, scale (q, pos, ws, out per row below)
  const float *q;
  int q_stride;
  const int32_t *pos_rows;
  char *ws;
  size_t ws_stride;
  float *out;
  int T;
};
hipError_t launch_attention_rows(const AttnRows &r, hipStream_t st);

// Row kernels of the batched step (elementwise.hip).  A row b with pos[b] < 0 is idle.
// h[b] = bf16 -> fp32 E[tokens[b]]; rope_cs[b] = the fp64 (cos, sin) table of pos[b] (D/2 pairs);
// ssq (if non-null) [B][ceil(H / 64)]: the sums of squares of h[b] per 64-value tile
hipError_t launch_embed_rows(const uint16_t *E, const int32_t *tokens, const int32_t *pos, int B, int H, int V,
                             float *h, float *ssq, float rope_base, int D, double *rope_cs, hipStream_t st);
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
