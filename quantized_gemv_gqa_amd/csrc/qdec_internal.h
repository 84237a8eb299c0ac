// Internal declarations shared by the qdec HIP sources (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qdec.h"

namespace qdec {

constexpr int kWave = 64;
constexpr int kTile = QDEC_TILE_ROWS;  // rows per packed tile = lanes per wave

// ---------------------------------------------------------------------------------- errors
void set_error(const char *fmt, ...);
#define QDEC_REQUIRE(cond, code, ...)        \
  do {                                       \
    if (!(cond)) {                           \
      ::qdec::set_error(__VA_ARGS__);        \
      return (code);                         \
    }                                        \
  } while (0)
qdec_status check_launch(const char *what);

// ---------------------------------------------------------------------------------- GEMV
enum GemvEpilogue : int {
  EPI_STORE = 0,   // y[n] = acc (+bias) (+residual)
  EPI_SWIGLU = 1,  // packed rows pair gate/up by half tile; y[i] = silu(g_i) * u_i
  EPI_ARGMAX = 2,  // y[n] = acc, then greedy token over all rows (lm head): *token, log, pos += 1
};

struct GemvArgs {
  const uint8_t *W;        // packed weights
  const void *S;           // packed scales (q8: fp32 [Npad], q4: fp16 [tiles][K/group][64])
  const float *x;          // activation [K]
  const float *gamma;      // RMSNorm gain [K] or null: x' = gamma * x, finalizer multiplies by r
  const float *ssq;        // per-tile partial sums of x^2 (ssq_n of them), used with gamma
  int ssq_n;
  float eps;
  const float *bias;       // [N] or null
  const float *residual;   // [N] or null (may alias y)
  float *y;                // output
  float *ssq_out;          // if non-null: per-tile sum of y^2 over the tile's valid rows
  float *part;             // split-K partials [tiles][ks][64]
  unsigned *counters;      // arrival counters (one per 128-byte line), zero between launches
  int N, K, group;
  int ks, cps;             // k splits, chunks per split
  int epi;
  // EPI_ARGMAX: per-tile then per-group (value, index) candidates and the step scalars
  float *cand;
  int32_t *token, *pos, *token_log, *step_count;
  int log_len;
  // Step-synchronised units of the fused layer kernels (null/0 otherwise).  *epoch is the step
  // number e (>= 1).  A consumer unit waits until wait_flags[f] >= e for every f covering its
  // k-range (f = k / wait_div).  A producer unit, after its device-coherent output stores, adds 1
  // to done[KV head of its rows * kLine] (the qkv GEMV, whose Hq, Hkv, hd give the head layout).
  const unsigned *epoch;
  const unsigned *wait_flags;
  int wait_div;
  unsigned *done;
  int Hq, Hkv, hd;
  unsigned *err;  // set on a wait that times out
  unsigned long long *timeline;  // diagnostics: 8 clock marks per unit of a plain launch, or null
  // Consumer form with tagged activations: x is read as (value, tag) pairs from xt, polled until
  // every tag equals *epoch * xt_tag_mul + xt_tag_add (no separate wait).
  const uint32_t *xt;
  unsigned xt_tag_mul, xt_tag_add;
};
// Device atomics to one cache line serialize (about 13 ns each on MI355X), so every arrival
// counter sits on a 128-byte line of its own.
constexpr int kLine = 32;                        // unsigned per 128-byte line
constexpr size_t kCounterBytes = 256 * 1024;     // GEMV arrival-counter region of a workspace
constexpr int kCounterLines = (int)(kCounterBytes / 128);
constexpr int kArgGroups = 64;                   // argmax reduction groups (tile mod 64)
constexpr int kArgGroupLine0 = kCounterLines - kArgGroups;
constexpr int kArgTopLine = kArgGroupLine0 - 1;
constexpr int kMaxSplitTiles = kArgTopLine;      // tiles 0 .. kMaxSplitTiles-1 own lines 0 ..

// A plain GEMV launch deals its units over the workgroups first (unit w * blocks + b to wave w
// of workgroup b), with at most one workgroup per compute unit, so every compute unit streams an
// equal share.
constexpr int kComputeUnits = 256;  // MI355X
constexpr int kMaxGemvWaves = 16;   // waves per workgroup (1024 threads)
struct GemvPlan {
  int tiles, nch, ks, cps, units, blocks, wpb;  // wpb: waves per workgroup
};
// target_small > 0: the waves a launch aims for on matrices of up to 128 tiles, in place of the
// decode GEMV's default
GemvPlan gemv_plan(int wfmt, int N, int K, bool allow_split, int target_small = 0);
void gemv_set_grid(GemvPlan &p);  // blocks and waves per workgroup of a plain launch
// Copy the plan into the arguments a kernel reads (k-splits, runs per split, INT4 group as a
// shift): every launch path calls it once, after the arguments are filled.
void gemv_apply_plan(GemvArgs &a, const GemvPlan &p, int wfmt);
size_t gemv_workspace_bytes(int wfmt, int N, int K, bool argmax = false);
void gemv_bind_workspace(GemvArgs &a, const GemvPlan &p, void *ws);
hipError_t launch_gemv(int wfmt, const GemvArgs &a, const GemvPlan &p, hipStream_t st);

// INT8 activations (gemv_a8.hip): per-group quantisation, and the GEMV on packed weights.
hipError_t launch_quantize_act_i8(const float *x, int K, int group, int8_t *q, float *sx, hipStream_t st);
hipError_t launch_gemv_a8(int wfmt, const uint8_t *W, const void *S, const int8_t *q, const float *sx, int group,
                          const float *bias, const float *residual, float *y, int N, int K, void *ws, hipStream_t st);

// Sampling (sample.hip): temperature / top-k / top-p with a Philox-keyed Gumbel-max draw.
constexpr int kSampleMaxTopK = 256;
size_t sample_workspace_bytes();
hipError_t launch_sample(const float *logits, int V, float temperature, int top_k, float top_p, uint64_t seed,
                         const int32_t *step, int32_t *token, int32_t *token_log, int32_t *step_count, int32_t *pos,
                         int log_len, void *ws, hipStream_t st);

hipError_t launch_pack_q8(const int8_t *W, const float *S, int N, int K, uint8_t *Wp, float *Sp,
                          hipStream_t st);
hipError_t launch_pack_q4(const uint8_t *W, const uint16_t *S, int N, int K, int group, uint8_t *Wp,
                          uint16_t *Sp, hipStream_t st);

// ---------------------------------------------------------------------------------- attention
struct AttnArgs {
  const float *q;          // [Hq][D] (already rotated); unused when qkv is set
  // Step form: when qkv != null, q, k and v are read raw from the fused vector [(Hq + 2 Hkv) D];
  // the kernel applies the optional per-head q/k RMSNorm (g_q, g_k, eps) and RoPE from rope_cs
  // ([D/2] fp64 (cos, sin) pairs of the angle pos * theta_i), appends the rotated k and v at pos,
  // and uses them for the newest token.
  const float *qkv;
  const float *g_q, *g_k;
  float eps;
  const double *rope_cs;
  void *k_pool, *v_pool;
  int kv_fmt;
  const int32_t *page_table;
  int n_pages;
  const int32_t *pos;      // device scalar: token index of the newest key (T = pos + 1)
  int Hq, Hkv, D;
  float scale_log2;        // sm_scale * log2(e)
  int splits;              // <= kMaxMergeSplits
  float *ws;               // [splits][Hq][D + 2] partials
  unsigned *counters;      // arrival counter of KV head j at [j * kLine], zero between launches
  float *out;              // [Hq][D]
  // Step-synchronised form (fused layer kernel; null otherwise): wait until
  // wait_cnt[j * kLine] >= *epoch * wait_per_step (the qkv tiles of KV head j are stored), read qkv
  // with device-coherent loads, publish the split's partial as (value, tag) pairs in tws
  // ([splits][Hq][D] pairs, then [splits][Hq] (m, tag, l, tag); tag = *epoch * tag_mul + tag_add),
  // merge query head h on split h % G % splits of its KV head and store its output as tagged
  // pairs in tout.
  const unsigned *epoch;
  const unsigned *wait_cnt;
  unsigned wait_per_step;
  unsigned *err;
  uint32_t *tws;
  uint32_t *tout;  // merged output as tagged pairs [Hq][D] (fused launch)
  unsigned tag_mul, tag_add;
};
constexpr int kMaxMergeSplits = 256;
// The attention kernels address a layer's K or V pool through one buffer resource with 32-bit
// byte offsets, so a pool must stay below 4 GiB.
inline bool kv_pool_fits(long long n_pages, int Hkv, int D, int kv_fmt) {
  const long long eb = kv_fmt == QDEC_KV_BF16 ? 2 : 4;
  return n_pages >= 1 && n_pages * Hkv * QDEC_PAGE_SIZE * D * eb < (1LL << 32);
}
// Error word values of the step handles: a bounded wait gave up, or the token being decoded has
// no cache slot (position < 0, past the page table, or an unmapped page-table entry).
constexpr unsigned kErrWait = 1u, kErrKvSlot = 2u;
constexpr size_t kAttnCounterBytes = 64 * 128;  // one line per KV head, up to 64 KV heads
size_t attn_workspace_bytes(int Hq, int D, int splits);
inline size_t attn_tagged_bytes(int Hq, int D, int splits) { return (size_t)splits * Hq * (2 * D + 4) * 4; }
hipError_t launch_attention(const AttnArgs &a, hipStream_t st);

// Append one token's k, v ([Hkv][D] fp32) into the pools at *pos.
hipError_t launch_kv_append(const float *k, const float *v, void *k_pool, void *v_pool, int kv_fmt,
                            const int32_t *page_table, int n_pages, const int32_t *pos, int Hkv,
                            int D, hipStream_t st);

// ---------------------------------------------------------------------------------- fused layer
// The attention half of a decoder layer as one launch (see layer.hip): nblk workgroups (one per
// compute unit) of attn_layer_waves() waves; wave w of workgroup b holds qkv unit b * waves + w
// and o unit (nblk - 1 - b) * waves + w, workgroup b < Hkv * splits attention unit (b / splits,
// b % splits).  The o units' runs (at most attn_layer_stash_runs()) are staged in LDS.
struct LayerArgs {
  GemvArgs qkv, o;
  AttnArgs at;
  int nblk;
  int o_waves;  // waves per workgroup holding o units (the last ones)
  unsigned long long *timeline;  // diagnostics: [nblk * waves][16] clock marks, or null
};
bool layer_fusion_supported(int G, int D);
int attn_layer_waves();
int attn_layer_o_waves();  // waves per workgroup that hold o GEMV units
int attn_layer_stash_runs();
int attn_layer_blocks_per_cu(int wfmt, int kv_fmt, int G);  // 0: the kernel does not fit a CU
hipError_t launch_attn_layer(const LayerArgs &a, int wfmt, hipStream_t st);

// ---------------------------------------------------------------------------------- small ops
// Per-head post-processing of a fused qkv vector: optional per-head RMSNorm of q and k, RoPE of
// q and k at *pos, then k and v stored into the pools (when k_pool != null).
struct QkvPostArgs {
  float *qkv;              // [(Hq + 2 Hkv) D], q and k rewritten in place
  const float *g_q, *g_k;  // [D] or null
  float eps;
  float rope_base;         // <= 0: no rotation
  const int32_t *pos;
  int Hq, Hkv, D;
  void *k_pool, *v_pool;   // null: no append
  int kv_fmt;
  const int32_t *page_table;
  int n_pages;
};
hipError_t launch_qkv_post(const QkvPostArgs &a, hipStream_t st);

hipError_t launch_rmsnorm_rope(const float *x, const float *gamma, float *y, int rows, int dim,
                               float eps, float rope_base, const int32_t *pos, hipStream_t st);
hipError_t launch_swiglu(const float *g, const float *u, float *m, int n, hipStream_t st);
// h = bf16 -> fp32 row E[*token] (E null: h is given), ssq[t] = sum of h^2 over rows 64t..64t+63.
// With rope_cs != null it also writes the RoPE table of *pos: rope_cs[2i], rope_cs[2i+1] =
// cos, sin of pos * base^(-2i/D) in fp64, i < D/2.  With epoch != null it advances the step
// number *epoch by one (the fused layer kernels' flag target).
hipError_t launch_embed(const uint16_t *E, const int32_t *token, int H, int V, float *h, float *ssq,
                        const int32_t *pos, float rope_base, int D, double *rope_cs, unsigned *epoch,
                        hipStream_t st);
// argmax over logits; writes *token, token_log[*step_count] (if log), advances *pos and
// *step_count.  With logits == null it only advances *pos.
hipError_t launch_argmax_finish(const float *logits, int n, int32_t *token, int32_t *pos,
                                int32_t *token_log, int32_t *step_count, int log_len,
                                hipStream_t st);
hipError_t launch_copy(const float *src, float *dst, int n, hipStream_t st);
// Bandwidth reference: reads bytes (a multiple of 16) at src once; *sink is written only in the
// unlikely case that the bytes' XOR is one fixed value.
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st);

}  // namespace qdec
