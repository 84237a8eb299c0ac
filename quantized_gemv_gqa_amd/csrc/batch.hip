// Batched decode step: up to 8 sequences advance by one token each in one pass over the weights.
//
// What it computes ("Chapter 2 Systems Foundations for LLMs": PagedAttention, Continuous
// Batching, Request Lifecycle): every running slot b (pos[b] >= 0) takes the single-sequence
// decode step with its own token, position and block table row, which maps its logical 16-token
// blocks to physical pages of one shared KV pool per layer; idle slots (pos[b] < 0) are left as
// they are.  The host owns the block tables, allocating a block on demand before the step that
// writes its first token, and may change any slot (a sequence finishing, another joining) between
// steps: everything a kernel needs is read from device memory, so one captured graph serves every
// step.
//
// How: per layer, skinny GEMM (RMSNorm folded in, qkv, bias) -> attention unit per (sequence, KV
// head, split) (q/k norm, RoPE, KV append and split-K attention, as in the single-sequence step) ->
// skinny GEMM (o, + residual) -> skinny GEMM (RMSNorm folded in, gate/up + SwiGLU) -> skinny GEMM
// (down, + residual); then the lm head (final RMSNorm folded in) and a per-row argmax.  Each
// weight byte is read once per step for all running sequences.  The RMSNorms cost no launch: the
// kernels that write the residual stream (the embedding, the o and down GEMMs) also write its sums
// of squares per 64-row tile, and the next GEMM normalises its activations while staging them.
#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "qdec_batch.h"

struct qdec_batch {
  qdec_config cfg;
  std::vector<qdec_layer_weights> layers;
  qdec_model model;
  std::vector<void *> kpools, vpools;
  qdec_batch_state state;
  int B = 0, nb_max = 0;
  float *ssq = nullptr, *qkv = nullptr, *attn = nullptr, *mlp = nullptr;
  double *rope_cs = nullptr;
  char *attn_ws = nullptr;
  size_t attn_ws_stride = 0;
  void *gemm_ws = nullptr;
  void *arg_ws = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipStream_t graph_stream = nullptr;
  int n_kernels = 0;
};

namespace qdec {
namespace {

size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

struct BLayout {
  size_t ssq, qkv, attn, mlp, rope_cs, attn_ws, attn_stride, gemm_ws, arg_ws, total;
};

BLayout blayout(const qdec_config &c, int B) {
  BLayout L{};
  const int nqkv = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim, qd = c.n_heads * c.head_dim;
  const int nbm = gemm_b_columns(B);
  size_t o = 0;
  L.ssq = o; o += al256((size_t)B * ((c.hidden + 63) / 64) * 4);
  L.qkv = o; o += al256((size_t)B * nqkv * 4);
  L.attn = o; o += al256((size_t)B * qd * 4);
  L.mlp = o; o += al256((size_t)B * c.inter * 4);
  L.rope_cs = o; o += al256((size_t)B * c.head_dim * 8);
  L.attn_stride = al256(attn_workspace_bytes(c.n_heads, c.head_dim, c.num_splits));
  L.attn_ws = o; o += (size_t)B * L.attn_stride;
  size_t g = gemm_b_workspace_bytes(c.wfmt, nqkv, c.hidden, nbm);
  g = std::max(g, gemm_b_workspace_bytes(c.wfmt, c.hidden, qd, nbm));
  g = std::max(g, gemm_b_workspace_bytes(c.wfmt, 2 * c.inter, c.hidden, nbm));
  g = std::max(g, gemm_b_workspace_bytes(c.wfmt, c.hidden, c.inter, nbm));
  g = std::max(g, gemm_b_workspace_bytes(c.wfmt, c.vocab, c.hidden, nbm));
  L.gemm_ws = o; o += al256(g);
  L.arg_ws = o; o += al256(argmax_rows_workspace_bytes(B));
  L.total = o;
  return L;
}

#define QDEC_BCK(expr)                                     \
  do {                                                     \
    hipError_t e_ = (expr);                                \
    if (e_ != hipSuccess) {                                \
      set_error("%s: %s", #expr, hipGetErrorString(e_));   \
      return QDEC_EHIP;                                    \
    }                                                      \
    ++n;                                                   \
  } while (0)

GemmBArgs gargs(const qdec_batch *h, const void *W, const void *S, const float *X, int ldx, float *Y, int ldy, int N,
                int K) {
  GemmBArgs g{};
  g.W = reinterpret_cast<const uint8_t *>(W);
  g.S = S;
  g.X = X;
  g.ldx = ldx;
  g.Y = Y;
  g.ldy = ldy;
  g.N = N;
  g.K = K;
  g.group = h->cfg.group;
  g.nb = h->B;
  g.nb_max = h->nb_max;
  g.epi = EPI_STORE;
  g.pos = h->state.pos;
  return g;
}

qdec_status enqueue_batch(qdec_batch *h, hipStream_t st, int *count) {
  const qdec_config &c = h->cfg;
  const qdec_batch_state &s = h->state;
  const int B = h->B, H = c.hidden, Hq = c.n_heads, Hkv = c.n_kv_heads, D = c.head_dim, I = c.inter, V = c.vocab;
  const int nqkv = (Hq + 2 * Hkv) * D, qd = Hq * D;
  const int wf = c.wfmt;
  int n = 0;
  // the residual stream's per-tile sums of squares: written by each kernel that writes s.hidden,
  // read by the next GEMM, which normalises while staging
  const auto normed = [&](GemmBArgs &g, const float *gamma) {
    g.gamma = gamma;
    g.ssq = h->ssq;
    g.ssq_n = (H + 63) / 64;
    g.eps = c.rms_eps;
  };
  QDEC_BCK(launch_embed_rows(h->model.embed, s.tokens, s.pos, B, H, V, s.hidden, h->ssq, c.rope_base, D, h->rope_cs,
                             st));
  for (int l = 0; l < c.n_layers; ++l) {
    const qdec_layer_weights &w = h->layers[l];
    GemmBArgs q = gargs(h, w.w_qkv, w.s_qkv, s.hidden, H, h->qkv, nqkv, nqkv, H);
    normed(q, w.g_attn);
    q.bias = c.has_qkv_bias ? w.b_qkv : nullptr;
    QDEC_BCK(launch_gemm_b(wf, q, h->gemm_ws, st));
    AttnBatch ab{};
    ab.a.g_q = c.has_qk_norm ? w.g_q : nullptr;
    ab.a.g_k = c.has_qk_norm ? w.g_k : nullptr;
    ab.a.eps = c.rms_eps;
    ab.a.k_pool = h->kpools[l];
    ab.a.v_pool = h->vpools[l];
    ab.a.kv_fmt = c.kv_fmt;
    ab.a.n_pages = c.n_pages;
    ab.a.Hq = Hq;
    ab.a.Hkv = Hkv;
    ab.a.D = D;
    ab.a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
    ab.a.splits = c.num_splits;
    ab.qkv = h->qkv;
    ab.rope_cs = h->rope_cs;
    ab.pos = s.pos;
    ab.tables = s.block_tables;
    ab.max_blocks = s.max_blocks;
    ab.ws = h->attn_ws;
    ab.ws_stride = h->attn_ws_stride;
    ab.out = h->attn;
    ab.B = B;
    QDEC_BCK(launch_attention_batch(ab, st));
    GemmBArgs o = gargs(h, w.w_o, w.s_o, h->attn, qd, s.hidden, H, H, qd);
    o.residual = s.hidden;
    o.ssq_out = h->ssq;
    QDEC_BCK(launch_gemm_b(wf, o, h->gemm_ws, st));
    GemmBArgs g = gargs(h, w.w_gu, w.s_gu, s.hidden, H, h->mlp, I, 2 * I, H);
    normed(g, w.g_ffn);
    g.epi = EPI_SWIGLU;
    QDEC_BCK(launch_gemm_b(wf, g, h->gemm_ws, st));
    GemmBArgs d = gargs(h, w.w_down, w.s_down, h->mlp, I, s.hidden, H, H, I);
    d.residual = s.hidden;
    d.ssq_out = h->ssq;
    QDEC_BCK(launch_gemm_b(wf, d, h->gemm_ws, st));
  }
  GemmBArgs lm = gargs(h, h->model.w_lm, h->model.s_lm, s.hidden, H, s.logits, V, V, H);
  normed(lm, h->model.g_out);
  QDEC_BCK(launch_gemm_b(wf, lm, h->gemm_ws, st));
  QDEC_BCK(launch_argmax_rows(s.logits, B, V, s.tokens, s.pos, h->arg_ws, st));
  ++n;  // (two launches)
  if (count) *count = n;
  return QDEC_OK;
}

qdec_status validate_batch(const qdec_config *c, int B) {
  QDEC_REQUIRE(c, QDEC_EINVAL, "qdec_batch: null config");
  QDEC_REQUIRE(B >= 1 && B <= 8, QDEC_EUNSUPPORTED, "qdec_batch: max_batch must be in [1, 8] (got %d)", B);
  QDEC_REQUIRE(c->n_layers >= 1 && c->hidden >= 16 && c->n_heads >= 1 && c->n_kv_heads >= 1 && c->inter >= 32 &&
                   c->vocab >= 1,
               QDEC_EINVAL, "qdec_batch: bad model sizes");
  QDEC_REQUIRE(c->n_heads % c->n_kv_heads == 0 && c->n_heads / c->n_kv_heads <= 8, QDEC_EUNSUPPORTED,
               "qdec_batch: need n_heads a multiple of n_kv_heads with at most 8 q heads per kv head");
  QDEC_REQUIRE(c->head_dim == 64 || c->head_dim == 128, QDEC_EUNSUPPORTED, "qdec_batch: head_dim must be 64 or 128");
  QDEC_REQUIRE(c->wfmt == QDEC_W_Q8_ROW || c->wfmt == QDEC_W_Q4_G_ZP8, QDEC_EUNSUPPORTED,
               "qdec_batch: unknown weight format %d", c->wfmt);
  QDEC_REQUIRE(c->kv_fmt == QDEC_KV_F32 || c->kv_fmt == QDEC_KV_BF16, QDEC_EUNSUPPORTED,
               "qdec_batch: unknown kv format %d", c->kv_fmt);
  QDEC_REQUIRE(c->page_size == QDEC_PAGE_SIZE && c->n_pages >= 1, QDEC_EUNSUPPORTED,
               "qdec_batch: page_size must be 16 and n_pages >= 1");
  QDEC_REQUIRE(kv_pool_fits(c->n_pages, c->n_kv_heads, c->head_dim, c->kv_fmt), QDEC_EUNSUPPORTED,
               "qdec_batch: a layer's KV pool (%d pages) must stay below 4 GiB", c->n_pages);
  QDEC_REQUIRE(c->num_splits >= 1 && c->num_splits <= kMaxMergeSplits, QDEC_EINVAL, "qdec_batch: num_splits in [1, %d]",
               kMaxMergeSplits);
  QDEC_REQUIRE(c->n_kv_heads <= (int)(kAttnCounterBytes / 128), QDEC_EUNSUPPORTED, "qdec_batch: too many KV heads");
  QDEC_REQUIRE(c->inter % 32 == 0, QDEC_EUNSUPPORTED, "qdec_batch: inter must be a multiple of 32");
  QDEC_REQUIRE(c->hidden % 4 == 0 && c->hidden <= 16384, QDEC_EUNSUPPORTED,
               "qdec_batch: hidden must be a multiple of 4, at most 16384");
  const int qd = c->n_heads * c->head_dim;
  if (c->wfmt == QDEC_W_Q8_ROW) {
    QDEC_REQUIRE(c->hidden % 16 == 0 && qd % 16 == 0 && c->inter % 16 == 0, QDEC_EINVAL,
                 "qdec_batch: Q8 needs hidden, n_heads*head_dim, inter multiples of 16");
  } else {
    QDEC_REQUIRE(c->group >= 32 && c->group <= 4096 && (c->group & (c->group - 1)) == 0, QDEC_EUNSUPPORTED,
                 "qdec_batch: bad Q4 group");
    QDEC_REQUIRE(c->hidden % c->group == 0 && qd % c->group == 0 && c->inter % c->group == 0, QDEC_EINVAL,
                 "qdec_batch: Q4 needs hidden, n_heads*head_dim, inter multiples of group");
  }
  QDEC_REQUIRE(std::isfinite(c->rms_eps) && c->rms_eps >= 0.f && c->rope_base > 0.f, QDEC_EINVAL,
               "qdec_batch: bad eps / rope_base");
  return QDEC_OK;
}

}  // namespace
}  // namespace qdec

using namespace qdec;

extern "C" {

size_t qdec_batch_workspace_bytes(const qdec_config *cfg, int max_batch) {
  if (validate_batch(cfg, max_batch) != QDEC_OK) return 0;
  return blayout(*cfg, max_batch).total;
}

qdec_status qdec_batch_create(const qdec_config *cfg, const qdec_model *m, const qdec_batch_state *s, qdec_batch **out) {
  QDEC_REQUIRE(s && m && out && m->layers, QDEC_EINVAL, "qdec_batch_create: null argument");
  qdec_status r = validate_batch(cfg, s->max_batch);
  if (r != QDEC_OK) return r;
  QDEC_REQUIRE(m->embed && m->w_lm && m->s_lm && m->g_out, QDEC_EINVAL,
               "qdec_batch_create: the batched step needs the embedding and the lm head");
  QDEC_REQUIRE(s->k_pools && s->v_pools && s->block_tables && s->pos && s->tokens && s->hidden && s->logits &&
                   s->workspace,
               QDEC_EINVAL, "qdec_batch_create: state is missing a buffer");
  QDEC_REQUIRE(s->max_blocks >= 1 && s->max_blocks <= cfg->n_pages, QDEC_EINVAL,
               "qdec_batch_create: max_blocks must be in [1, n_pages] (got %d)", s->max_blocks);
  const BLayout L = blayout(*cfg, s->max_batch);
  QDEC_REQUIRE(s->workspace_bytes >= L.total, QDEC_EINVAL, "qdec_batch_create: workspace too small (%zu < %zu bytes)",
               s->workspace_bytes, L.total);
  QDEC_REQUIRE((reinterpret_cast<uintptr_t>(s->workspace) % 256) == 0, QDEC_EINVAL,
               "qdec_batch_create: workspace must be 256-byte aligned");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const qdec_layer_weights &w = m->layers[l];
    QDEC_REQUIRE(w.w_qkv && w.s_qkv && w.w_o && w.s_o && w.w_gu && w.s_gu && w.w_down && w.s_down && w.g_attn && w.g_ffn,
                 QDEC_EINVAL, "qdec_batch_create: layer %d is missing a weight", l);
    QDEC_REQUIRE(!cfg->has_qkv_bias || w.b_qkv, QDEC_EINVAL, "qdec_batch_create: layer %d has no qkv bias", l);
    QDEC_REQUIRE(!cfg->has_qk_norm || (w.g_q && w.g_k), QDEC_EINVAL, "qdec_batch_create: layer %d has no q/k norm gains",
                 l);
    QDEC_REQUIRE(s->k_pools[l] && s->v_pools[l], QDEC_EINVAL, "qdec_batch_create: layer %d has no KV pool", l);
  }
  qdec_batch *h = new qdec_batch();
  h->cfg = *cfg;
  h->layers.assign(m->layers, m->layers + cfg->n_layers);
  h->model = *m;
  h->model.layers = h->layers.data();
  h->kpools.assign(s->k_pools, s->k_pools + cfg->n_layers);
  h->vpools.assign(s->v_pools, s->v_pools + cfg->n_layers);
  h->state = *s;
  h->state.k_pools = h->kpools.data();
  h->state.v_pools = h->vpools.data();
  h->B = s->max_batch;
  h->nb_max = gemm_b_columns(h->B);
  char *ws = reinterpret_cast<char *>(s->workspace);
  h->ssq = reinterpret_cast<float *>(ws + L.ssq);
  h->qkv = reinterpret_cast<float *>(ws + L.qkv);
  h->attn = reinterpret_cast<float *>(ws + L.attn);
  h->mlp = reinterpret_cast<float *>(ws + L.mlp);
  h->rope_cs = reinterpret_cast<double *>(ws + L.rope_cs);
  h->attn_ws = ws + L.attn_ws;
  h->attn_ws_stride = L.attn_stride;
  h->gemm_ws = ws + L.gemm_ws;
  h->arg_ws = ws + L.arg_ws;
  *out = h;
  return QDEC_OK;
}

qdec_status qdec_batch_decode_step(qdec_batch *h, int mode, void *stream) {
  QDEC_REQUIRE(h, QDEC_EINVAL, "qdec_batch_decode_step: null handle");
  hipStream_t st = (hipStream_t)stream;
  if (mode == QDEC_STEP_EAGER) return enqueue_batch(h, st, &h->n_kernels);
  QDEC_REQUIRE(mode == QDEC_STEP_GRAPH, QDEC_EINVAL, "qdec_batch_decode_step: mode must be EAGER or GRAPH (got %d)", mode);
  if (!h->exec) {
    QDEC_REQUIRE(st != nullptr, QDEC_ESTATE, "qdec_batch_decode_step: graph capture needs a non-default stream");
    hipError_t e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
      set_error("hipStreamBeginCapture: %s", hipGetErrorString(e));
      return QDEC_EHIP;
    }
    int nk = 0;
    qdec_status r = enqueue_batch(h, st, &nk);
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(st, &g);
    if (r != QDEC_OK) {
      if (g) (void)hipGraphDestroy(g);
      return r;
    }
    if (e != hipSuccess) {
      set_error("hipStreamEndCapture: %s", hipGetErrorString(e));
      return QDEC_EHIP;
    }
    e = hipGraphInstantiate(&h->exec, g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      (void)hipGraphDestroy(g);
      set_error("hipGraphInstantiate: %s", hipGetErrorString(e));
      return QDEC_EHIP;
    }
    h->graph = g;
    h->graph_stream = st;
    h->n_kernels = nk;
  }
  QDEC_REQUIRE(st == h->graph_stream, QDEC_ESTATE, "qdec_batch_decode_step: graph was captured on another stream");
  hipError_t e = hipGraphLaunch(h->exec, st);
  if (e != hipSuccess) {
    set_error("hipGraphLaunch: %s", hipGetErrorString(e));
    return QDEC_EHIP;
  }
  return QDEC_OK;
}

int qdec_batch_kernel_count(const qdec_batch *h) { return h ? h->n_kernels : 0; }

void qdec_batch_destroy(qdec_batch *h) {
  if (!h) return;
  if (h->exec) (void)hipGraphExecDestroy(h->exec);
  if (h->graph) (void)hipGraphDestroy(h->graph);
  delete h;
}

}  // extern "C"
