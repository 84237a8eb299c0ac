// One batch-1 decode step of a Qwen-style GQA decoder as a fixed list of kernel launches, run
// eagerly or captured once into a hipGraph and replayed.
//
// Every per-step scalar the kernels need (token id, position, step count) lives in device memory
// and is read by the kernels themselves, so one captured graph stays valid as the context grows
// and across page boundaries (FlashQwen README, "Optimization study", stage 6: a single graph
// whose kernels read token id / position from device buffers; the H100 runtime instead captured
// two graphs and patched scalars before each launch, "How To Construct Your Personal LLM Runtime
// From Scratch", section 6).  Region order per layer follows that post's ITL breakdown:
// qkv_gemv -> append_tail_kv (with RoPE) -> paged_attention -> o_proj -> gate_up_gemv ->
// swiglu_down.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "qdec_batch.h"

struct qdec_step {
  qdec_config cfg;
  std::vector<qdec_layer_weights> layers;
  qdec_model model;
  std::vector<void *> kpools, vpools;
  qdec_state state;
  // workspace carve-up
  float *qkv = nullptr, *attn = nullptr, *mlp = nullptr, *ssq = nullptr, *attn_ws = nullptr;
  uint32_t *attn_tws = nullptr;   // the fused launch's tagged split partials
  uint32_t *attn_tout = nullptr;  // and its tagged merged attention output
  double *rope_cs = nullptr;  // this step's RoPE (cos, sin) table, written by the embed kernel
  // fused attention kernel (three launches per layer)
  bool layer_ok = false;
  float *hB = nullptr, *ssqB = nullptr;  // second residual buffer and its per-tile sums of squares
  void *gemv_ws2 = nullptr;              // GEMV workspace of the roles that run beside the first
  unsigned *lsync = nullptr;             // [0]: step number; then per layer: qkv counts, attention flags
  size_t lsync_layer_words = 0;
  void *gemv_ws = nullptr;
  qdec::GemvPlan p_qkv, p_o, p_gu, p_down, p_lm;
  int nblk = 0;    // workgroups of the fused attention launch (one per compute unit)
  int o_waves = 0;  // its waves per workgroup that hold o units
  unsigned long long *timeline = nullptr;  // diagnostics: per-wave clock marks of the fused launches
  unsigned long long *mlp_timeline = nullptr;  // diagnostics: per-unit clock marks of gate/up and down
  int splits = 1;  // attention splits per KV head in use (the config's, capped for the fused launch)
  int ssq_n = 0;
  hipGraph_t graph[2] = {nullptr, nullptr};      // [per-op]: captured step
  hipGraphExec_t exec[2] = {nullptr, nullptr};
  hipStream_t graph_stream[2] = {nullptr, nullptr};
  int graph_kernels[2] = {0, 0};
  int n_kernels = 0;
  // sampling of the next token (temperature > 0) instead of the greedy argmax
  float temperature = 0.f, top_p = 1.f;
  int top_k = 0;
  uint64_t seed = 0;
  void *sample_ws = nullptr;
  unsigned *err = nullptr;
  // per-kernel timing of one eager step (qdec_step_kernel_times): an event after every launch
  std::vector<hipEvent_t> tev;
  size_t tev_n = 0;
  bool timing = false;
};

namespace qdec {
namespace {

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct Layout {
  size_t qkv, attn, mlp, ssq, attn_ws, attn_tws, attn_tout, rope_cs, gemv_ws, gemv_ws2, lsync, err, sample_ws, hB, ssqB, total;
};

// The fused attention launch has one workgroup per compute unit, at most this many (the GEMV
// workspaces hold one split-K partial tile per wave of that grid).
constexpr int kMaxLayerBlocks = 512;

// GEMV plan of the fused attention launch: the fewest runs per unit, at least one pipeline batch
// (or the whole row), such that every unit has a wave of the grid; an o unit's runs must also fit
// the LDS stash (max_cps).  units == 0: no split fits.
GemvPlan layer_plan(int wfmt, int N, int K, int waves, int max_cps) {
  GemvPlan p{};
  const int ck = (wfmt == QDEC_W_Q4_G_ZP8) ? 32 : 16;
  p.tiles = (N + kTile - 1) / kTile;
  p.nch = K / ck;
  for (int cps = std::min(4, p.nch); cps <= std::min(max_cps, p.nch); ++cps) {
    const int ks = (p.nch + cps - 1) / cps;
    if ((long)p.tiles * ks > waves) continue;
    p.cps = (p.nch + ks - 1) / ks;
    p.ks = (p.nch + p.cps - 1) / p.cps;
    p.units = p.tiles * p.ks;
    gemv_set_grid(p);
    return p;
  }
  p.units = 0;
  return p;
}

// Per layer: the qkv tile counts (one 128-byte line per KV head).
size_t lsync_layer_words(int Hkv) { return (size_t)Hkv * kLine; }

Layout layout_of(const qdec_config &c) {
  Layout L{};
  const int nqkv = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const int qd = c.n_heads * c.head_dim;
  size_t off = 0;
  L.qkv = off; off += align256((size_t)nqkv * 4);
  L.attn = off; off += align256((size_t)qd * 4);
  L.mlp = off; off += align256((size_t)c.inter * 4);
  L.ssq = off; off += align256((size_t)((c.hidden + 63) / 64) * 4);
  L.attn_ws = off; off += align256(attn_workspace_bytes(c.n_heads, c.head_dim, c.num_splits));
  L.attn_tws = off; off += align256(attn_tagged_bytes(c.n_heads, c.head_dim, c.num_splits));
  L.attn_tout = off; off += align256((size_t)c.n_heads * c.head_dim * 8);
  L.rope_cs = off; off += align256((size_t)c.head_dim * sizeof(double));
  size_t g = gemv_workspace_bytes(c.wfmt, nqkv, c.hidden);
  g = std::max(g, gemv_workspace_bytes(c.wfmt, c.hidden, qd));
  g = std::max(g, gemv_workspace_bytes(c.wfmt, 2 * c.inter, c.hidden));
  g = std::max(g, gemv_workspace_bytes(c.wfmt, c.hidden, c.inter));
  if (c.vocab > 0) g = std::max(g, gemv_workspace_bytes(c.wfmt, c.vocab, c.hidden, true));
  g = std::max(g, kCounterBytes + (size_t)kMaxLayerBlocks * attn_layer_waves() * kTile * sizeof(float));
  L.gemv_ws = off; off += align256(g);
  L.gemv_ws2 = off; off += align256(g);
  L.lsync = off; off += align256((32 + (size_t)c.n_layers * lsync_layer_words(c.n_kv_heads)) * 4);
  L.err = off; off += 256;
  L.sample_ws = off; off += align256(sample_workspace_bytes());
  L.hB = off; off += align256((size_t)c.hidden * 4);
  L.ssqB = off; off += align256(std::max<size_t>(256, (size_t)((c.hidden + 63) / 64) * 4));
  L.total = off;
  return L;
}

qdec_status validate(const qdec_config *c) {
  QDEC_REQUIRE(c, QDEC_EINVAL, "qdec_step: null config");
  QDEC_REQUIRE(c->n_layers >= 1 && c->hidden >= 16 && c->n_heads >= 1 && c->n_kv_heads >= 1 &&
                   c->inter >= 32 && c->vocab >= 0,
               QDEC_EINVAL, "qdec_step: bad model sizes");
  QDEC_REQUIRE(c->n_heads % c->n_kv_heads == 0 && c->n_heads / c->n_kv_heads <= 8, QDEC_EUNSUPPORTED,
               "qdec_step: need n_heads a multiple of n_kv_heads with at most 8 q heads per kv head");
  QDEC_REQUIRE(c->head_dim == 64 || c->head_dim == 128, QDEC_EUNSUPPORTED,
               "qdec_step: head_dim must be 64 or 128");
  QDEC_REQUIRE(c->wfmt == QDEC_W_Q8_ROW || c->wfmt == QDEC_W_Q4_G_ZP8, QDEC_EUNSUPPORTED,
               "qdec_step: unknown weight format %d", c->wfmt);
  QDEC_REQUIRE(c->kv_fmt == QDEC_KV_F32 || c->kv_fmt == QDEC_KV_BF16, QDEC_EUNSUPPORTED,
               "qdec_step: unknown kv format %d", c->kv_fmt);
  QDEC_REQUIRE(c->page_size == QDEC_PAGE_SIZE && c->n_pages >= 1, QDEC_EUNSUPPORTED,
               "qdec_step: page_size must be 16 and n_pages >= 1");
  QDEC_REQUIRE(kv_pool_fits(c->n_pages, c->n_kv_heads, c->head_dim, c->kv_fmt), QDEC_EUNSUPPORTED,
               "qdec_step: a layer's KV pool (%d pages) must stay below 4 GiB", c->n_pages);
  QDEC_REQUIRE(c->num_splits >= 1 && c->num_splits <= kMaxMergeSplits, QDEC_EINVAL,
               "qdec_step: num_splits in [1, %d]", kMaxMergeSplits);
  QDEC_REQUIRE(c->n_kv_heads <= (int)(kAttnCounterBytes / 128), QDEC_EUNSUPPORTED, "qdec_step: too many KV heads");
  QDEC_REQUIRE(c->inter % 32 == 0, QDEC_EUNSUPPORTED, "qdec_step: inter must be a multiple of 32");
  const int qd = c->n_heads * c->head_dim;
  if (c->wfmt == QDEC_W_Q8_ROW) {
    QDEC_REQUIRE(c->hidden % 16 == 0 && qd % 16 == 0 && c->inter % 16 == 0, QDEC_EINVAL,
                 "qdec_step: Q8 needs hidden, n_heads*head_dim, inter multiples of 16");
  } else {
    QDEC_REQUIRE(c->group >= 32 && c->group <= 4096 && (c->group & (c->group - 1)) == 0, QDEC_EUNSUPPORTED, "qdec_step: bad Q4 group");
    QDEC_REQUIRE(c->hidden % c->group == 0 && qd % c->group == 0 && c->inter % c->group == 0,
                 QDEC_EINVAL, "qdec_step: Q4 needs hidden, n_heads*head_dim, inter multiples of group");
  }
  QDEC_REQUIRE(std::isfinite(c->rms_eps) && c->rms_eps >= 0.f && c->rope_base > 0.f, QDEC_EINVAL,
               "qdec_step: bad eps / rope_base");
  return QDEC_OK;
}

GemvArgs gemv_args(const qdec_step *h, const void *W, const void *S, const float *x, float *y, int N,
                   int K, const GemvPlan &p) {
  GemvArgs a{};
  a.W = reinterpret_cast<const uint8_t *>(W);
  a.S = S;
  a.x = x;
  a.y = y;
  a.N = N;
  a.K = K;
  a.group = h->cfg.group;
  a.eps = h->cfg.rms_eps;
  a.ssq = h->ssq;
  a.ssq_n = h->ssq_n;
  a.epi = EPI_STORE;
  gemv_bind_workspace(a, p, h->gemv_ws);
  return a;
}

// The MLP timeline records of layer l: gate/up units, then down units, 8 marks each.
unsigned long long *mlp_rec(const qdec_step *h, int l, bool down) {
  if (!h->mlp_timeline) return nullptr;
  const size_t per_layer = (size_t)(h->p_gu.units + h->p_down.units) * 8;
  return h->mlp_timeline + l * per_layer + (down ? (size_t)h->p_gu.units * 8 : 0);
}

// Captured graphs hold the launch list with its arguments: a change of those drops them (the
// next GRAPH call captures again).
void drop_graphs(qdec_step *h) {
  for (int v = 0; v < 2; ++v) {
    if (h->exec[v]) (void)hipGraphExecDestroy(h->exec[v]);
    if (h->graph[v]) (void)hipGraphDestroy(h->graph[v]);
    h->exec[v] = nullptr;
    h->graph[v] = nullptr;
    h->graph_stream[v] = nullptr;
  }
}

// Records the next timing event after a launch while qdec_step_kernel_times runs a step.
void step_mark(qdec_step *h, hipStream_t st) {
  if (h->timing && h->tev_n < h->tev.size()) (void)hipEventRecord(h->tev[h->tev_n++], st);
}

#define QDEC_CK(expr)                                      \
  do {                                                     \
    hipError_t e_ = (expr);                                \
    if (e_ != hipSuccess) {                                \
      set_error("%s: %s", #expr, hipGetErrorString(e_));   \
      return QDEC_EHIP;                                    \
    }                                                      \
    ++n;                                                   \
    step_mark(h, st);                                      \
  } while (0)

AttnArgs step_attn_args(const qdec_step *h, int l) {
  const qdec_config &c = h->cfg;
  const qdec_state &s = h->state;
  const qdec_layer_weights &w = h->layers[l];
  AttnArgs at{};
  at.qkv = h->qkv;
  at.g_q = c.has_qk_norm ? w.g_q : nullptr;
  at.g_k = c.has_qk_norm ? w.g_k : nullptr;
  at.eps = c.rms_eps;
  at.rope_cs = h->rope_cs;
  at.k_pool = h->kpools[l];
  at.v_pool = h->vpools[l];
  at.kv_fmt = c.kv_fmt;
  at.page_table = s.page_table;
  at.n_pages = c.n_pages;
  at.pos = s.pos;
  at.Hq = c.n_heads;
  at.Hkv = c.n_kv_heads;
  at.D = c.head_dim;
  at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
  at.splits = h->splits;
  at.counters = reinterpret_cast<unsigned *>(h->attn_ws);
  at.ws = reinterpret_cast<float *>(reinterpret_cast<char *>(h->attn_ws) + kAttnCounterBytes);
  at.out = h->attn;
  return at;
}

// One layer as the attention kernel (qkv GEMV, attention, o GEMV), then the gate/up and down
// GEMVs.  Residual stream: hA = state.hidden (read by qkv and o's residual, written by down), hB
// (written by o, read by gate/up and down's residual), each with its own sums of squares.
hipError_t enqueue_layer(qdec_step *h, int l, hipStream_t st) {
  const qdec_config &c = h->cfg;
  const qdec_state &s = h->state;
  const qdec_layer_weights &w = h->layers[l];
  const int H = c.hidden, Hq = c.n_heads, Hkv = c.n_kv_heads, D = c.head_dim, I = c.inter, G = Hq / Hkv;
  const int qd = Hq * D, nqkv = (Hq + 2 * Hkv) * D;
  unsigned *const epoch = h->lsync;
  unsigned *const ls = h->lsync + 32 + (size_t)l * h->lsync_layer_words;
  unsigned *const qkv_cnt = ls;                            // [Hkv lines]
  float *const hA = s.hidden;
  LayerArgs la{};
  la.qkv = gemv_args(h, w.w_qkv, w.s_qkv, hA, h->qkv, nqkv, H, h->p_qkv);
  la.qkv.gamma = w.g_attn;
  la.qkv.bias = c.has_qkv_bias ? w.b_qkv : nullptr;
  la.qkv.epoch = epoch;
  la.qkv.done = qkv_cnt;
  la.qkv.Hq = Hq;
  la.qkv.Hkv = Hkv;
  la.qkv.hd = D;
  la.qkv.err = h->err;
  la.at = step_attn_args(h, l);
  la.at.epoch = epoch;
  la.at.wait_cnt = qkv_cnt;
  la.at.wait_per_step = (unsigned)((G + 2) * (D / kTile));
  la.at.err = h->err;
  la.at.tws = h->attn_tws;
  la.at.tout = h->attn_tout;
  la.at.tag_mul = (unsigned)c.n_layers;
  la.at.tag_add = (unsigned)l;
  la.o = gemv_args(h, w.w_o, w.s_o, h->attn, h->hB, H, qd, h->p_o);
  gemv_bind_workspace(la.o, h->p_o, h->gemv_ws2);
  la.o.residual = hA;
  la.o.ssq_out = h->ssqB;
  la.o.epoch = epoch;
  la.o.xt = h->attn_tout;  // the merged attention output, tagged like the split partials
  la.o.xt_tag_mul = (unsigned)c.n_layers;
  la.o.xt_tag_add = (unsigned)l;
  la.o.err = h->err;
  gemv_apply_plan(la.qkv, h->p_qkv, c.wfmt);
  gemv_apply_plan(la.o, h->p_o, c.wfmt);
  la.nblk = h->nblk;
  la.o_waves = h->o_waves;
  la.timeline = h->timeline ? h->timeline + (size_t)l * h->nblk * attn_layer_waves() * 16 : nullptr;
  hipError_t e = launch_attn_layer(la, c.wfmt, st);
  if (e != hipSuccess) return e;
  step_mark(h, st);
  // the MLP block as two plain launches: its gate/up tiles all finish together, so a down GEMV
  // in the same launch could only wait for them
  GemvArgs g = gemv_args(h, w.w_gu, w.s_gu, h->hB, h->mlp, 2 * I, H, h->p_gu);
  g.gamma = w.g_ffn;
  g.ssq = h->ssqB;
  g.epi = EPI_SWIGLU;
  g.timeline = mlp_rec(h, l, false);
  e = launch_gemv(c.wfmt, g, h->p_gu, st);
  if (e != hipSuccess) return e;
  step_mark(h, st);
  GemvArgs d = gemv_args(h, w.w_down, w.s_down, h->mlp, hA, H, I, h->p_down);
  d.residual = h->hB;
  d.ssq_out = h->ssq;
  d.timeline = mlp_rec(h, l, true);
  return launch_gemv(c.wfmt, d, h->p_down, st);
}

// Enqueue one whole step; returns the number of kernels launched through `count`.  Unless
// per_op is set (or the model's shape has no fused layer kernels), each layer is two launches.
qdec_status enqueue_step(qdec_step *h, hipStream_t st, int *count, bool per_op) {
  const qdec_config &c = h->cfg;
  const qdec_state &s = h->state;
  const int H = c.hidden, Hq = c.n_heads, Hkv = c.n_kv_heads, D = c.head_dim, I = c.inter;
  const int qd = Hq * D, nqkv = (Hq + 2 * Hkv) * D;
  const int wf = c.wfmt;
  int n = 0;
  const bool fuse = h->layer_ok && !per_op;
  QDEC_CK(launch_embed(h->model.embed, s.token, H, c.vocab, s.hidden, h->ssq, s.pos, c.rope_base, D, h->rope_cs,
                       fuse ? h->lsync : nullptr, st));
  if (s.trace) QDEC_CK(launch_copy(s.hidden, s.trace, H, st));
  for (int l = 0; l < c.n_layers; ++l) {
    const qdec_layer_weights &w = h->layers[l];
    if (fuse) {
      QDEC_CK(enqueue_layer(h, l, st));
      n += 2;  // three launches
      if (s.trace) QDEC_CK(launch_copy(s.hidden, s.trace + (size_t)(l + 1) * H, H, st));
      continue;
    }
    // attention block
    GemvArgs a = gemv_args(h, w.w_qkv, w.s_qkv, s.hidden, h->qkv, nqkv, H, h->p_qkv);
    a.gamma = w.g_attn;
    a.bias = c.has_qkv_bias ? w.b_qkv : nullptr;
    QDEC_CK(launch_gemv(wf, a, h->p_qkv, st));
    // attention takes q, k, v raw: it applies the q/k norm and RoPE and appends k, v itself
    AttnArgs at{};
    at.qkv = h->qkv;
    at.g_q = c.has_qk_norm ? w.g_q : nullptr;
    at.g_k = c.has_qk_norm ? w.g_k : nullptr;
    at.eps = c.rms_eps;
    at.rope_cs = h->rope_cs;
    at.k_pool = h->kpools[l];
    at.v_pool = h->vpools[l];
    at.kv_fmt = c.kv_fmt;
    at.page_table = s.page_table;
    at.n_pages = c.n_pages;
    at.pos = s.pos;
    at.Hq = Hq;
    at.Hkv = Hkv;
    at.D = D;
    at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
    at.splits = h->splits;
    at.counters = reinterpret_cast<unsigned *>(h->attn_ws);
    at.ws = reinterpret_cast<float *>(reinterpret_cast<char *>(h->attn_ws) + kAttnCounterBytes);
    at.out = h->attn;
    at.err = h->err;
    QDEC_CK(launch_attention(at, st));
    GemvArgs o = gemv_args(h, w.w_o, w.s_o, h->attn, s.hidden, H, qd, h->p_o);
    o.residual = s.hidden;
    o.ssq_out = h->ssq;
    QDEC_CK(launch_gemv(wf, o, h->p_o, st));
    // MLP block
    GemvArgs g = gemv_args(h, w.w_gu, w.s_gu, s.hidden, h->mlp, 2 * I, H, h->p_gu);
    g.gamma = w.g_ffn;
    g.epi = EPI_SWIGLU;
    g.timeline = mlp_rec(h, l, false);
    QDEC_CK(launch_gemv(wf, g, h->p_gu, st));
    GemvArgs d = gemv_args(h, w.w_down, w.s_down, h->mlp, s.hidden, H, I, h->p_down);
    d.residual = s.hidden;
    d.ssq_out = h->ssq;
    d.timeline = mlp_rec(h, l, true);
    QDEC_CK(launch_gemv(wf, d, h->p_down, st));
    if (s.trace) QDEC_CK(launch_copy(s.hidden, s.trace + (size_t)(l + 1) * H, H, st));
  }
  if (h->model.w_lm && h->temperature > 0.f) {
    // lm head storing the logits, then the sampler (draw counter: the step count), which writes
    // the token and advances the step scalars
    GemvArgs a = gemv_args(h, h->model.w_lm, h->model.s_lm, s.hidden, s.logits, c.vocab, H, h->p_lm);
    a.gamma = h->model.g_out;
    a.epi = EPI_STORE;
    QDEC_CK(launch_gemv(wf, a, h->p_lm, st));
    QDEC_CK(launch_sample(s.logits, c.vocab, h->temperature, h->top_k, h->top_p, h->seed, s.step_count, s.token,
                          s.token_log, s.step_count, s.pos, s.log_len, h->sample_ws, st));
    ++n;  // (two launches)
  } else if (h->model.w_lm) {
    // lm head with the greedy argmax, token write and position advance fused in its epilogue
    GemvArgs a = gemv_args(h, h->model.w_lm, h->model.s_lm, s.hidden, s.logits, c.vocab, H, h->p_lm);
    a.gamma = h->model.g_out;
    a.epi = EPI_ARGMAX;
    a.token = s.token;
    a.pos = s.pos;
    a.token_log = s.token_log;
    a.step_count = s.step_count;
    a.log_len = s.log_len;
    QDEC_CK(launch_gemv(wf, a, h->p_lm, st));
  } else {
    QDEC_CK(launch_argmax_finish(nullptr, 0, nullptr, s.pos, nullptr, s.step_count, 0, st));
  }
  if (count) *count = n;
  return QDEC_OK;
}

// ------------------------------------------------------------------ prefill
struct PLayout {
  size_t x32, a16, a16l, qkv, att, att16, att16l, mlp16, mlp16l, pos_rows, attn_ws, attn_stride, a_last, part, total;
};

PLayout playout(const qdec_config &c, int T) {
  PLayout L{};
  const int nqkv = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim, qd = c.n_heads * c.head_dim;
  size_t o = 0;
  L.x32 = o; o += align256((size_t)T * c.hidden * 4);
  L.a16 = o; o += align256((size_t)T * c.hidden * 2);
  L.a16l = o; o += align256((size_t)T * c.hidden * 2);
  L.qkv = o; o += align256((size_t)T * nqkv * 4);
  L.att = o; o += align256((size_t)T * qd * 4);
  L.att16 = o; o += align256((size_t)T * qd * 2);
  L.att16l = o; o += align256((size_t)T * qd * 2);
  L.mlp16 = o; o += align256((size_t)T * c.inter * 2);
  L.mlp16l = o; o += align256((size_t)T * c.inter * 2);
  L.pos_rows = o; o += align256((size_t)T * 4);
  L.attn_stride = align256(attn_workspace_bytes(c.n_heads, c.head_dim, 1));
  L.attn_ws = o; o += (size_t)T * L.attn_stride;
  L.a_last = o; o += align256((size_t)c.hidden * 4);
  size_t pb = 0;  // k-split partials of the largest split GEMM
  const int Ns[3] = {nqkv, c.hidden, c.hidden}, Ks[3] = {c.hidden, qd, c.inter};
  for (int i = 0; i < 3; ++i)
    pb = std::max(pb, (size_t)gemm_p_splits(T, Ns[i], Ks[i], EPI_STORE) * T * Ns[i] * 4);
  L.part = o; o += align256(pb);
  L.total = o;
  return L;
}

qdec_status prefill_supported(const qdec_config &c) {
  const int qd = c.n_heads * c.head_dim;
  QDEC_REQUIRE(c.hidden % 32 == 0 && qd % 32 == 0 && c.inter % 32 == 0 && c.hidden <= 16384, QDEC_EUNSUPPORTED,
               "qdec_prefill: hidden, n_heads*head_dim and inter must be multiples of 32 (hidden <= 16384)");
  return QDEC_OK;
}

qdec_status enqueue_prefill(qdec_step *h, const int32_t *tokens, int T, char *ws, hipStream_t st) {
  const qdec_config &c = h->cfg;
  const qdec_state &s = h->state;
  const int H = c.hidden, Hq = c.n_heads, Hkv = c.n_kv_heads, D = c.head_dim, I = c.inter, V = c.vocab;
  const int nqkv = (Hq + 2 * Hkv) * D, qd = Hq * D;
  const int wf = c.wfmt;
  const PLayout L = playout(c, T);
  float *x32 = reinterpret_cast<float *>(ws + L.x32);
  uint16_t *a16 = reinterpret_cast<uint16_t *>(ws + L.a16);
  uint16_t *a16l = reinterpret_cast<uint16_t *>(ws + L.a16l);
  float *qkv = reinterpret_cast<float *>(ws + L.qkv);
  float *att = reinterpret_cast<float *>(ws + L.att);
  uint16_t *att16 = reinterpret_cast<uint16_t *>(ws + L.att16);
  uint16_t *att16l = reinterpret_cast<uint16_t *>(ws + L.att16l);
  uint16_t *mlp16 = reinterpret_cast<uint16_t *>(ws + L.mlp16);
  uint16_t *mlp16l = reinterpret_cast<uint16_t *>(ws + L.mlp16l);
  int32_t *pos_rows = reinterpret_cast<int32_t *>(ws + L.pos_rows);
  float *a_last = reinterpret_cast<float *>(ws + L.a_last);
  int n = 0;
  QDEC_CK(launch_prefill_positions(s.pos, T, pos_rows, st));
  QDEC_CK(launch_embed_tokens(h->model.embed, tokens, T, H, V, x32, st));
  for (int l = 0; l < c.n_layers; ++l) {
    const qdec_layer_weights &w = h->layers[l];
    QDEC_CK(launch_rmsnorm_rows_h(x32, w.g_attn, a16, a16l, T, H, c.rms_eps, st));
    GemmPArgs g{};
    g.W = reinterpret_cast<const uint8_t *>(w.w_qkv);
    g.S = w.s_qkv;
    g.X = a16;
    g.Xl = a16l;
    g.ldx = H;
    g.bias = c.has_qkv_bias ? w.b_qkv : nullptr;
    g.Y = qkv;
    g.ldy = nqkv;
    g.M = T;
    g.N = nqkv;
    g.K = H;
    g.group = c.group;
    g.epi = EPI_STORE;
    g.part = reinterpret_cast<float *>(ws + L.part);
    g.ks = gemm_p_splits(T, nqkv, H, EPI_STORE);
    QDEC_CK(launch_gemm_p(wf, g, st));
    QkvRows qr{};
    qr.a.g_q = c.has_qk_norm ? w.g_q : nullptr;
    qr.a.g_k = c.has_qk_norm ? w.g_k : nullptr;
    qr.a.eps = c.rms_eps;
    qr.a.rope_base = c.rope_base;
    qr.a.Hq = Hq;
    qr.a.Hkv = Hkv;
    qr.a.D = D;
    qr.a.k_pool = h->kpools[l];
    qr.a.v_pool = h->vpools[l];
    qr.a.kv_fmt = c.kv_fmt;
    qr.a.page_table = s.page_table;
    qr.a.n_pages = c.n_pages;
    qr.qkv = qkv;
    qr.pos_rows = pos_rows;
    qr.T = T;
    QDEC_CK(launch_qkv_post_rows(qr, st));
    AttnRows ar{};
    ar.a.k_pool = h->kpools[l];
    ar.a.v_pool = h->vpools[l];
    ar.a.kv_fmt = c.kv_fmt;
    ar.a.page_table = s.page_table;
    ar.a.n_pages = c.n_pages;
    ar.a.Hq = Hq;
    ar.a.Hkv = Hkv;
    ar.a.D = D;
    ar.a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
    ar.a.splits = 1;
    ar.q = qkv;
    ar.q_stride = nqkv;
    ar.pos_rows = pos_rows;
    ar.ws = ws + L.attn_ws;
    ar.ws_stride = L.attn_stride;
    ar.out = att;
    ar.T = T;
    QDEC_CK(launch_attention_rows(ar, st));
    QDEC_CK(launch_to_half(att, att16, att16l, (size_t)T * qd, st));
    GemmPArgs o = g;
    o.W = reinterpret_cast<const uint8_t *>(w.w_o);
    o.S = w.s_o;
    o.X = att16;
    o.Xl = att16l;
    o.ldx = qd;
    o.bias = nullptr;
    o.residual = x32;
    o.Y = x32;
    o.ldy = H;
    o.N = H;
    o.K = qd;
    o.ks = gemm_p_splits(T, H, qd, EPI_STORE);
    QDEC_CK(launch_gemm_p(wf, o, st));
    QDEC_CK(launch_rmsnorm_rows_h(x32, w.g_ffn, a16, a16l, T, H, c.rms_eps, st));
    GemmPArgs gu = g;
    gu.W = reinterpret_cast<const uint8_t *>(w.w_gu);
    gu.S = w.s_gu;
    gu.bias = nullptr;
    gu.Y = nullptr;
    gu.Yh = mlp16;
    gu.Yl = mlp16l;
    gu.ldy = I;
    gu.N = 2 * I;
    gu.epi = EPI_SWIGLU;
    gu.ks = 1;
    QDEC_CK(launch_gemm_p(wf, gu, st));
    GemmPArgs d = o;
    d.W = reinterpret_cast<const uint8_t *>(w.w_down);
    d.S = w.s_down;
    d.X = mlp16;
    d.Xl = mlp16l;
    d.ldx = I;
    d.K = I;
    d.ks = gemm_p_splits(T, H, I, EPI_STORE);
    QDEC_CK(launch_gemm_p(wf, d, st));
  }
  // the last token: hidden state, final RMSNorm, lm head with the greedy argmax (it advances the
  // position by one, so the prompt's other tokens are added first) and the step bookkeeping
  QDEC_CK(launch_copy(x32 + (size_t)(T - 1) * H, s.hidden, H, st));
  QDEC_CK(launch_rmsnorm_rows(x32 + (size_t)(T - 1) * H, h->model.g_out, a_last, 1, H, c.rms_eps, st));
  if (T > 1) QDEC_CK(launch_add_pos(s.pos, T - 1, st));
  GemvArgs a = gemv_args(h, h->model.w_lm, h->model.s_lm, a_last, s.logits, V, H, h->p_lm);
  a.epi = EPI_ARGMAX;
  a.token = s.token;
  a.pos = s.pos;
  a.token_log = s.token_log;
  a.step_count = s.step_count;
  a.log_len = s.log_len;
  QDEC_CK(launch_gemv(wf, a, h->p_lm, st));
  (void)n;
  return QDEC_OK;
}

}  // namespace
}  // namespace qdec

using namespace qdec;

extern "C" {

size_t qdec_prefill_workspace_bytes(const qdec_config *cfg, int max_tokens) {
  if (validate(cfg) != QDEC_OK || max_tokens < 1 || prefill_supported(*cfg) != QDEC_OK) return 0;
  return playout(*cfg, max_tokens).total;
}

qdec_status qdec_prefill(qdec_step *h, const int32_t *tokens, int n_tokens, void *workspace, size_t workspace_bytes,
                         void *stream) {
  const char *nm = "qdec_prefill";
  QDEC_REQUIRE(h && tokens && workspace, QDEC_EINVAL, "%s: null argument", nm);
  QDEC_REQUIRE(n_tokens >= 1, QDEC_EINVAL, "%s: n_tokens must be >= 1", nm);
  QDEC_REQUIRE(h->model.embed && h->model.w_lm, QDEC_EINVAL, "%s: needs the embedding and the lm head", nm);
  qdec_status r = prefill_supported(h->cfg);
  if (r != QDEC_OK) return r;
  QDEC_REQUIRE((reinterpret_cast<uintptr_t>(workspace) % 256) == 0, QDEC_EINVAL, "%s: workspace must be 256-byte aligned",
               nm);
  QDEC_REQUIRE(workspace_bytes >= playout(h->cfg, n_tokens).total, QDEC_EINVAL, "%s: workspace too small (%zu < %zu bytes)",
               nm, workspace_bytes, playout(h->cfg, n_tokens).total);
  return enqueue_prefill(h, tokens, n_tokens, reinterpret_cast<char *>(workspace), (hipStream_t)stream);
}

size_t qdec_step_workspace_bytes(const qdec_config *cfg) {
  if (validate(cfg) != QDEC_OK) return 0;
  return layout_of(*cfg).total;
}

qdec_status qdec_step_create(const qdec_config *cfg, const qdec_model *m, const qdec_state *s,
                             qdec_step **out) {
  qdec_status r = validate(cfg);
  if (r != QDEC_OK) return r;
  QDEC_REQUIRE(m && s && out && m->layers, QDEC_EINVAL, "qdec_step_create: null argument");
  QDEC_REQUIRE(s->k_pools && s->v_pools && s->page_table && s->pos && s->hidden && s->workspace,
               QDEC_EINVAL, "qdec_step_create: state is missing pools, page table, pos, hidden or workspace");
  const bool lm = m->w_lm != nullptr;
  QDEC_REQUIRE(!lm || (cfg->vocab >= 1 && m->s_lm && m->g_out && s->logits && s->token), QDEC_EINVAL,
               "qdec_step_create: an lm head needs vocab, s_lm, g_out, logits and token");
  QDEC_REQUIRE(!m->embed || (cfg->vocab >= 1 && s->token), QDEC_EINVAL,
               "qdec_step_create: an embedding needs vocab and token");
  QDEC_REQUIRE(!s->token_log || (s->step_count && s->log_len >= 1), QDEC_EINVAL,
               "qdec_step_create: token_log needs step_count and log_len");
  const Layout L = layout_of(*cfg);
  QDEC_REQUIRE(s->workspace_bytes >= L.total, QDEC_EINVAL,
               "qdec_step_create: workspace too small (%zu < %zu bytes)", s->workspace_bytes, L.total);
  QDEC_REQUIRE((reinterpret_cast<uintptr_t>(s->workspace) % 256) == 0, QDEC_EINVAL, "qdec_step_create: workspace must be 256-byte aligned");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const qdec_layer_weights &w = m->layers[l];
    QDEC_REQUIRE(w.w_qkv && w.s_qkv && w.w_o && w.s_o && w.w_gu && w.s_gu && w.w_down && w.s_down &&
                     w.g_attn && w.g_ffn,
                 QDEC_EINVAL, "qdec_step_create: layer %d is missing a weight", l);
    QDEC_REQUIRE(!cfg->has_qkv_bias || w.b_qkv, QDEC_EINVAL, "qdec_step_create: layer %d has no qkv bias", l);
    QDEC_REQUIRE(!cfg->has_qk_norm || (w.g_q && w.g_k), QDEC_EINVAL,
                 "qdec_step_create: layer %d has no q/k norm gains", l);
    QDEC_REQUIRE(s->k_pools[l] && s->v_pools[l], QDEC_EINVAL, "qdec_step_create: layer %d has no KV pool", l);
  }
  qdec_step *h = new qdec_step();
  h->cfg = *cfg;
  h->layers.assign(m->layers, m->layers + cfg->n_layers);
  h->model = *m;
  h->model.layers = h->layers.data();
  h->kpools.assign(s->k_pools, s->k_pools + cfg->n_layers);
  h->vpools.assign(s->v_pools, s->v_pools + cfg->n_layers);
  h->state = *s;
  h->state.k_pools = h->kpools.data();
  h->state.v_pools = h->vpools.data();
  char *ws = reinterpret_cast<char *>(s->workspace);
  h->qkv = reinterpret_cast<float *>(ws + L.qkv);
  h->attn = reinterpret_cast<float *>(ws + L.attn);
  h->mlp = reinterpret_cast<float *>(ws + L.mlp);
  h->ssq = reinterpret_cast<float *>(ws + L.ssq);
  h->attn_ws = reinterpret_cast<float *>(ws + L.attn_ws);
  h->attn_tws = reinterpret_cast<uint32_t *>(ws + L.attn_tws);
  h->attn_tout = reinterpret_cast<uint32_t *>(ws + L.attn_tout);
  h->rope_cs = reinterpret_cast<double *>(ws + L.rope_cs);
  h->gemv_ws = ws + L.gemv_ws;
  h->sample_ws = ws + L.sample_ws;
  h->ssq_n = (cfg->hidden + 63) / 64;
  const int qd = cfg->n_heads * cfg->head_dim;
  const int nqkv = (cfg->n_heads + 2 * cfg->n_kv_heads) * cfg->head_dim;
  h->p_qkv = gemv_plan(cfg->wfmt, nqkv, cfg->hidden, true);
  h->p_o = gemv_plan(cfg->wfmt, cfg->hidden, qd, true);
  h->splits = cfg->num_splits;
  h->p_gu = gemv_plan(cfg->wfmt, 2 * cfg->inter, cfg->hidden, true);
  h->p_down = gemv_plan(cfg->wfmt, cfg->hidden, cfg->inter, true);
  if (lm) h->p_lm = gemv_plan(cfg->wfmt, cfg->vocab, cfg->hidden, true);
  h->err = reinterpret_cast<unsigned *>(ws + L.err);
  const int G = cfg->n_heads / cfg->n_kv_heads;
  h->gemv_ws2 = ws + L.gemv_ws2;
  h->hB = reinterpret_cast<float *>(ws + L.hB);
  h->ssqB = reinterpret_cast<float *>(ws + L.ssqB);
  h->lsync = reinterpret_cast<unsigned *>(ws + L.lsync);
  h->lsync_layer_words = lsync_layer_words(cfg->n_kv_heads);
  // The fused attention launch, when the shape has one and a workgroup per compute unit covers
  // its work; the per-op launches then use the same GEMV plans and splits, so the two agree bit
  // for bit.
  h->layer_ok = false;
  if (layer_fusion_supported(G, cfg->head_dim) && cfg->n_kv_heads <= kLine &&
      attn_layer_blocks_per_cu(cfg->wfmt, cfg->kv_fmt, G) >= 1) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus >= 1) {
      const int nblk = std::min(cus, kMaxLayerBlocks);
      const int waves = nblk * attn_layer_waves();
      const GemvPlan pq = layer_plan(cfg->wfmt, nqkv, cfg->hidden, waves, 1 << 30);
      int ow = attn_layer_o_waves();
      GemvPlan po = layer_plan(cfg->wfmt, cfg->hidden, qd, nblk * ow, attn_layer_stash_runs());
      if (po.units == 0) {
        ow = attn_layer_waves();
        po = layer_plan(cfg->wfmt, cfg->hidden, qd, nblk * ow, attn_layer_stash_runs());
      }
      const int S = std::min(cfg->num_splits, nblk / cfg->n_kv_heads);
      if (pq.units > 0 && po.units > 0 && S >= 1) {
        h->layer_ok = true;
        h->nblk = nblk;
        h->o_waves = ow;
        h->p_qkv = pq;
        h->p_o = po;
        h->splits = S;
      }
    }
  }
  *out = h;
  return QDEC_OK;
}

qdec_status qdec_decode_step(qdec_step *h, int mode, void *stream) {
  QDEC_REQUIRE(h, QDEC_EINVAL, "qdec_decode_step: null handle");
  hipStream_t st = (hipStream_t)stream;
  const bool per_op = (mode & QDEC_STEP_PER_OP) != 0;
  const int base = mode & ~QDEC_STEP_PER_OP;
  if (base == QDEC_STEP_EAGER) return enqueue_step(h, st, &h->n_kernels, per_op);
  QDEC_REQUIRE(base == QDEC_STEP_GRAPH, QDEC_EINVAL, "qdec_decode_step: unknown mode %d", mode);
  const int v = per_op ? 1 : 0;
  if (!h->exec[v]) {
    QDEC_REQUIRE(st != nullptr, QDEC_ESTATE,
                 "qdec_decode_step: graph capture needs a non-default stream");
    hipError_t e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
      set_error("hipStreamBeginCapture: %s", hipGetErrorString(e));
      return QDEC_EHIP;
    }
    int nk = 0;
    qdec_status r = enqueue_step(h, st, &nk, per_op);
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
    e = hipGraphInstantiate(&h->exec[v], g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      (void)hipGraphDestroy(g);
      set_error("hipGraphInstantiate: %s", hipGetErrorString(e));
      return QDEC_EHIP;
    }
    h->graph[v] = g;
    h->graph_stream[v] = st;
    h->graph_kernels[v] = nk;
  }
  QDEC_REQUIRE(st == h->graph_stream[v], QDEC_ESTATE,
               "qdec_decode_step: graph was captured on another stream");
  hipError_t e = hipGraphLaunch(h->exec[v], st);
  if (e != hipSuccess) {
    set_error("hipGraphLaunch: %s", hipGetErrorString(e));
    return QDEC_EHIP;
  }
  h->n_kernels = h->graph_kernels[v];
  return QDEC_OK;
}

int qdec_step_kernel_count(const qdec_step *h) { return h ? h->n_kernels : 0; }

int qdec_step_kernel_times(qdec_step *h, int mode, float *us, int max, void *stream) {
  const char *nm = "qdec_step_kernel_times";
  QDEC_REQUIRE(h && (us || max == 0) && max >= 0, QDEC_EINVAL, "%s: null argument", nm);
  QDEC_REQUIRE((mode & ~QDEC_STEP_PER_OP) == QDEC_STEP_EAGER, QDEC_EINVAL, "%s: mode must be EAGER (| PER_OP)", nm);
  hipStream_t st = (hipStream_t)stream;
  const size_t need = 8 + 8 * (size_t)h->cfg.n_layers;  // more than any step launches
  while (h->tev.size() < need) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
      set_error("%s: hipEventCreate failed", nm);
      return QDEC_EHIP;
    }
    h->tev.push_back(e);
  }
  h->tev_n = 0;
  h->timing = true;
  step_mark(h, st);
  int nk = 0;
  const qdec_status r = enqueue_step(h, st, &nk, (mode & QDEC_STEP_PER_OP) != 0);
  h->timing = false;
  const size_t marks = h->tev_n;
  hipError_t e = hipStreamSynchronize(st);
  if (r != QDEC_OK) return r;
  if (e != hipSuccess) {
    set_error("%s: %s", nm, hipGetErrorString(e));
    return QDEC_EHIP;
  }
  const int n = (int)marks - 1;
  for (int i = 0; i < n && i < max; ++i) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, h->tev[i], h->tev[i + 1]);
    if (e != hipSuccess) {
      set_error("%s: %s", nm, hipGetErrorString(e));
      return QDEC_EHIP;
    }
    us[i] = ms * 1000.f;
  }
  h->n_kernels = nk;
  return n;
}

qdec_status qdec_step_set_sampling(qdec_step *h, float temperature, int top_k, float top_p, uint64_t seed) {
  const char *nm = "qdec_step_set_sampling";
  QDEC_REQUIRE(h, QDEC_EINVAL, "%s: null handle", nm);
  QDEC_REQUIRE(!std::isnan(temperature), QDEC_EINVAL, "%s: temperature is NaN", nm);
  QDEC_REQUIRE(top_p > 0.f && top_p <= 1.f, QDEC_EINVAL, "%s: top_p must be in (0, 1] (got %g)", nm, (double)top_p);
  QDEC_REQUIRE(top_k >= 0, QDEC_EINVAL, "%s: top_k must be >= 0", nm);
  if (temperature > 0.f) {
    QDEC_REQUIRE(h->model.w_lm && h->state.step_count, QDEC_EINVAL, "%s: sampling needs an lm head and step_count", nm);
    const int V = h->cfg.vocab;
    QDEC_REQUIRE(top_k <= kSampleMaxTopK || top_k >= V, QDEC_EUNSUPPORTED, "%s: top_k above %d is not supported", nm,
                 kSampleMaxTopK);
    QDEC_REQUIRE(top_p >= 1.f || (top_k >= 1 && top_k <= kSampleMaxTopK), QDEC_EUNSUPPORTED,
                 "%s: top_p < 1 needs 1 <= top_k <= %d", nm, kSampleMaxTopK);
  }
  h->temperature = temperature > 0.f ? temperature : 0.f;
  h->top_k = top_k;
  h->top_p = top_p;
  h->seed = seed;
  drop_graphs(h);
  return QDEC_OK;
}


int qdec_step_layer_blocks(const qdec_step *h) { return h && h->layer_ok ? h->nblk : 0; }

qdec_status qdec_step_layer_timeline(qdec_step *h, uint64_t *ts) {
  QDEC_REQUIRE(h, QDEC_EINVAL, "qdec_step_layer_timeline: null handle");
  QDEC_REQUIRE(!ts || h->layer_ok, QDEC_EUNSUPPORTED, "qdec_step_layer_timeline: this step has no fused attention launch");
  h->timeline = reinterpret_cast<unsigned long long *>(ts);
  drop_graphs(h);
  return QDEC_OK;
}

qdec_status qdec_step_mlp_timeline(qdec_step *h, uint64_t *ts, int *units) {
  QDEC_REQUIRE(h, QDEC_EINVAL, "qdec_step_mlp_timeline: null handle");
  if (units) {
    units[0] = h->p_gu.units;
    units[1] = h->p_down.units;
  }
  h->mlp_timeline = reinterpret_cast<unsigned long long *>(ts);
  drop_graphs(h);
  return QDEC_OK;
}

qdec_status qdec_step_read_error(qdec_step *h, int *flag) {
  QDEC_REQUIRE(h && flag, QDEC_EINVAL, "qdec_step_read_error: null argument");
  unsigned v = 0;
  hipError_t e = hipMemcpy(&v, h->err, sizeof(v), hipMemcpyDeviceToHost);
  if (e == hipSuccess && v) {
    const unsigned z = 0;
    e = hipMemcpy(h->err, &z, sizeof(z), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    set_error("qdec_step_read_error: %s", hipGetErrorString(e));
    return QDEC_EHIP;
  }
  *flag = (int)v;
  return QDEC_OK;
}

void qdec_step_destroy(qdec_step *h) {
  if (!h) return;
  for (hipEvent_t e : h->tev) (void)hipEventDestroy(e);
  for (int v = 0; v < 2; ++v) {
    if (h->exec[v]) (void)hipGraphExecDestroy(h->exec[v]);
    if (h->graph[v]) (void)hipGraphDestroy(h->graph[v]);
  }
  delete h;
}

}  // extern "C"
