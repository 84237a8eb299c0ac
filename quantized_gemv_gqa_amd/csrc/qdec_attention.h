// Split-K paged GQA decode attention: the per-unit device code, shared by the standalone
// attention kernel and the fused layer kernel (gfx950, wave64).  The method and the layout are
// described in attention.hip.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>

#include "qdec_device.h"

namespace qdec {
namespace attn {

using namespace dev;

// One lane's piece of a token row: DPL = D / 16 values, kept packed as W dwords until used.
template <int D, int KVF>
struct Row {
  static constexpr int DPL = D / 16;
  static constexpr int EB = KVF == QDEC_KV_BF16 ? 2 : 4;  // bytes per element
  static constexpr int W = DPL * EB / 4;
  uint32_t w[W];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (W == 2) {
      // (a 64-bit load is read as one 64-bit integer: a two-lane vector view of it compiles to a
      // single dword load)
      const uint64_t v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
      w[0] = (uint32_t)v; w[1] = (uint32_t)(v >> 32);
    } else {
#pragma unroll
      for (int c = 0; c < W / 4; ++c) {
        const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * c, 0, 0));
        w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
      }
    }
  }
  __device__ __forceinline__ float get(int e) const {
    if constexpr (KVF == QDEC_KV_BF16)
      return __builtin_bit_cast(float, (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
    else
      return __builtin_bit_cast(float, w[e]);
  }
  // the stored form of fp32 values: bf16 round-to-nearest-even, or the fp32 bits
  __device__ __forceinline__ void set(const float (&v)[DPL]) {
    if constexpr (KVF == QDEC_KV_BF16) {
#pragma unroll
      for (int i = 0; i < W; ++i)
        w[i] = (uint32_t)float_to_bf16_rne(v[2 * i]) | ((uint32_t)float_to_bf16_rne(v[2 * i + 1]) << 16);
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) w[i] = __builtin_bit_cast(uint32_t, v[i]);
    }
  }
  __device__ __forceinline__ void store(void *pool, size_t elem) const {
    uint32_t *d = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(pool) + elem * EB);
#pragma unroll
    for (int i = 0; i < W; ++i) d[i] = w[i];
  }
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = 0u;
  }
};

// Online-softmax update of one wave with up to four 4-token quarters of the context: token
// t0[sub] + slot sits in this lane's kp[sub] / vp[sub] for sub < nsub (uniform); tokens at or past
// T are masked (an unmapped quarter has t0 = T).  Subs from nsub on are skipped.
template <int D, int G, int KVF>
__device__ __forceinline__ void attend_quarters(Row<D, KVF> (&kp)[4], Row<D, KVF> (&vp)[4], const int (&t0)[4],
                                                int nsub, int T, int slot, const float (&q)[G][D / 16],
                                                float (&m)[G], float (&l)[G], float (&o)[G][D / 16]) {
  constexpr int DPL = D / 16;
  float sc[4][G];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    if (sub >= nsub) {
#pragma unroll
      for (int h = 0; h < G; ++h) sc[sub][h] = -INFINITY;
      continue;
    }
    const bool valid = t0[sub] + slot < T;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) d = fmaf(q[h][e], kp[sub].get(e), d);
      d = sum16(d);
      sc[sub][h] = valid ? d : -INFINITY;
    }
    // slots past the newest token may hold stale bits (even NaN): zero them, never multiply
    // them by a zero weight
    if (!valid) vp[sub].clear();
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mx = fmaxf(fmaxf(m[h], fmaxf(sc[0][h], sc[1][h])), fmaxf(sc[2][h], sc[3][h]));
    const float alpha = __builtin_amdgcn_exp2f(m[h] - mx);
    m[h] = mx;
    float ls = 0.f;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      sc[sub][h] = __builtin_amdgcn_exp2f(sc[sub][h] - mx);
      ls += sc[sub][h];
    }
    l[h] = fmaf(l[h], alpha, ls);
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] *= alpha;
  }
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    if (sub >= nsub) break;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float vv = vp[sub].get(e);
#pragma unroll
      for (int h = 0; h < G; ++h) o[h][e] = fmaf(sc[sub][h], vv, o[h][e]);
    }
  }
}

// Optional RMSNorm over the head (DPL dims per lane, 16 lanes) and RoPE rotation of one head
// vector: `own` are the lane's dims, `mate` the dims D/2 away; cs holds the fp64 (cos, sin) of
// the lane's DPL rotation pairs.
template <int D>
__device__ __forceinline__ void norm_rope(float (&own)[D / 16], float (&mate)[D / 16], int part, const float *gamma,
                                          float eps, const double *cs) {
  constexpr int DPL = D / 16, HALF = D / 2;
  const int d0 = part * DPL;
  const bool lo = d0 < HALF;
  if (gamma) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) ss = fmaf(own[e], own[e], ss);
    ss = sum16(ss);
    const float r = rsqrtf(ss / (float)D + eps);
    const int dm = lo ? d0 + HALF : d0 - HALF;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      own[e] = gamma[d0 + e] * (own[e] * r);
      mate[e] = gamma[dm + e] * (mate[e] * r);
    }
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const double c = cs[2 * e], sn = cs[2 * e + 1];
    const double x = own[e], y = mate[e];
    // low half: x' = x c - y s (y = x[i + D/2]); high half: x' = x c + y s (y = x[i - D/2])
    own[e] = (float)(lo ? (x * c - y * sn) : (x * c + y * sn));
  }
}

constexpr int kAttnWaves = 8;                  // waves per workgroup
constexpr int kAttnThreads = 64 * kAttnWaves;

__device__ __forceinline__ void store_sc1_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kAuxSc1);
}

// ROPE: q, k and v come raw from the fused qkv vector; the kernel applies the optional q/k
// RMSNorm and RoPE itself, appends the new token's k and v (split 0), and takes the newest key
// and value from registers.  Otherwise q is given rotated and the new token's k and v were
// appended before the launch.
template <int D, int G, bool ROPE>
struct AttnSmem {
  static constexpr int NW = kAttnWaves;
  static constexpr int C = G * D / 4;  // f32x4 columns of a split's partial output
  float m[NW][G], l[NW][G];
  // per-wave partial outputs, then a merged head's per-row sums (kAttnThreads of them), or the
  // split weights of all G heads (standalone merge)
  f32x4 o[NW * C > kAttnThreads ? NW * C : kAttnThreads];
  float w[kMaxMergeSplits], ls[kMaxMergeSplits];  // a merged head's split weights and sums
  float q[ROPE ? (G + 2) * D : 1];
  unsigned flag;
};

// One (KV head j, split s) attention unit, run by a whole workgroup of kAttnThreads threads.
// SYNC: the step-synchronised form of the fused layer kernels (AttnArgs: epoch, wait_cnt, tws,
// tout).  start() requests the RoPE table and the wave's first KV page (nothing else happens
// before it); pages() waits for the inputs and attends to the wave's pages; publish() merges the
// workgroup's waves and publishes (and merges) the split.  A kernel can issue other roles' loads,
// or compute, between the three; finish() is pages() then publish().
template <int D, int G, int KVF, bool ROPE, bool SYNC>
struct AttnUnit {
  static constexpr int DPL = D / 16;
  static constexpr int EB = Row<D, KVF>::EB;
  static constexpr int NW = kAttnWaves;
  // (A second page buffer spilled registers of the 7-query-head unit and was slower at every
  // context and batch measured.)
  static constexpr int PF = 1;
  // Waves 0 .. kRopeWaves - 1 stage the q, k, v rows and norm + rotate the heads; the others may
  // carry long-running loads of other roles (which in-order memory counters would make these
  // steps wait for).
  static constexpr int kRopeWaves = 4;
  int pos, T, Q, npw, pw, gb, nq, last_page;
  int nwp;       // waves of this split that hold quarters (the first ones)
  unsigned ep;   // the step number (SYNC)
  __amdgpu_buffer_rsrc_t kr, vr;
  Row<D, KVF> kp[PF][4], vp[PF][4];
  int t0[PF][4];
  double cs[ROPE ? 2 * DPL : 1];  // fp64 (cos, sin) of the lane's rotation pairs

  __device__ __forceinline__ void start(const AttnArgs &a, int j, int s) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slot = lane >> 4;
    const int part = lane & 15;
    pos = *a.pos;
    T = pos + 1;
    // The context is dealt in quarters of a page (4 tokens; quarter g is sub-block g % 4 of page
    // g / 4) so that the work spreads evenly over the SIMDs and no wave waits for a second round
    // trip it could have shared out: per KV head npw = W splits waves hold quarters, splits
    // first: wave pw = s + splits * wave takes quarters gb + pw, gb + pw + npw, ..., four at a
    // time.  With x = Q / (4 splits) quarter groups per split:
    //   x <= 4: W = ceil(x) waves (one per SIMD), each with at most one group;
    //   4 < x <= 8: waves 0 .. 3 take the first 16 splits quarters, exactly one group each, and
    //     waves 4 .. 7 (gb = 16 splits) the rest, at most one group each: a group beyond the
    //     first on one wave would cost its split a serial round trip (the step just past a
    //     context of 16 splits pages leaves one such quarter);
    //   x > 8: all 8 waves (two per SIMD, evenly loaded).
    Q = max(0, min((T + 3) >> 2, 4 * a.n_pages));  // never index outside the page table
    const int q4 = 4 * a.splits;
    static_assert(NW == 8, "the wave counts above assume 8 waves on 4 SIMDs");
    gb = 0;
    if (Q > 4 * q4 && Q <= 8 * q4) {
      const int hi = wave >= 4;
      const int Qh = hi ? Q - 4 * q4 : 4 * q4;  // the quarters of this half of the waves
      gb = hi ? 4 * q4 : 0;
      npw = q4;
      pw = s + a.splits * (wave - 4 * hi);
      nq = pw < Qh ? (Qh - pw + npw - 1) / npw : 0;
      const int R = Q - 4 * q4;
      nwp = 4 + (R > s ? min(4, (R - s + a.splits - 1) / a.splits) : 0);  // wave < nwp  <=>  nq > 0
    } else {
      const int W = Q <= 4 * q4 ? max(1, (Q + q4 - 1) / q4) : NW;
      npw = W * a.splits;
      pw = s + a.splits * wave;
      nq = (wave < W && pw < Q) ? (Q - pw + npw - 1) / npw : 0;
      nwp = Q > s ? min(W, (Q - s + a.splits - 1) / a.splits) : 0;  // wave < nwp  <=>  nq > 0
    }
    last_page = ((T + 15) >> 4) - 1;
    if constexpr (ROPE) {
      if (wave < kRopeWaves) {
        const int i0 = (part * DPL) % (D / 2);
#pragma unroll
        for (int e = 0; e < 2 * DPL; ++e) cs[e] = a.rope_cs[2 * i0 + e];
      }
    }
    const uint32_t pool_bytes = (uint32_t)((size_t)a.n_pages * a.Hkv * 16 * D * EB);
    kr = rsrc(a.k_pool, pool_bytes);
    vr = rsrc(a.v_pool, pool_bytes);
#pragma unroll
    for (int i = 0; i < PF; ++i) load_group(a, j, i, i, slot, part);
  }

  // Requests quarters 4 k .. 4 k + 3 of this wave into buffer b (t0 = T for a quarter past the
  // wave's share or on an unmapped page: its tokens are masked, nothing is read).
  // The page-table entries of quarters 4 k .. 4 k + 3 of this wave, one per lane 0 .. 3 (-1
  // past the wave's share): one load for the group.
  __device__ __forceinline__ int group_entries(const AttnArgs &a, int k, int lane) const {
    return (lane < 4 && 4 * k + lane < nq) ? a.page_table[(gb + pw + npw * (4 * k + lane)) >> 2] : -1;
  }

  // Requests the rows of quarters 4 k .. 4 k + 3 into buffer b, their page-table entries from
  // group_entries (lane sub holds the entry of quarter 4 k + sub).
  __device__ __forceinline__ void rows_of(int ent, int j, int k, int b, int slot, int part, const AttnArgs &a) {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const int i = 4 * k + sub;
      t0[b][sub] = T;
      if (i < nq) {
        const int g = gb + pw + npw * i;
        const int phys = __builtin_amdgcn_readlane(ent, sub);
        if (phys >= 0 && phys < a.n_pages) {  // documented precondition; never read outside
          t0[b][sub] = 4 * g;
          const size_t row = (((size_t)phys * a.Hkv + j) * 16 + (g & 3) * 4 + slot) * D + part * DPL;
          kp[b][sub].load(kr, (uint32_t)(row * EB));
          vp[b][sub].load(vr, (uint32_t)(row * EB));
        }
      }
    }
  }

  __device__ __forceinline__ void load_group(const AttnArgs &a, int j, int k, int b, int slot, int part) {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const int i = 4 * k + sub;
      t0[b][sub] = T;
      if (i < nq) {
        const int g = gb + pw + npw * i;
        const int phys = a.page_table[g >> 2];
        if (phys >= 0 && phys < a.n_pages) {  // documented precondition; never read outside
          t0[b][sub] = 4 * g;
          const size_t row = (((size_t)phys * a.Hkv + j) * 16 + (g & 3) * 4 + slot) * D + part * DPL;
          kp[b][sub].load(kr, (uint32_t)(row * EB));
          vp[b][sub].load(vr, (uint32_t)(row * EB));
        }
      }
    }
  }

  __device__ __forceinline__ bool holds_page() const { return nq > 0; }

  __device__ __forceinline__ void finish(const AttnArgs &a, int j, int s, AttnSmem<D, G, ROPE> &sm,
                                        unsigned long long *rec = nullptr) {
    if (pages(a, j, s, sm, rec)) publish(a, j, s, sm, rec);
  }

  // Waits for the inputs (SYNC), stages q, k, v (ROPE), attends to the wave's pages and leaves
  // each page-holding wave's (m, l, o) in LDS.  Returns false (for the whole workgroup) if the
  // wait gave up.
  __device__ __forceinline__ bool pages(const AttnArgs &a, int j, int s, AttnSmem<D, G, ROPE> &sm,
                                        unsigned long long *rec = nullptr) {
  constexpr int C = G * D / 4;                                                // f32x4 columns
  auto &sm_m = sm.m;
  auto &sm_l = sm.l;
  auto &sm_o = sm.o;
  auto &sq = sm.q;
  unsigned &last = sm.flag;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = lane >> 4;
  const int part = lane & 15;

  unsigned e = 0;
  if constexpr (SYNC) {
    // the qkv tiles of KV head j (its G q heads, its k and v) are stored; the pages above are
    // already on their way
    e = __builtin_amdgcn_readfirstlane(*a.epoch);
    if (threadIdx.x == 0) last = poll_count(a.wait_cnt + j * kLine, e * a.wait_per_step, a.err) ? 1u : 0u;
    __syncthreads();
    if (!last) return false;  // (every thread of the workgroup leaves together)
    __syncthreads();          // everyone has read the flag before it is reused
  }
  ep = e;
  mark(rec, 0);
  float q[G][DPL];
  Row<D, KVF> knew, vnew;
  if constexpr (ROPE) {
    // stage this KV head's q heads and its new k, v (one pass); then wave h norms and rotates
    // head h (q heads, then k) in place, once per workgroup; then every lane reads its dims
    const __amdgpu_buffer_rsrc_t qr = rsrc(a.qkv, (uint32_t)((a.Hq + 2 * a.Hkv) * D * 4));
    if (wave < kRopeWaves) {
      for (int i = threadIdx.x; i < (G + 2) * D / 4; i += 64 * kRopeWaves) {
        const int h = (i * 4) / D, d = i * 4 - h * D;
        const int row = h < G ? (j * G + h) : (h == G ? a.Hq + j : a.Hq + a.Hkv + j);
        *reinterpret_cast<f32x4 *>(&sq[h * D + d]) = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, (uint32_t)((row * D + d) * 4), 0, SYNC ? kAuxSc1 : 0));
      }
    }
    __syncthreads();
    mark(rec, 8);
    const int dmate = part * DPL < D / 2 ? part * DPL + D / 2 : part * DPL - D / 2;
    for (int h = wave; wave < kRopeWaves && h < G + 1; h += kRopeWaves) {
      float own[DPL], mate[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        own[e] = sq[h * D + part * DPL + e];
        mate[e] = sq[h * D + dmate + e];
      }
      norm_rope<D>(own, mate, part, h < G ? a.g_q : a.g_k, a.eps, cs);
      // (the wave's reads above all precede its writes; the four token slots hold copies)
      if (slot == 0) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) sq[h * D + part * DPL + e] = own[e];
      }
    }
    __syncthreads();
    mark(rec, 9);
    if (nq > 0) {  // (waves without quarters need no q)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < DPL; ++e) q[h][e] = sq[h * D + part * DPL + e] * a.scale_log2;
    }
    float kk[DPL], vv[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      kk[e] = sq[G * D + part * DPL + e];
      vv[e] = sq[(G + 1) * D + part * DPL + e];
    }
    knew.set(kk);
    vnew.set(vv);
    // split 0 appends them for later steps (every split uses the register copy for this token).
    // A token without a cache slot (pos < 0, past the page table, or an unmapped entry) is not
    // stored and sets the error word: its attention would leave the newest key out.
    if (s == 0 && wave == 0 && slot == 0) {
      bool stored = false;
      if (pos >= 0 && last_page < a.n_pages) {
        const int phys = a.page_table[last_page];
        if (phys >= 0 && phys < a.n_pages) {
          const size_t e0 = (((size_t)phys * a.Hkv + j) * 16 + (pos & 15)) * D + part * DPL;
          knew.store(a.k_pool, e0);
          vnew.store(a.v_pool, e0);
          stored = true;
        }
      }
      if (!stored && part == 0 && a.err) __hip_atomic_store(a.err, kErrKvSlot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < DPL; ++e) q[h][e] = a.q[(size_t)(j * G + h) * D + part * DPL + e] * a.scale_log2;
  }
  const int new_slot = pos & 3;

  float m[G], l[G], o[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] = 0.f;
  }
  const int qnew = pos >> 2;  // the newest token's quarter
  auto group = [&](Row<D, KVF> (&kq)[4], Row<D, KVF> (&vq)[4], const int (&tq)[4], int nsub) {
    if (ROPE) {  // the newest token's row comes from registers
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
        if (tq[sub] == 4 * qnew && slot == new_slot) {
          kq[sub] = knew;
          vq[sub] = vnew;
        }
    }
    attend_quarters<D, G, KVF>(kq, vq, tq, nsub, T, slot, q, m, l, o);
  };
  // later groups (long contexts): each group's four page-table entries come in one load, made
  // one group ahead, so a group costs one round trip for its rows only
  int ent = 4 * PF < nq ? group_entries(a, PF, lane) : -1;
#pragma unroll
  for (int i = 0; i < PF; ++i)
    if (4 * i < nq) group(kp[i], vp[i], t0[i], min(4, nq - 4 * i));
  for (int k = PF; 4 * k < nq; ++k) {
    rows_of(ent, j, k, 0, slot, part, a);
    if (4 * (k + 1) < nq) ent = group_entries(a, k + 1, lane);
    group(kp[0], vp[0], t0[0], min(4, nq - 4 * k));
  }

  // Merge the four token slots of this wave (lanes part, part + 16, part + 32, part + 48):
  // rescale every slot to the heads' common maximum, then sum the slots' (o, l) values with a
  // butterfly of row swaps that reduces four values at once (3 swaps and 3 adds per four
  // values; each row of lanes ends up holding the sums of a different one of the four).
  mark(rec, 1);
  // (waves without pages hold nothing to merge and leave the SIMDs to the ones with pages)
  if (wave < nwp) {
    constexpr int CPH = DPL / 4;                    // float4 chunks of a head per lane
    constexpr int NCH = G * CPH;                    // chunk slots, then the l slots
    constexpr int NS = NCH + (G + 3) / 4;
    constexpr int K = (NS + 3) / 4;                 // blocks of 16 values (4 slots x 4)
    float M[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x, y;
      pair16(m[h], x, y);
      pair32(fmaxf(x, y), x, y);
      M[h] = fmaxf(x, y);
    }
    // value 16 k + 4 j + r: element j of slot 4 k + r (chunk (h, c) = slot 2 h + c or, past the
    // chunks, l of heads 4 (slot - NCH) + j)
    float v[16 * K];
#pragma unroll
    for (int i = 0; i < 16 * K; ++i) v[i] = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float al = __builtin_amdgcn_exp2f(m[h] - M[h]);
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const int sl = h * CPH + e / 4;
        v[16 * (sl / 4) + 4 * (e % 4) + sl % 4] = o[h][e] * al;
      }
      const int sl = NCH + h / 4;
      v[16 * (sl / 4) + 4 * (h % 4) + sl % 4] = l[h] * al;
    }
    auto rowsum16 = [](float x, float y) {
      const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                      false, false);
      const unsigned r0 = r[0], r1 = r[1];  // (copied out before the casts: see pair16)
      return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
    };
    auto rowsum32 = [](float x, float y) {
      const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                      false, false);
      const unsigned r0 = r[0], r1 = r[1];
      return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
    };
    auto butterfly = [&](float a0, float a1, float a2, float a3) {
      return rowsum32(rowsum16(a0, a1), rowsum16(a2, a3));
    };
    // which of the four values this lane's row ends up with (the same for every group): found
    // by running the butterfly on markers
    const float mk = butterfly(1.f, 2.f, 4.f, 8.f);  // 4, 8, 16 or 32
    const int q = mk < 6.f ? 0 : (mk < 12.f ? 1 : (mk < 24.f ? 2 : 3));
    float t[4 * K];
#pragma unroll
    for (int g = 0; g < 4 * K; ++g) t[g] = butterfly(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
    // lane (q, part) holds element j of slot 4 k + q in t[4 k + j]
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int sl = 4 * k + q;
      if (sl < NCH) {
        const int h = sl / CPH, c = sl % CPH;
        sm_o[wave * C + (h * D + part * DPL) / 4 + c] = f32x4{t[4 * k], t[4 * k + 1], t[4 * k + 2], t[4 * k + 3]};
      } else if (sl < NS && part == 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int h = 4 * (sl - NCH) + jj;
          if (h < G) sm_l[wave][h] = t[4 * k + jj];
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) sm_m[wave][h] = M[h];
    }
  }
  return true;
  }

  // Merges the page-holding waves' states into the split's partial and publishes it; SYNC: then
  // merges the query heads this split is responsible for.
  __device__ __forceinline__ void publish(const AttnArgs &a, int j, int s, AttnSmem<D, G, ROPE> &sm,
                                          unsigned long long *rec = nullptr) {
  constexpr int C = G * D / 4;  // f32x4 columns
  auto &sm_m = sm.m;
  auto &sm_l = sm.l;
  auto &sm_o = sm.o;
  unsigned &last = sm.flag;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned e = ep;
  // the heads' (m, l) go out from the last wave, which merges no columns (C <= 256 columns sit on
  // the first four waves), beside the columns rather than after them
  static_assert(C <= 64 * (kAttnWaves - 1), "the last wave holds no column");
  const int hml = (int)threadIdx.x - 64 * (kAttnWaves - 1);
  // (an LDS-only barrier: a wave of another role may have its LDS DMA copies still in flight,
  // into a stash no other wave reads, and must not hold the split's publish for them)
  lds_barrier();
  // merge the page-holding waves into the split's partial: o (G heads x D) and per head (m, l);
  // a split without pages publishes m = -1e30, l = 0, o = 0
  const int nw = nwp;
  auto column = [&](int c) {
    const int h = c / (D / 4);
    float mx = kNegBig;
    for (int w = 0; w < nw; ++w) mx = fmaxf(mx, sm_m[w][h]);
    f32x4 val = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < nw; ++w) val += __builtin_amdgcn_exp2f(sm_m[w][h] - mx) * sm_o[w * C + c];
    return val;
  };
  auto head_ml = [&](int h, float &mx, float &lsum) {
    mx = kNegBig;
    for (int w = 0; w < nw; ++w) mx = fmaxf(mx, sm_m[w][h]);
    lsum = 0.f;
    for (int w = 0; w < nw; ++w) lsum += __builtin_amdgcn_exp2f(sm_m[w][h] - mx) * sm_l[w][h];
  };
  if constexpr (SYNC) {
    // Published as (value, tag) pairs, each pair one 8-byte store that a reader sees whole or not
    // at all, so no counter is needed: the mergers poll the tags (tag: this step's number times
    // the layer count plus the layer).  Pairs o at [s][head][D], then (m, tag, l, tag) at [s][head].
    const unsigned tag = e * a.tag_mul + a.tag_add;
    const __amdgpu_buffer_rsrc_t tor = rsrc(a.tws, (uint32_t)((size_t)a.splits * a.Hq * D * 8));
    const __amdgpu_buffer_rsrc_t tmr = rsrc(a.tws + (size_t)a.splits * a.Hq * D * 2, (uint32_t)((size_t)a.splits * a.Hq * 16));
    for (int c = threadIdx.x; c < C; c += kAttnThreads) {
      const u32x4 vb = __builtin_bit_cast(u32x4, column(c));
      const uint32_t off = (uint32_t)((((size_t)s * a.Hq + j * G) * D + 4 * c) * 8);
      u32x4 lo, hi;
      lo.x = vb.x; lo.y = tag; lo.z = vb.y; lo.w = tag;
      hi.x = vb.z; hi.y = tag; hi.z = vb.w; hi.w = tag;
      __builtin_amdgcn_raw_buffer_store_b128(lo, tor, off, 0, kAuxSc1);
      __builtin_amdgcn_raw_buffer_store_b128(hi, tor, off + 16, 0, kAuxSc1);
    }
    if (hml >= 0 && hml < G) {
      float mx, lsum;
      head_ml(hml, mx, lsum);
      u32x4 v;
      v.x = __builtin_bit_cast(uint32_t, mx); v.y = tag; v.z = __builtin_bit_cast(uint32_t, lsum); v.w = tag;
      __builtin_amdgcn_raw_buffer_store_b128(v, tmr, (uint32_t)(((size_t)s * a.Hq + j * G + hml) * 16), 0, kAuxSc1);
    }
    // every wave is done with this unit's LDS before any leaves (a kernel may reuse it next; an
    // LDS-only barrier, so that the split's stores just issued are not waited for here)
    lds_barrier();
    mark(rec, 2);
    // query head j G + hh is merged by split hh % splits, as soon as its partials are all seen
    // (its output goes out as tagged pairs too: the o GEMV polls them, no flag needed)
    for (int hh = s; hh < G; hh += a.splits)
      if (!merge_head<true>(a, j * G + hh, sm, tag)) return;
    mark(rec, 3);
    return;
  }
  // merge the NW waves and publish the split's partial through device-coherent stores (the
  // merging block may sit on another XCD): o at [s][head][D], (m, l) at [s][head][2]
  float *wso = a.ws;
  float *wsml = a.ws + (size_t)a.splits * a.Hq * D;
  const __amdgpu_buffer_rsrc_t orr = rsrc(wso, (uint32_t)((size_t)a.splits * a.Hq * D * 4));
  const __amdgpu_buffer_rsrc_t mlr = rsrc(wsml, (uint32_t)((size_t)a.splits * a.Hq * 2 * 4));
  for (int c = threadIdx.x; c < C; c += kAttnThreads)
    store_sc1_b128(orr, (uint32_t)((((size_t)s * a.Hq + j * G) * D + 4 * c) * 4), column(c));
  if (hml >= 0 && hml < G) {
    float mx, lsum;
    head_ml(hml, mx, lsum);
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = {__builtin_bit_cast(uint32_t, mx), __builtin_bit_cast(uint32_t, lsum)};
    __builtin_amdgcn_raw_buffer_store_b64(v, mlr, (uint32_t)((((size_t)s * a.Hq + j * G + hml) * 2) * 4), 0, kAuxSc1);
  }
  // the waves that stored wait for the acknowledgements
  if (wave * 64 < C || wave == kAttnWaves - 1) drain_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&a.counters[j * kLine], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (unsigned)(a.splits - 1);
  __syncthreads();
  mark(rec, 2);
  if (!last) return;
  // the last split block of KV head j merges its G query heads, all at once
  merge_heads_all(a, j, sm);
  if (threadIdx.x == 0) __hip_atomic_store(&a.counters[j * kLine], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  mark(rec, 3);
  }

  // The merge of query head h's split partials (m_s, l_s, o_s; a split without keys has
  // m = -1e30, l = 0, o = 0 and weighs nothing):
  //   out[h][d] = sum_s 2^(m_s - M) o_s[d] / sum_s 2^(m_s - M) l_s,  M = max_s m_s,
  // in a fixed order whatever the caller: row r of RH takes splits r, r + RH, r + 2 RH, ... in
  // bursts of kBurst (MergeState::add, a running maximum with its rescaled sums), then the rows
  // are folded in row order (MergeState::fold).  The fused and standalone kernels agree bit for
  // bit.
  static constexpr int CH = D / 4;                // f32x4 columns of one head
  static constexpr int RH = kAttnThreads / CH;    // split rows: 16 at D = 128, 32 at D = 64
  static constexpr int kBurst = 4;                // splits of a row in flight at once

  struct MergeState {
    float M, l;
    f32x4 acc;
    __device__ __forceinline__ MergeState() : M(kNegBig), l(0.f), acc{0.f, 0.f, 0.f, 0.f} {}
    __device__ __forceinline__ void rescale(float Mn) {
      const float sc = __builtin_amdgcn_exp2f(M - Mn);
      acc.x *= sc; acc.y *= sc; acc.z *= sc; acc.w *= sc;
      l *= sc;
      M = Mn;
    }
    __device__ __forceinline__ void add_one(float p, float lv, f32x4 o) {
      acc.x = fmaf(p, o.x, acc.x); acc.y = fmaf(p, o.y, acc.y);
      acc.z = fmaf(p, o.z, acc.z); acc.w = fmaf(p, o.w, acc.w);
      l = fmaf(p, lv, l);
    }
    // splits u < n of a burst
    __device__ __forceinline__ void add(const float (&m)[kBurst], const float (&lv)[kBurst], const f32x4 (&o)[kBurst], int n) {
      float Mn = M;
#pragma unroll
      for (int u = 0; u < kBurst; ++u)
        if (u < n) Mn = fmaxf(Mn, m[u]);
      rescale(Mn);
#pragma unroll
      for (int u = 0; u < kBurst; ++u)
        if (u < n) add_one(__builtin_amdgcn_exp2f(m[u] - Mn), lv[u], o[u]);
    }
    // the next row's state
    __device__ __forceinline__ void fold(float Mr, float lr, f32x4 ar) {
      rescale(fmaxf(M, Mr));
      add_one(__builtin_amdgcn_exp2f(Mr - M), lr, ar);
    }
    __device__ __forceinline__ f32x4 out() const {
      const float inv = 1.0f / l;
      return f32x4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    }
  };

  // TAGGED (the fused launch): the partials are (value, tag) pairs; a thread requests the (m, l)
  // pair and the column of each split of its burst at once and requests again, all together,
  // whichever came back with another tag, until every tag equals `tag` (so the last split to
  // publish costs one round trip once its stores are visible, and the polls after the first
  // reread only the splits still missing); the output is stored as tagged pairs in tout.  Else
  // plain values of a finished launch phase, and the output is stored in out.  Returns false if
  // a poll gave up (the error word is then set).
  template <bool TAGGED>
  __device__ __forceinline__ bool merge_head(const AttnArgs &a, int h, AttnSmem<D, G, ROPE> &sm, unsigned tag) {
    const int t = threadIdx.x;
    const int r = t / CH, c = t - r * CH;
    const int S = a.splits;
    bool ok = true;
    MergeState row;
    if constexpr (TAGGED) {
      const __amdgpu_buffer_rsrc_t tor = rsrc(a.tws, (uint32_t)((size_t)S * a.Hq * D * 8));
      const __amdgpu_buffer_rsrc_t tmr = rsrc(a.tws + (size_t)S * a.Hq * D * 2, (uint32_t)((size_t)S * a.Hq * 16));
      for (int s0 = r; s0 < S; s0 += RH * kBurst) {
        const int n = min(kBurst, (S - s0 + RH - 1) / RH);
        u32x4 ml[kBurst], lo[kBurst], hi[kBurst];
        bool have[kBurst];
#pragma unroll
        for (int u = 0; u < kBurst; ++u) have[u] = u >= n;
        for (unsigned spins = 0;;) {
#pragma unroll
          for (int u = 0; u < kBurst; ++u) {
            if (have[u]) continue;
            const int ss = s0 + RH * u;
            const uint32_t oo = (uint32_t)((((size_t)ss * a.Hq + h) * D + 4 * c) * 8);
            ml[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(tmr, (uint32_t)(((size_t)ss * a.Hq + h) * 16), 0, kAuxSc1));
            lo[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(tor, oo, 0, kAuxSc1));
            hi[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(tor, oo + 16, 0, kAuxSc1));
          }
          bool all = true;
#pragma unroll
          for (int u = 0; u < kBurst; ++u) {
            if (!have[u])
              have[u] = ml[u].y == tag && ml[u].w == tag && lo[u].y == tag && lo[u].w == tag && hi[u].y == tag && hi[u].w == tag;
            all = all && have[u];
          }
          if (all) break;
          if (!poll_step(spins, a.err)) {
            ok = false;
            break;
          }
        }
        if (!ok) break;
        float m[kBurst], lv[kBurst];
        f32x4 o[kBurst];
#pragma unroll
        for (int u = 0; u < kBurst; ++u) {
          // (whole-vector bit casts: a bit cast of one element of a vector compiles to element 0)
          const f32x4 mf = __builtin_bit_cast(f32x4, ml[u]);
          const f32x4 lf = __builtin_bit_cast(f32x4, lo[u]), hf = __builtin_bit_cast(f32x4, hi[u]);
          m[u] = mf.x;
          lv[u] = mf.z;
          o[u] = f32x4{lf.x, lf.z, hf.x, hf.z};
        }
        row.add(m, lv, o, n);
      }
    } else {
      load_row(a, h, r, c, row);
    }
    sm.o[r * CH + c] = row.acc;
    if (c == 0) {
      sm.w[r] = row.M;
      sm.ls[r] = row.l;
    }
    __syncthreads();
    if (t < CH) {
      MergeState tot;
#pragma unroll
      for (int rr = 0; rr < RH; ++rr) tot.fold(sm.w[rr], sm.ls[rr], sm.o[rr * CH + t]);
      const f32x4 out = tot.out();
      if constexpr (TAGGED) {
        const u32x4 vb = __builtin_bit_cast(u32x4, out);
        u32x4 p0, p1;
        p0.x = vb.x; p0.y = tag; p0.z = vb.y; p0.w = tag;
        p1.x = vb.z; p1.y = tag; p1.z = vb.w; p1.w = tag;
        const __amdgpu_buffer_rsrc_t tr = rsrc(a.tout, (uint32_t)(a.Hq * D * 8));
        const uint32_t off = (uint32_t)(((size_t)h * D + 4 * t) * 8);
        __builtin_amdgcn_raw_buffer_store_b128(p0, tr, off, 0, kAuxSc1);
        __builtin_amdgcn_raw_buffer_store_b128(p1, tr, off + 16, 0, kAuxSc1);
      } else {
        *reinterpret_cast<f32x4 *>(a.out + (size_t)h * D + 4 * t) = out;
      }
    }
    __syncthreads();  // (the next head reuses the LDS above)
    return ok;
  }

  // Row r of head h's merge from the plain partials of a finished phase: o at [s][head][D],
  // (m, l) at [s][head][2].
  __device__ __forceinline__ static void load_row(const AttnArgs &a, int h, int r, int c, MergeState &row) {
    const int S = a.splits;
    const __amdgpu_buffer_rsrc_t orr = rsrc(a.ws, (uint32_t)((size_t)S * a.Hq * D * 4));
    const __amdgpu_buffer_rsrc_t mlr = rsrc(a.ws + (size_t)S * a.Hq * D, (uint32_t)((size_t)S * a.Hq * 2 * 4));
    for (int s0 = r; s0 < S; s0 += RH * kBurst) {
      const int n = min(kBurst, (S - s0 + RH - 1) / RH);
      float m[kBurst], lv[kBurst];
      f32x4 o[kBurst];
#pragma unroll
      for (int u = 0; u < kBurst; ++u) {
        const int ss = s0 + RH * u;
        const bool in = u < n;
        const uint64_t v = __builtin_bit_cast(
            uint64_t, __builtin_amdgcn_raw_buffer_load_b64(mlr, in ? (uint32_t)(((size_t)ss * a.Hq + h) * 8) : 0x80000000u, 0, kAuxSc1));
        m[u] = __builtin_bit_cast(float, (uint32_t)v);
        lv[u] = __builtin_bit_cast(float, (uint32_t)(v >> 32));
        o[u] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(orr, in ? (uint32_t)((((size_t)ss * a.Hq + h) * D + 4 * c) * 4) : 0x80000000u, 0, kAuxSc1));
      }
      row.add(m, lv, o, n);
    }
  }

  // The merge of all G query heads of KV head j in the standalone kernels (the last split to
  // arrive), by the whole workgroup: the row states (head, row r, column c) of a share of the rows
  // at a time (as many as the LDS holds), every thread taking several with all their loads in
  // flight, go to LDS; thread (head, c) then folds them in row order, so the result is
  // merge_head's bit for bit.
  static constexpr int kMergeSlots = (int)(sizeof(AttnSmem<D, G, ROPE>::o) / sizeof(f32x4));
  static constexpr int merge_passes() {
    int p = 1;
    while (p < RH && (RH % p != 0 || G * (RH / p) * CH > kMergeSlots)) p *= 2;
    return p;
  }
  __device__ __forceinline__ void merge_heads_all(const AttnArgs &a, int j, AttnSmem<D, G, ROPE> &sm) {
    constexpr int NPASS = merge_passes();
    constexpr int HALF = RH / NPASS;                      // rows per pass
    constexpr int ITEMS = G * HALF * CH;                  // row states per pass
    constexpr int PER = (ITEMS + kAttnThreads - 1) / kAttnThreads;
    static_assert(ITEMS <= kMergeSlots, "a pass's row states fit");
    static_assert(G * RH <= kMaxMergeSplits, "the rows' (M, l) fit");
    static_assert(G * CH <= kAttnThreads, "one folding thread per head and column");
    const int t = threadIdx.x;
    const int fh = t / CH, fc = t - fh * CH;              // the folding thread's head and column
    MergeState tot;
    __syncthreads();  // (every wave is done with the partials in sm.o)
#pragma unroll
    for (int half = 0; half < NPASS; ++half) {
      MergeState row[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int i = t + kAttnThreads * u;
        if (i < ITEMS) {
          const int h = i / (HALF * CH), rem = i - h * (HALF * CH);
          const int r = half * HALF + rem / CH, c = rem - (rem / CH) * CH;
          load_row(a, j * G + h, r, c, row[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int i = t + kAttnThreads * u;
        if (i < ITEMS) {
          const int h = i / (HALF * CH), rem = i - h * (HALF * CH);
          const int r = half * HALF + rem / CH, c = rem - (rem / CH) * CH;
          sm.o[i] = row[u].acc;
          if (c == 0) {
            sm.w[h * RH + r] = row[u].M;
            sm.ls[h * RH + r] = row[u].l;
          }
        }
      }
      __syncthreads();
      if (t < G * CH) {
#pragma unroll
        for (int rr = 0; rr < HALF; ++rr) {
          const int r = half * HALF + rr;
          tot.fold(sm.w[fh * RH + r], sm.ls[fh * RH + r], sm.o[(fh * HALF + rr) * CH + fc]);
        }
      }
      __syncthreads();
    }
    if (t < G * CH) *reinterpret_cast<f32x4 *>(a.out + (size_t)(j * G + fh) * D + 4 * fc) = tot.out();
  }
};

template <int D, int G, int KVF, bool ROPE, bool SYNC>
__device__ __forceinline__ void attn_unit(const AttnArgs &a, int j, int s, AttnSmem<D, G, ROPE> &sm) {
  AttnUnit<D, G, KVF, ROPE, SYNC> u;
  u.start(a, j, s);
  u.finish(a, j, s, sm);
}


}  // namespace attn
}  // namespace qdec
