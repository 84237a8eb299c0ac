// C-ABI entry points of libqdec: host-side argument checks, then kernel launches.
// Every check happens before the first HIP call, so a rejected call leaves the device untouched.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "qdec_batch.h"

namespace qdec {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

qdec_status check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return QDEC_EHIP;
  }
  return QDEC_OK;
}

static bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Scratch of qdec_gemv_q4_noalloc: the layout of a GEMV workspace (arrival counters, then split-K
// partial sums) in a static device array, one copy per GPU for the life of the process.  Host code
// never passes the array's name to a kernel (on the host it is a stand-in, not a device address):
// it uses the address hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = kCounterBytes + 512 * 1024;  // 768 KiB: up to 2048 split units
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_dev[kMaxDevices];

// Device address of this GPU's scratch, looked up once per device with that device current.
static qdec_status scratch_address(void **out, void *stream, const char *name) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("%s: hipGetDevice: %s", name, hipGetErrorString(e));
    return QDEC_EHIP;
  }
  QDEC_REQUIRE(dev >= 0 && dev < kMaxDevices, QDEC_EUNSUPPORTED, "%s: device %d is beyond the %d devices supported",
               name, dev, kMaxDevices);
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) {
      set_error("%s: hipStreamGetDevice: %s", name, hipGetErrorString(e));
      return QDEC_EHIP;
    }
    QDEC_REQUIRE(sdev == dev, QDEC_EINVAL, "%s: the stream belongs to device %d, the current device is %d", name,
                 sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      set_error("%s: hipGetSymbolAddress(scratch) on device %d: %s", name, dev, hipGetErrorString(e));
      return QDEC_EHIP;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return QDEC_OK;
}

// Zeroes the first `lines` arrival counters (one per 128-byte line).  A kernel, not a memset, so
// that a captured graph replays it correctly.
__global__ void clear_counter_lines(unsigned *counters, int lines) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < lines) counters[(size_t)i * kLine] = 0u;
}

}  // namespace qdec

using namespace qdec;

extern "C" {

const char *qdec_last_error(void) { return g_err; }
const char *qdec_version(void) { return "qdec 0.1 (gfx950)"; }

size_t qdec_packed_weight_bytes(int wfmt, int N, int K) {
  if (N < 1 || K < 1) return 0;
  const size_t npad = (size_t)((N + kTile - 1) / kTile) * kTile;
  if (wfmt == QDEC_W_Q8_ROW) return npad * (size_t)K;
  if (wfmt == QDEC_W_Q4_G_ZP8) return npad * (size_t)K / 2;
  return 0;
}

size_t qdec_packed_scale_bytes(int wfmt, int N, int K, int group) {
  if (N < 1 || K < 1) return 0;
  const size_t npad = (size_t)((N + kTile - 1) / kTile) * kTile;
  if (wfmt == QDEC_W_Q8_ROW) return npad * sizeof(float);
  if (wfmt == QDEC_W_Q4_G_ZP8 && group > 0 && K % group == 0) return npad * (size_t)(K / group) * 2;
  return 0;
}

qdec_status qdec_pack_q8(const int8_t *W, const float *scale, int N, int K, void *Wp, float *Sp,
                         void *stream) {
  QDEC_REQUIRE(W && scale && Wp && Sp, QDEC_EINVAL, "qdec_pack_q8: null pointer");
  QDEC_REQUIRE(N >= 1 && K >= 16 && K % 16 == 0, QDEC_EINVAL,
               "qdec_pack_q8: need N >= 1 and K a positive multiple of 16 (N=%d K=%d)", N, K);
  QDEC_REQUIRE(aligned(W, 16) && aligned(Wp, 16) && aligned(Sp, 4) && aligned(scale, 4), QDEC_EINVAL,
               "qdec_pack_q8: W and Wp must be 16-byte aligned");
  if (launch_pack_q8(W, scale, N, K, reinterpret_cast<uint8_t *>(Wp), Sp, (hipStream_t)stream) !=
      hipSuccess)
    return check_launch("qdec_pack_q8");
  return QDEC_OK;
}

qdec_status qdec_pack_q4(const uint8_t *W, const uint16_t *scale, int N, int K, int group, void *Wp,
                         uint16_t *Sp, void *stream) {
  QDEC_REQUIRE(W && scale && Wp && Sp, QDEC_EINVAL, "qdec_pack_q4: null pointer");
  QDEC_REQUIRE(group >= 32 && group <= 4096 && (group & (group - 1)) == 0, QDEC_EUNSUPPORTED,
               "qdec_pack_q4: group must be 32 times a power of two (got %d)", group);
  QDEC_REQUIRE(N >= 1 && K >= group && K % group == 0, QDEC_EINVAL,
               "qdec_pack_q4: need N >= 1 and K a multiple of group (N=%d K=%d group=%d)", N, K, group);
  QDEC_REQUIRE(aligned(W, 16) && aligned(Wp, 16) && aligned(Sp, 2) && aligned(scale, 2), QDEC_EINVAL,
               "qdec_pack_q4: W and Wp must be 16-byte aligned");
  if (launch_pack_q4(W, scale, N, K, group, reinterpret_cast<uint8_t *>(Wp), Sp,
                     (hipStream_t)stream) != hipSuccess)
    return check_launch("qdec_pack_q4");
  return QDEC_OK;
}

size_t qdec_gemv_workspace_bytes(int wfmt, int N, int K) {
  if (N < 1 || K < 1 || (wfmt != QDEC_W_Q8_ROW && wfmt != QDEC_W_Q4_G_ZP8)) return 0;
  return gemv_workspace_bytes(wfmt, N, K);
}

static qdec_status gemv_check(int wfmt, const void *Wp, const void *Sp, int group, const float *x, const float *y,
                              int N, int K, const char *name) {
  QDEC_REQUIRE(Wp && Sp && x && y, QDEC_EINVAL, "%s: null pointer", name);
  QDEC_REQUIRE(N >= 1 && K >= 1, QDEC_EINVAL, "%s: N and K must be >= 1 (N=%d K=%d)", name, N, K);
  if (wfmt == QDEC_W_Q8_ROW) {
    QDEC_REQUIRE(K % 16 == 0, QDEC_EINVAL, "%s: K must be a multiple of 16 (K=%d)", name, K);
  } else {
    QDEC_REQUIRE(group >= 32 && group <= 4096 && (group & (group - 1)) == 0, QDEC_EUNSUPPORTED,
                 "%s: group must be 32 times a power of two (got %d)", name, group);
    QDEC_REQUIRE(K % group == 0, QDEC_EINVAL, "%s: K must be a multiple of group (K=%d group=%d)",
                 name, K, group);
  }
  QDEC_REQUIRE(aligned(Wp, 16) && aligned(x, 16) && aligned(y, 4), QDEC_EINVAL,
               "%s: packed weights and x must be 16-byte aligned", name);
  QDEC_REQUIRE(x != y && !(x < y + N && y < x + K), QDEC_EINVAL, "%s: x must not overlap y", name);
  return QDEC_OK;
}

static qdec_status gemv_launch(int wfmt, const void *Wp, const void *Sp, int group, const float *x,
                               const float *bias, const float *residual, float *y, int N, int K,
                               const GemvPlan &p, void *ws, void *stream, const char *name) {
  GemvArgs a{};
  a.W = reinterpret_cast<const uint8_t *>(Wp);
  a.S = Sp;
  a.x = x;
  a.bias = bias;
  a.residual = residual;
  a.y = y;
  a.N = N;
  a.K = K;
  a.group = group;
  a.epi = EPI_STORE;
  gemv_bind_workspace(a, p, ws);
  if (launch_gemv(wfmt, a, p, (hipStream_t)stream) != hipSuccess) return check_launch(name);
  return QDEC_OK;
}

static qdec_status gemv_common(int wfmt, const void *Wp, const void *Sp, int group, const float *x,
                               const float *bias, const float *residual, float *y, int N, int K,
                               void *ws, size_t ws_bytes, void *stream, const char *name) {
  const qdec_status c = gemv_check(wfmt, Wp, Sp, group, x, y, N, K, name);
  if (c != QDEC_OK) return c;
  const bool split = ws != nullptr;
  if (split) {
    QDEC_REQUIRE(aligned(ws, 256), QDEC_EINVAL, "%s: workspace must be 256-byte aligned", name);
    QDEC_REQUIRE(ws_bytes >= gemv_workspace_bytes(wfmt, N, K), QDEC_EINVAL,
                 "%s: workspace too small (%zu < %zu bytes)", name, ws_bytes,
                 gemv_workspace_bytes(wfmt, N, K));
  }
  return gemv_launch(wfmt, Wp, Sp, group, x, bias, residual, y, N, K, gemv_plan(wfmt, N, K, split), ws, stream,
                     name);
}

qdec_status qdec_gemv_q8(const void *Wp, const float *Sp, const float *x, const float *bias,
                         const float *residual, float *y, int N, int K, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return gemv_common(QDEC_W_Q8_ROW, Wp, Sp, 0, x, bias, residual, y, N, K, workspace,
                     workspace_bytes, stream, "qdec_gemv_q8");
}

qdec_status qdec_gemv_q4(const void *Wp, const uint16_t *Sp, int group, const float *x,
                         const float *bias, const float *residual, float *y, int N, int K,
                         void *workspace, size_t workspace_bytes, void *stream) {
  return gemv_common(QDEC_W_Q4_G_ZP8, Wp, Sp, group, x, bias, residual, y, N, K, workspace,
                     workspace_bytes, stream, "qdec_gemv_q4");
}

qdec_status qdec_gemv_q4_noalloc(const void *Wp, const uint16_t *Sp, int group, const float *x, const float *bias,
                                 const float *residual, float *y, int N, int K, void *stream) {
  const char *name = "qdec_gemv_q4_noalloc";
  const qdec_status c = gemv_check(QDEC_W_Q4_G_ZP8, Wp, Sp, group, x, y, N, K, name);
  if (c != QDEC_OK) return c;
  const size_t need = gemv_workspace_bytes(QDEC_W_Q4_G_ZP8, N, K);
  QDEC_REQUIRE(need <= kNoAllocScratchBytes, QDEC_EINVAL,
               "%s: N=%d K=%d needs %zu bytes of scratch, more than the library's static %zu bytes "
               "(use qdec_gemv_q4 with a workspace)",
               name, N, K, need, kNoAllocScratchBytes);
  void *ws = nullptr;
  const qdec_status sa = scratch_address(&ws, stream, name);
  if (sa != QDEC_OK) return sa;
  const GemvPlan p = gemv_plan(QDEC_W_Q4_G_ZP8, N, K, true);
  if (p.ks > 1) {  // the counters a split launch uses start at zero whatever an earlier call left
    hipLaunchKernelGGL(clear_counter_lines, dim3((p.tiles + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<unsigned *>(ws), p.tiles);
    const qdec_status lc = check_launch(name);
    if (lc != QDEC_OK) return lc;
  }
  return gemv_launch(QDEC_W_Q4_G_ZP8, Wp, Sp, group, x, bias, residual, y, N, K, p, ws, stream, name);
}

static bool pow2_group(int group) { return group >= 32 && group <= 4096 && (group & (group - 1)) == 0; }

qdec_status qdec_quantize_act_i8(const float *x, int K, int group, int8_t *q, float *sx, void *stream) {
  const char *nm = "qdec_quantize_act_i8";
  QDEC_REQUIRE(x && q && sx, QDEC_EINVAL, "%s: null pointer", nm);
  QDEC_REQUIRE(pow2_group(group), QDEC_EUNSUPPORTED, "%s: group must be 32 times a power of two (got %d)", nm, group);
  QDEC_REQUIRE(K >= group && K % group == 0, QDEC_EINVAL, "%s: K must be a positive multiple of group (K=%d group=%d)",
               nm, K, group);
  const char *xb = reinterpret_cast<const char *>(x), *qb = reinterpret_cast<const char *>(q);
  QDEC_REQUIRE(!(qb < xb + (size_t)K * 4 && xb < qb + K), QDEC_EINVAL, "%s: q must not overlap x", nm);
  if (launch_quantize_act_i8(x, K, group, q, sx, (hipStream_t)stream) != hipSuccess) return check_launch(nm);
  return QDEC_OK;
}

static qdec_status gemv_a8_common(int wfmt, const void *Wp, const void *Sp, int group, const int8_t *q,
                                  const float *sx, const float *bias, const float *residual, float *y, int N,
                                  int K, void *ws, size_t ws_bytes, void *stream, const char *name) {
  QDEC_REQUIRE(Wp && Sp && q && sx && y, QDEC_EINVAL, "%s: null pointer", name);
  QDEC_REQUIRE(N >= 1 && K >= 1, QDEC_EINVAL, "%s: N and K must be >= 1 (N=%d K=%d)", name, N, K);
  QDEC_REQUIRE(pow2_group(group), QDEC_EUNSUPPORTED, "%s: group must be 32 times a power of two (got %d)", name,
               group);
  QDEC_REQUIRE(K % group == 0, QDEC_EINVAL, "%s: K must be a multiple of group (K=%d group=%d)", name, K, group);
  QDEC_REQUIRE(aligned(Wp, 16) && aligned(q, 16) && aligned(sx, 4) && aligned(y, 4), QDEC_EINVAL,
               "%s: packed weights and q must be 16-byte aligned", name);
  if (ws) {
    QDEC_REQUIRE(aligned(ws, 256), QDEC_EINVAL, "%s: workspace must be 256-byte aligned", name);
    QDEC_REQUIRE(ws_bytes >= gemv_workspace_bytes(wfmt, N, K), QDEC_EINVAL, "%s: workspace too small (%zu < %zu bytes)",
                 name, ws_bytes, gemv_workspace_bytes(wfmt, N, K));
  }
  if (launch_gemv_a8(wfmt, reinterpret_cast<const uint8_t *>(Wp), Sp, q, sx, group, bias, residual, y, N, K, ws,
                     (hipStream_t)stream) != hipSuccess)
    return check_launch(name);
  return QDEC_OK;
}

qdec_status qdec_gemv_q8_a8(const void *Wp, const float *Sp, const int8_t *q, const float *sx, int group,
                            const float *bias, const float *residual, float *y, int N, int K, void *workspace,
                            size_t workspace_bytes, void *stream) {
  return gemv_a8_common(QDEC_W_Q8_ROW, Wp, Sp, group, q, sx, bias, residual, y, N, K, workspace, workspace_bytes,
                        stream, "qdec_gemv_q8_a8");
}

qdec_status qdec_gemv_q4_a8(const void *Wp, const uint16_t *Sp, int group, const int8_t *q, const float *sx,
                            const float *bias, const float *residual, float *y, int N, int K, void *workspace,
                            size_t workspace_bytes, void *stream) {
  return gemv_a8_common(QDEC_W_Q4_G_ZP8, Wp, Sp, group, q, sx, bias, residual, y, N, K, workspace, workspace_bytes,
                        stream, "qdec_gemv_q4_a8");
}

size_t qdec_gemm_workspace_bytes(int wfmt, int N, int K, int nb) {
  if (N < 1 || K < 1 || nb < 1 || nb > 8 || (wfmt != QDEC_W_Q8_ROW && wfmt != QDEC_W_Q4_G_ZP8)) return 0;
  return gemm_b_workspace_bytes(wfmt, N, K, gemm_b_columns(nb));
}

static qdec_status gemm_common(int wfmt, const void *Wp, const void *Sp, int group, const float *X, int ldx, int nb,
                               const float *bias, const float *residual, float *Y, int ldy, int N, int K, void *ws,
                               size_t ws_bytes, void *stream, const char *name) {
  QDEC_REQUIRE(Wp && Sp && X && Y, QDEC_EINVAL, "%s: null pointer", name);
  QDEC_REQUIRE(N >= 1 && K >= 1 && nb >= 1 && nb <= 8, QDEC_EINVAL, "%s: need N, K >= 1 and nb in [1, 8] (N=%d K=%d nb=%d)",
               name, N, K, nb);
  if (wfmt == QDEC_W_Q8_ROW) {
    QDEC_REQUIRE(K % 16 == 0, QDEC_EINVAL, "%s: K must be a multiple of 16 (K=%d)", name, K);
  } else {
    QDEC_REQUIRE(group >= 32 && group <= 4096 && (group & (group - 1)) == 0, QDEC_EUNSUPPORTED,
                 "%s: group must be 32 times a power of two (got %d)", name, group);
    QDEC_REQUIRE(K % group == 0, QDEC_EINVAL, "%s: K must be a multiple of group (K=%d group=%d)", name, K, group);
  }
  QDEC_REQUIRE(ldx >= K && ldx % 4 == 0 && ldy >= N, QDEC_EINVAL, "%s: need ldx >= K, ldx %% 4 == 0, ldy >= N", name);
  QDEC_REQUIRE(aligned(Wp, 16) && aligned(X, 16) && aligned(Y, 4), QDEC_EINVAL,
               "%s: packed weights and X must be 16-byte aligned", name);
  const char *xb = reinterpret_cast<const char *>(X), *yb = reinterpret_cast<const char *>(Y);
  const size_t xn = ((size_t)(nb - 1) * ldx + K) * 4, yn = ((size_t)(nb - 1) * ldy + N) * 4;
  QDEC_REQUIRE(!(xb < yb + yn && yb < xb + xn), QDEC_EINVAL, "%s: X must not overlap Y", name);
  if (ws) {
    QDEC_REQUIRE(aligned(ws, 256), QDEC_EINVAL, "%s: workspace must be 256-byte aligned", name);
    QDEC_REQUIRE(ws_bytes >= gemm_b_workspace_bytes(wfmt, N, K, gemm_b_columns(nb)), QDEC_EINVAL,
                 "%s: workspace too small", name);
  }
  GemmBArgs a{};
  a.W = reinterpret_cast<const uint8_t *>(Wp);
  a.S = Sp;
  a.X = X;
  a.ldx = ldx;
  a.bias = bias;
  a.residual = residual;
  a.Y = Y;
  a.ldy = ldy;
  a.N = N;
  a.K = K;
  a.group = group;
  a.nb = nb;
  a.nb_max = gemm_b_columns(nb);
  a.epi = EPI_STORE;
  if (launch_gemm_b(wfmt, a, ws, (hipStream_t)stream) != hipSuccess) return check_launch(name);
  return QDEC_OK;
}

qdec_status qdec_gemm_q8(const void *Wp, const float *Sp, const float *X, int ldx, int nb, const float *bias,
                         const float *residual, float *Y, int ldy, int N, int K, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return gemm_common(QDEC_W_Q8_ROW, Wp, Sp, 0, X, ldx, nb, bias, residual, Y, ldy, N, K, workspace, workspace_bytes,
                     stream, "qdec_gemm_q8");
}

qdec_status qdec_gemm_q4(const void *Wp, const uint16_t *Sp, int group, const float *X, int ldx, int nb,
                         const float *bias, const float *residual, float *Y, int ldy, int N, int K, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return gemm_common(QDEC_W_Q4_G_ZP8, Wp, Sp, group, X, ldx, nb, bias, residual, Y, ldy, N, K, workspace,
                     workspace_bytes, stream, "qdec_gemm_q4");
}

qdec_status qdec_gemm_mfma(int wfmt, const void *Wp, const void *Sp, int group, const uint16_t *X16, const uint16_t *X16lo,
                           int ldx, int M, const float *bias, const float *residual, float *Y, int ldy, int N, int K,
                           void *stream) {
  const char *nm = "qdec_gemm_mfma";
  QDEC_REQUIRE(Wp && Sp && X16 && Y, QDEC_EINVAL, "%s: null pointer", nm);
  QDEC_REQUIRE(wfmt == QDEC_W_Q8_ROW || wfmt == QDEC_W_Q4_G_ZP8, QDEC_EUNSUPPORTED, "%s: unknown weight format %d", nm,
               wfmt);
  QDEC_REQUIRE(M >= 1 && N >= 1 && K >= 32 && K % 32 == 0, QDEC_EINVAL, "%s: need M, N >= 1 and K a multiple of 32 (K=%d)",
               nm, K);
  if (wfmt == QDEC_W_Q4_G_ZP8)
    QDEC_REQUIRE(group >= 32 && group <= 4096 && (group & (group - 1)) == 0 && K % group == 0, QDEC_EUNSUPPORTED,
                 "%s: group must be 32 times a power of two dividing K (got %d)", nm, group);
  QDEC_REQUIRE(ldx >= K && ldx % 8 == 0 && ldy >= N, QDEC_EINVAL, "%s: need ldx >= K, ldx %% 8 == 0, ldy >= N", nm);
  QDEC_REQUIRE(aligned(Wp, 16) && aligned(X16, 16) && aligned(X16lo, 16) && aligned(Y, 4), QDEC_EINVAL,
               "%s: packed weights and X16 must be 16-byte aligned", nm);
  GemmPArgs a{};
  a.W = reinterpret_cast<const uint8_t *>(Wp);
  a.S = Sp;
  a.X = X16;
  a.Xl = X16lo;
  a.ldx = ldx;
  a.bias = bias;
  a.residual = residual;
  a.Y = Y;
  a.ldy = ldy;
  a.M = M;
  a.N = N;
  a.K = K;
  a.group = group;
  a.epi = EPI_STORE;
  if (launch_gemm_p(wfmt, a, (hipStream_t)stream) != hipSuccess) return check_launch(nm);
  return QDEC_OK;
}

size_t qdec_sample_workspace_bytes(void) { return sample_workspace_bytes(); }

qdec_status qdec_sample(const float *logits, int V, float temperature, int top_k, float top_p, uint64_t seed,
                        const int32_t *step, int32_t *token, void *workspace, size_t workspace_bytes, void *stream) {
  const char *nm = "qdec_sample";
  QDEC_REQUIRE(logits && token && workspace, QDEC_EINVAL, "%s: null pointer", nm);
  QDEC_REQUIRE(V >= 1, QDEC_EINVAL, "%s: V must be >= 1 (V=%d)", nm, V);
  QDEC_REQUIRE(!std::isnan(temperature), QDEC_EINVAL, "%s: temperature is NaN", nm);
  QDEC_REQUIRE(top_p > 0.f && top_p <= 1.f, QDEC_EINVAL, "%s: top_p must be in (0, 1] (got %g)", nm, (double)top_p);
  QDEC_REQUIRE(top_k >= 0, QDEC_EINVAL, "%s: top_k must be >= 0 (got %d)", nm, top_k);
  if (temperature > 0.f) {
    QDEC_REQUIRE(top_k <= kSampleMaxTopK || top_k >= V, QDEC_EUNSUPPORTED, "%s: top_k above %d is not supported (got %d)",
                 nm, kSampleMaxTopK, top_k);
    QDEC_REQUIRE(top_p >= 1.f || (top_k >= 1 && top_k <= kSampleMaxTopK), QDEC_EUNSUPPORTED,
                 "%s: top_p < 1 needs 1 <= top_k <= %d (got top_k=%d)", nm, kSampleMaxTopK, top_k);
  }
  QDEC_REQUIRE(aligned(workspace, 256), QDEC_EINVAL, "%s: workspace must be 256-byte aligned", nm);
  QDEC_REQUIRE(workspace_bytes >= sample_workspace_bytes(), QDEC_EINVAL, "%s: workspace too small (%zu < %zu bytes)",
               nm, workspace_bytes, sample_workspace_bytes());
  if (launch_sample(logits, V, temperature, top_k, top_p, seed, step, token, nullptr, nullptr, nullptr, 0, workspace,
                    (hipStream_t)stream) != hipSuccess)
    return check_launch(nm);
  return QDEC_OK;
}

qdec_status qdec_rmsnorm_rope(const float *x, const float *gamma, float *y, int rows, int dim,
                              float eps, float rope_base, const int32_t *pos, void *stream) {
  QDEC_REQUIRE(x && y, QDEC_EINVAL, "qdec_rmsnorm_rope: null pointer");
  QDEC_REQUIRE(rows >= 1 && dim >= 2 && dim <= 256 && dim % 2 == 0, QDEC_EINVAL,
               "qdec_rmsnorm_rope: need rows >= 1 and even dim in [2, 256] (rows=%d dim=%d)", rows,
               dim);
  QDEC_REQUIRE(!(rope_base > 0.f) || pos, QDEC_EINVAL, "qdec_rmsnorm_rope: RoPE needs pos");
  QDEC_REQUIRE(!gamma || (eps >= 0.f && std::isfinite(eps)), QDEC_EINVAL,
               "qdec_rmsnorm_rope: eps must be finite and >= 0");
  if (launch_rmsnorm_rope(x, gamma, y, rows, dim, eps, rope_base, pos, (hipStream_t)stream) !=
      hipSuccess)
    return check_launch("qdec_rmsnorm_rope");
  return QDEC_OK;
}

qdec_status qdec_swiglu(const float *gate, const float *up, float *out, int n, void *stream) {
  QDEC_REQUIRE(gate && up && out, QDEC_EINVAL, "qdec_swiglu: null pointer");
  QDEC_REQUIRE(n >= 1, QDEC_EINVAL, "qdec_swiglu: n must be >= 1 (n=%d)", n);
  if (launch_swiglu(gate, up, out, n, (hipStream_t)stream) != hipSuccess) return check_launch("qdec_swiglu");
  return QDEC_OK;
}

qdec_status qdec_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  QDEC_REQUIRE(src && sink, QDEC_EINVAL, "qdec_stream_read: null pointer");
  QDEC_REQUIRE(bytes >= 16 && bytes % 16 == 0 && aligned(src, 16), QDEC_EINVAL,
               "qdec_stream_read: bytes must be a positive multiple of 16 and src 16-byte aligned");
  if (launch_stream_read(src, bytes, sink, (hipStream_t)stream) != hipSuccess) return check_launch("qdec_stream_read");
  return QDEC_OK;
}

qdec_status qdec_argmax(const float *logits, int n, int32_t *token, void *stream) {
  QDEC_REQUIRE(logits && token, QDEC_EINVAL, "qdec_argmax: null pointer");
  QDEC_REQUIRE(n >= 1, QDEC_EINVAL, "qdec_argmax: n must be >= 1 (n=%d)", n);
  if (launch_argmax_finish(logits, n, token, nullptr, nullptr, nullptr, 0, (hipStream_t)stream) !=
      hipSuccess)
    return check_launch("qdec_argmax");
  return QDEC_OK;
}

size_t qdec_attn_workspace_bytes(int n_heads, int head_dim, int num_splits) {
  if (n_heads < 1 || head_dim < 1 || num_splits < 1) return 0;
  return attn_workspace_bytes(n_heads, head_dim, num_splits);
}

qdec_status qdec_attn_decode_paged(const float *q, const float *k_new, const float *v_new,
                                   void *k_pool, void *v_pool, int kv_fmt, const int32_t *page_table,
                                   int n_pages, int page_size, const int32_t *pos, int n_heads,
                                   int n_kv_heads, int head_dim, float sm_scale, int num_splits,
                                   void *workspace, size_t workspace_bytes, float *out, void *stream) {
  const char *nm = "qdec_attn_decode_paged";
  QDEC_REQUIRE(q && k_pool && v_pool && page_table && pos && workspace && out, QDEC_EINVAL,
               "%s: null pointer", nm);
  QDEC_REQUIRE((k_new == nullptr) == (v_new == nullptr), QDEC_EINVAL,
               "%s: k_new and v_new must both be given or both be NULL", nm);
  QDEC_REQUIRE(kv_fmt == QDEC_KV_F32 || kv_fmt == QDEC_KV_BF16, QDEC_EUNSUPPORTED,
               "%s: unknown kv_fmt %d", nm, kv_fmt);
  QDEC_REQUIRE(page_size == QDEC_PAGE_SIZE, QDEC_EUNSUPPORTED, "%s: page_size must be 16 (got %d)", nm,
               page_size);
  QDEC_REQUIRE(n_heads >= 1 && n_kv_heads >= 1 && n_heads % n_kv_heads == 0, QDEC_EINVAL,
               "%s: n_heads must be a positive multiple of n_kv_heads (%d, %d)", nm, n_heads, n_kv_heads);
  QDEC_REQUIRE(n_heads / n_kv_heads <= 8, QDEC_EUNSUPPORTED,
               "%s: at most 8 query heads per KV head (got %d)", nm, n_heads / n_kv_heads);
  QDEC_REQUIRE(head_dim == 64 || head_dim == 128, QDEC_EUNSUPPORTED,
               "%s: head_dim must be 64 or 128 (got %d)", nm, head_dim);
  QDEC_REQUIRE(num_splits >= 1 && num_splits <= kMaxMergeSplits, QDEC_EINVAL, "%s: num_splits in [1, %d]", nm,
               kMaxMergeSplits);
  QDEC_REQUIRE(n_kv_heads <= (int)(kAttnCounterBytes / 128), QDEC_EUNSUPPORTED, "%s: at most %d KV heads", nm,
               (int)(kAttnCounterBytes / 128));
  QDEC_REQUIRE(n_pages >= 1, QDEC_EINVAL, "%s: n_pages must be >= 1", nm);
  QDEC_REQUIRE(kv_pool_fits(n_pages, n_kv_heads, head_dim, kv_fmt), QDEC_EUNSUPPORTED,
               "%s: a KV pool of %d pages x %d heads x 16 x %d must stay below 4 GiB", nm, n_pages, n_kv_heads, head_dim);
  QDEC_REQUIRE(std::isfinite(sm_scale), QDEC_EINVAL, "%s: sm_scale must be finite", nm);
  QDEC_REQUIRE(workspace_bytes >= attn_workspace_bytes(n_heads, head_dim, num_splits), QDEC_EINVAL,
               "%s: workspace too small", nm);
  QDEC_REQUIRE(aligned(k_pool, 16) && aligned(v_pool, 16) && aligned(q, 16) && aligned(workspace, 256),
               QDEC_EINVAL, "%s: q and pools must be 16-byte, workspace 256-byte aligned", nm);
  hipStream_t st = (hipStream_t)stream;
  if (k_new) {
    if (launch_kv_append(k_new, v_new, k_pool, v_pool, kv_fmt, page_table, n_pages, pos, n_kv_heads,
                         head_dim, st) != hipSuccess)
      return check_launch(nm);
  }
  AttnArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.kv_fmt = kv_fmt;
  a.page_table = page_table;
  a.n_pages = n_pages;
  a.pos = pos;
  a.Hq = n_heads;
  a.Hkv = n_kv_heads;
  a.D = head_dim;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.splits = num_splits;
  a.counters = reinterpret_cast<unsigned *>(workspace);
  a.ws = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + kAttnCounterBytes);
  a.out = out;
  if (launch_attention(a, st) != hipSuccess) return check_launch(nm);
  return QDEC_OK;
}

}  // extern "C"
