// C ABI of libcoalesce: argument validation on the host, tile/grid choice,
// and the launch on the caller's stream.  Nothing is launched unless every
// check passes; no device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/coalesce.h"
#include "launch.hpp"

using namespace coalesce;

namespace {

thread_local char g_last_error[512] = "";

coalesce_status fail(coalesce_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

coalesce_status ok() {
  g_last_error[0] = '\0';
  return COALESCE_OK;
}

coalesce_status device_fail(hipError_t e, const char* what) {
  return fail(COALESCE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
std::mutex g_props_mutex;
int g_cu_count[kMaxDevices] = {0};

// CU count of the current device, queried once per device.
coalesce_status current_cus(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(COALESCE_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_props_mutex);
  if (g_cu_count[dev] == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return device_fail(e, "hipDeviceGetAttribute");
    if (cus <= 0) return fail(COALESCE_ERR_DEVICE, "device reports %d compute units", cus);
    g_cu_count[dev] = cus;
  }
  *out = g_cu_count[dev];
  return COALESCE_OK;
}

bool valid_dtype(int d) { return d == COALESCE_F32 || d == COALESCE_F16 || d == COALESCE_BF16; }
bool valid_act(int a) {
  return a == COALESCE_ACT_NONE || a == COALESCE_ACT_GELU_ERF || a == COALESCE_ACT_SOFTPLUS || a == COALESCE_ACT_RELU;
}
int64_t dsize(int d) { return d == COALESCE_F32 ? 4 : 2; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
const int64_t kMaxExtent = (int64_t)INT32_MAX;

// Byte range [lo, hi) covered by a rows x cols matrix with leading dimension ld.
struct Range {
  uintptr_t lo, hi;
};
Range span(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t es) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  if (!p || rows <= 0 || cols <= 0) return {lo, lo};
  return {lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * es)};
}
bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

int act_code(coalesce_act a) {
  return a == COALESCE_ACT_GELU_ERF ? ACT_GELU
         : a == COALESCE_ACT_SOFTPLUS ? ACT_SOFTPLUS
         : a == COALESCE_ACT_RELU     ? ACT_RELU
                                      : ACT_NONE;
}

}  // namespace

namespace {

// A launch configuration the autotuner may choose (0 in a field: the
// launcher's own default).
struct TuneCfg {
  int grid = 0, group_m = 0, variant = 0;
};

// Tuned configurations, per device and problem key.  The public entry points
// consult it (a relaxed flag keeps the untuned path free of the lock).
std::mutex g_tune_mutex;
std::map<std::string, TuneCfg> g_tuned;
std::atomic<bool> g_tuned_any{false};

std::string gemm_key(int dev, int64_t M, int64_t N, int64_t K, int in, int out, int act, bool bias) {
  char b[160];
  snprintf(b, sizeof(b), "gemm:%d:%lld:%lld:%lld:%d:%d:%d:%d", dev, (long long)M, (long long)N, (long long)K, in, out,
           act, (int)bias);
  return b;
}

std::string mlp_key(int dev, const int64_t* dims, int L, int64_t M, int act) {
  std::string k = "mlp:" + std::to_string(dev) + ":" + std::to_string(M) + ":" + std::to_string(act) + ":";
  for (int l = 0; l <= L; ++l) k += std::to_string(dims[l]) + ",";
  return k;
}

bool tuned_lookup(const std::string& key, TuneCfg* cfg) {
  if (!g_tuned_any.load(std::memory_order_relaxed)) return false;
  std::lock_guard<std::mutex> lock(g_tune_mutex);
  auto it = g_tuned.find(key);
  if (it == g_tuned.end()) return false;
  *cfg = it->second;
  return true;
}

int current_device() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess ? dev : -1;
}

coalesce_status gemm_impl(const void* A, int64_t lda, const void* B, int64_t ldb, const void* bias, void* Y,
                          int64_t ldy, int64_t M, int64_t N, int64_t K, coalesce_dtype in_dtype,
                          coalesce_dtype out_dtype, coalesce_act act, void* stream, const TuneCfg* cfg) {
  if (M < 0 || N < 0 || K < 0)
    return fail(COALESCE_ERR_INVALID_ARGUMENT, "negative extent (M=%lld N=%lld K=%lld)", (long long)M, (long long)N,
                (long long)K);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(COALESCE_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (!valid_act(act)) return fail(COALESCE_ERR_INVALID_ARGUMENT, "unknown activation %d", (int)act);
  const bool combo_ok = (in_dtype == COALESCE_F32 && out_dtype == COALESCE_F32) ||
                        (in_dtype == COALESCE_BF16 && (out_dtype == COALESCE_BF16 || out_dtype == COALESCE_F32)) ||
                        (in_dtype == COALESCE_F16 && (out_dtype == COALESCE_F16 || out_dtype == COALESCE_F32));
  if (!combo_ok)
    return fail(COALESCE_ERR_UNSUPPORTED, "dtype combination in=%d out=%d not supported", (int)in_dtype,
                (int)out_dtype);
  if (M > kMaxExtent || N > kMaxExtent || K > kMaxExtent)
    return fail(COALESCE_ERR_UNSUPPORTED, "extents must be below 2^31");
  if (M == 0 || N == 0) return ok();
  const int64_t is = dsize(in_dtype), os = dsize(out_dtype);
  if (!Y) return fail(COALESCE_ERR_INVALID_ARGUMENT, "Y is NULL");
  if (ldy < N) return fail(COALESCE_ERR_INVALID_ARGUMENT, "ldy (%lld) < N (%lld)", (long long)ldy, (long long)N);
  if (K > 0) {
    if (!A || !B) return fail(COALESCE_ERR_INVALID_ARGUMENT, "A or B is NULL with K > 0");
    if (lda < K) return fail(COALESCE_ERR_INVALID_ARGUMENT, "lda (%lld) < K (%lld)", (long long)lda, (long long)K);
    if (ldb < N) return fail(COALESCE_ERR_INVALID_ARGUMENT, "ldb (%lld) < N (%lld)", (long long)ldb, (long long)N);
    if (!aligned16(A) || !aligned16(B)) return fail(COALESCE_ERR_UNSUPPORTED, "A and B must be 16-byte aligned");
    if ((lda * is) % 16 || (ldb * is) % 16)
      return fail(COALESCE_ERR_UNSUPPORTED, "lda and ldb must span a multiple of 16 bytes");
    // the 16-bit kernel addresses a 256-row A tile and a 64-row B slab with
    // 32-bit byte offsets
    if (is == 2 && (lda > (int64_t(1) << 23) || ldb > (int64_t(1) << 25)))
      return fail(COALESCE_ERR_UNSUPPORTED, "16-bit inputs need lda <= 2^23 and ldb <= 2^25");
  }
  if (!aligned16(Y) || (ldy * os) % 16)
    return fail(COALESCE_ERR_UNSUPPORTED, "Y must be 16-byte aligned with ldy spanning a multiple of 16 bytes");
  if (bias && !aligned16(bias)) return fail(COALESCE_ERR_UNSUPPORTED, "bias must be 16-byte aligned");
  const Range ry = span(Y, M, N, ldy, os);
  if ((K > 0 && (overlap(ry, span(A, M, K, lda, is)) || overlap(ry, span(B, K, N, ldb, is)))) ||
      overlap(ry, span(bias, 1, N, N, is)))
    return fail(COALESCE_ERR_INVALID_ARGUMENT, "Y overlaps an input");

  int cus = 0;
  coalesce_status s = current_cus(&cus);
  if (s != COALESCE_OK) return s;
  GemmParams p{};
  p.A = A;
  p.B = B;
  p.bias = bias;
  p.Y = Y;
  p.lda = lda;
  p.ldb = ldb;
  p.ldy = ldy;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  TuneCfg tc;
  if (cfg)
    tc = *cfg;
  else if (g_tuned_any.load(std::memory_order_relaxed))  // (no key is built while nothing is recorded)
    tuned_lookup(gemm_key(current_device(), M, N, K, in_dtype, out_dtype, act, bias != nullptr), &tc);
  p.grid_override = tc.grid;
  p.group_m = tc.group_m;
  p.variant = tc.variant;
  hipError_t e;
  if (in_dtype == COALESCE_F32)
    e = launch_gemm32(p, act_code(act), (hipStream_t)stream, cus);
  else
    e = launch_gemm16(p, in_dtype == COALESCE_BF16 ? DT_BF16 : DT_F16, out_dtype == COALESCE_F32 ? DT_F32 : (in_dtype == COALESCE_BF16 ? DT_BF16 : DT_F16),
                      act_code(act), (hipStream_t)stream, cus);
  if (e != hipSuccess) return device_fail(e, "GEMM launch");
  return ok();
}

}  // namespace

extern "C" {

coalesce_status coalesce_gemm_bias_act(const void* A, int64_t lda, const void* B, int64_t ldb, const void* bias,
                                       void* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                       coalesce_dtype in_dtype, coalesce_dtype out_dtype, coalesce_act act,
                                       void* stream) {
  return gemm_impl(A, lda, B, ldb, bias, Y, ldy, M, N, K, in_dtype, out_dtype, act, stream, nullptr);
}

}  // extern "C"

namespace {

// Shared checks of the MLP entry points: the chain's widths, depth, dtype,
// activation and weights.  Widths are multiples of 8 and at most 128; the
// chain runs at kernel width P = 64 if every width is at most 64, else 128
// (then *square says whether every width equals P).  Depth: P = 128 holds at
// most 4 layers of weights in LDS, P = 64 at most 8.
// A chain the MLP kernels run: L = 1..16 layers, fp16, widths multiples of
// 8 up to 256.  *P_out: the width class (64, 128 or 256) of its widest
// layer; *resident: all weights fit in LDS at once (widths up to 128 and at
// most 4 layers, or up to 64 and at most 8), so the resident megakernel
// (mlp_kernel.hpp, and the fused backward) runs it -- else the layer-streaming one.
coalesce_status check_mlp_chain(const void* const* W, const int64_t* dims, int32_t L, int64_t M,
                                coalesce_dtype dtype, coalesce_act hidden_act, int64_t* P_out, bool* square,
                                bool* resident) {
  if (L < 1) return fail(COALESCE_ERR_INVALID_ARGUMENT, "L must be at least 1 (got %d)", (int)L);
  if (!W || !dims) return fail(COALESCE_ERR_INVALID_ARGUMENT, "W or dims is NULL");
  if (M < 0) return fail(COALESCE_ERR_INVALID_ARGUMENT, "negative M");
  if (!valid_dtype(dtype)) return fail(COALESCE_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (!valid_act(hidden_act)) return fail(COALESCE_ERR_INVALID_ARGUMENT, "unknown activation");
  if (L > kMaxStreamLayers) return fail(COALESCE_ERR_UNSUPPORTED, "at most %d layers (got %d)", kMaxStreamLayers, (int)L);
  int64_t mx = 0;
  for (int l = 0; l <= L; ++l) {
    if (dims[l] <= 0) return fail(COALESCE_ERR_INVALID_ARGUMENT, "dims[%d] = %lld is not positive", l, (long long)dims[l]);
    if (dims[l] % 8 || dims[l] > 256)
      return fail(COALESCE_ERR_UNSUPPORTED, "MLP width %lld not supported (a multiple of 8, at most 256)",
                  (long long)dims[l]);
    if (dims[l] > mx) mx = dims[l];
  }
  if (dtype != COALESCE_F16) return fail(COALESCE_ERR_UNSUPPORTED, "the MLP megakernel takes fp16 only");
  if (hidden_act == COALESCE_ACT_GELU_ERF)
    return fail(COALESCE_ERR_UNSUPPORTED, "the MLP megakernel supports softplus, relu or no hidden activation");
  const int64_t P = mx <= 64 ? 64 : mx <= 128 ? 128 : 256;
  *resident = P == 64 ? L <= 8 : P == 128 ? L <= 4 : false;
  bool sq = true;
  for (int l = 0; l <= L; ++l) sq = sq && dims[l] == P;
  if (M > kMaxExtent - 256) return fail(COALESCE_ERR_UNSUPPORTED, "M must be below 2^31 - 256");
  for (int l = 0; l < L; ++l) {
    if (!W[l]) return fail(COALESCE_ERR_INVALID_ARGUMENT, "W[%d] is NULL", l);
    if (!aligned16(W[l])) return fail(COALESCE_ERR_UNSUPPORTED, "W[%d] must be 16-byte aligned", l);
  }
  *P_out = P;
  *square = sq;
  return COALESCE_OK;
}

// An fp16 row-major M x D operand: present, pitch at least D and at most
// 2^24 (16-row tiles are addressed with 32-bit byte offsets), 16-byte
// aligned rows.
coalesce_status check_rows(const void* t, int64_t ld, int64_t D, int64_t es, const char* name) {
  if (!t) return fail(COALESCE_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (ld < D) return fail(COALESCE_ERR_INVALID_ARGUMENT, "the pitch of %s is shorter than the row", name);
  if (ld > (int64_t(1) << 24)) return fail(COALESCE_ERR_UNSUPPORTED, "the pitch of %s must be at most 2^24", name);
  if (!aligned16(t) || (ld * es) % 16)
    return fail(COALESCE_ERR_UNSUPPORTED, "%s must be 16-byte aligned with a 16-byte row pitch", name);
  return COALESCE_OK;
}

// variant: the resident kernel's launch configuration (0 the launcher's
// choice, 1 32-row wave tiles with fewer waves (inference forward only), 2
// 16-row wave tiles, 3 32-row wave tiles; the same bits).  num_workgroups ==
// 0 and variant == 0 let a tuned record of this shape, if any, choose both.
coalesce_status mlp_forward_impl(const void* x, int64_t ldx, const void* const* W, const int64_t* dims, int32_t L,
                                 void* out, int64_t ldo, float* const* acts, int64_t lda, int64_t M,
                                 coalesce_dtype dtype, coalesce_act hidden_act, int64_t num_workgroups, int variant,
                                 bool train, bool use_cache, void* stream) {
  int64_t P = 0;
  bool square = true, resident = true;
  coalesce_status s = check_mlp_chain(W, dims, L, M, dtype, hidden_act, &P, &square, &resident);
  if (s != COALESCE_OK) return s;
  if (num_workgroups < 0) return fail(COALESCE_ERR_INVALID_ARGUMENT, "negative workgroup count");
  if (num_workgroups > (int64_t)INT32_MAX) return fail(COALESCE_ERR_UNSUPPORTED, "workgroup count too large");
  if (M == 0) return ok();
  const int64_t D = dims[0], O = dims[L];
  if ((s = check_rows(x, ldx, D, 2, "x")) != COALESCE_OK) return s;
  if ((s = check_rows(out, ldo, O, 2, "out")) != COALESCE_OK) return s;
  const Range ro = span(out, M, O, ldo, 2);
  if (overlap(ro, span(x, M, D, ldx, 2))) return fail(COALESCE_ERR_INVALID_ARGUMENT, "out overlaps x");
  MlpParams p{};
  MlpStreamParams q{};
  for (int l = 0; l < L; ++l) {
    if (overlap(ro, span(W[l], dims[l], dims[l + 1], dims[l + 1], 2)))
      return fail(COALESCE_ERR_INVALID_ARGUMENT, "out overlaps W[%d]", l);
    if (resident)
      p.W[l] = W[l];
    else
      q.W[l] = W[l];
  }
  for (int l = 0; l <= L; ++l) {
    if (resident)
      p.dims[l] = (int)dims[l];
    else
      q.dims[l] = (int)dims[l];
  }
  if (train && L > 1) {
    if (!acts) return fail(COALESCE_ERR_INVALID_ARGUMENT, "acts is NULL");
    for (int l = 0; l + 1 < L; ++l) {
      char name[16];
      snprintf(name, sizeof(name), "acts[%d]", l);
      const int64_t H = dims[l + 1];
      if ((s = check_rows(acts[l], lda, H, 4, name)) != COALESCE_OK) return s;
      const Range ra = span(acts[l], M, H, lda, 4);
      if (overlap(ra, span(x, M, D, ldx, 2)) || overlap(ra, ro))
        return fail(COALESCE_ERR_INVALID_ARGUMENT, "acts[%d] overlaps x or out", l);
      for (int j = 0; j < L; ++j)
        if (overlap(ra, span(W[j], dims[j], dims[j + 1], dims[j + 1], 2)))
          return fail(COALESCE_ERR_INVALID_ARGUMENT, "acts[%d] overlaps W[%d]", l, j);
      for (int j = 0; j < l; ++j)
        if (overlap(ra, span(acts[j], M, dims[j + 1], lda, 4)))
          return fail(COALESCE_ERR_INVALID_ARGUMENT, "acts[%d] overlaps acts[%d]", l, j);
      if (resident)
        p.acts[l] = acts[l];
      else
        q.acts[l] = acts[l];
    }
  }
  int cus = 0;
  s = current_cus(&cus);
  if (s != COALESCE_OK) return s;
  if (!resident) {
    q.x = x;
    q.out = out;
    q.ldx = ldx;
    q.ldo = ldo;
    q.lda = train ? lda : 0;
    q.M = (int)M;
    q.L = (int)L;
    if (num_workgroups == 0 && !train && use_cache && g_tuned_any.load(std::memory_order_relaxed)) {
      TuneCfg tc;
      if (tuned_lookup(mlp_key(current_device(), dims, L, M, hidden_act), &tc)) num_workgroups = tc.grid;
    }
    hipError_t e = launch_mlp_stream(q, (int)P, act_code(hidden_act), train && L > 1, (int)num_workgroups, cus,
                                     (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "MLP (layer-streaming) launch");
    return ok();
  }
  p.x = x;
  p.out = out;
  p.ldx = ldx;
  p.ldo = ldo;
  p.lda = train ? lda : 0;
  p.M = (int)M;
  if (num_workgroups == 0 && variant == 0 && !train && use_cache && g_tuned_any.load(std::memory_order_relaxed)) {
    TuneCfg tc;
    if (tuned_lookup(mlp_key(current_device(), dims, L, M, hidden_act), &tc)) {
      num_workgroups = tc.grid;
      variant = tc.variant;
    }
  }
  hipError_t e = launch_mlp(p, (int)P, (int)L, act_code(hidden_act), train && L > 1, !square, variant,
                            (int)num_workgroups, cus, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "MLP launch");
  return ok();
}

}  // namespace

extern "C" {

coalesce_status coalesce_mlp_forward_grid(const void* x, int64_t ldx, const void* const* W, const int64_t* dims,
                                          int32_t L, void* out, int64_t ldo, int64_t M, coalesce_dtype dtype,
                                          coalesce_act hidden_act, int64_t num_workgroups, void* stream) {
  return mlp_forward_impl(x, ldx, W, dims, L, out, ldo, nullptr, 0, M, dtype, hidden_act, num_workgroups, 0, false, true,
                          stream);
}

coalesce_status coalesce_mlp_forward_train(const void* x, int64_t ldx, const void* const* W, const int64_t* dims,
                                           int32_t L, void* out, int64_t ldo, float* const* acts, int64_t lda,
                                           int64_t M, coalesce_dtype dtype, coalesce_act hidden_act, void* stream) {
  return mlp_forward_impl(x, ldx, W, dims, L, out, ldo, acts, lda, M, dtype, hidden_act, 0, 0, true, false, stream);
}

// Workspace of the backward: the fused kernel's per-workgroup partial sums
// (chains whose weights fit in LDS), or the layer-by-layer kernels' partial
// sums of one layer plus the fp16 dz buffers of M rows.
size_t backward_workspace(const int64_t* dims, int L, int64_t M, int64_t P, bool resident, int cus) {
  if (resident) return mlp_backward_workspace((int)P, L, cus);
  int d[kMaxStreamLayers + 1];
  for (int l = 0; l <= L; ++l) d[l] = (int)dims[l];
  return mlp_backward_stream_workspace(d, L, M, cus);
}

size_t coalesce_mlp_backward_workspace_size(const int64_t* dims, int32_t L, int64_t M) {
  if (!dims || L < 1 || L > kMaxStreamLayers || M < 0 || M > kMaxExtent - 256) return 0;
  int64_t mx = 0;
  for (int l = 0; l <= L; ++l) {
    if (dims[l] <= 0 || dims[l] % 8 || dims[l] > 256) return 0;
    if (dims[l] > mx) mx = dims[l];
  }
  const int64_t P = mx <= 64 ? 64 : mx <= 128 ? 128 : 256;
  const bool resident = P == 64 ? L <= 8 : P == 128 ? L <= 4 : false;
  int cus = 0;
  if (current_cus(&cus) != COALESCE_OK) return 0;
  return backward_workspace(dims, L, M, P, resident, cus);
}

coalesce_status coalesce_mlp_backward(const void* x, int64_t ldx, const void* const* W, const int64_t* dims,
                                      int32_t L, const float* const* acts, int64_t lda, const void* dout,
                                      int64_t ldd, float* const* dW, void* dx, int64_t ldq, int64_t M,
                                      coalesce_dtype dtype, coalesce_act hidden_act, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  int64_t P = 0;
  bool square = true, resident = true;
  coalesce_status s = check_mlp_chain(W, dims, L, M, dtype, hidden_act, &P, &square, &resident);
  if (s != COALESCE_OK) return s;
  if (!dW) return fail(COALESCE_ERR_INVALID_ARGUMENT, "dW is NULL");
  const int64_t D = dims[0], O = dims[L];
  auto wspan = [&](const void* t, int l, int64_t es) { return span(t, dims[l], dims[l + 1], dims[l + 1], es); };
  for (int l = 0; l < L; ++l) {
    if (!dW[l]) return fail(COALESCE_ERR_INVALID_ARGUMENT, "dW[%d] is NULL", l);
    if (((uintptr_t)dW[l]) & 3u) return fail(COALESCE_ERR_UNSUPPORTED, "dW[%d] must be 4-byte aligned", l);
  }
  if (M > 0) {
    if ((s = check_rows(x, ldx, D, 2, "x")) != COALESCE_OK) return s;
    if ((s = check_rows(dout, ldd, O, 2, "dout")) != COALESCE_OK) return s;
    if (L > 1) {
      if (!acts) return fail(COALESCE_ERR_INVALID_ARGUMENT, "acts is NULL");
      for (int l = 0; l + 1 < L; ++l) {
        char name[16];
        snprintf(name, sizeof(name), "acts[%d]", l);
        if ((s = check_rows(acts[l], lda, dims[l + 1], 4, name)) != COALESCE_OK) return s;
      }
    }
    if (dx) {
      if ((s = check_rows(dx, ldq, D, 2, "dx")) != COALESCE_OK) return s;
      const Range rq = span(dx, M, D, ldq, 2);
      bool bad = overlap(rq, span(x, M, D, ldx, 2)) || overlap(rq, span(dout, M, O, ldd, 2));
      for (int l = 0; l < L; ++l) bad = bad || overlap(rq, wspan(W[l], l, 2)) || overlap(rq, wspan(dW[l], l, 4));
      for (int l = 0; l + 1 < L; ++l) bad = bad || overlap(rq, span(acts[l], M, dims[l + 1], lda, 4));
      if (bad) return fail(COALESCE_ERR_INVALID_ARGUMENT, "dx overlaps an input or a weight gradient");
    }
  }
  int cus = 0;
  s = current_cus(&cus);
  if (s != COALESCE_OK) return s;
  const size_t need = backward_workspace(dims, L, M, P, resident, cus);
  if (!workspace) return fail(COALESCE_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned16(workspace)) return fail(COALESCE_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(COALESCE_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                need);
  const Range rw = {(uintptr_t)workspace, (uintptr_t)workspace + need};
  for (int l = 0; l < L; ++l) {
    const Range rg = wspan(dW[l], l, 4);
    if (overlap(rg, rw)) return fail(COALESCE_ERR_INVALID_ARGUMENT, "dW[%d] overlaps the workspace", l);
    for (int j = 0; j < L; ++j)
      if ((j != l && overlap(rg, wspan(dW[j], j, 4))) || overlap(rg, wspan(W[j], j, 2)))
        return fail(COALESCE_ERR_INVALID_ARGUMENT, "dW[%d] overlaps another weight or gradient", l);
    if (overlap(rw, wspan(W[l], l, 2))) return fail(COALESCE_ERR_INVALID_ARGUMENT, "W[%d] overlaps the workspace", l);
  }
  if (M > 0) {
    bool bad = overlap(rw, span(x, M, D, ldx, 2)) || overlap(rw, span(dout, M, O, ldd, 2)) ||
               (dx && overlap(rw, span(dx, M, D, ldq, 2)));
    for (int l = 0; l + 1 < L; ++l) bad = bad || overlap(rw, span(acts[l], M, dims[l + 1], lda, 4));
    if (bad) return fail(COALESCE_ERR_INVALID_ARGUMENT, "the workspace overlaps x, dout, dx or an activation");
  }
  hipError_t e;
  if (resident) {
    MlpBwdParams p{};
    for (int l = 0; l < L; ++l) {
      p.W[l] = W[l];
      p.dW[l] = dW[l];
    }
    for (int l = 0; l <= L; ++l) p.dims[l] = (int)dims[l];
    for (int l = 0; M > 0 && l + 1 < L; ++l) p.acts[l] = acts[l];
    p.x = x;
    p.dout = dout;
    p.dx = M > 0 ? dx : nullptr;
    p.partial = (float*)workspace;
    p.ldx = ldx;
    p.ldd = ldd;
    p.lda = lda;
    p.ldq = ldq;
    p.M = (int)M;
    (void)square;
    e = launch_mlp_backward(p, (int)P, (int)L, act_code(hidden_act), cus, (hipStream_t)stream);
  } else {
    MlpStreamBwdParams q{};
    for (int l = 0; l < L; ++l) {
      q.W[l] = W[l];
      q.dW[l] = dW[l];
    }
    for (int l = 0; l <= L; ++l) q.dims[l] = (int)dims[l];
    for (int l = 0; M > 0 && l + 1 < L; ++l) q.acts[l] = acts[l];
    q.x = x;
    q.dout = dout;
    q.dx = M > 0 ? dx : nullptr;
    q.ldx = ldx;
    q.ldd = ldd;
    q.lda = lda;
    q.ldq = ldq;
    q.M = (int)M;
    q.L = L;
    e = launch_mlp_backward_stream(q, (int)P, act_code(hidden_act), cus, workspace, (hipStream_t)stream);
  }
  if (e != hipSuccess) return device_fail(e, "MLP backward launch");
  return ok();
}

coalesce_status coalesce_mlp_backward_noalloc(const void* x, int64_t ldx, const void* const* W, const int64_t* dims,
                                              int32_t L, const float* const* acts, int64_t lda, const void* dout,
                                              int64_t ldd, float* const* dW, void* dx, int64_t ldq, int64_t M,
                                              coalesce_dtype dtype, coalesce_act hidden_act, void* stream) {
  int64_t P = 0;
  bool square = true, resident = true;
  coalesce_status s = check_mlp_chain(W, dims, L, M, dtype, hidden_act, &P, &square, &resident);
  if (s != COALESCE_OK) return s;
  int cus = 0;
  if ((s = current_cus(&cus)) != COALESCE_OK) return s;
  const size_t need = backward_workspace(dims, L, M, P, resident, cus);
  const size_t have = mlp_backward_scratch_bytes();
  if (need > have)
    return fail(COALESCE_ERR_UNSUPPORTED,
                "this chain needs %zu bytes of workspace, more than the %zu bytes of the library's scratch", need,
                have);
  void* scratch = nullptr;
  hipError_t e = mlp_backward_scratch(&scratch);
  if (e != hipSuccess) return device_fail(e, "scratch address (hipGetSymbolAddress)");
  return coalesce_mlp_backward(x, ldx, W, dims, L, acts, lda, dout, ldd, dW, dx, ldq, M, dtype, hidden_act, scratch,
                               have, stream);
}

coalesce_status coalesce_mlp_forward(const void* x, int64_t ldx, const void* const* W, const int64_t* dims, int32_t L,
                                     void* out, int64_t ldo, int64_t M, coalesce_dtype dtype, coalesce_act hidden_act,
                                     void* stream) {
  return coalesce_mlp_forward_grid(x, ldx, W, dims, L, out, ldo, M, dtype, hidden_act, 0, stream);
}

// Shared checks of the weight-normalisation entry points: a chain of L
// (1..16) layers of positive widths, fp16, every pointer present.
static coalesce_status check_wn(const int64_t* dims, int32_t L, coalesce_dtype dtype, const void* const* a,
                                const char* an, const void* const* b, const char* bn, WnParams* p) {
  if (!dims) return fail(COALESCE_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (L < 1) return fail(COALESCE_ERR_INVALID_ARGUMENT, "L must be at least 1 (got %d)", (int)L);
  if (L > kMaxWnLayers) return fail(COALESCE_ERR_UNSUPPORTED, "at most %d layers per call", kMaxWnLayers);
  if (!valid_dtype(dtype)) return fail(COALESCE_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (dtype != COALESCE_F16) return fail(COALESCE_ERR_UNSUPPORTED, "weight normalisation takes fp16 v and g");
  for (int l = 0; l <= L; ++l)
    if (dims[l] <= 0) return fail(COALESCE_ERR_INVALID_ARGUMENT, "dims[%d] = %lld is not positive", l, (long long)dims[l]);
  for (int l = 0; l < L; ++l)
    if (dims[l] * dims[l + 1] > kMaxExtent || dims[l + 1] > 65535LL * 64)
      return fail(COALESCE_ERR_UNSUPPORTED, "layer %d is too large", l);
  if (!a || !b) return fail(COALESCE_ERR_INVALID_ARGUMENT, "%s or %s is NULL", an, bn);
  p->L = L;
  for (int l = 0; l < L; ++l) {
    if (!a[l]) return fail(COALESCE_ERR_INVALID_ARGUMENT, "%s[%d] is NULL", an, l);
    if (!b[l]) return fail(COALESCE_ERR_INVALID_ARGUMENT, "%s[%d] is NULL", bn, l);
    if ((reinterpret_cast<uintptr_t>(a[l]) | reinterpret_cast<uintptr_t>(b[l])) & 1u)
      return fail(COALESCE_ERR_UNSUPPORTED, "%s[%d] and %s[%d] must be 2-byte aligned", an, l, bn, l);
    p->din[l] = (int)dims[l];
    p->dout[l] = (int)dims[l + 1];
  }
  return COALESCE_OK;
}

static coalesce_status check_elementwise(const void* X, int64_t ldx, void* Y, int64_t ldy, int64_t M, int64_t N,
                                         int64_t es) {
  if (M < 0 || N < 0) return fail(COALESCE_ERR_INVALID_ARGUMENT, "negative extent");
  if (M > kMaxExtent || N > kMaxExtent) return fail(COALESCE_ERR_UNSUPPORTED, "extents must be below 2^31");
  if (M == 0 || N == 0) return COALESCE_OK;
  if (!X || !Y) return fail(COALESCE_ERR_INVALID_ARGUMENT, "X or Y is NULL");
  if (ldx < N || ldy < N) return fail(COALESCE_ERR_INVALID_ARGUMENT, "leading dimension shorter than the row");
  if (!aligned16(X) || !aligned16(Y) || (ldx * es) % 16 || (ldy * es) % 16)
    return fail(COALESCE_ERR_UNSUPPORTED, "X and Y must be 16-byte aligned with 16-byte row pitch");
  if (X != Y && overlap(span(X, M, N, ldx, es), span(Y, M, N, ldy, es)))
    return fail(COALESCE_ERR_INVALID_ARGUMENT, "X and Y overlap without being identical");
  if (X == Y && ldx != ldy) return fail(COALESCE_ERR_INVALID_ARGUMENT, "in-place call with different pitches");
  return COALESCE_OK;
}

coalesce_status coalesce_bias_add(const void* X, int64_t ldx, const void* bias, void* Y, int64_t ldy, int64_t M,
                                  int64_t N, coalesce_dtype x_dtype, coalesce_dtype bias_dtype, coalesce_dtype y_dtype,
                                  void* stream) {
  if (!valid_dtype(x_dtype) || !valid_dtype(bias_dtype) || !valid_dtype(y_dtype))
    return fail(COALESCE_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (x_dtype != bias_dtype || x_dtype != y_dtype)
    return fail(COALESCE_ERR_UNSUPPORTED, "bias_add needs one dtype for X, bias and Y");
  coalesce_status s = check_elementwise(X, ldx, Y, ldy, M, N, dsize(x_dtype));
  if (s != COALESCE_OK) return s;
  if (M == 0 || N == 0) return ok();
  if (!bias) return fail(COALESCE_ERR_INVALID_ARGUMENT, "bias is NULL");
  int cus = 0;
  s = current_cus(&cus);
  if (s != COALESCE_OK) return s;
  const DType dt = x_dtype == COALESCE_F32 ? DT_F32 : x_dtype == COALESCE_F16 ? DT_F16 : DT_BF16;
  hipError_t e = launch_bias_add(X, ldx, bias, Y, ldy, (int)M, (int)N, dt, dt, dt, (hipStream_t)stream, cus);
  if (e != hipSuccess) return device_fail(e, "bias_add launch");
  return ok();
}

coalesce_status coalesce_activation(const void* X, int64_t ldx, void* Y, int64_t ldy, int64_t M, int64_t N,
                                    coalesce_dtype dtype, coalesce_act act, void* stream) {
  if (!valid_dtype(dtype)) return fail(COALESCE_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (!valid_act(act)) return fail(COALESCE_ERR_INVALID_ARGUMENT, "unknown activation");
  coalesce_status s = check_elementwise(X, ldx, Y, ldy, M, N, dsize(dtype));
  if (s != COALESCE_OK) return s;
  if (M == 0 || N == 0) return ok();
  int cus = 0;
  s = current_cus(&cus);
  if (s != COALESCE_OK) return s;
  const DType dt = dtype == COALESCE_F32 ? DT_F32 : dtype == COALESCE_F16 ? DT_F16 : DT_BF16;
  hipError_t e = launch_activation(X, ldx, Y, ldy, (int)M, (int)N, dt, act_code(act), (hipStream_t)stream, cus);
  if (e != hipSuccess) return device_fail(e, "activation launch");
  return ok();
}

coalesce_status coalesce_flush_caches(const void* buf, size_t bytes, void* sink, void* stream) {
  if (bytes == 0) return ok();
  if (!buf || !sink) return fail(COALESCE_ERR_INVALID_ARGUMENT, "buf or sink is NULL");
  if (!aligned16(buf) || bytes % 16) return fail(COALESCE_ERR_UNSUPPORTED, "buf must be 16-byte aligned, bytes a multiple of 16");
  int cus = 0;
  coalesce_status s = current_cus(&cus);
  if (s != COALESCE_OK) return s;
  hipError_t e = launch_flush(buf, bytes, sink, (hipStream_t)stream, cus);
  if (e != hipSuccess) return device_fail(e, "flush launch");
  return ok();
}

coalesce_status coalesce_matrix_rate(const void* ops, int32_t nsets, int32_t iters, void* sink, void* clocks,
                                     int64_t max_waves, int32_t* waves, int64_t* wallclock_khz, void* stream) {
  if (!waves || !wallclock_khz) return fail(COALESCE_ERR_INVALID_ARGUMENT, "waves or wallclock_khz is NULL");
  int cus = 0;
  coalesce_status s = current_cus(&cus);
  if (s != COALESCE_OK) return s;
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return device_fail(e, "hipDeviceGetAttribute");
  *waves = matrix_rate_waves(cus);
  *wallclock_khz = khz;
  if (!ops || !sink || !clocks) return fail(COALESCE_ERR_INVALID_ARGUMENT, "ops, sink or clocks is NULL");
  if (!aligned16(ops)) return fail(COALESCE_ERR_UNSUPPORTED, "ops must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(sink) & 3u || reinterpret_cast<uintptr_t>(clocks) & 7u)
    return fail(COALESCE_ERR_UNSUPPORTED, "sink must be 4-byte and clocks 8-byte aligned");
  if (nsets <= 0 || iters <= 0) return fail(COALESCE_ERR_INVALID_ARGUMENT, "nsets and iters must be positive");
  if (max_waves < *waves) return fail(COALESCE_ERR_INVALID_ARGUMENT, "sink and clocks hold %lld waves, the launch has %d",
                                      (long long)max_waves, *waves);
  e = launch_matrix_rate(ops, nsets, iters, sink, clocks, (hipStream_t)stream, cus);
  if (e != hipSuccess) return device_fail(e, "matrix_rate launch");
  return ok();
}

coalesce_status coalesce_weight_norm(const void* const* v, const void* const* g, void* const* W, const int64_t* dims,
                                     int32_t L, coalesce_dtype dtype, void* stream) {
  WnParams p{};
  coalesce_status s = check_wn(dims, L, dtype, v, "v", g, "g", &p);
  if (s != COALESCE_OK) return s;
  if (!W) return fail(COALESCE_ERR_INVALID_ARGUMENT, "W is NULL");
  for (int l = 0; l < L; ++l) {
    if (!W[l]) return fail(COALESCE_ERR_INVALID_ARGUMENT, "W[%d] is NULL", l);
    if (reinterpret_cast<uintptr_t>(W[l]) & 1u) return fail(COALESCE_ERR_UNSUPPORTED, "W[%d] must be 2-byte aligned", l);
    const Range rw = span(W[l], dims[l], dims[l + 1], dims[l + 1], 2);
    for (int j = 0; j < L; ++j)
      if (overlap(rw, span(v[j], dims[j], dims[j + 1], dims[j + 1], 2)) || overlap(rw, span(g[j], 1, dims[j + 1], dims[j + 1], 2)) ||
          (j != l && overlap(rw, span(W[j], dims[j], dims[j + 1], dims[j + 1], 2))))
        return fail(COALESCE_ERR_INVALID_ARGUMENT, "W[%d] overlaps an input or another output", l);
    p.v[l] = v[l];
    p.g[l] = g[l];
    p.W[l] = W[l];
  }
  hipError_t e = launch_weight_norm(p, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "weight_norm launch");
  return ok();
}

coalesce_status coalesce_weight_norm_backward(const void* const* v, const void* const* g, const float* const* dW,
                                              float* const* dv, float* const* dg, const int64_t* dims, int32_t L,
                                              coalesce_dtype dtype, void* stream) {
  WnParams p{};
  coalesce_status s = check_wn(dims, L, dtype, v, "v", g, "g", &p);
  if (s != COALESCE_OK) return s;
  if (!dW || !dv || !dg) return fail(COALESCE_ERR_INVALID_ARGUMENT, "dW, dv or dg is NULL");
  for (int l = 0; l < L; ++l) {
    if (!dW[l] || !dv[l] || !dg[l]) return fail(COALESCE_ERR_INVALID_ARGUMENT, "dW, dv or dg[%d] is NULL", l);
    if ((reinterpret_cast<uintptr_t>(dW[l]) | reinterpret_cast<uintptr_t>(dv[l]) | reinterpret_cast<uintptr_t>(dg[l])) & 3u)
      return fail(COALESCE_ERR_UNSUPPORTED, "dW, dv and dg[%d] must be 4-byte aligned", l);
    const Range rv = span(dv[l], dims[l], dims[l + 1], dims[l + 1], 4), rg = span(dg[l], 1, dims[l + 1], dims[l + 1], 4);
    if (overlap(rv, rg)) return fail(COALESCE_ERR_INVALID_ARGUMENT, "dv[%d] overlaps dg[%d]", l, l);
    for (int j = 0; j < L; ++j) {
      const Range ins[3] = {span(v[j], dims[j], dims[j + 1], dims[j + 1], 2), span(g[j], 1, dims[j + 1], dims[j + 1], 2),
                            span(dW[j], dims[j], dims[j + 1], dims[j + 1], 4)};
      for (const Range& r : ins)
        if (overlap(rv, r) || overlap(rg, r))
          return fail(COALESCE_ERR_INVALID_ARGUMENT, "dv[%d] or dg[%d] overlaps an input", l, l);
      if (j != l && (overlap(rv, span(dv[j], dims[j], dims[j + 1], dims[j + 1], 4)) ||
                     overlap(rg, span(dg[j], 1, dims[j + 1], dims[j + 1], 4))))
        return fail(COALESCE_ERR_INVALID_ARGUMENT, "outputs of layers %d and %d overlap", l, j);
    }
    p.v[l] = v[l];
    p.g[l] = g[l];
    p.dW[l] = dW[l];
    p.dv[l] = dv[l];
    p.dg[l] = dg[l];
  }
  hipError_t e = launch_weight_norm_backward(p, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "weight_norm_backward launch");
  return ok();
}

}  // extern "C"

namespace {

// Time `iters` back-to-back launches of run() on the stream (after one
// untimed launch) and check the output against the reference with the
// compare kernel.  Synchronises the stream.
struct Trial {
  float us = 0.f;
  bool valid = false;
  coalesce_status status = COALESCE_OK;
};

template <typename Run>
Trial trial(Run run, int iters, hipStream_t st, const void* out, int64_t out_pitch_bytes, const void* ref,
            int64_t rows, int64_t row_bytes, unsigned int* counter, int cus) {
  Trial t;
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
    if (a) hipEventDestroy(a);
    t.status = fail(COALESCE_ERR_DEVICE, "hipEventCreate failed");
    return t;
  }
  t.status = run();
  if (t.status == COALESCE_OK) {
    hipEventRecord(a, st);
    for (int i = 0; i < iters && t.status == COALESCE_OK; ++i) t.status = run();
    hipEventRecord(b, st);
  }
  unsigned int diff = 1;
  if (t.status == COALESCE_OK) {
    hipError_t e = hipMemsetAsync(counter, 0, sizeof(unsigned int), st);
    if (e == hipSuccess) e = launch_compare(out, out_pitch_bytes, ref, row_bytes, rows, row_bytes, counter, st, cus);
    if (e == hipSuccess) e = hipMemcpyAsync(&diff, counter, sizeof(diff), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    if (e != hipSuccess) t.status = device_fail(e, "autotune timing");
    t.us = ms * 1e3f / (float)(iters > 0 ? iters : 1);
    t.valid = diff == 0;
  }
  hipEventDestroy(a);
  hipEventDestroy(b);
  return t;
}

// The autotuner's own arguments: iters in range, a workspace large enough
// for the reference copy of the output (rows x row_bytes, rounded up to 256
// bytes) and the counter, apart from every operand.
coalesce_status check_tune_args(int iters, const void* workspace, size_t workspace_bytes, int64_t rows,
                                int64_t row_bytes, const std::vector<Range>& operands) {
  if (iters < 1 || iters > 10000) return fail(COALESCE_ERR_INVALID_ARGUMENT, "iters must be in 1..10000");
  const size_t need = (((size_t)rows * (size_t)row_bytes + 255) & ~(size_t)255) + 256;
  if (!workspace) return fail(COALESCE_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned16(workspace)) return fail(COALESCE_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(COALESCE_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  const Range rw = {(uintptr_t)workspace, (uintptr_t)workspace + need};
  for (const Range& r : operands)
    if (overlap(rw, r)) return fail(COALESCE_ERR_INVALID_ARGUMENT, "the workspace overlaps an operand");
  return COALESCE_OK;
}

// Run the default, keep its output as the reference, try every candidate
// (the default first), keep the fastest whose output equals the reference
// bit for bit.
template <typename Run>
coalesce_status tune(const std::vector<TuneCfg>& cands, Run run, int iters, void* stream, void* out,
                     int64_t out_pitch_bytes, int64_t rows, int64_t row_bytes, void* workspace, size_t workspace_bytes,
                     const std::vector<Range>& operands, const std::string& key, coalesce_tune_report* report) {
  const size_t ref_bytes = (size_t)rows * (size_t)row_bytes;
  coalesce_status s = check_tune_args(iters, workspace, workspace_bytes, rows, row_bytes, operands);
  if (s != COALESCE_OK) return s;
  int cus = 0;
  s = current_cus(&cus);
  if (s != COALESCE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  char* ref = (char*)workspace;
  unsigned int* counter = (unsigned int*)(ref + ((ref_bytes + 255) & ~(size_t)255));
  const TuneCfg dflt{};
  if ((s = run(dflt)) != COALESCE_OK) return s;
  hipError_t e = hipMemcpy2DAsync(ref, (size_t)row_bytes, out, (size_t)out_pitch_bytes, (size_t)row_bytes, (size_t)rows,
                                  hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return device_fail(e, "autotune reference copy");
  // Two passes over the candidates, the second in reverse order, keeping
  // each one's faster time: the clocks drift while the GPU warms up, and a
  // single pass would favour whichever candidates come late.  A candidate
  // is valid only if both of its runs reproduced the reference.
  const size_t n = cands.size();
  std::vector<float> us(n, 0.f), worst(n, 0.f);
  std::vector<char> ok_run(n, 1);
  for (int pass = 0; pass < 2; ++pass)
    for (size_t j = 0; j < n; ++j) {
      const size_t i = pass == 0 ? j : n - 1 - j;
      const TuneCfg c = cands[i];
      Trial t = trial([&]() { return run(c); }, iters, st, out, out_pitch_bytes, ref, rows, row_bytes, counter, cus);
      if (t.status != COALESCE_OK) return t.status;
      us[i] = pass == 0 ? t.us : std::min(us[i], t.us);
      worst[i] = pass == 0 ? t.us : std::max(worst[i], t.us);
      ok_run[i] = ok_run[i] && t.valid;
    }
  const float default_us = us[0];
  const bool default_valid = ok_run[0] != 0;
  int valid = 0;
  for (size_t i = 0; i < n; ++i) valid += ok_run[i] ? 1 : 0;
  if (valid == 0) return fail(COALESCE_ERR_DEVICE, "no configuration reproduced the default's output");
  // A candidate replaces the default only if both of its passes beat the
  // default's faster pass by more than 1 %: on launches of a few
  // microseconds a single fast pass is often noise (measured: a 5 x 64
  // chain on 16384 rows once tuned to a configuration 7 % slower).  Among
  // those, the fastest.  Without a valid default, the fastest valid one.
  TuneCfg best = dflt;
  float best_us = default_us;
  bool have = default_valid;
  for (size_t i = 1; i < n; ++i) {
    if (!ok_run[i]) continue;
    const bool beats = default_valid ? worst[i] < 0.99f * default_us : true;
    if (beats && (!have || us[i] < best_us)) {
      best = cands[i];
      best_us = us[i];
      have = true;
    }
  }
  {
    std::lock_guard<std::mutex> lock(g_tune_mutex);
    g_tuned[key] = best;
    g_tuned_any.store(true);
  }
  if ((s = run(best)) != COALESCE_OK) return s;
  if (report) {
    report->candidates = (int32_t)cands.size();
    report->valid = valid;
    report->default_us = default_us;
    report->best_us = best_us;
    report->grid = best.grid;
    report->group_m = best.group_m;
    report->variant = best.variant;
  }
  return ok();
}

void add_unique(std::vector<TuneCfg>& v, TuneCfg c) {
  for (const TuneCfg& x : v)
    if (x.grid == c.grid && x.group_m == c.group_m && x.variant == c.variant) return;
  v.push_back(c);
}

}  // namespace

extern "C" {

coalesce_status coalesce_autotune_gemm_bias_act(const void* A, int64_t lda, const void* B, int64_t ldb,
                                                const void* bias, void* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                                coalesce_dtype in_dtype, coalesce_dtype out_dtype, coalesce_act act,
                                                int32_t iters, void* workspace, size_t workspace_bytes,
                                                coalesce_tune_report* report, void* stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(COALESCE_ERR_INVALID_ARGUMENT, "unknown dtype");
  const int64_t is = dsize(in_dtype), os = dsize(out_dtype);
  std::vector<Range> operands;
  const bool work = M > 0 && N > 0 && M <= kMaxExtent && N <= kMaxExtent;
  if (work) {
    operands = {span(Y, M, N, ldy, os), span(bias, 1, N, N, is)};
    if (K > 0) {
      operands.push_back(span(A, M, K, lda, is));
      operands.push_back(span(B, K, N, ldb, is));
    }
    coalesce_status s = check_tune_args(iters, workspace, workspace_bytes, M, N * os, operands);
    if (s != COALESCE_OK) return s;
  }
  // the entry point's own checks (and a first launch) through the untuned path
  const TuneCfg dflt{};
  coalesce_status s = gemm_impl(A, lda, B, ldb, bias, Y, ldy, M, N, K, in_dtype, out_dtype, act, stream, &dflt);
  if (s != COALESCE_OK) return s;
  if (!work) return ok();
  int cus = 0;
  if ((s = current_cus(&cus)) != COALESCE_OK) return s;
  std::vector<TuneCfg> cands;
  cands.push_back(dflt);
  if (in_dtype == COALESCE_F32) {
    // the tile shapes that split K into as many groups as the default's
    // (the others add the partial sums in another order: other bits)
    const int kg = gemm32_kgroups(gemm32_variant(M, N, cus));
    for (int variant : {1, 2, 3, 4})
      if (gemm32_kgroups(variant) == kg)
        for (int gm : {4, 8, 16}) add_unique(cands, TuneCfg{0, gm, variant});
  } else {
    // every tile shape (1 = 256 x 256, one workgroup per CU; 2 = 128 x 128,
    // two; 3 = 64 x 64, four), each with persistent grids of all, half and
    // three quarters of its workgroup slots, or one workgroup per tile
    for (int variant : {1, 2, 3}) {
      const int64_t bt = variant == 1 ? 256 : variant == 2 ? 128 : 64;
      const int64_t slots = (int64_t)cus * (variant == 1 ? 1 : variant == 2 ? 2 : 4);
      const int64_t tiles = ((M + bt - 1) / bt) * ((N + bt - 1) / bt);
      std::vector<int64_t> grids = {0, slots / 2, (3 * slots) / 4};
      if (tiles <= 4 * slots) grids.push_back(tiles);
      for (int64_t g : grids)
        for (int gm : {4, 8, 16})
          if (g >= 0 && g <= tiles) add_unique(cands, TuneCfg{(int)g, gm, variant});
    }
  }
  const std::string key = gemm_key(current_device(), M, N, K, in_dtype, out_dtype, act, bias != nullptr);
  return tune(
      cands,
      [&](const TuneCfg& c) {
        return gemm_impl(A, lda, B, ldb, bias, Y, ldy, M, N, K, in_dtype, out_dtype, act, stream, &c);
      },
      iters, stream, Y, ldy * os, M, N * os, workspace, workspace_bytes, operands, key, report);
}

coalesce_status coalesce_autotune_mlp_forward(const void* x, int64_t ldx, const void* const* W, const int64_t* dims,
                                              int32_t L, void* out, int64_t ldo, int64_t M, coalesce_dtype dtype,
                                              coalesce_act hidden_act, int32_t iters, void* workspace,
                                              size_t workspace_bytes, coalesce_tune_report* report, void* stream) {
  int64_t P = 0;
  bool square = true, resident = true;
  coalesce_status s = check_mlp_chain(W, dims, L, M, dtype, hidden_act, &P, &square, &resident);
  if (s != COALESCE_OK) return s;
  std::vector<Range> operands = {span(x, M, dims[0], ldx, 2), span(out, M, dims[L], ldo, 2)};
  for (int l = 0; l < L; ++l) operands.push_back(span(W[l], dims[l], dims[l + 1], dims[l + 1], 2));
  if (M > 0 && (s = check_tune_args(iters, workspace, workspace_bytes, M, dims[L] * 2, operands)) != COALESCE_OK)
    return s;
  s = mlp_forward_impl(x, ldx, W, dims, L, out, ldo, nullptr, 0, M, dtype, hidden_act, 0, 0, false, false, stream);
  if (s != COALESCE_OK) return s;
  if (M == 0) return ok();
  int cus = 0;
  if ((s = current_cus(&cus)) != COALESCE_OK) return s;
  // the compiled launch configurations of the resident kernel (variant 0:
  // the launcher's choice, 1: 32-row wave tiles with fewer waves and more
  // registers each, 2: 16-row wave tiles, 3: 32-row wave tiles), each with
  // its occupancy-derived grid and fixed grids around one workgroup per CU;
  // the layer-streaming kernel has one configuration (grids only)
  std::vector<TuneCfg> cands;
  cands.push_back(TuneCfg{});
  for (int v : resident ? std::vector<int>{0, 1, 2, 3} : std::vector<int>{0})
    for (int g : {0, cus / 4, cus / 2, cus, 2 * cus, 3 * cus}) add_unique(cands, TuneCfg{g, 0, v});
  const std::string key = mlp_key(current_device(), dims, L, M, hidden_act);
  return tune(
      cands,
      [&](const TuneCfg& c) {
        return mlp_forward_impl(x, ldx, W, dims, L, out, ldo, nullptr, 0, M, dtype, hidden_act, c.grid, c.variant,
                                false, false, stream);
      },
      iters, stream, out, ldo * 2, M, dims[L] * 2, workspace, workspace_bytes, operands, key, report);
}

coalesce_status coalesce_autotune_clear(void) {
  std::lock_guard<std::mutex> lock(g_tune_mutex);
  g_tuned.clear();
  g_tuned_any.store(false);
  return ok();
}

int32_t coalesce_device_cu_count(void) {
  int cus = 0;
  if (current_cus(&cus) != COALESCE_OK) return -1;
  return cus;
}

const char* coalesce_status_string(coalesce_status s) {
  switch (s) {
    case COALESCE_OK: return "COALESCE_OK";
    case COALESCE_ERR_INVALID_ARGUMENT: return "COALESCE_ERR_INVALID_ARGUMENT";
    case COALESCE_ERR_UNSUPPORTED: return "COALESCE_ERR_UNSUPPORTED";
    case COALESCE_ERR_DEVICE: return "COALESCE_ERR_DEVICE";
  }
  return "COALESCE_ERR_UNKNOWN";
}

const char* coalesce_last_error(void) { return g_last_error; }

int32_t coalesce_version(void) { return 100; }

}  // extern "C"
