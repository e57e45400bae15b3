// Weight normalisation of every layer of a chain in one launch ("MLP
// Megakernel" README, "Key ideas": W = g v / ||v|| for all weight matrices in
// a single kernel, so that per-layer launch overhead does not dominate at
// small sizes), and its backward, also one launch.
//
//   W_l[k][n] = g_l[n] v_l[k][n] / ||v_l[:, n]||        (norm per output unit)
//   dg_l[n]    = <dW_l[:, n], v_l[:, n]> / ||v_l[:, n]||
//   dv_l[k][n] = g_l[n] / ||v_l[:, n]|| (dW_l[k][n] - v_l[k][n] <dW_l[:, n], v_l[:, n]> / ||v_l[:, n]||^2)
//
// The matrices are a few to a few hundred KB, so what costs is the launch,
// not the bytes: the kernel is one memory round trip deep.  Grid (column
// blocks, layers): workgroup (c, l) owns the 64 output units 64 c .. 64 c + 63
// of layer l; its 1024 threads are 64 columns x 16 row slices (a thread reads
// d_in / 16 rows, loads issued back to back), so each wave reads one 128-byte
// run (64 fp16) per row.  The slices' partial sums (fp32, each element's
// square exact in fp32) meet in LDS and are added in slice order: repeated
// calls give the same bits.  A column of zeros gives 0 x g / 0 = NaN, as the
// formula does.
#include "common.hpp"
#include "launch.hpp"

namespace coalesce {
namespace {

constexpr int WN_COLS = 64, WN_SLICES = 16;

__device__ __forceinline__ float ld16(const _Float16* p, size_t i) { return (float)p[i]; }

__global__ __launch_bounds__(WN_COLS* WN_SLICES) void weight_norm_kernel(WnParams p) {
  __shared__ float part[WN_SLICES][WN_COLS];
  const int l = blockIdx.y;
  const int din = p.din[l], dout = p.dout[l];
  const int c = threadIdx.x % WN_COLS, sl = threadIdx.x / WN_COLS;
  const int n = blockIdx.x * WN_COLS + c;
  const _Float16* v = (const _Float16*)p.v[l];
  float ss = 0.0f;
  if (n < dout)
#pragma unroll 4
    for (int k = sl; k < din; k += WN_SLICES) {
      const float x = ld16(v, (size_t)k * dout + n);
      ss = __builtin_fmaf(x, x, ss);
    }
  part[sl][c] = ss;
  __syncthreads();
  if (n >= dout) return;
  float tot = part[0][c];
#pragma unroll
  for (int i = 1; i < WN_SLICES; ++i) tot += part[i][c];
  const float scale = ld16((const _Float16*)p.g[l], n) / __builtin_sqrtf(tot);
  _Float16* W = (_Float16*)p.W[l];
  for (int k = sl; k < din; k += WN_SLICES) W[(size_t)k * dout + n] = (_Float16)(ld16(v, (size_t)k * dout + n) * scale);
}

__global__ __launch_bounds__(WN_COLS* WN_SLICES) void weight_norm_backward_kernel(WnParams p) {
  __shared__ float pss[WN_SLICES][WN_COLS], pdot[WN_SLICES][WN_COLS];
  const int l = blockIdx.y;
  const int din = p.din[l], dout = p.dout[l];
  const int c = threadIdx.x % WN_COLS, sl = threadIdx.x / WN_COLS;
  const int n = blockIdx.x * WN_COLS + c;
  const _Float16* v = (const _Float16*)p.v[l];
  const float* dW = p.dW[l];
  float ss = 0.0f, dot = 0.0f;
  if (n < dout)
#pragma unroll 4
    for (int k = sl; k < din; k += WN_SLICES) {
      const size_t i = (size_t)k * dout + n;
      const float x = ld16(v, i);
      ss = __builtin_fmaf(x, x, ss);
      dot = __builtin_fmaf(x, dW[i], dot);
    }
  pss[sl][c] = ss;
  pdot[sl][c] = dot;
  __syncthreads();
  if (n >= dout) return;
  float tss = pss[0][c], tdot = pdot[0][c];
#pragma unroll
  for (int i = 1; i < WN_SLICES; ++i) {
    tss += pss[i][c];
    tdot += pdot[i][c];
  }
  const float nrm = __builtin_sqrtf(tss);
  if (sl == 0) p.dg[l][n] = tdot / nrm;
  const float a = ld16((const _Float16*)p.g[l], n) / nrm;
  const float b = tdot / tss;
  float* dv = p.dv[l];
  for (int k = sl; k < din; k += WN_SLICES) {
    const size_t i = (size_t)k * dout + n;
    dv[i] = a * (dW[i] - ld16(v, i) * b);
  }
}

dim3 wn_grid(const WnParams& p) {
  int cb = 1;
  for (int l = 0; l < p.L; ++l) {
    const int b = (p.dout[l] + WN_COLS - 1) / WN_COLS;
    if (b > cb) cb = b;
  }
  return dim3(cb, p.L);
}

}  // namespace

hipError_t launch_weight_norm(const WnParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(weight_norm_kernel, wn_grid(p), dim3(WN_COLS * WN_SLICES), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_weight_norm_backward(const WnParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(weight_norm_backward_kernel, wn_grid(p), dim3(WN_COLS * WN_SLICES), 0, stream, p);
  return hipGetLastError();
}

}  // namespace coalesce
