// Measurement helper: the rate at which this board's matrix cores run the
// 16-bit GEMM's instruction when nothing else shares the time.
//
// The published dense bf16 peak assumes every SIMD issues a 16x16x32 MFMA
// every 16 cycles at the 2.4 GHz peak engine clock.  Under load the clock
// follows the board's power budget, and the matrix cores' draw depends on the
// operand bits.  This kernel gives the GEMM's figure a measured ceiling on the
// same board and in the same process: one 8-wave workgroup per CU (two waves
// per SIMD, the 256 x 256 GEMM tile's occupancy), every wave repeating the
// GEMM wave's 4 x 8 block of v_mfma_f32_16x16x32_bf16 on two sets of operand
// fragments held in registers (no memory traffic, no LDS reads, no copies),
// and recording its shader-clock (s_memtime) and constant-rate
// (s_memrealtime) counters around the loop, so the caller obtains both the
// sustained FLOP rate and the engine clock it ran at.
#include "common.hpp"

namespace coalesce {
namespace {

constexpr int RATE_WAVES = 8;
// Per wave and lane: 2 sets x (4 A + 8 B) fragments of 8 bf16.
constexpr int RATE_FRAGS = 24;

__global__ __launch_bounds__(RATE_WAVES * 64, 1) void matrix_rate_kernel(const i16x8* __restrict__ ops, int nsets,
                                                                          int iters, float* __restrict__ sink,
                                                                          unsigned long long* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * RATE_WAVES + (threadIdx.x >> 6);
  const i16x8* src = ops + (size_t)(wave % nsets) * RATE_FRAGS * 64 + lane;
  i16x8 a[2][4], b[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int m = 0; m < 4; ++m) a[s][m] = src[(s * 12 + m) * 64];
#pragma unroll
    for (int n = 0; n < 8; ++n) b[s][n] = src[(s * 12 + 4 + n) * 64];
  }
  f32x4 acc[4][8];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[m][n] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // The operands are in registers before the first counter read: each empty
  // asm consumes one fragment, so its load has completed there.
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int m = 0; m < 4; ++m) asm volatile("" ::"v"(a[s][m]));
#pragma unroll
    for (int n = 0; n < 8; ++n) asm volatile("" ::"v"(b[s][n]));
  }
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = mfma16x16x32(a[s][m], b[s][n], acc[m][n], __bf16());
  }
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);

  float sum = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 8; ++n) sum += (acc[m][n][0] + acc[m][n][1]) + (acc[m][n][2] + acc[m][n][3]);
  sink[(size_t)wave * 64 + lane] = sum;
  if (lane == 0) {
    clocks[2 * (size_t)wave] = t1 - t0;
    clocks[2 * (size_t)wave + 1] = r1 - r0;
  }
}

}  // namespace

int matrix_rate_waves(int num_cus) { return num_cus * RATE_WAVES; }

hipError_t launch_matrix_rate(const void* ops, int nsets, int iters, void* sink, void* clocks, hipStream_t stream,
                              int num_cus) {
  hipLaunchKernelGGL(matrix_rate_kernel, dim3(num_cus), dim3(RATE_WAVES * 64), 0, stream, (const i16x8*)ops, nsets,
                     iters, (float*)sink, (unsigned long long*)clocks);
  return hipGetLastError();
}

}  // namespace coalesce
