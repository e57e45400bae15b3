// Internal launch interface between the C ABI (abi.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coalesce {

enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum Act { ACT_NONE = 0, ACT_GELU = 1, ACT_SOFTPLUS = 2, ACT_RELU = 3 };

struct GemmParams {
  const void* A;
  const void* B;
  const void* bias;  // nullptr: no bias
  void* Y;
  int64_t lda, ldb, ldy;
  int M, N, K;
  int tiles_m, tiles_n, group_m;
};

// Each launcher picks its tile configuration, fills tiles_* and launches on
// `stream`; it returns the hipError_t of the launch.
hipError_t launch_gemm16(GemmParams p, DType in, DType out, int act, hipStream_t stream, int num_cus);
hipError_t launch_gemm32(GemmParams p, int act, hipStream_t stream, int num_cus);

struct MlpParams {
  const void* x;
  void* out;
  const void* W[8];
  int64_t ldx, ldo;
  int M;
  int num_tiles;  // row tiles (set by the launcher)
};
// Widths all equal to D (64 or 128), L layers (1..8 for 64, 1..4 for 128).
// num_workgroups <= 0: min(#CUs x occupancy, workgroups with work).
hipError_t launch_mlp(const MlpParams& p, int D, int L, int hidden_act, int num_workgroups, int num_cus,
                      hipStream_t stream);

hipError_t launch_bias_add(const void* X, int64_t ldx, const void* bias, void* Y, int64_t ldy, int M, int N,
                           DType xt, DType bt, DType yt, hipStream_t stream, int num_cus);
hipError_t launch_activation(const void* X, int64_t ldx, void* Y, int64_t ldy, int M, int N, DType dt, int act,
                             hipStream_t stream, int num_cus);
hipError_t launch_flush(const void* buf, size_t bytes, void* sink, hipStream_t stream, int num_cus);

}  // namespace coalesce
