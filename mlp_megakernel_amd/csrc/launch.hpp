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
  int tiles_m, tiles_n;
  int group_m;        // tile rows per group of the tile order (0: the launcher's default)
  int grid_override;  // workgroups to launch (0: the launcher's default); persistent kernels walk the rest
  int variant;        // tile shape, 0 heuristic.  FP32: 1 = 128 x 128, 2 = 64 x 64, 3 = 32 x 32, 4 = 64 x 32;
                      // bf16 / fp16: 1 = 256 x 256, 2 = 128 x 128, 3 = 64 x 64
};

// Each launcher picks its tile configuration, fills tiles_* and launches on
// `stream`; it returns the hipError_t of the launch.
hipError_t launch_gemm16(GemmParams p, DType in, DType out, int act, hipStream_t stream, int num_cus);
hipError_t launch_gemm32(GemmParams p, int act, hipStream_t stream, int num_cus);
// The FP32 GEMM's tile shape for an M x N problem (the variant numbers of
// GemmParams::variant), and the number of K groups a variant splits K into
// (variants with the same count give the same bits).
int gemm32_variant(int64_t M, int64_t N, int num_cus);
int gemm32_kgroups(int variant);

struct MlpParams {
  const void* x;
  void* out;
  const void* W[8];
  float* acts[8];  // training forward: acts[l] receives h_{l+1} (fp32, M x dims[l+1], pitch lda), l = 0..L-2
  int dims[9];     // the chain's true widths (each a multiple of 8, at most the kernel width)
  int64_t ldx, ldo, lda;
  int M;
  int num_tiles;  // row tiles (set by the launcher)
};
// The chain runs at kernel width D (64 or 128), L layers (1..8 for 64, 1..4
// for 128).  pad = false: every width equals D; pad = true: p.dims holds the
// true widths (multiples of 8, at most D) and the kernel runs the chain with
// the weights zero-padded to D x D in LDS, x loads and out / activation stores
// masked to the true columns.  num_workgroups <= 0: a workgroup per #WAVES
// tiles, at least min(#tiles, #CUs), at most #CUs x occupancy.  store_acts: also write the hidden activations to
// p.acts (training forward).
// variant: the launch configuration (all give the same bits): 0 = the
// launcher's choice (mlp_default_variant), 1 = 32-row wave tiles with fewer
// waves per workgroup (inference only), 2 = 16-row wave tiles, 3 = 32-row
// wave tiles.
hipError_t launch_mlp(const MlpParams& p, int D, int L, int hidden_act, bool store_acts, bool pad, int variant,
                      int num_workgroups, int num_cus, hipStream_t stream);
// The launcher's choice of variant for a batch of M rows at kernel width D.
int mlp_default_variant(int D, int64_t M, bool store_acts, int num_cus);
// Variants 1 and 2 (mlp_alt.hip, mlp_small.hip).
hipError_t launch_mlp_alt(const MlpParams& p, int D, int L, int hidden_act, bool pad, int num_workgroups, int num_cus,
                          hipStream_t stream);
hipError_t launch_mlp_small(const MlpParams& p, int D, int L, int hidden_act, bool store_acts, bool pad,
                            int num_workgroups, int num_cus, hipStream_t stream);

// Chains for the layer-streaming megakernel (mlp_stream.hip): up to 16
// layers of widths up to 256, weights streamed through LDS chunk by chunk.
constexpr int kMaxStreamLayers = 16;
struct MlpStreamParams {
  const void* x;
  void* out;
  const void* W[kMaxStreamLayers];
  float* acts[kMaxStreamLayers];  // training forward: acts[l] = h_{l+1}, fp32, pitch lda
  int dims[kMaxStreamLayers + 1];
  int64_t ldx, ldo, lda;
  int M, L;
  int num_tiles;  // batches of wave tiles (set by the launcher)
};
// P: the width class (64, 128 or 256) the chain's widest layer fits.
hipError_t launch_mlp_stream(const MlpStreamParams& p, int P, int hidden_act, bool store_acts, int num_workgroups,
                             int num_cus, hipStream_t stream);

struct MlpBwdParams {
  const void* x;        // M x D fp16, pitch ldx
  const void* dout;     // M x D fp16, pitch ldd: dL/d(out)
  const void* W[8];     // D x D fp16, dense
  const float* acts[8]; // acts[l] = h_{l+1}, M x D fp32, pitch lda (l = 0..L-2)
  void* dx;             // M x D fp16, pitch ldq, or nullptr
  float* partial;       // grid x L x D x D fp32 per-workgroup weight-gradient sums
  float* dW[8];         // dims[l] x dims[l+1] fp32, dense: the reduced weight gradients
  int dims[9];          // the chain's true widths (multiples of 8, at most the kernel width D)
  int64_t ldx, ldd, lda, ldq;
  int M;
  int num_tiles;        // row tiles (set by the launcher)
};
// Weight-gradient workspace (bytes) the backward needs on a device with
// num_cus compute units.
size_t mlp_backward_workspace(int D, int L, int num_cus);
// Backward of the MLP chain: fills p.dW (and p.dx when set).  p.partial must
// hold mlp_backward_workspace(D, L, num_cus) bytes.
hipError_t launch_mlp_backward(MlpBwdParams p, int D, int L, int hidden_act, int num_cus, hipStream_t stream);
// The library's own device-resident scratch for the backward's partial sums
// (the no-allocation entry point): its size in bytes, and its address on the
// current device (looked up with hipGetSymbolAddress on the first call per
// device).
size_t mlp_backward_scratch_bytes();
hipError_t mlp_backward_scratch(void** ptr);

// Backward of a chain the layer-streaming forward runs (weights beyond LDS):
// one launch per layer, l = L-1 .. 0, each followed by the reduction of its
// per-workgroup weight-gradient sums.
struct MlpStreamBwdParams {
  const void* x;                         // M x dims[0] fp16 (ldx)
  const void* dout;                      // M x dims[L] fp16 (ldd)
  const void* W[kMaxStreamLayers];       // dims[l] x dims[l+1] fp16, dense
  const float* acts[kMaxStreamLayers];   // acts[l] = h_{l+1}, M x dims[l+1] fp32 (lda)
  void* dx;                              // M x dims[0] fp16 (ldq), or nullptr
  float* dW[kMaxStreamLayers];           // dims[l] x dims[l+1] fp32, dense
  int dims[kMaxStreamLayers + 1];
  int64_t ldx, ldd, lda, ldq;
  int M, L;
};
// Workspace (bytes) of launch_mlp_backward_stream: the per-workgroup partial
// sums of the largest layer and up to two M-row fp16 buffers for dz.
size_t mlp_backward_stream_workspace(const int* dims, int L, int64_t M, int num_cus);
hipError_t launch_mlp_backward_stream(const MlpStreamBwdParams& p, int P, int hidden_act, int num_cus,
                                      void* workspace, hipStream_t stream);

constexpr int kMaxWnLayers = 16;
struct WnParams {
  const void* v[kMaxWnLayers];  // fp16 din x dout, dense
  const void* g[kMaxWnLayers];  // fp16 dout
  void* W[kMaxWnLayers];        // fp16 din x dout (forward output)
  const float* dW[kMaxWnLayers];  // backward input
  float* dv[kMaxWnLayers];        // backward outputs
  float* dg[kMaxWnLayers];
  int din[kMaxWnLayers], dout[kMaxWnLayers];
  int L;
};
// Weight normalisation of p.L layers in one launch, and its backward.
hipError_t launch_weight_norm(const WnParams& p, hipStream_t stream);
hipError_t launch_weight_norm_backward(const WnParams& p, hipStream_t stream);

hipError_t launch_bias_add(const void* X, int64_t ldx, const void* bias, void* Y, int64_t ldy, int M, int N,
                           DType xt, DType bt, DType yt, hipStream_t stream, int num_cus);
hipError_t launch_activation(const void* X, int64_t ldx, void* Y, int64_t ldy, int M, int N, DType dt, int act,
                             hipStream_t stream, int num_cus);
hipError_t launch_flush(const void* buf, size_t bytes, void* sink, hipStream_t stream, int num_cus);
// Matrix-core rate probe: one 8-wave workgroup per CU, each wave `iters`
// rounds of 64 bf16 16x16x32 MFMAs on register operands; per wave two
// counter deltas (shader clock, constant-rate clock) into `clocks`.
int matrix_rate_waves(int num_cus);
hipError_t launch_matrix_rate(const void* ops, int nsets, int iters, void* sink, void* clocks, hipStream_t stream,
                              int num_cus);
// counter += number of 16-bit words that differ between two rows x row_bytes
// matrices (pitches in bytes; row_bytes even).
hipError_t launch_compare(const void* a, int64_t pitch_a, const void* b, int64_t pitch_b, int64_t rows,
                          int64_t row_bytes, unsigned int* counter, hipStream_t stream, int num_cus);

}  // namespace coalesce
