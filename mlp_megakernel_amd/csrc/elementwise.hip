// Elementwise kernels of the unfused baseline (GEMM -> bias add -> activation
// as three launches) and the cache-flush sweep of the timing harness.
//
// The elementwise kernels follow the design rules of the "Fuse Elementwise
// Ops" page: one thread per 8 consecutive elements of a row (128-bit loads
// and stores for 16-bit types, two of them for fp32), casts to fp32 after
// the load and back before the store, and bounds guards on the ragged end of
// every row.  Each is a pure HBM stream: 2 x M x N x element_size bytes.
#include "common.hpp"
#include "launch.hpp"

namespace coalesce {
namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* src, int valid, float (&f)[8]) {
  if (valid >= 8) {
    if constexpr (sizeof(T) == 4) {
      const f32x4 a = *(const f32x4*)src, b = *(const f32x4*)(src + 4);
      f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
      f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    } else {
      typedef T t8 __attribute__((ext_vector_type(8)));
      const t8 a = *(const t8*)src;
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (float)a[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = i < valid ? (float)src[i] : 0.f;
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* dst, int valid, const float (&f)[8]) {
  if (valid >= 8) {
    if constexpr (sizeof(T) == 4) {
      *(f32x4*)dst = (f32x4){f[0], f[1], f[2], f[3]};
      *(f32x4*)(dst + 4) = (f32x4){f[4], f[5], f[6], f[7]};
    } else {
      typedef T t8 __attribute__((ext_vector_type(8)));
      t8 a;
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = (T)f[i];
      *(t8*)dst = a;
    }
  } else {
    for (int i = 0; i < valid; ++i) dst[i] = (T)f[i];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void bias_add_kernel(const T* __restrict__ X, int64_t ldx, const T* __restrict__ bias,
                                                       T* Y, int64_t ldy, int M, int N) {
  const int chunks = (N + 7) >> 3;
  const int64_t total = (int64_t)M * chunks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / chunks);
    const int n = (int)(i - (int64_t)m * chunks) * 8;
    const int valid = min(8, N - n);
    float x[8], b[8];
    load8<T>(X + (int64_t)m * ldx + n, valid, x);
#pragma unroll
    for (int r = 0; r < 8; ++r) b[r] = r < valid ? (float)bias[n + r] : 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = x[r] + b[r];
    store8<T>(Y + (int64_t)m * ldy + n, valid, x);
  }
}

template <typename T, int ACT>
__global__ __launch_bounds__(256) void activation_kernel(const T* X, int64_t ldx, T* Y, int64_t ldy, int M, int N) {
  const int chunks = (N + 7) >> 3;
  const int64_t total = (int64_t)M * chunks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / chunks);
    const int n = (int)(i - (int64_t)m * chunks) * 8;
    const int valid = min(8, N - n);
    float x[8];
    load8<T>(X + (int64_t)m * ldx + n, valid, x);
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = apply_act<ACT, sizeof(T) == 2>(x[r]);
    store8<T>(Y + (int64_t)m * ldy + n, valid, x);
  }
}

__global__ __launch_bounds__(256) void flush_kernel(const u32x4* __restrict__ buf, size_t n16, unsigned* sink) {
  u32x4 acc = (u32x4){0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    acc ^= buf[i];
  const unsigned v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  // Practically never true; the data dependence keeps every read alive.
  if (v == 0x9e3779b9u) sink[0] = v;
}

// Autotuning's validation: count the 16-bit words in which two matrices of
// rows x row_bytes differ (grid-stride over rows and words; one atomic add
// per thread that saw a difference).
__global__ __launch_bounds__(256) void compare_kernel(const unsigned short* __restrict__ a, int64_t pitch_a,
                                                      const unsigned short* __restrict__ b, int64_t pitch_b,
                                                      int64_t rows, int64_t words, unsigned int* counter) {
  unsigned int diff = 0;
  const int64_t total = rows * words;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / words, c = i - r * words;
    diff += a[r * pitch_a + c] != b[r * pitch_b + c] ? 1u : 0u;
  }
  if (diff) atomicAdd(counter, diff);
}

int grid_for(int64_t work_items, int num_cus) {
  const int64_t blocks = (work_items + 255) / 256;
  const int64_t cap = (int64_t)num_cus * 16;
  return (int)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

template <typename T>
hipError_t bias_add_t(const void* X, int64_t ldx, const void* bias, void* Y, int64_t ldy, int M, int N,
                      hipStream_t stream, int num_cus) {
  const int64_t work = (int64_t)M * ((N + 7) / 8);
  hipLaunchKernelGGL((bias_add_kernel<T>), dim3(grid_for(work, num_cus)), dim3(256), 0, stream, (const T*)X, ldx,
                     (const T*)bias, (T*)Y, ldy, M, N);
  return hipGetLastError();
}

template <typename T, int ACT>
hipError_t act_t(const void* X, int64_t ldx, void* Y, int64_t ldy, int M, int N, hipStream_t stream, int num_cus) {
  const int64_t work = (int64_t)M * ((N + 7) / 8);
  hipLaunchKernelGGL((activation_kernel<T, ACT>), dim3(grid_for(work, num_cus)), dim3(256), 0, stream, (const T*)X,
                     ldx, (T*)Y, ldy, M, N);
  return hipGetLastError();
}

template <typename T>
hipError_t act_dispatch(const void* X, int64_t ldx, void* Y, int64_t ldy, int M, int N, int act, hipStream_t stream,
                        int num_cus) {
  switch (act) {
    case ACT_GELU: return act_t<T, ACT_GELU>(X, ldx, Y, ldy, M, N, stream, num_cus);
    case ACT_SOFTPLUS: return act_t<T, ACT_SOFTPLUS>(X, ldx, Y, ldy, M, N, stream, num_cus);
    case ACT_RELU: return act_t<T, ACT_RELU>(X, ldx, Y, ldy, M, N, stream, num_cus);
    default: return act_t<T, ACT_NONE>(X, ldx, Y, ldy, M, N, stream, num_cus);
  }
}

}  // namespace

hipError_t launch_bias_add(const void* X, int64_t ldx, const void* bias, void* Y, int64_t ldy, int M, int N, DType xt,
                           DType, DType, hipStream_t stream, int num_cus) {
  switch (xt) {
    case DT_F32: return bias_add_t<float>(X, ldx, bias, Y, ldy, M, N, stream, num_cus);
    case DT_F16: return bias_add_t<_Float16>(X, ldx, bias, Y, ldy, M, N, stream, num_cus);
    default: return bias_add_t<__bf16>(X, ldx, bias, Y, ldy, M, N, stream, num_cus);
  }
}

hipError_t launch_activation(const void* X, int64_t ldx, void* Y, int64_t ldy, int M, int N, DType dt, int act,
                             hipStream_t stream, int num_cus) {
  switch (dt) {
    case DT_F32: return act_dispatch<float>(X, ldx, Y, ldy, M, N, act, stream, num_cus);
    case DT_F16: return act_dispatch<_Float16>(X, ldx, Y, ldy, M, N, act, stream, num_cus);
    default: return act_dispatch<__bf16>(X, ldx, Y, ldy, M, N, act, stream, num_cus);
  }
}

hipError_t launch_compare(const void* a, int64_t pitch_a, const void* b, int64_t pitch_b, int64_t rows,
                          int64_t row_bytes, unsigned int* counter, hipStream_t stream, int num_cus) {
  const int64_t words = row_bytes / 2;
  if (rows <= 0 || words <= 0) return hipSuccess;
  hipLaunchKernelGGL(compare_kernel, dim3(grid_for(rows * words, num_cus)), dim3(256), 0, stream,
                     (const unsigned short*)a, pitch_a / 2, (const unsigned short*)b, pitch_b / 2, rows, words, counter);
  return hipGetLastError();
}

hipError_t launch_flush(const void* buf, size_t bytes, void* sink, hipStream_t stream, int num_cus) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(flush_kernel, dim3(num_cus * 8), dim3(256), 0, stream, (const u32x4*)buf, n16, (unsigned*)sink);
  return hipGetLastError();
}

}  // namespace coalesce
