// Device-side building blocks shared by the gfx950 kernels of libcoalesce.
//
// Lane layouts of the CDNA4 matrix instructions used here (64-lane waves;
// every GEMM and MLP parity test depends on them):
//   v_mfma_f32_16x16x32_{bf16,f16}: A operand lane l holds A[l%16][8(l/16)+e],
//     B operand lane l holds B[8(l/16)+e][l%16] (e = 0..7); result register r
//     of lane l is D[4(l/16)+r][l%16].
//   v_mfma_f32_16x16x4_f32: A lane l holds A[l%16][l/16], B lane l holds
//     B[l/16][l%16]; result as above.
//   ds_read_b64_tr_b16: within each 16-lane group, lanes 4r..4r+3 fetch 8
//     bytes each (together one 16-element row r); lane i of the group receives
//     element i of rows r = 0..3.
//   global_load_lds (16 bytes): lane l's 16 bytes land at the LDS base + 16 l.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace coalesce {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
struct u16x2x4 {
  u16x2 v[4];
};
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// GELU, erf form: 0.5 z (1 + erf(z / sqrt 2)) ("Coalesce" README notes: use
// erf, not the tanh approximation).  erf(z / sqrt 2) is evaluated as
// zc P(zc^2) / Q(zc^2), zc = clamp(z, -4 sqrt 2, 4 sqrt 2), a degree-5/5
// rational fitted to erf (coefficients and their derivation:
// mlp_megakernel_amd/erf_fit.py): 3.3e-7 absolute error on erf and 8.7e-7 on
// GELU in fp32 (the tanh approximation is off by ~1e-3), with no branch and
// 17 VALU operations instead of the library erff's ~30 plus divergent
// branches.
__device__ __forceinline__ float gelu_erf(float z) {
  const float zc = __builtin_amdgcn_fmed3f(z, -5.656854249f, 5.656854249f);
  const float u = zc * zc;
  float P = 4.390178103e-08f;
  P = __builtin_fmaf(P, u, 1.257623330e-05f);
  P = __builtin_fmaf(P, u, 3.432499626e-04f);
  P = __builtin_fmaf(P, u, 9.387202248e-03f);
  P = __builtin_fmaf(P, u, 6.842921802e-02f);
  P = __builtin_fmaf(P, u, 7.978845412e-01f);
  float Q = 1.169378502e-06f;
  Q = __builtin_fmaf(Q, u, 7.409945064e-05f);
  Q = __builtin_fmaf(Q, u, 1.900929089e-03f);
  Q = __builtin_fmaf(Q, u, 2.883771099e-02f);
  Q = __builtin_fmaf(Q, u, 2.524295846e-01f);
  Q = __builtin_fmaf(Q, u, 1.0f);
  const float e = zc * (P * __builtin_amdgcn_rcpf(Q));
  const float h = 0.5f * z;
  return __builtin_fmaf(h, e, h);
}

// The same GELU with a degree-3/4 rational (same derivation, erf_fit.py):
// 2.1e-5 absolute error on GELU in fp32, under 0.03 of an ulp of a bf16 or
// fp16 result at |y| = 1, for 13 VALU operations instead of 16.  Used where
// the result is rounded to a 16-bit type.
__device__ __forceinline__ float gelu_erf16(float z) {
  const float zc = __builtin_amdgcn_fmed3f(z, -5.656854249f, 5.656854249f);
  const float u = zc * zc;
  float P = 1.245941954e-04f;
  P = __builtin_fmaf(P, u, 8.630056566e-03f);
  P = __builtin_fmaf(P, u, 6.086595174e-02f);
  P = __builtin_fmaf(P, u, 7.978886278e-01f);
  float Q = 3.938829538e-06f;
  Q = __builtin_fmaf(Q, u, 1.491012022e-03f);
  Q = __builtin_fmaf(Q, u, 2.622371010e-02f);
  Q = __builtin_fmaf(Q, u, 2.430049890e-01f);
  Q = __builtin_fmaf(Q, u, 1.0f);
  const float e = zc * (P * __builtin_amdgcn_rcpf(Q));
  const float h = 0.5f * z;
  return __builtin_fmaf(h, e, h);
}

// softplus in the guarded form of the "MLP Megakernel" README's ablation
// findings: z above 20 passes through, otherwise ln(1 + e^z).  e^z and ln are
// the hardware base-2 exponential and logarithm with the base change folded
// into one multiply each.
__device__ __forceinline__ float softplus_guarded(float z) {
  float t = __builtin_amdgcn_exp2f(z * 1.44269504088896341f);
  float s = __builtin_amdgcn_logf(1.0f + t) * 0.693147180559945309f;
  return z > 20.0f ? z : s;
}

// relu(z) = z > 0 ? z : 0; v_max_f32 against +0 (a NaN z gives 0, as the
// comparison does).
__device__ __forceinline__ float relu(float z) { return __builtin_fmaxf(z, 0.0f); }

// OUT16: the result is rounded to bf16 / fp16 (the shorter GELU suffices).
template <int ACT, bool OUT16 = false>
__device__ __forceinline__ float apply_act(float z) {
  if constexpr (ACT == ACT_GELU) return OUT16 ? gelu_erf16(z) : gelu_erf(z);
  else if constexpr (ACT == ACT_SOFTPLUS) return softplus_guarded(z);
  else if constexpr (ACT == ACT_RELU) return relu(z);
  else return z;
}

// Conversions used at load and store time (round to nearest even).
template <typename T> __device__ __forceinline__ float to_f32(T v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return (T)v; }

// Asynchronous 16-byte global -> LDS copy (no VGPR staging): lane l's 16
// bytes land at LDS byte address lds_addr + 16 l.  lds_addr must be wave
// uniform.  Issued through inline asm so that the compiler does not guard
// every later LDS read with a wait for these copies (it cannot tell which
// LDS buffer they write); the kernels wait for them explicitly with
// wait_vmcnt0() before the barrier that publishes the buffer.  Nothing else
// in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr);
  // one wait state between the M0 write and the LDS-DMA instruction that reads it
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a __shared__ object (LDS addresses are 32-bit).
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) T*)(p);
}

__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

__device__ __forceinline__ f32x4 mfma16x16x32(i16x8 a, i16x8 b, f32x4 c, __bf16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(i16x8 a, i16x8 b, f32x4 c, _Float16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup -> tile mapping.  The hardware hands consecutive workgroup ids to
// the 8 XCDs in turn; when the tile count divides by 8, give every XCD one
// contiguous run of tiles so that the workgroups sharing an XCD's L2 work on
// neighbouring tiles.  Inside the run, tiles are walked in column groups of
// `group_m` tile rows so that concurrently running tiles share A and B panels.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  int total = tiles_m * tiles_n;
  int t = bid;
  if ((total & 7) == 0) t = (bid & 7) * (total >> 3) + (bid >> 3);
  int per_group = group_m * tiles_n;
  int g = t / per_group;
  int first_m = g * group_m;
  int gm = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
  int r = t - g * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

}  // namespace coalesce
