// Register and LDS layout helpers shared by the MLP megakernels (forward,
// training forward and backward): the chaining of one layer's MFMA result
// into the next layer's operand, the bank swizzle of weight rows in LDS and
// the paired 16-byte output store.
#pragma once
#include "common.hpp"

namespace coalesce {

// Two fp32 values rounded to nearest-even fp16 and packed into one dword.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}

// LDS position (within a weight row in LDS: a row of W^T in the forward, of W
// in the backward) of logical contraction unit k for layers whose B operand
// comes from the previous layer's registers.  Lane group g of the B operand holds, for
// k step ks, elements e = 0..7 = units 32 ks + 16 (e / 4) + 4 g + (e % 4); the
// A operand lane group g reads 8 consecutive LDS elements starting at
// 32 ks + 8 g, so unit k must sit at 32 ks + 8 g + e.
__device__ __forceinline__ int layer_k_slot(int k) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

// 16-byte chunk swizzle of weight rows in LDS: chunk c of row n sits at
// c ^ wswz(n).  A
// weight-fragment read is one 128-bit read by 16 lanes (rows n0..n0+15, one
// chunk); the swizzle puts those 16 reads in 16 distinct 16-byte slots of a
// 256-byte bank window (and any 8 consecutive rows in 8 distinct slots of a
// 128-byte one).  Rows are 256 B (16 chunks) for D = 128 and 128 B for D = 64.
// wswz(16 t + q) = wswz(q): the swizzle repeats every 16 rows.
template <int D>
__device__ __forceinline__ int wswz(int n) {
  if constexpr (D == 128)
    return n & 15;
  else
    return ((n >> 1) & 7) ^ ((n & 1) << 2);
}

// Logical input unit k that sits at LDS slot `slot` (inverse of
// layer_k_slot): slot = 32 a + 8 b + 4 c + d holds k = 32 a + 16 c + 4 b + d.
__device__ __forceinline__ int layer_slot_k(int slot) {
  return (slot & ~31) | (((slot >> 2) & 1) << 4) | (((slot >> 3) & 3) << 2) | (slot & 3);
}

__device__ __forceinline__ i16x8 lds_read128(uint32_t addr) {
  return *(const __attribute__((address_space(3))) i16x8*)(uintptr_t)addr;
}

// A value the compiler cannot see through.  The weight-fragment addresses of
// every layer of every tile pass through it, so that neither the fragments
// nor per-layer addresses are hoisted out of the tile loop into registers
// (they do not fit next to the activations); constant offsets added
// afterwards stay in the instructions' immediate fields.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Output of two neighbouring 16-unit sub-tiles u (even) and u + 1 of one
// 16-row sub-tile, fp16.  Lane group g (lanes 16 g .. 16 g + 15, one row
// each) holds 8 bytes of each: units 16 u + 4 g .. + 3 in a and
// 16 (u + 1) + 4 g .. + 3 in b.  One v_permlane16_swap per dword exchanges
// b of groups 0 and 2 with a of groups 1 and 3; then group g holds 16
// contiguous bytes, at unit 16 u + 16 (g & 1) + 8 (g >> 1), and the four
// groups cover 64 contiguous bytes of their row: one 16-byte store per lane
// instead of two 8-byte ones with 32 contiguous bytes per row.
__device__ __forceinline__ void store_pair(__amdgpu_buffer_rsrc_t rs, uint32_t off, u32x2 a, u32x2 b) {
  const auto s0 = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  __builtin_amdgcn_raw_buffer_store_b128((u32x4){s0[0], s1[0], s0[1], s1[1]}, rs, off, 0, 0);
}

// LDS stores of 8 and 16 bytes and the transposing 8-byte read at a byte
// address.
__device__ __forceinline__ void lds_write64(uint32_t addr, u32x2 v) {
  *(__attribute__((address_space(3))) u32x2*)(uintptr_t)addr = v;
}
__device__ __forceinline__ void lds_write128(uint32_t addr, u32x4 v) {
  *(__attribute__((address_space(3))) u32x4*)(uintptr_t)addr = v;
}
__device__ __forceinline__ i16x4 lds_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)addr);
}

// dz = g * act'(z) from the stored output h = act(z), in fp32:
//   softplus: act'(z) = sigmoid(z) = 1 - e^{-h} (e^{-h} = 1 / (1 + e^z) for
//     h = ln(1 + e^z)).  The hardware 2^x on -h log2(e) gives e^{-h} to about
//     one ulp, and 1 - e^{-h} is then exact, so the derivative is off by at
//     most 2^-23 in absolute terms: below the resolution of the fp16 dz it
//     feeds wherever dz is a normal fp16 number;
//   relu: g where h > 0, else 0 (a select, so an infinite g gives 0 there);
//   none: g.
template <int ACT>
__device__ __forceinline__ float apply_grad(float g, float h) {
  if constexpr (ACT == ACT_SOFTPLUS) {
    return g * (1.0f - __builtin_amdgcn_exp2f(h * -1.44269504088896341f));
  } else if constexpr (ACT == ACT_RELU) {
    return h > 0.0f ? g : 0.0f;
  } else {
    return g;
  }
}

}  // namespace coalesce
