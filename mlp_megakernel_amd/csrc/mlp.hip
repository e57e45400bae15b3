// Persistent softplus-MLP megakernel ("MLP Megakernel" README: all layers'
// GEMMs and activations in one launch, intermediate activations kept in
// registers, fp16 MFMA operands with fp32 accumulation, a persistent grid of
// min(#CUs x occupancy, #tiles) workgroups walking the row tiles round-robin).
//
//   h_0 = x;  h_l = act(h_{l-1} W_l) (l < L);  out = h_{L-1} W_L
//
// Design for gfx950, all widths D (64 or 128):
//   * one 512-thread workgroup per CU (8 waves, 2 per SIMD); it copies every
//     W_l into LDS once (L * D * D fp16: 96 KB for 3 x 128, 40 KB for 5 x 64)
//     and reuses it for all of its row tiles;
//   * a wave owns a tile of 64 rows; tiles go to waves round-robin, so every
//     row goes through the same instruction sequence whatever the grid size
//     (results are bit-identical for any grid);
//   * each layer is computed transposed, z^T = W^T h^T, with
//     v_mfma_f32_16x16x32_f16: the A operand is W^T read from LDS (one
//     128-bit read per 16 output units and 32 k, shared by the wave's four
//     16-row sub-tiles), the B operand is h^T straight from registers;
//   * the MFMA result layout (lane holds 4 consecutive output units of one
//     row) is reused as the next layer's B operand without any data
//     movement: the 8 fp16 values a lane needs for one 32-deep k step are its
//     own results of two neighbouring 16-unit sub-tiles.  The k order this
//     induces is fixed and is absorbed into how W_{l+1} is laid out in LDS
//     (layer_k_slot below);
//   * activation in fp32 on the accumulators, rounded to fp16 only as the
//     next layer's operand; the last layer stores fp16 directly;
//   * two waves per SIMD: one wave's global loads and activations overlap the
//     other's MFMAs.
#include "common.hpp"
#include "launch.hpp"

namespace coalesce {
namespace {

constexpr int THREADS = 512, WAVES = 8, TILE_ROWS = 64, MT = TILE_ROWS / 16;

// LDS position (within a row of W^T) of logical input unit k for layers fed
// by a previous layer's registers.  Lane group g of the B operand holds, for
// k step ks, elements e = 0..7 = units 32 ks + 16 (e / 4) + 4 g + (e % 4); the
// A operand lane group g reads 8 consecutive LDS elements starting at
// 32 ks + 8 g, so unit k must sit at 32 ks + 8 g + e.
__device__ __forceinline__ int layer_k_slot(int k) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

// 16-byte chunk swizzle of W^T rows (row n: chunk c at c ^ (n & 7)).
template <int D>
__device__ __forceinline__ int w_offset(int l, int n, int slot) {
  return (l * D + n) * D + ((((slot >> 3) ^ (n & 7))) << 3) + (slot & 7);
}

template <int D, int L>
__device__ __forceinline__ void stage_weights(const MlpParams& p, _Float16* sW) {
  constexpr int CHUNKS = D / 8;  // 16-byte chunks per weight row
  for (int idx = threadIdx.x; idx < L * D * CHUNKS; idx += THREADS) {
    const int l = idx / (D * CHUNKS);
    const int rem = idx - l * D * CHUNKS;
    const int k = rem / CHUNKS;
    const int c = rem - k * CHUNKS;
    const f16x8 v = *(const f16x8*)((const _Float16*)p.W[l] + (int64_t)k * D + c * 8);
    const int slot = l == 0 ? k : layer_k_slot(k);
#pragma unroll
    for (int i = 0; i < 8; ++i) sW[w_offset<D>(l, c * 8 + i, slot)] = v[i];
  }
}

template <int D>
__device__ __forceinline__ void load_x(const MlpParams& p, int tile, int lane, i16x8 (&h)[MT][D / 32]) {
  const _Float16* x = (const _Float16*)p.x;
  const int q = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < MT; ++s) {
    const int row = min(tile * TILE_ROWS + 16 * s + q, p.M - 1);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) h[s][ks] = *(const i16x8*)(x + (int64_t)row * p.ldx + 32 * ks + 8 * g);
  }
}

template <int ACT>
__device__ __forceinline__ f16x4 act_to_f16(f32x4 v) {
  return (f16x4){(_Float16)apply_act<ACT>(v[0]), (_Float16)apply_act<ACT>(v[1]), (_Float16)apply_act<ACT>(v[2]),
                 (_Float16)apply_act<ACT>(v[3])};
}

// One layer for one 64-row tile.  Output sub-tile t (16 units) is finished
// before t + 1 starts, so its activation overlaps the next sub-tile's MFMAs.
template <int D, int L, int l, int ACT>
__device__ __forceinline__ void layer(const MlpParams& p, const _Float16* sW, int tile, int lane,
                                      const i16x8 (&hin)[MT][D / 32], i16x8 (&hout)[MT][D / 32]) {
  constexpr int NT = D / 16, KS = D / 32;
  const int q = lane & 15, g = lane >> 4;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    f32x4 acc[MT];
#pragma unroll
    for (int s = 0; s < MT; ++s) acc[s] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int n = 16 * t + q;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const i16x8 a = *(const i16x8*)(sW + w_offset<D>(l, n, 32 * ks + 8 * g));
#pragma unroll
      for (int s = 0; s < MT; ++s) acc[s] = mfma16x16x32(a, hin[s][ks], acc[s], _Float16());
    }
    if constexpr (l + 1 < L) {
#pragma unroll
      for (int s = 0; s < MT; ++s) {
        const f16x4 o = act_to_f16<ACT>(acc[s]);
        const i16x4 ob = __builtin_bit_cast(i16x4, o);
#pragma unroll
        for (int r = 0; r < 4; ++r) hout[s][t >> 1][(t & 1) * 4 + r] = ob[r];
      }
    } else {
      _Float16* out = (_Float16*)p.out;
#pragma unroll
      for (int s = 0; s < MT; ++s) {
        const int row = tile * TILE_ROWS + 16 * s + q;
        if (row < p.M) {
          const f16x4 o = (f16x4){(_Float16)acc[s][0], (_Float16)acc[s][1], (_Float16)acc[s][2], (_Float16)acc[s][3]};
          *(f16x4*)(out + (int64_t)row * p.ldo + 16 * t + 4 * g) = o;
        }
      }
    }
  }
}

template <int D, int L, int l, int ACT>
__device__ __forceinline__ void run_layers(const MlpParams& p, const _Float16* sW, int tile, int lane,
                                           i16x8 (&h0)[MT][D / 32], i16x8 (&h1)[MT][D / 32]) {
  if constexpr (l % 2 == 0)
    layer<D, L, l, ACT>(p, sW, tile, lane, h0, h1);
  else
    layer<D, L, l, ACT>(p, sW, tile, lane, h1, h0);
  if constexpr (l + 1 < L) run_layers<D, L, l + 1, ACT>(p, sW, tile, lane, h0, h1);
}

template <int D, int L, int ACT>
__global__ __launch_bounds__(THREADS, 1) void mlp_kernel(MlpParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 sW[L * D * D];
  stage_weights<D, L>(p, sW);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * WAVES + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * WAVES;
  i16x8 h0[MT][D / 32], h1[MT][D / 32];
  for (int tile = wave; tile < p.num_tiles; tile += nwaves) {
    // An offset the compiler cannot see through: the weight fragments are
    // re-read from LDS for every tile instead of being hoisted into
    // registers (they do not fit next to the activations).
    int woff = 0;
    asm volatile("" : "+v"(woff));
    load_x<D>(p, tile, lane, h0);
    run_layers<D, L, 0, ACT>(p, sW + woff, tile, lane, h0, h1);
  }
}

template <int D, int L, int ACT>
hipError_t launch_dl(const MlpParams& p, int num_workgroups, hipStream_t stream) {
  hipLaunchKernelGGL((mlp_kernel<D, L, ACT>), dim3(num_workgroups), dim3(THREADS), 0, stream, p);
  return hipGetLastError();
}

template <int D, int ACT>
hipError_t launch_d(const MlpParams& p, int L, int nwg, hipStream_t stream) {
  if constexpr (D == 128) {
    switch (L) {
      case 1: return launch_dl<D, 1, ACT>(p, nwg, stream);
      case 2: return launch_dl<D, 2, ACT>(p, nwg, stream);
      case 3: return launch_dl<D, 3, ACT>(p, nwg, stream);
      case 4: return launch_dl<D, 4, ACT>(p, nwg, stream);
    }
  } else {
    switch (L) {
      case 1: return launch_dl<D, 1, ACT>(p, nwg, stream);
      case 2: return launch_dl<D, 2, ACT>(p, nwg, stream);
      case 3: return launch_dl<D, 3, ACT>(p, nwg, stream);
      case 4: return launch_dl<D, 4, ACT>(p, nwg, stream);
      case 5: return launch_dl<D, 5, ACT>(p, nwg, stream);
      case 6: return launch_dl<D, 6, ACT>(p, nwg, stream);
      case 7: return launch_dl<D, 7, ACT>(p, nwg, stream);
      case 8: return launch_dl<D, 8, ACT>(p, nwg, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

int mlp_tile_rows() { return TILE_ROWS; }
int mlp_waves_per_workgroup() { return WAVES; }

hipError_t launch_mlp(const MlpParams& p, int D, int L, int act, int num_workgroups, hipStream_t stream) {
  if (D == 128) {
    if (act == ACT_NONE) return launch_d<128, ACT_NONE>(p, L, num_workgroups, stream);
    return launch_d<128, ACT_SOFTPLUS>(p, L, num_workgroups, stream);
  }
  if (act == ACT_NONE) return launch_d<64, ACT_NONE>(p, L, num_workgroups, stream);
  return launch_d<64, ACT_SOFTPLUS>(p, L, num_workgroups, stream);
}

}  // namespace coalesce
