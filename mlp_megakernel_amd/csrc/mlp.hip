// Persistent softplus-MLP megakernel ("MLP Megakernel" README: all layers'
// GEMMs and activations in one launch, intermediate activations kept in
// registers, fp16 MFMA operands with fp32 accumulation, a persistent grid of
// min(#CUs x occupancy, #tiles) workgroups walking the row tiles round-robin).
//
//   h_0 = x;  h_l = act(h_{l-1} W_l) (l < L);  out = h_{L-1} W_L
//
// Design for gfx950, widths D of 64 or 128:
//   * a workgroup copies every W_l into LDS once (L * D * D fp16: 96 KB for
//     3 x 128, 40 KB for 5 x 64) and reuses it for all of its row tiles;
//   * a wave owns a tile of 32 (D = 128) or 64 (D = 64) rows; tiles go to
//     waves round-robin, so every row goes through the same instruction
//     sequence whatever the grid size (results are bit-identical for any
//     grid);
//   * each layer is computed transposed, z^T = W^T h^T, with
//     v_mfma_f32_16x16x32_f16: the A operand is W^T read from LDS (one
//     128-bit read per 16 output units and 32 k, shared by the wave's 16-row
//     sub-tiles), the B operand is h^T straight from registers;
//   * the MFMA result layout (lane holds 4 consecutive output units of one
//     row) is reused as the next layer's B operand without any data
//     movement: the 8 fp16 values a lane needs for one 32-deep k step are its
//     own results of two neighbouring 16-unit sub-tiles.  The k order this
//     induces is fixed and is absorbed into how W_{l+1} is laid out in LDS
//     (layer_k_slot below);
//   * activation in fp32 on the accumulators, rounded to fp16 only as the
//     next layer's operand; the last layer stores fp16 directly;
//   * at most 128 VGPRs, so 4 waves share a SIMD: one wave's global loads
//     and activations overlap the others' MFMAs.
#include "common.hpp"
#include "launch.hpp"

namespace coalesce {
namespace {

// Per-width geometry.  A wave owns a tile of 16 * MT rows; a workgroup has
// WAVES waves.  Width 128: 32-row tiles and 16-wave workgroups, so one
// workgroup (its 96 KB of weights fill the LDS) still gives 4 waves per SIMD
// within 128 VGPRs.  Width 64: 64-row tiles, 8-wave workgroups, two per CU.
template <int D>
struct MlpCfg;
template <>
struct MlpCfg<128> {
  static constexpr int MT = 2, WAVES = 16;
};
template <>
struct MlpCfg<64> {
  static constexpr int MT = 4, WAVES = 8;
};
template <int D>
constexpr int tile_rows() { return 16 * MlpCfg<D>::MT; }
template <int D>
constexpr int threads() { return 64 * MlpCfg<D>::WAVES; }

// LDS position (within a row of W^T) of logical input unit k for layers fed
// by a previous layer's registers.  Lane group g of the B operand holds, for
// k step ks, elements e = 0..7 = units 32 ks + 16 (e / 4) + 4 g + (e % 4); the
// A operand lane group g reads 8 consecutive LDS elements starting at
// 32 ks + 8 g, so unit k must sit at 32 ks + 8 g + e.
__device__ __forceinline__ int layer_k_slot(int k) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

// 16-byte chunk swizzle of W^T rows: chunk c of row n sits at c ^ wswz(n).  A
// weight-fragment read is one 128-bit read by 16 lanes (rows n0..n0+15, one
// chunk); the swizzle puts those 16 reads in 16 distinct 16-byte slots of a
// 256-byte bank window (and any 8 consecutive rows in 8 distinct slots of a
// 128-byte one).  Rows are 256 B (16 chunks) for D = 128 and 128 B for D = 64.
template <int D>
__device__ __forceinline__ int wswz(int n) {
  if constexpr (D == 128)
    return n & 15;
  else
    return ((n >> 1) & 7) ^ ((n & 1) << 2);
}

template <int D>
__device__ __forceinline__ int w_offset(int l, int n, int slot) {
  return (l * D + n) * D + ((((slot >> 3) ^ wswz<D>(n))) << 3) + (slot & 7);
}

template <int D, int L>
__device__ __forceinline__ void stage_weights(const MlpParams& p, _Float16* sW) {
  constexpr int CHUNKS = D / 8;  // 16-byte chunks per weight row
  for (int idx = threadIdx.x; idx < L * D * CHUNKS; idx += threads<D>()) {
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

// Uniform (SGPR) base of a row tile: per-lane offsets from it fit in 32 bits
// (at most 64 rows x a pitch the host limits), which keeps 64-bit address arithmetic
// out of the loop.
__device__ __forceinline__ const char* tile_base(const void* p, int64_t first_row, int64_t ld) {
  const uint64_t v = (uint64_t)(uintptr_t)((const char*)p + first_row * ld * 2);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

template <int D>
__device__ __forceinline__ void load_x(const MlpParams& p, int tile, int lane,
                                       i16x8 (&h)[MlpCfg<D>::MT][D / 32]) {
  const char* base = tile_base(p.x, (int64_t)tile * tile_rows<D>(), p.ldx);
  const int q = lane & 15, g = lane >> 4;
  const int rows_left = p.M - 1 - tile * tile_rows<D>();  // last valid row within the tile
#pragma unroll
  for (int s = 0; s < MlpCfg<D>::MT; ++s) {
    const uint32_t r = (uint32_t)min(16 * s + q, rows_left);
    const uint32_t off = r * (uint32_t)(p.ldx * 2) + (uint32_t)(16 * g);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) h[s][ks] = *(const i16x8*)(base + off + 64 * ks);
  }
}

// Hidden activations travel between layers in base-2 units, g = h / ln 2
// (h = softplus(z)), instead of h itself.  Then the next layer's accumulator
// is a = g W = z / ln 2 = z log2(e), exactly the argument the hardware
// exponential (2^x) wants, and
//   g' = softplus(z') / ln 2 = log2(1 + 2^a')
// costs exp2, add, log2 and the page's threshold (z > 20, i.e. a > 20 log2 e,
// passes a through), with no base-change multiplies.  The first layer, whose
// input x is in natural units, scales its accumulator by log2(e) once; the
// last layer scales its output by ln 2 once.  In exact arithmetic nothing
// changes; the fp16 operand is g rather than h (the same relative rounding).
__device__ __forceinline__ float softplus_b2(float a) {
  const float s = __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(a));
  return a > 28.853900817779268f ? a : s;
}

template <int ACT, bool IN_B2>
__device__ __forceinline__ float hidden_act(float acc) {
  if constexpr (ACT == ACT_SOFTPLUS) {
    if constexpr (IN_B2)
      return softplus_b2(acc);
    else
      return softplus_b2(acc * 1.44269504088896341f);
  } else {
    return acc;
  }
}

template <int ACT, bool IN_B2>
__device__ __forceinline__ f16x4 act_to_f16(f32x4 v) {
  return (f16x4){(_Float16)hidden_act<ACT, IN_B2>(v[0]), (_Float16)hidden_act<ACT, IN_B2>(v[1]),
                 (_Float16)hidden_act<ACT, IN_B2>(v[2]), (_Float16)hidden_act<ACT, IN_B2>(v[3])};
}

// One layer for one row tile.  Output sub-tile t (16 units) is finished
// before t + 1 starts, so its activation overlaps the next sub-tile's MFMAs.
template <int D, int L, int l, int ACT>
__device__ __forceinline__ void layer(const MlpParams& p, const _Float16* sW, int tile, int lane,
                                      const i16x8 (&hin)[MlpCfg<D>::MT][D / 32],
                                      i16x8 (&hout)[MlpCfg<D>::MT][D / 32]) {
  constexpr int NT = D / 16, KS = D / 32, MT = MlpCfg<D>::MT;
  // does this layer's input arrive in base-2 units (see softplus_b2)?
  constexpr bool IN_B2 = ACT == ACT_SOFTPLUS && l > 0;
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
        const f16x4 o = act_to_f16<ACT, IN_B2>(acc[s]);
        const i16x4 ob = __builtin_bit_cast(i16x4, o);
#pragma unroll
        for (int r = 0; r < 4; ++r) hout[s][t >> 1][(t & 1) * 4 + r] = ob[r];
      }
    } else {
      char* obase = (char*)tile_base(p.out, (int64_t)tile * tile_rows<D>(), p.ldo);
      const int rows_left = p.M - tile * tile_rows<D>();
#pragma unroll
      for (int s = 0; s < MT; ++s) {
        const int r = 16 * s + q;
        if (r < rows_left) {
          const float sc = IN_B2 ? 0.693147180559945309f : 1.0f;
          const f16x4 o = (f16x4){(_Float16)(acc[s][0] * sc), (_Float16)(acc[s][1] * sc), (_Float16)(acc[s][2] * sc),
                                  (_Float16)(acc[s][3] * sc)};
          *(f16x4*)(obase + (uint32_t)r * (uint32_t)(p.ldo * 2) + (uint32_t)(32 * t + 8 * g)) = o;
        }
      }
    }
  }
}

template <int D, int L, int l, int ACT>
__device__ __forceinline__ void run_layers(const MlpParams& p, const _Float16* sW, int tile, int lane,
                                           i16x8 (&h0)[MlpCfg<D>::MT][D / 32],
                                           i16x8 (&h1)[MlpCfg<D>::MT][D / 32]) {
  if constexpr (l % 2 == 0)
    layer<D, L, l, ACT>(p, sW, tile, lane, h0, h1);
  else
    layer<D, L, l, ACT>(p, sW, tile, lane, h1, h0);
  if constexpr (l + 1 < L) run_layers<D, L, l + 1, ACT>(p, sW, tile, lane, h0, h1);
}

// Every configuration is held to 128 VGPRs (at least 4 waves per SIMD, the
// second launch-bounds argument) so that memory latency and the activation
// chains of some waves hide behind the MFMAs of others.
template <int D, int L, int ACT>
__global__ __launch_bounds__(threads<D>(), 4) void mlp_kernel(MlpParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 sW[L * D * D];
  stage_weights<D, L>(p, sW);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * MlpCfg<D>::WAVES + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * MlpCfg<D>::WAVES;
  i16x8 h0[MlpCfg<D>::MT][D / 32], h1[MlpCfg<D>::MT][D / 32];
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

// Persistent grid: min(#CUs x workgroups that fit on a CU, #workgroups with
// work), unless the caller fixed the count.  The per-CU occupancy comes from
// the runtime for the compiled kernel (its VGPR and LDS use) and is cached.
template <int D, int L, int ACT>
hipError_t launch_dl(MlpParams p, int num_workgroups, int num_cus, hipStream_t stream) {
  p.num_tiles = (int)(((int64_t)p.M + tile_rows<D>() - 1) / tile_rows<D>());
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mlp_kernel<D, L, ACT>, threads<D>(), 0);
    if (e != hipSuccess) return e;
    per_cu = n > 0 ? n : 1;
  }
  int nwg = num_workgroups;
  if (nwg <= 0) {
    const int need = (p.num_tiles + MlpCfg<D>::WAVES - 1) / MlpCfg<D>::WAVES;
    const long cap = (long)num_cus * per_cu;
    nwg = need < cap ? need : (int)cap;
    if (nwg < 1) nwg = 1;
  }
  hipLaunchKernelGGL((mlp_kernel<D, L, ACT>), dim3(nwg), dim3(threads<D>()), 0, stream, p);
  return hipGetLastError();
}

template <int D, int ACT>
hipError_t launch_d(const MlpParams& p, int L, int nwg, int cus, hipStream_t stream) {
  if constexpr (D == 128) {
    switch (L) {
      case 1: return launch_dl<D, 1, ACT>(p, nwg, cus, stream);
      case 2: return launch_dl<D, 2, ACT>(p, nwg, cus, stream);
      case 3: return launch_dl<D, 3, ACT>(p, nwg, cus, stream);
      case 4: return launch_dl<D, 4, ACT>(p, nwg, cus, stream);
    }
  } else {
    switch (L) {
      case 1: return launch_dl<D, 1, ACT>(p, nwg, cus, stream);
      case 2: return launch_dl<D, 2, ACT>(p, nwg, cus, stream);
      case 3: return launch_dl<D, 3, ACT>(p, nwg, cus, stream);
      case 4: return launch_dl<D, 4, ACT>(p, nwg, cus, stream);
      case 5: return launch_dl<D, 5, ACT>(p, nwg, cus, stream);
      case 6: return launch_dl<D, 6, ACT>(p, nwg, cus, stream);
      case 7: return launch_dl<D, 7, ACT>(p, nwg, cus, stream);
      case 8: return launch_dl<D, 8, ACT>(p, nwg, cus, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace


hipError_t launch_mlp(const MlpParams& p, int D, int L, int act, int num_workgroups, int num_cus, hipStream_t stream) {
  if (D == 128) {
    if (act == ACT_NONE) return launch_d<128, ACT_NONE>(p, L, num_workgroups, num_cus, stream);
    return launch_d<128, ACT_SOFTPLUS>(p, L, num_workgroups, num_cus, stream);
  }
  if (act == ACT_NONE) return launch_d<64, ACT_NONE>(p, L, num_workgroups, num_cus, stream);
  return launch_d<64, ACT_SOFTPLUS>(p, L, num_workgroups, num_cus, stream);
}

}  // namespace coalesce
