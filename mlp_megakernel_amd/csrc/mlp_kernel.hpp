// Persistent softplus-MLP megakernel ("MLP Megakernel" README: all layers'
// GEMMs and activations in one launch, intermediate activations kept in
// registers, fp16 MFMA operands with fp32 accumulation, a persistent grid
// walking the row tiles).
//
//   h_0 = x;  h_l = act(h_{l-1} W_l) (l < L);  out = h_{L-1} W_L
//
// Design for gfx950, widths D of 64 or 128:
//   * a workgroup copies every W_l into LDS once (L * D * D fp16: 96 KB for
//     3 x 128, 40 KB for 5 x 64) and reuses it for all of its row tiles;
//   * a wave works on a tile of 32 rows at a time (16 for small batches,
//     see MlpCfg); workgroup b owns the
//     tiles b, b + G, b + 2G, ... (G workgroups) and its waves claim them one
//     at a time from a counter in LDS.  The SIMD issues from its oldest
//     ready wave first, so waves sharing a SIMD progress at very different
//     rates (with a fixed share each, the youngest finished ~2.7x later than
//     the oldest and ran alone at the end); claiming on demand keeps all of
//     them busy to the end.  Every row goes through the same instruction
//     sequence whatever wave or grid takes it, so results are bit-identical
//     for any grid and any timing;
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
//   * software pipeline inside a layer: the MFMAs of output sub-tile t are
//     interleaved, instruction by instruction, with the activation of
//     sub-tile t - 1, so the matrix core and the vector ALU work at the same
//     time even within one wave; the x of a wave's next row tile is loaded
//     when the current one starts, into a third register buffer;
//   * the output of two neighbouring 16-unit sub-tiles is exchanged between
//     lane groups (v_permlane16_swap) so that every lane stores 16 bytes and
//     each store instruction writes 64 contiguous bytes per row;
//   * the activation is VALU-bound (two transcendentals per element), so
//     the softplus guard is taken out of the per-element path: see
//     softplus_b2_fast and the check at the end of mlp_kernel.
#pragma once
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "mlp_common.hpp"

namespace coalesce {
namespace {

// Per-width geometry.  A wave owns a tile of 16 * MT rows; a workgroup has
// WAVES waves, and the kernel is held to the VGPR budget of MINW waves per
// SIMD (the second launch-bounds argument).  Large batches use 32-row tiles:
// one 128-bit weight read from LDS then feeds two MFMAs, which keeps the LDS
// port below its limit, and the activations of a tile take 2 x 16 (D = 128)
// or 2 x 8 (D = 64) VGPRs.  Three launch configurations per width, V, all
// compiled (the launcher picks 0 or 2 by batch size, the autotuner may pick
// any; every row gets the same bits):
//   V = 0            D = 128: 12 waves, one workgroup per CU (its 96 KB of
//                    weights fill the LDS), 3 waves per SIMD within 168
//                    VGPRs;  D = 64: 16 waves, 4 per SIMD within 128 VGPRs;
//   V = 1            D = 128: 8 waves, 2 per SIMD within 256 VGPRs;
//                    D = 64: 12 waves, 3 per SIMD within 168 VGPRs;
//   V = 2            as V = 0 with 16-row tiles: a batch of few tiles per
//                    wave runs each tile's layer chain in half the time.
template <int D, int V>
struct MlpCfg;
template <>
struct MlpCfg<128, 0> {
  static constexpr int WAVES = 12, MINW = 3, MT = 2;
};
template <>
struct MlpCfg<64, 0> {
  static constexpr int WAVES = 16, MINW = 4, MT = 2;
};
template <>
struct MlpCfg<128, 1> {
  static constexpr int WAVES = 8, MINW = 2, MT = 2;
};
template <>
struct MlpCfg<64, 1> {
  static constexpr int WAVES = 12, MINW = 3, MT = 2;
};
template <>
struct MlpCfg<128, 2> {
  static constexpr int WAVES = 12, MINW = 3, MT = 1;
};
template <>
struct MlpCfg<64, 2> {
  static constexpr int WAVES = 16, MINW = 4, MT = 1;
};

template <int D, int V = 0>
struct Geo {
  static constexpr int MT = MlpCfg<D, V>::MT;        // 16-row sub-tiles per wave tile
  static constexpr int WAVES = MlpCfg<D, V>::WAVES;  // waves per workgroup
  static constexpr int MINW = MlpCfg<D, V>::MINW;    // waves per SIMD the VGPR budget allows
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int TR = 16 * MT;  // rows per wave tile
  static constexpr int KS = D / 32;   // 32-deep k steps per layer
  static constexpr int NT = D / 16;   // 16-unit output sub-tiles per layer
};

// Activations of one row tile in MFMA B-operand form: v[s][ks] holds, for
// rows 16 s .. 16 s + 15, the 8 fp16 inputs of k step ks that this lane feeds
// (two per dword).
template <int D, int V>
struct HTile {
  u32x4 v[Geo<D, V>::MT][Geo<D, V>::KS];
};

template <int D>
__device__ __forceinline__ int w_offset(int l, int n, int slot) {
  return (l * D + n) * D + ((((slot >> 3) ^ wswz<D>(n))) << 3) + (slot & 7);
}

// Copy every W_l into LDS in the layout above.  One work item fills the
// 16-byte chunk cb of the 8 W^T rows n = 8 nb .. 8 nb + 7: it loads the 8
// rows of W_l (16 bytes each) whose units land in that chunk, transposes the
// 8 x 8 block in registers and writes 8 chunks of 16 bytes.
// With PAD the layer is the true dims[l] x dims[l+1] matrix (pitch dims[l+1])
// and every unit outside it is staged as zero.
template <int D, int L, bool PAD, int THREADS>
__device__ __forceinline__ void stage_weights(const MlpParams& p, _Float16* sW) {
  constexpr int NB = D / 8;  // 8-row blocks (and 16-byte chunks) per layer
  for (int idx = threadIdx.x; idx < L * NB * NB; idx += THREADS) {
    const int l = idx / (NB * NB);
    const int rem = idx - l * NB * NB;
    const int nb = rem / NB;
    const int cb = rem - nb * NB;
    const _Float16* Wl = (const _Float16*)p.W[l];
    const int K = PAD ? p.dims[l] : D, N = PAD ? p.dims[l + 1] : D;
    f16x8 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int slot = 8 * cb + j;
      const int k = l == 0 ? slot : layer_slot_k(slot);
      if (PAD && (k >= K || 8 * nb >= N))
        v[j] = (f16x8){0, 0, 0, 0, 0, 0, 0, 0};
      else
        v[j] = *(const f16x8*)(Wl + (int64_t)k * N + 8 * nb);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f16x8 o = (f16x8){v[0][i], v[1][i], v[2][i], v[3][i], v[4][i], v[5][i], v[6][i], v[7][i]};
      *(f16x8*)(sW + w_offset<D>(l, 8 * nb + i, 8 * cb)) = o;
    }
  }
}

// Per-lane constants of a wave.
template <int D>
struct Lane {
  uint32_t wk[Geo<D>::KS];  // LDS byte address of the lane's W^T fragment: layer 0, sub-tile 0, k step ks
  uint32_t xoff;            // byte offset of the lane's first x element in a 16-row sub-tile
  uint32_t ooff;            // byte offset of the lane's 16-byte output piece of sub-tiles 0 and 1 (see last_layer)
  uint32_t aoff;            // byte offset of the lane's first fp32 activation in a 16-row sub-tile (training forward)
};

template <int D>
__device__ __forceinline__ Lane<D> lane_setup(const MlpParams& p, const _Float16* sW, int lane) {
  Lane<D> c;
  const int q = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < Geo<D>::KS; ++ks) c.wk[ks] = lds_addr(sW) + 2u * (uint32_t)w_offset<D>(0, q, 32 * ks + 8 * g);
  const uint32_t xrow = (uint32_t)p.ldx * 2u, orow = (uint32_t)p.ldo * 2u;
  c.xoff = (uint32_t)q * xrow + 16u * (uint32_t)g;
  c.ooff = (uint32_t)q * orow + 32u * (uint32_t)(g & 1) + 16u * (uint32_t)(g >> 1);
  c.aoff = (uint32_t)q * (uint32_t)p.lda * 4u + 16u * (uint32_t)g;
  return c;
}

// Buffer resource over 16-row sub-tile s of row tile `tile` of a row-major
// fp16 matrix with pitch ld (elements) and M rows.  All arguments are
// wave-uniform.  The resource covers only the sub-tile's rows that exist:
// accesses at byte offsets at or beyond its size are dropped by the hardware
// (stores) or read as zero (loads), so the ragged last tile needs no branch.
// The host bounds the pitch by 2^24 elements, so 16 rows span less than 2^32
// bytes.
template <int D, int V>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sub_rsrc(const void* base, int M, int tile, int s, int64_t ld) {
  const int64_t first = (int64_t)tile * Geo<D, V>::TR + 16 * s;
  const int64_t rows = min((int64_t)16, max((int64_t)0, (int64_t)M - first));
  char* p = (char*)base + first * ld * 2;
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)((uint32_t)rows * (uint32_t)(ld * 2)), 0x00020000);
}

// As sub_rsrc, over the fp32 activation matrix acts[l] (pitch ld elements;
// the host bounds it by 2^24).
template <int D, int V>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t act_rsrc(float* base, int M, int tile, int s, int64_t ld) {
  const int64_t first = (int64_t)tile * Geo<D, V>::TR + 16 * s;
  const int64_t rows = min((int64_t)16, max((int64_t)0, (int64_t)M - first));
  char* p = (char*)base + first * ld * 4;
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)((uint32_t)rows * (uint32_t)(ld * 4)), 0x00020000);
}

// Stored activation of the training forward: h = act(z) in fp32 and natural
// units (the base-2 softplus output times ln 2), four consecutive units of
// one row per lane.
__device__ __forceinline__ void store_act(__amdgpu_buffer_rsrc_t rs, uint32_t off, float a0, float a1, float a2,
                                          float a3) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, (f32x4){a0, a1, a2, a3}), rs, off, 0, 0);
}

// Narrower chains (PAD): a lane's access to columns at or beyond the true
// width goes to a buffer offset past every resource's size (the host bounds
// 16 rows of any operand below 2^31 bytes), so the load reads zero and the
// store is dropped.
constexpr uint32_t OFF_NONE = 0x80000000u;
__device__ __forceinline__ uint32_t masked(bool ok, uint32_t off) { return ok ? off : OFF_NONE; }
__device__ __forceinline__ int lane_group() { return (int)(threadIdx.x & 63) >> 4; }

template <int D, int V, bool PAD>
__device__ __forceinline__ void load_x(const MlpParams& p, const Lane<D>& c, int tile, HTile<D, V>& h) {
  const uint32_t xoff = opaque(c.xoff);  // keeps the k-step offsets in the instructions' immediate field
#pragma unroll
  for (int s = 0; s < Geo<D, V>::MT; ++s) {
    const __amdgpu_buffer_rsrc_t rs = sub_rsrc<D, V>(p.x, p.M, tile, s, p.ldx);
#pragma unroll
    for (int ks = 0; ks < Geo<D>::KS; ++ks) {
      // units 32 ks + 8 g .. + 7 of the row
      const uint32_t off = PAD ? masked(32 * ks + 8 * lane_group() < p.dims[0], xoff + 64u * ks) : xoff + 64u * ks;
      h.v[s][ks] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    }
  }
}

// Hidden activations travel between layers in base-2 units, g = h / ln 2
// (h = softplus(z)), instead of h itself.  Then the next layer's accumulator
// is a = g W = z / ln 2 = z log2(e), exactly the argument the hardware
// exponential (2^x) wants, and
//   g' = softplus(z') / ln 2 = log2(1 + 2^a')
// costs exp2, add and log2, with no base-change multiplies.  The first
// layer, whose input x is in natural units, scales its accumulator by log2(e)
// once; the last layer scales its output by ln 2 once.  In exact arithmetic
// nothing changes; the fp16 operand is g rather than h (the same relative
// rounding).
//
// The page's guard (z > 20 passes z through) reads a > 20 log2(e) here.
// Below that threshold the guarded form is log2(1 + 2^a) exactly, so the
// per-element path computes only that (softplus_b2_fast) and keeps the
// maximum fp16 output of each lane.  log2(1 + 2^a) >= a, so an argument
// above the threshold (or +inf) shows as an output of at least 28 (a bound
// below the threshold that the rounding of exp2, log2 and fp16 cannot cross);
// a workgroup any of whose waves saw one recomputes all of its tiles from x
// with the guarded form (softplus_b2).  Both forms execute the same
// exp2/add/log2 instructions, so every result equals what the guarded form
// gives.  A NaN argument gives NaN in both forms; the maximum below
// propagates NaN (IEEE maximum), so a NaN also triggers the recompute (a slow
// path, not a different result).
constexpr float SP_THRESHOLD_B2 = 28.853900817779268f;  // 20 log2(e)
constexpr _Float16 SP_FLAG_B2_F16 = (_Float16)28.0f;

// Maximum of n packed fp16 pairs and m, in a tree of three-input packed
// maxima (v_pk_maximum3_f16: NaN in, NaN out): about n / 2 instructions with
// a short dependency chain.
template <int N>
__device__ __forceinline__ f16x2 max_tree(const f16x2 (&v)[N], f16x2 m) {
  if constexpr (N == 1) {
    return __builtin_elementwise_maximum(m, v[0]);
  } else if constexpr (N == 2) {
    return __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(v[0], v[1]));
  } else {
    constexpr int R = (N + 2) / 3;
    f16x2 r[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (3 * i + 2 < N)
        r[i] = __builtin_elementwise_maximum(v[3 * i], __builtin_elementwise_maximum(v[3 * i + 1], v[3 * i + 2]));
      else if (3 * i + 1 < N)
        r[i] = __builtin_elementwise_maximum(v[3 * i], v[3 * i + 1]);
      else
        r[i] = v[3 * i];
    }
    return max_tree<R>(r, m);
  }
}

__device__ __forceinline__ float softplus_b2_fast(float a) {
  return __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(a));
}
__device__ __forceinline__ float softplus_b2(float a) {
  const float s = softplus_b2_fast(a);
  return a > SP_THRESHOLD_B2 ? a : s;
}

// Issue order of one pipeline step: NM MFMAs, each followed by VPM VALU
// instructions (transcendentals included), a DS read after every DS_EVERY-th
// MFMA when DS is set, and a buffer store after every ST_EVERY-th MFMA when
// ST is set.
template <int NM, int VPM, bool DS, int DS_EVERY, bool ST, int ST_EVERY>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (DS && i % DS_EVERY == DS_EVERY - 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (ST && i % ST_EVERY == ST_EVERY - 1) __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, VPM, 0);
  }
}

// Hidden layer l for one row tile: hout = act(hin W_l), in the step pipeline
// described at the top, with the unguarded softplus; the largest output is
// folded into mx.
template <int D, int V, int l, int ACT, bool ST, bool PAD>
__device__ __forceinline__ void hidden_layer(const MlpParams& p, const Lane<D>& c, const HTile<D, V>& hin,
                                             HTile<D, V>& hout, f16x2& mx, int tile) {
  using G = Geo<D, V>;
  constexpr bool SP = ACT == ACT_SOFTPLUS;
  __amdgpu_buffer_rsrc_t ra[G::MT];
  uint32_t aoff = 0;
  if constexpr (ST) {
#pragma unroll
    for (int s = 0; s < G::MT; ++s) ra[s] = act_rsrc<D, V>(p.acts[l], p.M, tile, s, p.lda);
    aoff = opaque(c.aoff);
  }
  constexpr bool IN_B2 = SP && l > 0;  // does the accumulator arrive in base-2 units?
  // twice the VALU instructions per element: [scale] exp2 add log2, 1/2 pack
  constexpr int VPE2 = SP ? (IN_B2 ? 7 : 9) : 1;
  constexpr int VPM = (G::MT * 4 * VPE2 / 2 + G::KS * G::MT - 1) / (G::KS * G::MT);
  uint32_t wk[G::KS];
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) wk[ks] = opaque(c.wk[ks]) + 2u * (uint32_t)(l * D * D);
  // The first layer of a narrower chain runs only the k steps that hold
  // input units (k0 of them; the others would add products of zeros): k step
  // 0 inside the pipelined step, the rest in a branch after it.
  constexpr bool SKIPK = PAD && l == 0 && G::KS > 1;
  const int k0 = SKIPK ? (p.dims[0] + 31) >> 5 : G::KS;
  i16x8 wa[G::KS];
  f32x4 acc[G::MT], prv[G::MT];
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) wa[ks] = lds_read128(wk[ks]);
#pragma unroll
  for (int t = 0; t <= G::NT; ++t) {
    if (t < G::NT) {
#pragma unroll
      for (int s = 0; s < G::MT; ++s) acc[s] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < (SKIPK ? 1 : G::KS); ++ks) {
#pragma unroll
        for (int s = 0; s < G::MT; ++s) acc[s] = mfma16x16x32(wa[ks], __builtin_bit_cast(i16x8, hin.v[s][ks]), acc[s], _Float16());
        if (t + 1 < G::NT) wa[ks] = lds_read128(wk[ks] + 2u * (uint32_t)(16 * D * (t + 1)));
      }
    }
    if (t > 0) {
      const int u = t - 1;
#pragma unroll
      for (int s = 0; s < G::MT; ++s) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float a = prv[s][r];
          if constexpr (SP) {
            if constexpr (!IN_B2) a *= 1.44269504088896341f;
            v[r] = softplus_b2_fast(a);
          } else if constexpr (ACT == ACT_RELU) {
            v[r] = relu(a);
          } else {
            v[r] = a;
          }
        }
        hout.v[s][u >> 1][(u & 1) * 2] = pack_f16(v[0], v[1]);
        hout.v[s][u >> 1][(u & 1) * 2 + 1] = pack_f16(v[2], v[3]);
        if constexpr (ST) {
          const float sc = SP ? 0.693147180559945309f : 1.0f;
          // units 16 u + 4 g .. + 3
          const uint32_t off = PAD ? masked(16 * u + 4 * lane_group() < p.dims[l + 1], aoff + 64u * (uint32_t)u)
                                   : aoff + 64u * (uint32_t)u;
          store_act(ra[s], off, v[0] * sc, v[1] * sc, v[2] * sc, v[3] * sc);
        }
      }
    }
    if (t > 0 && t < G::NT) interleave<G::KS * G::MT, VPM, true, G::MT, ST, G::KS>();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (SKIPK) {
      if (t < G::NT && k0 > 1) {
#pragma unroll
        for (int ks = 1; ks < G::KS; ++ks) {
          if (ks < k0) {
#pragma unroll
            for (int s = 0; s < G::MT; ++s)
              acc[s] = mfma16x16x32(wa[ks], __builtin_bit_cast(i16x8, hin.v[s][ks]), acc[s], _Float16());
            if (t + 1 < G::NT) wa[ks] = lds_read128(wk[ks] + 2u * (uint32_t)(16 * D * (t + 1)));
          }
        }
      }
    }
#pragma unroll
    for (int s = 0; s < G::MT; ++s) prv[s] = acc[s];
  }
  if constexpr (SP) {
    // running maximum of the layer's fp16 outputs (two per dword)
    f16x2 h[G::MT * G::KS * 4];
#pragma unroll
    for (int s = 0; s < G::MT; ++s)
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) h[(s * G::KS + ks) * 4 + i] = __builtin_bit_cast(f16x2, hout.v[s][ks][i]);
    mx = max_tree(h, mx);
    // here, not later: deferring the maximum would keep every layer's
    // outputs alive until the end of the tile
    asm volatile("" : "+v"(mx));
  }
}

// Last layer l = L - 1 for one row tile: out = hin W_L (times ln 2 when hin
// is in base-2 units), fp16, stored through a buffer resource that drops the
// rows beyond M.
template <int D, int V, int l, int ACT, bool PAD>
__device__ __forceinline__ void last_layer(const MlpParams& p, const Lane<D>& c, const HTile<D, V>& hin,
                                           int tile) {
  using G = Geo<D, V>;
  constexpr bool IN_B2 = ACT == ACT_SOFTPLUS && l > 0;
  constexpr int VPM = (G::MT * 4 * (IN_B2 ? 3 : 1) / 2 + G::KS * G::MT - 1) / (G::KS * G::MT);
  constexpr int ST_EVERY = G::KS;  // MT stores per step (every other step) over KS * MT MFMAs
  __amdgpu_buffer_rsrc_t rs[G::MT];
#pragma unroll
  for (int s = 0; s < G::MT; ++s) rs[s] = sub_rsrc<D, V>(p.out, p.M, tile, s, p.ldo);
  const uint32_t ooff = opaque(c.ooff);  // keeps the sub-tile offsets in the instructions' immediate field
  uint32_t wk[G::KS];
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) wk[ks] = opaque(c.wk[ks]) + 2u * (uint32_t)(l * D * D);
  // A narrower chain computes only the pairs of 16-unit sub-tiles that hold
  // output units (nt of them), and a single-layer one only the k steps that
  // hold input units.
  const int nt = PAD ? 2 * ((p.dims[l + 1] + 31) >> 5) : G::NT;
  const int k0 = PAD && l == 0 ? (p.dims[0] + 31) >> 5 : G::KS;
  i16x8 wa[G::KS];
  f32x4 acc[G::MT], prv[G::MT];
  u32x2 ev[G::MT];  // packed output of the even sub-tile of a pair
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) wa[ks] = lds_read128(wk[ks]);
#pragma unroll
  for (int t = 0; t <= G::NT; ++t) {
    if (t < G::NT && (!PAD || t < nt)) {
#pragma unroll
      for (int s = 0; s < G::MT; ++s) acc[s] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) {
        if (PAD && l == 0 && ks >= k0) continue;
#pragma unroll
        for (int s = 0; s < G::MT; ++s) acc[s] = mfma16x16x32(wa[ks], __builtin_bit_cast(i16x8, hin.v[s][ks]), acc[s], _Float16());
        if (t + 1 < G::NT) wa[ks] = lds_read128(wk[ks] + 2u * (uint32_t)(16 * D * (t + 1)));
      }
    }
    if (t > 0 && (!PAD || t - 1 < nt)) {
      const int u = t - 1;
#pragma unroll
      for (int s = 0; s < G::MT; ++s) {
        const float sc = IN_B2 ? 0.693147180559945309f : 1.0f;
        const u32x2 o = (u32x2){pack_f16(prv[s][0] * sc, prv[s][1] * sc), pack_f16(prv[s][2] * sc, prv[s][3] * sc)};
        if (u % 2 == 0)
          ev[s] = o;
        else
          store_pair(rs[s],
                     PAD ? masked(16 * (u - 1) + 16 * (lane_group() & 1) + 8 * (lane_group() >> 1) < p.dims[l + 1],
                                  ooff + 32u * (uint32_t)(u - 1))
                         : ooff + 32u * (uint32_t)(u - 1),
                     ev[s], o);
      }
    }
    if (t > 0 && t < G::NT) interleave<G::KS * G::MT, VPM, true, G::MT, true, ST_EVERY>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < G::MT; ++s) prv[s] = acc[s];
  }
}

// One row tile with the guarded softplus, one 16-row sub-tile at a time and
// without the step pipeline: the rarely taken path, kept small in registers.
// Per element it executes the same MFMA accumulation order and the same
// exp2/add/log2/pack instructions as the pipelined path, so it reproduces
// that path's bits wherever the guard does not apply.
template <int D, int V, int L, int ACT, bool ST, bool PAD>
__device__ __forceinline__ void tile_guarded(const MlpParams& p, const Lane<D>& c, int tile) {
  using G = Geo<D, V>;
  constexpr bool SP = ACT == ACT_SOFTPLUS;
#pragma unroll 1
  for (int s = 0; s < G::MT; ++s) {
    const __amdgpu_buffer_rsrc_t rx = sub_rsrc<D, V>(p.x, p.M, tile, s, p.ldx);
    const __amdgpu_buffer_rsrc_t ro = sub_rsrc<D, V>(p.out, p.M, tile, s, p.ldo);
    const uint32_t xoff = opaque(c.xoff), ooff = opaque(c.ooff);
    // hn and ev fully defined on every path (the last layer writes neither,
    // and h is not copied from hn after it): with undefined lanes in that
    // loop-carried copy, the 16-row-tile build of this path reused the
    // registers of the loaded x before the first layer read them
    u32x4 h[G::KS], hn[G::KS];
    u32x2 ev = (u32x2){0u, 0u};
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) hn[ks] = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks)
      h[ks] = __builtin_amdgcn_raw_buffer_load_b128(
          rx, PAD ? masked(32 * ks + 8 * lane_group() < p.dims[0], xoff + 64u * ks) : xoff + 64u * ks, 0, 0);
    // the k steps and output sub-tiles the pipelined path computes (it skips
    // products of zeros), so that both paths give the same bits
    const int k0 = PAD ? (p.dims[0] + 31) >> 5 : G::KS;
    const int ntl = PAD ? 2 * ((p.dims[L] + 31) >> 5) : G::NT;
#pragma unroll 1
    for (int l = 0; l < L; ++l) {
      const bool in_b2 = SP && l > 0;
#pragma unroll
      for (int t = 0; t < G::NT; ++t) {
        if (l == L - 1 && t >= ntl) continue;
        f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
          if (l == 0 && ks >= k0) continue;
          const i16x8 wa = lds_read128(opaque(c.wk[ks]) + 2u * (uint32_t)(l * D * D + 16 * D * t));
          acc = mfma16x16x32(wa, __builtin_bit_cast(i16x8, h[ks]), acc, _Float16());
        }
        if (l + 1 < L) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float a = acc[r];
            if (SP) {
              if (!in_b2) a *= 1.44269504088896341f;
              v[r] = softplus_b2(a);
            } else {
              v[r] = a;
            }
          }
          hn[t >> 1][(t & 1) * 2] = pack_f16(v[0], v[1]);
          hn[t >> 1][(t & 1) * 2 + 1] = pack_f16(v[2], v[3]);
          if constexpr (ST) {
            const float sc = SP ? 0.693147180559945309f : 1.0f;
            const uint32_t off = opaque(c.aoff) + 64u * (uint32_t)t;
            store_act(act_rsrc<D, V>(p.acts[l], p.M, tile, s, p.lda),
                      PAD ? masked(16 * t + 4 * lane_group() < p.dims[l + 1], off) : off, v[0] * sc, v[1] * sc,
                      v[2] * sc, v[3] * sc);
          }
        } else {
          const float sc = in_b2 ? 0.693147180559945309f : 1.0f;
          const u32x2 o = (u32x2){pack_f16(acc[0] * sc, acc[1] * sc), pack_f16(acc[2] * sc, acc[3] * sc)};
          if (t % 2 == 0)
            ev = o;
          else
            store_pair(ro,
                       PAD ? masked(16 * (t - 1) + 16 * (lane_group() & 1) + 8 * (lane_group() >> 1) < p.dims[L],
                                    ooff + 32u * (uint32_t)(t - 1))
                           : ooff + 32u * (uint32_t)(t - 1),
                       ev, o);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (l + 1 < L) {
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) h[ks] = hn[ks];
      }
    }
  }
}

// One row tile, layers l .. L-1.  hin holds the layer-l input; hfree is free.
// mx collects the largest unguarded softplus output.
template <int D, int V, int L, int l, int ACT, bool ST, bool PAD>
__device__ __forceinline__ void tile_chain(const MlpParams& p, const Lane<D>& c, int tile, HTile<D, V>& hin,
                                           HTile<D, V>& hfree, f16x2& mx) {
  if constexpr (l < L - 1) {
    hidden_layer<D, V, l, ACT, ST, PAD>(p, c, hin, hfree, mx, tile);
    tile_chain<D, V, L, l + 1, ACT, ST, PAD>(p, c, tile, hfree, hin, mx);
  } else {
    last_layer<D, V, l, ACT, PAD>(p, c, hin, tile);
  }
}

// The next of the workgroup's tiles for the calling wave: one LDS atomic by
// lane 0, its result broadcast to the wave.  Workgroup b's k-th tile is
// b + k G.
__device__ __forceinline__ int claim_tile(int* counter) {
  int k = 0;
  if ((threadIdx.x & 63) == 0) k = atomicAdd(counter, 1);
  return (int)blockIdx.x + __builtin_amdgcn_readfirstlane(k) * (int)gridDim.x;
}

// Several waves per SIMD (MINW) so that memory latency and the dependent
// activation chains of some waves hide behind the work of others.
template <int D, int L, int ACT, bool ST, bool PAD, int V>
__global__ __launch_bounds__((Geo<D, V>::THREADS), (Geo<D, V>::MINW)) void mlp_kernel(MlpParams p) {
  using G = Geo<D, V>;
  __shared__ __attribute__((aligned(16))) _Float16 sW[L * D * D];
  __shared__ int s_next;      // the workgroup's next unclaimed tile (local index)
  __shared__ unsigned s_flag;  // some wave saw a softplus argument past the guard
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (threadIdx.x == 0) {
    s_next = G::WAVES;  // local tiles 0 .. WAVES - 1 are the waves' first ones
    s_flag = 0;
  }
  stage_weights<D, L, PAD, G::THREADS>(p, sW);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const Lane<D> c = lane_setup<D>(p, sW, lane);
  f16x2 mx = (f16x2){0, 0};
  int tile = (int)blockIdx.x + wv * (int)gridDim.x;
  // Three activation buffers in rotation: the x of the next tile is loaded
  // into the third one when a tile starts, a whole tile ahead of its use.
  // The load is issued even past the last tile (its buffer resources cover
  // zero rows, so it reads zeros without touching memory): a conditional
  // load would make the compiler wait for every outstanding memory operation
  // where the paths join, stores included.
  HTile<D, V> ha, hb, hc;
  if (tile < p.num_tiles) load_x<D, V, PAD>(p, c, tile, ha);
  // The compiler's memory-counter waits at the loop head are those of the
  // loop entry and of the back edge merged.  Entered with this load still in
  // flight, the first use of ha waited as if it had just been issued -- on
  // every pass, which then also waited for the previous tile's output stores
  // (the counter completes in order).  Waiting here once leaves only the
  // back edge's wait: for data loaded a whole tile earlier.  (The builtin,
  // not inline asm: the compiler's wait insertion sees only the former.)
  // Encoding: vmcnt 0, expcnt 7 and lgkmcnt 15 (no wait on those two).
  __builtin_amdgcn_s_waitcnt(0x0F70);
  while (tile < p.num_tiles) {
    int next = claim_tile(&s_next);
    load_x<D, V, PAD>(p, c, next, hc);
    tile_chain<D, V, L, 0, ACT, ST, PAD>(p, c, tile, ha, hb, mx);
    tile = next;
    if (tile >= p.num_tiles) break;
    next = claim_tile(&s_next);
    load_x<D, V, PAD>(p, c, next, hb);
    tile_chain<D, V, L, 0, ACT, ST, PAD>(p, c, tile, hc, ha, mx);
    tile = next;
    if (tile >= p.num_tiles) break;
    next = claim_tile(&s_next);
    load_x<D, V, PAD>(p, c, next, ha);
    tile_chain<D, V, L, 0, ACT, ST, PAD>(p, c, tile, hb, hc, mx);
    tile = next;
  }
  if constexpr (ACT == ACT_SOFTPLUS && L > 1) {
    // Some softplus argument of the workgroup's tiles may have exceeded the
    // guard threshold: then its waves recompute all of the workgroup's tiles
    // with the guarded form.  Tiles without such an argument get the same
    // bits again; the others are corrected.  Every wave's first results are
    // complete in memory (its own wait, then the barrier) before any wave
    // overwrites them.
    const bool big = !(mx[0] < SP_FLAG_B2_F16 && mx[1] < SP_FLAG_B2_F16);  // also for NaN
    if (__builtin_amdgcn_ballot_w64(big) != 0 && lane == 0) s_flag = 1u;
    __syncthreads();
    if (s_flag != 0u) {
      wait_vmcnt0();
      __syncthreads();
      for (int t = (int)blockIdx.x + wv * (int)gridDim.x; t < p.num_tiles; t += G::WAVES * (int)gridDim.x)
        tile_guarded<D, V, L, ACT, ST, PAD>(p, c, t);
    }
  }
}

// Persistent grid (unless the caller fixed the count): see below; at most
// #CUs x workgroups that fit on a CU.  The per-CU occupancy comes from
// the runtime for the compiled kernel (its VGPR and LDS use) and is cached.
template <int D, int L, int ACT, bool ST, bool PAD, int V>
hipError_t launch_dl(MlpParams p, int num_workgroups, int num_cus, hipStream_t stream) {
  using G = Geo<D, V>;
  p.num_tiles = (int)(((int64_t)p.M + G::TR - 1) / G::TR);
  // (atomic: concurrent first calls from several host threads store the
  // same value)
  static std::atomic<int> per_cu_cache{0};
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int n = 0;
    hipError_t e =
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mlp_kernel<D, L, ACT, ST, PAD, V>, G::THREADS, 0);
    if (e != hipSuccess) return e;
    per_cu = n > 0 ? n : 1;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  int nwg = num_workgroups;
  if (nwg <= 0) {
    // enough workgroups to give every wave a tile, but at least one per CU
    // while there are tiles for them: a small batch spread over the CUs (one
    // or two tiles per workgroup) finishes sooner than the same tiles packed
    // into full workgroups on a few CUs (4096 rows of 3 x 128: 8.7 against
    // 14.7 us)
    const long need = (p.num_tiles + G::WAVES - 1) / G::WAVES;
    const long spread = p.num_tiles < num_cus ? p.num_tiles : num_cus;
    const long want = need > spread ? need : spread;
    const long cap = (long)num_cus * per_cu;
    nwg = (int)(want < cap ? want : cap);
    if (nwg < 1) nwg = 1;
  }
  hipLaunchKernelGGL((mlp_kernel<D, L, ACT, ST, PAD, V>), dim3(nwg), dim3(G::THREADS), 0, stream, p);
  return hipGetLastError();
}

template <int D, int ACT, bool ST, bool PAD, int V>
hipError_t launch_d(const MlpParams& p, int L, int nwg, int cus, hipStream_t stream) {
  if constexpr (D == 128) {
    switch (L) {
      case 1: return launch_dl<D, 1, ACT, ST, PAD, V>(p, nwg, cus, stream);
      case 2: return launch_dl<D, 2, ACT, ST, PAD, V>(p, nwg, cus, stream);
      case 3: return launch_dl<D, 3, ACT, ST, PAD, V>(p, nwg, cus, stream);
      case 4: return launch_dl<D, 4, ACT, ST, PAD, V>(p, nwg, cus, stream);
    }
  } else {
    switch (L) {
      case 1: return launch_dl<D, 1, ACT, ST, PAD, V>(p, nwg, cus, stream);
      case 2: return launch_dl<D, 2, ACT, ST, PAD, V>(p, nwg, cus, stream);
      case 3: return launch_dl<D, 3, ACT, ST, PAD, V>(p, nwg, cus, stream);
      case 4: return launch_dl<D, 4, ACT, ST, PAD, V>(p, nwg, cus, stream);
      case 5: return launch_dl<D, 5, ACT, ST, PAD, V>(p, nwg, cus, stream);
      case 6: return launch_dl<D, 6, ACT, ST, PAD, V>(p, nwg, cus, stream);
      case 7: return launch_dl<D, 7, ACT, ST, PAD, V>(p, nwg, cus, stream);
      case 8: return launch_dl<D, 8, ACT, ST, PAD, V>(p, nwg, cus, stream);
    }
  }
  return hipErrorInvalidValue;
}

template <int D, bool ST, bool PAD, int V>
hipError_t launch_da(const MlpParams& p, int L, int act, int nwg, int cus, hipStream_t stream) {
  if (act == ACT_NONE) return launch_d<D, ACT_NONE, ST, PAD, V>(p, L, nwg, cus, stream);
  if (act == ACT_RELU) return launch_d<D, ACT_RELU, ST, PAD, V>(p, L, nwg, cus, stream);
  return launch_d<D, ACT_SOFTPLUS, ST, PAD, V>(p, L, nwg, cus, stream);
}

}  // namespace
}  // namespace coalesce
