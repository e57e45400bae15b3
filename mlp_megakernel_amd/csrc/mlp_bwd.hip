// Backward of the softplus-MLP chain in one persistent launch ("MLP
// Megakernel" README, "Key ideas": the training forward stores the hidden
// activations in fp32, the backward recovers the softplus derivative from
// them and casts to fp16 only for the matrix-core operands; the weight
// gradients of all layers come out of the same fused kernel).
//
// With h_0 = x, z_{l+1} = h_l W_l (0-based W_0..W_{L-1}), h_l = act(z_l) and
// the upstream gradient dz_L = dout, per row tile and per layer
// l = L-1 .. 0:
//   dW_l += h_l^T dz_{l+1}                    (contraction over rows)
//   dz_l  = (dz_{l+1} W_l^T) * act'(z_l)      (l > 0; contraction over units)
//   dx    =  dz_1 W_0^T                       (l = 0, optional)
// act'(z_l) is recovered from the stored h_l = act(z_l):
//   softplus: sigmoid(z) = 1 - exp(-h) (a four-term series below h = 2^-6,
//             where the subtraction would cancel);
//   relu: h > 0;  none: 1.
//
// Design for gfx950:
//   * a workgroup of 4 waves (one per SIMD, 512 registers a lane) owns a
//     tile of R rows per step; the grid is one workgroup per CU and walks the
//     row tiles round-robin;
//   * data gradients: each wave owns 16 MT rows of the tile and computes
//     dz_l^T = W_l dz_{l+1}^T with v_mfma_f32_16x16x32_f16, A = a W_l
//     fragment from LDS, B = dz_{l+1} in registers.  The result layout (4
//     consecutive units of one row per lane) is the next layer's B operand
//     without data movement, exactly as in the forward megakernel, with the
//     induced unit order absorbed into how W_l sits in LDS;
//   * weight gradients: dW_l is split into four D/2 x D/2 blocks, one per
//     wave, and accumulated in registers over all of the workgroup's tiles.
//     The contraction runs over rows, so h_l and dz_{l+1} of the whole tile
//     are staged in LDS as fp16 (row-major, 32-byte chunks XOR-swizzled by
//     row) and read back with the transposing ds_read_b64_tr_b16, which
//     hands every lane 4 consecutive rows of one column;
//   * h_l comes from the fp32 activations loaded once per layer: the same
//     registers give the fp16 staging copy and the derivative;
//   * the loads of the next layer's activations (and of the next tile's
//     dout) are issued a layer ahead, and the barriers around the staging
//     buffers do not wait for them;
//   * at the end every workgroup writes its partial dW to a workspace and a
//     second kernel sums the partials in workgroup order: the result is
//     deterministic for a given grid (the pages' design accumulates with
//     atomics below 32K rows and calls GEMMs above).
#include "common.hpp"
#include "launch.hpp"
#include "mlp_common.hpp"

namespace coalesce {
namespace {

template <int D>
struct BGeo {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int MT = D == 128 ? 1 : 2;  // 16-row sub-tiles per wave
  static constexpr int R = 16 * MT * WAVES;     // rows per workgroup tile
  static constexpr int KS = D / 32;             // 32-deep k steps of a data-gradient product
  static constexpr int NT = D / 16;             // 16-unit output sub-tiles
  static constexpr int QB = D / 32;             // 16 x 16 dW blocks per wave along each side
  static constexpr int CH = R / 32;             // 32-row chunks of a tile
};

// Staging buffers sH (h_l) and sZ (dz_{l+1}): R rows x D fp16, rows of 2D
// bytes, 32-byte chunk c (16 units) of row r at chunk position c ^ sfz(r).
// Both access patterns then spread over all banks:
//   * writes by 16 consecutive rows (one 8-byte piece each, lane groups
//     side by side) hit every 32-byte position of a 256-byte window twice;
//   * a transposing read by the 4 lane groups (rows 8 g + 4 h + 0..3 of a
//     32-row chunk, one chunk each) hits every position twice.
template <int D>
__device__ __forceinline__ int sfz(int r) {
  if constexpr (D == 128)
    return (r & 3) | (((r >> 3) & 1) << 2);
  else
    return ((r >> 1) & 1) | (((r >> 3) & 1) << 1);
}

// Weights in LDS: W_l as D rows k of D fp16, 16-byte chunks swizzled by
// wswz.  Layer L-1 is fed by dout (natural unit order); the others by the
// registers of the layer above, whose unit order is that of layer_k_slot.
template <int D, int L>
__device__ __forceinline__ void stage_weights_bwd(const MlpBwdParams& p, _Float16* sW) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  for (int idx = threadIdx.x; idx < L * D * CPR; idx += BGeo<D>::THREADS) {
    const int l = idx / (D * CPR);
    const int rem = idx - l * D * CPR;
    const int k = rem / CPR;
    const int cb = rem - k * CPR;
    const _Float16* row = (const _Float16*)p.W[l] + (int64_t)k * D;
    f16x8 v;
    if (l == L - 1) {
      v = *(const f16x8*)(row + 8 * cb);
    } else {
      // slots 8 cb .. 8 cb + 7 (cb = 4 a + b) hold units 32 a + 4 b + 0..3
      // and 32 a + 16 + 4 b + 0..3
      const int a = cb >> 2, b = cb & 3;
      const f16x4 lo = *(const f16x4*)(row + 32 * a + 4 * b);
      const f16x4 hi = *(const f16x4*)(row + 32 * a + 16 + 4 * b);
      v = (f16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    *(f16x8*)(sW + (l * D + k) * D + ((cb ^ wswz<D>(k)) << 3)) = v;
  }
}

// Per-lane constants.
template <int D>
struct BLane {
  uint32_t wk[BGeo<D>::KS];  // LDS byte address of the lane's W fragment: layer 0, sub-tile 0, k step ks
  uint32_t st8;              // staging byte offset of the lane's 8-byte piece (D layout), sub-tile 0, unit block 0
  uint32_t st16;             // staging byte offset of the lane's 16-byte piece (B layout), sub-tile 0, k step 0
  uint32_t trk;              // staging byte offset of the lane's transposing read, chunk 0 (before the block XOR)
  uint32_t boff;             // global byte offset of the lane's 16-byte fp16 piece in a 16-row sub-tile (x, dout)
  uint32_t aoff;             // global byte offset of the lane's 16-byte fp32 piece in a 16-row sub-tile (acts)
  uint32_t qoff;             // global byte offset of the lane's paired dx store (see store_pair)
};

template <int D>
__device__ __forceinline__ BLane<D> blane_setup(const MlpBwdParams& p, const _Float16* sW, int w, int lane) {
  using G = BGeo<D>;
  BLane<D> c;
  const int q = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks)
    c.wk[ks] = lds_addr(sW) + 2u * (uint32_t)(q * D + (((4 * ks + g) ^ wswz<D>(q)) << 3));
  const int r = 16 * G::MT * w + q;  // the lane's row in sub-tile 0 of its wave
  c.st8 = (uint32_t)(r * 2 * D + (sfz<D>(r) << 5) + (g << 3));
  c.st16 = (uint32_t)(r * 2 * D + (((g >> 1) ^ sfz<D>(r)) << 5) + ((g & 1) << 4));
  const int rt = 8 * g + (q >> 2);  // row of the first transposing read in a 32-row chunk
  c.trk = (uint32_t)(rt * 2 * D + (sfz<D>(rt) << 5) + ((q & 3) << 3));
  c.boff = (uint32_t)q * (uint32_t)p.ldx * 2u + 16u * (uint32_t)g;  // x; dout uses its own pitch below
  c.aoff = (uint32_t)q * (uint32_t)p.lda * 4u + 16u * (uint32_t)g;
  c.qoff = (uint32_t)q * (uint32_t)p.ldq * 2u + 32u * (uint32_t)(g & 1) + 16u * (uint32_t)(g >> 1);
  return c;
}

// Buffer resource over 16-row sub-tile s of wave w of row tile `tile` of a
// matrix with pitch ld elements of es bytes and M rows: rows past M read as
// zero and are never written.  The host bounds ld * es * 16 below 2^32.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void* base, int M, int tile, int w, int s, int64_t ld,
                                                        int es) {
  using G = BGeo<D>;
  const int64_t first = (int64_t)tile * G::R + 16 * (G::MT * w + s);
  const int64_t rows = min((int64_t)16, max((int64_t)0, (int64_t)M - first));
  const char* p = (const char*)base + first * ld * es;
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)((uint32_t)rows * (uint32_t)(ld * es)),
                                           0x00020000);
}

template <int D>
struct FragB {  // fp16 B-operand layout: v[s][ks] = 8 units of k step ks of the lane's row in sub-tile s
  u32x4 v[BGeo<D>::MT][BGeo<D>::KS];
};
template <int D>
struct RowsF32 {  // fp32 result layout: v[s][t] = units 16 t + 4 g .. + 3 of the lane's row in sub-tile s
  f32x4 v[BGeo<D>::MT][BGeo<D>::NT];
};

template <int D>
__device__ __forceinline__ void load_b(const void* base, int64_t ld, uint32_t off, int M, int tile, int w,
                                       FragB<D>& f) {
#pragma unroll
  for (int s = 0; s < BGeo<D>::MT; ++s) {
    const __amdgpu_buffer_rsrc_t rs = brsrc<D>(base, M, tile, w, s, ld, 2);
#pragma unroll
    for (int ks = 0; ks < BGeo<D>::KS; ++ks) f.v[s][ks] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64u * ks, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void load_acts(const float* base, int64_t ld, uint32_t off, int M, int tile, int w,
                                          RowsF32<D>& f) {
#pragma unroll
  for (int s = 0; s < BGeo<D>::MT; ++s) {
    const __amdgpu_buffer_rsrc_t rs = brsrc<D>(base, M, tile, w, s, ld, 4);
#pragma unroll
    for (int t = 0; t < BGeo<D>::NT; ++t)
      f.v[s][t] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64u * t, 0, 0));
  }
}

__device__ __forceinline__ void lds_write64(uint32_t addr, u32x2 v) {
  *(__attribute__((address_space(3))) u32x2*)(uintptr_t)addr = v;
}
__device__ __forceinline__ void lds_write128(uint32_t addr, u32x4 v) {
  *(__attribute__((address_space(3))) u32x4*)(uintptr_t)addr = v;
}
__device__ __forceinline__ i16x4 lds_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)addr);
}

// Stage a B-layout fp16 tile (dout or x) into a staging buffer.
template <int D>
__device__ __forceinline__ void stage_b(uint32_t buf, const BLane<D>& c, const FragB<D>& f) {
#pragma unroll
  for (int s = 0; s < BGeo<D>::MT; ++s)
#pragma unroll
    for (int ks = 0; ks < BGeo<D>::KS; ++ks)
      lds_write128((buf + c.st16 + 16u * 2 * D * s) ^ (uint32_t)(2 * ks << 5), f.v[s][ks]);
}

// Stage the packed fp16 D-layout pieces held in B-operand form: unit block t
// of sub-tile s is dwords (t & 1) * 2, + 1 of v[s][t / 2].
template <int D>
__device__ __forceinline__ void stage_d(uint32_t buf, const BLane<D>& c, const FragB<D>& f) {
#pragma unroll
  for (int s = 0; s < BGeo<D>::MT; ++s)
#pragma unroll
    for (int t = 0; t < BGeo<D>::NT; ++t)
      lds_write64((buf + c.st8 + 16u * 2 * D * s) ^ (uint32_t)(t << 5),
                  (u32x2){f.v[s][t >> 1][(t & 1) * 2], f.v[s][t >> 1][(t & 1) * 2 + 1]});
}

// fp32 activations -> fp16 pieces in B-operand form (the same packing the
// data-gradient step produces), for staging.
template <int D>
__device__ __forceinline__ void pack_rows(const RowsF32<D>& a, FragB<D>& f) {
#pragma unroll
  for (int s = 0; s < BGeo<D>::MT; ++s)
#pragma unroll
    for (int t = 0; t < BGeo<D>::NT; ++t) {
      f.v[s][t >> 1][(t & 1) * 2] = pack_f16(a.v[s][t][0], a.v[s][t][1]);
      f.v[s][t >> 1][(t & 1) * 2 + 1] = pack_f16(a.v[s][t][2], a.v[s][t][3]);
    }
}

// Derivative of the hidden activation from its stored output h = act(z).
template <int ACT>
__device__ __forceinline__ float act_grad(float h) {
  if constexpr (ACT == ACT_SOFTPLUS) {
    // sigmoid(z) = 1 - e^{-h}; below h = 2^-6 the series
    // h (1 - h (1/2 - h (1/6 - h / 24))) (truncation below 2^-25 relative)
    const float big = 1.0f - __builtin_amdgcn_exp2f(h * -1.44269504088896341f);
    const float small = h * __builtin_fmaf(-h, __builtin_fmaf(-h, __builtin_fmaf(-h, 0.0416666679f, 0.166666672f), 0.5f), 1.0f);
    return h < 0.015625f ? small : big;
  } else if constexpr (ACT == ACT_RELU) {
    return h > 0.0f ? 1.0f : 0.0f;
  } else {
    return 1.0f;
  }
}

// dW_l(wave block) += sH^T sZ over the tile's R rows.
template <int D>
__device__ __forceinline__ void weight_grad(uint32_t sH, uint32_t sZ, const BLane<D>& c, int w,
                                            f32x4 (&dw)[BGeo<D>::QB][BGeo<D>::QB]) {
  using G = BGeo<D>;
  const uint32_t kb0 = (uint32_t)(G::QB * (w >> 1)), nb0 = (uint32_t)(G::QB * (w & 1));
  uint32_t ha[G::QB], zb[G::QB];
#pragma unroll
  for (int b = 0; b < G::QB; ++b) {
    ha[b] = (sH + c.trk) ^ ((kb0 + b) << 5);
    zb[b] = (sZ + c.trk) ^ ((nb0 + b) << 5);
  }
#pragma unroll
  for (int j = 0; j < G::CH; ++j) {
    i16x8 a[G::QB], b[G::QB];
#pragma unroll
    for (int i = 0; i < G::QB; ++i) {
      const uint32_t r0 = (uint32_t)(32 * j * 2 * D), r4 = (uint32_t)((32 * j + 4) * 2 * D);
      const i16x4 a0 = lds_tr(ha[i] + r0), a1 = lds_tr(ha[i] + r4);
      const i16x4 b0 = lds_tr(zb[i] + r0), b1 = lds_tr(zb[i] + r4);
      a[i] = (i16x8){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      b[i] = (i16x8){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    }
#pragma unroll
    for (int i = 0; i < G::QB; ++i)
#pragma unroll
      for (int k = 0; k < G::QB; ++k) dw[i][k] = mfma16x16x32(a[i], b[k], dw[i][k], _Float16());
  }
}

// dz_l = (dz_{l+1} W_l^T) * act'(h_l) for the wave's rows: B operand dz
// (registers), A operand W_l (LDS), result packed to fp16 in B form.
template <int D, int l, int ACT>
__device__ __forceinline__ void data_grad(const BLane<D>& c, const FragB<D>& dz, const RowsF32<D>& h,
                                          FragB<D>& out) {
  using G = BGeo<D>;
#pragma unroll
  for (int t = 0; t < G::NT; ++t) {
    f32x4 acc[G::MT];
#pragma unroll
    for (int s = 0; s < G::MT; ++s) acc[s] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      const i16x8 wa = lds_read128(opaque(c.wk[ks]) + 2u * (uint32_t)((l * D + 16 * t) * D));
#pragma unroll
      for (int s = 0; s < G::MT; ++s) acc[s] = mfma16x16x32(wa, __builtin_bit_cast(i16x8, dz.v[s][ks]), acc[s], _Float16());
    }
#pragma unroll
    for (int s = 0; s < G::MT; ++s) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = ACT == ACT_NONE ? acc[s][i] : acc[s][i] * act_grad<ACT>(h.v[s][t][i]);
      out.v[s][t >> 1][(t & 1) * 2] = pack_f16(v[0], v[1]);
      out.v[s][t >> 1][(t & 1) * 2 + 1] = pack_f16(v[2], v[3]);
    }
  }
}

// dx = dz_1 W_0^T for the wave's rows, stored as fp16 in pairs of unit blocks.
template <int D>
__device__ __forceinline__ void input_grad(const MlpBwdParams& p, const BLane<D>& c, const FragB<D>& dz, int tile,
                                           int w) {
  using G = BGeo<D>;
  __amdgpu_buffer_rsrc_t rs[G::MT];
#pragma unroll
  for (int s = 0; s < G::MT; ++s) rs[s] = brsrc<D>(p.dx, p.M, tile, w, s, p.ldq, 2);
  const uint32_t qoff = opaque(c.qoff);
  u32x2 ev[G::MT];
#pragma unroll
  for (int t = 0; t < G::NT; ++t) {
    f32x4 acc[G::MT];
#pragma unroll
    for (int s = 0; s < G::MT; ++s) acc[s] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      const i16x8 wa = lds_read128(opaque(c.wk[ks]) + 2u * (uint32_t)(16 * t * D));
#pragma unroll
      for (int s = 0; s < G::MT; ++s) acc[s] = mfma16x16x32(wa, __builtin_bit_cast(i16x8, dz.v[s][ks]), acc[s], _Float16());
    }
#pragma unroll
    for (int s = 0; s < G::MT; ++s) {
      const u32x2 o = (u32x2){pack_f16(acc[s][0], acc[s][1]), pack_f16(acc[s][2], acc[s][3])};
      if (t % 2 == 0)
        ev[s] = o;
      else
        store_pair(rs[s], qoff + 32u * (uint32_t)(t - 1), ev[s], o);
    }
  }
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Barrier that waits only for the wave's own LDS accesses, not for its
// outstanding global loads (the prefetches stay in flight across it).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
#pragma clang diagnostic pop

// Registers carried through a tile.
template <int D>
struct BState {
  FragB<D> dz;    // dz_{l+1} of the wave's rows (B form)
  FragB<D> nz;    // dz_l being produced
  RowsF32<D> h;   // h_l of the wave's rows (fp32): derivative source
  RowsF32<D> ha;  // prefetch: the next fp32 activation layer
  FragB<D> hx;    // prefetch: x (B form)
  FragB<D> dn;    // prefetch: dout of the next tile
};

// Issue the load of h_j for `tile` (j >= 1: fp32 acts[j - 1]; j == 0: x).
template <int D>
__device__ __forceinline__ void prefetch_h(const MlpBwdParams& p, const BLane<D>& c, int j, int tile, int w,
                                           BState<D>& st) {
  if (j >= 1)
    load_acts<D>(p.acts[j - 1], p.lda, opaque(c.aoff), p.M, tile, w, st.ha);
  else
    load_b<D>(p.x, p.ldx, opaque(c.boff), p.M, tile, w, st.hx);
}

// Layers l .. 0 of one tile.  On entry sH holds h_l and sZ holds dz_{l+1}
// (this wave's rows written, the barrier not yet passed), st.dz holds
// dz_{l+1}, st.h holds h_l (l >= 1), and the load of h_{l-1} (or of the
// next tile's h_{L-1} when l == 0) is in flight.
template <int D, int L, int l, int ACT, bool DX>
__device__ __forceinline__ void tile_layers(const MlpBwdParams& p, const BLane<D>& c, uint32_t sH, uint32_t sZ,
                                            int tile, int next, int w, BState<D>& st,
                                            f32x4 (&dw)[L][BGeo<D>::QB][BGeo<D>::QB]) {
  lds_barrier();
  weight_grad<D>(sH, sZ, c, w, dw[l]);
  if constexpr (l >= 1) {
    data_grad<D, l, ACT>(c, st.dz, st.h, st.nz);
    lds_barrier();
    st.dz = st.nz;
    stage_d<D>(sZ, c, st.dz);
    if constexpr (l - 1 >= 1) {
      FragB<D> hp;
      pack_rows<D>(st.ha, hp);
      stage_d<D>(sH, c, hp);
      st.h = st.ha;
    } else {
      stage_b<D>(sH, c, st.hx);
    }
    if constexpr (l - 2 >= 0)
      prefetch_h<D>(p, c, l - 2, tile, w, st);
    else if (next < p.num_tiles)
      prefetch_h<D>(p, c, L - 1, next, w, st);
    tile_layers<D, L, l - 1, ACT, DX>(p, c, sH, sZ, tile, next, w, st, dw);
  } else {
    if constexpr (DX) input_grad<D>(p, c, st.dz, tile, w);
    lds_barrier();
  }
}

template <int D, int L, int ACT, bool DX>
__global__ __launch_bounds__(BGeo<D>::THREADS, 1) void mlp_bwd_kernel(MlpBwdParams p) {
  using G = BGeo<D>;
  __shared__ __attribute__((aligned(16))) _Float16 sW[L * D * D];
  __shared__ __attribute__((aligned(256))) _Float16 sHbuf[G::R * D];
  __shared__ __attribute__((aligned(256))) _Float16 sZbuf[G::R * D];
  stage_weights_bwd<D, L>(p, sW);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BLane<D> c = blane_setup<D>(p, sW, w, lane);
  const uint32_t sH = lds_addr(sHbuf), sZ = lds_addr(sZbuf);
  const uint32_t doff = (uint32_t)(lane & 15) * (uint32_t)p.ldd * 2u + 16u * (uint32_t)(lane >> 4);

  f32x4 dw[L][G::QB][G::QB];
#pragma unroll
  for (int l = 0; l < L; ++l)
#pragma unroll
    for (int i = 0; i < G::QB; ++i)
#pragma unroll
      for (int k = 0; k < G::QB; ++k) dw[l][i][k] = (f32x4){0.f, 0.f, 0.f, 0.f};

  BState<D> st;
  int tile = blockIdx.x;
  if (tile < p.num_tiles) {
    load_b<D>(p.dout, p.ldd, doff, p.M, tile, w, st.dn);
    prefetch_h<D>(p, c, L - 1, tile, w, st);
  }
  __syncthreads();  // weights staged
  while (tile < p.num_tiles) {
    const int next = tile + (int)gridDim.x;
    // the tile's first layer: sZ <- dout, sH <- h_{L-1}
    st.dz = st.dn;
    stage_b<D>(sZ, c, st.dz);
    if constexpr (L >= 2) {
      FragB<D> hp;
      pack_rows<D>(st.ha, hp);
      stage_d<D>(sH, c, hp);
      st.h = st.ha;
    } else {
      stage_b<D>(sH, c, st.hx);
    }
    if (next < p.num_tiles) load_b<D>(p.dout, p.ldd, doff, p.M, next, w, st.dn);
    if constexpr (L >= 2)
      prefetch_h<D>(p, c, L - 2, tile, w, st);
    else if (next < p.num_tiles)
      prefetch_h<D>(p, c, 0, next, w, st);
    tile_layers<D, L, L - 1, ACT, DX>(p, c, sH, sZ, tile, next, w, st, dw);
    tile = next;
  }

  // this workgroup's partial sums: block (kb, nb) of layer l, lane, register
  float* part = p.partial + (size_t)blockIdx.x * L * D * D;
  const int kb0 = G::QB * (w >> 1), nb0 = G::QB * (w & 1);
#pragma unroll
  for (int l = 0; l < L; ++l)
#pragma unroll
    for (int i = 0; i < G::QB; ++i)
#pragma unroll
      for (int k = 0; k < G::QB; ++k) {
        const int blk = (kb0 + i) * (D / 16) + nb0 + k;
        *(f32x4*)(part + (size_t)l * D * D + (size_t)blk * 256 + 4 * lane) = dw[l][i][k];
      }
}

// dW_l = sum over the grid's partials, in workgroup order.  One thread per
// (layer, 16 x 16 block, lane): register i of lane (g, q) of block (kb, nb)
// is dW[16 kb + 4 g + i][16 nb + q].
template <int D>
__global__ __launch_bounds__(256) void mlp_bwd_reduce(const float* __restrict__ partial, int nparts, int L,
                                                      MlpBwdParams p) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int per_layer = D * D / 4;
  if (idx >= L * per_layer) return;
  const int l = idx / per_layer;
  const int rem = idx - l * per_layer;
  const int blk = rem >> 6, lane = rem & 63;
  const size_t stride = (size_t)L * D * D;
  const float* src = partial + (size_t)l * D * D + 4 * (size_t)rem;
  f32x4 acc = *(const f32x4*)src;
  for (int b = 1; b < nparts; ++b) acc += *(const f32x4*)(src + (size_t)b * stride);
  const int kb = blk / (D / 16), nb = blk - kb * (D / 16);
  const int k = 16 * kb + 4 * (lane >> 4), n = 16 * nb + (lane & 15);
  float* dst = p.dW[l];
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[(k + i) * D + n] = acc[i];
}

template <int D, int L, int ACT, bool DX>
hipError_t launch_bwd_dl(MlpBwdParams p, int num_cus, hipStream_t stream) {
  using G = BGeo<D>;
  p.num_tiles = (int)(((int64_t)p.M + G::R - 1) / G::R);
  int nwg = p.num_tiles < num_cus ? p.num_tiles : num_cus;
  if (nwg < 1) nwg = 1;
  hipLaunchKernelGGL((mlp_bwd_kernel<D, L, ACT, DX>), dim3(nwg), dim3(G::THREADS), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int threads = L * D * D / 4;
  hipLaunchKernelGGL((mlp_bwd_reduce<D>), dim3((threads + 255) / 256), dim3(256), 0, stream, p.partial, nwg, L, p);
  return hipGetLastError();
}

template <int D, int ACT, bool DX>
hipError_t launch_bwd_d(const MlpBwdParams& p, int L, int cus, hipStream_t stream) {
  if constexpr (D == 128) {
    switch (L) {
      case 1: return launch_bwd_dl<D, 1, ACT, DX>(p, cus, stream);
      case 2: return launch_bwd_dl<D, 2, ACT, DX>(p, cus, stream);
      case 3: return launch_bwd_dl<D, 3, ACT, DX>(p, cus, stream);
      case 4: return launch_bwd_dl<D, 4, ACT, DX>(p, cus, stream);
    }
  } else {
    switch (L) {
      case 1: return launch_bwd_dl<D, 1, ACT, DX>(p, cus, stream);
      case 2: return launch_bwd_dl<D, 2, ACT, DX>(p, cus, stream);
      case 3: return launch_bwd_dl<D, 3, ACT, DX>(p, cus, stream);
      case 4: return launch_bwd_dl<D, 4, ACT, DX>(p, cus, stream);
      case 5: return launch_bwd_dl<D, 5, ACT, DX>(p, cus, stream);
      case 6: return launch_bwd_dl<D, 6, ACT, DX>(p, cus, stream);
      case 7: return launch_bwd_dl<D, 7, ACT, DX>(p, cus, stream);
      case 8: return launch_bwd_dl<D, 8, ACT, DX>(p, cus, stream);
    }
  }
  return hipErrorInvalidValue;
}

template <int D, bool DX>
hipError_t launch_bwd_da(const MlpBwdParams& p, int L, int act, int cus, hipStream_t stream) {
  if (act == ACT_NONE) return launch_bwd_d<D, ACT_NONE, DX>(p, L, cus, stream);
  if (act == ACT_RELU) return launch_bwd_d<D, ACT_RELU, DX>(p, L, cus, stream);
  return launch_bwd_d<D, ACT_SOFTPLUS, DX>(p, L, cus, stream);
}

}  // namespace

size_t mlp_backward_workspace(int D, int L, int num_cus) {
  return (size_t)num_cus * (size_t)L * (size_t)D * (size_t)D * sizeof(float);
}

hipError_t launch_mlp_backward(MlpBwdParams p, int D, int L, int act, int num_cus, hipStream_t stream) {
  const bool dx = p.dx != nullptr;
  if (D == 128)
    return dx ? launch_bwd_da<128, true>(p, L, act, num_cus, stream) : launch_bwd_da<128, false>(p, L, act, num_cus, stream);
  return dx ? launch_bwd_da<64, true>(p, L, act, num_cus, stream) : launch_bwd_da<64, false>(p, L, act, num_cus, stream);
}

}  // namespace coalesce
