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
//   softplus: sigmoid(z) = 1 - exp(-h);  relu: h > 0;  none: 1.
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
//     are staged in LDS as fp16 (row-major, 16-byte pieces XOR-swizzled by
//     row) and read back with the transposing ds_read_b64_tr_b16, which
//     hands every lane 4 rows of one column;
//   * h_l comes from the fp32 activations loaded once per layer: the same
//     registers give the fp16 staging copy and the derivative;
//   * every input of a tile (dout, each activation layer, x) has its own
//     register buffer that is reloaded with the next tile's rows as soon as
//     the current rows are staged, so the loads run a whole tile ahead (the
//     deepest chains keep one activation buffer, loaded a layer ahead); the
//     barriers around the staging buffers do not wait for them;
//   * at the end every workgroup writes its partial dW to a workspace and a
//     second kernel sums the partials in a fixed order: the result is
//     deterministic for a given grid (the pages' design accumulates with
//     atomics below 32K rows and calls GEMMs above).
#include <mutex>

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
// bytes, 16-byte piece c (units 8 c .. 8 c + 7) of row r at piece position
// c ^ sfz(r), where sfz depends on r mod 16 only.  The LDS serves 128 bytes
// per pass (measured on this GPU with a probe of these access patterns and
// SQ_LDS_BANK_CONFLICT): 8 lanes of a 16-byte access, 16 lanes of an 8-byte
// access or of a transposing read.  Then:
//   * 16-byte writes: 8 lanes cover 8 consecutive rows (from a multiple of
//     8) at one piece index; sfz mod 8 (D = 128: the 128-byte position of a
//     piece in a 256-byte row) or sfz (D = 64: 128-byte rows) takes 8
//     distinct values over those rows: one pass;
//   * transposing reads: 16 lanes cover 4 consecutive rows (from a multiple
//     of 4), two neighbouring pieces each; (sfz >> 1) mod 4 takes 4 distinct
//     values over them: one pass.  The 32 rows of a weight-gradient
//     contraction step are paired as kk = 8 g + 4 h + rho <-> row 16 h + 4 g
//     + rho, so that the second read is 16 rows further (sfz unchanged: the
//     offset stays an immediate);
//   * 8-byte writes (4 units of one row per lane): 16 lanes cover 16 rows
//     at the same half of one piece index, which a piece layout can spread
//     over 8 positions of a pass only: two passes.
// (The earlier sfz, ((r & 7) << 1) | ((r >> 3) & 1) and (((r >> 1) & 3) << 1)
// | ((r >> 3) & 1), was laid out for 256-byte passes and took two passes for
// every 16-byte write.)
template <int D>
__device__ __forceinline__ int sfz(int r) {
  if constexpr (D == 128)
    return ((r & 7) << 1) ^ ((r >> 2) & 1) ^ ((r >> 3) & 1);
  else
    return ((r & 3) << 1) | ((r >> 2) & 1);
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
  // units 16 t + 4 g .. + 3 sit in piece 2 t + g / 2 (XOR t << 5 selects t)
  c.st8 = (uint32_t)(r * 2 * D + (((g >> 1) ^ sfz<D>(r)) << 4) + ((g & 1) << 3));
  // units 32 ks + 8 g .. + 7 are piece 4 ks + g (XOR ks << 6 selects ks)
  c.st16 = (uint32_t)(r * 2 * D + ((g ^ sfz<D>(r)) << 4));
  // transposing read: row 4 g + q / 4 of a 32-row chunk, units 16 b + 4 (q % 4)
  // .. + 3, i.e. piece 2 b + (q % 4) / 2 (XOR b << 5 selects the block b)
  const int rt = 4 * g + (q >> 2);
  c.trk = (uint32_t)(rt * 2 * D + ((((q & 3) >> 1) ^ sfz<D>(rt)) << 4) + ((q & 1) << 3));
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

// A lane's access to columns at or beyond the operand's true width goes to a
// buffer offset past every resource's size (16 rows of any operand span
// less than 2^31 bytes), so the load reads zero and the store is dropped.
constexpr uint32_t OFF_NONE = 0x80000000u;
__device__ __forceinline__ uint32_t masked(bool ok, uint32_t off) { return ok ? off : OFF_NONE; }
__device__ __forceinline__ int lane_group() { return (int)(threadIdx.x & 63) >> 4; }

// Weights in LDS: W_l as D rows k of D fp16, 16-byte chunks swizzled by
// wswz.  Layer L-1 is fed by dout (natural unit order); the others by the
// registers of the layer above, whose unit order is that of layer_k_slot.
// The true layer is dims[l] x dims[l+1] (pitch dims[l+1]); units outside it
// are staged as zero (a narrower chain run at width D): their loads go to
// OFF_NONE.  Each thread issues all its loads of a layer before its first
// LDS write, and the layer index is a constant, so a layer costs one memory
// round trip instead of one per 16-byte chunk.
template <int D, int L>
__device__ __forceinline__ void stage_weights_bwd(const MlpBwdParams& p, _Float16* sW) {
  constexpr int CPR = D / 8;                             // 16-byte chunks per row
  constexpr int PER = D * CPR / BGeo<D>::THREADS;        // chunks of one layer per thread
  static_assert(D * CPR % BGeo<D>::THREADS == 0, "whole chunks per thread");
#pragma unroll
  for (int l = 0; l < L; ++l) {
    const int K = p.dims[l], N = p.dims[l + 1];
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.W[l], (short)0, K * N * 2, 0x00020000);
    u32x4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = (int)threadIdx.x + i * BGeo<D>::THREADS;
      const int k = idx / CPR, cb = idx % CPR;
      const uint32_t row = (uint32_t)(k * N) * 2u;
      if (l == L - 1) {
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, masked(k < K && 8 * cb < N, row + 16u * cb), 0, 0);
      } else {
        // slots 8 cb .. 8 cb + 7 (cb = 4 a + b) hold units 32 a + 4 b + 0..3
        // and 32 a + 16 + 4 b + 0..3 (each group of 4 is inside or outside N
        // as a whole, N being a multiple of 8)
        const int u = 32 * (cb >> 2) + 4 * (cb & 3);
        const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(rs, masked(k < K && u < N, row + 2u * u), 0, 0);
        const u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(rs, masked(k < K && u + 16 < N, row + 2u * (u + 16)), 0, 0);
        v[i] = (u32x4){lo[0], lo[1], hi[0], hi[1]};
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = (int)threadIdx.x + i * BGeo<D>::THREADS;
      const int k = idx / CPR, cb = idx % CPR;
      *(u32x4*)(sW + (l * D + k) * D + ((cb ^ wswz<D>(k)) << 3)) = v[i];
    }
  }
}

// B-form fp16 rows (x, dout) of `width` true columns: units 32 ks + 8 g .. + 7.
template <int D>
__device__ __forceinline__ void load_b(const void* base, int64_t ld, uint32_t off, int M, int tile, int w, int width,
                                       FragB<D>& f) {
#pragma unroll
  for (int s = 0; s < BGeo<D>::MT; ++s) {
    const __amdgpu_buffer_rsrc_t rs = brsrc<D>(base, M, tile, w, s, ld, 2);
#pragma unroll
    for (int ks = 0; ks < BGeo<D>::KS; ++ks)
      f.v[s][ks] = __builtin_amdgcn_raw_buffer_load_b128(rs, masked(32 * ks + 8 * lane_group() < width, off + 64u * ks),
                                                         0, 0);
  }
}

// fp32 activation rows of `width` true columns: units 16 t + 4 g .. + 3.
template <int D>
__device__ __forceinline__ void load_acts(const float* base, int64_t ld, uint32_t off, int M, int tile, int w,
                                          int width, RowsF32<D>& f) {
#pragma unroll
  for (int s = 0; s < BGeo<D>::MT; ++s) {
    const __amdgpu_buffer_rsrc_t rs = brsrc<D>(base, M, tile, w, s, ld, 4);
#pragma unroll
    for (int t = 0; t < BGeo<D>::NT; ++t)
      f.v[s][t] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, masked(16 * t + 4 * lane_group() < width, off + 64u * t), 0, 0));
  }
}

// Stage a B-layout fp16 tile (dout or x) into a staging buffer.
template <int D>
__device__ __forceinline__ void stage_b(uint32_t buf, const BLane<D>& c, const FragB<D>& f) {
#pragma unroll
  for (int s = 0; s < BGeo<D>::MT; ++s)
#pragma unroll
    for (int ks = 0; ks < BGeo<D>::KS; ++ks)
      lds_write128((buf + c.st16 + 16u * 2 * D * s) ^ (uint32_t)(ks << 6), f.v[s][ks]);
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

// Issue order of one pipeline step (as in the forward megakernel): NM MFMAs,
// each followed by VPM VALU instructions and, after every DS_EVERY-th one, a
// DS read.
template <int NM, int VPM, int DS_EVERY>
__device__ __forceinline__ void interleave_bwd() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i % DS_EVERY == DS_EVERY - 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, VPM, 0);
  }
}

// VALU issue slots per element of the derivative step (the transcendental
// counted twice).
template <int ACT>
constexpr int act_grad_ops() {
  return ACT == ACT_SOFTPLUS ? 5 : ACT == ACT_RELU ? 2 : 0;
}

// One layer's matrix work for the wave, software-pipelined over the NT
// 16-unit output sub-tiles of the data-gradient product.  Step t (0..NT)
// issues the MFMAs of sub-tile t (its W fragments were read one step ahead),
// the derivative and packing of sub-tile t - 1 (on results that are already
// complete), and a share of the weight-gradient MFMAs (their transposing
// reads one step ahead), so the matrix core, the VALU and the LDS all work
// within the one wave a SIMD holds.
//   weight gradient: dW_l(wave block) += sH^T sZ over the tile's R rows.  The
//     wave's block is QB x QB 16 x 16 tiles: k tiles QB (w / 2) + i, n tiles
//     QB (w % 2) + k; MFMA m = (j QB + i) QB + k covers rows 32 j .. + 31.
//   MODE 1: dz_l = (dz_{l+1} W_l^T) * act'(h_l) for the wave's rows, packed
//     to fp16 in B-operand form into out;
//   MODE 2: dx = dz_1 W_0^T, stored as fp16 in pairs of sub-tiles;
//   MODE 0: weight gradient only.
template <int D, int l, int ACT, int MODE>
__device__ __forceinline__ void layer_grads(const MlpBwdParams& p, const BLane<D>& c, uint32_t sH, uint32_t sZ,
                                            int w, int tile, f32x4 (&dw)[BGeo<D>::QB][BGeo<D>::QB],
                                            const FragB<D>& dz, const RowsF32<D>& h, FragB<D>& out) {
  using G = BGeo<D>;
  constexpr int NT = G::NT, MT = G::MT, KS = G::KS, QB = G::QB, CH = G::CH;
  constexpr int NWG = CH * QB * QB;       // weight-gradient MFMAs
  constexpr int PER = (NWG + NT - 1) / NT;  // of them per step
  constexpr int NDG = MODE ? KS * MT : 0;   // data-gradient MFMAs per step
  constexpr int VPE = MODE == 1 ? act_grad_ops<ACT>() : 0;
  constexpr int VPS = MT * (4 * VPE + 2) + (MODE == 2 ? 2 : 0);  // VALU per step
  constexpr int NM = NDG + PER;
  constexpr int VPM = (VPS + NM - 1) / NM;

  // transposing-read addresses of the wave's k tiles (sH) and n tiles (sZ)
  const uint32_t kb0 = (uint32_t)(QB * (w >> 1)), nb0 = (uint32_t)(QB * (w & 1));
  uint32_t ha[QB], zb[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    ha[b] = (sH + c.trk) ^ ((kb0 + b) << 5);
    zb[b] = (sZ + c.trk) ^ ((nb0 + b) << 5);
  }
  i16x8 fa[CH][QB], fb[CH][QB];
  auto tr8 = [](uint32_t addr, int j) {
    const i16x4 x0 = lds_tr(addr + (uint32_t)(32 * j * 2 * D));
    const i16x4 x1 = lds_tr(addr + (uint32_t)((32 * j + 16) * 2 * D));
    return (i16x8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };
  // fragments first used by the MFMAs of step u
  auto load_frags = [&](int u) {
#pragma unroll
    for (int m = u * PER; m < (u + 1) * PER && m < NWG; ++m) {
      const int j = m / (QB * QB), i = (m / QB) % QB, k = m % QB;
      if (k == 0) fa[j][i] = tr8(ha[i], j);
      if (i == 0) fb[j][k] = tr8(zb[k], j);
    }
  };

  uint32_t wk[KS];
  i16x8 wa[KS];
  f32x4 acc[MT], prv[MT];
  __amdgpu_buffer_rsrc_t rq[MT];
  uint32_t qoff = 0;
  u32x2 ev[MT];
  if constexpr (MODE != 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      wk[ks] = opaque(c.wk[ks]) + 2u * (uint32_t)(l * D * D);
      wa[ks] = lds_read128(wk[ks]);
    }
  }
  if constexpr (MODE == 2) {
#pragma unroll
    for (int s = 0; s < MT; ++s) rq[s] = brsrc<D>(p.dx, p.M, tile, w, s, p.ldq, 2);
    qoff = opaque(c.qoff);
  }
  load_frags(0);
#pragma unroll
  for (int t = 0; t <= NT; ++t) {
    if constexpr (MODE != 0) {
      if (t < NT) {
#pragma unroll
        for (int s = 0; s < MT; ++s) acc[s] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int s = 0; s < MT; ++s) acc[s] = mfma16x16x32(wa[ks], __builtin_bit_cast(i16x8, dz.v[s][ks]), acc[s], _Float16());
          if (t + 1 < NT) wa[ks] = lds_read128(wk[ks] + 2u * (uint32_t)(16 * D * (t + 1)));
        }
      }
    }
    if (t < NT) {
#pragma unroll
      for (int m = t * PER; m < (t + 1) * PER && m < NWG; ++m) {
        const int j = m / (QB * QB), i = (m / QB) % QB, k = m % QB;
        dw[i][k] = mfma16x16x32(fa[j][i], fb[j][k], dw[i][k], _Float16());
      }
      if (t + 1 < NT) load_frags(t + 1);
    }
    if constexpr (MODE != 0) {
      if (t > 0) {
        const int u = t - 1;
#pragma unroll
        for (int s = 0; s < MT; ++s) {
          if constexpr (MODE == 1) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = apply_grad<ACT>(prv[s][i], h.v[s][u][i]);
            out.v[s][u >> 1][(u & 1) * 2] = pack_f16(v[0], v[1]);
            out.v[s][u >> 1][(u & 1) * 2 + 1] = pack_f16(v[2], v[3]);
          } else {
            const u32x2 o = (u32x2){pack_f16(prv[s][0], prv[s][1]), pack_f16(prv[s][2], prv[s][3])};
            if (u % 2 == 0)
              ev[s] = o;
            else
              store_pair(rq[s],
                         masked(16 * (u - 1) + 16 * (lane_group() & 1) + 8 * (lane_group() >> 1) < p.dims[0],
                                qoff + 32u * (uint32_t)(u - 1)),
                         ev[s], o);
          }
        }
      }
    }
    if (t < NT) interleave_bwd<NM, VPM, 1>();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MODE != 0) {
#pragma unroll
      for (int s = 0; s < MT; ++s) prv[s] = acc[s];
    }
  }
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Barrier that waits only for the wave's own LDS accesses, not for its
// outstanding global loads (the prefetches stay in flight across it).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
#pragma clang diagnostic pop

// Register and LDS policy of a chain.
//   FULL: every input of a tile has its own register buffer, reloaded with
//     the next tile's rows right after its last use (an activation buffer
//     after the derivative step of its layer, x and dout after staging), so
//     the loads run most of a tile ahead of their use and no buffer is copied
//     while its load is in flight.  Chains whose buffers would not fit next
//     to their weight-gradient accumulators (4 layers of 128, 7 or 8 of 64)
//     share one activation buffer, loaded one layer ahead.
//   DB: two sets of staging buffers, used by alternate layers, so that one
//     barrier per layer suffices (the set written for layer l - 1 was last
//     read in layer l + 1, before the barrier of layer l).  4 layers of 128
//     leave no LDS for it and keep one set with two barriers per layer.
template <int D, int L>
struct BPolicy {
  static constexpr bool FULL = D == 128 ? L <= 3 : L <= 6;
  static constexpr int NA = L == 1 ? 1 : (FULL ? L - 1 : 1);  // activation buffers
  static constexpr bool DB = L * D * D * 2 + 4 * BGeo<D>::R * D * 2 <= 160 * 1024;
  static constexpr int SETS = DB ? 2 : 1;
  static constexpr uint32_t SZ = BGeo<D>::R * D * 2;  // bytes of one staging buffer
};

template <int D, int L>
struct BState {
  RowsF32<D> h;                      // !FULL: h_l of the wave's rows (fp32), the derivative source
  RowsF32<D> a[BPolicy<D, L>::NA];   // FULL: a[j - 1] holds h_j; otherwise the next activation layer
  FragB<D> hx;                       // x of the rows to stage next (B form)
  FragB<D> dn;                       // dout of the next tile
};

// Issue the load of h_j of `tile` into its buffer (j >= 1: fp32 acts[j - 1];
// j == 0: x).  Loads for a tile past the last one are issued anyway: their
// buffer resources cover zero rows, so they read zeros without touching
// memory, and the issue stream stays free of branches (a conditional load
// makes the compiler wait for every outstanding load where the paths join).
template <int D, int L>
__device__ __forceinline__ void load_h(const MlpBwdParams& p, const BLane<D>& c, int j, int tile, int w,
                                       BState<D, L>& st) {
  if (j >= 1)
    load_acts<D>(p.acts[j - 1], p.lda, opaque(c.aoff), p.M, tile, w, p.dims[j], st.a[BPolicy<D, L>::FULL ? j - 1 : 0]);
  else
    load_b<D>(p.x, p.ldx, opaque(c.boff), p.M, tile, w, p.dims[0], st.hx);
}

// Stage h_j of the current tile into the staging set `set` (sH = set, sZ =
// set + SZ) and issue the loads that policy attaches to this point.
template <int D, int L, int j>
__device__ __forceinline__ void stage_h(const MlpBwdParams& p, const BLane<D>& c, uint32_t set, int tile, int next,
                                        int w, BState<D, L>& st) {
  constexpr bool FULL = BPolicy<D, L>::FULL;
  if constexpr (j >= 1) {
    FragB<D> hp;
    pack_rows<D>(st.a[FULL ? j - 1 : 0], hp);
    stage_d<D>(set, c, hp);
    if constexpr (!FULL) {
      st.h = st.a[0];
      load_h<D, L>(p, c, j - 1, tile, w, st);  // the layer below, one layer ahead
    }
  } else {
    stage_b<D>(set, c, st.hx);
    if constexpr (FULL)
      load_h<D, L>(p, c, 0, next, w, st);
    else
      load_h<D, L>(p, c, L - 1, next, w, st);  // the next tile's first activation layer
  }
}

// Layers l .. 0 of one tile.  On entry the staging set `cur` holds h_l and
// dz_{l+1} (this wave's rows written, the barrier not yet passed), dz holds
// dz_{l+1}; nz receives dz_l.  With DB, layer l - 1 stages into `nxt`.
template <int D, int L, int l, int ACT, bool DX>
__device__ __forceinline__ void tile_layers(const MlpBwdParams& p, const BLane<D>& c, uint32_t cur, uint32_t nxt,
                                            int tile, int next, int w, BState<D, L>& st, FragB<D>& dz,
                                            FragB<D>& nz, f32x4 (&dw)[L][BGeo<D>::QB][BGeo<D>::QB]) {
  using P = BPolicy<D, L>;
  lds_barrier();
  if constexpr (l >= 1) {
    if constexpr (P::FULL) {
      layer_grads<D, l, ACT, 1>(p, c, cur, cur + P::SZ, w, tile, dw[l], dz, st.a[l - 1], nz);
      load_h<D, L>(p, c, l, next, w, st);  // h_l of the next tile, after its last use here
    } else {
      layer_grads<D, l, ACT, 1>(p, c, cur, cur + P::SZ, w, tile, dw[l], dz, st.h, nz);
    }
    if constexpr (!P::DB) lds_barrier();
    const uint32_t dst = P::DB ? nxt : cur;
    stage_d<D>(dst + P::SZ, c, nz);
    stage_h<D, L, l - 1>(p, c, dst, tile, next, w, st);
    tile_layers<D, L, l - 1, ACT, DX>(p, c, dst, P::DB ? cur : nxt, tile, next, w, st, nz, dz, dw);
  } else {
    layer_grads<D, 0, ACT, DX ? 2 : 0>(p, c, cur, cur + P::SZ, w, tile, dw[0], dz, st.h, nz);
    if constexpr (!P::DB) lds_barrier();
  }
}

template <int D, int L, int ACT, bool DX>
__global__ __launch_bounds__(BGeo<D>::THREADS, 1) void mlp_bwd_kernel(MlpBwdParams p) {
  using G = BGeo<D>;
  using P = BPolicy<D, L>;
  __shared__ __attribute__((aligned(16))) _Float16 sW[L * D * D];
  __shared__ __attribute__((aligned(256))) _Float16 sStage[P::SETS * 2 * G::R * D];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BLane<D> c = blane_setup<D>(p, sW, w, lane);
  uint32_t cur = lds_addr(sStage), nxt = cur + (P::DB ? 2 * P::SZ : 0);
  const uint32_t doff = (uint32_t)(lane & 15) * (uint32_t)p.ldd * 2u + 16u * (uint32_t)(lane >> 4);

  f32x4 dw[L][G::QB][G::QB];
#pragma unroll
  for (int l = 0; l < L; ++l)
#pragma unroll
    for (int i = 0; i < G::QB; ++i)
#pragma unroll
      for (int k = 0; k < G::QB; ++k) dw[l][i][k] = (f32x4){0.f, 0.f, 0.f, 0.f};

  BState<D, L> st;
  FragB<D> dz, nz;
  int tile = blockIdx.x;
  if (tile < p.num_tiles) {
    load_b<D>(p.dout, p.ldd, doff, p.M, tile, w, p.dims[L], st.dn);
    if constexpr (P::FULL) {
#pragma unroll
      for (int j = L - 1; j >= 0; --j) load_h<D, L>(p, c, j, tile, w, st);
    } else {
      load_h<D, L>(p, c, L - 1, tile, w, st);
    }
  }
  // the weights' loads go out behind the first tile's
  stage_weights_bwd<D, L>(p, sW);
  __syncthreads();  // weights staged
  while (tile < p.num_tiles) {
    const int next = tile + (int)gridDim.x;
    // the tile's first layer: sZ <- dout, sH <- h_{L-1}
    dz = st.dn;
    stage_b<D>(cur + P::SZ, c, dz);
    load_b<D>(p.dout, p.ldd, doff, p.M, next, w, p.dims[L], st.dn);  // zero rows past the last tile
    stage_h<D, L, L - 1>(p, c, cur, tile, next, w, st);
    tile_layers<D, L, L - 1, ACT, DX>(p, c, cur, nxt, tile, next, w, st, dz, nz, dw);
    // layer l used set cur when L - 1 - l is even: the next tile starts on the
    // set that layer 0 did not use
    if constexpr (P::DB && (L % 2 == 1)) {
      const uint32_t t = cur;
      cur = nxt;
      nxt = t;
    }
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

// dW_l = sum over the grid's partials.  The partials are viewed as rows of
// E = L D D / 4 float4 groups; a workgroup owns 32 groups and splits the
// partial index over 8 slices (slice s adds partials s, s + 8, ... in order),
// then adds the 8 slice sums in slice order: a fixed order, so the result is
// the same on every call with the same grid.  Register i of lane (g, q) of
// block (kb, nb) is dW[16 kb + 4 g + i][16 nb + q].
constexpr int RED_GROUPS = 32, RED_SLICES = 8;

template <int D>
__global__ __launch_bounds__(RED_GROUPS* RED_SLICES) void mlp_bwd_reduce(const float* __restrict__ partial, int nparts,
                                                                         int L, MlpBwdParams p) {
  __shared__ f32x4 red[RED_SLICES][RED_GROUPS];
  const int gi = threadIdx.x % RED_GROUPS, slice = threadIdx.x / RED_GROUPS;
  const int E = L * D * D / 4;
  const int e = blockIdx.x * RED_GROUPS + gi;
  f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (e < E) {
    const f32x4* src = (const f32x4*)partial + e;
#pragma unroll 8
    for (int b = slice; b < nparts; b += RED_SLICES) acc += src[(size_t)b * E];
  }
  red[slice][gi] = acc;
  __syncthreads();
  if (slice != 0 || e >= E) return;
  f32x4 sum = red[0][gi];
#pragma unroll
  for (int k = 1; k < RED_SLICES; ++k) sum += red[k][gi];
  const int per_layer = D * D / 4;
  const int l = e / per_layer;
  const int rem = e - l * per_layer;
  const int blk = rem >> 6, lane = rem & 63;
  const int kb = blk / (D / 16), nb = blk - kb * (D / 16);
  const int k = 16 * kb + 4 * (lane >> 4), n = 16 * nb + (lane & 15);
  const int K = p.dims[l], N = p.dims[l + 1];  // the true layer (a narrower chain writes its part only)
  float* dst = p.dW[l];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (k + i < K && n < N) dst[(k + i) * N + n] = sum[i];
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
  const int groups = L * D * D / 4;
  hipLaunchKernelGGL((mlp_bwd_reduce<D>), dim3((groups + RED_GROUPS - 1) / RED_GROUPS), dim3(RED_GROUPS * RED_SLICES),
                     0, stream, p.partial, nwg, L, p);
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

// Scratch of the no-allocation backward entry point: the per-workgroup
// partial weight gradients (mlp_backward_workspace bytes) in a file-scope
// device array instead of a caller-lent workspace.  Every device the library
// runs on holds its own copy until the process ends.  In host code the
// array's name is only a host-side stand-in: the kernels get the address
// that hipGetSymbolAddress returns on the current device (cached per device
// below), never the name.  All calls on one device share it.
constexpr size_t kBwdScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

size_t mlp_backward_scratch_bytes() { return kBwdScratchBytes; }

hipError_t mlp_backward_scratch(void** ptr) {
  constexpr int kDevices = 64;
  static std::mutex mutex;
  static void* addr[kDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mutex);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_mlp_backward(MlpBwdParams p, int D, int L, int act, int num_cus, hipStream_t stream) {
  const bool dx = p.dx != nullptr;
  if (D == 128)
    return dx ? launch_bwd_da<128, true>(p, L, act, num_cus, stream) : launch_bwd_da<128, false>(p, L, act, num_cus, stream);
  return dx ? launch_bwd_da<64, true>(p, L, act, num_cus, stream) : launch_bwd_da<64, false>(p, L, act, num_cus, stream);
}

}  // namespace coalesce
