// Layer-by-layer backward of the MLP chains whose weights do not all fit in
// LDS at once (the chains the layer-streaming forward runs: up to 16 layers,
// widths up to 256, each layer at its own width).  The quantities are those
// of the fused backward ("MLP Megakernel" README, "Key ideas": the fp32
// activations of the training forward, the softplus derivative recovered
// from them, fp16 only for the matrix-core operands, fp32 accumulation),
// computed one layer per launch, l = L-1 .. 0, with dz_L = dout:
//   dW_l = h_l^T dz_{l+1}                    (summed over all rows)
//   dz_l = (dz_{l+1} W_l^T) * act'(z_l)      (l > 0, stored as fp16)
//   dx   =  dz_1 W_0^T                       (l = 0, optional)
// Both products of a layer read the same two row tiles (dz_{l+1} and h_l),
// so one kernel computes them together and reads each tile from HBM once.
// dz_l goes to a workspace in fp16, the precision in which the next layer's
// MFMAs take it anyway: the results are those of one fused pass over all
// layers, up to the order in which per-workgroup dW sums are added.  (The
// README's own backward switches to per-layer GEMMs for large row counts;
// here each layer is one fused kernel instead of two GEMMs and an
// elementwise pass.)
//
// Design for gfx950 (one workgroup of 8 waves per CU, persistent over
// 32-row tiles; I = dims[l], J = dims[l+1]):
//   * W_l (I x J fp16, at most 128 KiB) sits in LDS for the whole launch in
//     its natural layout: a row of W_l is the A operand of the data product
//     dz_l^T = W_l dz_{l+1}^T, read as 16-byte pieces;
//   * each wave owns TI 16-unit tiles of the I units: it computes dz_l of
//     those units for the tile's rows (B = dz_{l+1} rows, from LDS) and sums
//     dW_l over the same units and all J in registers;
//   * the weight-gradient contraction runs over rows, so dz_{l+1} and h_l
//     (as fp16) are staged in LDS and read back with the transposing
//     ds_read_b64_tr_b16.  Computing dW^T = dz^T h leaves 4 consecutive j of
//     one i in each lane, so the partial sums leave in 16-byte stores;
//   * the next tile's dz_{l+1} and h_l are loaded into registers while the
//     current tile is computed; h_l's fp32 registers sit in the data
//     product's result layout (4 units of one row per lane), so the
//     derivative needs no data movement, and the same registers give the
//     fp16 copy staged for the weight gradient;
//   * each workgroup writes its partial dW_l; a second kernel adds the
//     partials in a fixed order, so repeated calls give the same bits.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "mlp_common.hpp"

namespace coalesce {
namespace {

// Geometry per width class P (the chain's widest layer, 128 or 256; chains
// up to 64 wide run at 128 with the units past their widths skipped).
template <int P>
struct LGeo {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int TI = P / 128;                    // 16-unit i tiles per wave: 8 waves cover P units
  static constexpr int R = 32;                          // rows per tile: one 32-deep weight-gradient k step
  static constexpr int ROWB = 2 * P;                    // bytes of a staged LDS row (W_l, dz, h)
  static constexpr int PIECES = P / 8;                  // 16-byte pieces per staged row
  static constexpr int KS = P / 32;                     // 32-deep data-product k steps at most
  static constexpr int NJ = P / 16;                     // 16-unit j tiles at most
  static constexpr int ZP = R * PIECES / THREADS;       // dz pieces a thread loads per tile
};

struct LayerArgs {
  const void* dz;    // M x J fp16 (ldz): dLoss/dz_{l+1}
  const void* h;     // M x I: h_l in fp32 (l > 0) or x in fp16 (l = 0), pitch ldh
  const void* W;     // I x J fp16, dense
  void* out;         // M x I fp16 (ldo): dz_l (l > 0), dx (l = 0), or nullptr
  float* partial;    // grid x I x J fp32
  int64_t ldz, ldh, ldo;
  int I, J, M, num_tiles;
};

// LDS bank model (measured on this GPU with a probe of each access pattern
// below and SQ_LDS_BANK_CONFLICT): a pass serves 128 bytes, i.e. 8 lanes of
// a 16-byte access, 16 lanes of an 8-byte access or of a transposing read.
//
// Staged dz rows: 16-byte piece c of row r sits at c ^ zsw(r).  zsw depends
// on r mod 16 only; zsw mod 8 takes 8 distinct values over each 8
// consecutive rows starting at a multiple of 8 (the 16-byte reads of the
// data product: 8 lanes = 8 rows, one piece each), and (zsw >> 1) mod 4
// takes 4 distinct values over each 4 consecutive rows starting at a
// multiple of 4 (a transposing read: 16 lanes = 4 rows, 32 bytes each).
// The row-major 16-byte staging writes cover 8 pieces of one row per pass.
// (The earlier ((r & 7) << 1) | ((r >> 3) & 1) repeats mod 8 within 8 rows:
// every data-product read took two passes.)  Weight rows use c ^ (i mod
// 16): 8 consecutive rows, one piece.
__device__ __forceinline__ int zsw(int r) { return ((r & 7) << 1) ^ ((r >> 2) & 1) ^ ((r >> 3) & 1); }

// Staged h rows (written 8 bytes per lane, read only by transposing reads):
// 8-byte chunk k of row r sits at k ^ hsw(r).  hsw mod 16 takes 16 distinct
// values over 16 consecutive rows (a write pass: 16 rows, the same chunk),
// and (hsw >> 2) mod 4 4 distinct values over each aligned 4 rows (a
// transposing read: 4 rows, 4 chunks each).  With the piece layout of zsw
// the 16 rows of a write pass fall on 8 chunk positions (two passes).
__device__ __forceinline__ int hsw(int r) { return ((r & 3) << 2) ^ (((r >> 2) & 1) * 17) ^ (((r >> 3) & 1) << 1); }

constexpr uint32_t L_OFF_NONE = 0x80000000u;  // past every resource (all span less than 2^31 bytes)
__device__ __forceinline__ uint32_t lmask(bool ok, uint32_t off) { return ok ? off : L_OFF_NONE; }

// Stage W (rows x cols fp16, dense, rows <= MAXR, cols <= 8 PIECES) as LDS
// rows of 16 PIECES bytes, 16-byte piece c of row i at c ^ (i mod 16), zero
// past the matrix up to the next 16 rows and 8 PIECES columns.  A thread
// issues up to 16 loads before its first LDS write (pieces outside the
// matrix read zero through the buffer's range check), so the copy costs one
// or two memory round trips, not one per piece.
template <int THREADS, int PIECES, int MAXR>
__device__ __forceinline__ void stage_w_rows(uint32_t sWr, const void* W, int rows, int cols) {
  constexpr int TOTAL = MAXR * PIECES / THREADS;  // pieces per thread at most
  constexpr int B = TOTAL < 16 ? TOTAL : 16;
  static_assert(MAXR * PIECES % THREADS == 0, "whole pieces per thread");
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)W, (short)0, rows * cols * 2, 0x00020000);
  const int n = ((rows + 15) & ~15) * PIECES;
  for (int base = threadIdx.x; base < n; base += B * THREADS) {
    u32x4 v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int idx = base + u * THREADS, i = idx / PIECES, c = idx % PIECES;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, lmask(i < rows && 8 * c < cols, (uint32_t)(i * cols + 8 * c) * 2u),
                                                   0, 0);
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int idx = base + u * THREADS, i = idx / PIECES, c = idx % PIECES;
      if (idx < n) lds_write128(sWr + (uint32_t)(i * 16 * PIECES + ((c ^ (i & 15)) << 4)), v[u]);
    }
  }
}

// Buffer resource over rows [first, first + n) of a matrix (pitch ld
// elements of es bytes, M rows): rows past M read as zero, stores to them
// are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int M, int64_t first, int n, int64_t ld,
                                                            int es) {
  const int64_t rows = min((int64_t)n, max((int64_t)0, (int64_t)M - first));
  const char* p = (const char*)base + first * ld * es;
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)((uint32_t)rows * (uint32_t)(ld * es)),
                                           0x00020000);
}

template <int P, int MODE>
struct TileRegs {
  // dz_{l+1}: pieces threadIdx.x + THREADS e of the tile (row-major, PIECES per row)
  u32x4 z[LGeo<P>::ZP];
  // h_l of the wave's units: rows 16 nt + q, units 16 it + 4 g .. + 3; fp32
  // for hidden layers, fp16 (x) for the first layer
  typename std::conditional<MODE == 1, f32x4, u32x2>::type h[LGeo<P>::TI][2];
};

template <int P, int MODE>
__device__ __forceinline__ void load_tile(const LayerArgs& a, int tile, int w, int q, int g, TileRegs<P, MODE>& r) {
  using G = LGeo<P>;
  const int64_t row0 = (int64_t)tile * G::R;
  const __amdgpu_buffer_rsrc_t rz = rows_rsrc(a.dz, a.M, row0, G::R, a.ldz, 2);
#pragma unroll
  for (int e = 0; e < G::ZP; ++e) {
    const int idx = threadIdx.x + G::THREADS * e;
    const int row = idx / G::PIECES, c = idx % G::PIECES;
    r.z[e] = __builtin_amdgcn_raw_buffer_load_b128(
        rz, lmask(8 * c < a.J, (uint32_t)row * (uint32_t)(a.ldz * 2) + 16u * (uint32_t)c), 0, 0);
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const __amdgpu_buffer_rsrc_t rh = rows_rsrc(a.h, a.M, row0 + 16 * nt, 16, a.ldh, MODE == 1 ? 4 : 2);
#pragma unroll
    for (int t = 0; t < G::TI; ++t) {
      const int u = 16 * (G::TI * w + t) + 4 * g;  // the lane's first unit
      if constexpr (MODE == 1)
        r.h[t][nt] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rh, lmask(u < a.I, (uint32_t)q * (uint32_t)(a.ldh * 4) + 4u * (uint32_t)u), 0, 0));
      else
        r.h[t][nt] = __builtin_amdgcn_raw_buffer_load_b64(
            rh, lmask(u < a.I, (uint32_t)q * (uint32_t)(a.ldh * 2) + 2u * (uint32_t)u), 0, 0);
    }
  }
}

// MODE 1: hidden layer l > 0 (dz_l with the derivative, h_l in fp32);
// MODE 2: first layer with dx (no derivative, h_0 = x in fp16);
// MODE 0: first layer, weight gradient only.
template <int P, int ACT, int MODE>
__global__ __launch_bounds__(LGeo<P>::THREADS, 1) void mlp_layer_bwd_kernel(LayerArgs a) {
  using G = LGeo<P>;
  constexpr int TI = G::TI, R = G::R, ROWB = G::ROWB, PIECES = G::PIECES, KS = G::KS, NJ = G::NJ;
  constexpr bool DATA = MODE != 0;
  constexpr int WROWS = DATA ? P : 0;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[(WROWS + 2 * R) * ROWB];
  const uint32_t sW = lds_addr(lds), sZ = sW + WROWS * ROWB, sH = sZ + R * ROWB;
  const int I = a.I, J = a.J;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, q = lane & 15, g = lane >> 4;

  const int ksn = (J + 31) >> 5;  // data-product k steps
  const int njn = (J + 15) >> 4;  // j tiles
  bool on[TI];                    // the wave's i tiles that hold units below I
#pragma unroll
  for (int t = 0; t < TI; ++t) on[t] = 16 * (TI * w + t) < I;

  // per-lane LDS offsets
  const uint32_t zrow = (uint32_t)(q * ROWB);
  const uint32_t bz = zrow + (uint32_t)((g ^ zsw(q)) << 4);           // data-product B piece, k step 0
  const int rt = 4 * g + (q >> 2);                                    // transposing read: row of a 32-row chunk
  const uint32_t trk = (uint32_t)(rt * ROWB + ((((q & 3) >> 1) ^ zsw(rt)) << 4) + ((q & 1) << 3));
  const uint32_t trkh = (uint32_t)(rt * ROWB + (((q & 3) ^ hsw(rt)) << 3));  // the same read in the h layout
  const uint32_t hst = zrow + (uint32_t)((g ^ hsw(q)) << 3);                 // h staging, i tile 0

  f32x4 dw[TI][NJ];
#pragma unroll
  for (int t = 0; t < TI; ++t)
#pragma unroll
    for (int j = 0; j < NJ; ++j) dw[t][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  TileRegs<P, MODE> nx;
  int tile = blockIdx.x;
  if (tile < a.num_tiles) load_tile<P, MODE>(a, tile, w, q, g, nx);
  // W_l rows (zero past I up to the next 16, and past J up to P), loaded
  // behind the first tile
  if constexpr (DATA) stage_w_rows<G::THREADS, PIECES, P>(sW, a.W, I, J);
  // nothing of the prologue stays in flight into the loop
  __builtin_amdgcn_s_waitcnt(0x0F70);

  for (; tile < a.num_tiles; tile += gridDim.x) {
    const int next = tile + gridDim.x;
    __syncthreads();  // the previous tile's reads of sZ are done (and W_l is staged)
#pragma unroll
    for (int e = 0; e < G::ZP; ++e) {
      const int idx = threadIdx.x + G::THREADS * e;
      const int row = idx / PIECES, c = idx % PIECES;
      lds_write128(sZ + (uint32_t)(row * ROWB + ((c ^ zsw(row)) << 4)), nx.z[e]);
    }
    // the wave's own h columns (only this wave reads them back)
    typename std::conditional<MODE == 1, f32x4, u32x2>::type hc[TI][2];
#pragma unroll
    for (int t = 0; t < TI; ++t)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        hc[t][nt] = nx.h[t][nt];
        u32x2 v;
        if constexpr (MODE == 1)
          v = (u32x2){pack_f16(hc[t][nt][0], hc[t][nt][1]), pack_f16(hc[t][nt][2], hc[t][nt][3])};
        else
          v = hc[t][nt];
        lds_write64(sH + ((hst + (uint32_t)(16 * nt * ROWB)) ^ (uint32_t)((TI * w + t) << 5)), v);
      }
    if (next < a.num_tiles) load_tile<P, MODE>(a, next, w, q, g, nx);
    __syncthreads();  // sZ holds the tile

    if constexpr (DATA) {
      // dz_l^T (or dx^T) of the wave's units: C[16 it + 4 g + e][16 nt + q]
      f32x4 acc[TI][2];
#pragma unroll
      for (int t = 0; t < TI; ++t)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[t][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks < ksn) {
          const i16x8 b0 = lds_read128(sZ + (bz ^ (uint32_t)(ks << 6)));
          const i16x8 b1 = lds_read128(sZ + (bz ^ (uint32_t)(ks << 6)) + 16 * ROWB);
#pragma unroll
          for (int t = 0; t < TI; ++t) {
            if (!on[t]) continue;
            const int i = 16 * (TI * w + t) + q;
            const i16x8 av = lds_read128(sW + (uint32_t)(i * ROWB) + ((uint32_t)((g ^ q) << 4) ^ (uint32_t)(ks << 6)));
            acc[t][0] = mfma16x16x32(av, b0, acc[t][0], _Float16{});
            acc[t][1] = mfma16x16x32(av, b1, acc[t][1], _Float16{});
          }
        }
      }
      // derivative, fp16, store: rows 16 nt + q, units 16 it + 4 g .. + 3
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        u32x2 pk[TI];
#pragma unroll
        for (int t = 0; t < TI; ++t) {
          f32x4 v = acc[t][nt];
          if constexpr (MODE == 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = apply_grad<ACT>(v[e], hc[t][nt][e]);
          }
          pk[t] = (u32x2){pack_f16(v[0], v[1]), pack_f16(v[2], v[3])};
        }
        const __amdgpu_buffer_rsrc_t ro = rows_rsrc(a.out, a.M, (int64_t)tile * R + 16 * nt, 16, a.ldo, 2);
        const uint32_t rowoff = (uint32_t)q * (uint32_t)(a.ldo * 2);
        if constexpr (TI == 2) {
          // i tiles 2 w and 2 w + 1 are neighbours: one 16-byte store per lane
          const int u = 32 * w + 16 * (g & 1) + 8 * (g >> 1);
          store_pair(ro, lmask(u < I, rowoff + 2u * (uint32_t)u), pk[0], pk[1]);
        } else {
          const int u = 16 * w + 4 * g;
          __builtin_amdgcn_raw_buffer_store_b64(pk[0], ro, lmask(u < I, rowoff + 2u * (uint32_t)u), 0, 0);
        }
      }
    }

    // dW^T += dz_{l+1}^T h_l over the tile's 32 rows: C[16 jt + 4 g + e][16 it + q]
    i16x8 hb[TI];
#pragma unroll
    for (int t = 0; t < TI; ++t) {
      const uint32_t ad = sH + (trkh ^ (uint32_t)((TI * w + t) << 5));
      const i16x4 lo = lds_tr(ad), hi = lds_tr(ad + 16 * ROWB);
      hb[t] = (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
      if (jt < njn) {
        const uint32_t ad = sZ + (trk ^ (uint32_t)(jt << 5));
        const i16x4 lo = lds_tr(ad), hi = lds_tr(ad + 16 * ROWB);
        const i16x8 za = (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int t = 0; t < TI; ++t)
          if (on[t]) dw[t][jt] = mfma16x16x32(za, hb[t], dw[t][jt], _Float16{});
      }
    }
  }

  // this workgroup's partial dW_l: row i = 16 it + q, columns 16 jt + 4 g .. + 3
  float* part = a.partial + (size_t)blockIdx.x * (size_t)I * (size_t)J;
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    const int i = 16 * (TI * w + t) + q;
    if (i >= I) continue;
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
      const int j = 16 * jt + 4 * g;
      if (j < J) *(f32x4*)(part + (size_t)i * J + j) = dw[t][jt];
    }
  }
}

// Two consecutive layers per launch at width <= 128: the top layer t = l and
// the bottom layer b = l - 1.  The top layer's dz_l never leaves the
// workgroup: its epilogue writes it (fp16, the precision the next MFMAs take
// it in either way) into an LDS tile that the bottom layer's data product and
// weight gradient read, so a pair of layers reads dz_{l+1}, h_l and h_{l-1}
// and writes dz_{l-1} (or dx) once -- the HBM round trip of dz_l is gone.
// Same arithmetic per element as two single-layer launches, so the same bits.
struct Layer2Args {
  const void* dz;    // M x Jt fp16 (ldz): dLoss/dz_{l+1}
  const float* ht;   // M x It fp32 (ldht): h_l
  const void* hb;    // M x Ib: h_{l-1} in fp32 (l - 1 > 0) or x in fp16, pitch ldhb
  const void* Wt;    // It x Jt fp16, dense (W_l)
  const void* Wb;    // Ib x It fp16, dense (W_{l-1})
  void* out;         // M x Ib fp16 (ldo): dz_{l-1}, dx, or nullptr
  float* pt;         // grid x It x Jt fp32: partial dW_l
  float* pb;         // grid x Ib x It fp32: partial dW_{l-1}
  int64_t ldz, ldht, ldhb, ldo;
  int It, Jt, Ib, M, num_tiles;
};

template <int MODE>
struct Tile2Regs {
  u32x4 z;                                                   // dz_{l+1}: piece threadIdx.x of the tile
  f32x4 ht[2];                                               // h_l: rows 16 nt + q, units 16 w + 4 g .. + 3
  typename std::conditional<MODE == 1, f32x4, u32x2>::type hb[2];  // h_{l-1} (or x), same places
};

template <int MODE>
__device__ __forceinline__ void load_tile2(const Layer2Args& a, int tile, int w, int q, int g, Tile2Regs<MODE>& r) {
  using G = LGeo<128>;
  const int64_t row0 = (int64_t)tile * G::R;
  {
    const __amdgpu_buffer_rsrc_t rz = rows_rsrc(a.dz, a.M, row0, G::R, a.ldz, 2);
    const int row = threadIdx.x / G::PIECES, c = threadIdx.x % G::PIECES;
    r.z = __builtin_amdgcn_raw_buffer_load_b128(
        rz, lmask(8 * c < a.Jt, (uint32_t)row * (uint32_t)(a.ldz * 2) + 16u * (uint32_t)c), 0, 0);
  }
  const int u = 16 * w + 4 * g;  // the lane's first unit
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const __amdgpu_buffer_rsrc_t rt = rows_rsrc(a.ht, a.M, row0 + 16 * nt, 16, a.ldht, 4);
    r.ht[nt] = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                   rt, lmask(u < a.It, (uint32_t)q * (uint32_t)(a.ldht * 4) + 4u * (uint32_t)u), 0, 0));
    const __amdgpu_buffer_rsrc_t rb = rows_rsrc(a.hb, a.M, row0 + 16 * nt, 16, a.ldhb, MODE == 1 ? 4 : 2);
    if constexpr (MODE == 1)
      r.hb[nt] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rb, lmask(u < a.Ib, (uint32_t)q * (uint32_t)(a.ldhb * 4) + 4u * (uint32_t)u), 0, 0));
    else
      r.hb[nt] = __builtin_amdgcn_raw_buffer_load_b64(
          rb, lmask(u < a.Ib, (uint32_t)q * (uint32_t)(a.ldhb * 2) + 2u * (uint32_t)u), 0, 0);
  }
}

// One wave's share of a layer's data product over a 32-row tile: the 16
// units 16 w .. of the output side (A = rows of W from LDS, B = the staged
// input-gradient tile), k steps < ksn.  acc[nt] = C[16 w + 4 g + e][16 nt + q].
__device__ __forceinline__ void data_product128(uint32_t sWr, uint32_t sIn, uint32_t bz, int w, int q, int g,
                                                int ksn, f32x4 (&acc)[2]) {
  using G = LGeo<128>;
  acc[0] = acc[1] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const uint32_t arow = sWr + (uint32_t)((16 * w + q) * G::ROWB);
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    if (ks < ksn) {
      const i16x8 b0 = lds_read128(sIn + (bz ^ (uint32_t)(ks << 6)));
      const i16x8 b1 = lds_read128(sIn + (bz ^ (uint32_t)(ks << 6)) + 16 * G::ROWB);
      const i16x8 av = lds_read128(arow + ((uint32_t)((g ^ q) << 4) ^ (uint32_t)(ks << 6)));
      acc[0] = mfma16x16x32(av, b0, acc[0], _Float16{});
      acc[1] = mfma16x16x32(av, b1, acc[1], _Float16{});
    }
  }
}

// One wave's weight-gradient terms of a 32-row tile: dW^T (rows j of the
// input-gradient side, columns the wave's 16 units) += sIn^T sH over the
// rows, j tiles < njn (sIn in the zsw layout, read at trk; sH in the hsw
// layout, read at trkh).
__device__ __forceinline__ void weight_grad128(uint32_t sIn, uint32_t sH, uint32_t trk, uint32_t trkh, int w,
                                               int njn, f32x4 (&dw)[LGeo<128>::NJ]) {
  using G = LGeo<128>;
  const uint32_t ah = sH + (trkh ^ (uint32_t)(w << 5));
  const i16x4 hl = lds_tr(ah), hh = lds_tr(ah + 16 * G::ROWB);
  const i16x8 hb = (i16x8){hl[0], hl[1], hl[2], hl[3], hh[0], hh[1], hh[2], hh[3]};
#pragma unroll
  for (int jt = 0; jt < G::NJ; ++jt) {
    if (jt < njn) {
      const uint32_t ad = sIn + (trk ^ (uint32_t)(jt << 5));
      const i16x4 lo = lds_tr(ad), hi = lds_tr(ad + 16 * G::ROWB);
      const i16x8 za = (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      dw[jt] = mfma16x16x32(za, hb, dw[jt], _Float16{});
    }
  }
}

// Stage W (rows x cols fp16, dense, rows <= 128) as LDS rows of 256 bytes,
// zero past the matrix up to the next 16 rows and 128 columns.
__device__ __forceinline__ void stage_w128(uint32_t sWr, const void* W, int rows, int cols) {
  stage_w_rows<LGeo<128>::THREADS, LGeo<128>::PIECES, 128>(sWr, W, rows, cols);
}

// ACT: the hidden activation (the top layer's derivative, and the bottom
// layer's in MODE 1).  MODE of the bottom layer: 1 hidden (dz_{l-1} with the
// derivative), 2 the first layer with dx, 0 the first layer without dx.
template <int ACT, int MODE>
__global__ __launch_bounds__(LGeo<128>::THREADS, 1) void mlp_layer2_bwd_kernel(Layer2Args a) {
  using G = LGeo<128>;
  constexpr int R = G::R, ROWB = G::ROWB, NJ = G::NJ;
  // W_l, W_{l-1} (128 rows each), then dz_{l+1}, h_l, dz_l, h_{l-1} tiles (32 rows each)
  __shared__ __attribute__((aligned(1024))) unsigned char lds[(2 * 128 + 4 * R) * ROWB];
  const uint32_t sWt = lds_addr(lds), sWb = sWt + 128 * ROWB, sZ = sWb + 128 * ROWB, sH = sZ + R * ROWB,
                 sZ2 = sH + R * ROWB, sH2 = sZ2 + R * ROWB;
  const int It = a.It, Jt = a.Jt, Ib = a.Ib;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, q = lane & 15, g = lane >> 4;

  const bool on_t = 16 * w < It, on_b = 16 * w < Ib;
  const int ksn_t = (Jt + 31) >> 5, njn_t = (Jt + 15) >> 4;
  const int ksn_b = (It + 31) >> 5, njn_b = (It + 15) >> 4;
  const uint32_t zrow = (uint32_t)(q * ROWB);
  const uint32_t bz = zrow + (uint32_t)((g ^ zsw(q)) << 4);
  const int rt = 4 * g + (q >> 2);
  const uint32_t trk = (uint32_t)(rt * ROWB + ((((q & 3) >> 1) ^ zsw(rt)) << 4) + ((q & 1) << 3));
  const uint32_t trkh = (uint32_t)(rt * ROWB + (((q & 3) ^ hsw(rt)) << 3));
  // the lane's 8-byte staging place (rows q and 16 + q, units 16 w + 4 g .. + 3):
  // dz_l (read by the bottom data product's 16-byte reads too) in the zsw
  // layout, h_l and h_{l-1} in the hsw layout
  const uint32_t hst = (zrow + (uint32_t)((((g >> 1) ^ zsw(q)) << 4) + ((g & 1) << 3))) ^ (uint32_t)(w << 5);
  const uint32_t hsth = (zrow + (uint32_t)((g ^ hsw(q)) << 3)) ^ (uint32_t)(w << 5);

  f32x4 dwt[NJ], dwb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) dwt[j] = dwb[j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  Tile2Regs<MODE> nx;
  int tile = blockIdx.x;
  if (tile < a.num_tiles) load_tile2<MODE>(a, tile, w, q, g, nx);
  // the weights, loaded behind the first tile
  stage_w128(sWt, a.Wt, It, Jt);
  if constexpr (MODE != 0) stage_w128(sWb, a.Wb, Ib, It);
  __builtin_amdgcn_s_waitcnt(0x0F70);

  for (; tile < a.num_tiles; tile += gridDim.x) {
    const int next = tile + gridDim.x;
    __syncthreads();  // the previous tile's reads of the tiles are done (and the weights are staged)
    {
      const int row = threadIdx.x / G::PIECES, c = threadIdx.x % G::PIECES;
      lds_write128(sZ + (uint32_t)(row * ROWB + ((c ^ zsw(row)) << 4)), nx.z);
    }
    f32x4 hct[2];
    typename std::conditional<MODE == 1, f32x4, u32x2>::type hcb[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      hct[nt] = nx.ht[nt];
      hcb[nt] = nx.hb[nt];
      lds_write64(sH + hsth + (uint32_t)(16 * nt * ROWB),
                  (u32x2){pack_f16(hct[nt][0], hct[nt][1]), pack_f16(hct[nt][2], hct[nt][3])});
      u32x2 vb;
      if constexpr (MODE == 1)
        vb = (u32x2){pack_f16(hcb[nt][0], hcb[nt][1]), pack_f16(hcb[nt][2], hcb[nt][3])};
      else
        vb = hcb[nt];
      lds_write64(sH2 + hsth + (uint32_t)(16 * nt * ROWB), vb);
    }
    if (next < a.num_tiles) load_tile2<MODE>(a, next, w, q, g, nx);
    __syncthreads();  // sZ holds dz_{l+1}

    // top layer: dz_l = (dz_{l+1} W_l^T) * act'(h_l) into sZ2 (zeros where
    // the wave's units lie past It, so the bottom product reads finite values)
    {
      f32x4 acc[2];
      if (on_t) {
        data_product128(sWt, sZ, bz, w, q, g, ksn_t, acc);
      } else {
        acc[0] = acc[1] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 v = acc[nt];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = apply_grad<ACT>(v[e], hct[nt][e]);
        lds_write64(sZ2 + hst + (uint32_t)(16 * nt * ROWB), (u32x2){pack_f16(v[0], v[1]), pack_f16(v[2], v[3])});
      }
    }
    if (on_t) weight_grad128(sZ, sH, trk, trkh, w, njn_t, dwt);
    __syncthreads();  // sZ2 holds dz_l

    // bottom layer: dz_{l-1} (MODE 1) or dx (MODE 2) from dz_l, and dW_{l-1}
    if constexpr (MODE != 0) {
      if (on_b) {
        f32x4 acc[2];
        data_product128(sWb, sZ2, bz, w, q, g, ksn_b, acc);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          f32x4 v = acc[nt];
          if constexpr (MODE == 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = apply_grad<ACT>(v[e], hcb[nt][e]);
          }
          const __amdgpu_buffer_rsrc_t ro = rows_rsrc(a.out, a.M, (int64_t)tile * R + 16 * nt, 16, a.ldo, 2);
          const int u = 16 * w + 4 * g;
          __builtin_amdgcn_raw_buffer_store_b64((u32x2){pack_f16(v[0], v[1]), pack_f16(v[2], v[3])}, ro,
                                                lmask(u < Ib, (uint32_t)q * (uint32_t)(a.ldo * 2) + 2u * (uint32_t)u),
                                                0, 0);
        }
      }
    }
    if (on_b) weight_grad128(sZ2, sH2, trk, trkh, w, njn_b, dwb);
  }

  // partial sums: rows i = 16 w + q, columns 16 jt + 4 g .. + 3
  {
    const int i = 16 * w + q;
    float* pt = a.pt + (size_t)blockIdx.x * (size_t)It * (size_t)Jt;
    float* pb = a.pb + (size_t)blockIdx.x * (size_t)Ib * (size_t)It;
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
      const int j = 16 * jt + 4 * g;
      if (i < It && j < Jt) *(f32x4*)(pt + (size_t)i * Jt + j) = dwt[jt];
      if (i < Ib && j < It) *(f32x4*)(pb + (size_t)i * It + j) = dwb[jt];
    }
  }
}

// dW = sum of nparts partials of E float4 groups each (row-major, as dW).  A
// workgroup owns 32 groups and splits the partial index over 8 slices (slice
// s adds partials s, s + 8, ... in order), then adds the slice sums in slice
// order: a fixed order for a given grid.  One launch sums up to two layers
// (a two-layer launch's partials): the first blocks0 workgroups the first,
// the rest the second.
constexpr int LRED_GROUPS = 32, LRED_SLICES = 8;

struct ReduceSeg {
  const float* partial;
  float* dW;
  int E;
};

__global__ __launch_bounds__(LRED_GROUPS* LRED_SLICES) void layer_bwd_reduce(ReduceSeg s0, ReduceSeg s1, int blocks0,
                                                                              int nparts) {
  __shared__ f32x4 red[LRED_SLICES][LRED_GROUPS];
  const bool second = (int)blockIdx.x >= blocks0;
  const float* __restrict__ partial = second ? s1.partial : s0.partial;
  float* __restrict__ dW = second ? s1.dW : s0.dW;
  const int E = second ? s1.E : s0.E;
  const int gi = threadIdx.x % LRED_GROUPS, slice = threadIdx.x / LRED_GROUPS;
  const int e = ((int)blockIdx.x - (second ? blocks0 : 0)) * LRED_GROUPS + gi;
  f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (e < E) {
    const f32x4* src = (const f32x4*)partial + e;
#pragma unroll 8
    for (int b = slice; b < nparts; b += LRED_SLICES) acc += src[(size_t)b * E];
  }
  red[slice][gi] = acc;
  __syncthreads();
  if (slice != 0 || e >= E) return;
  f32x4 sum = red[0][gi];
#pragma unroll
  for (int k = 1; k < LRED_SLICES; ++k) sum += red[k][gi];
  float* d = dW + 4 * (size_t)e;  // dW is only 4-byte aligned
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = sum[i];
}

template <int P, int ACT, int MODE>
hipError_t launch_layer(const LayerArgs& a, int nwg, hipStream_t stream) {
  hipLaunchKernelGGL((mlp_layer_bwd_kernel<P, ACT, MODE>), dim3(nwg), dim3(LGeo<P>::THREADS), 0, stream, a);
  return hipGetLastError();
}

template <int P>
hipError_t launch_layer_p(const LayerArgs& a, int mode, int act, int nwg, hipStream_t stream) {
  if (mode == 0) return launch_layer<P, ACT_NONE, 0>(a, nwg, stream);
  if (mode == 2) return launch_layer<P, ACT_NONE, 2>(a, nwg, stream);
  if (act == ACT_SOFTPLUS) return launch_layer<P, ACT_SOFTPLUS, 1>(a, nwg, stream);
  if (act == ACT_RELU) return launch_layer<P, ACT_RELU, 1>(a, nwg, stream);
  return launch_layer<P, ACT_NONE, 1>(a, nwg, stream);
}

constexpr int kRowsPerTile = 32;

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct StreamBwdLayout {
  size_t partial_bytes;  // per-workgroup partial sums (a pair's two layers share it: it holds
                         // 2 x #CUs partials of the largest layer)
  size_t dz_bytes;       // one M-row fp16 buffer of hidden gradients
  int ldz;
  int max_groups;        // workgroups of a launch at most
  bool pairs;            // width <= 128: two layers per launch
  int nbuf;              // dz buffers needed
};

StreamBwdLayout stream_bwd_layout(const int* dims, int L, int64_t M, int num_cus) {
  StreamBwdLayout s{};
  size_t maxij = 0;
  int ldz = 8, mx = 0;
  for (int l = 0; l < L; ++l) maxij = std::max(maxij, (size_t)dims[l] * (size_t)dims[l + 1]);
  for (int l = 1; l < L; ++l) ldz = std::max(ldz, dims[l]);
  for (int l = 0; l <= L; ++l) mx = std::max(mx, dims[l]);
  // Width <= 128: a single-layer launch takes 48 KB of LDS and under 128
  // VGPRs a lane, so two of its workgroups share a CU (twice the row tiles
  // in flight); the two-layer launch (96 KB) one.  Width 256 fills the LDS
  // with one layer's weights.
  s.pairs = mx <= 128;
  s.max_groups = std::max(num_cus, 1) * (mx > 128 ? 1 : 2);
  s.partial_bytes = align256((size_t)s.max_groups * maxij * sizeof(float));
  s.dz_bytes = align256((size_t)std::max<int64_t>(M, 0) * (size_t)ldz * 2);
  s.ldz = ldz;
  // hidden gradients that leave a launch: every dz_l (l = L-1 .. 1) one layer
  // at a time; with pairs only the dz_{l-1} at the bottom of each pair
  int writes = 0;
  for (int l = L - 1; l >= 0;) {
    const int step = s.pairs && l >= 1 ? 2 : 1;
    if (l - step + 1 > 0) ++writes;
    l -= step;
  }
  s.nbuf = std::min(writes, 2);
  return s;
}

}  // namespace

size_t mlp_backward_stream_workspace(const int* dims, int L, int64_t M, int num_cus) {
  const StreamBwdLayout s = stream_bwd_layout(dims, L, M, num_cus);
  return s.partial_bytes + (size_t)s.nbuf * s.dz_bytes;
}

hipError_t launch_mlp_backward_stream(const MlpStreamBwdParams& p, int P, int hidden_act, int num_cus,
                                      void* workspace, hipStream_t stream) {
  const StreamBwdLayout s = stream_bwd_layout(p.dims, p.L, p.M, num_cus);
  const int tiles = (int)(((int64_t)p.M + kRowsPerTile - 1) / kRowsPerTile);
  const int nwg = std::max(1, std::min(tiles, s.max_groups));
  const int nwg2 = std::max(1, std::min(tiles, std::max(num_cus, 1)));
  char* ws = (char*)workspace;
  float* partial = (float*)ws;
  char* zbase = ws + s.partial_bytes;
  // The hidden gradients that leave a launch alternate between two buffers:
  // a launch reads the previous one's and writes the other.
  void* zbuf[2] = {zbase, zbase + s.dz_bytes};
  const void* zin = p.dout;
  int64_t ldzin = p.ldd;
  int zsel = 0;
  // the sums of one or two layers' partials (nparts each) in one launch
  auto reduce = [&](int nparts, ReduceSeg s0, ReduceSeg s1) -> hipError_t {
    const int b0 = (s0.E + LRED_GROUPS - 1) / LRED_GROUPS, b1 = (s1.E + LRED_GROUPS - 1) / LRED_GROUPS;
    hipLaunchKernelGGL(layer_bwd_reduce, dim3(b0 + b1), dim3(LRED_GROUPS * LRED_SLICES), 0, stream, s0, s1, b0,
                       nparts);
    return hipGetLastError();
  };
  hipError_t e = hipSuccess;
  for (int l = p.L - 1; l >= 0;) {
    if (s.pairs && l >= 1) {
      // layers l (top) and l - 1 (bottom) in one launch
      const int b = l - 1;
      Layer2Args a{};
      a.dz = zin;
      a.ldz = ldzin;
      a.ht = p.acts[l - 1];
      a.ldht = p.lda;
      a.Wt = p.W[l];
      a.Wb = p.W[b];
      a.It = p.dims[l];
      a.Jt = p.dims[l + 1];
      a.Ib = p.dims[b];
      a.M = p.M;
      a.num_tiles = tiles;
      // the top layer's partials, then the bottom layer's: nwg2 x (It Jt + Ib
      // It) floats, within 2 #CUs x the largest layer
      a.pt = partial;
      a.pb = partial + (size_t)nwg2 * (size_t)a.It * (size_t)a.Jt;
      int mode;
      if (b > 0) {
        mode = 1;
        a.hb = p.acts[b - 1];
        a.ldhb = p.lda;
        a.out = zbuf[zsel];
        a.ldo = s.ldz;
      } else {
        mode = p.dx ? 2 : 0;
        a.hb = p.x;
        a.ldhb = p.ldx;
        a.out = p.dx;
        a.ldo = p.ldq;
      }
      // (ACT is the top layer's activation, whose derivative every pair applies)
      if (mode == 0 && hidden_act == ACT_SOFTPLUS)
        hipLaunchKernelGGL((mlp_layer2_bwd_kernel<ACT_SOFTPLUS, 0>), dim3(nwg2), dim3(LGeo<128>::THREADS), 0, stream,
                           a);
      else if (mode == 0 && hidden_act == ACT_RELU)
        hipLaunchKernelGGL((mlp_layer2_bwd_kernel<ACT_RELU, 0>), dim3(nwg2), dim3(LGeo<128>::THREADS), 0, stream, a);
      else if (mode == 0)
        hipLaunchKernelGGL((mlp_layer2_bwd_kernel<ACT_NONE, 0>), dim3(nwg2), dim3(LGeo<128>::THREADS), 0, stream, a);
      else if (mode == 2 && hidden_act == ACT_SOFTPLUS)
        hipLaunchKernelGGL((mlp_layer2_bwd_kernel<ACT_SOFTPLUS, 2>), dim3(nwg2), dim3(LGeo<128>::THREADS), 0, stream,
                           a);
      else if (mode == 2 && hidden_act == ACT_RELU)
        hipLaunchKernelGGL((mlp_layer2_bwd_kernel<ACT_RELU, 2>), dim3(nwg2), dim3(LGeo<128>::THREADS), 0, stream, a);
      else if (mode == 2)
        hipLaunchKernelGGL((mlp_layer2_bwd_kernel<ACT_NONE, 2>), dim3(nwg2), dim3(LGeo<128>::THREADS), 0, stream, a);
      else if (hidden_act == ACT_SOFTPLUS)
        hipLaunchKernelGGL((mlp_layer2_bwd_kernel<ACT_SOFTPLUS, 1>), dim3(nwg2), dim3(LGeo<128>::THREADS), 0, stream,
                           a);
      else if (hidden_act == ACT_RELU)
        hipLaunchKernelGGL((mlp_layer2_bwd_kernel<ACT_RELU, 1>), dim3(nwg2), dim3(LGeo<128>::THREADS), 0, stream, a);
      else
        hipLaunchKernelGGL((mlp_layer2_bwd_kernel<ACT_NONE, 1>), dim3(nwg2), dim3(LGeo<128>::THREADS), 0, stream, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = reduce(nwg2, ReduceSeg{partial, p.dW[l], a.It * a.Jt / 4}, ReduceSeg{a.pb, p.dW[b], a.Ib * a.It / 4})) !=
          hipSuccess)
        return e;
      if (b > 0) {
        zin = zbuf[zsel];
        ldzin = s.ldz;
        zsel ^= 1;
      }
      l -= 2;
      continue;
    }
    LayerArgs a{};
    a.I = p.dims[l];
    a.J = p.dims[l + 1];
    a.M = p.M;
    a.num_tiles = tiles;
    a.W = p.W[l];
    a.partial = partial;
    a.dz = zin;
    a.ldz = ldzin;
    int mode;
    if (l > 0) {
      mode = 1;
      a.h = p.acts[l - 1];
      a.ldh = p.lda;
      a.out = zbuf[zsel];
      a.ldo = s.ldz;
    } else {
      mode = p.dx ? 2 : 0;
      a.h = p.x;
      a.ldh = p.ldx;
      a.out = p.dx;
      a.ldo = p.ldq;
    }
    e = P == 256 ? launch_layer_p<256>(a, mode, hidden_act, nwg, stream)
                 : launch_layer_p<128>(a, mode, hidden_act, nwg, stream);
    if (e != hipSuccess) return e;
    if ((e = reduce(nwg, ReduceSeg{partial, p.dW[l], a.I * a.J / 4}, ReduceSeg{partial, p.dW[l], 0})) != hipSuccess)
      return e;
    if (l > 0) {
      zin = zbuf[zsel];
      ldzin = s.ldz;
      zsel ^= 1;
    }
    l -= 1;
  }
  return hipSuccess;
}

}  // namespace coalesce
