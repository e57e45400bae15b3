// Fused GEMM + bias + activation for bf16 / fp16 inputs on gfx950 MFMA.
//
// Y = act(A . B + bias) ("Coalesce" README, "Fusion study"): the bias add and
// the activation run on the fp32 accumulators in registers and Y is written
// once.  Tile plan (hand-budgeted against the 256 registers a lane has when
// two waves share a SIMD), given for the 256 x 256 tile of large problems;
// smaller problems take 128 x 128 tiles (4 waves of 64 x 64) or 64 x 64
// tiles (4 waves of 32 x 32), the same code at a smaller scale (see Geo and
// the tile choice in launch_gemm16):
//   * workgroup tile 256 (m) x 256 (n), K step 64, 8 waves in a 2 x 4 grid,
//     each wave owning a 128 (m) x 64 (n) block of Y;
//   * the wave computes Y^T blocks with v_mfma_f32_16x16x32 -- A operand =
//     B^T (rows n), B operand = A^T (columns m) -- so every lane ends up with
//     4 consecutive n of one row m, which makes bias loads contiguous;
//   * accumulators: 4 x 8 sub-tiles x 4 fp32 = 128 registers; operand
//     fragments for one 32-deep k slice: 4 + 8 x 4 = 48 registers, double
//     buffered;
//   * global -> LDS copies are 16-byte direct-to-LDS loads (no VGPR staging)
//     addressed as an SGPR base plus a per-lane 32-bit offset; two LDS stages
//     of 64 KB; K step k + 2 is copied while step k + 1 is consumed;
//   * B is K x N with n contiguous, so its MFMA fragments (8 consecutive k of
//     one n) come from the transposing LDS read ds_read_b64_tr_b16;
//   * LDS rows are XOR-swizzled in 16-byte chunks so that fragment reads
//     spread over the banks;
//   * each 32-deep slice is issued as 4 groups of {2 copies, 8 MFMAs, a
//     share of the next slice's fragment reads, those its first group needs
//     first}, fenced so the compiler keeps that interleave: the copies never
//     arrive as a burst that stalls the wave's in-order issue, and the MFMA
//     pipe is fed between them;
//   * the epilogue stages each wave's block in the (then free) LDS and stores
//     whole 128-byte lines of Y;
//   * the kernel is persistent (as many workgroups as fit on the CUs walking
//     the tiles), and the next tile's first copies are issued while the
//     current tile's stores drain.
// The last, partial K step (K not a multiple of 64) goes through masked
// register loads that zero every element past K.  Rows past M read a
// clamped (valid) row and are never stored; columns past N are masked.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace coalesce {
namespace {

constexpr int BK = 64;

// Tile configurations (BM x BN workgroup tile, NW waves in a 2 x NW/2 grid):
//   * 256 x 256, 8 waves: two waves per SIMD, each owning 128 (m) x 64 (n)
//     (128 accumulators), so that one wave's memory stalls are covered by the
//     other wave's MFMAs; one workgroup per CU (the two LDS stages take
//     128 KB).  The large problems' tile.
//   * 128 x 128, 4 waves of 64 x 64 (64 accumulators): two workgroups per CU
//     (64 KB of LDS each), again two waves per SIMD.  Four times the tiles of
//     the 256 x 256 plan, for problems whose 256 x 256 tiles would leave CUs
//     idle; it moves twice the operand bytes per flop.
//   * 64 x 64, 4 waves of 32 x 32: four workgroups per CU (32 KB of LDS
//     each), four waves per SIMD, for problems whose 128 x 128 tiles would
//     still leave most CUs idle.
// MINW is the launch-bounds floor of waves per SIMD, which caps the registers
// a wave may use (256 at two waves per SIMD).
template <int BM_, int BN_, int NW_, int MINW_>
struct Geo {
  static constexpr int BM = BM_, BN = BN_, NW = NW_, MINW = MINW_;
  static constexpr int THREADS = NW * 64;
  static constexpr int WGN = NW / 2;        // waves along n (two along m)
  static constexpr int WM = BM / 2;         // wave tile height (m)
  static constexpr int WN = BN / WGN;       // wave tile width (n)
  static constexpr int NT = WN / 16;        // 16-wide n sub-tiles per wave
  static constexpr int MT = WM / 16;        // 16-row m sub-tiles per wave
  static constexpr int CA = BM / 8 / NW;    // 1 KB A copies per wave per K step (8 rows of 64 k each)
  static constexpr int CB = BN / 8 / NW;    // 1 KB B copies per wave per K step
  static constexpr int CPRB = BN / 8;       // 16-byte chunks per B row
  static constexpr int CPRB_LOG = CPRB == 32 ? 5 : CPRB == 16 ? 4 : 3;
  static constexpr int BRPC = 64 / CPRB;    // B rows (k) per 1 KB copy
  static_assert((1 << CPRB_LOG) == CPRB && BRPC * CPRB == 64 && CA * NW * 8 == BM && CB * NW * BRPC == BK, "copy plan does not cover the tile");
};
typedef Geo<256, 256, 8, 1> Geo256;
typedef Geo<128, 128, 4, 2> Geo128;
typedef Geo<64, 64, 4, 4> Geo64;

// LDS layouts, 16-byte chunks XOR-swizzled so that every fragment read is
// free of bank conflicts whether the LDS serves 128 or 256 bytes per clock:
//   A tile: BM rows of 64 k (128 B = 8 chunks); chunk c of row m sits at slot
//     c ^ swzA(m).  A 128-bit read by 16 lanes (rows m0..m0+15, one chunk)
//     hits 16 distinct 16-byte slots of a 256-byte window, and any 8
//     consecutive rows hit 8 distinct slots of a 128-byte window.
//   B tile: 64 rows of BN n (512, 256 or 128 B = 32, 16 or 8 chunks); chunk c
//     of row k sits at slot c ^ swzB(k) (below the row's chunk count, and
//     below 16, so a chunk stays in its 256-byte part of a row).  A
//     transposing read by 32 lanes (rows k0..k0+3 and k0+8..k0+11, two chunks,
//     two 8-byte halves) hits 32 distinct 8-byte slots of a 256-byte window
//     (which holds two rows when they are 128 bytes long).
// Neither swizzle depends on the sub-tile index s, the slice ks or the half of
// a transposing read, so those stay immediate offsets of the LDS reads.
__device__ __forceinline__ int swzA(int m) { return ((m >> 1) & 7) ^ ((m & 1) << 2); }
template <typename G>
__device__ __forceinline__ int swzB(int k) {
  if constexpr (G::CPRB >= 16)
    return ((k & 3) << 1) | (((k >> 3) & 1) << 3);
  else  // 128-byte rows: a 256-byte window holds two rows, k and k ^ 1
    return (((k >> 1) & 1) << 1) | (((k >> 3) & 1) << 2);
}

template <typename T>
struct Stage {
  T* a;
  T* b;
};

// Direct copies of one K step: copy j < CA fills A rows 8 (w CA + j) .. + 7
// (one 1 KB LDS block, lane l's 16 bytes at slot l); copy CA + j fills the
// BRPC B rows from BRPC (w CB + j) on.  The per-lane byte offsets, relative to
// the tile's A base (A + m0 * lda + k0) and B base (B + n0 + k0 * ldb), do not
// depend on k0; they are written as computed from the lane index at each copy
// and the compiler keeps them in registers across the K loop where it can.
struct DmaPlan {
  const GemmParams* p;
  int m0, n0, w, lane;
};

__device__ __forceinline__ DmaPlan make_plan(const GemmParams& p, int m0, int n0, int w, int lane) {
  return DmaPlan{&p, m0, n0, w, lane};
}

template <typename T, typename G>
__device__ __forceinline__ uint32_t dma_offset(const DmaPlan& d, int j) {
  const GemmParams& p = *d.p;
  // 32-bit arithmetic is exact here: the host checks 256 * lda and 64 * ldb
  // bytes fit in 32 bits.
  if (j < G::CA) {
    const uint32_t lda_b = (uint32_t)p.lda * (uint32_t)sizeof(T);
    const int row = (d.w * G::CA + j) * 8 + (d.lane >> 3);
    const int cA = (d.lane & 7) ^ swzA(row);
    const int gm = min(d.m0 + row, p.M - 1);
    return (uint32_t)(gm - d.m0) * lda_b + (uint32_t)(cA * 8 * (int)sizeof(T));
  } else {
    const uint32_t ldb_b = (uint32_t)p.ldb * (uint32_t)sizeof(T);
    const int nlast = ((p.N - 1) >> 3) << 3;
    const int row = (d.w * G::CB + j - G::CA) * G::BRPC + (d.lane >> G::CPRB_LOG);
    const int cB = (d.lane & (G::CPRB - 1)) ^ swzB<G>(row);
    const int gn = min(d.n0 + cB * 8, nlast);
    return (uint32_t)row * ldb_b + (uint32_t)((gn - d.n0) * (int)sizeof(T));
  }
}

// Uniform (SGPR) 64-bit base for a direct copy.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16-byte direct copy: global (SGPR base + per-lane 32-bit offset) -> LDS
// (wave-uniform byte address + 16 * lane).
__device__ __forceinline__ void dma16_off(const void* base, uint32_t off, uint32_t lds) {
  // one wait state between the M0 write and the LDS-DMA instruction that reads it
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Copy j (0 .. CA + CB - 1) of a K step into stage st.
template <typename T, typename G>
__device__ __forceinline__ void dma_copy(int j, const DmaPlan& d, const void* abase, const void* bbase, Stage<T> st,
                                         int wu) {
  if (j < G::CA)
    dma16_off(abase, dma_offset<T, G>(d, j), lds_addr(st.a) + (uint32_t)((wu * G::CA + j) * 8) * (BK * (int)sizeof(T)));
  else
    dma16_off(bbase, dma_offset<T, G>(d, j),
              lds_addr(st.b) + (uint32_t)((wu * G::CB + j - G::CA) * G::BRPC) * (G::BN * (int)sizeof(T)));
}

template <typename T>
__device__ __forceinline__ const void* a_base(const GemmParams& p, int m0, int k0) {
  return uniform_ptr((const T*)p.A + (int64_t)m0 * p.lda + k0);
}
template <typename T>
__device__ __forceinline__ const void* b_base(const GemmParams& p, int n0, int k0) {
  return uniform_ptr((const T*)p.B + (int64_t)k0 * p.ldb + n0);
}

// All copies of a full K step at once (prologue only).
template <typename T, typename G>
__device__ __forceinline__ void dma_all(const GemmParams& p, const DmaPlan& d, int m0, int n0, int k0, Stage<T> st,
                                        int wu) {
  const void* ab = a_base<T>(p, m0, k0);
  const void* bb = b_base<T>(p, n0, k0);
#pragma unroll
  for (int j = 0; j < G::CA + G::CB; ++j) dma_copy<T, G>(j, d, ab, bb, st, wu);
}

// Partial last K step: masked loads (elements at k >= K become 0), written to
// the same LDS slots the direct copies would use.
template <typename T, typename G>
__device__ __forceinline__ void tail_fill(const GemmParams& p, int m0, int n0, int k0, Stage<T> st, int w, int lane) {
  const T* A = (const T*)p.A;
  const T* B = (const T*)p.B;
  const int rsub = lane >> 3;
  const int nlast = ((p.N - 1) >> 3) << 3;
  i16x8 ra[G::CA], rb[G::CB];
#pragma unroll
  for (int j = 0; j < G::CA; ++j) {
    const int row = (w * G::CA + j) * 8 + rsub;
    const int kA = k0 + ((lane & 7) ^ swzA(row)) * 8;
    const int gm = min(m0 + row, p.M - 1);
    i16x8 v = (i16x8){0, 0, 0, 0, 0, 0, 0, 0};
    if (kA < p.K) {
      v = *(const i16x8*)(A + (int64_t)gm * p.lda + kA);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (kA + e >= p.K) v[e] = 0;
    }
    ra[j] = v;
  }
#pragma unroll
  for (int j = 0; j < G::CB; ++j) {
    const int row = (w * G::CB + j) * G::BRPC + (lane >> G::CPRB_LOG);
    const int cB = (lane & (G::CPRB - 1)) ^ swzB<G>(row);
    const int gn = min(n0 + cB * 8, nlast);
    i16x8 v = (i16x8){0, 0, 0, 0, 0, 0, 0, 0};
    if (k0 + row < p.K) v = *(const i16x8*)(B + (int64_t)(k0 + row) * p.ldb + gn);
    rb[j] = v;
  }
#pragma unroll
  for (int j = 0; j < G::CA; ++j) *(i16x8*)(st.a + (w * G::CA + j) * 8 * BK + lane * 8) = ra[j];
#pragma unroll
  for (int j = 0; j < G::CB; ++j) *(i16x8*)(st.b + (w * G::CB + j) * G::BRPC * G::BN + lane * 8) = rb[j];
}

// Operand fragments of one 32-deep k slice (ks = 0 or 1 of a stage):
//   b[s]: B operand = A^T, rows m = WM wm + 16 s + (lane & 15), k = 8 (lane >> 4) + e
//         (WM = 128 / 64 / 32 for the 256 / 128 / 64 tiles);
//   a[t]: A operand = B^T, rows n = WN wn + 16 t + (lane & 15), same k, as two
//         transposing reads of 4 k (lo: e = 0..3, hi: e = 4..7).
template <typename G>
struct Frags {
  i16x8 a[G::NT];
  i16x8 b[G::MT];
};

template <typename T, typename G>
__device__ __forceinline__ i16x8 read_bf(Stage<T> st, int ks, int wm, int s, int lane) {
  const int m = wm * G::WM + 16 * s + (lane & 15);
  const int c = (4 * ks + (lane >> 4)) ^ swzA(m);
  return *(const i16x8*)(st.a + m * BK + c * 8);
}

template <typename T, typename G>
__device__ __forceinline__ i16x4 read_af_half(Stage<T> st, int ks, int wn, int t, int half, int lane) {
  const int q = lane & 15;
  const int n = wn * G::WN + 16 * t + 4 * (q & 3);
  const int k = 32 * ks + 8 * (lane >> 4) + 4 * half + (q >> 2);
  return lds_read_tr16(st.b + k * G::BN + (((n >> 3) ^ swzB<G>(k)) << 3) + (n & 7));
}

// One slice: NT groups of {2 copies of K step k + 2 when `copy` (a uniform
// branch around the copies only), the MT MFMAs of sub-tile t, a share of the
// next slice's fragment reads}.  The next slice's first group needs every
// m-side fragment and a[0], so those are read in the first two groups and the
// later a[t] after them: no MFMA at the start of a slice waits for a read
// issued just before it (1.8 % faster than reading a[t] and two m-side
// fragments in group t).  A scheduling fence closes every group.  The MFMAs
// never sit inside a branch, so the accumulators stay in AGPRs.  On the last
// K step the "next" reads fetch stale but in-bounds LDS and are unused.
template <typename T, typename G>
__device__ __forceinline__ void slice(const Frags<G>& cur, f32x4 (&acc)[G::NT][G::MT], Frags<G>& nxt, Stage<T> rst,
                                      int rks, int wm, int wn, int lane, bool copy, const DmaPlan& d, const void* ab,
                                      const void* bb, Stage<T> cst, int wu) {
  static_assert(((G::NT == 4 && (G::MT == 8 || G::MT == 4)) || (G::NT == 2 && G::MT == 2)) &&
                    G::CA + G::CB == 2 * G::NT,
                "the read plan assumes 4 x 8, 4 x 4 or 2 x 2 sub-tiles and two copies per group");
  auto read_a = [&](int t) {
    const i16x4 lo = read_af_half<T, G>(rst, rks, wn, t, 0, lane);
    const i16x4 hi = read_af_half<T, G>(rst, rks, wn, t, 1, lane);
    nxt.a[t] = (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
#pragma unroll
  for (int t = 0; t < G::NT; ++t) {
    if (copy) {
      dma_copy<T, G>(2 * t, d, ab, bb, cst, wu);
      dma_copy<T, G>(2 * t + 1, d, ab, bb, cst, wu);
    }
#pragma unroll
    for (int s = 0; s < G::MT; ++s) acc[t][s] = mfma16x16x32(cur.a[t], cur.b[s], acc[t][s], T());
    // The reads after the MFMAs: nxt.a[t] may then take the registers of
    // cur.a[t], which the MFMAs above were its last use of.
    __builtin_amdgcn_sched_barrier(0);
    if (t == 0) {
      read_a(0);
#pragma unroll
      for (int i = 0; i < (G::MT < 4 ? G::MT : 4); ++i) nxt.b[i] = read_bf<T, G>(rst, rks, wm, i, lane);
    } else if (G::MT == 8) {
      if (t == 1) {
#pragma unroll
        for (int i = 4; i < G::MT; ++i) nxt.b[i] = read_bf<T, G>(rst, rks, wm, i, lane);
      } else if (t == 2) {
        read_a(1);
        read_a(2);
      } else {
        read_a(3);
      }
    } else {
      read_a(t);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <typename T, typename G>
__device__ __forceinline__ void read_all(Frags<G>& f, Stage<T> st, int ks, int wm, int wn, int lane) {
#pragma unroll
  for (int t = 0; t < G::NT; ++t) {
    const i16x4 lo = read_af_half<T, G>(st, ks, wn, t, 0, lane);
    const i16x4 hi = read_af_half<T, G>(st, ks, wn, t, 1, lane);
    f.a[t] = (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
#pragma unroll
  for (int s = 0; s < G::MT; ++s) f.b[s] = read_bf<T, G>(st, ks, wm, s, lane);
}

template <typename TO>
__device__ __forceinline__ void store4(TO* dst, f32x4 v, int valid) {
  if constexpr (sizeof(TO) == 2) {
    typedef TO to4 __attribute__((ext_vector_type(4)));
    const to4 o = (to4){(TO)v[0], (TO)v[1], (TO)v[2], (TO)v[3]};
    if (valid >= 4) {
      *(to4*)dst = o;
    } else {
      for (int r = 0; r < valid; ++r) dst[r] = o[r];
    }
  } else {
    if (valid >= 4) {
      *(f32x4*)dst = v;
    } else {
      for (int r = 0; r < valid; ++r) dst[r] = v[r];
    }
  }
}

// Epilogue through LDS for a wave's full WM x WN block of a 16-bit Y (the
// 256 x 256 and 128 x 128 tiles; the 64 x 64 tile stores from the
// accumulators).  The
// accumulator layout gives each lane 4 consecutive n of one row (8 bytes),
// 32 contiguous bytes per row per store instruction; instead the wave writes
// act(acc + bias), rounded, into its own LDS region (row-major, 16-byte
// chunks XOR-swizzled by row so that both the 8-byte writes and the 16-byte
// reads are free of bank conflicts) and reads it back row-contiguously:
// every store instruction then writes whole 128-byte lines of Y (8 rows of
// 128 bytes, or 4 of 256).  Only the wave's own region is touched, so no
// workgroup barrier is needed between the write and the read-back.
template <int ROWB>
__device__ __forceinline__ int stage_swz(int row) {
  if constexpr (ROWB == 128)
    return (row >> 1) & 7;
  else
    return row & 15;
}

template <typename T, typename TO, int ACT, bool HAS_BIAS, typename G>
__device__ __forceinline__ void epilogue_staged(const GemmParams& p, const f32x4 (&acc)[G::NT][G::MT], char* region,
                                                int wr0, int wc0, int lane) {
  constexpr int ROWB = G::WN * 2;      // bytes per staged row
  constexpr int CPR = ROWB / 16;       // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;        // rows per 1 KB read-back
  static_assert(ROWB == 128 || ROWB == 256, "staging swizzle assumes 128- or 256-byte rows");
  const int q = lane & 15, b = lane >> 4;
  const T* bias = (const T*)p.bias;
  typedef TO to4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int t = 0; t < G::NT; ++t) {
    f32x4 bv = (f32x4){0.f, 0.f, 0.f, 0.f};
    if constexpr (HAS_BIAS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[r] = to_f32(bias[wc0 + 16 * t + 4 * b + r]);
    }
    const int chunk = 2 * t + (b >> 1);
#pragma unroll
    for (int s = 0; s < G::MT; ++s) {
      const int row = 16 * s + q;
      to4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = from_f32<TO>(apply_act<ACT, sizeof(TO) == 2>(acc[t][s][r] + bv[r]));
      *(to4*)(region + row * ROWB + ((chunk ^ stage_swz<ROWB>(row)) << 4) + ((b & 1) << 3)) = o;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  TO* Y = (TO*)p.Y;
  const int rsub = lane / CPR, c = lane % CPR;
#pragma unroll
  for (int i = 0; i < G::WM / RPI; ++i) {
    const int row = RPI * i + rsub;
    const u32x4 v = *(const u32x4*)(region + row * ROWB + ((c ^ stage_swz<ROWB>(row)) << 4));
    *(u32x4*)(Y + (int64_t)(wr0 + row) * p.ldy + wc0 + 8 * c) = v;
  }
}

// Workgroup barrier for LDS reuse: the wave's own LDS accesses are complete
// (lgkmcnt 0) but its global stores and direct copies may still be in
// flight (no vmcnt wait, unlike __syncthreads' fence); the "memory" clobber
// keeps the compiler from moving memory accesses across it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
#pragma clang diagnostic pop

// Persistent kernel: the workgroups that fit on the CUs (one of 256 x 256,
// whose two LDS stages take 128 KB, two of 128 x 128, or four or five of
// 64 x 64) walk the tiles v = blockIdx.x, + gridDim.x, ...  Once a tile's Y stores
// are issued, the next tile's first two K steps are copied in without
// waiting for them, so the copies' latency and the stores' drain overlap.
// With gridDim.x a multiple of 8 a workgroup stays on one XCD, which is what
// tile_coords assumes.
template <typename T, typename TO, int ACT, bool HAS_BIAS, typename G>
__global__ __launch_bounds__(G::THREADS, G::MINW) void gemm16_kernel(GemmParams p) {
  constexpr int BM = G::BM, BN = G::BN, NW = G::NW;
  // The two stages of A (and of B) are adjacent (BM x 64 and 64 x BN
  // elements apart), so switching
  // stage is an immediate offset on every LDS read rather than new address
  // registers.
  __shared__ __attribute__((aligned(1024))) T sA[2][BM * BK];
  __shared__ __attribute__((aligned(1024))) T sB[2][BK * BN];
  const Stage<T> st0{sA[0], sB[0]}, st1{sA[1], sB[1]};

  const int total = p.tiles_m * p.tiles_n;
  int v = blockIdx.x;
  if (v >= total) return;
  const int lane0 = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int wm = w & 1, wn = w >> 1;
  const int kfull = p.K / BK;
  const int ktiles = (p.K + BK - 1) / BK;

  // Steps 0 and 1 of the tile at (m0, n0) into the two stages.
  auto prologue = [&](int m0, int n0, const DmaPlan& d, int lane) {
    if (ktiles > 0) {
      if (kfull > 0)
        dma_all<T, G>(p, d, m0, n0, 0, st0, wu);
      else
        tail_fill<T, G>(p, m0, n0, 0, st0, wu, lane);
    }
    if (ktiles > 1) {
      if (kfull > 1)
        dma_all<T, G>(p, d, m0, n0, BK, st1, wu);
      else
        tail_fill<T, G>(p, m0, n0, BK, st1, wu, lane);
    }
  };

  int tm, tn;
  tile_coords(v, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  int m0 = tm * BM, n0 = tn * BN;
  DmaPlan d = make_plan(p, m0, n0, wu, lane0);
  prologue(m0, n0, d, lane0);

  while (true) {
    // The lane index through an opaque copy: everything derived from it
    // (fragment and epilogue addresses) is recomputed per tile instead of
    // being hoisted out of the tile loop and held in registers across the
    // K loop, where there are none to spare.
    int lane = lane0;
    asm volatile("" : "+v"(lane));
    const int q = lane & 15, b = lane >> 4;
    f32x4 acc[G::NT][G::MT];
#pragma unroll
    for (int t = 0; t < G::NT; ++t)
#pragma unroll
      for (int s = 0; s < G::MT; ++s) acc[t][s] = (f32x4){0.f, 0.f, 0.f, 0.f};
    Frags<G> f0, f1;
    if (ktiles > 0) {
      wait_vmcnt0();
      __syncthreads();
      read_all<T, G>(f0, st0, 0, wm, wn, lane);
    }
    // Per K step k (stage cur; the other stage holds step k + 1 or is filling):
    //   slice 0: MFMAs on f0 while f1 (slice 1 of cur) is read;
    //   barrier: every wave has its fragments of cur, so cur is free, and the
    //            copies of step k + 1 have landed;
    //   slice 1: MFMAs on f1 while step k + 2 is copied into cur and f0
    //            (slice 0 of step k + 1) is read.
    for (int kt = 0; kt < ktiles; kt += 2) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int k = kt + half;
        if (k < ktiles) {
          const Stage<T> cur = half ? st1 : st0;
          const Stage<T> nxt = half ? st0 : st1;
          slice<T, G>(f0, acc, f1, cur, 1, wm, wn, lane, false, d, nullptr, nullptr, cur, wu);
          if (k + 1 < ktiles) {
            wait_vmcnt0();
            __syncthreads();
          }
          if (k + 2 < ktiles && k + 2 >= kfull) tail_fill<T, G>(p, m0, n0, (k + 2) * BK, cur, wu, lane);
          const bool copy = k + 2 < kfull;
          const void* ab = a_base<T>(p, m0, (k + 2) * BK);
          const void* bb = b_base<T>(p, n0, (k + 2) * BK);
          slice<T, G>(f1, acc, f0, nxt, 0, wm, wn, lane, copy, d, ab, bb, cur, wu);
        }
      }
    }

    // Epilogue: + bias, activation, one rounding, one store.  A wave whose
    // whole WM x WN block lies inside a 16-bit Y stages it in LDS (the
    // stages are free once every wave is past its last fragment read) and
    // stores it as full rows.
    const int wr0 = m0 + wm * G::WM, wc0 = n0 + wn * G::WN;
    constexpr bool STAGE = sizeof(TO) == 2 && G::WN >= 64;  // staging needs 128-byte rows
    const bool staged = STAGE && wr0 + G::WM <= p.M && wc0 + G::WN <= p.N;
    __syncthreads();
    if (staged) {
      if constexpr (STAGE) {
        // waves 0 .. NW/2 - 1 stage in the A stages, the others in the B
        // stages (NW/2 regions of WM x WN x 2 bytes in each)
        constexpr int RB = G::WM * G::WN * 2;
        static_assert((NW / 2) * RB <= (int)sizeof(sA), "staging regions exceed the stage buffers");
        char* region = wu < NW / 2 ? (char*)sA + wu * RB : (char*)sB + (wu - NW / 2) * RB;
        epilogue_staged<T, TO, ACT, HAS_BIAS, G>(p, acc, region, wr0, wc0, lane);
      }
    } else {
      // edge block (or 32-bit Y): element stores straight from the
      // accumulators
      const T* bias = (const T*)p.bias;
      TO* Y = (TO*)p.Y;
#pragma unroll
      for (int t = 0; t < G::NT; ++t) {
        const int n = n0 + wn * G::WN + 16 * t + 4 * b;
        if (n >= p.N) continue;
        const int valid = min(4, p.N - n);
        f32x4 bv = (f32x4){0.f, 0.f, 0.f, 0.f};
        if constexpr (HAS_BIAS) {
#pragma unroll
          for (int r = 0; r < 4; ++r) bv[r] = r < valid ? to_f32(bias[n + r]) : 0.f;
        }
#pragma unroll
        for (int s = 0; s < G::MT; ++s) {
          const int m = m0 + wm * G::WM + 16 * s + q;
          if (m < p.M) {
            f32x4 o = acc[t][s];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = apply_act<ACT, sizeof(TO) == 2>(o[r] + bv[r]);
            store4<TO>(Y + (int64_t)m * p.ldy + n, o, valid);
          }
        }
      }
    }
    // Every wave is done with the LDS (its stores may still be in flight):
    // copy the next tile's first two K steps in while they drain.
    lds_barrier();
    const int vn = v + (int)gridDim.x;
    if (vn < total) {
      tile_coords(vn, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
      m0 = tm * BM;
      n0 = tn * BN;
      d = make_plan(p, m0, n0, wu, lane);
      prologue(m0, n0, d, lane);
    }
    if (vn >= total) break;
    v = vn;
  }
}

// Grid: min(#tiles, #CUs x workgroups per CU), the per-CU count from the
// runtime for the compiled kernel, cached per instantiation (or the caller's
// grid_override, an autotuning knob).
template <typename T, typename TO, int ACT, bool HAS_BIAS, typename G>
hipError_t launch_cfg(GemmParams p, hipStream_t stream, int num_cus) {
  p.tiles_m = (p.M + G::BM - 1) / G::BM;
  p.tiles_n = (p.N + G::BN - 1) / G::BN;
  // (atomic: concurrent first calls from several host threads store the
  // same value)
  static std::atomic<int> per_cu_cache{0};
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int n = 0;
    hipError_t e =
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm16_kernel<T, TO, ACT, HAS_BIAS, G>, G::THREADS, 0);
    if (e != hipSuccess) return e;
    per_cu = n > 0 ? n : 1;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  const long total = (long)p.tiles_m * p.tiles_n;
  const long cap = p.grid_override > 0 ? (long)p.grid_override : (long)num_cus * per_cu;
  const int grid = (int)(total < cap ? total : cap);
  hipLaunchKernelGGL((gemm16_kernel<T, TO, ACT, HAS_BIAS, G>), dim3(grid), dim3(G::THREADS), 0, stream, p);
  return hipGetLastError();
}

template <typename T, typename TO, int ACT, typename G>
hipError_t launch_bias(const GemmParams& p, hipStream_t stream, int num_cus) {
  if (p.bias) return launch_cfg<T, TO, ACT, true, G>(p, stream, num_cus);
  return launch_cfg<T, TO, ACT, false, G>(p, stream, num_cus);
}

// p.variant is resolved by launch_gemm16: 1 = 256 x 256, 2 = 128 x 128, 3 = 64 x 64.
template <typename T, typename TO, int ACT>
hipError_t launch_typed(const GemmParams& p, hipStream_t stream, int num_cus) {
  if (p.variant == 3) return launch_bias<T, TO, ACT, Geo64>(p, stream, num_cus);
  if (p.variant == 2) return launch_bias<T, TO, ACT, Geo128>(p, stream, num_cus);
  return launch_bias<T, TO, ACT, Geo256>(p, stream, num_cus);
}

template <typename T, typename TO>
hipError_t launch_act(const GemmParams& p, int act, hipStream_t stream, int num_cus) {
  switch (act) {
    case ACT_GELU: return launch_typed<T, TO, ACT_GELU>(p, stream, num_cus);
    case ACT_SOFTPLUS: return launch_typed<T, TO, ACT_SOFTPLUS>(p, stream, num_cus);
    case ACT_RELU: return launch_typed<T, TO, ACT_RELU>(p, stream, num_cus);
    default: return launch_typed<T, TO, ACT_NONE>(p, stream, num_cus);
  }
}

}  // namespace

hipError_t launch_gemm16(GemmParams p, DType in, DType out, int act, hipStream_t stream, int num_cus) {
  // 64 x 64 tiles while 128 x 128 ones number fewer than the CUs; 128 x 128
  // while all of them run at once (at most two workgroups per CU); else
  // 256 x 256.  Measured, bf16 + bias + GELU, the outputs the same bits
  // throughout: 128 x 128 is 1.3-2.2x faster than 256 x 256 on problems
  // whose 128 x 128 tiles fit in one round (1024^3, 2048^2 x 8192, 4096 x
  // 2048 x 4096, 16384 x 512 x 2048) and 0.82-0.86x on those that need more
  // (3072^2 x 4096: 144 tiles of 256 x 256 but 576 of 128 x 128; 4096^2 x
  // 4096); 64 x 64 is 1.2-1.7x faster than 128 x 128 below one 128 x 128
  // tile per CU (512^3, 1024^3, 1024 x 2048 x 2048, 4096 x 512 x 1024) and
  // level with it at exactly one per CU (2048^3: 611 against 591 TFLOP/s,
  // within the run-to-run spread), where the threshold keeps 128 x 128.  Variant 1 / 2 / 3 forces 256 x 256 / 128 x 128 /
  // 64 x 64: an autotuning knob.
  if (p.variant == 0) {
    const long tiles128 = (long)((p.M + 127) / 128) * ((p.N + 127) / 128);
    p.variant = tiles128 < num_cus ? 3 : tiles128 <= 2L * num_cus ? 2 : 1;
  }
  if (p.group_m <= 0) p.group_m = 8;
  if (in == DT_BF16) {
    if (out == DT_F32) return launch_act<__bf16, float>(p, act, stream, num_cus);
    return launch_act<__bf16, __bf16>(p, act, stream, num_cus);
  }
  if (out == DT_F32) return launch_act<_Float16, float>(p, act, stream, num_cus);
  return launch_act<_Float16, _Float16>(p, act, stream, num_cus);
}

}  // namespace coalesce
