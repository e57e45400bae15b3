// Fused GEMM + bias + activation for fp32 inputs on the gfx950 fp32 MFMA.
//
// Same method as the 16-bit kernel (bias and activation applied to the fp32
// accumulators in registers, one store of Y), on v_mfma_f32_16x16x4_f32:
//   * workgroup tile BM x BN (128 x 128; 64 x 64, 64 x 32 or 32 x 32 when the
//     problem has too few larger tiles to occupy the GPU), K step 32, 4 waves
//     in a 2 x 2 grid; each wave computes Y^T blocks (A operand = B^T,
//     B operand = A^T) so each lane holds 4 consecutive n of one row m;
//   * per 16-deep k group a wave reads its A^T operand as one 128-bit LDS read
//     per 16 rows (4 consecutive k, one per MFMA) and its B^T operand as 32-bit
//     reads; fp32 MFMA takes one k per lane, so no transpose is needed;
//   * 2 LDS stages filled by 16-byte direct-to-LDS copies one K step ahead;
//     2 workgroups per CU (64 KB of LDS each at 128 x 128);
//   * the smaller tiles split K inside the workgroup: KG groups of 4 waves
//     (2 at 64 x 64 and 64 x 32, 4 at 32 x 32) each take a contiguous run of
//     K steps with LDS stages of their own, and the groups' accumulators are
//     added through LDS in a fixed order (group 0 + 1 + ...) before the
//     epilogue.  A small problem has one such tile per CU or fewer, whose
//     K loop is a chain of dependent steps (copy, barrier, 8 MFMAs on one
//     accumulator); the groups run their chains side by side.
// The fp32 MFMA accumulates in fp32 with the hardware's own summation order,
// which is the same for the fused kernel and for the same kernel run with
// act = NONE and no bias (the unfused baseline's GEMM step), so the fused and
// unfused results agree bit for bit.  Tile shapes with the same number of K
// groups accumulate in the same order (the autotuner only exchanges those).
#include "common.hpp"
#include "launch.hpp"

namespace coalesce {
namespace {

constexpr int BK = 32;


__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// A tile: BM rows of 32 floats (8 chunks of 4); chunk c of row m at slot
// c ^ swzA(m): a 128-bit read by 16 lanes (16 rows, one chunk) hits 16
// distinct 16-byte slots of a 256-byte window (8 of a 128-byte one).
// B tile: 32 rows of BN floats (BN / 4 chunks); chunk c of row k at slot
// c ^ 4 ((k >> 2) & 3): the 32-bit reads of one MFMA (rows k, k+4, k+8, k+12,
// 16 consecutive n each) land in 4 disjoint 64-byte segments.  With 32-float
// rows (BN = 32) only two 64-byte segments fit in a row, so c ^ 4 ((k >> 2) &
// 1) and the rows k and k+8 share banks (a 2-way conflict the small
// problems that use this tile can afford).
__device__ __forceinline__ int swzA(int m) { return ((m >> 1) & 7) ^ ((m & 1) << 2); }
template <int BN>
__device__ __forceinline__ int swzB(int k) {
  if constexpr (BN >= 64)
    return ((k >> 2) & 3) << 2;
  else
    return ((k >> 2) & 1) << 2;
}

template <int BM, int BN, int KG_>
struct Cfg {
  static constexpr int KG = KG_;  // K groups of 4 waves
  static constexpr int NS = 2;    // LDS stages per K group (copies one K step ahead)
  static constexpr int THREADS = 256 * KG;
  static constexpr int STAGE = BM * BK + BK * BN;  // floats of one LDS stage (A then B)
  static constexpr int A_BLOCKS = BM * BK * 4 / 1024;  // 1 KB copies per stage for A
  static constexpr int B_BLOCKS = BK * BN * 4 / 1024;
  static constexpr int B_ROWS_PER_BLOCK = 1024 / (BN * 4);
  static constexpr int B_CHUNKS = BN / 4;
  static constexpr int WM = BM / 2, WN = BN / 2;  // wave tile
  static constexpr int MT = WM / 16, NT = WN / 16;
};

template <int BM, int BN>
__device__ __forceinline__ void fill_dma(const GemmParams& p, int m0, int n0, int k0, int nlast, float* sa, float* sb,
                                         int wu, int lane) {
  typedef Cfg<BM, BN, 1> C;
  const float* A = (const float*)p.A;
  const float* B = (const float*)p.B;
#pragma unroll
  for (int j = 0; j < C::A_BLOCKS / 4; ++j) {
    const int blk = wu * (C::A_BLOCKS / 4) + j;
    const int row = blk * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swzA(row);
    const int gm = min(m0 + row, p.M - 1);
    dma16(A + (int64_t)gm * p.lda + k0 + c * 4, lds_addr(sa) + blk * 1024);
  }
#pragma unroll
  for (int j = 0; j < C::B_BLOCKS / 4; ++j) {
    const int blk = wu * (C::B_BLOCKS / 4) + j;
    const int row = blk * C::B_ROWS_PER_BLOCK + lane / C::B_CHUNKS;
    const int c = (lane % C::B_CHUNKS) ^ swzB<BN>(row);
    const int gn = min(n0 + c * 4, nlast);
    dma16(B + (int64_t)(k0 + row) * p.ldb + gn, lds_addr(sb) + blk * 1024);
  }
}

template <int BM, int BN>
__device__ __forceinline__ void fill_tail(const GemmParams& p, int m0, int n0, int k0, int nlast, float* sa, float* sb,
                                          int w, int lane) {
  typedef Cfg<BM, BN, 1> C;
  const float* A = (const float*)p.A;
  const float* B = (const float*)p.B;
  f32x4 ra[C::A_BLOCKS / 4], rb[C::B_BLOCKS / 4];
#pragma unroll
  for (int j = 0; j < C::A_BLOCKS / 4; ++j) {
    const int blk = w * (C::A_BLOCKS / 4) + j;
    const int row = blk * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swzA(row);
    const int gm = min(m0 + row, p.M - 1);
    const int k = k0 + c * 4;
    f32x4 v = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (k < p.K) {
      v = *(const f32x4*)(A + (int64_t)gm * p.lda + k);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (k + e >= p.K) v[e] = 0.f;
    }
    ra[j] = v;
  }
#pragma unroll
  for (int j = 0; j < C::B_BLOCKS / 4; ++j) {
    const int blk = w * (C::B_BLOCKS / 4) + j;
    const int row = blk * C::B_ROWS_PER_BLOCK + lane / C::B_CHUNKS;
    const int c = (lane % C::B_CHUNKS) ^ swzB<BN>(row);
    const int gn = min(n0 + c * 4, nlast);
    f32x4 v = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (k0 + row < p.K) v = *(const f32x4*)(B + (int64_t)(k0 + row) * p.ldb + gn);
    rb[j] = v;
  }
#pragma unroll
  for (int j = 0; j < C::A_BLOCKS / 4; ++j) *(f32x4*)(sa + (w * (C::A_BLOCKS / 4) + j) * 256 + lane * 4) = ra[j];
#pragma unroll
  for (int j = 0; j < C::B_BLOCKS / 4; ++j) *(f32x4*)(sb + (w * (C::B_BLOCKS / 4) + j) * 256 + lane * 4) = rb[j];
}

template <int BM, int BN>
__device__ __forceinline__ void compute_stage(const float* sa, const float* sb,
                                              f32x4 (&acc)[Cfg<BM, BN, 1>::NT][Cfg<BM, BN, 1>::MT], int wm, int wn,
                                              int lane) {
  typedef Cfg<BM, BN, 1> C;
  const int q = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kg = 0; kg < BK / 16; ++kg) {
    f32x4 a4[C::MT];
#pragma unroll
    for (int s = 0; s < C::MT; ++s) {
      const int m = wm * C::WM + 16 * s + q;
      const int c = (4 * kg + g) ^ swzA(m);
      a4[s] = *(const f32x4*)(sa + m * BK + c * 4);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 16 * kg + 4 * g + e;
      float bt[C::NT];
#pragma unroll
      for (int t = 0; t < C::NT; ++t) {
        const int n = wn * C::WN + 16 * t + q;
        bt[t] = sb[k * BN + ((((n >> 2) ^ swzB<BN>(k))) << 2) + (n & 3)];
      }
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int s = 0; s < C::MT; ++s) acc[t][s] = mfma16x16x4(bt[t], a4[s][e], acc[t][s]);
    }
  }
}

// Wait for every copy this wave has in flight (the builtin, not inline asm,
// so that the compiler's own counter bookkeeping sees it).  Encoding: vmcnt
// 0, expcnt 7 and lgkmcnt 15 (those two untouched).
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier of the K loop: the wave's own LDS accesses complete
// (lgkmcnt 0), then s_barrier; the loop writes no global memory, so it needs
// none of __syncthreads' fences.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
#pragma clang diagnostic pop

template <int BM, int BN, int KG_, int ACT, bool HAS_BIAS>
__global__ __launch_bounds__((Cfg<BM, BN, KG_>::THREADS), 2) void gemm32_kernel(GemmParams p) {
  typedef Cfg<BM, BN, KG_> C;
  constexpr int KG = C::KG;
  constexpr int NS = C::NS;
  // per K group NS stages of A (BM x BK) and B (BK x BN)
  __shared__ __attribute__((aligned(1024))) float lds[KG * NS * C::STAGE];

  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // K group (a compile-time 0 for the one-group tile: with a run-time 0 the
  // 128 x 128 kernel fetched ~50 % more from HBM at 4096^3 and ran 2.5 %
  // slower)
  const int kg = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane(w >> 2);
  const int wl = w & 3;                                   // wave within the group
  const int wu = __builtin_amdgcn_readfirstlane(wl);
  const int wm = wl & 1, wn = wl >> 1;
  const int nlast = ((p.N - 1) >> 2) << 2;
  float* const stages = lds + (NS * kg) * C::STAGE;  // stage i: A at i STAGE, B after it

  f32x4 acc[C::NT][C::MT];
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int s = 0; s < C::MT; ++s) acc[t][s] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int kfull = p.K / BK;
  const int ktiles = (p.K + BK - 1) / BK;
  // the group's K steps [kbeg, kend); every group passes the same `per`
  // barriers
  const int per = (ktiles + KG - 1) / KG;
  const int kbeg = kg * per;
  const int kend = min(ktiles, kbeg + per);
  auto fill = [&](int i, int k) {  // K step k into stage i
    float* sa = stages + i * C::STAGE;
    if (k < kfull)
      fill_dma<BM, BN>(p, m0, n0, k * BK, nlast, sa, sa + BM * BK, wu, lane);
    else
      fill_tail<BM, BN>(p, m0, n0, k * BK, nlast, sa, sa + BM * BK, wu, lane);
  };
#pragma unroll
  for (int i = 0; i + 1 < NS; ++i)
    if (kbeg + i < kend) fill(i, kbeg + i);
  // Step j: wait for this wave's copies, barrier (every wave's copies of step
  // j have landed, and every wave is done with step j - 1, whose stage is
  // refilled next), copy step j + 1, compute step j.  (Written this way, with
  // the stage an immediate of the unrolled loop and the wait visible to the
  // compiler, the 128 x 128 tile runs 4096^3 in 1024 instead of 1058 us, the
  // other tiles unchanged.)
  for (int j0 = 0; j0 < per; j0 += NS) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int j = j0 + i;
      if (j < per) {
        const int k = kbeg + j;
        wait_copies();
        lds_barrier();
        if (k + NS - 1 < kend) fill((i + NS - 1) % NS, k + NS - 1);
        if (k < kend) {
          const float* sa = stages + i * C::STAGE;
          compute_stage<BM, BN>(sa, sa + BM * BK, acc, wm, wn, lane);
        }
      }
    }
  }

  if constexpr (KG > 1) {
    // groups 1 .. KG-1 hand their sums to group 0 through the (now free)
    // stages; group 0 adds them in group order
    f32x4* red = (f32x4*)lds;
    __syncthreads();
    if (kg > 0) {
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int s = 0; s < C::MT; ++s)
          red[((((kg - 1) * 4 + wl) * C::NT + t) * C::MT + s) * 64 + lane] = acc[t][s];
    }
    __syncthreads();
    if (kg > 0) return;
    for (int g2 = 1; g2 < KG; ++g2)
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int s = 0; s < C::MT; ++s) acc[t][s] += red[((((g2 - 1) * 4 + wl) * C::NT + t) * C::MT + s) * 64 + lane];
  }

  const int q = lane & 15, g = lane >> 4;
  const float* bias = (const float*)p.bias;
  float* Y = (float*)p.Y;
#pragma unroll
  for (int t = 0; t < C::NT; ++t) {
    const int n = n0 + wn * C::WN + 16 * t + 4 * g;
    if (n >= p.N) continue;
    const int valid = min(4, p.N - n);
    f32x4 bv = (f32x4){0.f, 0.f, 0.f, 0.f};
    if constexpr (HAS_BIAS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[r] = r < valid ? bias[n + r] : 0.f;
    }
#pragma unroll
    for (int s = 0; s < C::MT; ++s) {
      const int m = m0 + wm * C::WM + 16 * s + q;
      if (m < p.M) {
        f32x4 v = acc[t][s];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = apply_act<ACT>(v[r] + bv[r]);
        float* dst = Y + (int64_t)m * p.ldy + n;
        if (valid == 4) {
          *(f32x4*)dst = v;
        } else {
          for (int r = 0; r < valid; ++r) dst[r] = v[r];
        }
      }
    }
  }
}

template <int BM, int BN, int KG, int ACT>
hipError_t launch_cfg(GemmParams p, hipStream_t stream) {
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  if (p.group_m <= 0) p.group_m = 8;
  dim3 grid(p.tiles_m * p.tiles_n), block(Cfg<BM, BN, KG>::THREADS);
  if (p.bias)
    hipLaunchKernelGGL((gemm32_kernel<BM, BN, KG, ACT, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((gemm32_kernel<BM, BN, KG, ACT, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int BM, int BN, int KG>
hipError_t launch_act(GemmParams p, int act, hipStream_t stream) {
  switch (act) {
    case ACT_GELU: return launch_cfg<BM, BN, KG, ACT_GELU>(p, stream);
    case ACT_SOFTPLUS: return launch_cfg<BM, BN, KG, ACT_SOFTPLUS>(p, stream);
    case ACT_RELU: return launch_cfg<BM, BN, KG, ACT_RELU>(p, stream);
    default: return launch_cfg<BM, BN, KG, ACT_NONE>(p, stream);
  }
}

}  // namespace

int gemm32_variant(int64_t M, int64_t N, int num_cus) {
  // 128 x 128 tiles when they give at least one workgroup per CU; below,
  // 32 x 32 (four K groups) while 64 x 32 tiles would leave CUs idle, else
  // the two-group tiles: 64 x 64 while they number at most one per CU,
  // 64 x 32 beyond.  Measured with the K groups (the per-shape tuner, which
  // exchanges only same-group tiles): 64 x 64 faster on 768^3 (7 %), 1024^3
  // (7 %), 1024^2 x 4096 (9 %); 64 x 32 faster on 1536^2 x 1024 (13 %) and
  // 1280 x 1024^2 (2 %); 512^3 best on 32 x 32.
  //
  // Past one round of 128 x 128 tiles (two workgroups per CU) the last round
  // may be mostly empty; 64 x 64 tiles (two K groups, also two workgroups per
  // CU, a quarter of the work each) then sometimes finish sooner.  Cost model,
  // fitted to back-to-back times of both shapes on seven problems from 2560^3
  // to 6144^2 x 1024: a full round of 128 x 128 tiles takes ~0.125 us per
  // element of K (0.51 ms at K = 4096), one of 64 x 64 tiles ~0.037 (18 % more
  // per flop); a last round of at most one workgroup per CU costs ~0.55 of a
  // full one (each workgroup has its CU to itself).  Measured: 3072^3 590 ->
  // 511 us, 3584^3 908 -> 851 us, 3200^2 x 4096 784 -> 753 us; 4096^3,
  // 4608^3, 5120^3, 3328^3, 3456^2 x 2048, 3072 x 4096 x 2048 and 6144^2 x
  // 1024 stay on 128 x 128, 1-14 % faster there (the last four checked
  // after the fit, as predicted).
  const long tiles128 = (long)((M + 127) / 128) * ((N + 127) / 128);
  const long tiles64 = (long)((M + 63) / 64) * ((N + 63) / 64);
  const long tiles6432 = (long)((M + 63) / 64) * ((N + 31) / 32);
  const long slots = 2L * num_cus;
  if (tiles128 > slots) {
    auto rounds = [&](long n) {  // in hundredths of a full round
      const long rest = n % slots;
      return 100 * (n / slots) + (rest == 0 ? 0 : rest <= num_cus ? 55 : 100);
    };
    return 37 * rounds(tiles64) < 125 * rounds(tiles128) ? 2 : 1;
  }
  if (tiles128 >= num_cus) return 1;
  if (tiles6432 < num_cus) return 3;
  return tiles64 > num_cus ? 4 : 2;
}

int gemm32_kgroups(int variant) { return variant == 1 ? 1 : variant == 3 ? 4 : 2; }

hipError_t launch_gemm32(GemmParams p, int act, hipStream_t stream, int num_cus) {
  // Variant 1 / 2 / 3 / 4 forces 128 x 128 / 64 x 64 / 32 x 32 / 64 x 32: an
  // autotuning knob; 0 takes gemm32_variant's choice.
  int v = p.variant;
  if (v == 0) v = gemm32_variant(p.M, p.N, num_cus);
  if (v == 1) return launch_act<128, 128, 1>(p, act, stream);
  if (v == 2) return launch_act<64, 64, 2>(p, act, stream);
  if (v == 4) return launch_act<64, 32, 2>(p, act, stream);
  return launch_act<32, 32, 4>(p, act, stream);
}

}  // namespace coalesce
