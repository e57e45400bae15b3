// Fused GEMM + bias + activation for bf16 / fp16 inputs on gfx950 MFMA.
//
// Y = act(A . B + bias) ("Coalesce" README, "Fusion study"): the bias add and
// the activation run on the fp32 accumulators in registers and Y is written
// once.  Tile plan (hand-budgeted against the 512 VGPRs a lane has when one
// wave runs per SIMD):
//   * workgroup tile 256 (m) x 256 (n), K step 64, 4 waves in a 2 x 2 grid,
//     each wave owning a 128 x 128 block of Y;
//   * the wave computes Y^T blocks with v_mfma_f32_16x16x32 -- A operand =
//     B^T (rows n), B operand = A^T (columns m) -- so every lane ends up with
//     4 consecutive n of one row m, which makes bias loads and Y stores
//     contiguous;
//   * accumulators: 8 x 8 sub-tiles x 4 fp32 = 256 registers; operand
//     fragments for one 32-deep k slice: 8 + 8 x 4 = 64 registers;
//   * global -> LDS copies are 16-byte direct-to-LDS loads (no VGPR staging),
//     double-buffered (2 x 64 KB of the 160 KB LDS), issued one K step ahead;
//   * B is K x N with n contiguous, so its MFMA fragments (8 consecutive k of
//     one n) come from the transposing LDS read ds_read_b64_tr_b16;
//   * LDS rows are XOR-swizzled in 16-byte chunks so that the fragment reads
//     spread over the banks.
// The last, partial K step (K not a multiple of 64) goes through masked
// register loads that zero every element past K.  Rows past M read a
// clamped (valid) row and are never stored; columns past N are masked.
#include "common.hpp"
#include "launch.hpp"

namespace coalesce {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, THREADS = 256;

// A tile: 256 rows of 64 k (128 B = 8 chunks); chunk c of row m at slot c ^ (m & 7).
// B tile: 64 rows of 256 n (512 B = 32 chunks); chunk c of row k at slot c ^ 2 (k & 3).
__device__ __forceinline__ int swzA(int m) { return m & 7; }
__device__ __forceinline__ int swzB(int k) { return (k & 3) << 1; }

template <typename T>
struct Stage {
  T* a;
  T* b;
};

// Direct-to-LDS copy of the full K step starting at k0.  Wave w fills A rows
// [64 w, 64 w + 64) (8 copies of 8 rows) and B rows [16 w, 16 w + 16) (8
// copies of 2 rows); each copy is one 1 KB LDS block, lane l's 16 bytes going
// to slot l of the block.
template <typename T>
__device__ __forceinline__ void issue_dma(const GemmParams& p, int m0, int n0, int k0, int nlast, Stage<T> st,
                                          int w_uniform, int lane) {
  const T* A = (const T*)p.A;
  const T* B = (const T*)p.B;
  const int rsub = lane >> 3;
  const int cA = (lane & 7) ^ swzA(rsub);
  const uint32_t a_base = lds_addr(st.a) + (uint32_t)w_uniform * (64 * BK * (int)sizeof(T));
  const uint32_t b_base = lds_addr(st.b) + (uint32_t)w_uniform * (16 * BN * (int)sizeof(T));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int row = w_uniform * 64 + j * 8 + rsub;
    int gm = min(m0 + row, p.M - 1);
    dma16(A + (int64_t)gm * p.lda + k0 + cA * 8, a_base + j * (8 * BK * (int)sizeof(T)));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int row = w_uniform * 16 + j * 2 + (lane >> 5);
    int cB = (lane & 31) ^ swzB(row);
    int gn = min(n0 + cB * 8, nlast);
    dma16(B + (int64_t)(k0 + row) * p.ldb + gn, b_base + j * (2 * BN * (int)sizeof(T)));
  }
}

// Partial last K step: masked loads (elements at k >= K become 0), written to
// the same LDS slots the direct copies would use.
template <typename T>
__device__ __forceinline__ void tail_fill(const GemmParams& p, int m0, int n0, int k0, int nlast, Stage<T> st, int w,
                                          int lane) {
  const T* A = (const T*)p.A;
  const T* B = (const T*)p.B;
  const int rsub = lane >> 3;
  const int cA = (lane & 7) ^ swzA(rsub);
  const int kA = k0 + cA * 8;
  i16x8 ra[8], rb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int row = w * 64 + j * 8 + rsub;
    int gm = min(m0 + row, p.M - 1);
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
  for (int j = 0; j < 8; ++j) {
    int row = w * 16 + j * 2 + (lane >> 5);
    int cB = (lane & 31) ^ swzB(row);
    int gn = min(n0 + cB * 8, nlast);
    i16x8 v = (i16x8){0, 0, 0, 0, 0, 0, 0, 0};
    if (k0 + row < p.K) v = *(const i16x8*)(B + (int64_t)(k0 + row) * p.ldb + gn);
    rb[j] = v;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) *(i16x8*)(st.a + (w * 64 + j * 8) * BK + lane * 8) = ra[j];
#pragma unroll
  for (int j = 0; j < 8; ++j) *(i16x8*)(st.b + (w * 16 + j * 2) * BN + lane * 8) = rb[j];
}

template <typename T>
__device__ __forceinline__ void fill_stage(const GemmParams& p, int kt, int kfull, int m0, int n0, int nlast,
                                           Stage<T> st, int w_uniform, int lane) {
  if (kt < kfull)
    issue_dma<T>(p, m0, n0, kt * BK, nlast, st, w_uniform, lane);
  else
    tail_fill<T>(p, m0, n0, kt * BK, nlast, st, w_uniform, lane);
}

// Operand fragments of one 32-deep k slice (ks = 0 or 1 of the stage).
//   bf[s]: B operand = A^T, rows m = 128 wm + 16 s + (lane & 15), k = 8 (lane >> 4) + e
//   af[t]: A operand = B^T, rows n = 128 wn + 16 t + (lane & 15), same k, via two
//          transposing reads of 4 k each.
template <typename T>
__device__ __forceinline__ void read_frags(Stage<T> st, int ks, int wm, int wn, int lane, i16x8 (&af)[8],
                                           i16x8 (&bf)[8]) {
  const int q = lane & 15, b = lane >> 4;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    int m = wm * 128 + 16 * s + q;
    int c = (4 * ks + b) ^ swzA(m);
    bf[s] = *(const i16x8*)(st.a + m * BK + c * 8);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    int n = wn * 128 + 16 * t + 4 * (q & 3);
    int k = 32 * ks + 8 * b + (q >> 2);
    i16x4 lo = lds_read_tr16(st.b + k * BN + (((n >> 3) ^ swzB(k)) << 3) + (n & 7));
    i16x4 hi = lds_read_tr16(st.b + (k + 4) * BN + (((n >> 3) ^ swzB(k + 4)) << 3) + (n & 7));
    af[t] = (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

template <typename T>
__device__ __forceinline__ void mfma_slice(const i16x8 (&af)[8], const i16x8 (&bf)[8], f32x4 (&acc)[8][8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[t][s] = mfma16x16x32(af[t], bf[s], acc[t][s], T());
}

// Interleave the 24 LDS reads of the next slice with the 64 MFMAs of this one.
__device__ __forceinline__ void interleave_reads_with_mfma() {
#pragma unroll
  for (int i = 0; i < 24; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
}

template <typename T, typename TO>
__device__ __forceinline__ void store4(TO* dst, f32x4 v, int valid) {
  if constexpr (sizeof(TO) == 2) {
    typedef TO to4 __attribute__((ext_vector_type(4)));
    to4 o = (to4){(TO)v[0], (TO)v[1], (TO)v[2], (TO)v[3]};
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

template <typename T, typename TO, int ACT, bool HAS_BIAS>
__global__ __launch_bounds__(THREADS, 1) void gemm16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) T sA0[BM * BK];
  __shared__ __attribute__((aligned(1024))) T sB0[BK * BN];
  __shared__ __attribute__((aligned(1024))) T sA1[BM * BK];
  __shared__ __attribute__((aligned(1024))) T sB1[BK * BN];
  const Stage<T> st0{sA0, sB0}, st1{sA1, sB1};

  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int nlast = ((p.N - 1) >> 3) << 3;
  f32x4 acc[8][8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[t][s] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Main loop.  Per K step (one LDS stage, two 32-deep slices):
  //   slice 0 MFMAs run while slice 1 fragments are read;
  //   then the barrier that frees the stage (all waves hold their fragments)
  //   and publishes the other stage (its copies waited for);
  //   the copy of K step kt + 2 is issued into the freed stage;
  //   slice 1 MFMAs run while slice 0 fragments of the next stage are read.
  const int kfull = p.K / BK;
  const int ktiles = (p.K + BK - 1) / BK;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  i16x8 fa0[8], fb0[8], fa1[8], fb1[8];
  if (ktiles > 0) {
    fill_stage<T>(p, 0, kfull, m0, n0, nlast, st0, wu, lane);
    wait_vmcnt0();
    __syncthreads();
    if (ktiles > 1) fill_stage<T>(p, 1, kfull, m0, n0, nlast, st1, wu, lane);
    read_frags<T>(st0, 0, wm, wn, lane, fa0, fb0);
  }
  for (int kt = 0; kt < ktiles; kt += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k = kt + half;
      if (k < ktiles) {
        const Stage<T> cur = half ? st1 : st0;
        const Stage<T> nxt = half ? st0 : st1;
        read_frags<T>(cur, 1, wm, wn, lane, fa1, fb1);
        mfma_slice<T>(fa0, fb0, acc);
        interleave_reads_with_mfma();
        if (k + 1 < ktiles) {
          wait_vmcnt0();
          __syncthreads();
          if (k + 2 < ktiles) fill_stage<T>(p, k + 2, kfull, m0, n0, nlast, cur, wu, lane);
          read_frags<T>(nxt, 0, wm, wn, lane, fa0, fb0);
        }
        mfma_slice<T>(fa1, fb1, acc);
        interleave_reads_with_mfma();
      }
    }
  }

  // Epilogue: + bias, activation, one rounding, one store.
  const int q = lane & 15, b = lane >> 4;
  const T* bias = (const T*)p.bias;
  TO* Y = (TO*)p.Y;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int n = n0 + wn * 128 + 16 * t + 4 * b;
    if (n >= p.N) continue;
    const int valid = min(4, p.N - n);
    f32x4 bv = (f32x4){0.f, 0.f, 0.f, 0.f};
    if constexpr (HAS_BIAS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[r] = r < valid ? to_f32(bias[n + r]) : 0.f;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int m = m0 + wm * 128 + 16 * s + q;
      if (m < p.M) {
        f32x4 v = acc[t][s];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = apply_act<ACT>(v[r] + bv[r]);
        store4<T, TO>(Y + (int64_t)m * p.ldy + n, v, valid);
      }
    }
  }
}

template <typename T, typename TO, int ACT>
hipError_t launch_typed(GemmParams p, hipStream_t stream) {
  dim3 grid(p.tiles_m * p.tiles_n), block(THREADS);
  if (p.bias)
    hipLaunchKernelGGL((gemm16_kernel<T, TO, ACT, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((gemm16_kernel<T, TO, ACT, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <typename T, typename TO>
hipError_t launch_act(GemmParams p, int act, hipStream_t stream) {
  switch (act) {
    case ACT_GELU: return launch_typed<T, TO, ACT_GELU>(p, stream);
    case ACT_SOFTPLUS: return launch_typed<T, TO, ACT_SOFTPLUS>(p, stream);
    default: return launch_typed<T, TO, ACT_NONE>(p, stream);
  }
}

}  // namespace

hipError_t launch_gemm16(GemmParams p, DType in, DType out, int act, hipStream_t stream) {
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  p.group_m = 8;
  if (in == DT_BF16) {
    if (out == DT_F32) return launch_act<__bf16, float>(p, act, stream);
    return launch_act<__bf16, __bf16>(p, act, stream);
  }
  if (out == DT_F32) return launch_act<_Float16, float>(p, act, stream);
  return launch_act<_Float16, _Float16>(p, act, stream);
}

}  // namespace coalesce
