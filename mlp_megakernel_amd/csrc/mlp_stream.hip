// Layer-streaming MLP megakernel: the chain of "MLP Megakernel" README's
// "Architecture" (h_0 = x, h_l = act(h_{l-1} W_l), out = h_{L-1} W_L, fp16
// operands, fp32 accumulation) for chains whose weights do not all fit in LDS
// at once -- deeper chains, widths up to 256 -- and for non-square chains,
// whose layers it computes at their own widths (README: generalising the
// megakernel to N layers and to D != H != out).
//
// The resident kernel (mlp_kernel.hpp) keeps every W_l in LDS for the whole launch
// and lets each wave run its row tiles through the chain on its own.  Here
// the weights pass through LDS one chunk at a time instead:
//   * a chunk is the slice of one layer's W_l that produces up to 128 output
//     units: all of its input rows k (up to 256), 128 columns n; the chunks of
//     the chain (layer 0 chunk 0, ..., layer L-1 last chunk) are copied in
//     order into two LDS slots by direct buffer-to-LDS copies, the next chunk
//     while the current one is used, so the copies overlap the MFMAs;
//   * a workgroup of W waves works on up to W row tiles of 32 rows at a time
//     (one per wave; in round r workgroup b takes tiles r G W + b + w G, so a
//     small batch spreads over the workgroups) and takes them through the
//     chain in lockstep: a barrier per chunk publishes the slot its copies
//     filled; the activations stay in registers between layers, as in the
//     resident kernel; the next round's x is loaded during the current one;
//     a wave without a tile copies its share of the chunks but skips their
//     arithmetic;
//   * W_l stays in its natural layout (rows k, n contiguous).  The MFMA's A
//     operand is W^T, read with gfx950's transposing LDS read
//     (ds_read_b64_tr_b16), which gives each 16-lane group any 4 rows: so the
//     order in which the previous layer's results hold the units (the MFMA
//     result layout reused as the next B operand, see mlp_common.hpp) is
//     absorbed by the read addresses, with no permuted copy of W;
//   * the copies go through a buffer resource over the true dims[l] x
//     dims[l+1] matrix: rows k >= dims[l] and columns n >= dims[l+1] read as
//     zero, so padded units add exact zeros and the caller's weights need no
//     padding;
//   * every layer runs ceil(dims[l] / 32) k steps and ceil(dims[l+1] / 16)
//     output sub-tiles (run-time counts, uniform branches): a narrow layer
//     costs its own width, not the chain's widest;
//   * softplus in base-2 units as in the resident kernel, but in the form
//     max(a, 0) + log2(1 + 2^-|a|), exact for every argument, so there is no
//     guard and no recompute pass (the resident kernel's guard relies on all
//     weights staying in LDS); ReLU and none as there.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "mlp_common.hpp"

namespace coalesce {
namespace {

// Geometry per width class P (the widest layer, rounded up to 64, 128 or
// 256) and form (ST: the training forward): MT 16-row sub-tiles per wave
// tile, KSM 32-deep k steps at most.
template <int P, bool ST = false>
struct SGeo {
  static constexpr int MT = 2;            // 16-row sub-tiles per wave tile: one weight read feeds two MFMAs
  static constexpr int TR = 16 * MT;      // rows per wave tile
  static constexpr int KSM = P / 32;      // k steps of the widest layer
  // waves per workgroup (up to one wave tile each) and per SIMD: at width
  // 256 two (the registers of two 256-unit activation buffers); at 128 three
  // for the inference forward and two for the training forward, whose fp32
  // activation stores dominate (6 x 128 on 2^20 rows, alternating runs:
  // forward 0.342 / 0.361 ms with three / two, training forward 0.705 /
  // 0.651 ms); at 64 three
  static constexpr int MINW = P == 256 || (P == 128 && ST) ? 2 : 3;
  static constexpr int WAVES = 4 * MINW;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROWS = P;          // k rows of a slot
  static constexpr int SLOT = ROWS * 128;  // fp16 elements of a slot (128 units per row)
};

// A wave tile's activations in MFMA B-operand form (as in the resident
// kernel): v[s][ks] = the 8 fp16 inputs of k step ks this lane feeds.
template <int P>
struct STile {
  u32x4 v[SGeo<P>::MT][SGeo<P>::KSM];
};

// 16-byte chunk swizzle of a slot row (256 bytes = 16 chunks): chunk c of
// row k sits at c ^ sswz(k).  A transposing read by half a wave covers the
// 32-byte pieces of 8 rows, rows {k0..k0+3, k0+8..k0+11} for the first layer
// (natural k order) and {k0..k0+7} for the later ones (the result-layout
// order); f below is distinct on both sets, so either read touches each of
// the 64 banks once.  The swizzle moves whole 32-byte pieces (even values).
__device__ __forceinline__ int sswz(int k) {
  const int f = (k & 3) | ((((k >> 2) ^ (k >> 3)) & 1) << 2);
  return f << 1;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16-byte buffer-to-LDS copy: lane l's 16 bytes land at LDS byte address
// lds + 16 l; an offset at or past the resource's size reads zeros.  Issued
// through inline asm so that the compiler does not make every later LDS read
// wait for it; the kernel waits for the copies itself before the barrier
// that publishes a slot.
__device__ __forceinline__ void dma16_rsrc(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);  // (wave-uniform; an SGPR for M0)
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Raw buffer resource (wave-uniform) over n bytes at p.
__device__ __forceinline__ u32x4 rsrc_words(const void* p, uint32_t n) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t w0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t w1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  const uint32_t w2 = (uint32_t)__builtin_amdgcn_readfirstlane((int)n);
  return (u32x4){w0, w1, w2, 0x00020000u};
}

constexpr uint32_t S_OFF_NONE = 0x80000000u;  // past every resource (all are below 2^31 bytes)

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// The chunks of the chain in order: chunk j is (layer, column chunk).
struct ChunkPos {
  int l, cc;
};
__device__ __forceinline__ ChunkPos next_chunk(const MlpStreamParams& p, ChunkPos c) {
  if (c.cc + 1 < ceil_div(p.dims[c.l + 1], 128)) return ChunkPos{c.l, c.cc + 1};
  return ChunkPos{c.l + 1 < p.L ? c.l + 1 : 0, 0};
}

// Copy chunk c into the slot at LDS byte address slot: copy j (0 .. 8 KS_l
// - 1) fills the 4 rows 4 j .. 4 j + 3 (64 chunks of 16 bytes); wave w
// issues the copies j = w, w + WAVES, ...  Rows past the layer's k steps
// are not copied (never read).
template <int P, bool ST>
__device__ __forceinline__ void copy_chunk(const MlpStreamParams& p, ChunkPos c, uint32_t slot, int wu, int lane) {
  const int K = p.dims[c.l], N = p.dims[c.l + 1];
  const int ks = ceil_div(K, 32);
  const u32x4 rs = rsrc_words(p.W[c.l], (uint32_t)K * (uint32_t)N * 2u);
  const int sl = lane & 15;
  for (int j = wu; j < 8 * ks; j += SGeo<P, ST>::WAVES) {
    const int row = 4 * j + (lane >> 4);
    const int n = 128 * c.cc + 8 * (sl ^ sswz(row));
    const uint32_t off = row < K && n < N ? ((uint32_t)row * (uint32_t)N + (uint32_t)n) * 2u : S_OFF_NONE;
    dma16_rsrc(rs, off, slot + (uint32_t)j * 1024u);
  }
}

// Buffer resource over the 16-row sub-tile s of wave tile `tile` of a
// row-major matrix (pitch ld elements of `es` bytes; the host bounds 16 rows
// below 2^31 bytes): rows past M are outside it.
template <int P>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int M, int tile, int s, int64_t ld,
                                                            int es) {
  const int64_t first = (int64_t)tile * SGeo<P>::TR + 16 * s;
  const int64_t rows = min((int64_t)16, max((int64_t)0, (int64_t)M - first));
  char* q = (char*)base + first * ld * es;
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)((uint32_t)rows * (uint32_t)(ld * es)), 0x00020000);
}

// x of a wave tile: k step ks of sub-tile s holds units 32 ks + 8 g .. + 7 of
// row (lane & 15); columns past dims[0] read as zero.
template <int P>
__device__ __forceinline__ void load_x(const MlpStreamParams& p, int tile, int lane, STile<P>& h) {
  using G = SGeo<P>;
  const int q = lane & 15, g = lane >> 4;
  const int ks0 = ceil_div(p.dims[0], 32);
#pragma unroll
  for (int s = 0; s < G::MT; ++s) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc<P>(p.x, p.M, tile, s, p.ldx, 2);
#pragma unroll
    for (int ks = 0; ks < G::KSM; ++ks) {
      const int u = 32 * ks + 8 * g;
      const uint32_t off = ks < ks0 && u < p.dims[0] ? (uint32_t)q * (uint32_t)p.ldx * 2u + 2u * (uint32_t)u : S_OFF_NONE;
      h.v[s][ks] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    }
  }
}

// A operand (W^T rows n = 16 t + (lane & 15) of the chunk, 8 k of k step ks)
// from the slot: two transposing reads of 4 rows each.  first: the layer's
// input is x (lane group g holds k = 32 ks + 8 g + e); otherwise it is the
// previous layer's result layout (k = 32 ks + 16 (e / 4) + 4 g + e % 4).
// With q = lane & 15, r = q >> 2, the row is k = 32 ks + kr + (half term),
// kr = 8 g + r (first) or 4 g + r, and the swizzle sswz(k) = 2 f comes out
// independent of ks: f = r | (half ^ (g & 1)) << 2 (first) or
// r | ((g ^ (g >> 1)) & 1) << 2.  Column n = 16 t + 4 (q & 3) then sits at
// element 16 (t ^ f) + 8 ((q & 3) >> 1) + 4 (q & 1) of its row.  tbase()
// gives the byte address of half 0 for sub-tile t; k step ks adds 8192 ks
// bytes, half 1 adds 1024 (first: 4 rows, and f flips bit 2: t ^ 4 in the
// column term) or 4096 (16 rows, f unchanged) -- constant offsets.
__device__ __forceinline__ uint32_t tbase(uint32_t slot, int t, bool first, int lane) {
  const int q = lane & 15, g = lane >> 4, r = q >> 2;
  const int kr = first ? 8 * g + r : 4 * g + r;
  const int f = first ? (r | ((g & 1) << 2)) : (r | (((g ^ (g >> 1)) & 1) << 2));
  return slot + 2u * (uint32_t)(kr * 128 + 16 * (t ^ f) + 8 * ((q & 3) >> 1) + 4 * (q & 1));
}
__device__ __forceinline__ i16x8 read_w(uint32_t b0, uint32_t b1, int ks, bool first) {
  const uint32_t a0 = b0 + 8192u * (uint32_t)ks;
  const uint32_t a1 = b1 + 8192u * (uint32_t)ks + (first ? 1024u : 4096u);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)a0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)a1);
  return (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// softplus in base-2 units, exact for every argument: g = log2(1 + 2^a)
// written as max(a, 0) + log2(1 + 2^-|a|) (2^-|a| <= 1 never overflows).
__device__ __forceinline__ float softplus_b2_exact(float a) {
  return __builtin_fmaxf(a, 0.0f) + __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-__builtin_fabsf(a)));
}

// Wait until at most n of this wave's vector-memory operations are in
// flight (n uniform, 0 .. 63; the counter's immediate must be a constant).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int N = 0>
__device__ __forceinline__ void wait_vm_rt(int n) {
  if constexpr (N == 63) {
    wait_vm<63>();
  } else {
    if (n <= N)
      wait_vm<N>();
    else
      wait_vm_rt<N + 1>(n);
  }
}

// One chunk of layer l for the wave tile: output sub-tiles t < nt of the
// chunk (units 128 cc + 16 t ..), k steps < ks.  Hidden layers apply the
// activation and write the fp16 operand into hout (and, training forward,
// the fp32 activation to acts[l]); the last layer stores out.  Returns the
// number of store instructions the wave issued.
template <int P, int ACT, bool ST, int CC>
__device__ __forceinline__ int chunk(const MlpStreamParams& p, int l, uint32_t slot, const STile<P>& hin,
                                     STile<P>& hout, int tile, int lane) {
  using G = SGeo<P>;
  constexpr bool SP = ACT == ACT_SOFTPLUS;
  const ChunkPos c{l, CC};
  const bool first = l == 0, last = l == p.L - 1;
  const int ks = ceil_div(p.dims[l], 32);
  const int N = p.dims[l + 1];
  const int nt = min(8, ceil_div(N - 128 * c.cc, 16));
  // With softplus the hidden activations travel in base-2 units (as in the
  // resident kernel): a layer-0 accumulator is scaled by log2 e before the
  // activation; the last layer's output, when its input is in base-2 units,
  // by ln 2.
  const float pre = SP && first && !last ? 1.44269504088896341f : 1.0f;
  const float post = SP && !first && last ? 0.693147180559945309f : 1.0f;
  const int g = lane >> 4;
  __amdgpu_buffer_rsrc_t ro[G::MT];
#pragma unroll
  for (int s = 0; s < G::MT; ++s) {
    if (last)
      ro[s] = tile_rsrc<P>(p.out, p.M, tile, s, p.ldo, 2);
    else if (ST)
      ro[s] = tile_rsrc<P>(p.acts[l], p.M, tile, s, p.lda, 4);
  }
  const uint32_t orow = (uint32_t)(lane & 15) * (uint32_t)(last ? p.ldo * 2 : p.lda * 4);
  u32x2 ev[G::MT];
  const int stores = last ? G::MT * ((nt + 1) / 2) : ST ? G::MT * nt : 0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t < nt) {
      // (opaque: formed here, not hoisted out of the chunk loop into 16
      // registers held for the whole kernel)
      const uint32_t b0 = opaque(tbase(slot, t, first, lane));
      const uint32_t b1 = first ? opaque(tbase(slot, t ^ 4, first, lane)) : b0;
      f32x4 acc[G::MT];
#pragma unroll
      for (int s = 0; s < G::MT; ++s) acc[s] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < G::KSM; ++k) {
        if (k < ks) {
          const i16x8 wa = read_w(b0, b1, k, first);
#pragma unroll
          for (int s = 0; s < G::MT; ++s)
            acc[s] = mfma16x16x32(wa, __builtin_bit_cast(i16x8, hin.v[s][k]), acc[s], _Float16());
        }
      }
      const int u = 128 * c.cc + 16 * t;  // first unit of the sub-tile
#pragma unroll
      for (int s = 0; s < G::MT; ++s) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = acc[s][r] * pre;
          if (last)
            v[r] = acc[s][r] * post;
          else if constexpr (SP)
            v[r] = softplus_b2_exact(a);
          else if constexpr (ACT == ACT_RELU)
            v[r] = relu(a);
          else
            v[r] = a;
        }
        const u32x2 o = (u32x2){pack_f16(v[0], v[1]), pack_f16(v[2], v[3])};
        if (last) {
          // pairs of sub-tiles as in the resident kernel: 16 bytes per lane
          if ((t & 1) == 0) {
            ev[s] = o;
            if (t + 1 == nt) {  // odd count: the pair's second half is past N
              const uint32_t off = u + 16 * (g & 1) + 8 * (g >> 1) < N
                                       ? orow + 2u * (uint32_t)u + 32u * (uint32_t)(g & 1) + 16u * (uint32_t)(g >> 1)
                                       : S_OFF_NONE;
              store_pair(ro[s], off, ev[s], (u32x2){0u, 0u});
            }
          } else {
            const int u0 = u - 16;
            const uint32_t off = u0 + 16 * (g & 1) + 8 * (g >> 1) < N
                                     ? orow + 2u * (uint32_t)u0 + 32u * (uint32_t)(g & 1) + 16u * (uint32_t)(g >> 1)
                                     : S_OFF_NONE;
            store_pair(ro[s], off, ev[s], o);
          }
        } else {
          const int kk = u >> 5;  // the next layer's k step holding these units
          hout.v[s][kk][(t & 1) * 2] = o[0];
          hout.v[s][kk][(t & 1) * 2 + 1] = o[1];
          if constexpr (ST) {
            const float sc = SP ? 0.693147180559945309f : 1.0f;
            const uint32_t off = u + 4 * g < N ? orow + 4u * (uint32_t)(u + 4 * g) : S_OFF_NONE;
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, (f32x4){v[0] * sc, v[1] * sc, v[2] * sc, v[3] * sc}), ro[s], off, 0, 0);
          }
        }
      }
    } else if (!last && (t & 1) == 1 && t == nt) {
      // odd count of sub-tiles: the other half of the last k step is zero
      const int kk = (128 * c.cc + 16 * t) >> 5;
#pragma unroll
      for (int s = 0; s < G::MT; ++s) {
        hout.v[s][kk][2] = 0u;
        hout.v[s][kk][3] = 0u;
      }
    }
  }
  return stores;
}

// Issue order of one pipeline step of chunk_full: NM MFMAs, a transposing
// LDS read after each of the first NR, VPM VALU instructions (the
// transcendentals included) after each, and a buffer store after every
// ST_EVERY-th when NS stores are due.
template <int NM, int NR, int VPM, int NS, int ST_EVERY>
__device__ __forceinline__ void interleave_stream() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (NS > 0 && i % ST_EVERY == ST_EVERY - 1 && i / ST_EVERY < NS) __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, VPM, 0);
  }
}

// A chunk that spans the slot: all KSM k steps and 8 output sub-tiles, with
// the layer's role (first: input x in natural order; last: output to out)
// fixed at compile time.  Nothing inside depends on a run-time condition, so
// the steps are software-pipelined as in the resident kernel: step t issues
// the MFMAs of sub-tile t (their weight fragments read one step ahead)
// interleaved with the activation and stores of sub-tile t - 1.  Every unit
// of such a chunk lies inside the layer, so no column is masked.  The same
// arithmetic as chunk(), per element, so both give the same bits.
template <int P, int ACT, bool ST, int CC, bool FIRST, bool LAST>
__device__ __forceinline__ int chunk_full(const MlpStreamParams& p, int l, uint32_t slot, const STile<P>& hin,
                                          STile<P>& hout, int tile, int lane) {
  using G = SGeo<P>;
  constexpr int KS = G::KSM, MT = G::MT, NT = 8;
  constexpr bool SP = ACT == ACT_SOFTPLUS;
  constexpr float pre = SP && FIRST && !LAST ? 1.44269504088896341f : 1.0f;
  constexpr float post = SP && !FIRST && LAST ? 0.693147180559945309f : 1.0f;
  constexpr bool STORE = LAST || ST;
  // VALU issue slots per element (a transcendental counts twice): the
  // activation, the pre-scale, the fp32 copy's scale, half a pack
  constexpr int VPE2 = LAST ? 4 : (SP ? 15 : 3) + (pre != 1.0f ? 2 : 0) + (ST ? 2 : 0);
  constexpr int VPM = (MT * 4 * VPE2 / 2 + KS * MT - 1) / (KS * MT);
  const int g = lane >> 4;
  __amdgpu_buffer_rsrc_t ro[MT];
  uint32_t ooff = 0;
  if constexpr (STORE) {
#pragma unroll
    for (int s = 0; s < MT; ++s)
      ro[s] = LAST ? tile_rsrc<P>(p.out, p.M, tile, s, p.ldo, 2) : tile_rsrc<P>(p.acts[l], p.M, tile, s, p.lda, 4);
    // the lane's row, and its units of sub-tile 0 (of the pair, for out)
    ooff = LAST ? (uint32_t)(lane & 15) * (uint32_t)(p.ldo * 2) + 2u * (128u * CC) + 32u * (uint32_t)(g & 1) +
                      16u * (uint32_t)(g >> 1)
                : (uint32_t)(lane & 15) * (uint32_t)(p.lda * 4) + 4u * (128u * CC + 4u * (uint32_t)g);
    ooff = opaque(ooff);
  }
  // weight-fragment addresses of sub-tile 0 (halves 0 and 1, see tbase);
  // sub-tile t is the same XOR 32 t (the column term 16 (t ^ f) in fp16 units)
  const uint32_t w0 = opaque(tbase(slot, 0, FIRST, lane));
  const uint32_t w1 = FIRST ? (w0 ^ 128u) : w0;
  i16x8 wa[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) wa[ks] = read_w(w0, w1, ks, FIRST);
  f32x4 acc[MT], prv[MT];
  u32x2 ev[MT];
#pragma unroll
  for (int t = 0; t <= NT; ++t) {
    if (t < NT) {
      const uint32_t n0 = opaque(w0 ^ (uint32_t)(32 * (t + 1))), n1 = FIRST ? (n0 ^ 128u) : n0;
#pragma unroll
      for (int s = 0; s < MT; ++s) acc[s] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int s = 0; s < MT; ++s)
          acc[s] = mfma16x16x32(wa[ks], __builtin_bit_cast(i16x8, hin.v[s][ks]), acc[s], _Float16());
        if (t + 1 < NT) wa[ks] = read_w(n0, n1, ks, FIRST);
      }
    }
    if (t > 0) {
      const int u = t - 1;
#pragma unroll
      for (int s = 0; s < MT; ++s) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = prv[s][r] * pre;
          if constexpr (LAST)
            v[r] = prv[s][r] * post;
          else if constexpr (SP)
            v[r] = softplus_b2_exact(a);
          else if constexpr (ACT == ACT_RELU)
            v[r] = relu(a);
          else
            v[r] = a;
        }
        const u32x2 o = (u32x2){pack_f16(v[0], v[1]), pack_f16(v[2], v[3])};
        if constexpr (LAST) {
          if ((u & 1) == 0)
            ev[s] = o;
          else
            store_pair(ro[s], ooff + 32u * (uint32_t)(u - 1), ev[s], o);
        } else {
          const int kk = (128 * CC + 16 * u) >> 5;  // the next layer's k step holding these units
          hout.v[s][kk][(u & 1) * 2] = o[0];
          hout.v[s][kk][(u & 1) * 2 + 1] = o[1];
          if constexpr (ST) {
            const float sc = SP ? 0.693147180559945309f : 1.0f;
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, (f32x4){v[0] * sc, v[1] * sc, v[2] * sc, v[3] * sc}), ro[s],
                ooff + 64u * (uint32_t)u, 0, 0);
          }
        }
      }
    }
    if (t > 0 && t < NT) {
      constexpr int NR = 2 * KS;
      if constexpr (LAST) {
        if ((t - 1) & 1)
          interleave_stream<KS * MT, NR, VPM, MT, KS>();
        else
          interleave_stream<KS * MT, NR, VPM, 0, KS>();
      } else if constexpr (ST) {
        interleave_stream<KS * MT, NR, VPM, MT, KS>();
      } else {
        interleave_stream<KS * MT, NR, VPM, 0, KS>();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < MT; ++s) prv[s] = acc[s];
  }
  return LAST ? MT * NT / 2 : ST ? MT * NT : 0;
}

// One chunk of layer l: the pipelined form when the chunk spans the slot,
// else the general one.
template <int P, int ACT, bool ST, int CC>
__device__ __forceinline__ int run_chunk(const MlpStreamParams& p, int l, uint32_t slot, const STile<P>& hin,
                                         STile<P>& hout, int tile, int lane) {
  using G = SGeo<P>;
  const bool full = ceil_div(p.dims[l], 32) == G::KSM && p.dims[l + 1] - 128 * CC >= 128;
  if (full) {
    const bool first = l == 0, last = l == p.L - 1;
    if (first)
      return last ? chunk_full<P, ACT, ST, CC, true, true>(p, l, slot, hin, hout, tile, lane)
                  : chunk_full<P, ACT, ST, CC, true, false>(p, l, slot, hin, hout, tile, lane);
    return last ? chunk_full<P, ACT, ST, CC, false, true>(p, l, slot, hin, hout, tile, lane)
                : chunk_full<P, ACT, ST, CC, false, false>(p, l, slot, hin, hout, tile, lane);
  }
  return chunk<P, ACT, ST, CC>(p, l, slot, hin, hout, tile, lane);
}

template <int P, int ACT, bool ST>
__global__ __launch_bounds__((SGeo<P, ST>::THREADS), (SGeo<P, ST>::MINW)) void mlp_stream_kernel(MlpStreamParams p) {
  using G = SGeo<P, ST>;
  __shared__ __attribute__((aligned(1024))) _Float16 sW[2 * G::SLOT];
  const int lane = threadIdx.x & 63;
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t slot0 = lds_addr(sW), slot1 = slot0 + 2u * G::SLOT;
  // Rounds: in round r workgroup b takes the wave tiles r G W + b + w G
  // (G workgroups, W waves, w the wave), so a batch of fewer tiles than
  // G W spreads over the workgroups (one tile each while there are at most
  // G) instead of filling the waves of a few; the round goes on while the
  // workgroup's first wave has a tile.
  const int ntiles = p.num_tiles;
  const int G_ = (int)gridDim.x;
  const int64_t per_round = (int64_t)G_ * G::WAVES;
  int64_t first = blockIdx.x;  // tile of wave 0 in this round
  if (first >= ntiles) return;

  // The chunk sequence repeats per round; copies run one chunk ahead.  The
  // memory counter completes in order, so waiting for a chunk's copies means
  // waiting until no more than the wave's later operations are in flight:
  // `after` counts them (the x loads and stores issued since), and the
  // x prefetch and the output stores stay in flight across the barrier.
  ChunkPos cur{0, 0};
  int js = 0;  // slot of cur
  copy_chunk<P, ST>(p, cur, slot0, wu, lane);
  // Two activation buffers: every layer reads ha and writes hb, which is
  // then copied into ha (a few register moves per layer, where alternating
  // the roles at run time would make the compiler address the buffers
  // indirectly).  The last layer writes to memory, so hb is free while it
  // runs: the next round's x is loaded into it there.
  STile<P> ha, hb;
  // (tile indices past the last are clamped to it: a zero-row tile whose
  // buffer resources start right after the rows)
  load_x<P>(p, (int)min(first + (int64_t)wu * G_, (int64_t)ntiles), lane, ha);
  int after = G::MT * G::KSM;
  while (first < ntiles) {
    const int64_t tile64 = first + (int64_t)wu * G_;
    const int tile = (int)min(tile64, (int64_t)ntiles);
    const int64_t next_first = first + per_round;
    const int next_tile = (int)min(next_first + (int64_t)wu * G_, (int64_t)ntiles);
    // A wave whose tile lies past the last row (a small batch, or the last
    // round) still copies its share of every chunk and passes the barriers,
    // but skips the chunk's arithmetic: zero rows would have come out of it.
    const bool has_rows = tile64 < ntiles;
    // one chunk: wait for its copies (the wave's own; the barrier makes every
    // wave's visible and retires the other slot's last reader), start the
    // next chunk's copies, compute.  CC (the column chunk) is a template
    // argument so that every register index stays a constant.
    auto step = [&](auto cc_tag, int l) {
      constexpr int CC = decltype(cc_tag)::value;
      wait_vm_rt(after);
      __syncthreads();
      const ChunkPos nxt = next_chunk(p, cur);
      if (!(nxt.l == 0 && nxt.cc == 0 && next_first >= ntiles)) copy_chunk<P, ST>(p, nxt, js ? slot0 : slot1, wu, lane);
      after = 0;
      if (l == p.L - 1 && CC == 0) {
        // the next round's x (a zero-row tile past the last tile reads nothing)
        load_x<P>(p, next_tile, lane, hb);
        after = G::MT * G::KSM;
      }
      if (has_rows) after += run_chunk<P, ACT, ST, CC>(p, l, js ? slot1 : slot0, ha, hb, tile, lane);
      cur = nxt;
      js ^= 1;
    };
    for (int l = 0; l < p.L; ++l) {
      step(std::integral_constant<int, 0>{}, l);
      if constexpr (P == 256)
        if (p.dims[l + 1] > 128) step(std::integral_constant<int, 1>{}, l);
      ha = hb;
    }
    first = next_first;
  }
}

// Grid: min(#CUs x workgroups per CU, #wave tiles) persistent workgroups
// (occupancy from the runtime, cached), or the caller's count.
template <int P, int ACT, bool ST>
hipError_t launch_pa(MlpStreamParams p, int num_workgroups, int num_cus, hipStream_t stream) {
  using G = SGeo<P, ST>;
  p.num_tiles = (int)(((int64_t)p.M + G::TR - 1) / G::TR);
  static std::atomic<int> per_cu_cache{0};
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int n = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mlp_stream_kernel<P, ACT, ST>, G::THREADS, 0);
    if (e != hipSuccess) return e;
    per_cu = n > 0 ? n : 1;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  int nwg = num_workgroups;
  if (nwg <= 0) {
    const long cap = (long)num_cus * per_cu;
    nwg = p.num_tiles < cap ? p.num_tiles : (int)cap;
  }
  if (nwg < 1) nwg = 1;
  hipLaunchKernelGGL((mlp_stream_kernel<P, ACT, ST>), dim3(nwg), dim3(G::THREADS), 0, stream, p);
  return hipGetLastError();
}

template <int P, bool ST>
hipError_t launch_p(const MlpStreamParams& p, int act, int nwg, int cus, hipStream_t stream) {
  if (act == ACT_NONE) return launch_pa<P, ACT_NONE, ST>(p, nwg, cus, stream);
  if (act == ACT_RELU) return launch_pa<P, ACT_RELU, ST>(p, nwg, cus, stream);
  return launch_pa<P, ACT_SOFTPLUS, ST>(p, nwg, cus, stream);
}

}  // namespace

hipError_t launch_mlp_stream(const MlpStreamParams& p, int P, int act, bool store_acts, int num_workgroups,
                             int num_cus, hipStream_t stream) {
  if (P == 256)
    return store_acts ? launch_p<256, true>(p, act, num_workgroups, num_cus, stream)
                      : launch_p<256, false>(p, act, num_workgroups, num_cus, stream);
  if (P == 128)
    return store_acts ? launch_p<128, true>(p, act, num_workgroups, num_cus, stream)
                      : launch_p<128, false>(p, act, num_workgroups, num_cus, stream);
  return store_acts ? launch_p<64, true>(p, act, num_workgroups, num_cus, stream)
                    : launch_p<64, false>(p, act, num_workgroups, num_cus, stream);
}

}  // namespace coalesce
