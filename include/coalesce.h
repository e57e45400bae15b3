/*
 * coalesce.h -- C ABI of the MI355X (gfx950) fused-epilogue GEMM and softplus
 * MLP megakernel library (libcoalesce.so).
 *
 * Every pointer argument named as device memory is a device pointer owned by
 * the caller; the library keeps no pointer after a call returns and never
 * allocates device memory on these paths.  `stream` is a hipStream_t passed
 * as void* (NULL = the legacy default stream).  Calls only enqueue work:
 * they return before the GPU has run it, and a fault inside a kernel shows
 * up at the caller's next synchronisation of that stream.
 *
 * Errors: every entry point validates its arguments on the host before it
 * launches anything.  On any return other than COALESCE_OK nothing has been
 * launched and no output has been written; coalesce_last_error() then gives
 * a one-line explanation (thread-local, valid until the next call on the
 * same thread).
 *   COALESCE_ERR_INVALID_ARGUMENT  a NULL pointer where data is needed, a
 *                                  negative extent, a leading dimension
 *                                  shorter than the row, an unknown enum.
 *   COALESCE_ERR_UNSUPPORTED       a valid request the library does not
 *                                  implement (alignment, dtype combination,
 *                                  MLP width or depth), see each function.
 *   COALESCE_ERR_DEVICE            a HIP call failed (launch or device query).
 *
 * Layout: every matrix is row-major with a leading dimension (elements
 * between consecutive rows) and unit inner stride.  Alignment: base
 * pointers must be 16-byte aligned and ld * element_size a multiple of 16
 * bytes, so that every row can be moved with 128-bit accesses.  The extents
 * M, N, K themselves are arbitrary (partial tiles are masked).
 */
#ifndef COALESCE_H
#define COALESCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  COALESCE_OK = 0,
  COALESCE_ERR_INVALID_ARGUMENT = 1,
  COALESCE_ERR_UNSUPPORTED = 2,
  COALESCE_ERR_DEVICE = 3
} coalesce_status;

typedef enum { COALESCE_F32 = 0, COALESCE_F16 = 1, COALESCE_BF16 = 2 } coalesce_dtype;

typedef enum {
  COALESCE_ACT_NONE = 0,
  COALESCE_ACT_GELU_ERF = 1, /* 0.5 z (1 + erf(z / sqrt 2)) */
  COALESCE_ACT_SOFTPLUS = 2, /* ln(1 + e^z), evaluated as z above 20 */
  COALESCE_ACT_RELU = 3      /* z > 0 ? z : 0 (the matmul-relu of the "Coalesce" README's MLIR pipeline) */
} coalesce_act;

/*
 * Y = act(A . B + bias) with the bias add and the activation applied to the
 * fp32 accumulators in registers, then one rounding to out_dtype and one
 * store of Y.  Defined by the "Coalesce" README ("Fusion study": GEMM + bias
 * + GELU fused into the GEMM kernel; "Notes for future sessions": GELU is
 * the erf form), with softplus as in the "MLP Megakernel" README.
 *
 *   A     device, M x K, in_dtype, leading dimension lda >= K
 *   B     device, K x N, in_dtype, leading dimension ldb >= N
 *   bias  device, N elements of in_dtype (added to every row), or NULL
 *   Y     device, M x N, out_dtype, leading dimension ldy >= N (written)
 * Accumulation is fp32 (fp32 MFMA for F32 inputs, bf16/fp16 MFMA otherwise);
 * bias and activation are computed in fp32; the store rounds to nearest even.
 * Supported (in_dtype -> out_dtype): F32->F32, BF16->BF16, BF16->F32,
 * F16->F16, F16->F32.  M, N, K must be below 2^31 (and, for 16-bit inputs,
 * lda <= 2^23, ldb <= 2^25); M == 0 or N == 0 is a
 * no-op; K == 0 gives Y = act(bias) (act(0) without a bias), and A, B may
 * then be NULL.  Y must not overlap A, B or bias.
 */
coalesce_status coalesce_gemm_bias_act(const void* A, int64_t lda, const void* B, int64_t ldb, const void* bias,
                                       void* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                       coalesce_dtype in_dtype, coalesce_dtype out_dtype, coalesce_act act,
                                       void* stream);

/*
 * Persistent MLP megakernel ("MLP Megakernel" README, "Architecture" and
 * "Key ideas"):
 *   h_0 = x;  h_l = act(h_{l-1} W_l) for l < L;  out = h_{L-1} W_L
 * with no biases and a linear last layer, in ONE launch whose intermediate
 * activations stay on chip (fp16 MFMA operands, fp32 accumulation, the
 * activation in fp32, h_l rounded to fp16 only as the next layer's operand).
 * The grid is G persistent workgroups: enough to give each of their waves a
 * row tile, and at least min(#tiles, #CUs) so that a small batch spreads over
 * the CUs, at most #CUs x occupancy; workgroup b owns the row tiles b, b + G,
 * b + 2G, ..., which its waves take one at a time as they become free.
 *
 *   x     device, M x dims[0] fp16, leading dimension ldx >= dims[0]
 *   W     HOST array of L device pointers; W[l] is dims[l] x dims[l+1] fp16,
 *         dense row-major (the x @ W orientation)
 *   dims  HOST array of L + 1 widths
 *   out   device, M x dims[L] fp16, leading dimension ldo >= dims[L] (written)
 * Supported: dtype F16; hidden_act SOFTPLUS, RELU or NONE (a linear chain);
 * widths multiples of 8 and at most 256, in any mix (the quick start's D, H,
 * out_features), L = 1..16 ("MLP Megakernel" README, Reports: the megakernel
 * generalised to N layers).  Chains whose weights fit in LDS (every width at
 * most 64 and L <= 8, or at most 128 and L <= 4) run the resident kernel
 * above: all W_l staged in LDS once per workgroup, each layer at the padded
 * kernel width 64 or 128 (the weights zero-padded in LDS, x loads and out
 * stores limited to the true columns, the k steps past dims[0] and the output
 * sub-tiles past dims[L] skipped: the padded units add exact zeros, so the
 * result is the one the narrower chain gives).  The other chains run the
 * layer-streaming kernel: the same layer arithmetic, each layer at its own
 * width, with the weights passed through LDS one 128-unit chunk at a time
 * (direct copies from the caller's unpadded W[l], double-buffered); softplus
 * there is evaluated in the exact form max(z, 0) + ln(1 + e^-|z|), equal
 * in real arithmetic to the resident kernel's guarded form up to the guard's
 * ln(1 + e^-20) ~ 2e-9 (the two round differently in fp32, so a chain run by
 * both kernels need not give the same bits).  x is M x dims[0], out
 * M x dims[L], W[l] dense dims[l] x dims[l+1].  M == 0 is a no-op.
 */
coalesce_status coalesce_mlp_forward(const void* x, int64_t ldx, const void* const* W, const int64_t* dims, int32_t L,
                                     void* out, int64_t ldo, int64_t M, coalesce_dtype dtype, coalesce_act hidden_act,
                                     void* stream);

/*
 * As coalesce_mlp_forward, with the persistent grid size chosen by the
 * caller: num_workgroups > 0 launches exactly that many workgroups (each
 * owns every num_workgroups-th row tile), 0 picks the default grid above.  The
 * result does not depend on the grid size, bit for bit.
 */
coalesce_status coalesce_mlp_forward_grid(const void* x, int64_t ldx, const void* const* W, const int64_t* dims,
                                          int32_t L, void* out, int64_t ldo, int64_t M, coalesce_dtype dtype,
                                          coalesce_act hidden_act, int64_t num_workgroups, void* stream);

/*
 * Training forward ("MLP Megakernel" README, "Key ideas": for training, the
 * forward keeps the hidden activations in fp32 so that the backward's
 * softplus derivative loses nothing).  Computes out exactly as
 * coalesce_mlp_forward does (the same bits) and also writes, for
 * l = 0 .. L-2,
 *   acts[l] = h_{l+1} = act(z_{l+1})
 * in fp32: the activation as computed on the fp32 accumulators, before its
 * rounding to the next layer's fp16 operand.
 *   acts  HOST array of L - 1 device pointers, each M x dims[l+1] fp32 with
 *         leading dimension lda (dims[l+1] <= lda <= 2^24, 16-byte aligned
 *         rows), not overlapping x, out, the weights or each other; may be
 *         NULL when L == 1.
 * Other arguments, support and errors as coalesce_mlp_forward.
 */
coalesce_status coalesce_mlp_forward_train(const void* x, int64_t ldx, const void* const* W, const int64_t* dims,
                                           int32_t L, void* out, int64_t ldo, float* const* acts, int64_t lda,
                                           int64_t M, coalesce_dtype dtype, coalesce_act hidden_act, void* stream);

/*
 * Device workspace in bytes that coalesce_mlp_backward needs for this chain
 * and M rows on the current device.  Chains whose weights fit in LDS (widths
 * up to 64 and at most 8 layers, or up to 128 and at most 4) need one
 * partial weight gradient per compute unit, whatever M; the others (run
 * layer by layer) need the partial sums of their largest layer plus, for
 * L >= 2, one (L == 2) or two fp16 buffers of M x max(dims[1..L-1]) for the
 * hidden gradients.  Returns 0 for an unsupported width or depth, a negative
 * or too large M, or a failed device query.
 */
size_t coalesce_mlp_backward_workspace_size(const int64_t* dims, int32_t L, int64_t M);

/*
 * Backward of the MLP chain ("MLP Megakernel" README, "Key ideas": the
 * backward reads the fp32 activations stored by the training forward,
 * multiplies by the derivative of softplus, and casts to fp16 only for the
 * matrix-core operands; the weight gradients come out of one fused kernel).
 * With h_0 = x, h_l = acts[l-1], the upstream gradient dz_L = dout and
 * 0-based layers l = L-1 .. 0:
 *   dW[l] = h_l^T dz_{l+1}               (fp32, summed over all M rows)
 *   dz_l  = (dz_{l+1} W_l^T) * act'(z_l)  (l > 0)
 *   dx    = dz_1 W_0^T                    (when dx is not NULL)
 * act'(z_l) is recovered from h_l in fp32: softplus -> 1 - exp(-h_l) (the
 * logistic sigmoid of z_l; absolute error at most 2^-23), relu -> 1 where
 * h_l > 0 else 0, none -> 1.  h_l and dz_l are rounded to fp16 (nearest
 * even) as MFMA operands; products accumulate in fp32.
 *   x         device, M x dims[0] fp16 (ldx)    the forward's input
 *   W, dims   as coalesce_mlp_forward
 *   acts      HOST array of L - 1 device pointers, M x dims[l+1] fp32 (lda),
 *             as written by coalesce_mlp_forward_train; may be NULL when L == 1
 *   dout      device, M x dims[L] fp16 (ldd)    dLoss/d(out)
 *   dW        HOST array of L device pointers, each dims[l] x dims[l+1] fp32,
 *             dense row-major (the x @ W orientation of W[l]), overwritten
 *   dx        device, M x dims[0] fp16 (ldq), written; or NULL to skip it
 *   workspace device, at least coalesce_mlp_backward_workspace_size(dims, L, M)
 *             bytes, 16-byte aligned, not overlapping any other argument;
 *             its contents on entry are ignored
 * Pitches are at least the operand's width and at most 2^24, with 16-byte
 * aligned rows.  Chains whose weights fit in LDS (widths up to 64 and at most
 * 8 layers, or up to 128 and at most 4) run two kernels on `stream`: the
 * fused backward over all layers (one persistent workgroup per compute unit;
 * each sums its rows' weight-gradient terms in registers) and a reduction
 * that adds the per-workgroup sums in a fixed order.  The other chains that
 * coalesce_mlp_forward supports (up to 16 layers, widths up to 256) run
 * layer by layer, l = L-1 .. 0: one fused kernel per layer (per pair of
 * layers at widths up to 128, the pair's inner gradient staying on chip)
 * computes dz_l (or dx) and the per-workgroup sums of dW[l] from the same
 * row tiles, with the dz_l passed between launches kept as fp16 in the
 * workspace (the precision in which the next layer uses it either way),
 * then the reduction of that launch's dW sums.  Either way repeated calls
 * give identical bits.  M == 0 gives dW = 0.  Non-square chains write only
 * the true dims[l] x dims[l+1] of each dW and the true columns of dx.
 * Outputs must not overlap the inputs, each other or the workspace.  Calls
 * that share a workspace must be ordered on one stream.
 */
coalesce_status coalesce_mlp_backward(const void* x, int64_t ldx, const void* const* W, const int64_t* dims,
                                      int32_t L, const float* const* acts, int64_t lda, const void* dout,
                                      int64_t ldd, float* const* dW, void* dx, int64_t ldq, int64_t M,
                                      coalesce_dtype dtype, coalesce_act hidden_act, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * coalesce_mlp_backward without the workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  The workspace (the per-workgroup
 * partial weight gradients, and for chains run layer by layer the fp16
 * hidden gradients) is a scratch array of 64 MiB (67108864 bytes) that the
 * library keeps in device memory, one per device, for the life of the
 * process; the call itself allocates nothing and clears nothing (the
 * backward overwrites every value it reads back).  A call whose workspace
 * (coalesce_mlp_backward_workspace_size(dims, L, M)) exceeds 64 MiB is
 * rejected with COALESCE_ERR_UNSUPPORTED before anything is launched: every
 * chain whose weights fit in LDS fits on a device of up to 256 compute
 * units, whatever M; a chain run layer by layer fits while its partial sums
 * and hidden-gradient buffers do (e.g. 6 layers 128 wide up to 65536
 * rows on 256 compute units).  Every call on one device shares that
 * device's scratch, which keeps
 * the last call's contents: calls that can overlap on one device (streams
 * without an order between them, several host threads) race and give wrong
 * gradients, so order them on one stream.  Otherwise the arguments, the
 * results (bit for bit the same as coalesce_mlp_backward's) and the errors
 * are those of coalesce_mlp_backward.
 */
coalesce_status coalesce_mlp_backward_noalloc(const void* x, int64_t ldx, const void* const* W, const int64_t* dims,
                                              int32_t L, const float* const* acts, int64_t lda, const void* dout,
                                              int64_t ldd, float* const* dW, void* dx, int64_t ldq, int64_t M,
                                              coalesce_dtype dtype, coalesce_act hidden_act, void* stream);

/*
 * Weight normalisation of every layer of a chain in ONE launch ("MLP
 * Megakernel" README, "Key ideas": the fused kernel normalises all weight
 * matrices, W = g * v / ||v||, so that per-layer launches do not dominate at
 * small sizes).  The norm is taken per output unit, i.e. over each column of
 * the x @ W matrix (torch's weight_norm on a Linear weight):
 *   W[l][k][n] = g[l][n] * v[l][k][n] / sqrt(sum_k v[l][k][n]^2)
 *   v, W  HOST arrays of L device pointers; layer l is dims[l] x dims[l+1]
 *         fp16, dense row-major; W[l] is written
 *   g     HOST array of L device pointers to dims[l+1] fp16 gains
 *   dims  HOST array of L + 1 positive widths; 1 <= L <= 16
 * Sums of squares in fp32 (added in a fixed order), the scale g / ||v|| in
 * fp32, one rounding of W to fp16.  A column of zeros gives NaN, as the
 * formula does.  dtype must be F16.  Outputs must not overlap inputs.
 */
coalesce_status coalesce_weight_norm(const void* const* v, const void* const* g, void* const* W, const int64_t* dims,
                                     int32_t L, coalesce_dtype dtype, void* stream);

/*
 * Backward of coalesce_weight_norm for all layers in one launch, from the
 * weight gradients dW (fp32, e.g. from coalesce_mlp_backward):
 *   dg[l][n]    = <dW[l][:, n], v[l][:, n]> / ||v[l][:, n]||
 *   dv[l][k][n] = g[l][n] / ||v[l][:, n]|| * (dW[l][k][n] - v[l][k][n] <dW, v>_n / ||v_n||^2)
 *   v, g, dims  as coalesce_weight_norm (fp16)
 *   dW          HOST array of L device pointers, dims[l] x dims[l+1] fp32
 *   dv, dg      HOST arrays of L device pointers, fp32, written
 * Everything in fp32; reductions in a fixed order.
 */
coalesce_status coalesce_weight_norm_backward(const void* const* v, const void* const* g, const float* const* dW,
                                              float* const* dv, float* const* dg, const int64_t* dims, int32_t L,
                                              coalesce_dtype dtype, void* stream);

/*
 * Unfused baseline, step 2: Y = X + bias (bias broadcast over rows), each
 * element converted to fp32, added, and rounded once to y_dtype.  The
 * elementwise-kernel design of the "Fuse Elementwise Ops" page (vectorised
 * 128-bit loads, bounds-guarded tails).
 *   X device M x N (x_dtype, ldx), bias device N elements (bias_dtype),
 *   Y device M x N (y_dtype, ldy); Y may equal X (in place) when the types
 *   and leading dimensions match.
 */
coalesce_status coalesce_bias_add(const void* X, int64_t ldx, const void* bias, void* Y, int64_t ldy, int64_t M,
                                  int64_t N, coalesce_dtype x_dtype, coalesce_dtype bias_dtype, coalesce_dtype y_dtype,
                                  void* stream);

/*
 * Unfused baseline, step 3: Y = act(X) elementwise in fp32, rounded once to
 * the storage type.  X and Y are device M x N of `dtype`; Y may equal X.
 */
coalesce_status coalesce_activation(const void* X, int64_t ldx, void* Y, int64_t ldy, int64_t M, int64_t N,
                                    coalesce_dtype dtype, coalesce_act act, void* stream);

/*
 * Benchmark helper: stream `bytes` of device memory at `buf` through the
 * cache hierarchy with 128-bit reads so that the L2 and the MALL hold none
 * of the operands of the next timed kernel (the "Coalesce" README's harness
 * flushes the cache before every timed run).  `sink` is a device pointer to
 * at least 4 bytes that receives a value derived from the data (it keeps
 * the reads alive).  buf must be 16-byte aligned, bytes a multiple of 16.
 */
coalesce_status coalesce_flush_caches(const void* buf, size_t bytes, void* sink, void* stream);

/*
 * Benchmark helper: the matrix-core rate and engine clock this board sustains
 * with nothing else sharing the time ("Coalesce" README, Results: figures are
 * taken after the boost clock has settled; Triton port and the notes for
 * future sessions: thermal throttling moves repeated runs by ~10 %).  One
 * 8-wave workgroup per CU (two waves per SIMD, as the 256 x 256 bf16 GEMM
 * tile); each wave runs `iters` rounds of the GEMM wave's 4 x 8 block of
 * v_mfma_f32_16x16x32_bf16 twice, on two sets of operand fragments held in
 * registers: 64 MFMAs = 2^20 FLOP per wave and round, no memory traffic.
 *   ops    device, 16-byte aligned: nsets x 24 x 64 fragments of 8 bf16
 *          (16 bytes); wave w takes set w mod nsets, fragment f of lane l at
 *          index (set * 24 + f) * 64 + l; fragments 0-3 and 12-15 are the A
 *          operands, 4-11 and 16-23 the B operands of the two sets.
 *   sink   device float[waves * 64]: each lane's sum of its accumulators
 *          (keeps the work alive).
 *   clocks device uint64[2 * waves]: per wave, the shader-clock counter
 *          (s_memtime) and the constant-rate counter (s_memrealtime) elapsed
 *          over its loop; engine clock = first / second x wallclock_khz.
 *   max_waves  capacity of sink and clocks in waves.
 *   *waves, *wallclock_khz (host): the launch's wave count (8 per CU) and the
 *          constant-rate counter's frequency; written before any other check,
 *          so a call with NULL buffers queries them and returns
 *          COALESCE_ERR_INVALID_ARGUMENT without a launch.
 * Errors: NULL or misaligned pointers, nsets or iters <= 0, max_waves below the
 * launch's wave count -> an error before any launch.
 */
coalesce_status coalesce_matrix_rate(const void* ops, int32_t nsets, int32_t iters, void* sink, void* clocks,
                                     int64_t max_waves, int32_t* waves, int64_t* wallclock_khz, void* stream);

/*
 * Per-shape autotuning ("Coalesce" README, plan's phase 4 and its finding that
 * tile shape was worth more than anything else measured; "MLP Megakernel"
 * README, "Autotuning": an exhaustive search per shape, a cached fast path,
 * and post-tune correctness validation).  An autotune call takes the same
 * arguments as the entry point it tunes and computes the same output; it
 * runs every candidate launch configuration `iters` times on the caller's
 * data (the tile shape -- three compiled tile configurations --, persistent
 * grid size and tile-group order of the bf16/fp16 GEMM; the tile shape -- four
 * compiled ones -- and group order of the FP32 GEMM; for the MLP megakernel
 * its two compiled launch configurations (waves per workgroup and the register
 * budget that goes with them) and the grid size), keeps the fastest whose
 * output equals the default
 * configuration's bit for bit (every candidate performs the same arithmetic
 * per output element, so equality is the exact test; the default is kept
 * unless a candidate is more than 1 % faster than the default's faster pass
 * in both of its own passes), and records it: later
 * calls of coalesce_gemm_bias_act / coalesce_mlp_forward with the same
 * device, shape, dtypes and activation use it.  Each candidate is timed in
 * two passes (the second in reverse order) and keeps its faster time, so
 * the warm-up drift of the clocks favours none of them.
 *   iters      timed launches per candidate and pass, 1..10000
 *   workspace  device, 16-byte aligned, at least
 *              round_up(rows * row_bytes of the output, 256) + 256 bytes
 *              (the reference copy and a counter)
 *   report     filled when not NULL
 * Autotuning synchronises `stream` and may take a while (candidates x iters
 * launches).  Errors as the tuned entry point; COALESCE_ERR_DEVICE also when
 * no candidate reproduced the default output (nothing is recorded then).
 */
typedef struct {
  int32_t candidates;  /* configurations tried (the default first) */
  int32_t valid;       /* of them, those whose output matched the default's bit for bit */
  float default_us;    /* mean launch time of the default configuration */
  float best_us;       /* mean launch time of the chosen one */
  int32_t grid;        /* the chosen workgroup count (0: the launcher's default) */
  int32_t group_m;     /* the chosen tile-group height (0: default) */
  int32_t variant;     /* GEMM tile shape, 0 = the launcher's heuristic.  FP32: 1 = 128 x 128,
                          2 = 64 x 64, 3 = 32 x 32, 4 = 64 x 32; bf16 / fp16: 1 = 256 x 256,
                          2 = 128 x 128, 3 = 64 x 64.  MLP (chains whose
                          weights fit in LDS): 0 = the launcher's choice (16-row wave tiles for
                          batches of at most ~96 rows per wave of the grid, else 32-row tiles),
                          1 = 32-row tiles with 8 / 12 waves per workgroup (width 128 / 64),
                          2 = 16-row tiles, 3 = 32-row tiles (12 / 16 waves) */
} coalesce_tune_report;

coalesce_status coalesce_autotune_gemm_bias_act(const void* A, int64_t lda, const void* B, int64_t ldb,
                                                const void* bias, void* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                                coalesce_dtype in_dtype, coalesce_dtype out_dtype, coalesce_act act,
                                                int32_t iters, void* workspace, size_t workspace_bytes,
                                                coalesce_tune_report* report, void* stream);

coalesce_status coalesce_autotune_mlp_forward(const void* x, int64_t ldx, const void* const* W, const int64_t* dims,
                                              int32_t L, void* out, int64_t ldo, int64_t M, coalesce_dtype dtype,
                                              coalesce_act hidden_act, int32_t iters, void* workspace,
                                              size_t workspace_bytes, coalesce_tune_report* report, void* stream);

/* Forget every tuned configuration (all devices). */
coalesce_status coalesce_autotune_clear(void);

/* Number of compute units of the current device (cached per device). */
int32_t coalesce_device_cu_count(void);

/*
 * Status reporting, after the status-checking helper of the vectorfold.studio
 * GPU-compilation tutorial (every runtime call's status is checked and a
 * failure is turned into a readable message naming the call):
 * coalesce_status_string gives the enumerator's name for a status code
 * (never NULL; "COALESCE_ERR_UNKNOWN" for a value outside the enum); coalesce_last_error gives
 * the detail of the calling thread's last non-OK return ("" if there was
 * none), valid until that thread's next call into the library.  Neither
 * launches anything or touches the device.
 */
const char* coalesce_status_string(coalesce_status s);
const char* coalesce_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int32_t coalesce_version(void);

#ifdef __cplusplus
}
#endif

#endif /* COALESCE_H */
