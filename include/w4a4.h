/*
 * w4a4.h -- C ABI of libw4a4: the SVDQuant W4A4 + 16-bit low-rank linear layer on AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (SVDQuant summary page, arXiv 2411.05007v4, §4.2 and Fig. 4):
 *
 *     Y = Q(X̂) · Q(R)ᵀ + bf16(bf16(X̂) · L1) · L2 (+ bias),   X̂ = X · diag(λ)^-1
 *     Ŵ = W · diag(λ),  Ŵᵀ ≈ L1 · L2 (rank r),  R = Ŵ − (L1 · L2)ᵀ
 *
 * λ are per-input-channel smoothing factors (App. D, after SmoothQuant), L1·L2 the rank-r SVD
 * of the smoothed weight kept in 16 bits, Q a 4-bit quantizer: per-group (64 along K) symmetric
 * INT4 with bf16 scales (App. D), or FP4 E2M1 with one power-of-two (E8M0) scale per block of 32.
 * Following §4.3 / Fig. 6 the down projection X̂·L1 is computed by the activation quantizer and
 * the up projection is added inside the 4-bit GEMM.
 *
 * Conventions
 *  - Ownership: the caller allocates and frees every buffer; host buffers are ordinary arrays,
 *    device buffers are device memory (e.g. from torch). The library never allocates device
 *    memory, never synchronizes a stream and keeps no mutable global state, with two exceptions
 *    described at their calls: the GELU table that the first GELU call on a device fills in the
 *    library's device data (waiting on that call's stream), and the fixed device scratch array of
 *    the no-allocation MLP call.
 *  - bf16 tensors are passed as uint16_t bit patterns. Row-major everywhere.
 *  - Library layouts: codes and scales of activations and weights, and the low-rank factors, use
 *    the private layouts described at w4a4_buffer_sizes(). Rows (M of X, N of W) are padded to a
 *    multiple of W4A4_ROW_ALIGN; padding rows are written as zero codes with zero scales.
 *    w4a4_codes_to_canonical() / w4a4_scales_to_canonical() convert to plain layouts.
 *  - Errors: every argument is validated on the host before anything is launched or written;
 *    a failed check returns a status and leaves outputs untouched. Device calls return
 *    W4A4_ERR_HIP if a launch fails; faults inside kernels surface at the caller's stream
 *    synchronization. No C++ exception crosses the ABI (host memory exhaustion returns
 *    W4A4_ERR_HOST_MEMORY).
 *  - Non-finite values: the host calls scan their bf16 / fp32 inputs (weights, given factors,
 *    channel maxima, LoRA factors) and return W4A4_ERR_NUMERIC, writing nothing, if one is Inf or
 *    NaN. The device calls do not scan activations: a non-finite activation gives unspecified codes,
 *    scales and outputs in its row (other rows are unaffected); it never makes a kernel read or
 *    write out of bounds.
 *  - Device pointers must be 16-byte aligned.
 */
#ifndef W4A4_H
#define W4A4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A4_ABI_VERSION 2   /* 2: + W8A8 format, refined preparation, the MLP-pair GELU calls */
#define W4A4_GROUP 64        /* INT4 group size along K (App. D) */
#define W4A4_MX_BLOCK 32     /* FP4 block size along K */
#define W4A4_ROW_ALIGN 256   /* M and N are padded to a multiple of this in library layouts */
#define W4A4_RANK_ALIGN 16   /* rank is zero-padded to a multiple of this (r_pad) */
#define W4A4_MAX_RANK 128    /* largest supported rank (after any LoRA merge) */
#define W4A4_W8A8_MAX_K 131072 /* W8A8: 127 * 127 * K stays below 2^31 (exact int32 sums) */
#define W4A4_NOALLOC_SCRATCH_BYTES (32u << 20) /* fixed per-GPU scratch of the no-allocation call */

typedef enum {
  W4A4_OK = 0,
  W4A4_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misalignment, rank out of range ... */
  W4A4_ERR_UNSUPPORTED = 2,  /* unknown format */
  W4A4_ERR_NUMERIC = 3,      /* non-finite input, non-normal smoothing factor, SVD failure */
  W4A4_ERR_HIP = 4,          /* a HIP launch or runtime call failed */
  W4A4_ERR_HOST_MEMORY = 5,  /* a host-side allocation failed */
  W4A4_ERR_TOO_LARGE = 6     /* the problem needs more than the no-allocation call's fixed scratch */
} w4a4_status_t;

typedef enum {
  W4A4_FMT_INT4_G64 = 0,     /* per-group-64 symmetric INT4, bf16 scales */
  W4A4_FMT_MXFP4_B32 = 1,    /* E2M1 codes, E8M0 scale per block of 32 */
  W4A4_FMT_W8A8 = 2          /* 8-bit setting (App. D): symmetric INT8 per row (activations per
                                token, weights per output channel), fp32 scales */
} w4a4_fmt_t;

/* Same object as hipStream_t; NULL is the default stream. */
typedef struct ihipStream_t* w4a4_stream_t;

/* Byte sizes of every library buffer for one layer (see w4a4_buffer_sizes). */
typedef struct {
  size_t wq, wscale, l1t, l2t;   /* weights side (prepare_weights outputs) */
  size_t xq, xscale, xl1;        /* activation side (quantize_act outputs) */
  int m_pad, n_pad, rank_pad;
} w4a4_sizes_t;

int w4a4_abi_version(void);
const char* w4a4_status_str(w4a4_status_t status);

/*
 * Buffer sizes and layouts. K must be a positive multiple of 64 for every format (the MXFP4
 * kernels step K by two 32-blocks). m_pad = roundup(M, 256), n_pad = roundup(N, 256),
 * rank_pad = roundup(rank, 16) (0 for rank 0). Layouts (G64 = K/64, B32 = K/32):
 *   wq     MXFP4: [G64][n_pad][32] bytes, the 64 codes of (row, group) 4 bits each: code k of the
 *            group at byte k/2, low nibble for even k (E2M1 codes).
 *          INT4 (FP6 images, n_pad·K·3/4 bytes): code q is carried as the FP6 E2M3 field
 *            F = (q < 0) << 5 | |q| (the encoding of q/8). The 64 codes of (row, group g) form four
 *            runs of 16; run j's fields F_f (f = 0..15, code 16j + f) make the 96-bit image
 *            Σ_f F_f << 6f, dwords o0 o1 o2 (little-endian). Half h (runs 2h, 2h+1) is stored as a
 *            16-byte main part [o0 o1 o2 of run 2h, o0 of run 2h+1] at byte (g·n_pad + row)·32 + 16h
 *            and an 8-byte extra part [o1 o2 of run 2h+1] at byte n_pad·K/2 + ((2g + h)·n_pad + row)·8.
 *            The GEMM feeds these images to its FP6 MFMAs as they are.
 *   wscale INT4: [G64][n_pad] bf16;  MXFP4: [B32][n_pad] E8M0 bytes (e + 127)
 *   W8A8:  wq [B32][n_pad][32] int8 codes (code k of the 32-slice at byte k);
 *          wscale [n_pad] fp32 (one scale per output channel)
 *   l1t    [rank_pad][K] bf16   : L1ᵀ, rows >= rank are zero
 *   l2t    [n_pad][rank_pad] bf16 : L2ᵀ, columns >= rank are zero
 *   xq, xscale : as wq, wscale with m_pad rows. W8A8: xscale holds the [m_pad] fp32 per-token
 *          scales first; the rest of the buffer is scratch for w4a4_quantize_act (per-K-slice
 *          partial row maxima).
 *   xl1    fp32, first [m_pad][rank_pad] : t = bf16(X̂)·L1 (fp32 accumulation); the rest of the
 *          buffer (when the size returned here exceeds m_pad·rank_pad·4 bytes) is scratch that
 *          w4a4_quantize_act uses for per-K-slice partial sums of t. 0 bytes when rank == 0.
 *          w4a4_lowrank_linear reads only the first m_pad·rank_pad floats.
 * Returns W4A4_ERR_INVALID_ARG for M, N < 1, K not a positive multiple of 64, rank outside
 * [0, min(N, K, W4A4_MAX_RANK)], or out == NULL; W4A4_ERR_UNSUPPORTED for an unknown fmt.
 */
w4a4_status_t w4a4_buffer_sizes(int M, int N, int K, int rank, int fmt, w4a4_sizes_t* out);

/* ----------------------------------------------------------------- host (CPU, synchronous) */

/*
 * out[j] = max_i |A[i, j]| for a bf16 matrix A [rows][lda] (the activation / weight channel
 * maxima the smoothing factor is built from, App. D). Thread-safe. W4A4_ERR_NUMERIC (out not
 * written) if A holds an Inf or NaN.
 */
w4a4_status_t w4a4_column_absmax(const uint16_t* A, int rows, int cols, int lda, float* out);

/*
 * Smoothing factors (App. D, after SmoothQuant): λ_j = max|X_j|^α / max|W_j|^(1-α).
 * α = 0.5 is computed as fp32(sqrt(double(ax)/double(aw))); other α in (0, 1) as
 * fp32(pow(ax, α) / pow(aw, 1 - α)) in double. λ_j = 1 when ax or aw is 0.
 * inv_lambda[j] = 1.0f / λ_j (IEEE float division). W4A4_ERR_NUMERIC if a maximum is not finite
 * or a λ_j is not a finite normal float; W4A4_ERR_INVALID_ARG for α outside (0, 1) or negative
 * maxima. Nothing is written on error.
 */
w4a4_status_t w4a4_smooth_factors(const float* amax_x, const float* amax_w, int K, float alpha,
                                  float* lambda, float* inv_lambda);

/*
 * Offline weight preparation (§4.2): Ŵ = W·diag(λ) (fp64); rank-r split Ŵᵀ ≈ L1·L2 with
 * L1 = bf16(U_r Σ_r), L2 = bf16(V_rᵀ); residual R = fp32(Ŵ − (L1·L2)ᵀ) with the rank sum in
 * fp64 in increasing rank order; R quantized per `fmt` into (wq, wscale); L1, L2 written
 * transposed and zero-padded into (l1t, l2t).
 *   W      [N][K] bf16 (host)
 *   lambda [K] fp32 (host)
 *   L1_in  [K][rank], L2_in [rank][N] bf16 (host) -- if both non-NULL they are used as the
 *          factors (no SVD); if both NULL the library computes its own truncated SVD
 *          (randomized subspace iteration + one-sided Jacobi; deterministic).
 *   wq, wscale, l1t, l2t  host outputs sized by w4a4_buffer_sizes (copy them to the device).
 *   L1_out [K][rank], L2_out [rank][N] bf16 (host, optional, may be NULL): the factors used.
 * Thread-safe; uses several CPU threads. W4A4_ERR_NUMERIC if W (or a given factor) holds an Inf
 * or NaN, or the SVD does not converge; W4A4_ERR_INVALID_ARG for a λ_j that is not a positive finite
 * float.
 */
w4a4_status_t w4a4_prepare_weights(const uint16_t* W, int N, int K, const float* lambda, int rank,
                                   int fmt, const uint16_t* L1_in, const uint16_t* L2_in,
                                   uint8_t* wq, void* wscale, uint16_t* l1t, uint16_t* l2t,
                                   uint16_t* L1_out, uint16_t* L2_out);

/*
 * Iterative refinement of the split (§4.2: iterative updates lower the quantization error and the
 * result with the smallest error after several iterations is kept). Iteration 0 is the split of
 * w4a4_prepare_weights (own SVD); iteration i >= 1 re-fits the low-rank branch to what the
 * current 4-bit branch misses, L1·L2 = rank-r SVD of (Ŵ − deq(Q(R_{i-1})))ᵀ, and quantizes
 * R_i = Ŵ − (L1·L2)ᵀ afresh. Each iteration is scored by ||Ŵ − (L1·L2)ᵀ − deq(Q(R))||_F (fp64);
 * the outputs (same buffers and layouts as w4a4_prepare_weights) hold the iteration with the
 * smallest score, the earliest on ties.
 *   iters      0 .. 64 further iterations (0 gives w4a4_prepare_weights' result)
 *   errors     [iters + 1] fp64 host output, the score of every iteration (may be NULL)
 *   best_iter  host output, the iteration kept (may be NULL)
 * Host buffers; synchronous; thread-safe; uses several CPU threads. Errors as
 * w4a4_prepare_weights (W4A4_ERR_INVALID_ARG also for iters outside 0 .. 64).
 */
w4a4_status_t w4a4_prepare_weights_refined(const uint16_t* W, int N, int K, const float* lambda, int rank,
                                           int fmt, int iters, uint8_t* wq, void* wscale, uint16_t* l1t,
                                           uint16_t* l2t, uint16_t* L1_out, uint16_t* L2_out, double* errors,
                                           int* best_iter);

/*
 * LoRA merge without re-quantization (§2, §5.2: the low-rank branch absorbs a LoRA by growing
 * its rank): L1' = [L1 | A], L2' = [L2 ; B], rank' = rank + ra. Reads the library-layout
 * factors (l1t [rank_pad][K], l2t [n_pad][rank_pad]) and writes the merged ones
 * (l1t_out [rank_pad'][K], l2t_out [n_pad][rank_pad']); A [K][ra], B [ra][N] bf16. Host
 * buffers. The 4-bit codes and scales are not touched (they are not even passed in).
 */
w4a4_status_t w4a4_append_lowrank(const uint16_t* l1t, const uint16_t* l2t, int K, int N, int rank,
                                  const uint16_t* A, const uint16_t* B, int ra,
                                  uint16_t* l1t_out, uint16_t* l2t_out);

/*
 * Library code layout -> canonical: out [rows][K/2] bytes, code 2i in the low nibble; INT4
 * codes become two's-complement nibbles, MXFP4 codes stay E2M1; W8A8: out [rows][K] int8.
 * `q` is a wq or xq buffer (host copy) with roundup(rows, 256) padded rows.
 */
w4a4_status_t w4a4_codes_to_canonical(const uint8_t* q, int rows, int K, int fmt, uint8_t* out);

/* Library scale layout -> canonical: INT4 out [rows][K/64] bf16; MXFP4 out [rows][K/32] bytes;
 * W8A8 out [rows] fp32. */
w4a4_status_t w4a4_scales_to_canonical(const void* s, int rows, int K, int fmt, void* out);

/* ----------------------------------------------------- device (asynchronous on `stream`) */

/*
 * Activation side, one pass over X (§4.3: the down projection shares the activations with the
 * quantizer). Per row m and group:
 *   X̂ = fp32(X · inv_lambda) (one fp32 multiply); codes and scales of X̂ per `fmt`
 *   (INT4: s = bf16(max|X̂|/7), q = rint(X̂ · (1/s)); MXFP4: e = min{e : 6·2^e >= max|X̂|},
 *   E2M1 round-half-even of X̂ / 2^e; W8A8, per row over all of K: s = fp32(max|X̂|/127),
 *   q = clamp(rint(X̂ · (1/s)), -127, 127)); t = bf16(X̂) · L1 accumulated in fp32.
 *   X          [M][ldx] bf16 device, K <= ldx <= 2^26, ldx % 8 == 0 (W4A4_ERR_INVALID_ARG otherwise)
 *   inv_lambda [K] fp32 device
 *   l1t        [rank_pad][K] bf16 device (NULL allowed when rank == 0)
 *   xq, xscale, xl1 device outputs in library layout (xl1 may be NULL when rank == 0).
 *   All m_pad rows of xq/xscale/xl1 are written (padding rows as zeros).
 */
w4a4_status_t w4a4_quantize_act(const uint16_t* X, int M, int K, int ldx, const float* inv_lambda,
                                const uint16_t* l1t, int rank, int fmt,
                                uint8_t* xq, void* xscale, float* xl1, w4a4_stream_t stream);

/*
 * The fused 4-bit GEMM with the low-rank up projection in its epilogue (§4.3):
 *   Y[m][n] = bf16( Σ_g s_x[m,g] s_w[n,g] Σ_{k∈g} q_x[m,k] q_w[n,k]      (INT4)
 *                   or Σ_b 2^(e_x+e_w) Σ_{k∈b} val(c_x) val(c_w)          (MXFP4)
 *                   or s_x[m] s_w[n] Σ_k q_x[m,k] q_w[n,k]                 (W8A8, App. D;
 *                      exact int32 sum, then fp32; requires K <= 131072)
 *                 + Σ_i bf16(t[m][i]) · L2[i][n]  + bias[n] )
 *   xq, xscale, xl1  outputs of w4a4_quantize_act (device)
 *   wq, wscale, l2t  outputs of w4a4_prepare_weights, copied to the device
 *   bias   [N] bf16 device or NULL
 *   Y      [M][ldy] bf16 device, ldy >= N. Only the M x N block is written.
 */
w4a4_status_t w4a4_lowrank_linear(const uint8_t* xq, const void* xscale, const float* xl1,
                                  const uint8_t* wq, const void* wscale, const uint16_t* l2t,
                                  const uint16_t* bias, uint16_t* Y, int ldy,
                                  int M, int N, int K, int rank, int fmt, w4a4_stream_t stream);

/* ------------------------------------- the MLP pair, fc1 -> GELU -> fc2 (device, asynchronous) */

/*
 * GELU used between the two layers of the MLP (this library's fixed reading; the SVDQuant page
 * names no formula): GELU(y) = (y/2)(1 + erf(y/sqrt 2)) in fp32 with erf from Abramowitz & Stegun
 * 7.1.28, 1 - (1 + a1 x + ... + a6 x^6)^-16, |error| <= 3e-7, evaluated one IEEE fp32 operation at a
 * time (Horner from a6, the 16th power by four squarings, correctly rounded division), so that
 * the bf16 rounding of X2 = bf16(GELU(Y1)) is reproducible on a host. The first GELU call on a
 * device evaluates it once for the bf16 inputs with 2^-20 <= |x| < 256 into a 14 KB table in the
 * library's device data (on the call's stream, waiting for it; not possible during stream capture,
 * where it returns W4A4_ERR_HIP and is retried by the next call); the kernels look those values up
 * and evaluate the function for every other input, with identical results.
 *
 * Consumer side: w4a4_quantize_act (INT4 only) applied to X = bf16(GELU(Y)) of a producer's bf16
 * output Y [M][ldy] (device; K <= ldy <= 2^26, ldy % 8 == 0); every other argument as for
 * w4a4_quantize_act.
 */
w4a4_status_t w4a4_gelu_quantize_act(const uint16_t* Y, int M, int K, int ldy, const float* inv_lambda,
                                     const uint16_t* l1t, int rank, int fmt,
                                     uint8_t* xq, void* xscale, float* xl1, w4a4_stream_t stream);

/*
 * Producer side (the quantizer fused into the producer's epilogue, §4.3's fusion principle one
 * step upstream): the 4-bit GEMM of fc1 (arguments as for w4a4_lowrank_linear) whose epilogue
 * emits fc2's activation side instead of fc1's output: X2 = bf16(GELU(bf16(Y1))) (padding rows:
 * 0), smoothed by inv_lambda2 [N] (fc2's 1/lambda over fc2's K = this layer's N), quantized to
 * fc2's INT4 codes xq2 [N/64][m_pad][32] and bf16 scales xscale2 [N/64][m_pad] (library layout,
 * as w4a4_quantize_act writes them), and t2 = bf16(X2_hat)·L1_2 into xl1_2 ([m_pad][rank2_pad] fp32
 * first, then per-256-column-tile partial planes as scratch; size from
 * w4a4_gelu_quant_xl1_bytes). l1t2 is fc2's [rank2_pad][N] L1 transpose. Y [M][ldy] bf16 receives
 * Y1 when not NULL (for checking; the fused path does not need it).
 * Requires fmt == W4A4_FMT_INT4_G64, N a multiple of 64, rank <= 32 and rank2 <= 32
 * (W4A4_ERR_UNSUPPORTED otherwise); xq2/xscale2/xl1_2 device buffers sized as w4a4_buffer_sizes
 * gives them for fc2 (M rows, K = N), except xl1_2.
 */
w4a4_status_t w4a4_lowrank_linear_gelu_quant(const uint8_t* xq, const void* xscale, const float* xl1,
                                             const uint8_t* wq, const void* wscale, const uint16_t* l2t,
                                             const uint16_t* bias, int M, int N, int K, int rank, int fmt,
                                             const float* inv_lambda2, const uint16_t* l1t2, int rank2,
                                             uint8_t* xq2, void* xscale2, float* xl1_2, uint16_t* Y, int ldy,
                                             w4a4_stream_t stream);

/* Bytes of the xl1_2 buffer of w4a4_lowrank_linear_gelu_quant (0 when rank2 < 1 or M, N < 1). */
size_t w4a4_gelu_quant_xl1_bytes(int M, int N, int rank2);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): w4a4_lowrank_linear_gelu_quant without any
 * caller-provided scratch. Same arguments and results, except that t2 is only fc2's t
 * ([m_pad][rank2_pad] fp32, m_pad * rank2_pad * 4 bytes) and the per-256-column-tile partial t2
 * planes go to a fixed device array owned by the library: W4A4_NOALLOC_SCRATCH_BYTES on every GPU
 * the library runs on, from the loading of its code on that GPU until the process ends. The call
 * allocates nothing (no hipMalloc, no allocating library routine); its first call on a GPU looks
 * up that GPU's copy of the array (hipGetSymbolAddress) with the GPU current.
 * Limit: ceil(N / 256) * m_pad * rank2_pad * 4 bytes must not exceed W4A4_NOALLOC_SCRATCH_BYTES
 * (e.g. M = 4608, N = 12288, rank2 = 32: 28.3 MB), else W4A4_ERR_TOO_LARGE before anything is
 * launched. Every call writes all the planes it reads, so nothing needs clearing between calls;
 * but all calls on one GPU share that GPU's array, so calls that overlap in time on one GPU (other
 * streams, other threads) race, and the caller must serialize them. W4A4_ERR_HIP if the array's
 * address cannot be looked up or a launch fails.
 */
w4a4_status_t w4a4_lowrank_linear_gelu_quant_noalloc(const uint8_t* xq, const void* xscale, const float* xl1,
                                                     const uint8_t* wq, const void* wscale, const uint16_t* l2t,
                                                     const uint16_t* bias, int M, int N, int K, int rank, int fmt,
                                                     const float* inv_lambda2, const uint16_t* l1t2, int rank2,
                                                     uint8_t* xq2, void* xscale2, float* t2, uint16_t* Y, int ldy,
                                                     w4a4_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* W4A4_H */
