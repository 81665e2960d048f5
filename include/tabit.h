/*
 * tabit.h -- C ABI of the timestep-adaptive-bit quantized linear for MI355X (gfx950).
 *
 * One quantized linear layer of a diffusion transformer whose weight
 * precision changes per layer and per denoising step:
 *
 *   - TASQ (Temporal-Adaptive Bit Sparsification Quantization; gist.science
 *     technical summary section 2 "Metodologia", and the newx.sg abstract):
 *     one shared maximum-precision (8-bit) weight buffer is stored; a learned
 *     per-(layer, stage) LSB mask truncates least-significant bits, giving an
 *     effective precision of 8 - k without per-stage weight copies; switching
 *     precision costs nothing because the engine simply reads fewer bit planes.
 *   - HQ-DM (gist.science technical summary section 2.1): activations are
 *     rotated by a block-diagonal Hadamard before symmetric quantization; the
 *     Hadamard normalization is moved into the fp scales so the core is an
 *     integer matrix product.
 *   - 6Bit-Diffusion (gist.science technical summary section 2A): per layer
 *     and step, INT8 for unstable layers or a 4-bit format for stable ones,
 *     after a local block Hadamard.  The 4-bit format here is OCP MXFP4
 *     (E2M1 elements, one E8M0 scale per 32), gfx950's native 4-bit format.
 *
 * Conventions (apply to every entry point):
 *   Ownership   The caller allocates and owns every device buffer; the library
 *               never allocates device memory.  A tabit_ctx owns host state only
 *               (schedule table, last error text, options).
 *   Layout      Row-major, K contiguous.  X is [M][K] (tokens x input features),
 *               W is [N][K] (the nn.Linear layout), Y is [M][N].  bf16 values
 *               are passed as their uint16_t bit patterns.
 *   Streams     `stream` is a hipStream_t passed as void* (NULL = default
 *               stream).  Work is enqueued asynchronously; nothing synchronizes.
 *               No entry point allocates, frees or memsets, so calls may be
 *               captured into a HIP graph.
 *   Errors      Every int-returning call returns TABIT_OK or a negative
 *               status.  Arguments are validated before any HIP call; a failed
 *               validation launches nothing.  tabit_last_error(ctx) gives text.
 *               Faults inside kernels surface at the caller's synchronize.
 *   Threads     A ctx is not thread-safe; separate ctxs are independent.
 *   Shapes      M >= 0 (M == 0 is a no-op), K % 32 == 0 and 32 <= K <= 32768,
 *               N % 32 == 0 (N == 0 is a no-op), K % had_block == 0;
 *               M * K and N * K below 2^31 (each operand under 2 GiB).
 *               had_block in {0, 32, 64, 128} (0 = no rotation); the MXFP4
 *               format takes had_block in {0, 32}.
 *   Alignment   bf16/int8/fp4 matrices 16-byte aligned; fp32 vectors 4-byte.
 *   Contract    Activations and weights must be rotated with the same
 *               had_block; the library cannot detect a mismatch.  Inputs must
 *               be finite with |x| * had_block below the fp32 range.
 */
#ifndef TABIT_H
#define TABIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tabit_ctx tabit_ctx;

enum tabit_status {
  TABIT_OK = 0,
  TABIT_EINVAL = -1,   /* null pointer, unknown enum value, bad option          */
  TABIT_ESHAPE = -2,   /* shape constraint violated (K % 32, N % 32, K % b, ...) */
  TABIT_EALIGN = -3,   /* pointer not aligned as required                        */
  TABIT_ERANGE = -4,   /* k outside [0, 7], block size not supported            */
  TABIT_ENOSCHED = -5, /* no schedule installed, or (step, layer) outside it    */
  TABIT_EHIP = -6,     /* HIP runtime error (launch or attribute query)          */
  TABIT_ENOMEM = -7    /* host allocation failed                                 */
};

enum tabit_fmt { TABIT_FMT_INT8 = 0, TABIT_FMT_MXFP4 = 1 };
enum tabit_path {
  TABIT_PATH_MASKED = 0,
  TABIT_PATH_BITSERIAL = 1,
  TABIT_PATH_PLANES = 3,
  TABIT_PATH_HQDM = 4
};

/* Create / destroy a context (host memory only; makes no HIP call).
 * tabit_create returns TABIT_EINVAL if out is NULL, TABIT_ENOMEM on failure. */
int tabit_create(tabit_ctx** out);
void tabit_destroy(tabit_ctx* ctx);

/* Text of the last error recorded on ctx ("" if none).  The pointer stays valid
 * until the next call on ctx.  ctx may be NULL (returns a static string). */
const char* tabit_last_error(const tabit_ctx* ctx);

/* Library version string, e.g. "tabit 0.1.0 gfx950". */
const char* tabit_version(void);

/*
 * Offline weight preparation into the single shared buffer.
 * TASQ section 2 (shared weight representation): one maximum-precision copy.
 * HQ-DM section 2.1: the block Hadamard; the same block size must be used for
 * the activations (the weights are rotated here so that both operands of the
 * INT8 product are integer codes; (XH)(WH)^T = b X W^T, so w_scale carries 1/b).
 *
 * Per output row n: y = blockFWHT_b(W[n, :]) in fp32 (stages h = 1, 2, 4, ...),
 * a = max|y|, codes = clamp(rint(y * (127/a)), -127, 127),
 * w_scale[n] = (a / 127) / max(b, 1).  A zero row gives codes 0, scale 0.
 *   w_bf16  device [N][K] bf16 input.
 *   w_q     device [N][K] int8 output, w_scale device [N] fp32 output.
 *   w_fp4   device [N][K/2] packed MXFP4 output (element 2i low nibble),
 *   w_e8m0  device [N][K/32] E8M0 output; the MX copy for layers scheduled to
 *           4 bits (6Bit-Diffusion section 2A).  Requires had_block in {0, 32}.
 * Either pair may be NULL (both members of a pair together); not both pairs.
 */
int tabit_quantize_weights(tabit_ctx* ctx, const uint16_t* w_bf16, int N, int K, int had_block,
                           int8_t* w_q, float* w_scale, uint8_t* w_fp4, uint8_t* w_e8m0,
                           void* stream);

/*
 * Install the per-(step, layer) precision table (host copy into ctx).
 * TASQ section 2: the Temporal-Spatial LSB mask M_{t,l} gives each layer and
 * denoising stage its number k of truncated LSBs.  6Bit-Diffusion section 2A:
 * INT8 or 4-bit chosen per layer and step.
 *   k_bits  host [num_steps][num_layers], each in [0, 7] (effective bits 8 - k).
 *   fmt     host [num_steps][num_layers] of TABIT_FMT_*, or NULL for all INT8.
 * Makes no HIP call.  Errors: EINVAL (null / bad fmt), ERANGE (k > 7),
 * ESHAPE (num_steps or num_layers < 1).
 */
int tabit_set_step_schedule(tabit_ctx* ctx, int num_steps, int num_layers,
                            const uint8_t* k_bits, const uint8_t* fmt);

/* Look up (k, fmt) for one (step, layer) of the installed table: the mask
 * M_{t,l} that TASQ section 2 learns per layer and denoising stage (k truncated
 * LSBs), and the INT8 / 4-bit choice 6Bit-Diffusion section 2A makes per layer
 * and step.  ENOSCHED when no table is installed or the pair is outside it.
 * Makes no HIP call. */
int tabit_schedule_lookup(const tabit_ctx* ctx, int step, int layer, int* k_bits, int* fmt);

/*
 * Activation quantizer: fused block FWHT + per-token quantization.
 * HQ-DM section 2.1 (X H, then quantize; unnormalized Hadamard) and section
 * 2.2 (symmetric); 6Bit-Diffusion section 2A (local block Hadamard first).
 *   fmt = TABIT_FMT_INT8:  per token m, y = blockFWHT_b(x_m) (fp32),
 *       a = max|y|, x_q int8 [M][K] = clamp(rint(y * (127/a)), -127, 127),
 *       x_scale fp32 [M] = a / 127 (0 for a zero row).
 *   fmt = TABIT_FMT_MXFP4 (had_block 0 or 32): per block of 32, X =
 *       clamp(floor(log2 amax) - 2, -127, 127); x_scale = uint8 E8M0 [M][K/32]
 *       holding X + 127 (127 for a zero block); x_q = packed E2M1 [M][K/2] of
 *       y * 2^-X, round to nearest even, saturating at 6.
 *   x_bf16 device [M][K].  Outputs device, caller-owned.
 */
int tabit_hadamard_quant_act(tabit_ctx* ctx, const uint16_t* x_bf16, int M, int K, int had_block,
                             int fmt, void* x_q, void* x_scale, void* stream);

/*
 * Masked W8A8 GEMM.  TASQ section 2: the operational weight at (step, layer)
 * is the stored code with its k least-significant bits truncated,
 * Q_M = (W >> k) << k (two's complement), applied to weight tiles as they are
 * staged; the same kernel serves every k (k is a scalar argument).
 *   acc[m][n] = sum_k x_q[m][k] * ((w_q[n][k] >> k_bits) << k_bits)   (int32, exact)
 *   y[m][n]   = bf16_rne(((float)acc[m][n] * x_scale[m]) * w_scale[n])
 * HQ-DM section 2.1: integer core, fp scales outside it.
 *   x_q device int8 [M][K], x_scale fp32 [M], w_q int8 [N][K], w_scale fp32 [N].
 *   y_bf16 device [M][N] (may be NULL), acc device int32 [M][N] (may be NULL);
 *   at least one output.  k_bits in [0, 7].
 */
int tabit_masked_qgemm(tabit_ctx* ctx, const int8_t* x_q, const float* x_scale,
                       const int8_t* w_q, const float* w_scale, int M, int N, int K, int k_bits,
                       uint16_t* y_bf16, int32_t* acc, void* stream);

/*
 * Bit-plane (bit-serial) GEMM over the 8 - k retained weight planes.
 * TASQ section 2 (Temporal-Precision Engine): in a bit-serial GEMM, cycles
 * scale with the weight bit width; activations stay resident and only the
 * selected weight planes are streamed.  Here the INT8 activation fragment is
 * loaded once per K-tile and multiplied against each retained plane:
 *   acc = sum_{b = k_bits}^{7} c_b * (x_q . W_b^T),  W_b = bit b of w_q,
 *   c_b = 2^b (b < 7), -2^7 (sign plane).  Equals tabit_masked_qgemm exactly.
 * Same arguments, layouts and errors as tabit_masked_qgemm.
 */
int tabit_qgemm_bitserial(tabit_ctx* ctx, const int8_t* x_q, const float* x_scale,
                          const int8_t* w_q, const float* w_scale, int M, int N, int K, int k_bits,
                          uint16_t* y_bf16, int32_t* acc, void* stream);

/*
 * Plane-major copy of the shared INT8 buffer.  TASQ section 2 (Temporal-
 * Precision Engine): only the weight bit-planes a layer-step keeps are
 * streamed (plane fetches 2LR -> L + R).  Stored plane by plane, a step with
 * mask k reads (8 - k)/8 of the buffer; the copy has the same size as w_q
 * (N * K bytes) and replaces it for tabit_plane_qgemm.
 *   w_q       device int8 [N][K] (from tabit_quantize_weights).
 *   w_planes  device uint32 [8][S][N][4], S = ceil(K/128), output
 *             (tabit_weight_planes_bytes(N, K) bytes, 16-byte aligned): word
 *             [b][s][n][j] holds bit b of the 32 codes w_q[n][128s + 32j + i],
 *             code i = 4u + q (u = 0..7, q = 0..3) at bit 8q + u; words past K
 *             are zero.  A plane's 128-code K-stage is 16 bytes per row.
 * Errors: EINVAL (null), ESHAPE (N % 32, K % 32, K range, size), EALIGN.
 */
int tabit_pack_weight_planes(tabit_ctx* ctx, const int8_t* w_q, int N, int K, uint32_t* w_planes,
                             void* stream);

/* Bytes of the plane-major copy of an N x K buffer: 128 * ceil(K/128) * N
 * (N * K when K % 128 == 0).  0 for N or K <= 0.  Makes no HIP call. */
size_t tabit_weight_planes_bytes(int N, int K);

/*
 * Masked W8A8 GEMM reading the plane-major weights: only planes b = k_bits..7
 * are fetched; each 16-byte weight fragment is rebuilt on chip as
 * sum_{b >= k} c_b * bit_b = (w >> k) << k (TASQ section 2), so the results
 * equal tabit_masked_qgemm bit for bit (acc exact, y by the same epilogue).
 * Same arguments, layouts and errors as tabit_masked_qgemm, with w_planes
 * from tabit_pack_weight_planes in place of w_q.
 */
int tabit_plane_qgemm(tabit_ctx* ctx, const int8_t* x_q, const float* x_scale,
                      const uint32_t* w_planes, const float* w_scale, int M, int N, int K,
                      int k_bits, uint16_t* y_bf16, int32_t* acc, void* stream);

/*
 * Producer-fused quantizer for the MLP down projection: the MLP's activation
 * (GELU, tanh form -- the pages fix none; the DiT convention) is applied while
 * the down projection's input is quantized, so the 4H-wide activation is read
 * once and never written in bf16.  Per element g = bf16_rne(gelu(x)) with
 *   gelu(x) = 0.5 x (1 + tanh(u)) = x / (1 + exp(-2u)),
 *   u = sqrt(2/pi) (x + 0.044715 x^3),
 * magnitudes below 2^-100 taken as 0; then exactly tabit_hadamard_quant_act on
 * g in the format `fmt` (INT8, or MXFP4 with had_block 0 or 32 for layer-steps
 * scheduled to 4 bits; 6Bit-Diffusion section 2A).  GELU is evaluated in fp32
 * with the hardware exp2 and reciprocal: within 16 ulp (x >= 0) or
 * (16|2u| + 24) ulp (x < 0) of the exact value (ulp = 2^-24 relative), so g is
 * the correctly rounded bf16 of the exact GELU except where that lies within
 * this bound of a rounding boundary.
 *   x_bf16 device [M][K] (the up projection's output); x_q and x_scale as
 *   tabit_hadamard_quant_act for `fmt`.  Errors as tabit_hadamard_quant_act.
 */
int tabit_gelu_quant_act(tabit_ctx* ctx, const uint16_t* x_bf16, int M, int K, int had_block,
                         int fmt, void* x_q, void* x_scale, void* stream);

/*
 * HQ-DM single-Hadamard activation quantizer (HQ-DM section 2.1: only the
 * activations are rotated; inference recovers X_hat = S (XH)_int H, the
 * Hadamard normalization living in the fp scale).  Per token m: codes q of
 * blockFWHT_b(x_m) exactly as tabit_hadamard_quant_act (INT8), then
 * Z = blockFWHT_b(q) (integers, |Z| <= 127 b), written as two planes
 * Z = 128 * x_hi + x_lo (x_hi = floor(Z / 128), x_lo in [0, 127]);
 * x_scale[m] = (a / 127) / max(b, 1), so X ~ x_scale * Z.
 *   x_bf16 device [M][K]; x_hi, x_lo device int8 [M][K]; x_scale fp32 [M].
 */
int tabit_hqdm_quant_act(tabit_ctx* ctx, const uint16_t* x_bf16, int M, int K, int had_block,
                         int8_t* x_hi, int8_t* x_lo, float* x_scale, void* stream);

/*
 * HQ-DM single-Hadamard GEMM against the untransformed weights (quantized with
 * had_block = 0), with the TASQ LSB mask (TASQ section 2):
 *   acc[m][n] = sum_k Z[m][k] * ((w_q[n][k] >> k_bits) << k_bits),
 *               Z = 128 x_hi + x_lo, computed as two INT8 products (exact)
 *   y[m][n]   = bf16_rne(((float)acc[m][n] * x_scale[m]) * w_scale[n])
 *   acc device int64 [M][N] (may be NULL), y_bf16 device [M][N] (may be NULL),
 *   at least one.  Other arguments, layouts and errors as tabit_masked_qgemm.
 * tabit_scheduled_linear / tabit_run_schedule run this pair for INT8 steps
 * with path = TABIT_PATH_HQDM (w_q then holds unrotated codes).
 */
int tabit_hqdm_qgemm(tabit_ctx* ctx, const int8_t* x_hi, const int8_t* x_lo, const float* x_scale,
                     const int8_t* w_q, const float* w_scale, int M, int N, int K, int k_bits,
                     uint16_t* y_bf16, int64_t* acc, void* stream);

/*
 * MXFP4 (W4A4) GEMM for layer-steps scheduled to 4 bits (6Bit-Diffusion
 * section 2A).  acc[m][n] = sum over 32-blocks j of 2^(xe[m][j] + we[n][j] - 254)
 * * sum_i e2m1(x)*e2m1(w), accumulated in fp32 by the scaled matrix cores
 * (order hardware-defined); y = bf16_rne(acc * out_scale).  With both operands
 * rotated by H_32, out_scale = 1/32.
 *   x_fp4 [M][K/2], x_e8m0 [M][K/32], w_fp4 [N][K/2], w_e8m0 [N][K/32] device.
 *   y_bf16 [M][N] and/or acc_f32 [M][N] device outputs (at least one).
 */
int tabit_mxfp4_qgemm(tabit_ctx* ctx, const uint8_t* x_fp4, const uint8_t* x_e8m0,
                      const uint8_t* w_fp4, const uint8_t* w_e8m0, int M, int N, int K,
                      float out_scale, uint16_t* y_bf16, float* acc_f32, void* stream);

/* Bytes of device workspace tabit_scheduled_linear needs for M x K activations
 * (quantized codes -- two int8 planes on the HQ-DM path -- plus scales, any
 * format). */
size_t tabit_act_workspace_bytes(int M, int K);

/*
 * One linear at denoising step `step`, layer `layer` (the per-step driver).
 * TASQ section 2 / abstract: the learned schedule maps to execution with no
 * switching overhead -- here a switch is one table lookup and a scalar kernel
 * argument.  Looks up (k, fmt); INT8: quantizes x into act_ws and runs the
 * masked GEMM (path = TABIT_PATH_MASKED), the bit-plane GEMM
 * (TABIT_PATH_BITSERIAL), the plane-major GEMM (TABIT_PATH_PLANES: w_q then
 * points at the words of tabit_pack_weight_planes) or HQ-DM's single-Hadamard
 * pair (TABIT_PATH_HQDM: tabit_hqdm_quant_act + tabit_hqdm_qgemm, w_q holding
 * unrotated codes) with k; MXFP4: MX-quantizes x and runs the MXFP4 GEMM
 * with out_scale 1/max(had_block, 1).
 *   w_q/w_scale required for INT8 steps, w_fp4/w_e8m0 for MXFP4 steps.
 *   act_ws device workspace of at least tabit_act_workspace_bytes(M, K),
 *   16-byte aligned.  y_bf16 device [M][N].
 */
int tabit_scheduled_linear(tabit_ctx* ctx, int step, int layer, int path,
                           const uint16_t* x_bf16, int M, int N, int K, int had_block,
                           const int8_t* w_q, const float* w_scale,
                           const uint8_t* w_fp4, const uint8_t* w_e8m0,
                           void* act_ws, size_t act_ws_bytes, uint16_t* y_bf16, void* stream);

/*
 * tabit_scheduled_linear for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same lookup, quantizer and GEMM, with the quantized
 * activations in a static device array owned by the library instead of a
 * caller workspace.  Nothing is allocated, freed or memset.  The array holds
 * tabit_noalloc_scratch_bytes() = 64 MiB per GPU (loaded with the library's
 * code object, kept until the process ends); a call needs
 *   INT8 (masked, bit-plane, plane-major): align256(M*K) + align256(4*M),
 *   INT8 on TABIT_PATH_HQDM:               2*align256(M*K) + align256(4*M),
 *   MXFP4:                                 align256(M*K/2) + align256(M*K/32)
 * bytes (align256 rounds up to a multiple of 256) and is rejected with
 * TABIT_ESHAPE, before anything is enqueued, when that exceeds the array.
 * Every call on one GPU shares that GPU's array: calls whose work overlaps on
 * one GPU (different streams, or other threads) race and must be ordered by
 * the caller.  Every byte a call reads from the array is written earlier in
 * the same call.  Arguments and errors otherwise as tabit_scheduled_linear;
 * the results equal its results bit for bit.
 */
size_t tabit_noalloc_scratch_bytes(void);
int tabit_scheduled_linear_noalloc(tabit_ctx* ctx, int step, int layer, int path,
                                   const uint16_t* x_bf16, int M, int N, int K, int had_block,
                                   const int8_t* w_q, const float* w_scale,
                                   const uint8_t* w_fp4, const uint8_t* w_e8m0,
                                   uint16_t* y_bf16, void* stream);

/*
 * DMPQ online format selection (6Bit-Diffusion section 2A): the relative L1
 * input-output change of a transformer block at step t-1 predicts, linearly,
 * the quantization sensitivity of its linear layers at step t; unstable
 * blocks keep INT8, stable ones go to 4 bits.  The page gives no predictor
 * coefficients or threshold, so the rule is a per-layer threshold:
 *   Gamma  = sum |x_out - x_in| / sum |x_in|   (0 if both sums are 0, +inf if
 *            only sum |x_in| is)
 *   fmt[l] = Gamma > theta[l] ? TABIT_FMT_INT8 : TABIT_FMT_MXFP4
 * The sums run in fp64 (terms |x_in| and |x_out - x_in| in fp64) in a fixed
 * order, so a given input always gives the same Gamma; each sum of n terms is
 * within (n - 1) 2^-53 of the exact sum (relative), so Gamma is within twice
 * that (plus the division's rounding) of the exact ratio, and a decision can
 * differ from the exact one only when Gamma is that close to theta[l].
 * Written on the device: a captured step needs no host round trip; the next
 * step's tabit_gated_linear calls read fmt.
 *   x_in, x_out  device bf16 [M][H] (block input and output at step t-1),
 *                H % 16 == 0, 16 <= H <= 32768, 16-byte aligned.
 *   theta        device fp32 [n_layers]; fmt device uint8 [n_layers] output
 *                (both may be NULL when n_layers == 0).
 *   gamma        device fp64 [1] output (may be NULL if n_layers > 0).
 *   ws           device workspace of tabit_dmpq_workspace_bytes(M) bytes.
 */
size_t tabit_dmpq_workspace_bytes(int M);
int tabit_dmpq_select(tabit_ctx* ctx, const uint16_t* x_in, const uint16_t* x_out, int M, int H,
                      const float* theta, int n_layers, uint8_t* fmt, double* gamma, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * One linear whose format is read on the device (6Bit-Diffusion section 2A
 * with the table from tabit_dmpq_select): enqueues the INT8 branch (quantizer
 * + masked GEMM with k_bits, or the plane-major GEMM when path =
 * TABIT_PATH_PLANES and w_q holds the plane words) and the MXFP4 branch
 * (MX quantizer + MXFP4 GEMM with out_scale 1/max(had_block, 1)); every kernel
 * first reads *fmt_dev and returns at once unless it is its own format, so
 * exactly one branch does work and no host synchronization is needed.
 *   fmt_dev  device uint8 (TABIT_FMT_*).  Both weight formats are required;
 *   had_block in {0, 32}.  Other arguments as tabit_scheduled_linear.
 */
int tabit_gated_linear(tabit_ctx* ctx, const uint8_t* fmt_dev, int k_bits, int path,
                       const uint16_t* x_bf16, int M, int N, int K, int had_block,
                       const void* w_q, const float* w_scale, const uint8_t* w_fp4,
                       const uint8_t* w_e8m0, void* act_ws, size_t act_ws_bytes, uint16_t* y_bf16,
                       void* stream);

/* Activation applied to a layer's input inside its quantizer (tabit_layer). */
enum tabit_act { TABIT_ACT_NONE = 0, TABIT_ACT_GELU = 1 };

/* One linear layer of a stack, for tabit_run_schedule. */
typedef struct tabit_layer {
  int M, N, K;               /* tokens, output and input features                     */
  const int8_t* w_q;         /* device [N][K] INT8 codes (NULL if never INT8); with   */
                             /* TABIT_PATH_PLANES the plane-major words instead       */
  const float* w_scale;      /* device [N]                                            */
  const uint8_t* w_fp4;      /* device [N][K/2] MXFP4 copy (NULL if never MXFP4)      */
  const uint8_t* w_e8m0;     /* device [N][K/32]                                      */
  uint16_t* y_bf16;          /* device [M][N] output                                  */
  int input_from;            /* 0: the input is x_bf16[step][layer]; j + 1: the       */
                             /* output y_bf16 of layer j (< this layer) of the same   */
                             /* step, e.g. the MLP's up projection for its down one   */
  int input_act;             /* TABIT_ACT_NONE, or TABIT_ACT_GELU: the quantizer      */
                             /* applies GELU first (tabit_gelu_quant_act); not on     */
                             /* TABIT_PATH_HQDM                                       */
} tabit_layer;

/*
 * Run steps [first_step, first_step + num_steps) of the installed schedule over
 * a stack of layers: for each step t, for each layer l, the same work as
 * tabit_scheduled_linear(t, l, ...) (TASQ section 2: the per-(layer, stage)
 * precision is applied by reading the table, with no weight copy).
 *   x_bf16      host array [num_steps][num_layers] of device pointers to the
 *               layer inputs ([M][K] bf16 each); ignored (may be NULL) for
 *               layers whose input_from names an earlier layer.  A chained
 *               layer reads that layer's y_bf16 of the same step, through the
 *               GELU-fused quantizer when input_act = TABIT_ACT_GELU (the MLP:
 *               up projection -> GELU -> down projection).
 *   gemm_events NULL, or a host array of 2 * num_steps * num_layers hipEvent_t
 *               (passed as void*): events[2i] and events[2i+1] become the start
 *               and stop events of the GEMM dispatch of layer-step i
 *               (hipExtLaunchKernel), stamped with that kernel's own start and
 *               end, so a caller can time the GEMM kernels alone.
 *   num_layers must equal the schedule's layer count.  Validation covers every
 *   layer before the first launch.
 */
int tabit_run_schedule(tabit_ctx* ctx, int first_step, int num_steps, const tabit_layer* layers,
                       int num_layers, const uint16_t* const* x_bf16, int had_block, int path,
                       void* act_ws, size_t act_ws_bytes, void* const* gemm_events, void* stream);

/*
 * Autotune the tile configuration for one GEMM problem: time every
 * configuration of the GEMM `path` (TABIT_PATH_MASKED, TABIT_PATH_BITSERIAL,
 * 2 for the MXFP4 GEMM, TABIT_PATH_PLANES) on the caller's buffers, `reps` launches each, and
 * remember the fastest for (path, M, N, K) in ctx; later calls with that shape
 * on that path use it (an explicit TABIT_OPT_*_CONFIG still wins).  The
 * buffers follow the layouts of tabit_masked_qgemm (path 0/1: x_q int8,
 * x_scale fp32, w_q int8, w_scale fp32), tabit_mxfp4_qgemm (path 2: x_fp4,
 * x_e8m0, w_fp4, w_e8m0) or tabit_plane_qgemm (path 3: w_q = the plane-major
 * words); y_bf16 [M][N] receives scratch results.
 * Synchronizes `stream` to read the timings: call it outside graph capture,
 * e.g. during warm-up.  *best_cfg (may be NULL) receives the winner.
 */
int tabit_autotune_gemm(tabit_ctx* ctx, int path, const void* x_q, const void* x_scale,
                        const void* w_q, const void* w_scale, int M, int N, int K, int k_bits,
                        uint16_t* y_bf16, int reps, int* best_cfg, void* stream);

/*
 * Options (tests and tuning).  TABIT_OPT_GEMM_CONFIG forces the INT8 GEMM tile
 * configuration (value = index from tabit_gemm_config_info, -1 = automatic);
 * TABIT_OPT_MXFP4_CONFIG, TABIT_OPT_PLANE_CONFIG and TABIT_OPT_HQDM_CONFIG
 * likewise for the MXFP4, plane-major and HQ-DM GEMMs.  EINVAL for an unknown option or value.  Makes no HIP call.
 */
enum tabit_option {
  TABIT_OPT_GEMM_CONFIG = 0,
  TABIT_OPT_MXFP4_CONFIG = 1,
  TABIT_OPT_PLANE_CONFIG = 2,
  TABIT_OPT_HQDM_CONFIG = 3
};
int tabit_set_option(tabit_ctx* ctx, int option, int value);

/* Describe INT8 GEMM tile configuration `index` (0 <= index < count): block
 * tile BM x BN and, in *k_groups, the number of wave groups that split the K
 * stages of one tile inside its workgroup (1 = no split; the groups' int32
 * sums are added exactly, so every configuration gives the same result; the
 * automatic choice, tabit_gemm_config_choose, takes a split tile only when the
 * one-group tile leaves at least half of the CUs idle).  Returns the number of
 * configurations when index < 0.  Makes no HIP call. */
int tabit_gemm_config_info(int index, int* bm, int* bn, int* k_groups);

/* As tabit_gemm_config_info, for the MXFP4 GEMM's tile configurations. */
int tabit_mxfp4_config_info(int index, int* bm, int* bn);

/* The MXFP4 GEMM configuration the library picks for M x N x K on a device
 * with num_cus compute units (<= 0: 256) when neither an option nor tuning
 * forces one: the busiest-CU model (ceil(tiles / CUs) x tile area / the tile's
 * measured rate); tiles whose variant for K not a multiple of 128 spills are
 * left out for such K.  EINVAL for negative sizes or K < 1.  Makes no HIP
 * call. */
int tabit_mxfp4_config_choose(int M, int N, int K, int num_cus);

/* As tabit_mxfp4_config_info, for the plane-major GEMM's tile configurations;
 * *k_groups (may be NULL) receives the number of wave groups that split the K
 * stages of one tile inside its workgroup (1 = no split; the groups' int32
 * sums are added exactly, so every configuration gives the same result). */
int tabit_plane_config_info(int index, int* bm, int* bn, int* k_groups);

/* The plane-major GEMM configuration the library picks for M x N x K on a
 * device with num_cus compute units (<= 0: 256) when neither an option nor
 * tuning forces one: the busiest-CU model over one-group tiles, then, when
 * that tile leaves at least half of the CUs idle, its K-split variant with the
 * fewest stages per group.  EINVAL for negative sizes or K < 1.  Makes no HIP
 * call. */
int tabit_plane_config_choose(int M, int N, int K, int num_cus);

/* As tabit_mxfp4_config_info, for the HQ-DM GEMM's tile configurations. */
int tabit_hqdm_config_info(int index, int* bm, int* bn);

/*
 * Sustained matrix-core rate of the current device at its running clock (the
 * measured side of the roofline beside the published peak): every CU runs four
 * workgroups of four waves, each wave `iters` rounds of independent MFMA
 * chains on register operands, with no memory traffic in the loop.
 *   kind   0: v_mfma_i32_32x32x32_i8 (INT8 ops), 1: the FP4 block-scaled
 *          32x32x64 MFMA (FP4 flops).
 *   iters  rounds per wave, 1 .. 2^24 (20000 runs for about 2 ms).
 *   sink   device int32 [tabit_mfma_probe_sink_ints(number of CUs)]: one word per
 *          thread keeps the chains live; its contents mean nothing.
 *   ops_per_s  host: operations per second of the launch, timed by its own
 *          start/stop events.
 * Enqueues on `stream` and synchronizes on the stop event: call it outside
 * graph capture.  EINVAL / ERANGE / ESHAPE for bad arguments, EHIP for a launch
 * error.
 */
int tabit_mfma_peak_probe(tabit_ctx* ctx, int kind, int iters, int32_t* sink, size_t sink_ints,
                          double* ops_per_s, void* stream);
size_t tabit_mfma_probe_sink_ints(int num_cus);

/* The configuration the automatic choice would take for (M, N, K) on a device
 * with num_cus compute units (num_cus <= 0: 256).  Makes no HIP call. */
int tabit_gemm_config_choose(int M, int N, int K, int num_cus);

#ifdef __cplusplus
}
#endif

#endif /* TABIT_H */
