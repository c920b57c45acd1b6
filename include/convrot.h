/*
 * convrot.h -- C ABI of the ConvRot / ConvLinear4bit (rotated W4A4 linear) library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow these pages (cited by title and section):
 *   [AUTHOR]  ComfyUI issue #14735, comment by the ConvRot author: group-wise rotation by a
 *             regular Hadamard matrix over non-overlapping windows whose size is a power of 4
 *             (16, 64, 256, 1024), with zero padding when K is not a multiple of the window.
 *   [PAPER]   "ConvRot: Rotation-Based Plug-and-Play 4-bit Quantization for Diffusion
 *             Transformers" (arXiv 2512.03673): Abstract (ConvLinear4bit = rotation,
 *             quantization, GEMM, dequantization), Fig. 3 (RHT on non-overlapping windows),
 *             Def. 2.1 / 2.3 (Hadamard and regular Hadamard matrices), Thm. 2.3 (Kronecker
 *             construction).
 *   [HSWQ]    HSWQ v2.3.4 release notes, "Mathematical Formulation & Format Layout" ->
 *             "Hadamard Orthogonal Rotation": W_rot = W H^T, per-row scale = absmax / q_max,
 *             codes = round(W_rot / scale).
 *   [KITCHEN] comfy-kitchen PR #65 "Basic convrot int4 support", review comments: the
 *             integer-only power-of-4 size check and its error text; int4_linear, which
 *             unpacks row-major int4 operands, accumulates x @ w^T exactly, scales by the
 *             per-row x scale and per-column w scale, adds the bias and casts last.
 *
 * Conventions fixed by this library where the pages are silent:
 *   - H_g = H4 (x) ... (x) H4 (log4 g factors) with H4 = J - 2I (symmetric, regular, every row
 *     and column sums to +2); the rotation applied to each window is H_g / sqrt(g).
 *   - Windows start at column 0.  K' = ceil(K / g) * g; columns K..K'-1 are zero and take
 *     part in the rotation and in the GEMM (depth K').
 *   - int4 is symmetric: scale = absmax(rotated row) / 7 (IEEE fp32 division); code =
 *     clamp(round_half_even(rotated / scale), -8, 7); an all-zero row has scale 0, codes 0.
 *     The rotated value is the correctly rounded fp32 of the exact rotation; the row scale
 *     is computed from exact values and is bit-identical to that definition.  Codes are
 *     computed from an fp32 butterfly and may differ by one from the definition where the
 *     quotient lies within a few ulp of a rounding tie.
 *   - Packing: two codes per byte, code 2j in the low nibble of byte j, code 2j+1 in the
 *     high nibble, two's complement; each row is K'/2 bytes.
 *   - Output: y = bf16_rne( fp32( fp32( fp32(acc) * x_scale[m] ) * w_scale[n] ) + bias[n] ),
 *     acc = exact integer sum over K'.  Output is always bf16.
 *
 * Memory and threading:
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except the host buffer
 *     of convrot_make_rht.  The library never allocates, frees or retains device memory,
 *     except the fixed scratch array of convrot_w4a4_linear_noalloc (below), which the
 *     code object holds on each device it is loaded on.  Its other global state is per-device
 *     caches of the compute-unit count and of that array's address (atomic); every other
 *     call is re-entrant and may come from several host threads.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Device work is
 *     enqueued asynchronously on it; no call synchronises the device or the stream.  Every
 *     call enqueues kernel launches only (no memset, copy or allocation), so calls may be
 *     recorded by stream capture into a HIP graph and replayed.
 *   - Every call validates its arguments on the host first and returns a status; on error
 *     nothing is enqueued and no output is written.
 *   - Non-finite rows: the rotation runs as an fp32 butterfly whose stage sums reach up to
 *     2^(k+1) max|x| (k = log4 g), so inputs above FLT_MAX / 2^(k+1) (4.2e37 for g = 16,
 *     2.1e37, 1.1e37, 5.3e36 for g = 64, 256, 1024; 8.5e37 for rows of equal values) can
 *     overflow it.  A row whose butterfly overflows, or that holds a NaN or an Inf, gets a
 *     NaN scale (int4, int8) and unspecified codes, so a layer's output row is NaN; with
 *     MXFP4 codes, every block of a window holding a non-finite rotated value gets the
 *     E8M0 NaN byte 0xFF.  No such input yields a finite scale.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define CONVROT_API __attribute__((visibility("default")))
#else
#define CONVROT_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
    CONVROT_OK = 0,
    CONVROT_ERR_GROUP = -1,        /* g is not an integer power of 4 (>= 4) */
    CONVROT_ERR_UNSUPPORTED = -2,  /* a valid power of 4 or shape the kernels do not implement:
                                      g must be 16, 64, 256 or 1024; the rotate+quantize row
                                      K' must be at most 16384 (g = 16), 32768 (g = 64, 256)
                                      or 61440 (g = 1024; 32768 for fp32 input); the GEMM
                                      depth at most CONVROT_MAX_KP */
    CONVROT_ERR_SHAPE = -3,        /* M < 0, N < 0, K < 1, ld < K, or a size that overflows */
    CONVROT_ERR_NULL = -4,         /* a required pointer is NULL */
    CONVROT_ERR_DTYPE = -5,        /* unknown dtype code */
    CONVROT_ERR_ALIGN = -6,        /* a pointer or row stride violates the stated alignment */
    CONVROT_ERR_WORKSPACE = -7,    /* workspace smaller than convrot_w4a4_workspace_bytes() */
    CONVROT_ERR_HIP = -8,          /* the HIP runtime reported an error at launch */
    CONVROT_ERR_SCRATCH = -9       /* convrot_w4a4_linear_noalloc: the problem needs more than
                                      CONVROT_NOALLOC_SCRATCH_BYTES of scratch */
};

/* Element type of activation / weight inputs. */
enum { CONVROT_F32 = 0, CONVROT_BF16 = 1 };

/* Largest padded depth K' any kernel accepts (the GEMM; rotate+quantize rows: see above). */
#define CONVROT_MAX_KP 65536

/* Human-readable text of a status code (static storage; never NULL). */
CONVROT_API const char* convrot_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
CONVROT_API int convrot_version(void);

/* K' = ceil(K / g) * g ([AUTHOR]: padding inside the algorithm).
 * Returns K' >= g, or a negative status: CONVROT_ERR_GROUP if g is not a power of 4,
 * CONVROT_ERR_SHAPE if K < 1 or K' would overflow. */
CONVROT_API int64_t convrot_padded_k(int64_t K, int64_t g);

/* Integer-only power-of-4 test ([KITCHEN] review of the size check): 1 if g = 4^k, k >= 1,
 * else 0.  Accepts every 4^k up to 4^31 (e.g. 2^58 = 4^29). */
CONVROT_API int convrot_is_power_of_4(int64_t g);

/* Dense regular Hadamard matrix H_g = H4^(x)k, H4 = J - 2I ([PAPER] Def. 2.3, Thm. 2.3),
 * written row-major into the HOST buffer h[g*g] (fp32).  normalized = 0: entries +-1;
 * normalized != 0: entries +-1/sqrt(g) (exact powers of two).  For reference and tests;
 * the GPU path never materialises H.  Errors: CONVROT_ERR_GROUP, CONVROT_ERR_NULL,
 * CONVROT_ERR_UNSUPPORTED if g > 4096. */
CONVROT_API int convrot_make_rht(int64_t g, float* h, int32_t normalized);

/* Online activation path ([AUTHOR]; [PAPER] Abstract, Fig. 3): for each of the M rows of x
 * (row stride ldx elements), zero-pad to K', rotate every window of g columns by H_g/sqrt(g),
 * take the per-row absmax scale and quantize to int4.
 *   x        device, dtype x_dtype, [M][ldx] with ldx >= K; any alignment of the element type
 *   xq       device, uint8 [M][K'/2] packed codes (layout above); 16-byte aligned
 *   xs       device, fp32 [M] per-row scales; 4-byte aligned
 *   xrot     device, fp32 [M][K'] rotated activations, or NULL (debug output)
 * M = 0 is a no-op.  Errors: GROUP, UNSUPPORTED, SHAPE, NULL, DTYPE, ALIGN, HIP. */
CONVROT_API int convrot_rotate_quant_act(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                             int64_t g, uint8_t* xq, float* xs, float* xrot, void* stream);

/* Offline weight path ([HSWQ] "Hadamard Orthogonal Rotation", per output channel): the same
 * operation on the N rows of w [N][K] (row stride K): wq uint8 [N][K'/2] (16-byte aligned),
 * ws fp32 [N].  Called once per layer; not on the forward path. */
CONVROT_API int convrot_quant_weight(const void* w, int32_t w_dtype, int64_t N, int64_t K, int64_t g,
                         uint8_t* wq, float* ws, void* stream);

/* W4A4 GEMM with fused dequantization ([KITCHEN] int4_linear semantics; int8 matrix cores):
 *   y[m][n] = bf16( fp32(fp32(fp32(sum_k qx[m][k] qw[n][k]) * xs[m]) * ws[n]) + bias[n] )
 *   xq [M][Kp/2], wq [N][Kp/2] packed int4 (16-byte aligned), xs fp32 [M], ws fp32 [N],
 *   bias bf16 [N] or NULL, y bf16 [M][N] row-major (4-byte aligned).
 *   Kp must be a positive multiple of 16 and <= CONVROT_MAX_KP.
 *   acc_dbg: int32 [M][N] (16-byte aligned) or NULL; when set, the exact integer sums are
 *   written there as well (debug / bit-exactness checks).
 * M = 0 or N = 0 is a no-op.  Errors: SHAPE, NULL, ALIGN, UNSUPPORTED, HIP. */
CONVROT_API int convrot_w4a4_gemm(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                      const void* bias, int64_t M, int64_t N, int64_t Kp, void* y,
                      int32_t* acc_dbg, void* stream);

/* Bytes of device workspace convrot_w4a4_linear needs: packed codes M*K'/2 and scales 4*M,
 * each rounded up to 256 bytes.  Returns 0 for an invalid g or shape. */
CONVROT_API size_t convrot_w4a4_workspace_bytes(int64_t M, int64_t K, int64_t g);

/* The ConvLinear4bit forward pass ([PAPER] Abstract, Fig. 3): rotate + quantize x [M][K]
 * (row stride K, dtype x_dtype) into the workspace, then the W4A4 GEMM against the offline
 * weights wq [N][K'/2] / ws [N] (from convrot_quant_weight with the same g and K) with the
 * dequant epilogue, writing y bf16 [M][N].  bias bf16 [N] or NULL.  The workspace (device,
 * 256-byte aligned, ws_bytes >= convrot_w4a4_workspace_bytes(M, K, g)) holds the packed
 * activation codes and scales afterwards.  Two kernels are enqueued on `stream`.
 * M = 0 or N = 0 is a no-op.  Errors: GROUP, UNSUPPORTED, SHAPE, NULL, DTYPE, ALIGN,
 * WORKSPACE, HIP. */
CONVROT_API int convrot_w4a4_linear(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t g,
                        const uint8_t* wq, const float* ws, int64_t N, const void* bias,
                        void* y, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * INT8 variant (W8A8): the same group-wise regular rotation with 8-bit symmetric codes
 * ([HSWQ] "Hadamard Orthogonal Rotation": per-row scale = absmax / 127, codes =
 * round(rotated / scale); [AUTHOR]: the rotation is independent of the code format).
 * Codes are int8, one per element, row stride K' bytes; scale = fp32(absmax / 127) (exact
 * absmax, bit-identical to the definition); codes may differ by one from the definition
 * where the quotient lies within a few ulp of a rounding tie.  The sums are exact int32
 * (|acc| <= 16384 K' < 2^31); y = bf16( fp32( fp32( fp32(acc) * xs[m] ) * ws[n] ) + bias[n] ),
 * fp32(acc) rounding to nearest even once |acc| >= 2^24.
 * --------------------------------------------------------------------------------------- */

/* Online activation path, INT8 codes: as convrot_rotate_quant_act, with
 *   xq  device, int8 [M][K'] codes, 16-byte aligned.
 * K' limits as for int4 codes except: g = 1024 with bf16 input, K' <= 53248; fp32 input,
 * K' <= 30720 (g = 64, 256) or 28672 (g = 1024).  Each row's packed codes and raw input
 * windows are staged in the workgroup's LDS, and int8 codes take twice the room of int4.
 * M = 0 is a no-op.  Errors: GROUP, UNSUPPORTED, SHAPE, NULL, DTYPE, ALIGN, HIP. */
CONVROT_API int convrot_rotate_quant_act_i8(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                                int64_t ldx, int64_t g, int8_t* xq, float* xs, float* xrot,
                                void* stream);

/* Offline INT8 weight path: wq int8 [N][K'] (16-byte aligned), ws fp32 [N]. */
CONVROT_API int convrot_quant_weight_i8(const void* w, int32_t w_dtype, int64_t N, int64_t K,
                            int64_t g, int8_t* wq, float* ws, void* stream);

/* W8A8 GEMM with fused dequantization (int8 matrix cores, no unpacking):
 *   xq [M][Kp], wq [N][Kp] int8 (16-byte aligned), xs fp32 [M], ws fp32 [N], bias bf16 [N]
 *   or NULL, y bf16 [M][N] (4-byte aligned); Kp a positive multiple of 16, <= CONVROT_MAX_KP;
 *   acc_dbg int32 [M][N] (16-byte aligned) or NULL, as for convrot_w4a4_gemm.
 * M = 0 or N = 0 is a no-op.  Errors: SHAPE, NULL, ALIGN, UNSUPPORTED, HIP. */
CONVROT_API int convrot_w8a8_gemm(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws,
                      const void* bias, int64_t M, int64_t N, int64_t Kp, void* y,
                      int32_t* acc_dbg, void* stream);

/* Bytes of device workspace convrot_w8a8_linear needs: codes M*K' and scales 4*M, each
 * rounded up to 256 bytes.  Returns 0 for an invalid g or shape. */
CONVROT_API size_t convrot_w8a8_workspace_bytes(int64_t M, int64_t K, int64_t g);

/* The W8A8 forward pass: rotate + quantize x to int8 codes in the workspace, then the W8A8
 * GEMM against wq int8 [N][K'] / ws [N] (from convrot_quant_weight_i8 with the same g and K),
 * writing y bf16 [M][N].  Arguments and errors as for convrot_w4a4_linear. */
CONVROT_API int convrot_w8a8_linear(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t g,
                        const int8_t* wq, const float* ws, int64_t N, const void* bias,
                        void* y, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Floating-point 4-bit variant (MXFP4).  [AUTHOR]: ConvRot also suits floating-point
 * quantization; the pages fix no format, and this library reads it as MXFP4 of the OCP
 * Microscaling (MX) Specification v1.0, the format gfx950's scaled FP4 matrix instructions
 * take.  The same group-wise regular rotation, then every 32 consecutive rotated values of
 * a row share one E8M0 scale byte e = floor(log2(absmax)) - 2 + 127 (clamped to >= 0; an
 * all-zero block takes 0), and each value becomes the E2M1 code nearest to value / 2^(e-127),
 * ties to the even mantissa, magnitudes beyond 6 saturating at 6, the sign bit following the
 * value (-0.0 -> 0x8).  Codes: two per byte, value 2j in the low nibble, row stride K'/2
 * bytes; scales: K'/32 bytes per row in rows of S = 4 ceil(K'/128) bytes (S = K'/32 unless
 * g = 64; the padding bytes are written as 0).  The block maxima are those of the fp32 rotation:
 * a block's exponent may differ from the definition's only where its maximum lies within
 * the rotation's rounding error of a power of two, and a code only at a rounding tie.
 * g must be 64, 256 or 1024 (g = 16: UNSUPPORTED).
 * --------------------------------------------------------------------------------------- */

/* Online activation path, MXFP4: as convrot_rotate_quant_act, with
 *   xq   device, uint8 [M][K'/2] E2M1 codes, 16-byte aligned;
 *   xbs  device, uint8 [M][S] E8M0 block scales, S = 4 ceil(K'/128) (no alignment).
 * K' limits as for int4 codes.  M = 0 is a no-op.
 * Errors: GROUP, UNSUPPORTED, SHAPE, NULL, DTYPE, ALIGN, HIP. */
CONVROT_API int convrot_rotate_quant_act_mxfp4(const void* x, int32_t x_dtype, int64_t M,
                                               int64_t K, int64_t ldx, int64_t g, uint8_t* xq,
                                               uint8_t* xbs, float* xrot, void* stream);

/* Offline MXFP4 weight path: wq uint8 [N][K'/2] (16-byte aligned), wbs uint8 [N][S]. */
CONVROT_API int convrot_quant_weight_mxfp4(const void* w, int32_t w_dtype, int64_t N, int64_t K,
                                           int64_t g, uint8_t* wq, uint8_t* wbs, void* stream);

/* MXFP4 GEMM (gfx950's scaled FP4 matrix instructions, fp32 accumulation):
 *   y[m][n] = bf16( fp32( sum_k x[m][k] w[n][k] ) + bias[n] ), x and w the decoded values
 *   (E2M1 code * 2^(E8M0 - 127) of its block).
 *   xq [M][Kp/2], wq [N][Kp/2] packed codes (16-byte aligned); xbs [M][S], wbs [N][S] E8M0
 *   bytes, S = 4 ceil(Kp/128) (4-byte aligned); bias bf16 [N] or NULL; y bf16 [M][N] (4-byte
 *   aligned); Kp a positive multiple of 64, <= CONVROT_MAX_KP; acc_dbg fp32 [M][N] (16-byte
 *   aligned) receives the sums before the bias, or NULL.
 * The order in which the products are added is not specified: the sum carries fp32 rounding
 * of at most about Kp/64 + 16 roundings of partial sums, not an exact result (for M <= 256 the
 * K range is split over up to 16 waves whose partial sums are added last).
 * M = 0 or N = 0 is a no-op.  Errors: SHAPE, NULL, ALIGN, UNSUPPORTED, HIP. */
CONVROT_API int convrot_mxfp4_gemm(const uint8_t* xq, const uint8_t* xbs, const uint8_t* wq,
                                   const uint8_t* wbs, const void* bias, int64_t M, int64_t N,
                                   int64_t Kp, void* y, float* acc_dbg, void* stream);

/* Bytes of device workspace convrot_mxfp4_linear needs: codes M*K'/2 and scales M*S, each
 * rounded up to 256 bytes.  Returns 0 for an invalid or unsupported g or shape. */
CONVROT_API size_t convrot_mxfp4_workspace_bytes(int64_t M, int64_t K, int64_t g);

/* The MXFP4 forward pass: rotate + quantize x to MXFP4 in the workspace, then the MXFP4 GEMM
 * against wq / wbs (from convrot_quant_weight_mxfp4 with the same g and K), writing y bf16
 * [M][N].  Arguments and errors as for convrot_w4a4_linear; g = 16 is UNSUPPORTED. */
CONVROT_API int convrot_mxfp4_linear(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                                     int64_t g, const uint8_t* wq, const uint8_t* wbs, int64_t N,
                                     const void* bias, void* y, void* workspace, size_t ws_bytes,
                                     void* stream);

/* The ConvLinear4bit forward pass in ONE kernel launch ([PAPER] Abstract: the module
 * integrates rotation, quantization, GEMM and dequantization): a persistent grid of one
 * workgroup per compute unit rotates and quantizes x into the workspace, meets at a grid
 * barrier, then runs the GEMM tiles.  Arguments, workspace layout and results as for
 * convrot_w4a4_linear (codes, scales and y bit-identical to it), plus
 *   status   device, uint32, 4-byte aligned; must be 0 on entry.  The kernel sets it to a
 *            nonzero value if its grid barrier waited 2^20 polls (of the order of a second) (all
 *            workgroups must be resident at once: another kernel holding compute units can
 *            delay them); y is then incomplete.  Read it after the stream has finished.
 * Supported: bf16 x, g = 256 or 1024, K'/2 a multiple of 16 bytes, K even, and one row
 * within eight waves (K' <= 16384 for g = 256, 32768 for g = 1024); otherwise
 * CONVROT_ERR_UNSUPPORTED before anything is enqueued.  The barrier keeps its counter in device
 * memory of the library, one per device: calls that overlap in time on one device must be
 * serialised by the caller.
 * Speed: on the attention-projection, MLP down-projection and proj_out layers it takes
 * 1.15-1.7x the time of convrot_w4a4_linear, since its rotation phase runs at the GEMM's
 * occupancy (two waves per SIMD) instead of the rotate kernel's; the two-launch path stays
 * the default and this entry point is the measured alternative.
 * Errors: as convrot_w4a4_linear, and UNSUPPORTED for the cases above. */
CONVROT_API int convrot_w4a4_linear_fused(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                                          int64_t g, const uint8_t* wq, const float* ws,
                                          int64_t N, const void* bias, void* y, void* workspace,
                                          size_t ws_bytes, uint32_t* status, void* stream);

/* ---------------------------------------------------------------------------------------
 * Analysis helpers, not on the layer's path: the int4 quantization rule of a3-a4 applied to
 * rows that are already transformed (no rotation), and the inverse mapping of packed codes.
 * The outlier-suppression tool uses them to quantize its comparison transforms (none,
 * Sylvester-type Hadamard) by the same rule as the layer ([HSWQ] "Hadamard Orthogonal
 * Rotation": per-row scale = max|row| / q_max, code = round(value / scale), here with q_max = 7,
 * round half to even, codes clamped to [-8, 7]; [KITCHEN]: two codes per byte, column 2j in
 * the low nibble).  Device pointers, owned by the caller; calls enqueue on `stream`.
 *
 * convrot_quant_rows_int4: y fp32 [M][ldy] (ldy >= K elements; y 4-byte aligned) ->
 *   q [M][(K + 1) / 2] packed codes (an odd K leaves a zero code in each row's last high
 *   nibble) and s [M] fp32 (4-byte aligned): s = fp32(max_k |y[m][k]| / 7) by IEEE division,
 *   code = clamp(rne(fp32(y / s)), -8, 7), all codes 0 where s == 0.  Rows holding NaN give
 *   unspecified codes.  Errors: NULL, SHAPE (M < 0, M >= 2^31, K < 1, ldy < K), ALIGN, HIP. */
CONVROT_API int convrot_quant_rows_int4(const float* y, int64_t M, int64_t K, int64_t ldy,
                                        uint8_t* q, float* s, void* stream);

/* convrot_dequant_int4: q [M][(K + 1) / 2] packed codes as above, s [M] fp32 (4-byte aligned)
 *   -> out fp64 [M][K] (8-byte aligned), out = code * s, exact.  Errors: NULL, SHAPE (M < 0,
 *   K < 1, M * K >= 2^40), ALIGN, HIP. */
CONVROT_API int convrot_dequant_int4(const uint8_t* q, const float* s, int64_t M, int64_t K,
                                     double* out, void* stream);

/* ---------------------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the ConvLinear4bit forward pass of
 * convrot_w4a4_linear without a workspace argument.  The packed activation codes and row
 * scales go to a fixed array of CONVROT_NOALLOC_SCRATCH_BYTES (72 MiB) of device memory inside
 * the library, one per device, held from the library's first use on that device until the
 * process ends.  The call allocates and frees nothing (no hipMalloc, no library routine that
 * allocates); the caller passes inputs and outputs as for convrot_w4a4_linear.
 *   Limit: convrot_w4a4_workspace_bytes(M, K, g) <= CONVROT_NOALLOC_SCRATCH_BYTES, else
 *   CONVROT_ERR_SCRATCH before anything is enqueued (e.g. K = 3072, g = 256: M <= 49024).
 *   Every call on one device shares that device's array, which keeps the last call's codes:
 *   calls that may overlap in time on one device (several streams, several host threads
 *   without ordering) race on it and must be serialised by the caller.  Output is identical
 *   to convrot_w4a4_linear's (the same kernels).
 * Errors: as convrot_w4a4_linear, with CONVROT_ERR_SCRATCH in place of CONVROT_ERR_WORKSPACE. */
#define CONVROT_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)

CONVROT_API int convrot_w4a4_linear_noalloc(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                                            int64_t g, const uint8_t* wq, const float* ws,
                                            int64_t N, const void* bias, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
