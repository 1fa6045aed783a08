/*
 * fp8q -- fine-grained FP8 (E4M3) quantization and block-scaled FP8 GEMMs
 * for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The method (DeepSeek-V3 FP8 mixed-precision training, as described on the
 * pages cited below):
 *   - activations are quantized per 1x128 tile (per token per 128 channels)
 *     and weights per 128x128 block, each tile/block scaled from its own
 *     max-abs, computed online;  [dssusan.co.kr FP8 excerpt, paragraphs 2
 *     and 4; youlimart.com FP8 excerpt, paragraph 1; "FP8 mixed precision -
 *     где и как DeepSeek снизили точность вычислений?", section "Точечное
 *     (fine-grained) квантование"]
 *   - the max-abs is mapped onto the largest E4M3 value (448);  ["Deepseek -
 *     Not For everyone", paragraph 3]
 *   - some scales are integral powers of two;  [dssusan.co.kr, paragraph 1]
 *   - for the backward pass activations are re-tiled 128x1 (along tokens);
 *     [dssusan.co.kr, paragraph 4]
 *   - GEMMs take per-group scales along the inner dimension K, multiply them
 *     in as dequantization and promote partial products to FP32 accumulation;
 *     [dssusan.co.kr, paragraph 3; "Deepseek - Not For everyone", paragraph 4]
 *   - Fprop, Dgrad and Wgrad all run in FP8 and write BF16 or FP32.
 *     [youlimart.com FP8 excerpt, paragraphs 2 and 3]
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller; the
 *     library allocates nothing and keeps no state between calls, so calls
 *     are thread-safe.
 *   - Status codes and enum-valued arguments (dtype, tile, scale mode, GEMM
 *     kind, power-of-two operand mask) are passed as plain int, so that the
 *     ABI does not depend on the size a C compiler picks for an enum; the
 *     FP8Q_* constants below are the valid values, anything else returns
 *     FP8Q_ERR_ARG.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream of the
 *     calling thread's current device).  All work is enqueued on it and runs
 *     on its device, so every pointer must be memory that device can access;
 *     the library never synchronises.
 *   - Return value: an fp8q_status.  Arguments are validated before anything
 *     is launched; on the first violation the matching error is returned and
 *     nothing runs.  A launch failure returns FP8Q_ERR_HIP.  Device faults
 *     surface at the caller's next synchronisation.  Nothing is printed and
 *     no C++ exception crosses the ABI.
 *   - Matrices are row-major with an explicit leading dimension (in
 *     elements).  FP8 data is OCP E4M3FN bytes (max 448, no infinities).
 *   - Inputs must be finite; non-finite input gives unspecified output.
 *   - Alignment: pointers 16-byte aligned, leading dimensions multiples of
 *     16 bytes (FP8Q_ERR_ALIGN otherwise).
 *   - Outputs may not overlap inputs (FP8Q_ERR_ALIAS for an overlap the
 *     library can see from the pointer ranges).
 *
 * Quantization rule (both quantizers), for each group G of 128 elements
 * (1x128, 128x1) or 128x128 elements (block):
 *   a   = max(max_{x in G} |x|, 448 * 2^-126)
 *   MAXABS: s = fl32(a / 448), inv = fl32(448 / a)  (IEEE divisions)
 *   POW2:   s = 2^k, inv = 2^-k, k the smallest integer with a <= 448 * 2^k
 *   q   = E4M3_RNE(clamp(fl32(x * inv), -448, 448))   (sign of zero kept)
 * The stored scale s is the dequantization multiplier: x ~= s * q.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8Q_OK = 0,
  FP8Q_ERR_NULL = 1,         /* a required pointer is NULL */
  FP8Q_ERR_SHAPE = 2,        /* negative size, leading dimension too small, bad group map size */
  FP8Q_ERR_ALIGN = 3,        /* pointer or leading dimension not 16-byte aligned */
  FP8Q_ERR_UNSUPPORTED = 4,  /* valid request outside this library's shape/dtype support */
  FP8Q_ERR_ALIAS = 5,        /* an output overlaps an input or another output */
  FP8Q_ERR_HIP = 6,          /* the HIP launch itself failed */
  FP8Q_ERR_ARG = 7           /* unknown enum value */
} fp8q_status;

typedef enum { FP8Q_BF16 = 0, FP8Q_F32 = 1 } fp8q_dtype;
typedef enum { FP8Q_SCALE_MAXABS = 0, FP8Q_SCALE_POW2 = 1 } fp8q_scale_mode;
typedef enum { FP8Q_TILE_1x128 = 0, FP8Q_TILE_128x1 = 1 } fp8q_tile;
typedef enum { FP8Q_FPROP = 0, FP8Q_DGRAD = 1, FP8Q_WGRAD = 2 } fp8q_gemm_kind;
typedef enum { FP8Q_POW2_A = 1, FP8Q_POW2_B = 2, FP8Q_POW2_AB = 3 } fp8q_pow2_operands;

/*
 * fp8_quant_tile -- online 1x128 or 128x1 tile quantization.
 * [dssusan.co.kr FP8 excerpt, paragraph 4: activations grouped per token per
 *  128 channels (1x128), re-tiled 1x128 -> 128x1 for the backward pass;
 *  paragraph 2: each tile's max-abs computed online and the scale derived
 *  from it; "Deepseek - Not For everyone", paragraph 3: the max-abs is mapped
 *  onto the largest FP8 value; dssusan.co.kr, paragraph 1: optional integral
 *  power-of-2 scales]
 *
 * x        : input X[rows][cols], leading dimension ld_x (elements), dtype x_dtype.
 * tile     : FP8Q_TILE_1x128 -- groups of 128 consecutive columns in one row
 *              (activations in the forward pass).
 *              q[rows][cols] with leading dimension ld_q (bytes);
 *              scales[cols/128][rows], packed (group-major).
 *              Requires cols % 128 == 0; rows arbitrary.
 *            FP8Q_TILE_128x1 -- groups of 128 consecutive rows in one column
 *              (activations / output gradients re-tiled for Wgrad), written
 *              TRANSPOSED so each group is 128 contiguous bytes:
 *              q[cols][rows] with leading dimension ld_q (bytes), i.e.
 *              q[c*ld_q + r] is the code of X[r][c];
 *              scales[rows/128][cols], packed.
 *              Requires rows % 128 == 0 and cols % 8 == 0.
 * mode     : FP8Q_SCALE_MAXABS or FP8Q_SCALE_POW2.
 * rows == 0 or cols == 0 is a no-op returning FP8Q_OK.
 */
int fp8_quant_tile(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                   int tile, int mode,
                   uint8_t* q, int64_t ld_q, float* scales,
                   void* stream);

/*
 * fp8_quant_block -- online 128x128 block quantization (weights).
 * [dssusan.co.kr FP8 excerpt, paragraph 4: per 128 input x 128 output channels]
 *
 * w        : input W[rows][cols], leading dimension ld_w (elements), dtype w_dtype.
 * q        : q[rows][cols], leading dimension ld_q (bytes).
 * scales   : scales[rows/128][cols/128], packed.
 * q_t      : optional (NULL to skip): the transposed codes q_t[cols][rows],
 *            leading dimension ld_qt (bytes); q_t[c*ld_qt + r] == q[r*ld_q + c].
 * scales_t : required iff q_t is given: scales_t[cols/128][rows/128] == scales^T
 *            (q_t without scales_t: FP8Q_ERR_NULL; scales_t without q_t:
 *            FP8Q_ERR_ARG).
 *            The transposed pair is the K-contiguous weight operand of Dgrad.
 * Requires rows % 128 == 0 and cols % 128 == 0.
 */
int fp8_quant_block(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ld_w,
                    int mode,
                    uint8_t* q, int64_t ld_q, float* scales,
                    uint8_t* q_t, int64_t ld_qt, float* scales_t,
                    void* stream);

/*
 * fp8_quant_tile_dual -- both tilings of one tensor in one pass: the 1x128
 * tiles of fp8_quant_tile(FP8Q_TILE_1x128) and the transposed 128x1 tiles of
 * fp8_quant_tile(FP8Q_TILE_128x1), read from X once.
 * [dssusan.co.kr FP8 excerpt, paragraph 4: the backward pass feeds the
 *  output gradient to Dgrad in 1x128 tiles and to Wgrad in 128x1 tiles]
 *
 * x        : input X[rows][cols], leading dimension ld_x (elements), dtype x_dtype.
 * q        : 1x128 codes q[rows][cols], leading dimension ld_q (bytes).
 * scales   : 1x128 scales[cols/128][rows], packed.
 * q_t      : 128x1 codes, transposed: q_t[cols][rows], leading dimension ld_qt
 *            (bytes); q_t[c*ld_qt + r] is the 128x1 code of X[r][c].
 * scales_t : 128x1 scales[rows/128][cols], packed.
 * mode     : FP8Q_SCALE_MAXABS or FP8Q_SCALE_POW2 (both tilings).
 * Every output is bit-identical to the two fp8_quant_tile calls.  All four
 * outputs are required (FP8Q_ERR_NULL otherwise).
 * Requires rows % 128 == 0 and cols % 128 == 0.
 * rows == 0 or cols == 0 is a no-op returning FP8Q_OK.
 */
int fp8_quant_tile_dual(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                        int mode,
                        uint8_t* q, int64_t ld_q, float* scales,
                        uint8_t* q_t, int64_t ld_qt, float* scales_t,
                        void* stream);

/*
 * fp8_gemm_blockscaled -- C[M][N] (+)= A . B^T with per-128-K-group scales,
 * FP32 promotion once per K-group.
 * [dssusan.co.kr FP8 excerpt, paragraph 3; youlimart.com FP8 excerpt, paragraphs 2-3]
 *
 *   C[m][n] = sum_g  sa(g,m) * sb(g,n) * sum_{k in group g} dec(a[m][k]) * dec(b[n][k])
 *
 * Each group's FP8 partial is formed exactly-ish by the matrix cores (FP32
 * accumulation inside one 128-deep MFMA) and then multiplied by its scales and
 * added into FP32 accumulators.
 *
 * a        : A[M][K] E4M3, leading dimension lda (bytes).  K-contiguous.
 * a_scales : [K/128][M] packed (the 1x128 quantizer's layout, or the 128x1
 *            quantizer's layout for Wgrad).
 * b        : B[N][K] E4M3, leading dimension ldb (bytes).  K-contiguous.
 * b_scales : FPROP / DGRAD: [N/128][K/128] packed (128x128 block scales of the
 *              weight as stored [N][K]; for Dgrad pass fp8_quant_block's q_t /
 *              scales_t).
 *            WGRAD: [K/128][N] packed (the 128x1 quantizer's scales).
 * kind     : FPROP  -- Y = X W:   A = X quantized 1x128, B = W stored [out][in].
 *            DGRAD  -- dX = dY W^T: A = dY quantized 1x128, B = W's transposed copy.
 *            WGRAD  -- dW = dY^T X: A = dY^T (128x1, transposed), B = X^T (128x1, transposed).
 * c        : C[M][N], leading dimension ldc (elements), dtype c_dtype
 *            (FP8Q_BF16, rounded to nearest-even, or FP8Q_F32).  With BF16
 *            output the call may use C's own rows as temporary FP32 storage
 *            before writing the result there (C is an output: nothing the
 *            caller put in it is read); only the columns [0, N) of C are ever
 *            touched, and C holds the result once the call's work completes.
 * accumulate : 0 -> C = result; 1 -> C += result (FP8Q_F32 output only).
 * Requires M, N, K multiples of 128, and lda, ldb of at most 4,194,176 bytes
 * (the kernels address a tile's rows with 32-bit offsets); otherwise
 * FP8Q_ERR_UNSUPPORTED.  M == 0 or N == 0 is a no-op; K == 0 with M, N > 0
 * writes zeros (or leaves C unchanged with accumulate).
 * Scale domain: each group's combined factor sa*sb is formed in FP32 (for
 * WGRAD per element, for FPROP / DGRAD per row and block) and multiplied into
 * the FP32 accumulation with one FMA; results follow the definition above to
 * FP32 rounding as long as every such product is an FP32 normal number
 * (2^-126 <= sa*sb < 2^128) and the output is finite.  Scales from
 * fp8_quant_tile / fp8_quant_block of data whose max-abs values lie between
 * about 2^-55 and 2^55 always satisfy this.
 */
int fp8_gemm_blockscaled(int kind, int64_t M, int64_t N, int64_t K,
                         const uint8_t* a, int64_t lda, const float* a_scales,
                         const uint8_t* b, int64_t ldb, const float* b_scales,
                         void* c, int c_dtype, int64_t ldc, int accumulate,
                         void* stream);

/*
 * fp8_gemm_blockscaled_pow2 -- the same GEMM when one or both operands carry
 * power-of-two scales (FP8Q_SCALE_POW2 quantizer output), with those scales
 * applied by the matrix cores themselves.
 * [dssusan.co.kr FP8 excerpt, paragraph 1: power-of-2 scales; paragraph 3 and
 *  "Deepseek - Not For everyone", paragraph 4: MMA with group scaling]
 *
 * Arguments, layouts, shape rules and status codes are those of
 * fp8_gemm_blockscaled, plus
 * pow2_operands : FP8Q_POW2_A, FP8Q_POW2_B or FP8Q_POW2_AB -- whose scales are
 *                 powers of two (anything else: FP8Q_ERR_ARG).
 * Each power-of-two scale is handed to gfx950's
 * v_mfma_scale_f32_16x16x128_f8f6f4 as an E8M0 code (its biased exponent),
 * so that operand is dequantized inside the MFMA:
 *   FP8Q_POW2_AB: every 128-deep group is dequantized and accumulated in the
 *                 MFMA's own FP32 accumulator across all K-groups; there is no
 *                 per-group VALU promotion at all;
 *   FP8Q_POW2_A / FP8Q_POW2_B: the other operand's scale is applied by the
 *                 per-group FP32 promotion as in fp8_gemm_blockscaled (for
 *                 Wgrad this saves one multiply per output element per group).
 * Only the exponent field of a scale declared power-of-two is used: such a
 * scale that is not a positive power of two in [2^-126, 2^127] gives
 * unspecified output.
 */
int fp8_gemm_blockscaled_pow2(int kind, int64_t M, int64_t N, int64_t K,
                              const uint8_t* a, int64_t lda, const float* a_scales,
                              const uint8_t* b, int64_t ldb, const float* b_scales,
                              void* c, int c_dtype, int64_t ldc, int accumulate,
                              int pow2_operands, void* stream);

/*
 * fp8_gemm_blockscaled_grouped -- grouped (MoE expert) Fprop.
 * [dssusan.co.kr FP8 excerpt, paragraph 3 and "Deepseek - Not For everyone",
 *  paragraph 4 for the scaling; MoE experts per "Deepseek - Not For everyone",
 *  paragraphs 1 and 4]
 *
 * The rows of A are the concatenation of per-group token slabs, each padded
 * to a multiple of 128 rows; every 128-row M tile belongs to one group.
 *
 * group_of_mtile : DEVICE int32[M_total/128]; entry t is the group of rows
 *                  [128t, 128t+128).  A tile whose entry is outside
 *                  [0, num_groups) is skipped (its C rows are left untouched).
 * a, lda, a_scales : A[M_total][K] E4M3, scales [K/128][M_total] packed.
 * b        : B[num_groups][N][K] E4M3, contiguous (row pitch K bytes).
 * b_scales : [num_groups][N/128][K/128] packed.
 * c        : C[M_total][N], leading dimension ldc (elements), c_dtype.
 * Requires M_total, N, K multiples of 128 and num_groups >= 1.
 */
int fp8_gemm_blockscaled_grouped(int32_t num_groups, int64_t M_total, int64_t N, int64_t K,
                                 const int32_t* group_of_mtile,
                                 const uint8_t* a, int64_t lda, const float* a_scales,
                                 const uint8_t* b, const float* b_scales,
                                 void* c, int c_dtype, int64_t ldc,
                                 void* stream);

/*
 * fp8_requant_1x128_to_128x1 -- FP8 -> FP8 re-tiling of 1x128-quantized
 * activations into 128x1 tiles for the backward pass, without a trip through
 * BF16.  [dssusan.co.kr FP8 excerpt, paragraph 4: 1x128 tiles converted to
 * 128x1 tiles in backward; paragraph 1: power-of-2 scales for these
 * activations]
 *
 * q        : input codes Q[rows][cols] (E4M3 bytes, 1x128 tiles), leading
 *            dimension ld_q (bytes).
 * scales   : their 1x128 scales, scales[cols/128][rows], packed (exactly what
 *            fp8_quant_tile(..., FP8Q_TILE_1x128, ...) writes).
 * mode     : scale rule of the OUTPUT tiles, FP8Q_SCALE_POW2 or MAXABS.
 * q_t      : output codes, TRANSPOSED: q_t[cols][rows], leading dimension
 *            ld_qt (bytes); q_t[c*ld_qt + r] is the new code of element (r, c).
 * scales_t : output scales[rows/128][cols], packed (the 128x1 layout of
 *            fp8_quant_tile).
 * Computes, for every element, xh = fl32(dec(Q[r][c]) * scales[c/128][r])
 * (exact when the input scales are powers of two) and quantizes xh with the
 * quantization rule above over each 128x1 group (128 rows of one column).
 * With power-of-2 scales on both sides, a column whose 128x1 scale equals
 * every row's 1x128 scale comes back with its codes unchanged.
 * Input codes must not be NaN (0x7F / 0xFF): unspecified output.
 * Requires rows % 128 == 0 and cols % 128 == 0.
 * rows == 0 or cols == 0 is a no-op returning FP8Q_OK.
 */
int fp8_requant_1x128_to_128x1(const uint8_t* q, int64_t rows, int64_t cols, int64_t ld_q,
                               const float* scales, int mode,
                               uint8_t* q_t, int64_t ld_qt, float* scales_t,
                               void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* fp8q_status_string(int status);

/* ABI version of this header/library pair (major*100 + minor). */
int fp8q_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
