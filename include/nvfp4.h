/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 linear-layer library.
 *
 * NVFP4 is the two-level 4-bit format of "Pretraining Large Language Models
 * with NVFP4" (arXiv 2509.25149).  Citations below name two web pages about
 * that paper:
 *   [Review]   "NVFP4 4-bit Pretraining, Made Practical: 12B up to 10T Tokens,
 *              Effectively On Par with FP8" (jaehun.me paper review), by its
 *              numbered sections ("s1 Step 2" = second step of section
 *              "1) The NVFP4 quantization pipeline").
 *   [Captions] the paper's figure-caption list, by figure number.
 *
 * Format of one quantised operand [rows, cols] (cols = contraction / block axis):
 *   codes   uint8 [rows][cols/2]; two E2M1 codes per byte, the even column in
 *           the low nibble; code = sign << 3 | magnitude index, magnitudes
 *           {0, .5, 1, 1.5, 2, 3, 4, 6}                     [Review s7]
 *   scales  uint8 E4M3 (OCP E4M3FN bit pattern) decode scales, one per block:
 *           1x16 mode  [rows][cols/16]  (16 consecutive elements of a row)
 *           16x16 mode [rows/16][cols/16] (one per 16x16 tile)  [Review s2]
 *   global  one fp32 g = 1/s_enc with s_enc = 2688/amax (6 x 448)
 *                                                    [Review s1 Step 1]
 *   value   x_hat = e2m1(code) * e4m3(scale) * g     [Review s1 Step 3]
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers; the caller owns every buffer.
 *     The library never allocates device memory; its only global state is
 *     the per-device scratch of nvfp4_quantize_static.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work on it and return; none synchronises except
 *     nvfp4_device_status().
 *   - Argument errors are returned synchronously and then NOTHING has been
 *     enqueued.  A failed launch returns NVFP4_ERR_HIP.  A non-finite tensor
 *     amax is only known on the device: the kernels then record
 *     NVFP4_ERR_NONFINITE in the workspace's status word (read it with
 *     nvfp4_device_status) and that operand's outputs are unspecified.
 *   - `workspace` is a device buffer of at least nvfp4_workspace_bytes()
 *     bytes holding the status word and per-call reduction slots.  Calls that
 *     share a workspace must be issued on one stream (they reuse its slots).
 *   - Shapes: rows and cols are multiples of 16 except where stated; leading
 *     dimensions are in elements and >= cols, with 256 * ld * element size
 *     below 2^31 bytes (rows are read in 256-row tiles with 32-bit offsets)
 *     and at most 65535 * 128 = 8388480 rows per source matrix;
 *     device pointers must be 16-byte aligned and ld * element size a
 *     multiple of 16 bytes; a GEMM operand's scales pointer must be 4-byte
 *     aligned.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,       /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,      /* sizes not supported / inconsistent */
  NVFP4_ERR_ALIGN = 3,      /* pointer, leading dimension or offset misaligned */
  NVFP4_ERR_DTYPE = 4,      /* unsupported dtype or enum value */
  NVFP4_ERR_WORKSPACE = 5,  /* workspace missing or too small */
  NVFP4_ERR_HIP = 6,        /* a HIP launch or runtime call failed */
  NVFP4_ERR_NONFINITE = 7   /* device-side: an operand's amax is Inf/NaN */
} nvfp4_status;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype;
typedef enum { NVFP4_RN = 0, NVFP4_SR = 1 } nvfp4_round;
/* NVFP4_SCALE_MX32 marks an MXFP4 operand, the comparator format the pages
 * weigh NVFP4 against [Review "secret weapon" items 1-2; Captions Fig. 6]:
 * the same codes, one E8M0 (power-of-two, bias 127) scale per 32 elements of a row,
 * scales [rows][cols/32], no tensor scale (global_scale unused, may be NULL). */
typedef enum {
  NVFP4_SCALE_1X16 = 0,
  NVFP4_SCALE_16X16 = 1,
  NVFP4_SCALE_MX32 = 2
} nvfp4_scale_mode;

/* One quantised operand (see the format above).  rows x cols is the
 * operand's own logical shape; cols is the block (contraction) axis. */
typedef struct {
  uint8_t* codes;
  uint8_t* scales;
  float* global_scale; /* device pointer to one fp32 (g = 1/s_enc) */
  int64_t rows;
  int64_t cols;
  int32_t scale_mode;  /* nvfp4_scale_mode */
} nvfp4_tensor;

/* Options of one 1x16 quantisation.
 *   round      NVFP4_RN: nearest-even (activations, weights)
 *              NVFP4_SR: stochastic (gradients)      [Review s1 Step 3, s4]
 *   transpose  0: the operand is x [rows, cols], blocks along cols;
 *              1: the operand is x^T [cols, rows], blocks along x's rows
 *                 (tokens) -- the column-wise copy the backward GEMMs need
 *                 because the contraction axis flips      [Review s2]
 *   rht        1: apply the 16-point random Hadamard transform to each
 *              16-element chunk along the operand's block axis first
 *              (Wgrad inputs only in the recipe)           [Review s3]
 *   rht_signs  sign diagonal, bit i set = s_i is -1
 *   seed, offset, stream_id
 *              stochastic-rounding draw of operand element (r, c) comes from
 *              the Philox4x32-10 counter-based generator with key = seed,
 *              counter = (e/8, stream_id, 0), e = offset + r*C + c in the
 *              operand's own [R, C] layout; offset % 16 == 0.
 *   rht_d      size of the transform with rht: 0 or 16 (the recipe), or 4
 *              (four 4-point transforms y = 1/2 H4 diag(s) x per 16-element
 *              chunk, signs bits 0-3 [Captions Fig. 12]; nvfp4_quantize only).
 *              Any other value is NVFP4_ERR_DTYPE. */
typedef struct {
  int32_t round;
  int32_t transpose;
  int32_t rht;
  uint32_t rht_signs;
  uint64_t seed;
  uint64_t offset;
  uint32_t stream_id;
  int32_t rht_d;
} nvfp4_quant_opts;

/* The layer recipe.  All-zero switches give the pages' recipe [Review "Core
 * idea" items (2)-(4); Captions Fig. 4, 5]: 16x16 weight scales, RHT on the
 * Wgrad inputs only, stochastic rounding on the gradient copies only.  The
 * pages fix one sign seed for the whole run: use nvfp4_rht_signs_from_seed(0)
 * unless another is wanted.  Each no_* switch removes one component, as the
 * pages' ablations do [Captions Fig. 4, 10, 11, 14]:
 *   no_2d_weights  W and W^T are each quantised with 1x16 blocks along their
 *                  own rows (W along K for Fprop, W^T along N for Dgrad), so
 *                  the two copies differ (w_fprop != w_bprop) [Review s2]
 *   no_rht         the Wgrad copies (X^T, dY^T) skip the RHT
 *   no_sr          the dY copies round to nearest-even
 *   bf16_fprop     the end-of-training precision switch [Review "Core
 *                  strengths" item 9; Captions Fig. 7]: Fprop runs as the
 *                  plain BF16 product Y = X W^T
 *                  (nvfp4_bf16_gemm) while the backward stays NVFP4.  Needs
 *                  dtype NVFP4_BF16 and K % 32 == 0, K >= 96; ctx->xq and
 *                  ctx->wq are then neither read nor written.
 * A backward must use the recipe of its forward. */
typedef struct {
  uint32_t rht_signs;   /* sign diagonal shared by every RHT of the layer */
  int32_t training;     /* forward also builds the Wgrad copy of X */
  int32_t no_2d_weights;
  int32_t no_rht;
  int32_t no_sr;
  int32_t bf16_fprop;
} nvfp4_recipe;

/* Buffers of one layer step Y = X W^T, X [M, K], W [N, K], dY [M, N].
 * The caller allocates each operand with nvfp4_tensor_bytes() and fills
 * codes/scales/global_scale pointers; shapes are set by the library.
 *   xq   X       [M, K] 1x16 RN          (Fprop A)
 *   wq   W       [N, K] 16x16 RN         (Fprop B)      (1x16 with no_2d_weights)
 *   wqt  W^T     [K, N] 16x16 RN, same codes transposed, same g (Dgrad B)
 *                (no_2d_weights: W^T quantised on its own, 1x16 along N, same g)
 *   xqt  (R X)^T [K, M] 1x16 along tokens, RHT, RN              (Wgrad B)
 *   dyq  dY      [M, N] 1x16 SR, stream 0                       (Dgrad A)
 *   dyqt (R dY)^T [N, M] 1x16 along tokens, RHT, SR, stream 1   (Wgrad A) */
typedef struct {
  int64_t M, K, N;
  nvfp4_tensor xq, wq, wqt, xqt, dyq, dyqt;
  /* Set by nvfp4_linear_fwd: the sign diagonal and whether the RHT was
   * applied to xqt, so that the backward can refuse a recipe whose dY^T copy
   * would get another transform than X^T (dW = (R dY)^T (R X) needs one R). */
  uint32_t rht_signs;
  int32_t rht;
  /* Optional fp32 scratch for the backward's fused Dgrad + Wgrad launch
   * (device memory, 16-byte aligned, NVFP4_LINEAR_SCRATCH_BYTES): with it the
   * last Wgrad tiles of each XCD's share run as two K halves and a short pass
   * adds the halves, which evens out the launch's last round.  The halves are
   * summed in another order than a whole tile's K loop, so dW may differ from
   * nvfp4_gemm's in the last bits (within the GEMM tolerance); NULL keeps
   * every tile whole.  nvfp4_linear_ctx_init places it in its buffer. */
  void* wgrad_scratch;
  size_t wgrad_scratch_bytes;
} nvfp4_linear_ctx;

/* Size of nvfp4_linear_ctx.wgrad_scratch: 8 XCD shares x 8 split tiles x 2
 * halves x 256 x 256 fp32. */
#define NVFP4_LINEAR_SCRATCH_BYTES ((size_t)32 << 20)

/* ------------------------------------------------------------ size queries */

/* Bytes of the codes and scales arrays of a [rows, cols] operand (codes
 * rows * cols / 2; scales per block: rows * cols / 16 for 1x16, / 256 for
 * 16x16, / 32 for MX32).  cols % 16 (MX32: % 32) and, for 16x16, rows % 16
 * must hold and the byte counts stay below 2^62, else NVFP4_ERR_SHAPE; an
 * unknown scale_mode is NVFP4_ERR_DTYPE. */
nvfp4_status nvfp4_tensor_bytes(int64_t rows, int64_t cols, int32_t scale_mode,
                                size_t* codes_bytes, size_t* scales_bytes);

/* Bytes of one device buffer that holds all six quantised operands of a
 * layer step (the buffers of nvfp4_linear_ctx), for nvfp4_linear_ctx_init.
 * M, K, N positive multiples of 16 whose operand sizes stay below 2^62
 * bytes, else NVFP4_ERR_SHAPE. */
nvfp4_status nvfp4_linear_ctx_bytes(int64_t M, int64_t K, int64_t N, size_t* bytes);

/* Point ctx's six operands into `buffer` (a device buffer of at least
 * nvfp4_linear_ctx_bytes(M, K, N) bytes, 256-byte aligned; the caller keeps
 * ownership) and set their shapes and ctx->M, K, N.  Codes, scales and tensor
 * scale of each operand start on 256-byte boundaries; scale arrays are sized
 * for 1x16 blocks, so either weight recipe fits.  Host bookkeeping only:
 * nothing is enqueued and the buffer is not touched.  A buffer that is too
 * small is NVFP4_ERR_SHAPE. */
nvfp4_status nvfp4_linear_ctx_init(nvfp4_linear_ctx* ctx, void* buffer, size_t bytes, int64_t M,
                                   int64_t K, int64_t N);

/* Minimum workspace size in bytes (a constant, 32 KB). */
size_t nvfp4_workspace_bytes(void);

/* Host-side: the sign diagonal from a seed = low 16 bits of word 0 of
 * Philox4x32-10(counter 0, key = seed)  [Review s3: one fixed seed]. */
uint32_t nvfp4_rht_signs_from_seed(uint64_t seed);

/* Zero the workspace (status word and slots) on `stream`. */
nvfp4_status nvfp4_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/* Synchronises `stream`, returns the device status word (NVFP4_OK or
 * NVFP4_ERR_NONFINITE) and clears it. */
nvfp4_status nvfp4_device_status(void* workspace, void* stream);

const char* nvfp4_status_string(nvfp4_status s);

/* -------------------------------------------------------------- operations */

/*
 * nvfp4_quantize: two-level NVFP4 quantisation of one operand with 1x16
 * blocks [Review s1 Steps 1-3; Captions Fig. 1]:
 *   1. tensor amax A of the operand (after the RHT when opts->rht),
 *      s_enc = 2688/A (FLT_MAX if that overflows; 1 when A == 0), g = 1/s_enc;
 *   2. per block: d_b = E4M3(amax_b * (s_enc/6)), nearest-even, saturating;
 *   3. per element: v = x * (s_enc/d_b), E2M1 code of v by opts->round.
 * x: [rows, cols] of `dtype` (NVFP4_F32 or NVFP4_BF16), leading dim ld.
 * out: operand [rows, cols] (transpose 0) or [cols, rows] (transpose 1);
 *      out->rows/cols/scale_mode are set by the call.
 * Ragged rows (rows % 16 != 0) are allowed for transpose 0 without RHT.
 */
nvfp4_status nvfp4_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                            int64_t ld, const nvfp4_quant_opts* opts, nvfp4_tensor* out,
                            void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_quantize_static: nvfp4_quantize for callers that cannot allocate or
 * hand over a workspace -- code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The operation, the arguments shared with
 * nvfp4_quantize and their errors are those of nvfp4_quantize; the call
 * allocates nothing and enqueues the same kernels.  Differences:
 *   - the tensor-amax reduction slots live in a library-owned device array
 *     of a fixed 8 KB per GPU, whatever the input size (so no input is too
 *     large for it); each GPU's copy is looked up (hipGetSymbolAddress) on
 *     the first call on that device and is held until the process ends;
 *   - status: caller-owned device word (4-byte aligned, not NULL, else
 *     NVFP4_ERR_NULL / NVFP4_ERR_ALIGN); a non-finite amax raises it to
 *     NVFP4_ERR_NONFINITE (atomic max), nothing ever clears it;
 *   - the stream must belong to the current device, else NVFP4_ERR_HIP.
 * Every call on one GPU shares that GPU's array: calls issued in order on one
 * stream are safe, calls that overlap on one GPU (two streams, two host
 * threads without ordering) race and give wrong scales.
 */
nvfp4_status nvfp4_quantize_static(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                   int64_t ld, const nvfp4_quant_opts* opts, nvfp4_tensor* out,
                                   uint32_t* status, void* stream);

/*
 * nvfp4_quantize_rowcol: both copies an operand needs for a training step
 * from one read of x [rows, cols]: `row` = x with 1x16 blocks along cols
 * (opts_row; transpose/rht must be 0) and `col` = (R x)^T with 1x16 blocks
 * along rows (opts_col; transpose must be 1, rht optional with rht_d 0 or
 * 16; rht_d 4 is NVFP4_ERR_DTYPE here).  Each copy has its
 * own tensor scale.  Equivalent to two nvfp4_quantize calls.  [Review s6
 * steps 1-3; Captions Fig. 5]
 */
nvfp4_status nvfp4_quantize_rowcol(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                   int64_t ld, const nvfp4_quant_opts* opts_row,
                                   const nvfp4_quant_opts* opts_col, nvfp4_tensor* row,
                                   nvfp4_tensor* col, void* workspace, size_t ws_bytes,
                                   void* stream);

/*
 * nvfp4_quantize_2d: weight quantisation with one E4M3 scale per 16x16 tile
 * and nearest-even rounding [Review s2; "Core idea" item (2)].  out = W
 * [rows, cols] with grid [rows/16][cols/16]; out_t (nullable) = the same
 * codes transposed, [cols, rows] with grid [cols/16][rows/16] and the same
 * g, so the backward GEMM sees exactly the forward weight.
 */
nvfp4_status nvfp4_quantize_2d(const void* w, int32_t dtype, int64_t rows, int64_t cols,
                               int64_t ld, nvfp4_tensor* out, nvfp4_tensor* out_t,
                               void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_rht: random Hadamard transform of size d = 4, 16 or 128 [Review s3
 * and its size note: d = 16 is the recipe, 4 and 128 the sizes compared with
 * it; Captions Fig. 12]: y = c * H_d * diag(s) * x per d-element chunk along
 * `axis` (1: rows, cols % d == 0 (cols % 8 for d = 4); 0: columns,
 * rows % d == 0), c = fp32(1/sqrt(d)) (exact for 4 and 16), fp32 order signs,
 * butterflies h = 1 .. d/2 as (a+b, a-b), then x c.  signs: HOST array of 4
 * words; sign bit i = bit i % 32 of signs[i / 32] (d = 16 uses the low 16
 * bits of signs[0], exactly nvfp4_rht16).  y: dense fp32 [rows, cols].  A
 * Wgrad operand with another size is nvfp4_rht(axis 0) followed by
 * nvfp4_quantize(transpose 1) of y.  Sign options [Captions Fig. 13]: all
 * zero (no randomisation), one seed for every layer, or a seed per layer via
 * nvfp4_rht_signs128_from_seed.
 */
nvfp4_status nvfp4_rht(const void* x, float* y, int32_t in_dtype, int64_t rows, int64_t cols,
                       int64_t ld, int32_t axis, int32_t d, const uint32_t* signs, void* stream);

/* Host-side: the 128 sign bits from a seed = the Philox4x32-10 block
 * (counter 0, key = seed), word 0 first; its low 16 bits are
 * nvfp4_rht_signs_from_seed(seed).  out: 4 words. */
void nvfp4_rht_signs128_from_seed(uint64_t seed, uint32_t* out);

/*
 * nvfp4_dequantize: decode an operand [Review s1 Step 3]: out[r][c] =
 * e2m1(code) * d_b * g for the 1x16 and 16x16 modes, e2m1(code) * 2^(s - 127)
 * for NVFP4_SCALE_MX32 (E8M0 code 0xFF decodes to NaN), in fp32 (e2m1 * d_b
 * is exact, so each value is the exact product rounded once).  out: fp32
 * [rows][ldo], ldo >= cols and a multiple of 4, 16-byte aligned.
 */
nvfp4_status nvfp4_dequantize(const nvfp4_tensor* t, float* out, int64_t ldo, void* stream);

/*
 * nvfp4_mx_quantize: MXFP4 quantisation of x [rows, cols] (leading dim ld,
 * F32 or BF16) with 32-element blocks along cols (cols % 32 == 0), the
 * comparator of [Review "secret weapon" items 1-2; Captions Fig. 6]: blocks
 * of 32, one power-of-two UE8M0 scale.  Scale rule (the OCP Microscaling one; the
 * pages describe only the format): e = floor(log2(amax_b)) - 2 clamped to
 * [-127, 127], stored as e + 127; so amax_b / 2^e is in [4, 8) and values at
 * or above 6 * 2^e saturate (the binade the pages say MXFP4 loses).  An
 * all-zero block stores 0; a block holding Inf/NaN stores 0xFF (E8M0 NaN)
 * and zero codes.  Elements: x * 2^-e (exact), nearest-even E2M1.  out
 * (codes >= rows*cols/2 bytes, scales >= rows*cols/32) becomes an
 * NVFP4_SCALE_MX32 operand [rows, cols]; ragged rows are allowed.
 */
nvfp4_status nvfp4_mx_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                               int64_t ld, nvfp4_tensor* out, void* stream);

/*
 * nvfp4_rht16: standalone 16-point random Hadamard transform
 * y = 1/4 * H16 * diag(s) * x on every 16-element chunk [Review s3].
 * axis 1: chunks along each row (cols % 16 == 0); axis 0: along each column
 * (rows % 16 == 0).  x: [rows, cols] F32 or BF16 with leading dim ld;
 * y: dense fp32 [rows, cols].  fp32 order: signs, butterflies h = 1, 2, 4, 8
 * as (a+b, a-b), then x 1/4.
 */
nvfp4_status nvfp4_rht16(const void* x, float* y, int32_t in_dtype, int64_t rows,
                         int64_t cols, int64_t ld, int32_t axis, uint32_t rht_signs,
                         void* stream);

/*
 * nvfp4_gemm: C[m][n] = g_a g_b sum_k (e2m1*d_b)_A[m][k] (e2m1*d_b)_B[n][k]
 * with FP32 accumulation [Review s6 step 1; Captions Fig. 5].  Both operands
 * are contiguous along k (a->cols == b->cols == K); either may use 1x16 or
 * 16x16 scales.  c: [M, N] row-major with leading dim ldc >= N, 4-byte aligned,
 * dtype NVFP4_F32 or NVFP4_BF16 (nearest-even).  M and N may be any positive
 * size (a 16x16-scaled operand needs rows % 16 == 0); K a multiple of 16.
 * Only C's [M, N] window is written.
 * With both operands in NVFP4_SCALE_MX32 mode it is the MXFP4 product
 * C = sum_k (e2m1 * 2^(s-127))_A (e2m1 * 2^(s-127))_B (no tensor scales), on
 * gfx950's scaled FP4 MFMA; that path needs K % 128 == 0, K >= 384 and
 * rows * K / 2 < 2^31 for each operand (else NVFP4_ERR_SHAPE), and mixing an
 * MX32 operand with an NVFP4 one is NVFP4_ERR_DTYPE.
 * workspace, ws_bytes: reserved, not read or written (no GEMM path uses
 * scratch memory); NULL and 0 are accepted.
 */
nvfp4_status nvfp4_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c, int32_t c_dtype,
                        int64_t ldc, void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_bf16_gemm: the plain BF16 product C = A B^T with FP32 accumulation,
 * the high-precision forward of the pages' precision switch [Review "Core
 * strengths" item 9; Captions Fig. 7].  a: bf16 [M, K], b: bf16 [N, K], both dense row-major
 * (row stride K) and 16-byte aligned; c: [M, N] row-major with leading dim
 * ldc >= N, c_dtype NVFP4_F32 or NVFP4_BF16 (rounded to nearest-even), aligned
 * to its element.  M, N >= 1 (any value); K % 32 == 0 and K >= 96; each
 * operand's rows rounded up to 256, times K * 2 bytes, below 2^31
 * (else NVFP4_ERR_SHAPE).  Needs no workspace.
 */
nvfp4_status nvfp4_bf16_gemm(const void* a, const void* b, void* c, int64_t M, int64_t N,
                             int64_t K, int32_t c_dtype, int64_t ldc, void* stream);

/*
 * nvfp4_linear_fwd: forward of one NVFP4 linear layer Y = X W^T [Review s6
 * step 1; Captions Fig. 5].  Quantises X (1x16 RN -> ctx->xq), W (16x16 RN ->
 * ctx->wq) and, when recipe->training, the backward copies W^T (-> ctx->wqt)
 * and (R X)^T (RHT along tokens, RN -> ctx->xqt), then runs the Fprop GEMM.
 * x [M, K], w [N, K] of `dtype`, dense; y [M, N] bf16.  M, K, N multiples of
 * 16.  ctx->wqt and ctx->xqt are only needed when training.  With
 * recipe->bf16_fprop only the backward copies are made (none for inference)
 * and Fprop is nvfp4_bf16_gemm(x, w).
 */
nvfp4_status nvfp4_linear_fwd(const void* x, const void* w, void* y, int64_t M, int64_t K,
                              int64_t N, int32_t dtype, const nvfp4_recipe* recipe,
                              nvfp4_linear_ctx* ctx, void* workspace, size_t ws_bytes,
                              void* stream);

/*
 * nvfp4_linear_bwd: backward of the same layer [Review s6 steps 2-3;
 * Captions Fig. 5].  Quantises dY twice from one read: dY 1x16 SR stream 0
 * (ctx->dyq) and (R dY)^T with the RHT along tokens, SR stream 1
 * (ctx->dyqt), both with key sr_seed; then Dgrad dX = dyq . wqt^T (bf16
 * [M, K]) and Wgrad dW = dyqt . xqt^T ([N, K], dw_dtype F32 or BF16).
 * Requires a preceding nvfp4_linear_fwd with recipe->training on ctx, and a
 * recipe with that forward's rht_signs and no_rht (else NVFP4_ERR_SHAPE:
 * the two Wgrad operands must carry the same transform [Review s3]).
 */
nvfp4_status nvfp4_linear_bwd(const void* dy, int32_t dtype, nvfp4_linear_ctx* ctx, void* dx,
                              void* dw, int32_t dw_dtype, uint64_t sr_seed,
                              const nvfp4_recipe* recipe, void* workspace, size_t ws_bytes,
                              void* stream);

/*
 * nvfp4_peak_mfma_f16: measurement helper, not part of the layer.  Enqueues
 * an fp16 MFMA loop shaped like the GEMM's inner loop
 * (v_mfma_f32_32x32x16_f16, FP32 accumulation, one wave per SIMD, 16
 * accumulators, no memory traffic) of `iters` iterations and returns in
 * *flops the floating-point operations it performs; timing it on the stream
 * gives the compute rate the card holds under that load, next to the
 * datasheet peak (which assumes the top clock).  toggle_mask picks the
 * operand bits that change (ANDed with 0x87FF87FF, the sign and mantissa bits
 * of two f16; 0 keeps the operands constant).  valu_per_mfma:
 *   0  no VALU work in the loop: the operands alternate between two random
 *      register sets, so each MFMA sees new bits at no instruction cost
 *      (the pure MFMA rate);
 *   4  four VALU instructions per MFMA make fresh random operands every
 *      iteration (about the GEMM's dequantisation load).
 * Any other value is NVFP4_ERR_DTYPE.  sink: a device buffer of 2048 floats
 * the kernel may write (it does not in practice).
 */
nvfp4_status nvfp4_peak_mfma_f16(int32_t iters, uint32_t toggle_mask, int32_t valu_per_mfma,
                                 float* sink, double* flops, void* stream);

/*
 * nvfp4_peak_mfma_fp4: measurement helper, not part of the layer.  The same
 * VALU-free loop on the MXFP4 comparator's instruction,
 * v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 x E2M1 operands and unit E8M0
 * scales (one wave per SIMD, 16 accumulators, `iters` iterations, no memory
 * traffic); operands alternate between two register sets differing in the
 * bits under toggle_mask (0 keeps them constant; every 4-bit pattern is a
 * finite E2M1 code).  *flops receives 2*32*32*64 per MFMA.  sink: a device
 * buffer of 2048 floats the kernel may write (it does not in practice).
 * NVFP4_ERR_NULL / NVFP4_ERR_SHAPE (iters <= 0) as for nvfp4_peak_mfma_f16.
 */
nvfp4_status nvfp4_peak_mfma_fp4(int32_t iters, uint32_t toggle_mask, float* sink, double* flops,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
