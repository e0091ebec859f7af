/*
 * NVFP4 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, step-by-step CPU statement of what the NVFP4 linear layer
 * computes.  It exists to check the GPU library and nothing else: only the
 * test-suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load it.  It shares no code, header, table or constant generator with the
 * GPU library, and the GPU library never calls it.
 *
 * Citations name two web pages about "Pretraining Large Language Models with
 * NVFP4" (arXiv 2509.25149):
 *   [Review]   "NVFP4 4-bit Pretraining, Made Practical: 12B up to 10T Tokens,
 *              Effectively On Par with FP8" (jaehun.me paper review), cited by
 *              its numbered sections, e.g. [Review s1 Step 2] for the second
 *              step of "1) The NVFP4 quantization pipeline".
 *   [Captions] the figure-caption list of the same paper, cited by figure.
 * Where the pages leave a step open, the reading taken is stated at the step
 * (the same readings are listed together in the project's design notes).
 *
 * Floating point: every fp32 step below is one IEEE binary32 operation rounded
 * to nearest even (built with -ffp-contract=off, no fast-math); dequantised
 * values and GEMM sums are float64.
 *
 * Parity status: every function here (NVFP4 and the MXFP4 comparator) is
 * pinned by a CPU test against values
 * the pages print, closed forms, invariants or brute force; see the test
 * files named test_oracle_*.py.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_NONFINITE 7
#define ORACLE_ERR_SHAPE 2

/* ------------------------------------------------------------------------ */
/* E2M1 (FP4) element values: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}                 */
/* [Review s7, the FP4 value set of the toy example]; code = sign bit 3 plus  */
/* magnitude index 0..7 (standard E2M1: 1 sign, 2 exponent, 1 mantissa bit). */
/* ------------------------------------------------------------------------ */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_decode(uint8_t code) {
  double mag = kE2M1[code & 7];
  return (code & 8) ? -mag : mag;
}

/* Nearest-even rounding of a non-negative magnitude onto the E2M1 grid, the
 * rounding used for activations and weights [Review s1 Step 3; s6 step 1].
 * Nearest grid value; an exact tie goes to the even code index.  Values past 6 saturate to 6 (the nearest
 * representable value). */
int oracle_e2m1_rn_index(float m) {
  if (m >= 6.0f) return 7;
  int best = 0;
  double best_d = fabs((double)m - kE2M1[0]);
  for (int i = 1; i < 8; ++i) {
    double d = fabs((double)m - kE2M1[i]);
    if (d < best_d || (d == best_d && (i % 2) == 0 && (best % 2) != 0)) {
      best = i;
      best_d = d;
    }
  }
  return best;
}

/* Stochastic rounding of a non-negative magnitude [Review s10 SR formula and
 * s7 SR mini-example]: with lo <= m < hi the neighbouring grid values, the
 * result is hi with probability (m-lo)/(hi-lo), else lo.  The random source
 * is a 16-bit integer r16, uniform on [0, 65536), and the fraction is taken
 * in 22-bit fixed point (exactly the fp32 mantissa bits below the E2M1
 * mantissa bit when m >= 1, truncated below that): with
 * T = floor((m-lo)/(hi-lo) * 2^22), round up iff 64 * r16 < T.  Magnitudes at
 * or beyond 6 give 6. */
int oracle_e2m1_sr_index(float m, uint32_t r16) {
  if (m >= 6.0f) return 7;
  int lo = 0;
  for (int i = 0; i < 8; ++i)
    if (kE2M1[i] <= (double)m) lo = i;
  float lo_v = (float)kE2M1[lo];
  float hi_v = (float)kE2M1[lo + 1];
  float frac = (m - lo_v) / (hi_v - lo_v);
  double T = floor((double)frac * 4194304.0);
  return (64.0 * (double)r16 < T) ? lo + 1 : lo;
}

/* ------------------------------------------------------------------------ */
/* E4M3 (FP8) block scale [Review s1 Step 2; Captions Fig. 1].  The pages do */
/* not name the variant; the reading taken is OCP E4M3FN: exponent bias 7, 3 */
/* mantissa bits, subnormals down to 2^-9, largest finite 448, no infinity.  */
/* ------------------------------------------------------------------------ */
double oracle_e4m3_decode(uint8_t b) {
  int s = (b >> 7) & 1;
  int e = (b >> 3) & 15;
  int f = b & 7;
  double v;
  if (e == 15 && f == 7) return NAN;
  if (e == 0)
    v = ldexp((double)f / 8.0, -6);
  else
    v = ldexp(1.0 + (double)f / 8.0, e - 7);
  return s ? -v : v;
}

/* Encode a non-negative finite fp32 value to E4M3FN, round to nearest with
 * ties to the even code, saturating at 448 (never NaN). */
uint8_t oracle_e4m3_encode(float t) {
  if (!(t > 0.0f)) return 0;
  if (t >= 448.0f) return 0x7E;
  double x = (double)t;
  if (x < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9 */
    double q = nearbyint(x * 512.0); /* default rounding: half to even */
    return (uint8_t)q;              /* q == 8 is the code of 2^-6 */
  }
  int ex;
  double fr = frexp(x, &ex);     /* x = fr * 2^ex, fr in [0.5, 1) */
  int e = ex - 1;                /* x = (2*fr) * 2^e, 2*fr in [1, 2) */
  double mant = (2.0 * fr - 1.0) * 8.0;
  double q = nearbyint(mant);    /* 0..8, half to even */
  if (q == 8.0) {
    q = 0.0;
    e += 1;
  }
  int code = ((e + 7) << 3) | (int)q;
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)code;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 counter-based generator (Salmon, Moraes, Dror & Shaw,       */
/* "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11).  The pages only    */
/* give SR's probabilities; the random source is a reading, chosen because a */
/* counter-based stream makes every element's draw independent of tiling.    */
/* ------------------------------------------------------------------------ */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                          uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
    uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += W0;
    k1 += W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 16 random bits of element e of a quantised operand: e is the element's
 * position (offset + row*C + col) in the operand's own [R, C] layout.  Eight
 * consecutive elements share one generator call with counter
 * (e/8 low word, e/8 high word, stream, 0) and key (seed low, seed high);
 * element e takes 16-bit half (e mod 8) of the 128-bit output, word (e mod 8)/2,
 * low half first. */
uint32_t oracle_sr_bits(uint64_t seed, uint32_t stream, uint64_t e) {
  uint64_t j = e / 8;
  uint32_t ctr[4] = {(uint32_t)j, (uint32_t)(j >> 32), stream, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  unsigned h = (unsigned)(e % 8);
  uint32_t w = out[h / 2];
  return (h % 2 == 0) ? (w & 0xFFFFu) : (w >> 16);
}

/* Sign diagonal of the random Hadamard transform from a seed: the low 16 bits
 * of word 0 of one generator call (counter 0, key = seed).  Bit i set means
 * sign s_i = -1.  [Review s3 and Captions Fig. 11/13: one fixed seed for the
 * whole run is enough.] */
uint32_t oracle_rht_signs_from_seed(uint64_t seed) {
  uint32_t ctr[4] = {0u, 0u, 0u, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  return out[0] & 0xFFFFu;
}

/* ------------------------------------------------------------------------ */
/* Random Hadamard transform of size 16 [Review s3, transform size d = 16;  */
/* s0 key terms; Captions Fig. 11/12].  y = (1/4) * H16 * diag(s) * x with   */
/* H16 the Sylvester Hadamard matrix, H[i][j] = (-1)^popcount(i & j).  The    */
/* 1/4 makes it orthonormal.  fp32 evaluation order (a reading, fixed so the */
/* result is reproducible): signs first, then the butterfly stages h = 1, 2,  */
/* 4, 8 with (u_i, u_{i+h}) <- (u_i + u_{i+h}, u_i - u_{i+h}), then x 1/4.    */
/* ------------------------------------------------------------------------ */
void oracle_rht16_chunk(const float* x, uint32_t signs, float* y) {
  float u[16];
  for (int i = 0; i < 16; ++i) u[i] = ((signs >> i) & 1u) ? -x[i] : x[i];
  for (int h = 1; h < 16; h *= 2) {
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      float a = u[i], b = u[i + h];
      u[i] = a + b;
      u[i + h] = a - b;
    }
  }
  for (int i = 0; i < 16; ++i) y[i] = u[i] * 0.25f;
}

/* Standalone RHT16 of a [rows, cols] fp32 matrix (leading dimension ld).
 * axis 1: 16-element chunks along each row; axis 0: along each column.
 * Output is dense [rows, cols]. */
int oracle_rht16(const float* x, int64_t rows, int64_t cols, int64_t ld,
                 int axis, uint32_t signs, float* y) {
  if (axis == 1) {
    if (cols % 16) return ORACLE_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t c = 0; c < cols; c += 16)
        oracle_rht16_chunk(x + r * ld + c, signs, y + r * cols + c);
  } else {
    if (rows % 16) return ORACLE_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
      for (int64_t r = 0; r < rows; r += 16) {
        float in[16], out[16];
        for (int i = 0; i < 16; ++i) in[i] = x[(r + i) * ld + c];
        oracle_rht16_chunk(in, signs, out);
        for (int i = 0; i < 16; ++i) y[(r + i) * cols + c] = out[i];
      }
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Two-level NVFP4 quantisation [Review s1 Steps 1-3; s10 formula summary;   */
/* Captions Fig. 1].                                                          */
/*                                                                            */
/* Step 1 (global FP32 scale).  The tensor is remapped into a range the E4M3 */
/* block scales can represent.  Reading: s_enc = 2688 / amax with 2688 = 6 x */
/* 448 (FP4 maximum x E4M3 maximum), so the largest block's scale lands on   */
/* E4M3's maximum.  The stored per-tensor FP32 value is g = 1 / s_enc.        */
/* Step 2 (E4M3 block scale).  Each block's amax maps to the FP4 maximum 6.   */
/* Reading: the stored E4M3 value is the decode scale d_b = E4M3(amax_b *     */
/* s_enc / 6); the element multiplier is r_b = s_enc / d_b (the page's        */
/* s_b * s_glob), and decoding multiplies by d_b * g (the page's              */
/* (s_b * s_glob)^-1).  This reproduces the toy example's 6/6.2 = 0.968.      */
/* Step 3 (FP4 conversion).  v = x * r_b rounded to E2M1: nearest-even for   */
/* activations and weights, stochastic for gradients.                        */
/* ------------------------------------------------------------------------ */
typedef struct {
  float s_enc, s6, g;
} oracle_tensor_scales;

static int tensor_scales_from_amax(float amax, oracle_tensor_scales* ts) {
  if (!isfinite(amax)) return ORACLE_ERR_NONFINITE;
  if (amax == 0.0f) {
    ts->s_enc = 1.0f;
    ts->g = 1.0f;
    ts->s6 = 1.0f / 6.0f;
    return ORACLE_OK;
  }
  float s_enc = 2688.0f / amax;
  if (isinf(s_enc)) s_enc = FLT_MAX;
  ts->s_enc = s_enc;
  ts->g = 1.0f / s_enc;
  ts->s6 = s_enc / 6.0f;
  return ORACLE_OK;
}

/* One block: n values -> d_b code + codes.  r16 may be NULL for RN. */
static void quantize_block(const float* vals, int n, const oracle_tensor_scales* ts,
                           const uint32_t* r16, uint8_t* codes, uint8_t* scale_code) {
  float amax_b = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = fabsf(vals[i]);
    if (a > amax_b) amax_b = a;
  }
  float t = amax_b * ts->s6;
  uint8_t d_code = oracle_e4m3_encode(t);
  float d_b = (float)oracle_e4m3_decode(d_code);
  float r_b = (d_b == 0.0f) ? 0.0f : ts->s_enc / d_b;
  /* Reading for tensors so small that s_enc saturated: the multiplier is
   * clamped to the largest finite fp32 as well, so v stays finite. */
  if (isinf(r_b)) r_b = FLT_MAX;
  for (int i = 0; i < n; ++i) {
    float v = vals[i] * r_b;
    float m = fabsf(v);
    int idx = r16 ? oracle_e2m1_sr_index(m, r16[i]) : oracle_e2m1_rn_index(m);
    uint8_t sign = signbit(vals[i]) ? 8 : 0;
    codes[i] = (uint8_t)(sign | idx);
  }
  *scale_code = d_code;
}

/*
 * Quantise one operand with 1x16 blocks.
 *   x          : fp32 source, [src_rows, src_cols], leading dimension ld.
 *   transpose  : 0 -> operand = x ([R, C] = [src_rows, src_cols]);
 *                1 -> operand = x^T ([R, C] = [src_cols, src_rows]).
 *   rht        : apply the RHT to each 16-chunk along the operand's C axis
 *                (the block axis) before anything else.
 *   round_mode : 0 = nearest-even, 1 = stochastic.
 *   seed, offset, stream : SR random source (see oracle_sr_bits).
 * Outputs: codes [R][C/2] (low nibble = even column), scales [R][C/16]
 * (E4M3 bytes), g_out = 1/s_enc.  Returns 0, or ORACLE_ERR_NONFINITE when
 * the operand's amax is not finite (outputs then untouched), or
 * ORACLE_ERR_SHAPE when C is not a multiple of 16.
 */
int oracle_quantize(const float* x, int64_t src_rows, int64_t src_cols, int64_t ld,
                    int transpose, int rht, uint32_t signs, int round_mode,
                    uint64_t seed, uint64_t offset, uint32_t stream,
                    uint8_t* codes, uint8_t* scales, float* g_out) {
  int64_t R = transpose ? src_cols : src_rows;
  int64_t C = transpose ? src_rows : src_cols;
  if (C % 16 != 0 || R <= 0) return ORACLE_ERR_SHAPE;
  float* op = (float*)malloc(sizeof(float) * (size_t)(R * C));
  if (!op) return ORACLE_ERR_SHAPE;
  /* the operand in its own layout */
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < R; ++i)
    for (int64_t j = 0; j < C; ++j)
      op[i * C + j] = transpose ? x[j * ld + i] : x[i * ld + j];
  if (rht) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i)
      for (int64_t j = 0; j < C; j += 16) {
        float y[16];
        oracle_rht16_chunk(op + i * C + j, signs, y);
        memcpy(op + i * C + j, y, sizeof(y));
      }
  }
  /* Step 1: tensor amax and the FP32 scale */
  float amax = 0.0f;
  int nonfinite = 0;
  for (int64_t k = 0; k < R * C; ++k) {
    float a = fabsf(op[k]);
    if (!isfinite(a)) nonfinite = 1;
    if (a > amax) amax = a;
  }
  oracle_tensor_scales ts;
  if (nonfinite || tensor_scales_from_amax(amax, &ts) != ORACLE_OK) {
    free(op);
    return ORACLE_ERR_NONFINITE;
  }
  /* Steps 2-3 per 1x16 block */
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < R; ++i) {
    for (int64_t b = 0; b < C / 16; ++b) {
      uint32_t r16[16];
      uint8_t blk_codes[16];
      if (round_mode == 1)
        for (int t = 0; t < 16; ++t)
          r16[t] = oracle_sr_bits(seed, stream, offset + (uint64_t)(i * C + b * 16 + t));
      quantize_block(op + i * C + b * 16, 16, &ts, round_mode == 1 ? r16 : NULL,
                     blk_codes, &scales[i * (C / 16) + b]);
      for (int t = 0; t < 8; ++t)
        codes[i * (C / 2) + b * 8 + t] =
            (uint8_t)(blk_codes[2 * t] | (blk_codes[2 * t + 1] << 4));
    }
  }
  *g_out = ts.g;
  free(op);
  return ORACLE_OK;
}

/*
 * 2D 16x16 weight quantisation [Review s2; Review "Core idea", recipe item
 * (2)]: weights get one scale per 16x16 tile so that the forward and the
 * backward GEMM read the identical quantised weight.  Nearest-even only.  w is [rows, cols] (output x
 * input channels); one E4M3 scale per 16x16 tile, grid [rows/16][cols/16].
 * The transposed copy (codes_t [cols][rows/2], grid_t [cols/16][rows/16]) is
 * the element-wise transpose of the same codes and scales with the same g:
 * the backward pass sees exactly the forward pass's quantised weight.
 * codes_t / grid_t may be NULL.
 */
int oracle_quantize_2d(const float* w, int64_t rows, int64_t cols, int64_t ld,
                       uint8_t* codes, uint8_t* grid, uint8_t* codes_t,
                       uint8_t* grid_t, float* g_out) {
  if (rows % 16 || cols % 16 || rows <= 0) return ORACLE_ERR_SHAPE;
  float amax = 0.0f;
  int nonfinite = 0;
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < cols; ++j) {
      float a = fabsf(w[i * ld + j]);
      if (!isfinite(a)) nonfinite = 1;
      if (a > amax) amax = a;
    }
  oracle_tensor_scales ts;
  if (nonfinite || tensor_scales_from_amax(amax, &ts) != ORACLE_OK)
    return ORACLE_ERR_NONFINITE;
  int64_t GR = rows / 16, GC = cols / 16;
  uint8_t* full = (uint8_t*)malloc((size_t)(rows * cols)); /* one code per byte */
  if (!full) return ORACLE_ERR_SHAPE;
#pragma omp parallel for schedule(static)
  for (int64_t bi = 0; bi < GR; ++bi) {
    for (int64_t bj = 0; bj < GC; ++bj) {
      float tile[256];
      uint8_t tc[256];
      for (int r = 0; r < 16; ++r)
        for (int c = 0; c < 16; ++c) tile[r * 16 + c] = w[(bi * 16 + r) * ld + bj * 16 + c];
      quantize_block(tile, 256, &ts, NULL, tc, &grid[bi * GC + bj]);
      for (int r = 0; r < 16; ++r)
        for (int c = 0; c < 16; ++c) full[(bi * 16 + r) * cols + bj * 16 + c] = tc[r * 16 + c];
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < cols; j += 2)
      codes[i * (cols / 2) + j / 2] =
          (uint8_t)(full[i * cols + j] | (full[i * cols + j + 1] << 4));
  if (codes_t) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < cols; ++j)
      for (int64_t i = 0; i < rows; i += 2)
        codes_t[j * (rows / 2) + i / 2] =
            (uint8_t)(full[i * cols + j] | (full[(i + 1) * cols + j] << 4));
  }
  if (grid_t) {
    for (int64_t bi = 0; bi < GR; ++bi)
      for (int64_t bj = 0; bj < GC; ++bj) grid_t[bj * GR + bi] = grid[bi * GC + bj];
  }
  *g_out = ts.g;
  free(full);
  return ORACLE_OK;
}

/*
 * Dequantise [Review s1 Step 3: decoding divides by the product of the block
 * and global encode scales]: x_hat = decode(code) * d_b * g in float64.  scale_mode 0: grid [R][C/16];
 * 1: grid [R/16][C/16].
 */
void oracle_dequant(const uint8_t* codes, const uint8_t* scales, float g, int64_t R,
                    int64_t C, int scale_mode, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < R; ++i) {
    for (int64_t j = 0; j < C; ++j) {
      uint8_t byte = codes[i * (C / 2) + j / 2];
      uint8_t code = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);
      uint8_t sc = scale_mode == 0 ? scales[i * (C / 16) + j / 16]
                                   : scales[(i / 16) * (C / 16) + j / 16];
      out[i * C + j] = oracle_e2m1_decode(code) * oracle_e4m3_decode(sc) * (double)g;
    }
  }
}

/*
 * NVFP4 GEMM entries [Review s6: y = GEMM(x_FP4, W_FP4); Captions Fig. 5:
 * every GEMM quantises its inputs]: C[m][n] = sum_k a_hat[m][k] * b_hat[n][k]
 * in float64 over dequantised operands (both contiguous along k), plus
 * S[m][n] = sum_k |a_hat[m][k] * b_hat[n][k]| for the tolerance bound.
 * Computed for a list of (m, n) pairs, one entry at a time.
 */
void oracle_gemm_entries(const double* a_hat, const double* b_hat, int64_t K,
                         const int64_t* ms, const int64_t* ns, int64_t count,
                         double* c_out, double* s_out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < count; ++t) {
    const double* a = a_hat + ms[t] * K;
    const double* b = b_hat + ns[t] * K;
    double c = 0.0, s = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double p = a[k] * b[k];
      c += p;
      s += fabs(p);
    }
    c_out[t] = c;
    s_out[t] = s;
  }
}

/* ------------------------------------------------------------------------ */
/* Array forms of the scalar steps, so tests can sweep many inputs.          */
/* ------------------------------------------------------------------------ */
void oracle_e4m3_encode_n(const float* t, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(t[i]);
}

void oracle_e2m1_rn_index_n(const float* m, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e2m1_rn_index(m[i]);
}

void oracle_e2m1_sr_index_n(const float* m, const uint32_t* r16, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e2m1_sr_index(m[i], r16[i]);
}

void oracle_sr_bits_n(uint64_t seed, uint32_t stream, uint64_t e0, int64_t n, uint32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_sr_bits(seed, stream, e0 + (uint64_t)i);
}

/* ------------------------------------------------------------------------ */
/* MXFP4, the comparator format the pages weigh NVFP4 against [Review      */
/* "secret weapon" items 1-2; Captions Fig. 6: blocks of 32 E2M1 values     */
/* sharing one power-of-two UE8M0 scale, no tensor scale; the pages         */
/* attribute its loss                                                       */
/* to that power-of-two rounding dropping a binade (values near +-4, +-6)].  */
/* The pages do not spell the scale rule out; the reading taken is the OCP  */
/* Microscaling rule: X = 2^e with e = floor(log2(amax_b)) - 2 (2 is E2M1's */
/* largest exponent), so amax_b / X lies in [4, 8) and anything at or above */
/* 6 X saturates to 6 X -- which is exactly the lost binade.  e is clamped  */
/* to E8M0's range [-127, 127]; an all-zero block stores e = -127 (code 0). */
/* Elements: v = x / X (exact: a power of two), nearest-even E2M1,          */
/* saturating.  A block holding Inf or NaN stores the E8M0 NaN code 0xFF    */
/* and its codes are unspecified (here 0).                                  */
/* ------------------------------------------------------------------------ */

/* floor(log2(a)) of a positive finite fp32 value, exactly (from its bits). */
static int floor_log2_f32(float a) {
  uint32_t b;
  memcpy(&b, &a, 4);
  const int ef = (int)((b >> 23) & 0xFF);
  if (ef > 0) return ef - 127;
  /* subnormal: value = mantissa * 2^-149 */
  uint32_t m = b & 0x7FFFFF;
  int lg = 0;
  while (m >>= 1) ++lg;
  return lg - 149;
}

/* One MX block of n (<= 32) values: returns the E8M0 scale code, writes the
 * 4-bit codes. */
uint8_t oracle_mx_block(const float* x, int n, uint8_t* codes) {
  float amax = 0.0f;
  int finite = 1;
  for (int i = 0; i < n; ++i) {
    if (!isfinite(x[i])) finite = 0;
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  if (!finite) {
    for (int i = 0; i < n; ++i) codes[i] = 0;
    return 0xFF;
  }
  int e = amax > 0.0f ? floor_log2_f32(amax) - 2 : -127;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  for (int i = 0; i < n; ++i) {
    const double v = ldexp((double)x[i], -e); /* exact */
    const double m = fabs(v);
    /* nearest-even onto the grid on the exact magnitude; m < 8 always, and
     * anything >= 6 saturates (the page's lost binade) */
    int idx;
    if (m >= 6.0)
      idx = 7;
    else
      idx = oracle_e2m1_rn_index((float)m); /* m = |x| 2^-e is exact in fp32 too */
    codes[i] = (uint8_t)((signbit(x[i]) ? 8 : 0) | idx);
  }
  return (uint8_t)(e + 127);
}

/* MXFP4 quantisation of x [rows, cols] (leading dim ld) with 32-element
 * blocks along cols (cols % 32 == 0): codes [rows][cols/2] (even column in the
 * low nibble), scales E8M0 [rows][cols/32]. */
int oracle_mx_quantize(const float* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                       uint8_t* scales) {
  if (rows <= 0 || cols <= 0 || cols % 32 != 0) return ORACLE_ERR_SHAPE;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < rows; ++i) {
    for (int64_t b = 0; b < cols / 32; ++b) {
      uint8_t c[32];
      scales[i * (cols / 32) + b] = oracle_mx_block(x + i * ld + b * 32, 32, c);
      for (int j = 0; j < 32; j += 2)
        codes[i * (cols / 2) + b * 16 + j / 2] = (uint8_t)(c[j] | (c[j + 1] << 4));
    }
  }
  return ORACLE_OK;
}

/* E8M0 scale value 2^(code - 127); code 0xFF is NaN. */
double oracle_e8m0_decode(uint8_t code) {
  return code == 0xFF ? NAN : ldexp(1.0, (int)code - 127);
}

/* Dequantise an MXFP4 operand: x_hat = e2m1(code) * 2^(scale - 127), float64. */
void oracle_mx_dequant(const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t C,
                       double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < R; ++i)
    for (int64_t j = 0; j < C; ++j) {
      uint8_t byte = codes[i * (C / 2) + j / 2];
      uint8_t code = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);
      out[i * C + j] = oracle_e2m1_decode(code) * oracle_e8m0_decode(scales[i * (C / 32) + j / 32]);
    }
}

/* ------------------------------------------------------------------------ */
/* Random Hadamard transforms of other sizes [Review s3 and its size note:  */
/* d = 16 is the recipe, d = 4 and d = 128 the sizes the pages compare it   */
/* against; Captions Fig. 12].  y = c * H_d * diag(s) * x per d-element     */
/* chunk, H_d Sylvester, c = fp32(1/sqrt(d)) (orthonormal; exact for d = 4  */
/* and 16).  fp32 order as for d = 16: signs, butterflies h = 1, 2, ...,    */
/* d/2 as (a+b, a-b), then x c.  Signs: bit i of the 128-bit Philox4x32-10  */
/* block (counter 0, key = seed), word 0 first, least significant bit      */
/* first -- the low 16 bits are exactly the d = 16 mask above.               */
/* ------------------------------------------------------------------------ */
void oracle_rht_signs128_from_seed(uint64_t seed, uint32_t out[4]) {
  const uint32_t ctr[4] = {0u, 0u, 0u, 0u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  oracle_philox4x32_10(ctr, key, out);
}

void oracle_rht_chunk_d(const float* x, int d, const uint32_t signs[4], float* y) {
  float u[128];
  for (int i = 0; i < d; ++i) u[i] = ((signs[i / 32] >> (i % 32)) & 1u) ? -x[i] : x[i];
  for (int h = 1; h < d; h *= 2) {
    for (int i = 0; i < d; ++i) {
      if (i & h) continue;
      float a = u[i], b = u[i + h];
      u[i] = a + b;
      u[i + h] = a - b;
    }
  }
  const float c = (float)(1.0 / sqrt((double)d));
  for (int i = 0; i < d; ++i) y[i] = u[i] * c;
}

/* RHT of size d (4, 16 or 128) of a [rows, cols] fp32 matrix: axis 1 chunks
 * along each row, axis 0 along each column; output dense [rows, cols]. */
int oracle_rht_d(const float* x, int64_t rows, int64_t cols, int64_t ld, int axis, int d,
                 const uint32_t signs[4], float* y) {
  if (d != 4 && d != 16 && d != 128) return ORACLE_ERR_SHAPE;
  if (axis == 1) {
    if (cols % d) return ORACLE_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t c = 0; c < cols; c += d) oracle_rht_chunk_d(x + r * ld + c, d, signs, y + r * cols + c);
  } else {
    if (rows % d) return ORACLE_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
      for (int64_t r = 0; r < rows; r += d) {
        float in[128], out[128];
        for (int i = 0; i < d; ++i) in[i] = x[(r + i) * ld + c];
        oracle_rht_chunk_d(in, d, signs, out);
        for (int i = 0; i < d; ++i) y[(r + i) * cols + c] = out[i];
      }
    }
  }
  return ORACLE_OK;
}
