/*
 * NVFP4 W4A4 + Residual Activation Compensation (RAC): the CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously-correct scalar C that
 * defines the numbers the GPU library must reproduce.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load this code; the
 * product path never does.  It shares no code, header or table with the HIP
 * library.
 *
 * Sources (cited by page title and section):
 *  [ABS]  QUADS arXiv abstract, as reproduced on the mlsanity paper page
 *         ("QUADS: Stabilizing NVFP4 Reinforcement Learning for MoE ...",
 *         section "Abstract (arXiv)"): NVFP4 pairs per-block scale factors
 *         with 4-bit E2M1 values and multiplies 4-bit weights by 4-bit
 *         activations; rollout activations are new at every step and are
 *         quantized at run time; RAC repairs the activation channels whose
 *         quantization error is worst and keeps the 4-bit GEMMs.
 *  [FAIL] Blog post "Why 4-bit RL rollout collapses - and it isn't the
 *         weights", section "The failure mode": E2M1 can represent eight
 *         magnitudes for each sign; every rollout engine quantizes the
 *         synchronized weights the same way.
 *  [FIX]  Same blog post, section "Two fixes, on two different sides": about
 *         half of the activation channels, those with the largest error,
 *         also go through a second 4-bit GEMM on their quantized residual,
 *         in the same kernels; the ordinary 4-bit pass is unchanged.
 *
 * The pages fix neither the block size, the scale encodings, the rounding
 * mode, the error metric nor the tie-breaks.  This file implements the
 * standard NVFP4 layout (E2M1 elements, one E4M3 scale per 16 consecutive
 * elements along K, one FP32 tensor scale amax/(6*448)), round-to-nearest-even
 * everywhere with saturation, and the readings stated at each function.
 *
 * Floating point: every step is one IEEE operation in the precision written;
 * build with -O2 -fno-fast-math -ffp-contract=off so that no step is fused.
 * Exact integer arithmetic is used where the definition is a sum (channel
 * score, GEMM) so that the result does not depend on summation order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#pragma STDC FP_CONTRACT OFF

/* ---------------------------------------------------------------- formats */

/* E2M1 magnitudes, indexed by the 3 low bits of a code [FAIL: 8 levels per
 * sign]; bit 3 is the sign. */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double or_e2m1_value(int code) {
  double g = E2M1_GRID[code & 7];
  return (code & 8) ? -g : g;
}

/* OCP E4M3 (FN variant): sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent field 0 is subnormal m*2^-9; 0x7F/0xFF are NaN; max 448. */
double or_e4m3_value(int byte) {
  int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

/* Nearest E4M3 value to rho >= 0, ties to the even code, saturating at 448.
 * Positive E4M3 codes are monotone in value, so "even code" is "even
 * mantissa LSB". */
int or_e4m3_encode(float rho) {
  double r = (double)rho;
  int ex, E, code;
  double f, sig, q;
  if (!(r > 0.0)) return 0;
  if (r >= 448.0) return 0x7E;
  if (r < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9; 8*2^-9 = 2^-6 is code 0x08 */
    return (int)nearbyint(ldexp(r, 9));
  }
  f = frexp(r, &ex); /* r = f * 2^ex, f in [0.5, 1) */
  E = ex - 1;
  sig = f * 2.0;                      /* [1, 2), exact */
  q = nearbyint((sig - 1.0) * 8.0);   /* 0..8, ties to even */
  if (q == 8.0) { E += 1; q = 0.0; }
  code = ((E + 7) << 3) | (int)q;
  if (code > 0x7E) code = 0x7E;       /* 464..480 would round to NaN: clamp */
  return code;
}

/* Index of the grid magnitude nearest to a >= 0, ties to the even index;
 * anything above 6 saturates to 6. */
static int e2m1_index(float a) {
  int best = 0, i;
  double bd, d;
  if ((double)a > 6.0) return 7;
  bd = fabs((double)a - E2M1_GRID[0]);
  for (i = 1; i < 8; i++) {
    d = fabs((double)a - E2M1_GRID[i]);
    if (d < bd || (d == bd && (i % 2) == 0)) { best = i; bd = d; }
  }
  return best;
}

int or_e2m1_encode(float v) {
  int idx = e2m1_index(fabsf(v));
  return (v < 0.0f && idx != 0) ? (8 | idx) : idx; /* never -0 */
}

/* ------------------------------------------------------------ quantizer */

/* Tensor scale s_t = RN32(amax / (6*448)); the division is done in double
 * and rounded once to float. */
float or_tensor_scale(float amax) {
  return (float)((double)amax / 2688.0);
}

/* Per-block scale code: rho = RN32(RN64(amax_b / RN64(6*s_t))), then the
 * nearest E4M3. */
int or_block_scale_code(float amax_b, float s_t) {
  float rho;
  if (s_t == 0.0f) return 0;
  rho = (float)((double)amax_b / (6.0 * (double)s_t));
  return or_e4m3_encode(rho);
}

static float e4m3_f(int byte) { return (float)or_e4m3_value(byte); }

/* Quantize one 16-element block (n elements at stride 1) with tensor scale
 * s_t: returns the scale code and writes 16 element codes. */
static int quantize_block(const float* x, float s_t, uint8_t* elem_codes) {
  float amax_b = 0.0f, sb, Sb, rb, v;
  int i, sc;
  for (i = 0; i < 16; i++) {
    float a = fabsf(x[i]);
    if (a > amax_b) amax_b = a;
  }
  sc = or_block_scale_code(amax_b, s_t);
  sb = e4m3_f(sc);
  Sb = sb * s_t;                                     /* RN32 */
  rb = (Sb > 0.0f) ? (float)(1.0 / (double)Sb) : 0.0f; /* RN32(1/Sb) */
  for (i = 0; i < 16; i++) {
    v = x[i] * rb;                                   /* RN32 */
    elem_codes[i] = (uint8_t)or_e2m1_encode(v);
  }
  return sc;
}

/* Block-quantize every row of x[rows, K] (row stride ldx) with the tensor
 * scale s_t: per 16-block scale byte and E2M1 codes, packed. */
static void quantize_rows(const float* x, int64_t rows, int64_t K, int64_t ldx, float s_t,
                          uint8_t* codes, uint8_t* scales) {
  int64_t r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < rows; r++) {
    uint8_t ec[16];
    for (int64_t b = 0; b < K / 16; b++) {
      int sc = quantize_block(x + r * ldx + b * 16, s_t, ec);
      scales[r * (K / 16) + b] = (uint8_t)sc;
      for (int i = 0; i < 16; i += 2)
        codes[r * (K / 2) + b * 8 + i / 2] = (uint8_t)(ec[i] | (ec[i + 1] << 4));
    }
  }
}

/* NVFP4-quantize x[rows, K] (row stride ldx floats).
 * codes[rows, K/2]: element 2j in the low nibble of byte j, 2j+1 in the high.
 * scales[rows, K/16]: E4M3 bytes.  *tscale_out = s_t.
 * amax_in (nullable) replaces max|x| as the tensor amax. */
int or_quantize(const float* x, int64_t rows, int64_t K, int64_t ldx,
                const float* amax_in, uint8_t* codes, uint8_t* scales,
                float* tscale_out) {
  float amax = 0.0f, s_t;
  int64_t r;
  if (K % 16 != 0) return 2;
  (void)r;
  if (amax_in) {
    amax = *amax_in;
  } else {
    for (r = 0; r < rows; r++)
      for (int64_t k = 0; k < K; k++) {
        float a = fabsf(x[r * ldx + k]);
        if (a > amax) amax = a;
      }
  }
  s_t = or_tensor_scale(amax);
  *tscale_out = s_t;
  quantize_rows(x, rows, K, ldx, s_t, codes, scales);
  return 0;
}

static int get_code(const uint8_t* codes, int64_t K, int64_t r, int64_t k) {
  uint8_t byte = codes[r * (K / 2) + k / 2];
  return (k & 1) ? (byte >> 4) : (byte & 15);
}

/* Dequantized element in FP32: RN32(RN32(g * s_b) * s_t); g*s_b is exact. */
float or_dequant(int code, int scale_byte, float s_t) {
  float t = (float)or_e2m1_value(code) * e4m3_f(scale_byte);
  return t * s_t;
}

void or_dequantize(const uint8_t* codes, const uint8_t* scales, float s_t,
                   int64_t rows, int64_t K, float* out) {
  int64_t r, k;
  for (r = 0; r < rows; r++)
    for (k = 0; k < K; k++)
      out[r * K + k] = or_dequant(get_code(codes, K, r, k),
                                  scales[r * (K / 16) + k / 16], s_t);
}

/* ----------------------------------------------------- RAC: error, score */

/* Quantization error e = x - deq(q(x)), one FP32 subtraction. */
static float quant_error(const float* x, int64_t ldx, const uint8_t* codes,
                         const uint8_t* scales, float s_t, int64_t K,
                         int64_t r, int64_t k) {
  float d = or_dequant(get_code(codes, K, r, k), scales[r * (K / 16) + k / 16], s_t);
  return x[r * ldx + k] - d;
}

/* Fixed-point exponent of the score: q = floor(|e| * 2^(8 - Es)) where Es is
 * the frexp exponent of s_t (s_t = f * 2^Es, f in [0.5, 1)).  Since
 * |e| <= S_b <= ~448 s_t, q < 2^17; q is clamped to 2^17 - 1 so that the
 * integer sums stay bounded even when a caller's amax under-estimates max|x|. */
int or_score_shift(float s_t) {
  int es = 0;
  if (s_t != 0.0f) frexp((double)s_t, &es);
  return 8 - es;
}

int64_t or_score_term(float e, int shift) {
  double q = floor(ldexp(fabs((double)e), shift));
  if (q > 131071.0) q = 131071.0;
  return (int64_t)q * (int64_t)q;
}

/* Per-channel quantization-error statistics over all rows of the call
 * [FIX: channels are ranked by their quantization error].
 * A channel is one K column of the GEMM input.  score[k] = sum over rows of
 * q^2 (exact int64: the sum of squared errors in fixed point);
 * chmax[k] = max over rows of |e|. */
void or_channel_stats(const float* x, int64_t rows, int64_t K, int64_t ldx,
                      const uint8_t* codes, const uint8_t* scales, float s_t,
                      int64_t* score, float* chmax) {
  int shift = or_score_shift(s_t);
  int64_t k;
#pragma omp parallel for schedule(static)
  for (k = 0; k < K; k++) {
    int64_t acc = 0;
    float mx = 0.0f;
    for (int64_t r = 0; r < rows; r++) {
      float e = quant_error(x, ldx, codes, scales, s_t, K, r, k);
      acc += or_score_term(e, shift);
      if (fabsf(e) > mx) mx = fabsf(e);
    }
    score[k] = acc;
    chmax[k] = mx;
  }
}

/* ------------------------------------------------------ RAC: selection */

typedef struct { int64_t score; int32_t k; } key_t_;

static int key_cmp(const void* a, const void* b) {
  const key_t_* x = (const key_t_*)a;
  const key_t_* y = (const key_t_*)b;
  if (x->score != y->score) return (x->score > y->score) ? -1 : 1; /* desc */
  return (x->k < y->k) ? -1 : (x->k > y->k);                       /* asc */
}

static int int_cmp(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x < y) ? -1 : (x > y);
}

/* Select the n_sel channels with the largest score, ties toward the lower
 * channel index [FIX: "roughly top-50%"; n_sel = K/2 exactly in the
 * workloads].  Outputs: selected[n_sel] ascending, mask[K], active[K/16]
 * (block holds a selected channel), and res_amax = max over the selected
 * channels of chmax[k], which is max|r| of the residual. */
void or_rac_select(const int64_t* score, const float* chmax, int64_t K,
                   int64_t n_sel, int32_t* selected, uint8_t* mask,
                   uint8_t* active, float* res_amax) {
  key_t_* keys = (key_t_*)malloc(sizeof(key_t_) * (size_t)(K > 0 ? K : 1));
  float amax_r = 0.0f;
  int64_t i;
  for (i = 0; i < K; i++) { keys[i].score = score[i]; keys[i].k = (int32_t)i; }
  qsort(keys, (size_t)K, sizeof(key_t_), key_cmp);
  memset(mask, 0, (size_t)K);
  for (i = 0; i < n_sel; i++) {
    selected[i] = keys[i].k;
    mask[keys[i].k] = 1;
    if (chmax[keys[i].k] > amax_r) amax_r = chmax[keys[i].k];
  }
  qsort(selected, (size_t)n_sel, sizeof(int32_t), int_cmp);
  for (i = 0; i < K / 16; i++) {
    int any = 0;
    for (int j = 0; j < 16; j++) any |= mask[i * 16 + j];
    active[i] = (uint8_t)any;
  }
  *res_amax = amax_r;
  free(keys);
}

/* Masked residual r = mask * e, re-quantized to NVFP4 in the same 16-element
 * blocks [FIX: the selected channels' residual goes through a second 4-bit
 * pass inside the same kernels].  Reading: the residual pass uses the main
 * pass's tensor scale s_t -- its block scales are E4M3(RN32(max|r_b| /
 * (6 s_t))) and its codes follow N2-N4 with that s_t -- so that both passes of
 * the GEMM share the activation's tensor scale.  *res_tscale_out = s_t.
 * Every residual block scale stays within E4M3's range: |r| <= max|x|. */
void or_rac_residual(const float* x, int64_t rows, int64_t K, int64_t ldx,
                     const uint8_t* codes, const uint8_t* scales, float s_t,
                     const uint8_t* mask, uint8_t* res_codes,
                     uint8_t* res_scales, float* res_tscale_out,
                     float* res_out /* nullable [rows, K] */) {
  float* r = (float*)malloc(sizeof(float) * (size_t)(rows * K > 0 ? rows * K : 1));
  int64_t i, k;
  for (i = 0; i < rows; i++)
    for (k = 0; k < K; k++)
      r[i * K + k] = mask[k] ? quant_error(x, ldx, codes, scales, s_t, K, i, k) : 0.0f;
  quantize_rows(r, rows, K, K, s_t, res_codes, res_scales);
  *res_tscale_out = s_t;
  if (res_out) memcpy(res_out, r, sizeof(float) * (size_t)(rows * K));
  free(r);
}

/* ------------------------------------------------------------- the GEMM */

/* Exact integer image of one dequantized operand element:
 * (2 g) * (s_b * 2^9); every E2M1 value is a multiple of 1/2 and every E4M3
 * value a multiple of 2^-9, so g * s_b = image * 2^-10. */
static int64_t elem_int(const uint8_t* codes, const uint8_t* scales, int64_t K,
                        int64_t r, int64_t k) {
  int c = get_code(codes, K, r, k);
  double v = or_e2m1_value(c) * 2.0 * or_e4m3_value(scales[r * (K / 16) + k / 16]) * 512.0;
  return (int64_t)v; /* exact */
}

static int64_t dot_int(const uint8_t* ac, const uint8_t* as, int64_t ar,
                       const uint8_t* wc, const uint8_t* ws, int64_t wr,
                       int64_t K) {
  int64_t acc = 0, k;
  for (k = 0; k < K; k++)
    acc += elem_int(ac, as, K, ar, k) * elem_int(wc, ws, K, wr, k);
  return acc;
}

static int64_t group_of(const int32_t* offsets, int64_t G, int64_t j) {
  int64_t g;
  for (g = 0; g < G; g++)
    if (j >= offsets[g] && j < offsets[g + 1]) return g;
  return -1;
}

/* One output of the grouped W4A4 GEMM with RAC:
 *   Y[j, n] = s_tw[g] * (s_ta * sum_k A[src,k] W_g[n,k] + s_tr * sum_k R[src,k] W_g[n,k])
 * where A, R, W are the dequantized g*s_b values, g is the group (expert) of
 * output row j, src = gather[j] (or j).  Both sums are exact int64 sums of
 * the integer images (scaled by 2^-20); they are combined in long double and
 * rounded once to float.  Residual terms are dropped when r_codes is NULL
 * (naive W4A4).  [ABS: 4-bit by 4-bit GEMMs; FIX: the ordinary pass is
 * unchanged and the residual pass adds to it.] */
static void gemm_one(int64_t G, int64_t N, int64_t K, const int32_t* offsets,
                     const int32_t* gather, const uint8_t* a_codes,
                     const uint8_t* a_scales, float a_ts,
                     const uint8_t* r_codes, const uint8_t* r_scales, float r_ts,
                     const uint8_t* w_codes, const uint8_t* w_scales,
                     const float* w_ts, const float* a_ts_g, const float* r_ts_g,
                     int64_t j, int64_t n, float* out, int64_t* main_sum, int64_t* res_sum) {
  int64_t g = group_of(offsets, G, j);
  if (a_ts_g) a_ts = a_ts_g[g];
  if (r_ts_g) r_ts = r_ts_g[g];
  int64_t src = gather ? gather[j] : j;
  int64_t wr = g * N + n; /* row of the [G*N, K] weight image */
  int64_t m = dot_int(a_codes, a_scales, src, w_codes, w_scales, wr, K);
  int64_t rs = 0;
  long double y;
  if (r_codes) rs = dot_int(r_codes, r_scales, src, w_codes, w_scales, wr, K);
  y = (long double)a_ts * ldexpl((long double)m, -20);
  if (r_codes) y += (long double)r_ts * ldexpl((long double)rs, -20);
  y *= (long double)w_ts[g];
  *out = (float)y;
  if (main_sum) *main_sum = m;
  if (res_sum) *res_sum = rs;
}

/* Integer images of a whole quantized matrix [rows, K] (see elem_int). */
static int32_t* int_image(const uint8_t* codes, const uint8_t* scales,
                          int64_t rows, int64_t K) {
  int32_t* img = (int32_t*)malloc(sizeof(int32_t) * (size_t)(rows * K > 0 ? rows * K : 1));
  int64_t r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < rows; r++)
    for (int64_t k = 0; k < K; k++)
      img[r * K + k] = (int32_t)elem_int(codes, scales, K, r, k);
  return img;
}

/* Full grouped GEMM: out[total_rows, N] (rows in group order), the same
 * definition as gemm_one with the operands decoded once.  src_rows is the
 * number of rows of A (and R); main_sum and res_sum (nullable) receive the
 * exact integer sums.  a_ts_g / r_ts_g (nullable, [G]) replace the scalar
 * activation and residual tensor scales by per-group ones (per-expert RAC). */
void or_grouped_gemm(int64_t G, int64_t N, int64_t K, int64_t total_rows,
                     int64_t src_rows, const int32_t* offsets,
                     const int32_t* gather,
                     const uint8_t* a_codes, const uint8_t* a_scales, float a_ts,
                     const uint8_t* r_codes, const uint8_t* r_scales, float r_ts,
                     const uint8_t* w_codes, const uint8_t* w_scales,
                     const float* w_ts, float* out, int64_t* main_sum,
                     int64_t* res_sum, const float* a_ts_g, const float* r_ts_g) {
  int32_t* ai = int_image(a_codes, a_scales, src_rows, K);
  int32_t* ri = r_codes ? int_image(r_codes, r_scales, src_rows, K) : NULL;
  int32_t* wi = int_image(w_codes, w_scales, G * N, K);
  int64_t idx;
#pragma omp parallel for schedule(dynamic, 64)
  for (idx = 0; idx < total_rows * N; idx++) {
    int64_t j = idx / N, n = idx % N;
    int64_t g = group_of(offsets, G, j);
    int64_t src = gather ? gather[j] : j;
    const int32_t* w = wi + (g * N + n) * K;
    int64_t m = 0, rs = 0, k;
    long double y;
    for (k = 0; k < K; k++) m += (int64_t)ai[src * K + k] * w[k];
    if (ri)
      for (k = 0; k < K; k++) rs += (int64_t)ri[src * K + k] * w[k];
    y = (long double)(a_ts_g ? a_ts_g[g] : a_ts) * ldexpl((long double)m, -20);
    if (ri) y += (long double)(r_ts_g ? r_ts_g[g] : r_ts) * ldexpl((long double)rs, -20);
    y *= (long double)w_ts[g];
    out[idx] = (float)y;
    if (main_sum) main_sum[idx] = m;
    if (res_sum) res_sum[idx] = rs;
  }
  free(ai);
  free(ri);
  free(wi);
}

/* Sampled outputs: out[i] = Y[rows[i], cols[i]]. */
void or_grouped_gemm_sample(int64_t G, int64_t N, int64_t K,
                            const int32_t* offsets, const int32_t* gather,
                            const uint8_t* a_codes, const uint8_t* a_scales, float a_ts,
                            const uint8_t* r_codes, const uint8_t* r_scales, float r_ts,
                            const uint8_t* w_codes, const uint8_t* w_scales,
                            const float* w_ts, int64_t n_samples,
                            const int64_t* rows, const int64_t* cols, float* out,
                            const float* a_ts_g, const float* r_ts_g) {
  int64_t i;
#pragma omp parallel for schedule(dynamic, 16)
  for (i = 0; i < n_samples; i++)
    gemm_one(G, N, K, offsets, gather, a_codes, a_scales, a_ts, r_codes,
             r_scales, r_ts, w_codes, w_scales, w_ts, a_ts_g, r_ts_g, rows[i],
             cols[i], out + i, NULL, NULL);
}

/* ---------------------------------------------------------- SiLU * mul */

/* bf16 round-to-nearest-even of a double, returned as the bf16 bit pattern
 * (8 significant bits, FP32 exponent range, subnormals down to 2^-133). */
uint16_t or_bf16_rne(double v) {
  double a = fabs(v), q;
  int ex;
  float f;
  uint32_t bits;
  if (a == 0.0) return (uint16_t)(signbit(v) ? 0x8000 : 0);
  frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1): quantum 2^(ex-8) */
  if (ex - 8 < -133) ex = -133 + 8;
  q = nearbyint(ldexp(a, 8 - ex));
  a = ldexp(q, ex - 8);
  f = (float)a; /* exact: at most 8 significant bits, in float range */
  if (v < 0) f = -f;
  memcpy(&bits, &f, 4);
  return (uint16_t)(bits >> 16);
}

/* h = bf16(silu(g) * u) with silu(g) = g / (1 + exp(-g)) evaluated in double;
 * y[rows, 2I] holds the gate in columns [0, I) and up in [I, 2I).
 * Also returns max|h|. */
void or_silu_mul(const float* y, int64_t rows, int64_t I, uint16_t* h,
                 float* amax_out) {
  int64_t i, j;
  float amax = 0.0f;
  for (i = 0; i < rows; i++)
    for (j = 0; j < I; j++) {
      double g = y[i * 2 * I + j], u = y[i * 2 * I + I + j];
      double s = g / (1.0 + exp(-g));
      uint16_t b = or_bf16_rne(s * u);
      uint32_t bits = (uint32_t)b << 16;
      float f;
      memcpy(&f, &bits, 4);
      h[i * I + j] = b;
      if (fabsf(f) > amax) amax = fabsf(f);
    }
  *amax_out = amax;
}

/* ------------------------------------------------------------- routing */

typedef struct { float logit; int32_t e; } rkey_t;

static int rkey_cmp(const void* a, const void* b) {
  const rkey_t* x = (const rkey_t*)a;
  const rkey_t* y = (const rkey_t*)b;
  if (x->logit != y->logit) return (x->logit > y->logit) ? -1 : 1;
  return (x->e < y->e) ? -1 : (x->e > y->e);
}

/* MoE top-k routing: per token the k experts with the largest logit (ties
 * toward the lower expert index), in (logit desc, index asc) order; softmax
 * weights of the chosen experts (not renormalized); per-expert offsets
 * (exclusive prefix sum of counts, E+1 entries); gather[j] = source token of
 * grouped row j, expert-major with tokens ascending; row_of[t*k+s] = grouped
 * row of token t's s-th expert. */
void or_route(const float* logits, int64_t T, int64_t E, int64_t k,
              int32_t* topk_ids, float* topk_w, int32_t* offsets,
              int32_t* gather, int32_t* row_of) {
  rkey_t* keys = (rkey_t*)malloc(sizeof(rkey_t) * (size_t)E);
  int64_t t, e, s, pos;
  int64_t* counts = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  for (t = 0; t < T; t++) {
    double mx = -INFINITY, den = 0.0;
    for (e = 0; e < E; e++) {
      keys[e].logit = logits[t * E + e];
      keys[e].e = (int32_t)e;
      if (logits[t * E + e] > mx) mx = logits[t * E + e];
    }
    for (e = 0; e < E; e++) den += exp((double)logits[t * E + e] - mx);
    qsort(keys, (size_t)E, sizeof(rkey_t), rkey_cmp);
    for (s = 0; s < k; s++) {
      topk_ids[t * k + s] = keys[s].e;
      if (topk_w) topk_w[t * k + s] = (float)(exp((double)keys[s].logit - mx) / den);
      counts[keys[s].e]++;
    }
  }
  offsets[0] = 0;
  for (e = 0; e < E; e++) offsets[e + 1] = offsets[e] + (int32_t)counts[e];
  pos = 0;
  for (e = 0; e < E; e++)
    for (t = 0; t < T; t++)
      for (s = 0; s < k; s++)
        if (topk_ids[t * k + s] == e) {
          gather[pos] = (int32_t)t;
          row_of[t * k + s] = (int32_t)pos;
          pos++;
        }
  free(counts);
  free(keys);
}

/* ------------------------------------------------ FP8 W8A8 comparator */

/* The pages measure QUADS against FP8 rollout (arXiv abstract; blog post,
 * section "What it buys": about 16% higher rollout throughput than FP8) but
 * do not say how the FP8 engine scales its tensors.  Reading: W8A8 with OCP
 * E4M3 elements, one FP32 scale per activation row (token) and one per
 * weight output channel, the usual dynamic per-token / static per-channel
 * form, with the same rounding conventions as the NVFP4 quantizer above:
 *   s = RN32(amax_row / 448)     (double quotient, rounded once)
 *   r = RN32(1 / s)              (0 when s == 0)
 *   code = sign(v) | E4M3(|v|),  v = RN32(x * r), nearest-even, saturating;
 * the sign bit is that of v, so a negative value that rounds to zero keeps
 * it (0x80).  A row of zeros gets s = 0 and zero codes. */
float or_fp8_row_scale(float amax) {
  return (float)((double)amax / 448.0);
}

int or_fp8_encode(float v) {
  int c = or_e4m3_encode(fabsf(v));
  return signbit(v) ? (0x80 | c) : c;
}

void or_fp8_quantize_rows(const float* x, int64_t rows, int64_t K, int64_t ldx,
                          uint8_t* codes, float* scales) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < rows; i++) {
    const float* xr = x + i * ldx;
    float amax = 0.0f, s, r;
    int64_t k;
    for (k = 0; k < K; k++)
      if (fabsf(xr[k]) > amax) amax = fabsf(xr[k]);
    s = or_fp8_row_scale(amax);
    r = (s > 0.0f) ? (float)(1.0 / (double)s) : 0.0f;
    for (k = 0; k < K; k++) {
      float v = xr[k] * r;
      codes[i * K + k] = (uint8_t)or_fp8_encode(v);
    }
    scales[i] = s;
  }
}

/* Exact integer image of an E4M3 byte: value * 2^9 (every E4M3 value is a
 * multiple of 2^-9 and at most 448, so the image fits 18 bits). */
static int32_t fp8_int(uint8_t b) {
  return (int32_t)(or_e4m3_value(b) * 512.0);
}

/* FP8 grouped GEMM, the same grouping and gather as or_grouped_gemm:
 *   Y[j, n] = RN32( s_a[src] * s_w[g*N + n] * sum_k A[src,k] W_g[n,k] )
 * with the sum exact in int64 (images scaled by 2^-18) and the product formed
 * in long double. */
static float fp8_one(int64_t G, int64_t N, int64_t K, const int32_t* offsets,
                     const int32_t* gather, const uint8_t* a_codes, const float* a_scales,
                     const uint8_t* w_codes, const float* w_scales, int64_t j, int64_t n) {
  int64_t g = group_of(offsets, G, j);
  int64_t src = gather ? gather[j] : j;
  const uint8_t* a = a_codes + src * K;
  const uint8_t* w = w_codes + (g * N + n) * K;
  int64_t acc = 0, k;
  long double y;
  for (k = 0; k < K; k++) acc += (int64_t)fp8_int(a[k]) * fp8_int(w[k]);
  y = (long double)a_scales[src] * (long double)w_scales[g * N + n] *
      ldexpl((long double)acc, -18);
  return (float)y;
}

void or_fp8_grouped_gemm(int64_t G, int64_t N, int64_t K, int64_t total_rows,
                         const int32_t* offsets, const int32_t* gather,
                         const uint8_t* a_codes, const float* a_scales,
                         const uint8_t* w_codes, const float* w_scales, float* out) {
  int64_t idx;
#pragma omp parallel for schedule(dynamic, 64)
  for (idx = 0; idx < total_rows * N; idx++)
    out[idx] = fp8_one(G, N, K, offsets, gather, a_codes, a_scales, w_codes, w_scales,
                       idx / N, idx % N);
}

void or_fp8_grouped_gemm_sample(int64_t G, int64_t N, int64_t K, const int32_t* offsets,
                                const int32_t* gather, const uint8_t* a_codes,
                                const float* a_scales, const uint8_t* w_codes,
                                const float* w_scales, int64_t n_samples,
                                const int64_t* rows, const int64_t* cols, float* out) {
  int64_t i;
#pragma omp parallel for schedule(dynamic, 16)
  for (i = 0; i < n_samples; i++)
    out[i] = fp8_one(G, N, K, offsets, gather, a_codes, a_scales, w_codes, w_scales,
                     rows[i], cols[i]);
}

/* ------------------------------------- trainer-side weight fake-quant */

/* Asymmetric QAT fake-quantizes the trainer's weights with the rollout's own
 * NVFP4 quantize-dequantize path and leaves activations unquantized (blog
 * post, section "Two fixes, on two different sides"; arXiv abstract: a shared
 * quantization-dequantization path aligns the weights).  Reading: the
 * trainer's weight is the rollout's dequantized value, formed in FP32 as
 * RN32(RN32(g * s_b) * s_t) (g * s_b is exact, so this is the exact product
 * rounded once), and, for a bf16 trainer, that value rounded to bf16
 * (nearest even).  out_f32 and out_bf16 are each optional. */
int or_qdq(const float* x, int64_t rows, int64_t K, const float* amax, float* out_f32,
           uint16_t* out_bf16, float* s_t_out) {
  uint8_t* codes = (uint8_t*)malloc((size_t)(rows * K / 2 > 0 ? rows * K / 2 : 1));
  uint8_t* scales = (uint8_t*)malloc((size_t)(rows * K / 16 > 0 ? rows * K / 16 : 1));
  float* deq = (float*)malloc(sizeof(float) * (size_t)(rows * K > 0 ? rows * K : 1));
  float s_t = 0.0f;
  int64_t i;
  int rc = or_quantize(x, rows, K, K, amax, codes, scales, &s_t);
  if (rc == 0) {
    or_dequantize(codes, scales, s_t, rows, K, deq);
    for (i = 0; i < rows * K; i++) {
      if (out_f32) out_f32[i] = deq[i];
      if (out_bf16) out_bf16[i] = or_bf16_rne((double)deq[i]);
    }
    if (s_t_out) *s_t_out = s_t;
  }
  free(codes);
  free(scales);
  free(deq);
  return rc;
}

/* ----------------------------------------------------------- MoE combine */

/* Weighted combine of the expert outputs back to token order, the last step
 * of the MoE layer whose expert GEMMs the pages quantize (arXiv abstract: MoE
 * rollout).  Reading: for token t,
 *   acc = 0; for s = 0 .. k-1: acc = RN32(acc + RN32(w[t,s] * y[row_of[t,s], :]))
 * in slot order (the routing's (logit desc, index asc) order), then FP32
 * out_f32 = acc and/or bf16 out_bf16 = bf16(acc) (nearest even). */
void or_moe_combine(const float* y, const int32_t* row_of, const float* w, int64_t T,
                    int64_t k, int64_t H, float* out_f32, uint16_t* out_bf16) {
  int64_t t;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; t++) {
    int64_t h, s;
    for (h = 0; h < H; h++) {
      float acc = 0.0f;
      for (s = 0; s < k; s++) {
        float p = w[t * k + s] * y[(int64_t)row_of[t * k + s] * H + h];
        acc = acc + p;
      }
      if (out_f32) out_f32[t * H + h] = acc;
      if (out_bf16) out_bf16[t * H + h] = or_bf16_rne((double)acc);
    }
  }
}


/* ------------------------------------------------------ per-expert RAC */

/* The pages do not say over which rows RAC's channel selection and the
 * activation tensor scale are taken (blog post, section "Two fixes, on two
 * different sides").  The per-tensor reading takes one GEMM input tensor;
 * this is the per-expert one: the grouped rows of each group g, j in
 * [offsets[g], offsets[g+1]), with input row gather[j] (or j), form their own
 * tensor -- own amax and tensor scale, own channel statistics, own selection
 * of n_sel channels, own residual tensor scale -- and each step is exactly
 * the per-tensor oracle above applied to that tensor.  Outputs are in
 * grouped row order (codes [rows, K/2], scales [rows, K/16], residual codes
 * and scales likewise); per-group arrays: s_t[G], score[G, K], chmax[G, K],
 * selected[G, n_sel], active[G, K/16], s_tr[G] (the residual's tensor scale,
 * which is the group's s_t).  score == NULL quantizes only (no RAC). */
void or_quantize_rac_grouped(const float* x, int64_t K, const int32_t* offsets, int64_t G,
                             const int32_t* gather, int64_t n_sel, uint8_t* codes,
                             uint8_t* scales, float* s_t, int64_t* score, float* chmax,
                             int32_t* selected, uint8_t* active, uint8_t* res_codes,
                             uint8_t* res_scales, float* s_tr) {
  int64_t g, i;
  uint8_t* mask = (uint8_t*)malloc((size_t)(K > 0 ? K : 1));
  for (g = 0; g < G; g++) {
    const int64_t j0 = offsets[g], rows = offsets[g + 1] - offsets[g];
    float* sub = (float*)malloc(sizeof(float) * (size_t)(rows * K > 0 ? rows * K : 1));
    float amax_r;
    for (i = 0; i < rows; i++) {
      const int64_t src = gather ? gather[j0 + i] : j0 + i;
      memcpy(sub + i * K, x + src * K, sizeof(float) * (size_t)K);
    }
    or_quantize(sub, rows, K, K, NULL, codes + j0 * (K / 2), scales + j0 * (K / 16), &s_t[g]);
    if (score) {
      or_channel_stats(sub, rows, K, K, codes + j0 * (K / 2), scales + j0 * (K / 16), s_t[g],
                       score + g * K, chmax + g * K);
      or_rac_select(score + g * K, chmax + g * K, K, n_sel, selected + g * n_sel, mask,
                    active + g * (K / 16), &amax_r);
      or_rac_residual(sub, rows, K, K, codes + j0 * (K / 2), scales + j0 * (K / 16), s_t[g],
                      mask, res_codes + j0 * (K / 2), res_scales + j0 * (K / 16), &s_tr[g],
                      NULL);
    }
    free(sub);
  }
  free(mask);
}
