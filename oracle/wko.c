/*
 * wko.c -- plain, slow, fp64 CPU reference ("the oracle") for the WUSH-KV
 * transformed low-bit KV cache: key transform, per-token percentile-clipped
 * affine quantizer, full-precision cache windows and decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the GPU library, and the GPU library never
 * loads it.
 *
 * Everything is scalar double-precision arithmetic, written for a reader to
 * check against the method's description by eye.  No blocking, fusion or
 * reordering is done beyond what each definition states.  Build with
 * -ffp-contract=off so that no multiply-add is fused.
 *
 * Sources (web pages on "WUSH-KV: KV Cache Quantization with Data-Adaptive
 * Transforms"):
 *   [P3 s4.1]  paper, section 4.1 "KV Cache in Grouped-Query Attention":
 *              per KV head the cache holds one column per position; keys are
 *              stored after head-norm and RoPE; query heads Q_{h,g} share KV
 *              head h.
 *   [P3 s4.2]  section 4.2 "WUSH-KV Transforms": a full d x d key transform
 *              applied after RoPE to every new key, with a query-side
 *              compensation.
 *   [P3 B.1]   appendix B.1: the transform acts as T X on column tokens and the
 *              compensation is T^{-T}; each column is one quantization group.
 *   [P3 s5.3]  section 5.3 "Downstream Benchmarks": the quantizer used end to
 *              end is percentile clipping plus asymmetric affine scaling with
 *              an adaptive zero point.
 *   [P3 B.3]   appendix B.3: 2^b equally spaced levels between the clip ends,
 *              spacing = range / (2^b - 1).
 *   [P3 s4.4]  section 4.4 "Full-Precision Cache Window": a fixed sink of the
 *              first S_sink positions, a rolling recent window of the newest
 *              S_keep positions, quantization in multiples of S_flush, and a
 *              quantized-region boundary S_quant that starts at zero.
 *   [P3 D.1]   appendix D.1: softmax with the model's native scaling.
 *
 * Readings taken where the pages are silent (each is also listed in the
 * design notes): percentile = linear interpolation at h = p (n - 1); scale
 * and zero are rounded to IEEE binary16 (round-to-nearest-even, saturating at
 * +-65504) and the codes are computed from the rounded values; codes are
 * round-half-to-even of (x - z16) / s16 clamped to [0, 2^b - 1]; a group whose
 * rounded scale is zero gets all-zero codes; full-precision window entries
 * are bfloat16 (round-to-nearest-even); softmax scale is 1/sqrt(d).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Rounding to a binary floating-point format with p significand bits.       */
/* ------------------------------------------------------------------------ */

/* Round x to the nearest value with p significand bits whose exponent is at
 * least emin (gradual underflow below 2^emin), ties to even.  |results| above
 * maxval become +-inf, or +-maxval when saturate is set. */
static double round_to_format(double x, int p, int emin, double maxval,
                              int saturate) {
  if (x == 0.0 || !isfinite(x)) return x;
  int E;
  (void)frexp(x, &E);          /* |x| = f 2^E, f in [0.5, 1): floor(log2|x|) = E-1 */
  int e = E - 1;
  if (e < emin) e = emin;       /* subnormal range: fixed quantum 2^(emin-p+1) */
  double quantum = ldexp(1.0, e - (p - 1));
  double r = rint(x / quantum) * quantum;   /* rint: nearest, ties to even */
  if (fabs(r) > maxval) {
    if (saturate) return x > 0 ? maxval : -maxval;
    return x > 0 ? INFINITY : -INFINITY;
  }
  return r;
}

/* bfloat16: 8 significand bits, min normal 2^-126, max 0x1.FEp127. */
double wko_bf16(double x) {
  return round_to_format(x, 8, -126, ldexp(255.0, 120), 0);
}

/* IEEE binary16: 11 significand bits, min normal 2^-14, max 65504.
 * Saturating (reading: scale/zero never become infinite). */
double wko_fp16(double x) {
  return round_to_format(x, 11, -14, 65504.0, 1);
}

void wko_bf16_array(const double* x, double* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = wko_bf16(x[i]);
}

void wko_fp16_array(const double* x, double* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = wko_fp16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Key transform k' = T k  [P3 s4.2, B.1]                                    */
/* ------------------------------------------------------------------------ */

/* T: d x d row-major, k'_i = sum_j T[i][j] k_j.  keys: n x d.  out: n x d.
 * absout (nullable): sum_j |T[i][j] k_j|, used by callers to bound the
 * rounding error of any other summation order of the same products. */
void wko_transform(const double* T, const double* keys, int64_t n, int d,
                   double* out, double* absout) {
  for (int64_t t = 0; t < n; ++t) {
    const double* k = keys + t * d;
    for (int i = 0; i < d; ++i) {
      double acc = 0.0, aacc = 0.0;
      for (int j = 0; j < d; ++j) {
        double prod = T[(int64_t)i * d + j] * k[j];
        acc += prod;
        aacc += fabs(prod);
      }
      out[t * d + i] = acc;
      if (absout) absout[t * d + i] = aacc;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Percentile by sorting  [P3 s5.3; reading: linear interpolation]           */
/* ------------------------------------------------------------------------ */

static int cmp_double(const void* a, const void* b) {
  double x = *(const double*)a, y = *(const double*)b;
  return (x > y) - (x < y);
}

/* Percentile p in [0, 1] of n values: sort ascending, h = p (n - 1),
 * j = floor(h), f = h - j; result x(j) + f (x(j+1) - x(j)), or x(n-1) when
 * j = n - 1.  scratch must hold n doubles. */
double wko_percentile(const double* x, int n, double p, double* scratch) {
  memcpy(scratch, x, sizeof(double) * (size_t)n);
  qsort(scratch, (size_t)n, sizeof(double), cmp_double);
  double h = p * (double)(n - 1);
  double jf = floor(h);
  int j = (int)jf;
  double f = h - jf;
  if (j >= n - 1) return scratch[n - 1];
  return scratch[j] + f * (scratch[j + 1] - scratch[j]);
}

/* ------------------------------------------------------------------------ */
/* Per-token percentile-clipped asymmetric affine quantizer                  */
/* [P3 s5.3 quantizer; B.1 one group per column; B.3 level spacing]          */
/* ------------------------------------------------------------------------ */

/* One group of n values with clip ends lo <= hi: s = (hi - lo)/(2^b - 1),
 * z = lo, both rounded to binary16; codes = rint((x - z16)/s16) clamped to
 * [0, 2^b - 1] (all 0 when s16 == 0); u = the unrounded code coordinate. */
static void quantize_group_ends(const double* xg, int n, int bits, double lo, double hi,
                                uint8_t* codes, double* s16, double* z16, double* u) {
  const double levels = (double)((1 << bits) - 1);
  double s = (hi - lo) / levels;   /* spacing of 2^b levels over [lo, hi] */
  double z = lo;                   /* zero point = lower clip end */
  double sr = wko_fp16(s), zr = wko_fp16(z);
  *s16 = sr;
  *z16 = zr;
  for (int i = 0; i < n; ++i) {
    double ui = 0.0, c = 0.0;
    if (sr != 0.0) {
      ui = (xg[i] - zr) / sr;
      c = rint(ui);                /* round half to even */
      if (c < 0.0) c = 0.0;
      if (c > levels) c = levels;
    }
    codes[i] = (uint8_t)c;
    if (u) u[i] = ui;
  }
}

/* Quantize n_groups groups of n values each (groups contiguous), clip ends
 * at the p_lo and p_hi percentiles of the group (asymmetric, adaptive zero
 * point).  Outputs per group: s16, z16 (the stored binary16 scale and zero
 * point), per element: code (0 .. 2^bits - 1) and u = (x - z16) / s16 (the
 * unrounded code coordinate, 0 when s16 == 0; lets callers see rounding
 * boundaries).  Returns 0, or -1 on bad arguments. */
int wko_quantize(const double* x, int64_t n_groups, int n, int bits,
                 double p_lo, double p_hi, uint8_t* codes, double* s16,
                 double* z16, double* u) {
  if (n < 1 || bits < 1 || bits > 8 || !(p_lo <= p_hi)) return -1;
  double* scratch = (double*)malloc(sizeof(double) * (size_t)n);
  if (!scratch) return -1;
  for (int64_t g = 0; g < n_groups; ++g) {
    const double* xg = x + g * n;
    double lo = wko_percentile(xg, n, p_lo, scratch);
    double hi = wko_percentile(xg, n, p_hi, scratch);
    quantize_group_ends(xg, n, bits, lo, hi, codes + g * n, s16 + g, z16 + g,
                        u ? u + g * n : 0);
  }
  free(scratch);
  return 0;
}

/* The QuEST-style symmetric quantizer [P3 B.3: 2^b equally spaced levels from
 * -alpha to alpha on the RMS-normalized group]: clip ends -alpha * rms and
 * +alpha * rms with rms = sqrt(sum_i x_i^2 / n), then the same binary16
 * scale / zero and codes as above.  Returns 0, or -1 on bad arguments. */
int wko_quantize_rms(const double* x, int64_t n_groups, int n, int bits, double alpha,
                     uint8_t* codes, double* s16, double* z16, double* u) {
  if (n < 1 || bits < 1 || bits > 8 || !(alpha >= 0.0)) return -1;
  for (int64_t g = 0; g < n_groups; ++g) {
    const double* xg = x + g * n;
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += xg[i] * xg[i];
    const double rms = sqrt(ss / (double)n);
    quantize_group_ends(xg, n, bits, -alpha * rms, alpha * rms, codes + g * n, s16 + g,
                        z16 + g, u ? u + g * n : 0);
  }
  return 0;
}

/* Dequantize: xhat = z16 + s16 * code. */
void wko_dequantize(const uint8_t* codes, const double* s16, const double* z16,
                    int64_t n_groups, int n, double* out) {
  for (int64_t g = 0; g < n_groups; ++g)
    for (int i = 0; i < n; ++i)
      out[g * n + i] = z16[g] + s16[g] * (double)codes[g * n + i];
}

/* ------------------------------------------------------------------------ */
/* Cache regions  [P3 s4.4]                                                  */
/* ------------------------------------------------------------------------ */

/* Quantized region [S, S_quant) after the cache reaches length L: the entries
 * outside the sink (first S) and outside the newest R, rounded down to a
 * multiple of F.  Returns S_quant. */
int64_t wko_squant(int64_t L, int64_t S, int64_t R, int64_t F) {
  int64_t outside = L - R - S;
  if (outside < 0) outside = 0;
  return S + F * (outside / F);
}

/* ------------------------------------------------------------------------ */
/* Decode attention  [P3 s4.1 GQA sharing; D.1 native 1/sqrt(d) scaling]     */
/* ------------------------------------------------------------------------ */

/* One decode query per query head over L cached positions.
 * qc:   n_q x d, compensated queries (already multiplied by T^{-T}).
 * K, V: n_kv x L x d, the cache as read back (window values or dequantized).
 * out:  n_q x d.  Query head j reads KV head j / (n_q / n_kv).
 * The single decode query is the newest position, so it sees all L entries
 * and no causal mask applies.  Softmax: subtract max, exp, divide by sum. */
int wko_attention(const double* qc, const double* K, const double* V, int n_q,
                  int n_kv, int64_t L, int d, double* out) {
  if (n_kv < 1 || n_q % n_kv != 0 || L < 1) return -1;
  int G = n_q / n_kv;
  double* e = (double*)malloc(sizeof(double) * (size_t)L);
  if (!e) return -1;
  double scale = 1.0 / sqrt((double)d);
  for (int j = 0; j < n_q; ++j) {
    int h = j / G;
    const double* q = qc + (int64_t)j * d;
    const double* Kh = K + (int64_t)h * L * d;
    const double* Vh = V + (int64_t)h * L * d;
    double m = -INFINITY;
    for (int64_t p = 0; p < L; ++p) {
      double dot = 0.0;
      for (int i = 0; i < d; ++i) dot += q[i] * Kh[p * d + i];
      e[p] = dot * scale;
      if (e[p] > m) m = e[p];
    }
    double l = 0.0;
    for (int64_t p = 0; p < L; ++p) {
      e[p] = exp(e[p] - m);
      l += e[p];
    }
    double* o = out + (int64_t)j * d;
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    for (int64_t p = 0; p < L; ++p) {
      double w = e[p] / l;
      for (int i = 0; i < d; ++i) o[i] += w * Vh[p * d + i];
    }
  }
  free(e);
  return 0;
}
