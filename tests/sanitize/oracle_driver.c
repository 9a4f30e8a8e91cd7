/* Driver of the fp64 oracle (oracle/wko.c) for AddressSanitizer and
 * UndefinedBehaviorSanitizer builds: every exported function on inputs that
 * include the edge cases (ties, constant groups, binary16 saturation,
 * subnormals, infinities).  Prints "oracle driver OK" and exits 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double wko_bf16(double x);
double wko_fp16(double x);
void wko_bf16_array(const double* x, double* y, int64_t n);
void wko_fp16_array(const double* x, double* y, int64_t n);
void wko_transform(const double* T, const double* keys, int64_t n, int d, double* out,
                   double* absout);
double wko_percentile(const double* x, int n, double p, double* scratch);
int wko_quantize(const double* x, int64_t n_groups, int n, int bits, double p_lo, double p_hi,
                 uint8_t* codes, double* s16, double* z16, double* u);
int wko_quantize_rms(const double* x, int64_t n_groups, int n, int bits, double alpha,
                     uint8_t* codes, double* s16, double* z16, double* u);
void wko_dequantize(const uint8_t* codes, const double* s16, const double* z16, int64_t n_groups,
                    int n, double* out);
int64_t wko_squant(int64_t L, int64_t S, int64_t R, int64_t F);
int wko_attention(const double* qc, const double* K, const double* V, int n_q, int n_kv, int64_t L,
                  int d, double* out);

static int fail = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); fail = 1; } } while (0)

int main(void) {
  enum { D = 128, NG = 6 };
  const double specials[] = {0.0, -0.0, 1.0, 65504.0, 65520.0, 1e5, -1e5, 5.96e-8, 2.98e-8,
                             1e-40, INFINITY, -INFINITY, 3.0e38, 3.4e38};
  for (unsigned i = 0; i < sizeof specials / sizeof *specials; ++i) {
    (void)wko_bf16(specials[i]);
    (void)wko_fp16(specials[i]);
  }
  CHECK(wko_fp16(1e5) == 65504.0 && wko_fp16(-1e5) == -65504.0);
  double* T = malloc(sizeof(double) * D * D);
  double* x = malloc(sizeof(double) * NG * D);
  double* y = malloc(sizeof(double) * NG * D);
  double* a = malloc(sizeof(double) * NG * D);
  double* u = malloc(sizeof(double) * NG * D);
  uint8_t* codes = malloc(NG * D);
  double s16[NG], z16[NG], scratch[D];
  srand(1);
  for (int i = 0; i < D * D; ++i) T[i] = (double)rand() / RAND_MAX - 0.5;
  for (int g = 0; g < NG; ++g)
    for (int i = 0; i < D; ++i) {
      double v = (double)(rand() % 16) * 0.5;
      if (g == 1) v = 3.25;                  /* constant group */
      if (g == 2) v = (i & 1) ? 9e4 : -9e4;  /* saturating scale and zero */
      if (g == 3) v = ldexp(1.0, -20) + ((i & 1) ? ldexp(1.0, -27) : 0.0);
      x[g * D + i] = v;
    }
  wko_transform(T, x, NG, D, y, a);
  wko_transform(T, x, NG, D, y, NULL);
  wko_bf16_array(y, y, NG * D);
  wko_fp16_array(x, a, NG * D);
  for (int p = 0; p <= 100; ++p) (void)wko_percentile(x, D, p / 100.0, scratch);
  (void)wko_percentile(x, 1, 0.5, scratch);
  for (int bits = 1; bits <= 8; ++bits) {
    CHECK(wko_quantize(x, NG, D, bits, 0.01, 0.99, codes, s16, z16, u) == 0);
    CHECK(s16[1] == 0.0);
    CHECK(wko_quantize(x, NG, D, bits, 0.0, 1.0, codes, s16, z16, NULL) == 0);
    CHECK(wko_quantize_rms(x, NG, D, bits, 1.5, codes, s16, z16, u) == 0);
    wko_dequantize(codes, s16, z16, NG, D, a);
  }
  CHECK(wko_quantize(x, NG, D, 0, 0.01, 0.99, codes, s16, z16, u) == -1);
  CHECK(wko_quantize(x, NG, D, 2, 0.9, 0.1, codes, s16, z16, u) == -1);
  CHECK(wko_quantize_rms(x, NG, D, 9, 1.5, codes, s16, z16, u) == -1);
  CHECK(wko_squant(0, 4, 128, 1) == 4 && wko_squant(1000, 4, 128, 1) == 872);
  CHECK(wko_squant(1000, 16, 128, 16) == 864);
  double q[4 * D], out[4 * D];
  for (int i = 0; i < 4 * D; ++i) q[i] = (double)rand() / RAND_MAX - 0.5;
  CHECK(wko_attention(q, y, x, 4, 2, 3, D, out) == 0);
  CHECK(wko_attention(q, y, x, 3, 2, 3, D, out) == -1);
  CHECK(wko_attention(q, y, x, 4, 2, 0, D, out) == -1);
  free(T); free(x); free(y); free(a); free(u); free(codes);
  if (fail) return 1;
  printf("oracle driver OK\n");
  return 0;
}
