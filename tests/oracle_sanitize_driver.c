/* Runs every entry point of the oracle (oracle/nvfp4_oracle.c) on small and edge inputs,
 * for a build with AddressSanitizer and UndefinedBehaviorSanitizer: any out-of-bounds
 * access, overflow or undefined conversion ends the run with a report. It also checks a
 * few facts the oracle's callers rely on (every code and scale byte survives an encode of
 * its own value; the quantizer's outputs decode within the tensor's range), so a build
 * that silently computes garbage fails too. Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e2m1_value(int code);
int oracle_e2m1_encode(float q);
double oracle_e4m3_value(int byte);
int oracle_e4m3_encode(float r);
double oracle_bf16_value(uint16_t bits);
uint16_t oracle_bf16_round(double v);
int oracle_quantize(const float* w, int64_t rows, int64_t K, int per_row, uint8_t* codes,
                    uint8_t* scales, float* ts);
void oracle_dequant(const uint8_t* codes, const uint8_t* scales, const float* ts, int per_row,
                    int64_t rows, int64_t K, double* out);
void oracle_linear(const double* x, int64_t M, const double* w, int64_t N, int64_t K, double* y,
                   double* bound);
int oracle_num_threads(void);
void oracle_bf16_round_batch(const double* v, int64_t n, uint16_t* out);
void oracle_e2m1_encode_batch(const float* q, int64_t n, int8_t* out);
void oracle_e4m3_encode_batch(const float* r, int64_t n, int16_t* out);

static int failures = 0;
#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");              \
      failures++;                         \
    }                                     \
  } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, in [0, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}

static void codecs(void) {
  for (int c = 0; c < 16; c++) {
    const double v = oracle_e2m1_value(c);
    const int back = oracle_e2m1_encode((float)v);
    /* -0 encodes as code 8, +0 as code 0 */
    CHECK(back == c, "e2m1 code %d -> %g -> %d", c, v, back);
  }
  for (int b = 0; b < 256; b++) {
    const double v = oracle_e4m3_value(b);
    if (isnan(v) || v < 0.0) continue; /* scales are non-negative; 0x7F / 0xFF are NaN */
    const int back = oracle_e4m3_encode((float)v);
    CHECK(back == b || v == 0.0, "e4m3 byte %d -> %g -> %d", b, v, back);
  }
  const float specials[] = {0.0f, -0.0f, 1e-30f, 0.25f, 0.75f, 5.0f, 6.0f, 7.0f, 1e30f,
                            -1e30f, INFINITY, -INFINITY, NAN};
  for (size_t i = 0; i < sizeof specials / sizeof specials[0]; i++) {
    (void)oracle_e2m1_encode(specials[i]);
    (void)oracle_e4m3_encode(specials[i]);
  }
  const double dspecials[] = {0.0, -0.0, 1e-300, 3.0e38, 3.4e38, 1e300, -1e300,
                              INFINITY, -INFINITY, NAN, 1.0 + 1.0 / 256.0};
  for (size_t i = 0; i < sizeof dspecials / sizeof dspecials[0]; i++)
    (void)oracle_bf16_value(oracle_bf16_round(dspecials[i]));
  for (uint32_t bits = 0; bits < 65536; bits += 7) {
    const double v = oracle_bf16_value((uint16_t)bits);
    if (!isnan(v)) CHECK(oracle_bf16_round(v) == bits, "bf16 %u does not round to itself", bits);
  }
}

static void batches(void) {
  enum { n = 1000 };
  float q[n];
  double v[n];
  int8_t c[n];
  int16_t s[n];
  uint16_t b[n];
  for (int i = 0; i < n; i++) {
    q[i] = (float)((uniform() - 0.5) * 16.0);
    v[i] = (uniform() - 0.5) * 1e6;
  }
  q[0] = NAN;
  q[1] = INFINITY;
  oracle_e2m1_encode_batch(q, n, c);
  oracle_e4m3_encode_batch(q, n, s);
  oracle_bf16_round_batch(v, n, b);
  for (int i = 2; i < n; i++) {
    CHECK(c[i] >= 0 && c[i] < 16, "e2m1 batch code out of range at %d", i);
    CHECK(c[i] == oracle_e2m1_encode(q[i]), "e2m1 batch differs at %d", i);
    CHECK(b[i] == oracle_bf16_round(v[i]), "bf16 batch differs at %d", i);
  }
}

/* quantize -> dequantize -> linear on one shape; w holds rows * K values */
static void round_trip(const float* w, int64_t rows, int64_t K, int per_row) {
  uint8_t* codes = malloc((size_t)(rows * K / 2));
  uint8_t* scales = malloc((size_t)(rows * K / 16));
  float* ts = malloc(sizeof(float) * (size_t)(per_row ? rows : 1));
  double* deq = malloc(sizeof(double) * (size_t)(rows * K));
  double* x = malloc(sizeof(double) * (size_t)(3 * K));
  double* y = malloc(sizeof(double) * (size_t)(3 * rows));
  double* bound = malloc(sizeof(double) * (size_t)(3 * rows));
  const int rc = oracle_quantize(w, rows, K, per_row, codes, scales, ts);
  CHECK(rc == 0, "quantize refused finite input (rows %ld, K %ld)", (long)rows, (long)K);
  oracle_dequant(codes, scales, ts, per_row, rows, K, deq);
  double amax = 0.0;
  for (int64_t i = 0; i < rows * K; i++) amax = fmax(amax, fabs((double)w[i]));
  for (int64_t i = 0; i < rows * K; i++) {
    CHECK(isfinite(deq[i]), "dequantized value not finite at %ld", (long)i);
    /* every value decodes within 6 * 448 * ts of zero, and ts = amax / 2688 */
    CHECK(fabs(deq[i]) <= amax * 1.0000001 + 1e-30, "dequantized %g beyond amax %g",
          deq[i], amax);
  }
  for (int64_t i = 0; i < 3 * K; i++) x[i] = uniform() - 0.5;
  oracle_linear(x, 3, deq, rows, K, y, bound);
  oracle_linear(x, 3, deq, rows, K, y, NULL); /* the bound is optional */
  for (int64_t i = 0; i < 3 * rows; i++) CHECK(isfinite(y[i]), "linear output not finite");
  free(codes);
  free(scales);
  free(ts);
  free(deq);
  free(x);
  free(y);
  free(bound);
}

static void quantizer(void) {
  const int64_t shapes[][2] = {{1, 16}, {3, 32}, {5, 48}, {2, 160}, {17, 64}};
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; s++) {
    const int64_t rows = shapes[s][0], K = shapes[s][1];
    float* w = malloc(sizeof(float) * (size_t)(rows * K));
    for (int per_row = 0; per_row < 2; per_row++) {
      for (int64_t i = 0; i < rows * K; i++) w[i] = (float)((uniform() - 0.5) * 8.0);
      round_trip(w, rows, K, per_row);
      memset(w, 0, sizeof(float) * (size_t)(rows * K)); /* all zero: ts = 0 */
      round_trip(w, rows, K, per_row);
      for (int64_t i = 0; i < rows * K; i++) w[i] = (i % 3 == 0) ? -3.0e38f : 1e-38f;
      round_trip(w, rows, K, per_row); /* the float range's ends */
      for (int64_t i = 0; i < rows * K; i++) w[i] = (i % 16 == 5) ? 2.5f : -0.0f;
      round_trip(w, rows, K, per_row); /* one value per block */
    }
    /* a non-finite input is refused without reading past the tensor */
    w[rows * K - 1] = NAN;
    uint8_t* codes = malloc((size_t)(rows * K / 2));
    uint8_t* scales = malloc((size_t)(rows * K / 16));
    float ts[32];
    CHECK(oracle_quantize(w, rows, K, 1, codes, scales, ts) == -1, "NaN not refused");
    w[rows * K - 1] = -INFINITY;
    CHECK(oracle_quantize(w, rows, K, 0, codes, scales, ts) == -1, "Inf not refused");
    free(codes);
    free(scales);
    free(w);
  }
}

int main(void) {
  CHECK(oracle_num_threads() >= 1, "no threads");
  codecs();
  batches();
  quantizer();
  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("oracle under sanitizers: ok\n");
  return 0;
}
