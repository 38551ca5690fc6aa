/* NVFP4 block-scaled linear layer: CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. This library exists to check the GPU library. Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark load it; the
 * product path (libnvfp4 and its Python binding) never links, loads or calls it, and
 * the two share no code, header, table or helper.
 *
 * Plain and slow on purpose: every function restates a definition in the most direct
 * form, in float64 wherever the format does not fix the precision. Sources:
 *
 *  - Weight format. The FP4-Local / ModelOpt NVFP4 checkpoints described in bloomery
 *    issue #565 ("NVIDIA FP4-Local checkpoints on DGX Spark (TP=1, TP=2): format, model
 *    and speed plan in rounds", section 4 "Round 1", PRs #489 and #490) store U8 bytes
 *    holding two 4-bit codes, an F8_E4M3 scale per 16 elements ("group-16", Rocket log
 *    entry "Rank-local E256 MoE misses the Qwen K1 and K4 step budgets", setup table)
 *    and one fp32 tensor scale per matrix. The pages do not spell out the element
 *    encodings; we take the public definitions: E2M1 as in the OCP Microscaling (MX)
 *    v1.0 specification (1 sign, 2 exponent, 1 mantissa bit, bias 1, no Inf/NaN) and
 *    E4M3 as the OCP 8-bit floating point "E4M3FN" encoding (bias 7, max 448, NaN =
 *    S.1111.111, no Inf).
 *  - Quantization rule, nibble order and operand layout: the problem statement of this
 *    library (per-tensor or per-row ts = amax / (6 * 448); per 16-block scale
 *    s = E4M3_RNE(amax_block / 6 / ts); codes E2M1_RNE(w / (s * ts)); two codes per
 *    byte, low nibble first; W is [N][K], y = x W^T). Each expression is evaluated left
 *    to right, one correctly rounded fp32 operation at a time.
 *  - Linear: the pages' model reference computes in f32 with every weight dequantized
 *    by its own rule (issue #565, section 9 "Rules and related work", accuracy item);
 *    here the dequantized product is summed in float64, and the tensor scale is part
 *    of the dequantized value.
 *
 * Readings where the pages are silent: ties round to the even code (RNE); E2M1 values
 * above 6 saturate to 6 and E4M3 values above 448 to 448; a negative value that rounds
 * to zero keeps its sign (code 0x8); an all-zero tensor (ts = 0) gives scale 0 and
 * codes +-0; a zero denominator s*ts gives q = +-0; non-finite inputs are refused.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- E2M1 ------------------------------------------------------------------------ */

/* magnitude of E2M1 code bits 0..2 (exponent e = bits 1..2, mantissa m = bit 0):
 * e = 0: m * 0.5;  e > 0: 2^(e-1) * (1 + m/2) */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_value(int code) {
  double m = E2M1_MAG[code & 7];
  return (code & 8) ? -m : m;
}

/* Round q to the nearest E2M1 value; a tie goes to the even code. The sign comes from
 * signbit(q), so -0 and small negatives give code 0x8. |q| > 6 saturates to 6 (the
 * nearest value); that case is taken first because for huge |q| the float64 distances
 * below stop being exact. Returns -1 for NaN or Inf. */
int oracle_e2m1_encode(float q) {
  if (isnan(q) || isinf(q)) return -1;
  int sign = signbit(q) ? 8 : 0;
  double a = fabs((double)q);
  if (a > 6.0) return sign | 7;
  int best = 0;
  double bestd = fabs(a - E2M1_MAG[0]);
  for (int c = 1; c < 8; c++) {
    double d = fabs(a - E2M1_MAG[c]);
    if (d < bestd || (d == bestd && (c % 2) == 0 && (best % 2) != 0)) {
      best = c;
      bestd = d;
    }
  }
  return sign | best;
}

/* ---- E4M3 (OCP E4M3FN) ------------------------------------------------------------ */

double oracle_e4m3_value(int byte) {
  int s = (byte >> 7) & 1, e = (byte >> 3) & 15, f = byte & 7;
  if (e == 15 && f == 7) return NAN;
  double v = (e == 0) ? (f / 8.0) * ldexp(1.0, -6) : (1.0 + f / 8.0) * ldexp(1.0, e - 7);
  return s ? -v : v;
}

/* Round r >= 0 to the nearest of the 127 finite non-negative E4M3 values (codes 0x00 to
 * 0x7E, increasing with the code); a tie goes to the even code; r >= 448 gives 0x7E.
 * Returns -1 for negative, NaN or Inf input (-0 is treated as 0). */
int oracle_e4m3_encode(float r) {
  if (isnan(r) || isinf(r) || r < 0.0f) return -1;
  double v = (double)r;
  if (v >= 448.0) return 0x7E;
  int lo = 0, hi = 0x7E; /* value(lo) <= v < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (oracle_e4m3_value(mid) <= v) lo = mid; else hi = mid;
  }
  double dlo = v - oracle_e4m3_value(lo), dhi = oracle_e4m3_value(hi) - v;
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo % 2 == 0) ? lo : hi;
}

/* ---- BF16 ------------------------------------------------------------------------- */

double oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest BF16 value (ties to even), one rounding, for finite
 * values within the BF16 range. Used for the BF16 SwiGLU output of the MoE reading. */
uint16_t oracle_bf16_round(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
  int sign = v < 0;
  double a = fabs(v);
  int e;
  frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
  int E = e - 1;         /* a in [2^E, 2^(E+1)) */
  if (E < -126) E = -126; /* subnormal spacing */
  double ulp = ldexp(1.0, E - 7);
  double q = a / ulp;    /* exact: scaling by a power of two */
  double fl = floor(q), rem = q - fl;
  double n = (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) ? fl + 1.0 : fl;
  float r = (float)(n * ulp);
  uint32_t u;
  memcpy(&u, &r, 4);
  return (uint16_t)((u >> 16) | (sign ? 0x8000 : 0));
}

/* ---- Quantizer -------------------------------------------------------------------- */

/* Quantize w [rows][K] (K % 16 == 0). per_row != 0: one ts per row (ts has `rows`
 * entries); per_row == 0: one ts for the whole tensor (ts has 1 entry).
 * codes [rows][K/2] (low nibble = even k), scales [rows][K/16] E4M3 bytes.
 * Returns 0, or -1 if any input is NaN or Inf (outputs then undefined). */
int oracle_quantize(const float* w, int64_t rows, int64_t K, int per_row,
                    uint8_t* codes, uint8_t* scales, float* ts) {
  for (int64_t i = 0; i < rows * K; i++)
    if (isnan(w[i]) || isinf(w[i])) return -1;
  if (!per_row) {
    float amax = 0.0f;
    for (int64_t i = 0; i < rows * K; i++) amax = fmaxf(amax, fabsf(w[i]));
    ts[0] = amax / 2688.0f;
  }
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    const float* wr = w + r * K;
    float t;
    if (per_row) {
      float amax = 0.0f;
      for (int64_t k = 0; k < K; k++) amax = fmaxf(amax, fabsf(wr[k]));
      t = amax / 2688.0f;
      ts[r] = t;
    } else {
      t = ts[0];
    }
    for (int64_t b = 0; b < K / 16; b++) {
      float amax_b = 0.0f;
      for (int j = 0; j < 16; j++) amax_b = fmaxf(amax_b, fabsf(wr[b * 16 + j]));
      float ratio = (t == 0.0f) ? 0.0f : (amax_b / 6.0f) / t;
      int s = oracle_e4m3_encode(ratio);
      scales[r * (K / 16) + b] = (uint8_t)s;
      float sd = (float)oracle_e4m3_value(s);
      float den = sd * t;
      int c[16];
      for (int j = 0; j < 16; j++) {
        float x = wr[b * 16 + j];
        float q = (den == 0.0f) ? copysignf(0.0f, x) : x / den;
        c[j] = oracle_e2m1_encode(q);
      }
      for (int j = 0; j < 8; j++)
        codes[r * (K / 2) + b * 8 + j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
    }
  }
  return 0;
}

/* ---- Dequantization and the linear layer -------------------------------------------- */

/* out[r][k] = e2m1(code) * e4m3(scale of block k/16) * ts, in float64 (exact: at most
 * 2 + 4 + 24 significant bits). per_row selects ts[r] or ts[0]. */
void oracle_dequant(const uint8_t* codes, const uint8_t* scales, const float* ts,
                    int per_row, int64_t rows, int64_t K, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    double t = (double)(per_row ? ts[r] : ts[0]);
    for (int64_t k = 0; k < K; k++) {
      uint8_t byte = codes[r * (K / 2) + k / 2];
      int code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
      double s = oracle_e4m3_value(scales[r * (K / 16) + k / 16]);
      out[r * K + k] = oracle_e2m1_value(code) * s * t;
    }
  }
}

/* y[m][n] = sum_k x[m][k] * w[n][k], summed in float64 in increasing k;
 * bound[m][n] = sum_k |x[m][k] * w[n][k]| (the scale of the accepted error). */
void oracle_linear(const double* x, int64_t M, const double* w, int64_t N, int64_t K,
                   double* y, double* bound) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < M; m++) {
    for (int64_t n = 0; n < N; n++) {
      double s = 0.0, b = 0.0;
      for (int64_t k = 0; k < K; k++) {
        double p = x[m * K + k] * w[n * K + k];
        s += p;
        b += fabs(p);
      }
      y[m * N + n] = s;
      if (bound) bound[m * N + n] = b;
    }
  }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Batch forms of the two encoders (used by the exhaustive checks of the tests) and of
 * the BF16 rounding (whole SwiGLU outputs of a prompt-sized MoE layer). */
void oracle_bf16_round_batch(const double* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_round(v[i]);
}

void oracle_e2m1_encode_batch(const float* q, int64_t n, int8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = (int8_t)oracle_e2m1_encode(q[i]);
}

void oracle_e4m3_encode_batch(const float* r, int64_t n, int16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = (int16_t)oracle_e4m3_encode(r[i]);
}
