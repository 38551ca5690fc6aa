/* Seeded random streams for the synthetic workloads (no NVFP4 arithmetic here).
 *
 * SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) in counter form: output i of the
 * stream with key k is mix(k + (i + 1) * 0x9E3779B97F4A7C15). Uniform doubles take
 * the top 53 bits. Normal variates come from the Box-Muller transform on consecutive
 * uniform pairs (u1, u2): r = sqrt(-2 ln(1 - u1)), theta = 2 pi u2, giving r cos theta
 * and r sin theta, all in double precision.
 */
#include <math.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

void synth_u64(uint64_t key, uint64_t start, int64_t n, uint64_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = mix64(key + (start + (uint64_t)i + 1) * GOLDEN);
}

static inline double unif(uint64_t key, uint64_t i) {
  return (double)(mix64(key + (i + 1) * GOLDEN) >> 11) * (1.0 / 9007199254740992.0);
}

void synth_uniform(uint64_t key, uint64_t start, int64_t n, double* out) {
  for (int64_t i = 0; i < n; i++) out[i] = unif(key, start + (uint64_t)i);
}

/* out[i] = (float)(scale * z_i), z_i standard normal; z_{2p}, z_{2p+1} use uniforms 2p, 2p+1 */
void synth_normal_f32(uint64_t key, int64_t n, double scale, float* out) {
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t p = 0; 2 * p < n; p++) {
    double u1 = unif(key, (uint64_t)(2 * p)), u2 = unif(key, (uint64_t)(2 * p + 1));
    double r = sqrt(-2.0 * log(1.0 - u1)), th = two_pi * u2;
    out[2 * p] = (float)(scale * (r * cos(th)));
    if (2 * p + 1 < n) out[2 * p + 1] = (float)(scale * (r * sin(th)));
  }
}

void synth_normal_f64(uint64_t key, int64_t n, double* out) {
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t p = 0; 2 * p < n; p++) {
    double u1 = unif(key, (uint64_t)(2 * p)), u2 = unif(key, (uint64_t)(2 * p + 1));
    double r = sqrt(-2.0 * log(1.0 - u1)), th = two_pi * u2;
    out[2 * p] = r * cos(th);
    if (2 * p + 1 < n) out[2 * p + 1] = r * sin(th);
  }
}
