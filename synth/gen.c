/* Counter-based Gaussian draws for the synthetic inputs (same recipe as rng.py).
 *
 * Element i of the stream with seed s is built from the splitmix64 outputs
 * mix(s + (2j+1)*G) and mix(s + (2j+2)*G), j = i/2, G = 0x9E3779B97F4A7C15
 * (Vigna's splitmix64), turned into uniforms in (0,1] from their top 53 bits,
 * and combined by Box-Muller: even i takes r*cos(2 pi u2), odd i r*sin(2 pi u2)
 * with r = sqrt(-2 ln u1).  Each element depends only on (s, i), so any thread
 * split gives the same bits. */
#include <math.h>
#include <stdint.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline double u01(uint64_t seed, uint64_t ctr) {
  uint64_t z = mix64(seed + ctr * 0x9E3779B97F4A7C15ULL);
  return ((double)(z >> 11) + 1.0) * (1.0 / 9007199254740992.0);
}

/* out[i] = (float)(std * N_i) for i in [0, n) */
void synth_normal_f64(uint64_t seed, int64_t n, double std_, double *out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (n + 1) / 2; ++j) {
    double u1 = u01(seed, (uint64_t)(2 * j + 1));
    double u2 = u01(seed, (uint64_t)(2 * j + 2));
    double r = sqrt(-2.0 * log(u1));
    double t = 2.0 * M_PI * u2;
    out[2 * j] = std_ * (r * cos(t));
    if (2 * j + 1 < n) out[2 * j + 1] = std_ * (r * sin(t));
  }
}

/* fp32 -> bf16 bit patterns, round to nearest even; NaN -> 0x7FC0 */
void synth_f32_to_bf16(const float *in, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    union { float f; uint32_t u; } c;
    c.f = in[i];
    if (c.f != c.f) { out[i] = 0x7FC0; continue; }
    out[i] = (uint16_t)((c.u + 0x7FFFu + ((c.u >> 16) & 1u)) >> 16);
  }
}
