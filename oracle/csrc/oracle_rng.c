/* Plain-C twin of oracle/rng.py (test infrastructure only).
 *
 * Same definition as the numpy code: splitmix64 (Steele, Lea and Flood, 2014)
 * feeding Box-Muller, counter based, element i of stream s under seed k is
 *   key = sm(k ^ sm(s)),  N(i) = sqrt(-2 ln(1 - u53(sm(key+2i)))) cos(2 pi u53(sm(key+2i+1))),
 * scaled by std and rounded nearest-even into the storage type. Built with
 * plain IEEE arithmetic (no fast-math). Used only to make the oracle's
 * multi-billion-element weight tensors affordable on the host.
 */
#include <math.h>
#include <stdint.h>

static inline uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ULL;
  uint64_t z = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline double u53(uint64_t x) { return (double)(x >> 11) * 0x1.0p-53; }

/* nearest-even rounding to 8 significant bits (bfloat16), normal range */
static inline double round_bf16(double x) {
  int e;
  double m = frexp(x, &e);
  return ldexp(nearbyint(m * 256.0) / 256.0, e);
}

/* storage: 0 = f64, 1 = f32, 2 = bf16. out_f32 != 0 writes float (exact for 1 and 2). */
void oracle_normal(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double std,
                   int storage, void* out, int out_f32) {
  const uint64_t key = sm64(seed ^ sm64(stream));
  const double two_pi = 2.0 * 3.14159265358979323846;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    const uint64_t i = start + (uint64_t)j;
    const double u1 = u53(sm64(key + 2 * i));
    const double u2 = u53(sm64(key + 2 * i + 1));
    double v = std * (sqrt(-2.0 * log(1.0 - u1)) * cos(two_pi * u2));
    if (storage == 1) v = (double)(float)v;
    else if (storage == 2) v = round_bf16(v);
    if (out_f32) ((float*)out)[j] = (float)v;
    else ((double*)out)[j] = v;
  }
}
